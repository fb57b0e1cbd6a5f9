"""Helpers shared by the GPU parity tests: device copies of the seeded inputs,
the oracle run per (b, h) slice on a thread pool, and error measures."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

WORKERS = min(16, os.cpu_count() or 1)

# Tolerances of the two arithmetic paths against the fp64 oracle run on the
# same (rounded) inputs: float32 inputs -> normwise relative error 1e-4 on
# every output; bf16 inputs with float32 accumulation -> max absolute error
# 1e-2 on every output.
F32_NORMWISE = 1e-4
BF16_MAXABS = 1e-2


def to_device(x: np.ndarray):
    import torch

    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(x).to("cuda")


def oracle_heads(S, K, V, s, heads):
    """Oracle (Qd, Z, Y) for the listed (b, h) pairs, one thread per pair."""
    H = K.shape[1]

    def one(bh):
        b, h = bh
        Sh = S[h] if S.ndim == 3 else S
        Qd, Z, Y = oracle.route(Sh, K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], s)
        return Qd[0, 0], Z[0, 0], Y[0, 0]

    with ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(one, heads))


def all_heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def errors(got: np.ndarray, ref: np.ndarray):
    """(max abs error, normwise relative error max|d| / max|ref|)."""
    d = np.abs(got.astype(np.float64) - ref)
    mx = float(d.max()) if d.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 1.0
    return mx, mx / max(scale, 1e-300)


def assert_close(name, got, ref, dtype):
    mx, rel = errors(got, ref)
    print(f"    {name}: max|err| {mx:.3e}  normwise {rel:.3e}", flush=True)
    if dtype == "f32":
        assert rel <= F32_NORMWISE, f"{name}: normwise error {rel:.3e} > {F32_NORMWISE}"
    else:
        assert mx <= BF16_MAXABS, f"{name}: max abs error {mx:.3e} > {BF16_MAXABS}"
    return mx, rel
