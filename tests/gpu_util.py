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


def poisoned(shape, dtype=None):
    """A device tensor filled with NaN bit patterns (every byte 0xFF), so a
    kernel that reads memory it never wrote, or leaves part of an output
    unwritten, cannot pass a comparison with the oracle."""
    import torch

    n = 1
    for x in shape:
        n *= int(x)
    dtype = dtype or torch.float32
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")[:nbytes].view(dtype).view(*shape)


def route_poisoned(fp, S, K, V, scale, tuning=None):
    """Y, Qd, Z of flarepp_route (flarepp_route_tuned when `tuning` is given),
    with the workspace and all three outputs NaN-poisoned before the call."""
    import torch

    desc = fp.desc_for(S, K, scale)
    B, H, N, D = K.shape
    M = desc.M
    Y, Qd, Z = poisoned((B, H, N, D)), poisoned((B, H, M, D)), poisoned((B, H, M, D))
    n = fp.flarepp_workspace_size_tuned(desc, fp.OP_ROUTE, tuning)
    ws = poisoned((max(n, 1),), torch.uint8)
    stream = fp._stream(None)
    if tuning is None:
        st = fp.flarepp_route(desc, S.data_ptr(), K.data_ptr(), V.data_ptr(), Y.data_ptr(), Qd.data_ptr(),
                              Z.data_ptr(), ws.data_ptr(), n, stream)
    else:
        st = fp.flarepp_route_tuned(desc, tuning, S.data_ptr(), K.data_ptr(), V.data_ptr(), Y.data_ptr(),
                                    Qd.data_ptr(), Z.data_ptr(), ws.data_ptr(), n, stream)
    if st != 0:
        raise fp.FlareppError(st, "flarepp_route")
    return Y, Qd, Z


def backward_poisoned(fp, S, K, V, scale, dY):
    """dS, dK, dV of flarepp_route_backward with the workspace and the three
    gradient outputs NaN-poisoned before the call."""
    import torch

    desc = fp.desc_for(S, K, scale)
    dS = poisoned(tuple(S.shape))
    dK, dV = poisoned(tuple(K.shape)), poisoned(tuple(K.shape))
    n = fp.flarepp_workspace_size(desc, fp.OP_ROUTE_BACKWARD)
    ws = poisoned((max(n, 1),), torch.uint8)
    st = fp.flarepp_route_backward(desc, S.data_ptr(), K.data_ptr(), V.data_ptr(), dY.data_ptr(), dS.data_ptr(),
                                   dK.data_ptr(), dV.data_ptr(), ws.data_ptr(), n, fp._stream(None))
    if st != 0:
        raise fp.FlareppError(st, "flarepp_route_backward")
    return dS, dK, dV


def spectrum_poisoned(fp, S, K, V, scale):
    """Eigenvalues and G of flarepp_spectrum with the workspace and both
    outputs NaN-poisoned before the call."""
    import torch

    desc = fp.desc_for(S, K, scale)
    B, H, N, D = K.shape
    M = desc.M
    eig, G = poisoned((B, H, M)), poisoned((B, H, M, M))
    n = fp.flarepp_workspace_size(desc, fp.OP_SPECTRUM)
    ws = poisoned((max(n, 1),), torch.uint8)
    st = fp.flarepp_spectrum(desc, S.data_ptr(), K.data_ptr(), V.data_ptr(), eig.data_ptr(), G.data_ptr(),
                             ws.data_ptr(), n, fp._stream(None))
    if st != 0:
        raise fp.FlareppError(st, "flarepp_spectrum")
    return eig, G


def compare_route(p, Y, Qd, Z, heads=None, ref=None):
    """Element-wise comparison of the route's three outputs with the oracle
    on the listed heads (all by default); returns the oracle results."""
    import torch

    torch.cuda.synchronize()
    Y, Qd, Z = Y.cpu().numpy(), Qd.cpu().numpy(), Z.cpu().numpy()
    heads = heads or all_heads(p.B, p.H)
    ref = ref or oracle_heads(p.S, p.K, p.V, p.scale, heads)
    out = {}
    out["Qd"] = assert_close("Qd", np.stack([Qd[b, h] for b, h in heads]), np.stack([r[0] for r in ref]), p.dtype)
    out["Z"] = assert_close("Z", np.stack([Z[b, h] for b, h in heads]), np.stack([r[1] for r in ref]), p.dtype)
    out["Y"] = assert_close("Y", np.stack([Y[b, h] for b, h in heads]), np.stack([r[2] for r in ref]), p.dtype)
    assert np.isfinite(Y).all()
    return ref, out


def saved_backward_poisoned(fp, S, K, V, scale, dY):
    """flarepp_route_save, then flarepp_route_backward_saved on its saved
    forward, every output and both workspaces NaN-poisoned before the calls:
    (Y, Qd, Z, lse) and (dS, dK, dV)."""
    import torch

    desc = fp.desc_for(S, K, scale)
    B, H, N, D = K.shape
    M = desc.M
    n = fp.flarepp_workspace_size(desc, fp.OP_ROUTE_BACKWARD)
    Y = poisoned((B, H, N, D))
    Qd, Z = poisoned((B, H, M, D)), poisoned((B, H, M, D))
    lse = poisoned((fp.saved_lse_count(desc),))
    ws = poisoned((max(n, 1),), torch.uint8)
    st = fp.flarepp_route_save(desc, S.data_ptr(), K.data_ptr(), V.data_ptr(), Y.data_ptr(), Qd.data_ptr(),
                               Z.data_ptr(), lse.data_ptr(), ws.data_ptr(), n, fp._stream(None))
    if st != 0:
        raise fp.FlareppError(st, "flarepp_route_save")
    dS = poisoned(tuple(S.shape))
    dK, dV = poisoned(tuple(K.shape)), poisoned(tuple(K.shape))
    ws2 = poisoned((max(n, 1),), torch.uint8)
    st = fp.flarepp_route_backward_saved(desc, S.data_ptr(), K.data_ptr(), V.data_ptr(), Qd.data_ptr(),
                                         Z.data_ptr(), lse.data_ptr(), dY.data_ptr(), dS.data_ptr(),
                                         dK.data_ptr(), dV.data_ptr(), ws2.data_ptr(), n, fp._stream(None))
    if st != 0:
        raise fp.FlareppError(st, "flarepp_route_backward_saved")
    return (Y, Qd, Z, lse), (dS, dK, dV)
