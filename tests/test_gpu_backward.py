"""GPU parity of flarepp_route_backward (float32 and bf16 inputs) against the
oracle's backward: dS, dK, dV element by element on the same seeded inputs
(the bf16 values, exactly, for the oracle), through the C ABI."""
import numpy as np
import pytest

from rank_latent_attention_seed_amd import inputs
from gpu_util import assert_close, backward_poisoned, oracle_heads, saved_backward_poisoned, to_device

pytestmark = pytest.mark.gpu

# tolerances, normwise per gradient tensor (max |err| over max |ref|): the
# float32 path 1e-4 as for the forward; the bf16 path (matrix-core products
# from bf16 operands and weights, float32 accumulation) 1e-2
BWD_NORMWISE = {"f32": 1e-4, "bf16": 1e-2}


@pytest.fixture(scope="module")
def fp():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rank_latent_attention_seed_amd import flarepp

    flarepp.library()
    return flarepp


def run_and_compare(fp, p, label, seed=0):
    import oracle
    import torch

    tol = BWD_NORMWISE[p.dtype]
    print(f"\n  case {label}: B{p.B} H{p.H} N{p.N} M{p.M} D{p.D} {p.dtype} s={p.scale:g}", flush=True)
    rng = np.random.default_rng(seed + 100)
    dY = rng.standard_normal((p.B, p.H, p.N, p.D)).astype(np.float32)
    S, K, V, G = to_device(p.S), to_device(p.K), to_device(p.V), to_device(dY)
    # workspace and gradients NaN-poisoned: every element must be written
    dS, dK, dV = backward_poisoned(fp, S, K, V, p.scale, G)
    torch.cuda.synchronize()
    rS, rK, rV = oracle.route_backward(p.S, p.K, p.V, p.scale, dY.astype(np.float64))
    # normwise per gradient tensor: max|err| / max|ref| of that tensor.  A
    # gradient that is exactly zero in the mathematics (dK at N = 1, dS and
    # dK at s = 0) has no scale of its own and is held to the largest of the
    # three instead.
    joint = max(float(np.abs(r).max()) for r in (rS, rK, rV))
    for name, got, ref in (("dS", dS, rS), ("dK", dK, rK), ("dV", dV, rV)):
        err = float(np.abs(got.cpu().numpy().astype(np.float64) - ref).max())
        own = float(np.abs(ref).max())
        scale = own if own > 0.0 else joint
        print(f"    {name}: max|err| {err:.3e}  normwise {err / scale:.3e} (scale {'own' if own > 0 else 'joint'})",
              flush=True)
        assert err <= tol * scale, f"{name}: {err:.3e} > {tol} x {scale:.3e}"


CASES = [
    # B, H, N, M, D, scale, per-head seeds
    (1, 2, 300, 20, 16, 0.25, False),
    (2, 1, 1000, 64, 32, 1 / np.sqrt(32), False),
    (1, 3, 777, 33, 32, 0.4, True),
    (1, 1, 2000, 256, 32, 1 / np.sqrt(32), False),
    (2, 2, 129, 100, 16, 1.0, False),
    (1, 1, 1, 5, 16, 0.5, False),
    (1, 2, 64, 1, 32, 0.7, True),
    (1, 2, 900, 48, 32, -1.0, False),      # s < 0: the bounds use |s|
]


@pytest.mark.parametrize("B,H,N,M,D,scale,per_head", CASES)
def test_backward_matches_oracle(fp, B, H, N, M, D, scale, per_head):
    p = inputs.random_problem(B, H, N, M, D, dtype="f32", scale=scale, seed=N + M, per_head_seeds=per_head)
    run_and_compare(fp, p, f"backward N{N} M{M} D{D}", seed=N)


def test_backward_scale_zero(fp):
    p = inputs.random_problem(1, 2, 500, 16, 32, dtype="f32", scale=0.0, seed=3)
    run_and_compare(fp, p, "backward s=0")


def test_backward_sharp_logits(fp):
    # keys of spread 4 and s = 1: the per-token bound exceeds the safe span,
    # so the decode pass takes its exact-max fallback
    p = inputs.random_problem(1, 1, 600, 48, 16, dtype="f32", scale=1.0, seed=8, sigma=4.0, sigma_v=1.0)
    run_and_compare(fp, p, "backward sharp logits")


def test_backward_linear_and_deterministic(fp):
    """At a larger size: doubling dY doubles every gradient exactly (powers
    of two scale float32 exactly through every linear step), and two calls
    agree bit for bit."""
    import torch

    p = inputs.random_problem(1, 2, 20000, 128, 32, dtype="f32", scale=0.2, seed=4)
    print("\n  case backward linearity / determinism", flush=True)
    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    G = torch.randn((p.B, p.H, p.N, p.D), generator=torch.Generator().manual_seed(1)).cuda()
    a = fp.route_backward(S, K, V, p.scale, G)
    b = fp.route_backward(S, K, V, p.scale, G)
    c = fp.route_backward(S, K, V, p.scale, 2.0 * G)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y), "two identical calls differ"
        assert torch.equal(2.0 * x, z), "gradients not exactly linear in dY"


BF16_CASES = [
    # B, H, N, M, D, scale, per-head seeds
    (1, 2, 300, 20, 16, 0.25, False),
    (2, 1, 1000, 64, 32, 1 / np.sqrt(32), False),
    (1, 3, 777, 33, 32, 0.4, True),
    (1, 1, 5000, 256, 32, 1 / np.sqrt(32), False),   # 20 token splits, all 256 latents
    (2, 2, 129, 100, 16, 1.0, False),
    (1, 1, 1, 5, 16, 0.5, False),
    (1, 2, 64, 1, 32, 0.7, True),
    (1, 2, 900, 48, 32, -1.0, False),                 # s < 0
    (1, 2, 3000, 128, 32, 1.0, False),                # sharp softmaxes
    (1, 1, 20000, 128, 16, 0.25, False),
]


@pytest.mark.parametrize("B,H,N,M,D,scale,per_head", BF16_CASES)
def test_backward_bf16_matches_oracle(fp, B, H, N, M, D, scale, per_head):
    p = inputs.random_problem(B, H, N, M, D, dtype="bf16", scale=scale, seed=N + M + 1, per_head_seeds=per_head)
    run_and_compare(fp, p, f"backward bf16 N{N} M{M} D{D}", seed=N + 1)


def test_backward_bf16_scale_zero(fp):
    p = inputs.random_problem(1, 2, 500, 16, 32, dtype="bf16", scale=0.0, seed=5)
    run_and_compare(fp, p, "backward bf16 s=0")


def test_backward_bf16_deterministic(fp):
    """Two calls on the million-point shapes' per-head slice agree bit for
    bit (no atomics; the split plan is a function of the descriptor)."""
    import torch

    p = inputs.random_problem(1, 2, 65536, 256, 32, dtype="bf16", scale=1 / np.sqrt(32), seed=6)
    print("\n  case backward bf16 determinism N65536 M256", flush=True)
    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    G = torch.randn((p.B, p.H, p.N, p.D), generator=torch.Generator().manual_seed(2)).cuda()
    a = fp.route_backward(S, K, V, p.scale, G)
    b = fp.route_backward(S, K, V, p.scale, G)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.isfinite(x).all(), "non-finite gradient"
        assert torch.equal(x, y), "two identical calls differ"


SAVED_CASES = [
    # B, H, N, M, D, scale, per-head seeds
    (1, 2, 300, 20, 16, 0.25, False),
    (1, 3, 777, 33, 32, 0.4, True),
    (1, 1, 5000, 256, 32, 1 / np.sqrt(32), False),
    (2, 2, 129, 100, 16, 1.0, False),
    (1, 2, 900, 48, 32, -1.0, False),
    (1, 2, 3000, 128, 32, 1.0, False),
]


@pytest.mark.parametrize("B,H,N,M,D,scale,per_head", SAVED_CASES)
def test_saved_forward_and_backward(fp, B, H, N, M, D, scale, per_head):
    """flarepp_route_save's outputs against the oracle's forward, and
    flarepp_route_backward_saved's gradients against the oracle's backward
    and against flarepp_route_backward on the same inputs (which recomputes
    the same forward stages: they differ only by the rounding of the latent
    norms that each path forms), all buffers NaN-poisoned."""
    import oracle
    import torch

    p = inputs.random_problem(B, H, N, M, D, dtype="bf16", scale=scale, seed=N + M + 7, per_head_seeds=per_head)
    print(f"\n  case saved forward/backward: B{B} H{H} N{N} M{M} D{D} s={scale:g}", flush=True)
    rng = np.random.default_rng(N + 9)
    dY = rng.standard_normal((B, H, N, D)).astype(np.float32)
    S, K, V, G = to_device(p.S), to_device(p.K), to_device(p.V), to_device(dY)
    (Y, Qd, Z, lse), (dS, dK, dV) = saved_backward_poisoned(fp, S, K, V, p.scale, G)
    rS, rK, rV = backward_poisoned(fp, S, K, V, p.scale, G)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all(), "log-sum-exp rows left unwritten"
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_heads(p.S, p.K, p.V, p.scale, heads)
    for name, got, k in (("Qd", Qd, 0), ("Z", Z, 1), ("Y", Y, 2)):
        g = got.cpu().numpy()
        assert_close(name, np.stack([g[b, h] for b, h in heads]), np.stack([r[k] for r in ref]), "bf16")
    oS, oK, oV = oracle.route_backward(p.S, p.K, p.V, p.scale, dY.astype(np.float64))
    joint = max(float(np.abs(r).max()) for r in (oS, oK, oV))
    for name, got, rec, ref in (("dS", dS, rS, oS), ("dK", dK, rK, oK), ("dV", dV, rV, oV)):
        g, r = got.cpu().numpy().astype(np.float64), rec.cpu().numpy().astype(np.float64)
        own = float(np.abs(ref).max())
        scale_ = own if own > 0.0 else joint
        err = float(np.abs(g - ref).max())
        diff = float(np.abs(g - r).max())
        print(f"    {name}: vs oracle {err / scale_:.3e} normwise, vs recomputing backward {diff / scale_:.3e}",
              flush=True)
        assert err <= BWD_NORMWISE["bf16"] * scale_, f"{name}: {err:.3e} vs oracle"
        assert diff <= 1e-3 * scale_, f"{name}: saved and recomputing backward differ by {diff:.3e}"
