"""Pins of the CPU oracle against what the pages and mathematics fix.

Every check takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees with an independent fact: a hand-derived worked example, a
closed form, an invariance, or a library implementation of the same
definition (torch's scaled_dot_product_attention).  The same checks run
against deliberately broken oracle builds in ``test_oracle_mutations.py``;
each plausible mistake there must trip at least one of them.
"""
from __future__ import annotations

import json
import math
import os
import re

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


# --------------------------------------------------------------- helpers ----

def _eval_expr(e) -> float:
    if isinstance(e, (int, float)):
        return float(e)
    expr = re.sub(r"(\d)(ln3|sqrt3)", r"\1*\2", e)
    expr = expr.replace("sqrt3", "math.sqrt(3)").replace("ln3", "math.log(3)")
    return float(eval(expr, {"__builtins__": {}}, {"math": math}))  # fixture strings only


def _leaves(x):
    if isinstance(x, list) and len(x) == 2 and isinstance(x[0], str) and isinstance(x[1], float):
        return [x]
    if isinstance(x, list):
        out = []
        for y in x:
            out.extend(_leaves(y))
        return out
    return [x]


def _expected(tree, shape):
    vals = []
    for expr, num in _leaves(tree):
        exact = _eval_expr(expr)
        assert abs(exact - num) <= 1e-15 * max(1.0, abs(exact)), (expr, num, exact)
        vals.append(exact)
    return np.array(vals).reshape(shape)


def _inputs(tree):
    return np.vectorize(_eval_expr, otypes=[float])(np.array(tree, dtype=object))


def _rng(seed):
    return np.random.default_rng(seed)


def _torch_route(S, K, V, s):
    """The three stages as three calls of torch's SDPA, float64, CPU."""
    import torch
    import torch.nn.functional as F

    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64))
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64))
    St = torch.from_numpy(np.asarray(S, dtype=np.float64))
    B, H, N, D = Kt.shape
    if St.dim() == 2:
        St = St.expand(B, H, *St.shape)
    else:
        St = St.unsqueeze(0).expand(B, *St.shape)
    St = St.contiguous()
    Qd = F.scaled_dot_product_attention(St, Kt, Vt, scale=s)
    Z = F.scaled_dot_product_attention(Qd, Kt, Vt, scale=s)
    Y = F.scaled_dot_product_attention(Kt, Qd, Z, scale=s)
    return Qd.numpy(), Z.numpy(), Y.numpy()


def _softmax_rows(x):
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=1, keepdims=True)


def _close(a, b, rtol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
    assert err <= rtol, f"{what}: normwise error {err:.3e} > {rtol:.1e}"


# ------------------------------------------------------------------ pins ----

def pin_worked_examples(orc):
    """Hand-derived closed forms (tests/golden/worked_examples.json)."""
    with open(GOLDEN) as f:
        data = json.load(f)
    for ex in data["examples"]:
        S = _inputs(ex["S"])
        K = _inputs(ex["K"])
        V = _inputs(ex["V"])
        B, H, N, D = K.shape
        M = S.shape[0]
        Qd, Z, Y = orc.route(S, K, V, ex["scale"])
        _close(Qd, _expected(ex["Qd"], (B, H, M, D)), 1e-14, ex["name"] + " Qd")
        _close(Z, _expected(ex["Z"], (B, H, M, D)), 1e-14, ex["name"] + " Z")
        _close(Y, _expected(ex["Y"], (B, H, N, D)), 1e-14, ex["name"] + " Y")


def pin_torch_sdpa(orc):
    """Each stage equals torch's SDPA (an independent implementation), float64."""
    rng = _rng(11)
    cases = [(2, 3, 37, 5, 4, 0.7), (1, 2, 64, 16, 16, 0.25), (2, 1, 9, 12, 3, 1.0),
             (1, 1, 1, 3, 2, 0.5), (1, 2, 130, 1, 8, 1 / math.sqrt(8))]
    for B, H, N, M, D, s in cases:
        K = rng.standard_normal((B, H, N, D))
        V = rng.standard_normal((B, H, N, D))
        S = rng.standard_normal((M, D))
        got = orc.route(S, K, V, s)
        ref = _torch_route(S, K, V, s)
        for g, r, name in zip(got, ref, ("Qd", "Z", "Y")):
            _close(g, r, 1e-12, f"torch {name} B{B} H{H} N{N} M{M} D{D}")
        Sh = rng.standard_normal((H, M, D))
        got = orc.route(Sh, K, V, s)
        ref = _torch_route(Sh, K, V, s)
        for g, r, name in zip(got, ref, ("Qd", "Z", "Y")):
            _close(g, r, 1e-12, f"torch per-head {name}")


def pin_low_rank_matrix(orc):
    """Y = W V with W = softmax(s K Qd^T) softmax(s Qd K^T): rank <= M, rows sum to 1, W >= 0."""
    rng = _rng(12)
    for N, M, D, s in [(200, 12, 8, 0.5), (96, 7, 5, 1.0)]:
        K = rng.standard_normal((1, 1, N, D))
        V = rng.standard_normal((1, 1, N, D))
        S = rng.standard_normal((M, D))
        Qd, Z, Y = orc.route(S, K, V, s)
        q, k = Qd[0, 0], K[0, 0]
        W = _softmax_rows(s * k @ q.T) @ _softmax_rows(s * q @ k.T)
        _close(Y[0, 0], W @ V[0, 0], 1e-12, "W V")
        sv = np.linalg.svd(W, compute_uv=False)
        assert sv[M] / sv[0] <= 1e-12, f"rank > M: sigma_M+1/sigma_1 = {sv[M] / sv[0]:.2e}"
        assert np.max(np.abs(W.sum(axis=1) - 1)) <= 1e-13
        assert W.min() >= 0


def pin_identical_tokens(orc):
    """All keys equal: every encode softmax is uniform, so Qd = Z = Y = mean(V)."""
    rng = _rng(13)
    N, M, D = 50, 6, 4
    k = rng.standard_normal(D)
    K = np.broadcast_to(k, (1, 2, N, D)).copy()
    V = rng.standard_normal((1, 2, N, D))
    S = rng.standard_normal((M, D))
    Qd, Z, Y = orc.route(S, K, V, 0.9)
    mean = V.mean(axis=2, keepdims=True)
    _close(Qd, np.broadcast_to(mean, Qd.shape), 1e-14, "identical-token Qd")
    _close(Z, np.broadcast_to(mean, Z.shape), 1e-14, "identical-token Z")
    _close(Y, np.broadcast_to(mean, Y.shape), 1e-14, "identical-token Y")
    V2 = np.broadcast_to(rng.standard_normal(D), V.shape).copy()
    _, _, Y2 = orc.route(S, K, V2, 0.9)
    _close(Y2, V2, 1e-14, "identical tokens and values")


def pin_fixed_query_flare(orc):
    """FLARE with parameter queries = brute-force W V; route(S) = FLARE(seed_encode(S))."""
    rng = _rng(14)
    N, M, D, s = 80, 9, 6, 0.6
    K = rng.standard_normal((1, 2, N, D))
    V = rng.standard_normal((1, 2, N, D))
    Q = rng.standard_normal((M, D))
    Zf, Yf = orc.flare(Q, K, V, s)
    for h in range(2):
        k, v = K[0, h], V[0, h]
        W = _softmax_rows(s * k @ Q.T) @ _softmax_rows(s * Q @ k.T)
        _close(Yf[0, h], W @ v, 1e-12, "FLARE Y vs W V")
        _close(Zf[0, h], _softmax_rows(s * Q @ k.T) @ v, 1e-12, "FLARE Z")
    Qd, Z, Y = orc.route(Q, K, V, s)
    Z2, Y2 = orc.flare(Qd[0], K, V, s)  # per-head queries = the synthesised ones
    _close(Z, Z2, 1e-13, "route Z = FLARE(Qd) Z")
    _close(Y, Y2, 1e-13, "route Y = FLARE(Qd) Y")
    Qd1 = np.stack([orc.sdpa(Q, K[0, h], V[0, h], s) for h in range(2)])
    _close(Qd[0], Qd1, 1e-14, "route Qd = seed encode")


def pin_scale_zero(orc):
    """s = 0: every softmax is uniform, every output row is mean(V)."""
    rng = _rng(15)
    K = rng.standard_normal((2, 2, 33, 5))
    V = rng.standard_normal((2, 2, 33, 5))
    S = rng.standard_normal((4, 5))
    Qd, Z, Y = orc.route(S, K, V, 0.0)
    mean = V.mean(axis=2, keepdims=True)
    for X, name in ((Qd, "Qd"), (Z, "Z"), (Y, "Y")):
        _close(X, np.broadcast_to(mean, X.shape), 1e-14, f"s=0 {name}")


def pin_single_latent(orc):
    """M = 1: the decode weight is 1, so Y_n = Z for every token."""
    rng = _rng(16)
    K = rng.standard_normal((1, 3, 40, 7))
    V = rng.standard_normal((1, 3, 40, 7))
    S = rng.standard_normal((1, 7))
    _, Z, Y = orc.route(S, K, V, 0.8)
    _close(Y, np.broadcast_to(Z, Y.shape), 1e-15, "M=1")


def pin_single_token(orc):
    """N = 1: every output equals the one value row."""
    rng = _rng(17)
    K = rng.standard_normal((2, 2, 1, 6))
    V = rng.standard_normal((2, 2, 1, 6))
    S = rng.standard_normal((5, 6))
    Qd, Z, Y = orc.route(S, K, V, 1.3)
    for X, name in ((Qd, "Qd"), (Z, "Z"), (Y, "Y")):
        _close(X, np.broadcast_to(V, X.shape), 1e-15, f"N=1 {name}")


def pin_permutations(orc):
    """Permuting tokens permutes Y only; permuting seeds permutes Qd and Z only."""
    rng = _rng(18)
    N, M, D, s = 45, 8, 6, 0.7
    K = rng.standard_normal((1, 2, N, D))
    V = rng.standard_normal((1, 2, N, D))
    S = rng.standard_normal((M, D))
    Qd, Z, Y = orc.route(S, K, V, s)
    p = rng.permutation(N)
    Qd2, Z2, Y2 = orc.route(S, K[:, :, p], V[:, :, p], s)
    _close(Qd2, Qd, 1e-13, "token perm Qd")
    _close(Z2, Z, 1e-13, "token perm Z")
    _close(Y2, Y[:, :, p], 1e-13, "token perm Y")
    q = rng.permutation(M)
    Qd3, Z3, Y3 = orc.route(S[q], K, V, s)
    _close(Qd3, Qd[:, :, q], 1e-13, "seed perm Qd")
    _close(Z3, Z[:, :, q], 1e-13, "seed perm Z")
    _close(Y3, Y, 1e-13, "seed perm Y")


def pin_rotation(orc):
    """(S R, K R, V R) for orthogonal R gives (Qd R, Z R, Y R): dot products and
    convex combinations commute with a rotation of the feature axis."""
    rng = _rng(19)
    N, M, D, s = 60, 5, 6, 0.8
    K = rng.standard_normal((1, 1, N, D))
    V = rng.standard_normal((1, 1, N, D))
    S = rng.standard_normal((M, D))
    R, _ = np.linalg.qr(rng.standard_normal((D, D)))
    Qd, Z, Y = orc.route(S, K, V, s)
    Qd2, Z2, Y2 = orc.route(S @ R, K @ R, V @ R, s)
    _close(Qd2, Qd @ R, 1e-13, "rotation Qd")
    _close(Z2, Z @ R, 1e-13, "rotation Z")
    _close(Y2, Y @ R, 1e-13, "rotation Y")


def pin_convexity(orc):
    """Row-stochastic weights: each output column lies within [min V, max V] of its head."""
    rng = _rng(20)
    K = rng.standard_normal((2, 2, 70, 4)) * 3
    V = rng.standard_normal((2, 2, 70, 4))
    S = rng.standard_normal((10, 4)) * 3
    Qd, Z, Y = orc.route(S, K, V, 1.0)
    lo = V.min(axis=2, keepdims=True) - 1e-12
    hi = V.max(axis=2, keepdims=True) + 1e-12
    for X, name in ((Qd, "Qd"), (Z, "Z"), (Y, "Y")):
        assert np.all(X >= lo) and np.all(X <= hi), f"{name} leaves the value range"


def pin_storage_types(orc):
    """bf16 bit patterns and float32 inputs are read as their exact values."""
    rng = _rng(21)
    x = rng.standard_normal((3, 1, 1, 2, 20, 4)).astype(np.float32)
    bits = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # truncation: any bf16 pattern
    exact = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    S_b, K_b, V_b = bits[0, 0, 0, 0, :6], bits[1, 0], bits[2, 0]
    S_e, K_e, V_e = exact[0, 0, 0, 0, :6], exact[1, 0], exact[2, 0]
    got = orc.route(S_b, K_b, V_b, 0.5)
    ref = orc.route(S_e, K_e, V_e, 0.5)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r), "bf16 widening differs from exact values"
    got = orc.route(x[0, 0, 0, 0, :6], x[1, 0], x[2, 0], 0.5)
    ref = orc.route(*(a.astype(np.float64) for a in (x[0, 0, 0, 0, :6], x[1, 0], x[2, 0])), 0.5)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r), "float32 widening differs from exact values"


PINS = [
    pin_worked_examples,
    pin_torch_sdpa,
    pin_low_rank_matrix,
    pin_identical_tokens,
    pin_fixed_query_flare,
    pin_scale_zero,
    pin_single_latent,
    pin_single_token,
    pin_permutations,
    pin_rotation,
    pin_convexity,
    pin_storage_types,
]
