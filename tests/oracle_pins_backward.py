"""Pins of the oracle's backward (gradients of <dY, Y> for the route) against
facts that do not come from its own formulas: central finite differences of
the oracle's forward, torch autograd through torch's SDPA (float64, CPU), a
closed form at s = 0, and linearity in dY.  Used by test_oracle_backward.py,
also against planted mistakes."""
from __future__ import annotations

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)), 1.0)
    assert err <= rtol, f"{what}: normwise error {err:.3e} > {rtol:.1e}"


def _loss(orc, S, K, V, s, dY):
    return float((orc.route(S, K, V, s)[2] * dY).sum())


def _fd(orc, S, K, V, s, dY, which, h=1e-5):
    """Central differences of <dY, Y> with respect to one input, element by element."""
    args = {"S": S, "K": K, "V": V}
    X = args[which]
    g = np.zeros_like(X)
    it = np.nditer(X, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        for sign in (1, -1):
            Xs = X.copy()
            Xs[i] += sign * h
            a = dict(args)
            a[which] = Xs
            g[i] += sign * _loss(orc, a["S"], a["K"], a["V"], s, dY) / (2 * h)
    return g


def pin_finite_differences(orc):
    """Every gradient entry equals the central difference of the forward (shared and per-head seeds)."""
    for per_head, (B, H, N, M, D, s) in ((False, (2, 2, 6, 3, 3, 0.8)), (True, (1, 2, 5, 4, 2, 1.3))):
        rng = _rng(11 + per_head)
        S = rng.standard_normal((H, M, D) if per_head else (M, D))
        K = rng.standard_normal((B, H, N, D))
        V = rng.standard_normal((B, H, N, D))
        dY = rng.standard_normal((B, H, N, D))
        dS, dK, dV = orc.route_backward(S, K, V, s, dY)
        for name, g in (("S", dS), ("K", dK), ("V", dV)):
            _close(g, _fd(orc, S, K, V, s, dY, name), 1e-7, f"d{name} vs finite differences")


def pin_torch_autograd(orc):
    """Gradients equal torch autograd through three calls of torch's SDPA (float64)."""
    import torch
    import torch.nn.functional as F

    rng = _rng(5)
    B, H, N, M, D, s = 2, 3, 40, 7, 4, 0.6
    S = rng.standard_normal((M, D))
    K = rng.standard_normal((B, H, N, D))
    V = rng.standard_normal((B, H, N, D))
    dY = rng.standard_normal((B, H, N, D))
    St = torch.tensor(S, requires_grad=True)
    Kt = torch.tensor(K, requires_grad=True)
    Vt = torch.tensor(V, requires_grad=True)
    Se = St.expand(B, H, M, D)
    Qd = F.scaled_dot_product_attention(Se, Kt, Vt, scale=s)
    Z = F.scaled_dot_product_attention(Qd, Kt, Vt, scale=s)
    Y = F.scaled_dot_product_attention(Kt, Qd, Z, scale=s)
    (Y * torch.tensor(dY)).sum().backward()
    dS, dK, dV = orc.route_backward(S, K, V, s, dY)
    _close(dS, St.grad.numpy(), 1e-12, "dS vs torch autograd")
    _close(dK, Kt.grad.numpy(), 1e-12, "dK vs torch autograd")
    _close(dV, Vt.grad.numpy(), 1e-12, "dV vs torch autograd")


def pin_scale_zero(orc):
    """s = 0: every output row is mean(V), so dS = dK = 0 and every dV_j = sum_n dY_n / N."""
    rng = _rng(6)
    B, H, N, M, D = 1, 2, 9, 4, 3
    S = rng.standard_normal((M, D))
    K = rng.standard_normal((B, H, N, D))
    V = rng.standard_normal((B, H, N, D))
    dY = rng.standard_normal((B, H, N, D))
    dS, dK, dV = orc.route_backward(S, K, V, 0.0, dY)
    assert np.max(np.abs(dS)) == 0.0 and np.max(np.abs(dK)) == 0.0
    ref = np.broadcast_to(dY.sum(axis=2, keepdims=True) / N, dV.shape)
    _close(dV, ref, 1e-14, "dV at s = 0")


def pin_linearity(orc):
    """Gradients are linear in dY."""
    rng = _rng(7)
    B, H, N, M, D, s = 1, 1, 12, 5, 4, 0.9
    S = rng.standard_normal((M, D))
    K = rng.standard_normal((B, H, N, D))
    V = rng.standard_normal((B, H, N, D))
    d1 = rng.standard_normal((B, H, N, D))
    d2 = rng.standard_normal((B, H, N, D))
    g1 = orc.route_backward(S, K, V, s, d1)
    g2 = orc.route_backward(S, K, V, s, d2)
    g12 = orc.route_backward(S, K, V, s, 2.0 * d1 - 3.0 * d2)
    for a, b, c, n in zip(g1, g2, g12, "SKV"):
        _close(c, 2.0 * a - 3.0 * b, 1e-12, f"d{n} linearity")


PINS = [pin_finite_differences, pin_torch_autograd, pin_scale_zero, pin_linearity]
