"""Pins of the spectral oracle (oracle/spectral.py) against facts that do not
come from its own code path: the N x N mixing matrix built by brute force,
closed forms at s = 0, M = 1 and identical keys, and the structure of
W_enc W_dec (nonnegative, rows summing to one, similar to a symmetric
positive semidefinite matrix: real eigenvalues in [0, 1] led by 1)."""
from __future__ import annotations

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _softmax_rows(x):
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def pin_brute_force_mixing_matrix(sp, orc):
    """The nonzero eigenvalues of the N x N W = W_dec W_enc built from the
    oracle's route outputs by explicit softmaxes equal the spectrum."""
    rng = _rng(1)
    B, H, N, M, D, s = 1, 2, 24, 5, 4, 0.9
    S = rng.standard_normal((M, D))
    K = rng.standard_normal((B, H, N, D))
    V = rng.standard_normal((B, H, N, D))
    Qd, _, _ = orc.route(S, K, V, s)
    ev = sp.spectrum(S, K, V, s)
    for h in range(H):
        L = s * Qd[0, h] @ K[0, h].T
        W = _softmax_rows(L.T) @ _softmax_rows(L)  # N x N
        evn = np.linalg.eigvals(W)
        evn = evn[np.argsort(-evn.real)]
        assert np.max(np.abs(evn[:M] - ev[0, h])) <= 1e-10, "spectrum differs from the N x N matrix"
        assert np.max(np.abs(evn[M:])) <= 1e-10, "N x N matrix has more than M nonzero eigenvalues"


def pin_structure(sp, orc):
    """Real eigenvalues in [0, 1], the largest equal to 1."""
    rng = _rng(2)
    S = rng.standard_normal((6, 3))
    K = rng.standard_normal((2, 1, 40, 3)) * 2.0
    V = rng.standard_normal((2, 1, 40, 3))
    ev = sp.spectrum(S, K, V, 0.7)
    assert np.max(np.abs(ev.imag)) <= 1e-10
    assert np.min(ev.real) >= -1e-10 and np.max(ev.real) <= 1 + 1e-10
    assert np.max(np.abs(ev[..., 0] - 1.0)) <= 1e-10


def pin_scale_zero(sp, orc):
    """s = 0: every softmax is uniform, W_enc W_dec = ones / M: spectrum {1, 0, ...}."""
    rng = _rng(3)
    S = rng.standard_normal((4, 3))
    K = rng.standard_normal((1, 1, 10, 3))
    V = rng.standard_normal((1, 1, 10, 3))
    ev = sp.spectrum(S, K, V, 0.0)[0, 0]
    assert abs(ev[0] - 1.0) <= 1e-12 and np.max(np.abs(ev[1:])) <= 1e-12


def pin_identical_keys(sp, orc):
    """All keys equal: W_enc is uniform over tokens, so W_enc W_dec = 1 w^T with
    w the (common) decode row: spectrum {sum(w) = 1, 0, ...}."""
    rng = _rng(4)
    k = rng.standard_normal(3)
    K = np.broadcast_to(k, (1, 1, 12, 3)).copy()
    V = rng.standard_normal((1, 1, 12, 3))
    S = rng.standard_normal((5, 3))
    ev = sp.spectrum(S, K, V, 1.1)[0, 0]
    assert abs(ev[0] - 1.0) <= 1e-12 and np.max(np.abs(ev[1:])) <= 1e-12


def pin_single_latent(sp, orc):
    """M = 1: the product is the 1 x 1 matrix [1]."""
    rng = _rng(5)
    ev = sp.spectrum(rng.standard_normal((1, 2)), rng.standard_normal((1, 1, 7, 2)),
                     rng.standard_normal((1, 1, 7, 2)), 0.5)
    assert abs(ev[0, 0, 0] - 1.0) <= 1e-12


PINS = [pin_brute_force_mixing_matrix, pin_structure, pin_scale_zero, pin_identical_keys, pin_single_latent]
