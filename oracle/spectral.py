"""Spectrum of the routing's mixing matrix -- TEST INFRASTRUCTURE ONLY (the
tests, the smoke check and the benchmark's CPU-baseline leg may call it; the
library never does).

The FLARE summary ("FLARE: Fast Low-rank Attention Routing Engine", section
"Спектральный анализ") analyses the learned communication matrices by an
eigendecomposition that costs O(M^3 + M^2 N): the N x N mixing matrix
W = W_dec W_enc (section "Матрица коммуникации низкого ранга") has rank <= M,
and its nonzero eigenvalues are those of the M x M product W_enc W_dec (AB and
BA share their nonzero spectrum).  For FLARE++ the routing queries are the
synthesised Qd of the seed encode.

Per (b, h), in float64 with numpy:
    W_enc[m, n] = softmax_n(s <Qd_m, K_n>)    (M x N, the encode weights)
    W_dec[n, m] = softmax_m(s <K_n, Qd_m>)    (N x M, the decode weights)
    eigenvalues of C = W_enc W_dec            (numpy.linalg.eigvals)
sorted by decreasing real part.
"""
from __future__ import annotations

import numpy as np

from . import route as _route


def _widen(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns: the top 16 bits of a float32
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _softmax_rows(x):
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def mixing_factors(S, K, V, s):
    """(W_enc, W_dec) per (b, h): arrays B x H x M x N and B x H x N x M."""
    Qd, _, _ = _route(S, K, V, s)
    Kw = _widen(K)
    L = s * np.einsum("bhmd,bhnd->bhmn", Qd, Kw)  # logits shared by both stages
    B, H, M, N = L.shape
    W_enc = np.empty_like(L)
    W_dec = np.empty((B, H, N, M))
    for b in range(B):
        for h in range(H):
            W_enc[b, h] = _softmax_rows(L[b, h])
            W_dec[b, h] = _softmax_rows(L[b, h].T)
    return W_enc, W_dec


def spectrum(S, K, V, s):
    """Eigenvalues of W_enc W_dec per (b, h): complex array B x H x M, by
    decreasing real part."""
    W_enc, W_dec = mixing_factors(S, K, V, s)
    B, H, M, _ = W_enc.shape
    out = np.empty((B, H, M), dtype=np.complex128)
    for b in range(B):
        for h in range(H):
            ev = np.linalg.eigvals(W_enc[b, h] @ W_dec[b, h])
            out[b, h] = ev[np.argsort(-ev.real, kind="stable")]
    return out
