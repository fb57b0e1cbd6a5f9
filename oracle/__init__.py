"""CPU oracle for the FLARE++ routing forward pass -- test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library in ``rank_latent_attention_seed_amd``
never imports it, and it imports nothing from that library.

The arithmetic lives in ``flarepp_oracle.c`` (plain C, IEEE double, one
thread); this module only marshals numpy arrays into it.  Array conventions:

* ``float32`` / ``float64`` arrays are read as those types;
* ``uint16`` arrays are bf16 bit patterns (the upper half of an fp32).

Functions follow the pages as follows:

* :func:`sdpa` -- one scaled-dot-product attention, softmax over the key
  index ("FLARE: Fast Low-rank Attention Routing Engine", section
  "Основной механизм FLARE", encode and decode steps).
* :func:`route` -- seed encode, encode, decode ("FLARE++: Low-rank attention
  with dynamic attention routing", abstract; French technical summary,
  "Méthodologie").
* :func:`flare` -- fixed-query FLARE (encode and decode with parameter
  queries), the special case the FLARE++ abstract starts from.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "flarepp_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2


def compile_oracle(src: str, out: str) -> str:
    """gcc, single-threaded, -O2, no vector intrinsics, no OpenMP."""
    tmp = out + ".tmp"
    subprocess.run(
        ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"],
        check=True,
    )
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_oracle(SOURCE, LIBRARY)
    return LIBRARY


def _typed(a: np.ndarray):
    """Return (contiguous array, dtype code) for a supported input array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle inputs must be float32, float64 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _heads(Q: np.ndarray, H: int, D: int):
    """(M, element stride between heads) for an M x D or H x M x D query block."""
    if Q.ndim == 2:
        M, stride = Q.shape[0], 0
    elif Q.ndim == 3 and Q.shape[0] == H:
        M = Q.shape[1]
        stride = M * D
    else:
        raise ValueError("queries must be M x D or H x M x D")
    if Q.shape[-1] != D:
        raise ValueError("query last dim must equal D")
    return M, stride


class Oracle:
    """The oracle functions bound to one compiled copy of flarepp_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.oracle_sdpa.argtypes = [vp, ci, i64, vp, ci, vp, ci, i64, i64, i64, dbl, vp]
        lib.oracle_sdpa.restype = ci
        lib.oracle_route.argtypes = [i64, i64, i64, i64, i64, ci, dbl, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_route.restype = ci
        lib.oracle_flare.argtypes = [i64, i64, i64, i64, i64, ci, dbl, i64, vp, vp, vp, vp, vp]
        lib.oracle_flare.restype = ci
        lib.oracle_sdpa_backward.argtypes = [vp, ci, i64, vp, ci, vp, ci, i64, i64, i64, dbl, vp, vp, vp,
                                             vp]
        lib.oracle_sdpa_backward.restype = ci
        lib.oracle_route_backward.argtypes = [i64, i64, i64, i64, i64, ci, dbl, i64, vp, vp, vp, vp, vp,
                                              vp, vp]
        lib.oracle_route_backward.restype = ci
        self._lib = lib
        self.path = path

    def sdpa(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, s: float) -> np.ndarray:
        """out[i] = sum_j softmax_j(s <q_i, k_j>) v_j; q: nq x d, k: nk x d, v: nk x dv."""
        q, qt = _typed(q)
        k, kt = _typed(k)
        v, vt = _typed(v)
        if q.ndim != 2 or k.ndim != 2 or v.ndim != 2:
            raise ValueError("sdpa takes 2-D arrays")
        nq, d = q.shape
        nk, dk = k.shape
        if dk != d or v.shape[0] != nk:
            raise ValueError("shape mismatch")
        dv = v.shape[1]
        out = np.empty((nq, dv), dtype=np.float64)
        rc = self._lib.oracle_sdpa(_ptr(q), qt, nq, _ptr(k), kt, _ptr(v), vt, nk, d, dv, float(s),
                                   _ptr(out))
        if rc != 0:
            raise ValueError("oracle_sdpa rejected its arguments")
        return out

    def route(self, S: np.ndarray, K: np.ndarray, V: np.ndarray, s: float):
        """Seed encode -> encode -> decode for every (b, h).

        K, V: B x H x N x D of one dtype; S: M x D (shared by all heads) or
        H x M x D (per-head seeds), same dtype as K.  Returns (Qd, Z, Y) as
        float64 arrays of shapes B x H x M x D, B x H x M x D, B x H x N x D.
        """
        K, kt = _typed(K)
        V, vt = _typed(V)
        S, st = _typed(S)
        if not (kt == vt == st):
            raise TypeError("S, K and V must share one dtype")
        if K.ndim != 4 or V.shape != K.shape:
            raise ValueError("K and V must be B x H x N x D of one shape")
        B, H, N, D = K.shape
        M, stride = _heads(S, H, D)
        Qd = np.empty((B, H, M, D), dtype=np.float64)
        Z = np.empty((B, H, M, D), dtype=np.float64)
        Y = np.empty((B, H, N, D), dtype=np.float64)
        rc = self._lib.oracle_route(B, H, N, M, D, kt, float(s), stride, _ptr(S), _ptr(K), _ptr(V),
                                    _ptr(Qd), _ptr(Z), _ptr(Y))
        if rc != 0:
            raise ValueError("oracle_route rejected its arguments")
        return Qd, Z, Y

    def flare(self, Q: np.ndarray, K: np.ndarray, V: np.ndarray, s: float):
        """Fixed-query FLARE: Z = SDPA(Q, K, V, s), Y = SDPA(K, Q, Z, s) per (b, h)."""
        K, kt = _typed(K)
        V, vt = _typed(V)
        Q, qt = _typed(Q)
        if not (kt == vt == qt):
            raise TypeError("Q, K and V must share one dtype")
        if K.ndim != 4 or V.shape != K.shape:
            raise ValueError("K and V must be B x H x N x D of one shape")
        B, H, N, D = K.shape
        M, stride = _heads(Q, H, D)
        Z = np.empty((B, H, M, D), dtype=np.float64)
        Y = np.empty((B, H, N, D), dtype=np.float64)
        rc = self._lib.oracle_flare(B, H, N, M, D, kt, float(s), stride, _ptr(Q), _ptr(K), _ptr(V),
                                    _ptr(Z), _ptr(Y))
        if rc != 0:
            raise ValueError("oracle_flare rejected its arguments")
        return Z, Y


    def sdpa_backward(self, q, k, v, s: float, dout):
        """Gradients (dq, dk, dv) of <dout, SDPA(q, k, v, s)> (float64 arrays)."""
        q, qt = _typed(q)
        k, kt = _typed(k)
        v, vt = _typed(v)
        dout = np.ascontiguousarray(dout, dtype=np.float64)
        nq, d = q.shape
        nk, dv = v.shape
        if k.shape != (nk, d) or dout.shape != (nq, dv):
            raise ValueError("shape mismatch")
        dq = np.zeros((nq, d))
        dk = np.zeros((nk, d))
        dvv = np.zeros((nk, dv))
        rc = self._lib.oracle_sdpa_backward(_ptr(q), qt, nq, _ptr(k), kt, _ptr(v), vt, nk, d, dv,
                                            float(s), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dvv))
        if rc != 0:
            raise ValueError("oracle_sdpa_backward rejected its arguments")
        return dq, dk, dvv

    def route_backward(self, S, K, V, s: float, dY):
        """Gradients (dS, dK, dV) of <dY, Y> for the route Y(S, K, V); dS has
        the shape of S (a shared seed block collects the gradient of every
        (b, h)).  float64 results."""
        K, kt = _typed(K)
        V, vt = _typed(V)
        S, st = _typed(S)
        if not (kt == vt == st):
            raise TypeError("S, K and V must share one dtype")
        B, H, N, D = K.shape
        M, stride = _heads(S, H, D)
        dY = np.ascontiguousarray(dY, dtype=np.float64)
        if dY.shape != K.shape:
            raise ValueError("dY must be B x H x N x D")
        dS = np.empty(S.shape, dtype=np.float64)
        dK = np.empty(K.shape, dtype=np.float64)
        dV = np.empty(K.shape, dtype=np.float64)
        rc = self._lib.oracle_route_backward(B, H, N, M, D, kt, float(s), stride, _ptr(S), _ptr(K),
                                             _ptr(V), _ptr(dY), _ptr(dS), _ptr(dK), _ptr(dV))
        if rc != 0:
            raise ValueError("oracle_route_backward rejected its arguments")
        return dS, dK, dV


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build(force=True)
        _default = Oracle(LIBRARY)
    return _default


def sdpa(q, k, v, s):
    return default().sdpa(q, k, v, s)


def route(S, K, V, s):
    return default().route(S, K, V, s)


def flare(Q, K, V, s):
    return default().flare(Q, K, V, s)


def sdpa_backward(q, k, v, s, dout):
    return default().sdpa_backward(q, k, v, s, dout)


def route_backward(S, K, V, s, dY):
    return default().route_backward(S, K, V, s, dY)
