"""Thin Python binding of libflarepp (ctypes).

The functions named ``flarepp_*`` mirror the C ABI in ``include/flarepp.h``
one to one: they take a :class:`FlareppDesc`, raw device addresses (ints) and
a stream handle, and only marshal arguments.  ``route``, ``seed_encode``,
``encode``, ``decode`` and ``flare`` are conveniences over them that take
torch tensors already on the GPU and allocate outputs and workspace with
torch (device memory and streams are all torch is used for).  Every step of
the computation runs in the library's HIP kernels; there is no fallback: if
``libflarepp.so`` is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libflarepp.so")

F32, BF16 = 0, 1
OP_SEED_ENCODE, OP_ENCODE, OP_DECODE, OP_ROUTE, OP_FLARE, OP_ROUTE_BACKWARD, OP_SPECTRUM = range(7)
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE_TOO_SMALL", 4: "ALIASING",
          5: "HIP_ERROR", 6: "SCRATCH_LIMIT"}
ABI_VERSION = 2
SYMBOLS = ("flarepp_abi_version", "flarepp_status_string", "flarepp_workspace_size",
           "flarepp_seed_encode", "flarepp_encode", "flarepp_decode", "flarepp_route",
           "flarepp_flare", "flarepp_route_backward", "flarepp_spectrum", "flarepp_route_profiled",
           "flarepp_workspace_size_tuned", "flarepp_route_tuned", "flarepp_route_noalloc",
           "flarepp_noalloc_scratch_bytes", "flarepp_shard_records_size", "flarepp_encode_shard",
           "flarepp_merge_shards", "flarepp_route_save", "flarepp_route_backward_saved")
KERNEL_KINDS = {0: "prep", 1: "seed_encode", 2: "encode", 3: "merge", 4: "decode"}


class FlareppDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("M", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("seed_head_stride", ctypes.c_int64),
    ]


class FlareppTuning(ctypes.Structure):
    """Explicit launch choices (0 = the library's own, a function of the descriptor)."""
    _fields_ = [
        ("splits", ctypes.c_int32),
        ("head_group", ctypes.c_int32),
        ("decode_kernel", ctypes.c_int32),
        ("decode_wg_per_cu", ctypes.c_int32),
    ]


class FlareppError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_lib().flarepp_status_string(status).decode()})")


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is not built; run `python -m rank_latent_attention_seed_amd.build` "
                "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(LIBRARY)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        dp = ctypes.POINTER(FlareppDesc)
        lib.flarepp_abi_version.restype = ctypes.c_int
        lib.flarepp_abi_version.argtypes = []
        lib.flarepp_status_string.restype = ctypes.c_char_p
        lib.flarepp_status_string.argtypes = [ctypes.c_int]
        lib.flarepp_workspace_size.restype = ctypes.c_int
        lib.flarepp_workspace_size.argtypes = [dp, i32, ctypes.POINTER(sz)]
        lib.flarepp_seed_encode.restype = ctypes.c_int
        lib.flarepp_seed_encode.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_encode.restype = ctypes.c_int
        lib.flarepp_encode.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_decode.restype = ctypes.c_int
        lib.flarepp_decode.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_route.restype = ctypes.c_int
        lib.flarepp_route.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_flare.restype = ctypes.c_int
        lib.flarepp_flare.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_route_backward.restype = ctypes.c_int
        lib.flarepp_route_backward.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_route_save.restype = ctypes.c_int
        lib.flarepp_route_save.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_route_backward_saved.restype = ctypes.c_int
        lib.flarepp_route_backward_saved.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_spectrum.restype = ctypes.c_int
        lib.flarepp_spectrum.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_route_profiled.restype = ctypes.c_int
        lib.flarepp_route_profiled.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                               ctypes.POINTER(vp), ctypes.POINTER(i32), i32,
                                               ctypes.POINTER(i32)]
        tp = ctypes.POINTER(FlareppTuning)
        lib.flarepp_workspace_size_tuned.restype = ctypes.c_int
        lib.flarepp_workspace_size_tuned.argtypes = [dp, i32, tp, ctypes.POINTER(sz)]
        lib.flarepp_route_tuned.restype = ctypes.c_int
        lib.flarepp_route_tuned.argtypes = [dp, tp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flarepp_route_noalloc.restype = ctypes.c_int
        lib.flarepp_route_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp]
        lib.flarepp_noalloc_scratch_bytes.restype = sz
        lib.flarepp_noalloc_scratch_bytes.argtypes = []
        lib.flarepp_shard_records_size.restype = ctypes.c_int
        lib.flarepp_shard_records_size.argtypes = [dp, i32, ctypes.POINTER(sz)]
        lib.flarepp_encode_shard.restype = ctypes.c_int
        lib.flarepp_encode_shard.argtypes = [dp, i32, vp, vp, vp, vp, i32, i32, vp, sz, vp]
        lib.flarepp_merge_shards.restype = ctypes.c_int
        lib.flarepp_merge_shards.argtypes = [dp, vp, i32, vp, vp]
        if lib.flarepp_abi_version() != ABI_VERSION:
            raise RuntimeError("libflarepp ABI version mismatch")
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def make_desc(B, H, N, M, D, dtype, scale, seed_head_stride=0) -> FlareppDesc:
    return FlareppDesc(int(B), int(H), int(N), int(M), int(D), int(dtype), float(scale),
                       int(seed_head_stride))


def _check(status: int, where: str):
    if status != 0:
        raise FlareppError(status, where)


# ---------------------------------------------------------------- C ABI ----

def flarepp_abi_version() -> int:
    return _lib().flarepp_abi_version()


def flarepp_status_string(status: int) -> str:
    return _lib().flarepp_status_string(status).decode()


def flarepp_workspace_size(desc: FlareppDesc, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib().flarepp_workspace_size(ctypes.byref(desc), op, ctypes.byref(n)),
           "flarepp_workspace_size")
    return n.value


def _tuning_ref(tuning):
    return None if tuning is None else ctypes.byref(tuning)


def flarepp_workspace_size_tuned(desc: FlareppDesc, op: int, tuning) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib().flarepp_workspace_size_tuned(ctypes.byref(desc), op, _tuning_ref(tuning),
                                               ctypes.byref(n)), "flarepp_workspace_size_tuned")
    return n.value


def flarepp_route_tuned(desc, tuning, S, K, V, Y, Qd_out, Z_out, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_route_tuned(ctypes.byref(desc), _tuning_ref(tuning), S, K, V, Y, Qd_out, Z_out,
                                      ws, ws_bytes, stream)


def flarepp_route_noalloc(desc, S, K, V, Y, Qd_out, Z_out, stream) -> int:
    return _lib().flarepp_route_noalloc(ctypes.byref(desc), S, K, V, Y, Qd_out, Z_out, stream)


def flarepp_shard_records_size(desc, nslots) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib().flarepp_shard_records_size(ctypes.byref(desc), int(nslots), ctypes.byref(n)),
           "flarepp_shard_records_size")
    return n.value


def flarepp_encode_shard(desc, stage, Q, K, V, rec, slot, nslots, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_encode_shard(ctypes.byref(desc), int(stage), Q, K, V, rec, int(slot), int(nslots), ws,
                                       ws_bytes, stream)


def flarepp_merge_shards(desc, rec, nslots, out, stream) -> int:
    return _lib().flarepp_merge_shards(ctypes.byref(desc), rec, int(nslots), out, stream)


def flarepp_noalloc_scratch_bytes() -> int:
    return _lib().flarepp_noalloc_scratch_bytes()


def make_tuning(splits=0, head_group=0, decode_kernel=0, decode_wg_per_cu=0) -> FlareppTuning:
    return FlareppTuning(int(splits), int(head_group), int(decode_kernel), int(decode_wg_per_cu))


def flarepp_seed_encode(desc, S, K, V, Qd, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_seed_encode(ctypes.byref(desc), S, K, V, Qd, ws, ws_bytes, stream)


def flarepp_encode(desc, Qd, K, V, Z, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_encode(ctypes.byref(desc), Qd, K, V, Z, ws, ws_bytes, stream)


def flarepp_decode(desc, Qd, Z, K, Y, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_decode(ctypes.byref(desc), Qd, Z, K, Y, ws, ws_bytes, stream)


def flarepp_route(desc, S, K, V, Y, Qd_out, Z_out, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_route(ctypes.byref(desc), S, K, V, Y, Qd_out, Z_out, ws, ws_bytes, stream)


def flarepp_flare(desc, Q, K, V, Y, Z_out, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_flare(ctypes.byref(desc), Q, K, V, Y, Z_out, ws, ws_bytes, stream)


def flarepp_spectrum(desc, S, K, V, eig, sym_out, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_spectrum(ctypes.byref(desc), S, K, V, eig, sym_out, ws, ws_bytes, stream)


def flarepp_route_backward(desc, S, K, V, dY, dS, dK, dV, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_route_backward(ctypes.byref(desc), S, K, V, dY, dS, dK, dV, ws, ws_bytes,
                                         stream)


def flarepp_route_save(desc, S, K, V, Y, Qd_out, Z_out, lse_out, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_route_save(ctypes.byref(desc), S, K, V, Y, Qd_out, Z_out, lse_out, ws, ws_bytes,
                                     stream)


def flarepp_route_backward_saved(desc, S, K, V, Qd, Z, lse, dY, dS, dK, dV, ws, ws_bytes, stream) -> int:
    return _lib().flarepp_route_backward_saved(ctypes.byref(desc), S, K, V, Qd, Z, lse, dY, dS, dK, dV, ws,
                                               ws_bytes, stream)


def saved_lse_count(desc: FlareppDesc) -> int:
    """Floats of the saved log-sum-exp buffer: [2][B H][16 ceil(M / 16)]."""
    return 2 * desc.B * desc.H * (-(-desc.M // 16) * 16)


def flarepp_route_profiled(desc, S, K, V, Y, Qd_out, Z_out, ws, ws_bytes, stream, events, kinds,
                           max_launches, n_launches) -> int:
    """events: ctypes array of 2*max_launches hipEvent_t; kinds: ctypes int32 array;
    n_launches: ctypes.c_int32 (by reference)."""
    return _lib().flarepp_route_profiled(ctypes.byref(desc), S, K, V, Y, Qd_out, Z_out, ws, ws_bytes,
                                         stream, events, kinds, max_launches,
                                         ctypes.byref(n_launches))


# ------------------------------------------------------ torch plumbing -----

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")


def desc_for(S, K, scale) -> FlareppDesc:
    """Descriptor from K (B x H x N x D) and S (M x D or H x M x D)."""
    B, H, N, D = K.shape
    if S.dim() == 2:
        M, shs = S.shape[0], 0
    elif S.dim() == 3 and S.shape[0] == H:
        M = S.shape[1]
        shs = M * D
    else:
        raise ValueError("S must be M x D or H x M x D")
    return make_desc(B, H, N, M, D, _dtype_code(K), scale, shs)


class Workspace:
    """A reusable device workspace (grown on demand, never shrunk)."""

    def __init__(self, device=None):
        self.buf = None
        self.device = device

    def get(self, nbytes: int):
        torch = _torch()
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device or "cuda")
        return self.buf, self.buf.numel()


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def route_sharded(S, K, V, scale, bounds, *, stream=None):
    """(Y, Qd, Z) of the route computed the context-parallel way over the token
    shards [bounds[i], bounds[i+1]): per stage every shard emits its records
    (flarepp_encode_shard), the records of all shards are merged
    (flarepp_merge_shards), and each shard decodes its own tokens.  Here the
    shards run one after another on one device, and the record buffer stands
    in for the exchange between devices."""
    torch = _torch()
    for t, n in ((S, "S"), (K, "K"), (V, "V")):
        _require(t, n)
    B, H, N, D = K.shape
    if bounds[0] != 0 or bounds[-1] != N or any(b1 <= b0 for b0, b1 in zip(bounds, bounds[1:])):
        raise ValueError("bounds must rise strictly from 0 to N")
    ns = len(bounds) - 1
    full = desc_for(S, K, scale)
    M = full.M
    shards = [(K[:, :, b0:b1].contiguous(), V[:, :, b0:b1].contiguous()) for b0, b1 in zip(bounds, bounds[1:])]
    descs = [desc_for(S, k, scale) for k, _ in shards]
    rec = torch.empty(flarepp_shard_records_size(full, ns) // 4, dtype=torch.float32, device=K.device)
    Qd = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    st = _stream(stream)
    for stage, q, out in ((1, S, Qd), (2, Qd, Z)):
        op = OP_SEED_ENCODE if stage == 1 else OP_ENCODE
        for i, ((k, v), d) in enumerate(zip(shards, descs)):
            n = flarepp_workspace_size(d, op)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=K.device)
            _check(flarepp_encode_shard(d, stage, _ptr(q), _ptr(k), _ptr(v), _ptr(rec), i, ns, _ptr(ws), n, st),
                   "flarepp_encode_shard")
        _check(flarepp_merge_shards(full, _ptr(rec), ns, _ptr(out), st), "flarepp_merge_shards")
    Ys = []
    for (k, _), d in zip(shards, descs):
        y = torch.empty(k.shape, dtype=torch.float32, device=K.device)
        n = flarepp_workspace_size(d, OP_DECODE)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=K.device)
        _check(flarepp_decode(d, _ptr(Qd), _ptr(Z), _ptr(k), _ptr(y), _ptr(ws), n, st), "flarepp_decode")
        Ys.append(y)
    return torch.cat(Ys, dim=2), Qd, Z


def route(S, K, V, scale, *, with_intermediates=False, workspace: Workspace | None = None, stream=None,
          out=None, tuning: FlareppTuning | None = None):
    """Y (and optionally Qd, Z) of the full route for GPU tensors S, K, V
    (with explicit launch choices through flarepp_route_tuned if `tuning`)."""
    torch = _torch()
    for t, n in ((S, "S"), (K, "K"), (V, "V")):
        _require(t, n)
    desc = desc_for(S, K, scale)
    B, H, N, D = K.shape
    M = desc.M
    Y = out if out is not None else torch.empty((B, H, N, D), dtype=torch.float32, device=K.device)
    Qd = Z = None
    if with_intermediates:
        Qd = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
        Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    ws = workspace or Workspace(K.device)
    if tuning is None:
        buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_ROUTE))
        _check(flarepp_route(desc, _ptr(S), _ptr(K), _ptr(V), _ptr(Y), _ptr(Qd), _ptr(Z), _ptr(buf),
                             nbytes, _stream(stream)), "flarepp_route")
    else:
        buf, nbytes = ws.get(flarepp_workspace_size_tuned(desc, OP_ROUTE, tuning))
        _check(flarepp_route_tuned(desc, tuning, _ptr(S), _ptr(K), _ptr(V), _ptr(Y), _ptr(Qd), _ptr(Z),
                                   _ptr(buf), nbytes, _stream(stream)), "flarepp_route_tuned")
    return (Y, Qd, Z) if with_intermediates else Y


def route_backward(S, K, V, scale, dY, *, workspace: Workspace | None = None, stream=None):
    """(dS, dK, dV): float32 gradients of <dY, route(S, K, V)>; S, K, V float32 or
    bfloat16 GPU tensors, dY float32."""
    torch = _torch()
    for t, n in ((S, "S"), (K, "K"), (V, "V"), (dY, "dY")):
        _require(t, n)
    if dY.dtype != torch.float32:
        raise TypeError("dY must be float32")
    desc = desc_for(S, K, scale)
    dS = torch.empty_like(S, dtype=torch.float32)
    dK = torch.empty(K.shape, dtype=torch.float32, device=K.device)
    dV = torch.empty(K.shape, dtype=torch.float32, device=K.device)
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_ROUTE_BACKWARD))
    _check(flarepp_route_backward(desc, _ptr(S), _ptr(K), _ptr(V), _ptr(dY), _ptr(dS), _ptr(dK),
                                  _ptr(dV), _ptr(buf), nbytes, _stream(stream)), "flarepp_route_backward")
    return dS, dK, dV


def route_save(S, K, V, scale, *, workspace: Workspace | None = None, stream=None):
    """(Y, saved): the route with the backward's forward stages, and what
    route_backward_saved needs (Qd, Z, the encodes' log-sum-exps); bf16 only."""
    torch = _torch()
    for t, n in ((S, "S"), (K, "K"), (V, "V")):
        _require(t, n)
    desc = desc_for(S, K, scale)
    B, H, N, D = K.shape
    Y = torch.empty((B, H, N, D), dtype=torch.float32, device=K.device)
    Qd = torch.empty((B, H, desc.M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty_like(Qd)
    lse = torch.empty(saved_lse_count(desc), dtype=torch.float32, device=K.device)
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_ROUTE_BACKWARD))
    _check(flarepp_route_save(desc, _ptr(S), _ptr(K), _ptr(V), _ptr(Y), _ptr(Qd), _ptr(Z), _ptr(lse),
                              _ptr(buf), nbytes, _stream(stream)), "flarepp_route_save")
    return Y, (Qd, Z, lse)


def route_backward_saved(S, K, V, scale, saved, dY, *, workspace: Workspace | None = None, stream=None):
    """(dS, dK, dV) as route_backward, from route_save's saved forward."""
    torch = _torch()
    Qd, Z, lse = saved
    for t, n in ((S, "S"), (K, "K"), (V, "V"), (dY, "dY"), (Qd, "Qd"), (Z, "Z"), (lse, "lse")):
        _require(t, n)
    desc = desc_for(S, K, scale)
    dS = torch.empty_like(S, dtype=torch.float32)
    dK = torch.empty(K.shape, dtype=torch.float32, device=K.device)
    dV = torch.empty(K.shape, dtype=torch.float32, device=K.device)
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_ROUTE_BACKWARD))
    _check(flarepp_route_backward_saved(desc, _ptr(S), _ptr(K), _ptr(V), _ptr(Qd), _ptr(Z), _ptr(lse), _ptr(dY),
                                        _ptr(dS), _ptr(dK), _ptr(dV), _ptr(buf), nbytes, _stream(stream)),
           "flarepp_route_backward_saved")
    return dS, dK, dV


def spectrum(S, K, V, scale, *, with_matrix=False, workspace: Workspace | None = None, stream=None):
    """Eigenvalues (B x H x M, decreasing) of each head's W_enc W_dec; with
    with_matrix also the symmetric matrix G similar to it (B x H x M x M)."""
    torch = _torch()
    for t, n in ((S, "S"), (K, "K"), (V, "V")):
        _require(t, n)
    desc = desc_for(S, K, scale)
    B, H, N, D = K.shape
    M = desc.M
    eig = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    G = torch.empty((B, H, M, M), dtype=torch.float32, device=K.device) if with_matrix else None
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_SPECTRUM))
    _check(flarepp_spectrum(desc, _ptr(S), _ptr(K), _ptr(V), _ptr(eig), _ptr(G), _ptr(buf), nbytes,
                            _stream(stream)), "flarepp_spectrum")
    return (eig, G) if with_matrix else eig


def seed_encode(S, K, V, scale, *, workspace: Workspace | None = None, stream=None):
    torch = _torch()
    for t, n in ((S, "S"), (K, "K"), (V, "V")):
        _require(t, n)
    desc = desc_for(S, K, scale)
    B, H, N, D = K.shape
    Qd = torch.empty((B, H, desc.M, D), dtype=torch.float32, device=K.device)
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_SEED_ENCODE))
    _check(flarepp_seed_encode(desc, _ptr(S), _ptr(K), _ptr(V), _ptr(Qd), _ptr(buf), nbytes,
                               _stream(stream)), "flarepp_seed_encode")
    return Qd


def encode(Qd, K, V, scale, *, workspace: Workspace | None = None, stream=None):
    torch = _torch()
    for t, n in ((Qd, "Qd"), (K, "K"), (V, "V")):
        _require(t, n)
    B, H, N, D = K.shape
    desc = make_desc(B, H, N, Qd.shape[2], D, _dtype_code(K), scale, 0)
    Z = torch.empty_like(Qd)
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_ENCODE))
    _check(flarepp_encode(desc, _ptr(Qd), _ptr(K), _ptr(V), _ptr(Z), _ptr(buf), nbytes,
                          _stream(stream)), "flarepp_encode")
    return Z


def decode(Qd, Z, K, scale, *, workspace: Workspace | None = None, stream=None):
    torch = _torch()
    for t, n in ((Qd, "Qd"), (Z, "Z"), (K, "K")):
        _require(t, n)
    B, H, N, D = K.shape
    desc = make_desc(B, H, N, Qd.shape[2], D, _dtype_code(K), scale, 0)
    Y = torch.empty((B, H, N, D), dtype=torch.float32, device=K.device)
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_DECODE))
    _check(flarepp_decode(desc, _ptr(Qd), _ptr(Z), _ptr(K), _ptr(Y), _ptr(buf), nbytes,
                          _stream(stream)), "flarepp_decode")
    return Y


def flare(Q, K, V, scale, *, with_latents=False, workspace: Workspace | None = None, stream=None):
    """Fixed-query FLARE: Y (and optionally Z) with parameter queries Q."""
    torch = _torch()
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _require(t, n)
    desc = desc_for(Q, K, scale)
    B, H, N, D = K.shape
    Y = torch.empty((B, H, N, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, desc.M, D), dtype=torch.float32, device=K.device) if with_latents else None
    ws = workspace or Workspace(K.device)
    buf, nbytes = ws.get(flarepp_workspace_size(desc, OP_FLARE))
    _check(flarepp_flare(desc, _ptr(Q), _ptr(K), _ptr(V), _ptr(Y), _ptr(Z), _ptr(buf), nbytes,
                         _stream(stream)), "flarepp_flare")
    return (Y, Z) if with_latents else Y
