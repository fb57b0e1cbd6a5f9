"""libflarepp's C ABI on the host: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments with the
documented status codes before touching the GPU (no compute call here
reaches a kernel launch, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from rank_latent_attention_seed_amd import flarepp as fp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flarepp.h")

OK, INVALID_ARG, UNSUPPORTED, WS_SMALL, ALIASING, SCRATCH_LIMIT = 0, 1, 2, 3, 4, 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flarepp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = fp.library()
    names = declared_functions()
    assert set(names) == set(fp.SYMBOLS), names
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_strings():
    assert fp.flarepp_abi_version() == fp.ABI_VERSION
    for code in range(7):
        assert isinstance(fp.flarepp_status_string(code), str)
    assert fp.flarepp_status_string(99) == "unknown status"


def desc(**kw):
    d = dict(B=2, H=3, N=1000, M=64, D=32, dtype=fp.BF16, scale=0.25, seed_head_stride=0)
    d.update(kw)
    return fp.make_desc(**d)


def ws_status(d, op):
    n = ctypes.c_size_t(0)
    return fp.library().flarepp_workspace_size(ctypes.byref(d), op, ctypes.byref(n)), n.value


@pytest.mark.parametrize("op", range(5))
def test_workspace_sizes(op):  # forward ops (the backward: test_backward_validation)
    st, n_bf16 = ws_status(desc(), op)
    assert st == OK
    st, n_f32 = ws_status(desc(dtype=fp.F32), op)
    assert st == OK
    if op == fp.OP_DECODE:
        assert n_f32 == 0 and n_bf16 > 0
    else:
        assert n_f32 > 0 and n_bf16 > 0
    # partial records grow with the latent count
    assert ws_status(desc(M=256), op)[1] >= n_bf16


def test_workspace_size_rejects():
    assert ws_status(desc(D=24), fp.OP_ROUTE)[0] == UNSUPPORTED
    assert ws_status(desc(M=257), fp.OP_ROUTE)[0] == UNSUPPORTED
    assert ws_status(desc(dtype=7), fp.OP_ROUTE)[0] == UNSUPPORTED
    assert ws_status(desc(N=0), fp.OP_ROUTE)[0] == INVALID_ARG
    assert ws_status(desc(scale=float("nan")), fp.OP_ROUTE)[0] == INVALID_ARG
    assert ws_status(desc(seed_head_stride=5), fp.OP_ROUTE)[0] == INVALID_ARG
    assert ws_status(desc(), 9)[0] == INVALID_ARG
    assert ws_status(desc(seed_head_stride=64 * 32), fp.OP_ROUTE)[0] == OK
    n = ctypes.c_size_t(0)
    assert fp.library().flarepp_workspace_size(None, 0, ctypes.byref(n)) == INVALID_ARG


# Fake, never-dereferenced device addresses: every call below fails
# validation on the host and returns before any HIP call.
A = 1 << 40


def addr(i):
    return A + i * (1 << 34)


def route(d, S=addr(0), K=addr(1), V=addr(2), Y=addr(3), Qd=addr(4), Z=addr(5), ws=addr(6), nbytes=None):
    if nbytes is None:
        nbytes = ws_status(d, fp.OP_ROUTE)[1]
    return fp.flarepp_route(d, S, K, V, Y, Qd, Z, ws, nbytes, None)


def test_route_validation():
    d = desc()
    assert route(d, S=None) == INVALID_ARG
    assert route(d, K=None) == INVALID_ARG
    assert route(d, Y=None) == INVALID_ARG
    assert route(d, K=addr(1) + 2) == INVALID_ARG        # misaligned
    assert route(d, ws=None) == INVALID_ARG
    assert route(d, nbytes=16) == WS_SMALL
    assert route(d, Y=addr(1) + 64) == ALIASING           # output inside K
    assert route(d, Qd=addr(3) + 16) == ALIASING          # two outputs overlap
    assert route(d, Z=addr(6)) == ALIASING                # output inside the workspace
    assert route(desc(D=64)) == UNSUPPORTED
    assert route(desc(M=0)) == INVALID_ARG


def test_stage_validation():
    d = desc()
    n = ws_status(d, fp.OP_SEED_ENCODE)[1]
    assert fp.flarepp_seed_encode(d, addr(0), addr(1), addr(2), None, addr(6), n, None) == INVALID_ARG
    n = ws_status(d, fp.OP_ENCODE)[1]
    assert fp.flarepp_encode(d, addr(0), addr(1), addr(2), addr(0), addr(6), n, None) == ALIASING
    n = ws_status(d, fp.OP_DECODE)[1]
    assert fp.flarepp_decode(d, addr(0), addr(1), addr(2), addr(3), addr(6), n - 1, None) == WS_SMALL
    n = ws_status(d, fp.OP_FLARE)[1]
    assert fp.flarepp_flare(d, addr(0), None, addr(2), addr(3), None, addr(6), n, None) == INVALID_ARG
    assert fp.library().flarepp_route(None, addr(0), addr(1), addr(2), addr(3), None, None, addr(6),
                                      1 << 30, None) == INVALID_ARG


@pytest.mark.parametrize("dt", [fp.F32, fp.BF16])
def test_backward_validation(dt):
    d = desc(dtype=dt)
    st, n = ws_status(d, fp.OP_ROUTE_BACKWARD)
    assert st == OK and n > 0
    assert ws_status(desc(dtype=dt, M=257), fp.OP_ROUTE_BACKWARD)[0] == UNSUPPORTED

    def bwd(dd=d, S=addr(0), K=addr(1), V=addr(2), dY=addr(3), dS=addr(4), dK=addr(5), dV=addr(7),
            ws=addr(6), nbytes=n):
        return fp.flarepp_route_backward(dd, S, K, V, dY, dS, dK, dV, ws, nbytes, None)

    # every case fails validation on the host, before any HIP call
    assert bwd(dd=desc(dtype=dt, D=24)) == UNSUPPORTED
    assert bwd(dS=None) == INVALID_ARG
    assert bwd(dY=None) == INVALID_ARG
    assert bwd(dV=addr(7) + 4) == INVALID_ARG      # misaligned
    assert bwd(nbytes=n - 1) == WS_SMALL
    assert bwd(dK=addr(2) + 256) == ALIASING       # output inside V
    assert bwd(dV=addr(5) + 16) == ALIASING        # two outputs overlap
    assert bwd(dS=addr(6)) == ALIASING             # output inside the workspace


def test_saved_forward_validation():
    d = desc()
    n = ws_status(d, fp.OP_ROUTE_BACKWARD)[1]
    assert fp.saved_lse_count(d) == 2 * 2 * 3 * 64
    assert fp.saved_lse_count(desc(M=17)) == 2 * 2 * 3 * 32

    def save(dd=d, Y=addr(3), Qd=addr(4), Z=addr(5), lse=addr(7), ws=addr(6), nbytes=n):
        return fp.flarepp_route_save(dd, addr(0), addr(1), addr(2), Y, Qd, Z, lse, ws, nbytes, None)

    def bwd(dd=d, Qd=addr(3), Z=addr(4), lse=addr(5), dS=addr(7), dK=addr(8), dV=addr(9), ws=addr(6), nbytes=n):
        return fp.flarepp_route_backward_saved(dd, addr(0), addr(1), addr(2), Qd, Z, lse, addr(10), dS, dK, dV, ws,
                                               nbytes, None)

    # every case fails validation on the host, before any HIP call
    for call in (save, bwd):
        assert call(dd=desc(dtype=fp.F32)) == UNSUPPORTED
        assert call(dd=desc(M=257)) == UNSUPPORTED
        assert call(nbytes=n - 1) == WS_SMALL
    assert save(lse=None) == INVALID_ARG
    assert save(Qd=None) == INVALID_ARG
    assert save(Z=addr(5) + 4) == INVALID_ARG           # misaligned
    assert save(lse=addr(2) + 256) == ALIASING          # output inside V
    assert save(Z=addr(4) + 64) == ALIASING             # two outputs overlap
    assert bwd(lse=None) == INVALID_ARG
    assert bwd(dK=addr(3) + 128) == ALIASING            # output inside the saved Qd
    assert bwd(dS=addr(5) + 16) == ALIASING             # output inside the saved log-sum-exps
    assert bwd(dV=addr(6)) == ALIASING                  # output inside the workspace


def test_shard_validation():
    lib = fp.library()
    d = desc()
    n = ctypes.c_size_t(0)
    assert lib.flarepp_shard_records_size(ctypes.byref(d), 3, ctypes.byref(n)) == OK
    assert n.value == 2 * 3 * 64 * 3 * (32 + 4) * 4  # B H Mp slots (D + 4) floats
    assert lib.flarepp_shard_records_size(ctypes.byref(d), 0, ctypes.byref(n)) == INVALID_ARG
    assert lib.flarepp_shard_records_size(ctypes.byref(desc(M=17)), 1, ctypes.byref(n)) == OK
    assert n.value == 2 * 3 * 32 * (32 + 4) * 4  # Mp = 32
    nws = ws_status(d, fp.OP_SEED_ENCODE)[1]

    def shard(stage=1, slot=0, nslots=2, rec=addr(4), nbytes=nws, dd=d):
        return fp.flarepp_encode_shard(dd, stage, addr(0), addr(1), addr(2), rec, slot, nslots, addr(6), nbytes, None)

    # every case fails validation on the host, before any HIP call
    assert shard(stage=3) == INVALID_ARG
    assert shard(slot=2) == INVALID_ARG
    assert shard(slot=-1) == INVALID_ARG
    assert shard(nslots=0) == INVALID_ARG
    assert shard(rec=None) == INVALID_ARG
    assert shard(rec=addr(4) + 8) == INVALID_ARG    # misaligned
    assert shard(nbytes=nws - 1) == WS_SMALL
    assert shard(rec=addr(1) + 256) == ALIASING     # records inside K
    assert shard(dd=desc(D=24)) == UNSUPPORTED
    assert fp.flarepp_merge_shards(d, addr(4), 0, addr(5), None) == INVALID_ARG
    assert fp.flarepp_merge_shards(d, addr(4), 2, None, None) == INVALID_ARG
    assert fp.flarepp_merge_shards(d, addr(4), 2, addr(4) + 64, None) == ALIASING


def test_spectrum_validation():
    for dt in (fp.BF16, fp.F32):
        st, n = ws_status(desc(dtype=dt), fp.OP_SPECTRUM)
        assert st == OK and n > 0
    d = desc()
    n = ws_status(d, fp.OP_SPECTRUM)[1]

    def spec(eig=addr(4), sym=addr(5), ws=addr(6), nbytes=n, K=addr(1)):
        return fp.flarepp_spectrum(d, addr(0), K, addr(2), eig, sym, ws, nbytes, None)

    # every case fails validation on the host, before any HIP call
    assert spec(eig=None) == INVALID_ARG
    assert spec(K=None) == INVALID_ARG
    assert spec(nbytes=n - 1) == WS_SMALL
    assert spec(eig=addr(1) + 64) == ALIASING        # output inside K
    assert spec(sym=addr(4) + 16) == ALIASING        # outputs overlap


def test_tuning_validation_and_sizes():
    """Explicit launch choices: a null tuning (or all-zero fields) is the
    library's own plan, split counts change the partial-record workspace, and
    bad fields are rejected before any HIP call."""
    d = desc(N=100000, M=256)
    lib = fp.library()
    n_default = ws_status(d, fp.OP_ROUTE)[1]
    assert fp.flarepp_workspace_size_tuned(d, fp.OP_ROUTE, None) == n_default
    assert fp.flarepp_workspace_size_tuned(d, fp.OP_ROUTE, fp.make_tuning()) == n_default
    n1 = fp.flarepp_workspace_size_tuned(d, fp.OP_ROUTE, fp.make_tuning(splits=1))
    n4 = fp.flarepp_workspace_size_tuned(d, fp.OP_ROUTE, fp.make_tuning(splits=4))
    assert n1 < n4 < n_default
    # more splits than tiles: clamped (a split is at least one 256-token tile)
    big = fp.flarepp_workspace_size_tuned(d, fp.OP_ROUTE, fp.make_tuning(splits=1 << 20))
    assert big == fp.flarepp_workspace_size_tuned(d, fp.OP_ROUTE, fp.make_tuning(splits=391))
    n = ctypes.c_size_t(0)
    for bad in (fp.make_tuning(splits=-1), fp.make_tuning(head_group=-2), fp.make_tuning(decode_kernel=3),
                fp.make_tuning(decode_wg_per_cu=65)):
        assert lib.flarepp_workspace_size_tuned(ctypes.byref(d), fp.OP_ROUTE, ctypes.byref(bad),
                                                ctypes.byref(n)) == INVALID_ARG
        assert fp.flarepp_route_tuned(d, bad, addr(0), addr(1), addr(2), addr(3), None, None, addr(6),
                                      1 << 30, None) == INVALID_ARG
    # the tuned route validates like the plain one
    t = fp.make_tuning(splits=4)
    assert fp.flarepp_route_tuned(d, t, addr(0), addr(1), addr(2), addr(3), None, None, addr(6), n4 - 1,
                                  None) == WS_SMALL
    assert fp.flarepp_route_tuned(d, t, addr(0), addr(1), addr(2), addr(1) + 64, None, None, addr(6), n4,
                                  None) == ALIASING


def test_plan_ignores_the_environment(monkeypatch):
    """The workspace (and with it the split count) depends on the descriptor
    only: variables that once tuned the plan have no effect."""
    d = desc(N=100000, M=256)
    n = ws_status(d, fp.OP_ROUTE)[1]
    for var in ("FLAREPP_SPLITS", "FLAREPP_HEAD_GROUP", "FLAREPP_DECODE_PAIR", "FLAREPP_DECODE_WG_PER_CU"):
        monkeypatch.setenv(var, "3")
    assert ws_status(d, fp.OP_ROUTE)[1] == n


def test_negative_scale_is_accepted():
    """A negative scale is a valid descriptor (the bounds use |s|)."""
    assert ws_status(desc(scale=-1.0), fp.OP_ROUTE)[0] == OK


def test_noalloc_validation():
    """The allocation-free route validates like flarepp_route and refuses, on
    the host, problems whose workspace exceeds its built-in scratch."""
    assert fp.flarepp_noalloc_scratch_bytes() == 64 << 20
    d = desc()
    assert fp.flarepp_route_noalloc(d, addr(0), addr(1), addr(2), None, None, None, None) == INVALID_ARG
    assert fp.flarepp_route_noalloc(d, addr(0), None, addr(2), addr(3), None, None, None) == INVALID_ARG
    assert fp.flarepp_route_noalloc(d, addr(0), addr(1), addr(2), addr(1) + 64, None, None, None) == ALIASING
    assert fp.flarepp_route_noalloc(desc(D=24), addr(0), addr(1), addr(2), addr(3), None, None, None) == UNSUPPORTED
    big = fp.make_desc(64, 64, 4096, 256, 32, fp.BF16, 0.2, 0)  # needs 344 MiB of workspace
    assert fp.flarepp_workspace_size(big, fp.OP_ROUTE) > fp.flarepp_noalloc_scratch_bytes()
    assert fp.flarepp_route_noalloc(big, addr(0), addr(1), addr(2), addr(3), None, None, None) == SCRATCH_LIMIT
