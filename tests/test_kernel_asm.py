"""Checks on the generated gfx950 code of libflarepp (CPU only: hipcc
cross-compiles the device code to assembly; nothing runs on a GPU).

The encode's direct-to-LDS tile loads are issued from an asm statement that
sets M0 (the LDS base) and issues the load.  The compiler reserves M0 and does
not see that write, so the library is only correct while no compiler-generated
instruction relies on M0 keeping a value across such a statement.  These tests
pin that, and that the packed-fp32 VALU forms stay disabled."""
import os
import re
import shutil
import subprocess

import pytest

from rank_latent_attention_seed_amd import build as fbuild

pytestmark = pytest.mark.skipif(not os.path.exists(fbuild.HIPCC), reason="hipcc not available")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "flarepp_gfx950.s"
    flags = [f for f in fbuild.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [fbuild.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), fbuild.SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return [l.split(";")[0].strip() for l in out.read_text().splitlines()]


def _instructions(lines):
    return [l for l in lines if l and not l.startswith((".", "_")) and not l.endswith(":")]


def test_m0_only_feeds_the_tile_loads(device_asm):
    ins = _instructions(device_asm)
    m0_uses = [(i, l) for i, l in enumerate(ins) if re.search(r"\bm0\b", l)]
    assert m0_uses, "expected the tile loads' M0 writes"
    n_dma = 0
    for i, l in m0_uses:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"unexpected M0 use: {l}"
        assert ins[i + 1].startswith("global_load_lds_dwordx4"), f"M0 write not followed by a tile load: {l}"
        n_dma += 1
    # and every tile load takes its M0 from the write just before it
    loads = [i for i, l in enumerate(ins) if l.startswith("global_load_lds")]
    assert len(loads) == n_dma
    assert all(re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 1]) for i in loads)


def test_no_packed_fp32_valu(device_asm):
    ins = _instructions(device_asm)
    bad = [l for l in ins if re.match(r"v_pk_(add|mul|fma|mov)_f32", l)]
    assert not bad, bad[:5]
