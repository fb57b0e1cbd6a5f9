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


def test_no_waterfall_loops(device_asm):
    """A buffer resource built from a value the compiler cannot prove
    wave-uniform (a wave index taken as threadIdx.x / 64 without
    readfirstlane, say) is lowered to a loop that peels one distinct value per
    iteration around every buffer access (readfirstlane, compare, exec mask,
    s_cbranch_execnz back).  Such loops cost a dozen instructions per access
    even when the value is uniform; none may appear in the library."""
    labels = {l[:-1]: i for i, l in enumerate(device_asm) if re.fullmatch(r"\.LBB\w+:", l)}
    loops = []
    for i, l in enumerate(device_asm):
        m = re.fullmatch(r"s_cbranch_execnz (\.LBB\w+)", l)
        if not m or m.group(1) not in labels or labels[m.group(1)] >= i:
            continue
        body = device_asm[labels[m.group(1)]:i]
        if any(x.startswith("v_readfirstlane_b32") for x in body) and \
                any(x.startswith(("buffer_load", "buffer_store")) for x in body):
            loops.append(m.group(1))
    assert not loops, f"{len(loops)} waterfall loops, e.g. at {loops[:3]}"


def test_no_register_spills(device_asm):
    """No kernel spills registers to scratch.  The split-N encode is compiled
    for four waves per SIMD (at most 128 VGPRs), the occupancy its speed
    depends on; a change that no longer fits shows up here as scratch use
    rather than as a silent slowdown."""
    kernels = [l.split()[1] for l in device_asm if l.startswith(".amdhsa_kernel ")]
    sizes = [int(l.split()[1]) for l in device_asm if l.startswith(".amdhsa_private_segment_fixed_size")]
    assert kernels and len(kernels) == len(sizes)
    spilled = [k for k, n in zip(kernels, sizes) if n != 0]
    assert not spilled, f"{len(spilled)} kernels use scratch, e.g. {spilled[:3]}"


def test_encode_fits_four_waves_per_simd(device_asm):
    """The eight-wave encode instantiations stay within 128 VGPRs (two
    workgroups per CU)."""
    name = None
    seen, over = 0, []
    for l in device_asm:
        if l.startswith(".amdhsa_kernel "):
            name = l.split()[1]
        elif l.startswith(".amdhsa_next_free_vgpr") and name and re.search(r"encode_split_bf16ILi(16|32)ELi8E", name):
            seen += 1
            if int(l.split()[1]) > 128:
                over.append(name)
    assert seen >= 6, seen
    assert not over, over[:3]


def test_16bit_denormals_kept(device_asm):
    # the fp16 logit products take keys and c * Qd down to fp16's subnormal
    # range; their error bound assumes that nothing there flushes to zero
    modes = [l.split()[1] for l in device_asm if l.startswith(".amdhsa_float_denorm_mode_16_64")]
    assert modes, "expected kernel descriptors"
    assert set(modes) == {"3"}, f"16/64-bit denormal modes {sorted(set(modes))}"


def test_fp16_logit_forms_present(device_asm):
    # the route's stage-2 encode and paired decode carry the single fp16
    # logit product (v_mfma_f32_16x16x32_f16 on the key operand)
    assert any(l.startswith("v_mfma_f32_16x16x32_f16") for l in device_asm)
    names = [l[:-1] for l in device_asm if l.endswith(":") and "decode_pair_bf16" in l and not l.startswith(".")]
    assert any("Lb1EEEvNS_10DecodeArgsE" in n for n in names), "no fp16-logit paired decode"
