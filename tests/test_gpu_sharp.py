"""GPU parity under sharp softmaxes, at sizes where every encode split spans
many tiles.

The named workloads route through broad softmaxes (every weight small, the
running max settled after the first step), so they leave three parts of the
split-N encode untested against the oracle: the per-tile decision whether a
tile's scores must be checked against the running max, raising that max in
the middle of a split (with the rescale of the accumulators), and the route's
fallback from the bound shift to the running max in its second encode.  The
cases here reach them: iid keys at scale 1 (support of a few tokens), and keys
whose norms grow along the token axis so that a split's largest scores arrive
late.  Every call writes into NaN-poisoned outputs and workspace.

The oracle is the definition (three SDPA calls in fp64, the encode softmaxes
over the tokens, the decode softmax over the latents: FLARE summary,
"Основной механизм FLARE" and "Матрица коммуникации низкого ранга"; the seed
encode of the FLARE++ abstract)."""
import numpy as np
import pytest

from rank_latent_attention_seed_amd import inputs
from gpu_util import all_heads, compare_route, errors, oracle_heads, route_poisoned, to_device

pytestmark = pytest.mark.gpu

_REF = {}


@pytest.fixture(scope="module")
def fp():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rank_latent_attention_seed_amd import flarepp

    flarepp.library()
    return flarepp


def _problem(key, **kw):
    """Draw a problem and its oracle once per module (several split counts share it)."""
    if key not in _REF:
        p = inputs.random_problem(**kw)
        _REF[key] = (p, oracle_heads(p.S, p.K, p.V, p.scale, all_heads(p.B, p.H)))
    return _REF[key]


def _run(fp, p, ref, splits, label):
    print(f"\n  case {label}: B{p.B} H{p.H} N{p.N} M{p.M} D{p.D} s={p.scale:g} splits={splits or 'default'}",
          flush=True)
    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    tuning = fp.make_tuning(splits=splits) if splits else None
    Y, Qd, Z = route_poisoned(fp, S, K, V, p.scale, tuning)
    return compare_route(p, Y, Qd, Z, ref=ref)[1]


@pytest.mark.parametrize("M", [64, 256])
@pytest.mark.parametrize("splits", [1, 4, 0])
def test_iid_scale_one_many_tiles(fp, M, splits):
    """iid N(0, 1) keys, values and seeds, s = 1, N = 65536: with one split the
    seed encode's running max lives through 256 tiles of 256 tokens."""
    p, ref = _problem(("iid", M), B=1, H=1, N=65536, M=M, D=32, dtype="bf16", scale=1.0, seed=100 + M)
    _run(fp, p, ref, splits, f"iid s=1 M{M}")


@pytest.mark.parametrize("splits", [1, 0])
def test_stress_recipe_long(fp, splits):
    """The stress recipe (iid N(0, 1), M = 128, s = 1) at N = 2^18."""
    p, ref = _problem("stress18", B=1, H=2, N=1 << 18, M=128, D=32, dtype="bf16", scale=1.0, seed=618)
    _run(fp, p, ref, splits, "stress N=2^18")


@pytest.mark.parametrize("M", [64, 256])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_rising_key_norms(fp, M, splits):
    """Key rows scaled by a ramp from 0.25 to 3 along the tokens (s = 1/2):
    the first tiles' scores are small, later ones exceed the running max by
    far more than its slack, so the seed encode switches from skipping the
    per-step check to checking and raises its max mid-split, many times; the
    largest key norms make the second encode's bound unsafe for most latents
    (the bound-to-running-max fallback) and the decode take exact maxima."""
    p, ref = _problem(("ramp", M), B=1, H=2, N=65536, M=M, D=32, dtype="bf16", scale=0.5, seed=200 + M,
                      k_ramp=(0.25, 3.0))
    _run(fp, p, ref, splits, f"rising key norms M{M}")


def test_falling_key_norms(fp):
    """The same ramp reversed: the first step of each split sets a high
    running max that is never raised; weights of later tiles underflow."""
    p, ref = _problem("fall", B=1, H=1, N=65536, M=128, D=32, dtype="bf16", scale=0.5, seed=301,
                      k_ramp=(3.0, 0.25))
    _run(fp, p, ref, 1, "falling key norms")


@pytest.mark.parametrize("scale", [-1.0, -0.5])
def test_negative_scale_many_tiles(fp, scale):
    """s < 0: every bound and shift is taken with |s| (a signed bound would sit
    below the scores and overflow the exponentials)."""
    p, ref = _problem(("neg", scale), B=1, H=2, N=20000, M=256, D=32, dtype="bf16", scale=scale, seed=401)
    _run(fp, p, ref, 0, f"negative scale {scale}")


@pytest.mark.parametrize("N,splits", [(4096, 0), (4096, 1), (16384, 0), (16384, 1)])
def test_fp16_weight_overflow_is_recomputed(fp, N, splits):
    """Keys aligned with a seed arrive after small keys set the running max,
    in tiles that skip the per-step check: their fp16 weights overflow
    (tests/test_spike_inputs.py shows the inputs do), and the merge recomputes
    those records.  N = 4096 merges 32 splits per row (merge_partials), N =
    16384 128 (merge_rows256); splits=1 is one split per head."""
    from spike_inputs import spike_problem

    spikes = [(300, 0), (2000, 5)] + ([(9000, 9)] if N > 9000 else [])
    p = spike_problem(N, spikes, H=2)
    ref = oracle_heads(p.S, p.K, p.V, p.scale, all_heads(p.B, p.H))
    _run(fp, p, ref, splits, f"fp16 overflow N{N}")


def test_fp16_weight_overflow_in_the_stand_alone_seed_encode(fp):
    import torch
    from spike_inputs import spike_problem
    from gpu_util import poisoned

    p = spike_problem(4096, [(300, 0), (2000, 5)])
    print("\n  case fp16 overflow, flarepp_seed_encode", flush=True)
    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    d = fp.desc_for(S, K, p.scale)
    n = fp.flarepp_workspace_size(d, fp.OP_SEED_ENCODE)
    ws = poisoned((n,), torch.uint8)
    Qd = poisoned((1, 1, p.M, p.D))
    assert fp.flarepp_seed_encode(d, S.data_ptr(), K.data_ptr(), V.data_ptr(), Qd.data_ptr(), ws.data_ptr(), n,
                                  fp._stream(None)) == 0
    torch.cuda.synchronize()
    ref = oracle_heads(p.S, p.K, p.V, p.scale, [(0, 0)])[0][0]
    from gpu_util import assert_close
    assert_close("Qd", Qd.cpu().numpy()[0, 0], ref, "bf16")
