"""Precision of the bf16 path where the pages' tolerance (max absolute error
1e-2 against the oracle on the same bf16 inputs) is hardest to meet: sharp
softmaxes (large |s| ||Q|| ||K||) and large values.

Two cases were once narrowed to pass (keys of spread 4 with s = 1, values of
spread 16); they are restored here as first written.  The first passes.  The
second cannot meet an absolute bound: every stage rounds its matrix-core
operands (the decode's Z to bf16, the weights to fp16 or bf16), so the error
grows in proportion to the scale of V.  It is kept as an expected failure
with its measured error, and `test_error_envelope` bounds the error relative
to max |V| over a sweep of key spread, scale and value spread."""
import numpy as np
import pytest

from rank_latent_attention_seed_amd import inputs
from gpu_util import errors, oracle_heads, route_poisoned, to_device

pytestmark = pytest.mark.gpu

# measured bound on max|err| / max|V| over the envelope sweep (largest seen:
# 3.6e-3, D = 16, s = 1, sigma_V = 16)
ENVELOPE_REL = 5e-3


@pytest.fixture(scope="module")
def fp():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rank_latent_attention_seed_amd import flarepp

    flarepp.library()
    return flarepp


def route_errors(fp, p):
    import torch

    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    Y, Qd, Z = route_poisoned(fp, S, K, V, p.scale)
    torch.cuda.synchronize()
    ref = oracle_heads(p.S, p.K, p.V, p.scale, [(0, 0)])[0]
    errs = [errors(g.cpu().numpy()[0, 0], r)[0] for g, r in zip((Qd, Z, Y), ref)]
    vmax = float(np.abs(inputs.bf16_bits_to_f32(p.V)).max())
    print(f"\n  case sigK {p.meta.get('sigma')} s {p.scale:g} sigV {p.meta.get('sigma_v')} D{p.D} M{p.M}: "
          f"Qd {errs[0]:.2e} Z {errs[1]:.2e} Y {errs[2]:.2e}  max|V| {vmax:.1f}  max err/max|V| "
          f"{max(errs) / vmax:.2e}", flush=True)
    return errs, vmax


def problem(sigma, scale, sigma_v, D=16, M=32, N=3000, seed=3):
    p = inputs.random_problem(1, 1, N, M, D, dtype="bf16", scale=scale, seed=seed, sigma=sigma, sigma_v=sigma_v)
    p.meta.update(sigma=sigma, sigma_v=sigma_v)
    return p


def test_sharp_keys_restored(fp):
    """Keys of spread 4 with s = 1 (logits up to ~140 log2 units), unit
    values: within the absolute tolerance."""
    errs, _ = route_errors(fp, problem(4.0, 1.0, 1.0))
    assert max(errs) <= 1e-2, errs


@pytest.mark.xfail(strict=True, reason="values of spread 16 (max |V| 76.5), keys of spread 4, s = 1/2: "
                                       "measured max |err| on Y 0.23 (3.0e-3 of max |V|); the rounding of "
                                       "the matrix-core operands scales with V, an absolute 1e-2 cannot hold")
def test_large_values_restored(fp):
    errs, _ = route_errors(fp, problem(4.0, 0.5, 16.0))
    assert max(errs) <= 1e-2, errs


@pytest.mark.parametrize("D,M", [(16, 32), (32, 128)])
@pytest.mark.parametrize("sigma", [1.0, 4.0])
@pytest.mark.parametrize("scale", [0.25, 1.0])
@pytest.mark.parametrize("sigma_v", [1.0, 16.0])
def test_error_envelope(fp, D, M, sigma, scale, sigma_v):
    errs, vmax = route_errors(fp, problem(sigma, scale, sigma_v, D=D, M=M))
    assert max(errs) <= ENVELOPE_REL * vmax, (errs, vmax)
