"""Seeded input generators: reproducible bytes, shapes, and bf16 rounding."""
import numpy as np
import pytest
import torch

from rank_latent_attention_seed_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0,
        # exact ties between two bf16 neighbours: mantissa low half = 0x8000
        ((rng.integers(0, 1 << 8, 1000, dtype=np.uint32) << 16) | np.uint32(0x3F008000)
         | (rng.integers(0, 2, 1000, dtype=np.uint32) << 31)).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -3e38, 65504.0], dtype=np.float32),
    ])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", ["tiny", "mesh", "stress"])
def test_problem_is_reproducible(name):
    a = inputs.make_problem(name)
    b = inputs.make_problem(name)
    for x, y in ((a.S, b.S), (a.K, b.K), (a.V, b.V)):
        assert x.dtype == y.dtype and np.array_equal(x, y)


@pytest.mark.parametrize("name,shape,M,dtype", [
    ("tiny", (1, 4, 1024, 16), 32, np.float32),
    ("mesh", (8, 8, 7225, 16), 64, np.uint16),
    ("cloud", (4, 8, 11271, 32), 128, np.uint16),
    ("stress", (1, 2, 4096, 32), 128, np.uint16),
])
def test_problem_shapes(name, shape, M, dtype):
    p = inputs.make_problem(name)
    assert p.K.shape == shape and p.V.shape == shape
    assert p.S.shape == (M, shape[-1])
    assert p.K.dtype == dtype and p.S.dtype == dtype
    vals = inputs.bf16_bits_to_f32(p.K) if dtype == np.uint16 else p.K
    assert np.isfinite(vals).all()


def test_mesh_structure():
    p = inputs.make_problem("mesh")
    assert p.N == 85 * 85 and abs(p.scale - 0.25) < 1e-15
    # three input features -> per-head K spans at most 3 dimensions (up to bf16 rounding)
    k = inputs.bf16_bits_to_f32(p.K[0, 0]).astype(np.float64)
    sv = np.linalg.svd(k, compute_uv=False)
    assert sv[3] / sv[0] < 1e-2


def test_random_problem_per_head_seeds():
    p = inputs.random_problem(2, 3, 17, 5, 16, dtype="bf16", per_head_seeds=True, seed=4)
    assert p.S.shape == (3, 5, 16) and p.K.shape == (2, 3, 17, 16)
    q = inputs.random_problem(1, 1, 9, 2, 32, dtype="f32", seed=1)
    assert q.K.dtype == np.float32
