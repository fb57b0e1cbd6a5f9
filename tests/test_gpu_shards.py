"""GPU parity of the token-shard path (flarepp_encode_shard +
flarepp_merge_shards + per-shard flarepp_decode): the route computed over
token shards, run one after another on one device with the record buffer
standing in for the exchange between devices, against the oracle and
against the unsharded calls."""
import numpy as np
import pytest

from rank_latent_attention_seed_amd import inputs
from gpu_util import compare_route, poisoned, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rank_latent_attention_seed_amd import flarepp

    flarepp.library()
    return flarepp


CASES = [
    # B, H, N, M, D, dtype, scale, per-head seeds, shard bounds
    (2, 2, 3001, 48, 32, "bf16", 1 / np.sqrt(32), False, (0, 700, 1701, 3001)),
    (1, 3, 5000, 256, 32, "bf16", 1 / np.sqrt(32), True, (0, 1250, 2500, 3750, 5000)),
    (1, 2, 2048, 33, 16, "bf16", 1.0, False, (0, 1, 1000, 2048)),
    (2, 1, 1500, 20, 16, "f32", 0.25, False, (0, 512, 1500)),
    (1, 2, 999, 100, 32, "f32", -0.5, True, (0, 333, 666, 999)),
]


@pytest.mark.parametrize("B,H,N,M,D,dtype,scale,per_head,bounds", CASES)
def test_sharded_route_matches_oracle(fp, B, H, N, M, D, dtype, scale, per_head, bounds):
    import torch

    p = inputs.random_problem(B, H, N, M, D, dtype=dtype, scale=scale, seed=N + M + 7, per_head_seeds=per_head)
    print(f"\n  case shards {list(bounds)}: B{B} H{H} N{N} M{M} D{D} {dtype} s={scale:g}", flush=True)
    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    Y, Qd, Z = fp.route_sharded(S, K, V, p.scale, list(bounds))
    torch.cuda.synchronize()
    compare_route(p, Y, Qd, Z)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_shard_equals_the_stage_calls(fp, dtype):
    """One shard: merging its records reproduces flarepp_seed_encode and
    flarepp_encode. The record merge rescales by exp(0) = 1 exactly, so the
    bf16 routes agree bit for bit; the float32 merge kernel normalises with a
    different product order than the record merge, which moves a few outputs
    by one unit in the last place, so there the bar is two ulp."""
    import torch

    p = inputs.random_problem(1, 2, 2500, 64, 32, dtype=dtype, seed=11)
    print(f"\n  case single shard {dtype}", flush=True)
    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    desc = fp.desc_for(S, K, p.scale)
    st = fp._stream(None)
    B, H, N, D = K.shape
    M = desc.M

    def ws_for(op):
        n = fp.flarepp_workspace_size(desc, op)
        return poisoned((max(n, 1),), torch.uint8), n

    rec = poisoned((fp.flarepp_shard_records_size(desc, 1) // 4,))
    for stage, op, q in ((1, fp.OP_SEED_ENCODE, S), (2, fp.OP_ENCODE, None)):
        if stage == 2:
            q = ref
        ws, n = ws_for(op)
        assert fp.flarepp_encode_shard(desc, stage, q.data_ptr(), K.data_ptr(), V.data_ptr(), rec.data_ptr(), 0, 1,
                                       ws.data_ptr(), n, st) == 0
        got = poisoned((B, H, M, D))
        assert fp.flarepp_merge_shards(desc, rec.data_ptr(), 1, got.data_ptr(), st) == 0
        ref = poisoned((B, H, M, D))
        ws2, n2 = ws_for(op)
        call = fp.flarepp_seed_encode if stage == 1 else fp.flarepp_encode
        assert call(desc, q.data_ptr(), K.data_ptr(), V.data_ptr(), ref.data_ptr(), ws2.data_ptr(), n2, st) == 0
        torch.cuda.synchronize()
        if dtype == "bf16":
            assert torch.equal(got, ref), f"stage {stage}: merged shard records differ from the stage call"
        else:
            ulp = torch.finfo(torch.float32).eps * ref.abs().clamp_min(torch.finfo(torch.float32).tiny)
            err = ((got - ref).abs() / ulp).max().item()
            assert err <= 2.0, f"stage {stage}: merged shard records differ from the stage call by {err:.1f} ulp"


def test_shard_slots_write_only_their_slot(fp):
    """A shard call writes its own slot of every record and nothing else."""
    import torch

    p = inputs.random_problem(1, 2, 1200, 40, 16, dtype="bf16", seed=12)
    S, K, V = to_device(p.S), to_device(p.K), to_device(p.V)
    desc = fp.desc_for(S, K, p.scale)
    n = fp.flarepp_workspace_size(desc, fp.OP_SEED_ENCODE)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    rec = torch.full((fp.flarepp_shard_records_size(desc, 3) // 4,), 7.5, device="cuda")
    assert fp.flarepp_encode_shard(desc, 1, S.data_ptr(), K.data_ptr(), V.data_ptr(), rec.data_ptr(), 1, 3,
                                   ws.data_ptr(), n, fp._stream(None)) == 0
    torch.cuda.synchronize()
    r = rec.view(p.B * p.H, -1, 3, p.D + 4).cpu()
    assert torch.all(r[:, :, 0] == 7.5) and torch.all(r[:, :, 2] == 7.5)
    assert torch.all(torch.isfinite(r[:, :, 1, : p.D + 2]))
