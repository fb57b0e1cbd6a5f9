"""Inputs that drive the fp16 weights of an encode past their range in a tile
whose steps skip the running-max check.

The encodes with a running max form P V in fp16.  A tile skips the per-step
comparison with the running max when the Cauchy-Schwarz bound |c| ||Q_m||
max ||K_n|| of its scores is within 32 binades of the max.  A key aligned
with one seed, arriving after small keys have set the max, can score more
than 16 binades above it while the tile still passes that rule: the fp16
weight overflows, and the merge recomputes the split's record
(refit_record).  `overflowing_tiles` models that rule on the CPU so a test can
show its input reaches the path."""
import numpy as np

from rank_latent_attention_seed_amd import inputs

LOG2E = 1.4426950408889634


def _bf16(x):
    return inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(np.asarray(x, np.float32)))


def spike_problem(N, spikes, alpha=18.0, M=16, D=32, seed=7, H=1):
    """iid N(0, 1/4) keys, N(0, 1) values and seeds; key row `pos` of every
    head replaced by alpha * S_m / ||S_m|| for each (pos, m) in spikes."""
    rng = np.random.default_rng(seed)
    S = _bf16(rng.standard_normal((M, D)))
    K = _bf16(rng.standard_normal((1, H, N, D)) * 0.5)
    V = _bf16(rng.standard_normal((1, H, N, D)))
    for pos, m in spikes:
        K[:, :, pos] = _bf16(alpha * S[m] / np.linalg.norm(S[m]))
    s = 1.0 / np.sqrt(D)
    return inputs.Problem(
        name=f"spike_N{N}", B=1, H=H, N=N, M=M, D=D, dtype="bf16", scale=float(s),
        S=inputs.f32_to_bf16_bits(S), K=inputs.f32_to_bf16_bits(K), V=inputs.f32_to_bf16_bits(V), seed=seed)


def overflowing_tiles(p, chunk, tile=128, h=0):
    """(first token of tile, score above the running max) for every tile of
    head h where the tile rule skips the checks and a score exceeds the
    running max by more than 16 binades (an fp16 weight above 65504)."""
    S = inputs.bf16_bits_to_f32(p.S).astype(np.float64)
    K = inputs.bf16_bits_to_f32(p.K[0, h]).astype(np.float64)
    q = p.scale * LOG2E * S
    qn = np.linalg.norm(q, axis=1)
    out = []
    for n0 in range(0, p.N, chunk):
        Ks = K[n0:n0 + chunk]
        T = Ks @ q.T
        mu = T[:32].max(axis=0)                  # the first step's exact max
        for t0 in range(0, Ks.shape[0], tile):
            km = np.linalg.norm(Ks[t0:t0 + tile], axis=1).max()
            tmax = T[t0:t0 + tile].max(axis=0)
            if np.any(qn * km - mu > 32):        # checked tile: the max follows the scores
                mu = np.maximum(mu, tmax)
            elif np.any(tmax - mu > 16):
                out.append((n0 + t0, float((tmax - mu).max())))
    return out
