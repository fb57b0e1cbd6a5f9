"""Seeded synthetic inputs for the FLARE++ routing forward pass.

This module only *draws* inputs (seeds S, keys K, values V); it holds none of
the routing arithmetic, so both the GPU path and the CPU oracle can be fed
from it.  The pages evaluate on PDE-surrogate meshes and point clouds
(Elasticity, Darcy, Airfoil, Pipe, DrivAerML) and on Long Range Arena; none
of those datasets is available here, so each named problem below is a
synthetic stand-in with the shape and structure of one of those workloads:

=========  =====================================================  =====
name       structure                                              dtype
=========  =====================================================  =====
tiny       B1 H4 N1024 M32 D16, K/V/S iid N(0,1)                  f32
mesh       B8 H8 N7225 (85x85 jittered grid) M64 D16              bf16
cloud      B4 H8 N11271 (denser near a random closed curve) M128  bf16
           D32
longseq    B32 H8 N4096 M128 D32, iid N(0,1) + low-frequency      bf16
           sinusoid per sequence
million    B1 H8 N2^20 (uniform in the unit cube) M256 D32        bf16
stress     B1 H2 N4096 M128 D32, iid N(0,1), scale 1 (sharp)      bf16
=========  =====================================================  =====

Recipe (fixed so that the bytes are reproducible):

* generator ``numpy.random.default_rng(1000 + id)`` with ids 1..6 in the
  table order, and a fixed draw order: points -> K map -> V map ->
  K noise -> V noise -> positional terms -> S (steps a problem does not
  use are skipped);
* linear maps ``W in R^{F x (H*D)}`` drawn iid N(0, 1/F), shared across the
  batch, no bias; the map's output for head h is columns h*D..h*D+D-1;
* noise is drawn as float32 N(0, sigma^2), block i of 2^22 elements from
  the i-th child of the problem's generator (``Generator.spawn``);
  everything else in float64;
* values are cast to float32, then (bf16 problems) rounded to bf16 with
  round-to-nearest-even.  bf16 arrays are returned as ``uint16`` bit
  patterns; float32 arrays as ``float32``;
* S is an M x D block of iid N(0, 1) seeds shared by every (b, h);
* the scale is 1/sqrt(D) except for ``stress`` (scale 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "Problem",
    "PROBLEMS",
    "make_problem",
    "random_problem",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclass
class Problem:
    name: str
    B: int
    H: int
    N: int
    M: int
    D: int
    dtype: str  # "bf16" or "f32"
    scale: float
    S: np.ndarray
    K: np.ndarray
    V: np.ndarray
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def tokens_heads(self) -> int:
        return self.B * self.H * self.N


_CHUNK = 1 << 22  # elements per independently seeded / converted block


def _pool():
    from concurrent.futures import ThreadPoolExecutor
    import os

    return ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def work(lo):
        u = flat[lo:lo + _CHUNK].view(np.uint32)
        r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
        out[lo:lo + _CHUNK] = (r >> np.uint32(16)).astype(np.uint16)

    with _pool() as ex:
        list(ex.map(work, range(0, flat.size, _CHUNK)))
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _finish(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _map_to_heads(feat: np.ndarray, W: np.ndarray, H: int, D: int) -> np.ndarray:
    """feat: B x N x F (float64), W: F x (H*D) -> float32 B x H x N x D.

    Written as a sum of F outer products (F is 3 or 4) over row blocks,
    in float64, rather than as a BLAS call: the same linear map, computed
    without large temporaries and independent of a BLAS library's threading.
    """
    B, N, F = feat.shape
    out = np.empty((B, H, N, D), dtype=np.float32)
    rows = 1 << 15
    jobs = [(b, h, lo) for b in range(B) for h in range(H) for lo in range(0, N, rows)]

    def work(job):
        b, h, lo = job
        f_blk = feat[b, lo:lo + rows]
        w = W[:, h * D:(h + 1) * D]
        acc = np.zeros((f_blk.shape[0], D))
        tmp = np.empty_like(acc)
        for f in range(F):
            np.multiply(f_blk[:, f, None], w[f][None, :], out=tmp)
            acc += tmp
        out[b, h, lo:lo + rows] = acc

    with _pool() as ex:
        list(ex.map(work, jobs))
    return out


def _noise(rng, shape, sigma: float) -> np.ndarray:
    """float32 N(0, sigma^2) of the given shape.

    The array is filled in blocks of 2^22 elements, block i from the i-th
    child generator spawned from ``rng`` (numpy SeedSequence spawning), so the
    bytes depend only on the seed and the shape, not on the thread count.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, _CHUNK))
    children = rng.spawn(len(starts))

    def work(i):
        lo = starts[i]
        blk = out[lo:lo + _CHUNK]
        children[i].standard_normal(size=blk.shape, dtype=np.float32, out=blk)
        if sigma != 1.0:
            blk *= np.float32(sigma)

    with _pool() as ex:
        list(ex.map(work, range(len(starts))))
    return out.reshape(shape)


def _seeds(rng, M: int, D: int) -> np.ndarray:
    return rng.standard_normal((M, D)).astype(np.float32)


def _tiny(rng):
    B, H, N, M, D = 1, 4, 1024, 32, 16
    K = _noise(rng, (B, H, N, D), 1.0)
    V = _noise(rng, (B, H, N, D), 1.0)
    S = _seeds(rng, M, D)
    return dict(B=B, H=H, N=N, M=M, D=D, dtype="f32", scale=1 / math.sqrt(D), S=S, K=K, V=V)


def _mesh(rng):
    B, H, M, D, side = 8, 8, 64, 16, 85
    N = side * side
    feat = np.empty((B, N, 3))
    for b in range(B):
        iy, ix = np.meshgrid(np.arange(side), np.arange(side), indexing="ij")  # row-major tokens
        x = (ix.reshape(-1) + rng.random(N)) / side
        y = (iy.reshape(-1) + rng.random(N)) / side
        feat[b, :, 0] = x
        feat[b, :, 1] = y
        feat[b, :, 2] = np.sin(2 * np.pi * x) * np.cos(2 * np.pi * y)
    WK = rng.normal(0.0, math.sqrt(1 / 3), size=(3, H * D))
    WV = rng.normal(0.0, math.sqrt(1 / 3), size=(3, H * D))
    K = _map_to_heads(feat, WK, H, D)
    V = _map_to_heads(feat, WV, H, D)
    S = _seeds(rng, M, D)
    return dict(B=B, H=H, N=N, M=M, D=D, dtype="bf16", scale=1 / math.sqrt(D), S=S, K=K, V=V)


def _curve(theta, a, b):
    r = 1.0
    for k in range(3):
        r = r + a[k] * np.cos((k + 1) * theta) + b[k] * np.sin((k + 1) * theta)
    r = 0.3 * r
    return np.stack([0.5 + r * np.cos(theta), 0.5 + r * np.sin(theta)], axis=-1)


def _dist_to_polyline(p: np.ndarray, poly: np.ndarray, k: int = 8) -> np.ndarray:
    """Euclidean distance from points p (n x 2) to the closed polyline poly (v x 2).

    The closest segment of a dense polyline touches one of the point's k
    nearest vertices, so only the segments adjacent to those are measured.
    """
    from scipy.spatial import cKDTree

    nv = poly.shape[0]
    _, idx = cKDTree(poly).query(p, k=k)
    best = np.full(p.shape[0], np.inf)
    for j in range(k):
        for step in (-1, 0):
            i0 = (idx[:, j] + step) % nv
            a = poly[i0]
            ab = poly[(i0 + 1) % nv] - a
            t = np.clip(((p - a) * ab).sum(-1) / np.maximum((ab * ab).sum(-1), 1e-300), 0.0, 1.0)
            d = np.sqrt(((p - a - t[:, None] * ab) ** 2).sum(-1))
            best = np.minimum(best, d)
    return best


def _cloud(rng):
    B, H, N, M, D = 4, 8, 11271, 128, 32
    feat = np.empty((B, N, 3))
    n_uni = N // 2
    n_cur = N - n_uni
    theta_poly = 2 * np.pi * np.arange(4096) / 4096
    for b in range(B):
        ca = rng.uniform(-0.05, 0.05, size=3)
        cb = rng.uniform(-0.05, 0.05, size=3)
        uni = rng.random((n_uni, 2))
        th = rng.uniform(0.0, 2 * np.pi, size=n_cur)
        cur = np.clip(_curve(th, ca, cb) + rng.normal(0.0, 0.03, size=(n_cur, 2)), 0.0, 1.0)
        pts = np.concatenate([uni, cur], axis=0)
        pts = pts[rng.permutation(N)]  # a point cloud carries no token order
        d = _dist_to_polyline(pts, _curve(theta_poly, ca, cb))
        feat[b, :, 0:2] = pts
        feat[b, :, 2] = d
    WK = rng.normal(0.0, math.sqrt(1 / 3), size=(3, H * D))
    WV = rng.normal(0.0, math.sqrt(1 / 3), size=(3, H * D))
    K = _map_to_heads(feat, WK, H, D)
    V = _map_to_heads(feat, WV, H, D)
    K += _noise(rng, K.shape, 0.1)
    V += _noise(rng, V.shape, 0.1)
    S = _seeds(rng, M, D)
    return dict(B=B, H=H, N=N, M=M, D=D, dtype="bf16", scale=1 / math.sqrt(D), S=S, K=K, V=V)


def _longseq(rng):
    B, H, N, M, D = 32, 8, 4096, 128, 32
    K = _noise(rng, (B, H, N, D), 1.0)
    V = _noise(rng, (B, H, N, D), 1.0)
    n = np.arange(N) / N
    for X in (K, V):
        f = rng.integers(1, 5, size=(B, D))
        phi = rng.uniform(0.0, 2 * np.pi, size=(B, D))
        pos = np.sin(2 * np.pi * f[:, None, :] * n[None, :, None] + phi[:, None, :])  # B x N x D
        X += pos[:, None, :, :].astype(np.float32)  # shared across heads
    S = _seeds(rng, M, D)
    return dict(B=B, H=H, N=N, M=M, D=D, dtype="bf16", scale=1 / math.sqrt(D), S=S, K=K, V=V)


def _million(rng):
    B, H, N, M, D = 1, 8, 1 << 20, 256, 32
    pts = rng.random((N, 3))
    feat = np.empty((B, N, 4))
    feat[0, :, :3] = pts
    feat[0, :, 3] = (pts * pts).sum(-1)
    WK = rng.normal(0.0, math.sqrt(1 / 4), size=(4, H * D))
    WV = rng.normal(0.0, math.sqrt(1 / 4), size=(4, H * D))
    K = _map_to_heads(feat, WK, H, D)
    V = _map_to_heads(feat, WV, H, D)
    K += _noise(rng, K.shape, 0.1)
    V += _noise(rng, V.shape, 0.1)
    S = _seeds(rng, M, D)
    return dict(B=B, H=H, N=N, M=M, D=D, dtype="bf16", scale=1 / math.sqrt(D), S=S, K=K, V=V)


def _stress(rng):
    B, H, N, M, D = 1, 2, 4096, 128, 32
    K = _noise(rng, (B, H, N, D), 1.0)
    V = _noise(rng, (B, H, N, D), 1.0)
    S = _seeds(rng, M, D)
    return dict(B=B, H=H, N=N, M=M, D=D, dtype="bf16", scale=1.0, S=S, K=K, V=V)


PROBLEMS = {
    "tiny": (1, _tiny),
    "mesh": (2, _mesh),
    "cloud": (3, _cloud),
    "longseq": (4, _longseq),
    "million": (5, _million),
    "stress": (6, _stress),
}


def make_problem(name: str) -> Problem:
    """Draw one of the named problems (see the module docstring)."""
    pid, fn = PROBLEMS[name]
    seed = 1000 + pid
    rng = np.random.default_rng(seed)
    d = fn(rng)
    dtype = d["dtype"]
    return Problem(
        name=name, B=d["B"], H=d["H"], N=d["N"], M=d["M"], D=d["D"], dtype=dtype,
        scale=d["scale"], S=_finish(d["S"], dtype), K=_finish(d["K"], dtype),
        V=_finish(d["V"], dtype), seed=seed,
    )


def random_problem(B: int, H: int, N: int, M: int, D: int, dtype: str = "bf16",
                   scale: float | None = None, seed: int = 0, per_head_seeds: bool = False,
                   sigma: float = 1.0, sigma_v: float | None = None,
                   k_ramp: tuple[float, float] | None = None) -> Problem:
    """iid N(0, sigma^2) K, N(0, sigma_v^2) V (sigma_v defaults to sigma), N(0, 1) seeds:
    for edge shapes (ragged N, small M, ...) and sharpness sweeps.

    k_ramp=(lo, hi) multiplies key row n by lo + (hi - lo) * n / (N - 1), so the
    key norms (and the sharpness of the encode softmaxes) grow along the
    token axis: the largest scores of a split arrive late."""
    rng = np.random.default_rng(seed)
    K = _noise(rng, (B, H, N, D), sigma)
    if k_ramp is not None:
        lo, hi = k_ramp
        ramp = lo + (hi - lo) * np.arange(N, dtype=np.float64) / max(N - 1, 1)
        K = (K * ramp[None, None, :, None]).astype(np.float32)
    V = _noise(rng, (B, H, N, D), sigma if sigma_v is None else sigma_v)
    S = rng.standard_normal((H, M, D) if per_head_seeds else (M, D)).astype(np.float32)
    if scale is None:
        scale = 1 / math.sqrt(D)
    return Problem(
        name=f"random_B{B}_H{H}_N{N}_M{M}_D{D}_{dtype}", B=B, H=H, N=N, M=M, D=D, dtype=dtype,
        scale=float(scale), S=_finish(S, dtype), K=_finish(K, dtype), V=_finish(V, dtype),
        seed=seed,
    )
