#!/usr/bin/env python3
"""Throughput of the fused FLARE++ route (libflarepp) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload million]

A step is one call of flarepp_route (seed encode -> encode -> decode for every
(b, h)) over the synthetic million-point problem (B1 H8 N2^20 M256 D32, bf16
inputs, float32 outputs), with inputs resident in HBM.  Warm-up runs at least
W steps and at least 200 ms of continuous work (the GPU's clocks settle over
tens of milliseconds); then exactly K timed steps, bracketed by device
synchronisations, with a HIP event before every step and after the last.
Rank 0 prints one JSON line:

* value = routed token*heads per second, B*H*N / (median seconds per step);
  ms_per_step is that median, ms_per_step_mean the mean over the K steps;
  mfma_frac_of_bf16_peak = 12*M*D flops per token*head at that rate over the
  2.5 PFLOP/s dense bf16 peak;
* roofline = the dominant kernel's algorithmic HBM bytes per launch over its
  average launch duration (HIP events recorded around every kernel by
  flarepp_route_profiled on the launch stream), with the copy-calibrated HBM
  traffic and the matrix-core busy fraction from the rocprofv3 counter
  summary in profiles/ when that summary was taken from the current kernel
  sources (null otherwise);
* configs = the other workloads (tiny, mesh, cloud, longseq): median time
  per route, token*heads/s, algorithmic rates against the peaks, and for the
  three whose K and V fit in the 256 MB Infinity Cache the median time with
  512 MB written between routes (cache flushed);
* flare, backward, spectrum = fixed-query FLARE (route/FLARE time ratio), the
  backward (bf16 inputs on the matrix cores, and float32 copies on the float32
  path, each with its time over the forward route's) and the mixing-matrix
  spectrum on the same inputs;
* token_shards = one GPU's share of the route split over --shards token
  ranges (its shard's encodes and decode plus the merges of all shards'
  records), against the route time over the shard count;
* cpu_baseline = the oracle (single-threaded C, fp64) on a bounded sample of
  the same problem, with the host's core count and CPU model.

Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 matrix cores, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
METRIC = "routed token·heads/sec + % bf16 MFMA peak, fused route, N=1M M=256"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "rank_latent_attention_seed_amd", "csrc")
WARMUP_SECONDS = 0.2
FLUSH_BYTES = 512 << 20
OTHER_WORKLOADS = ("tiny", "mesh", "cloud", "longseq")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def host_cpu() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_nproc": os.cpu_count(), "host_cpu_model": model}


class HipEvents:
    """hipEvent_t handles through the HIP runtime (ctypes)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev
        self.n = n

    def record(self, i: int, stream) -> None:
        if self.hip.hipEventRecord(self.arr[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def per_token_bytes(kind: str, D: int, elem: int) -> int:
    """Algorithmic HBM bytes per token*head of one kernel (inputs of `elem`
    bytes, float32 output)."""
    if kind in ("seed_encode", "encode"):
        return 2 * D * elem       # K and V rows read once
    if kind == "decode":
        return D * elem + D * 4   # K row read, Y row written
    return 0


def route_bytes(D: int, elem: int) -> int:
    """Algorithmic HBM bytes per token*head of the route: K read three times,
    V twice, Y written once."""
    return 5 * D * elem + 4 * D


class Route:
    """One workload resident on the GPU and its flarepp_route call."""

    def __init__(self, fp, torch, p):
        import numpy as np

        def dev(x):
            if x.dtype == np.uint16:
                return torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
            return torch.from_numpy(x).to("cuda")

        self.fp, self.torch, self.p = fp, torch, p
        self.S, self.K, self.V = dev(p.S), dev(p.K), dev(p.V)
        self.Y = torch.empty((p.B, p.H, p.N, p.D), dtype=torch.float32, device="cuda")
        self.desc = fp.desc_for(self.S, self.K, p.scale)
        self.nbytes = fp.flarepp_workspace_size(self.desc, fp.OP_ROUTE)
        self.ws = torch.empty(max(self.nbytes, 1), dtype=torch.uint8, device="cuda")
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.ptrs = (self.S.data_ptr(), self.K.data_ptr(), self.V.data_ptr(), self.Y.data_ptr())
        self.elem = 2 if p.dtype == "bf16" else 4
        self.tokens_heads = p.B * p.H * p.N

    def step(self):
        st = self.fp.flarepp_route(self.desc, *self.ptrs, None, None, self.ws.data_ptr(), self.nbytes,
                                   self.stream)
        if st != 0:
            raise self.fp.FlareppError(st, "flarepp_route")

    def kernel_stats(self, steps: int) -> dict:
        """Per kernel kind: launches per step and average launch duration, from
        events recorded around every launch (flarepp_route_profiled)."""
        fp = self.fp
        max_l = 256
        kev = HipEvents(2 * max_l)
        kinds = (ctypes.c_int32 * max_l)()
        n_l = ctypes.c_int32(0)
        per_kind = {}
        for _ in range(steps):
            st = fp.flarepp_route_profiled(self.desc, *self.ptrs, None, None, self.ws.data_ptr(), self.nbytes,
                                           self.stream, kev.arr, kinds, max_l, n_l)
            if st != 0:
                raise fp.FlareppError(st, "flarepp_route_profiled")
            self.torch.cuda.synchronize()
            if n_l.value > max_l:
                raise RuntimeError("more launches than recorded events")
            for i in range(n_l.value):
                per_kind.setdefault(fp.KERNEL_KINDS[kinds[i]], []).append(kev.elapsed_ms(2 * i, 2 * i + 1))
        kev.close()
        return {kind: {"launches_per_step": len(xs) // steps, "avg_us": 1e3 * sum(xs) / len(xs),
                       "ms_per_step": sum(xs) / steps}
                for kind, xs in per_kind.items()}


def warm(step, torch, min_steps: int) -> int:
    """At least min_steps calls and at least WARMUP_SECONDS of continuous work."""
    n, t0 = 0, time.perf_counter()
    while n < min_steps or time.perf_counter() - t0 < WARMUP_SECONDS:
        for _ in range(max(1, min_steps // 4)):
            step()
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(step, torch, stream, steps: int) -> list:
    """Exactly `steps` calls between two synchronisations, an event before
    each and after the last: per-step milliseconds."""
    ev = HipEvents(steps + 1)
    torch.cuda.synchronize()
    for i in range(steps):
        ev.record(i, stream)
        step()
    ev.record(steps, stream)
    torch.cuda.synchronize()
    ms = [ev.elapsed_ms(i, i + 1) for i in range(steps)]
    ev.close()
    return ms


def time_flushed(step, torch, stream, iters: int) -> list:
    """Per-call milliseconds with FLUSH_BYTES written to HBM before each call,
    so that no input is left in the last-level cache."""
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ev = HipEvents(2)
    ms = []
    for i in range(iters):
        buf.fill_(i & 0xFF)
        ev.record(0, stream)
        step()
        ev.record(1, stream)
        torch.cuda.synchronize()
        ms.append(ev.elapsed_ms(0, 1))
    ev.close()
    del buf
    return ms


def counter_summary(workload: str):
    """The rocprofv3 counter summary of this workload, if it was taken from the
    current kernel sources."""
    path = os.path.join(PROFILES, f"counters_route_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec if rec.get("source_hash") == kernel_source_hash() else None


def route_rates(p, ms: float, elem: int) -> dict:
    th = p.B * p.H * p.N
    sec = ms * 1e-3
    flops = 12.0 * p.M * p.D * th
    peak = BF16_PEAK_TFLOPS if p.dtype == "bf16" else FP32_VECTOR_PEAK_TFLOPS
    return {
        "token_heads_per_s": th / sec,
        "algorithmic_tflops": flops / sec / 1e12,
        "frac_of_compute_peak": flops / sec / (peak * 1e12),
        "compute_peak": "bf16 matrix cores 2500 TFLOP/s" if p.dtype == "bf16" else "fp32 vector 157.3 TFLOP/s",
        "algorithmic_hbm_gbs": route_bytes(p.D, elem) * th / sec / 1e9,
        "frac_of_hbm_peak": route_bytes(p.D, elem) * th / sec / 1e9 / HBM_PEAK_GBS,
    }


def graph_record(fp, torch, r: Route, steps: int) -> dict:
    """The route captured once in a HIP graph (through torch.cuda.CUDAGraph; the
    library launches its kernels on the stream it is given, allocates nothing
    and records no memset) and replayed: median time per replay, and every
    checked replay bitwise equal to the eager route."""
    Y0 = r.Y.clone()
    r.step()
    torch.cuda.synchronize()
    ref = r.Y.clone()

    def launch():
        st = fp.flarepp_route(r.desc, *r.ptrs, None, None, r.ws.data_ptr(), r.nbytes,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise fp.FlareppError(st, "flarepp_route (capture)")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    match = True
    for i in range(4):  # replays with eager work and synchronisations between them
        r.Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        match = match and bool(torch.equal(r.Y, ref))
        r.step()
        torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ms = time_steps(g.replay, torch, stream, steps)
    r.Y.copy_(Y0)
    del g
    return {"ms_per_step_graph": statistics.median(ms), "replays_match_eager": match}


def config_record(fp, torch, inputs, name: str, steps: int, warmup: int) -> dict:
    t0 = time.perf_counter()
    p = inputs.make_problem(name)
    r = Route(fp, torch, p)
    warm(r.step, torch, warmup)
    ms = time_steps(r.step, torch, r.stream, steps)
    med = statistics.median(ms)
    rec = {"B": p.B, "H": p.H, "N": p.N, "M": p.M, "D": p.D, "dtype": p.dtype, "scale": p.scale,
           "steps": steps, "ms_per_step": med, "ms_per_step_mean": sum(ms) / len(ms)}
    rec.update(route_rates(p, med, r.elem))
    rec["kernels_avg_us"] = {k: round(v["avg_us"], 2) for k, v in r.kernel_stats(10).items()}
    rec.update(graph_record(fp, torch, r, steps))
    kv_bytes = 2 * p.B * p.H * p.N * p.D * r.elem
    if kv_bytes < (256 << 20) and name != "tiny":
        fl = time_flushed(r.step, torch, r.stream, 20)
        rec["ms_per_step_cache_flushed"] = statistics.median(fl)
        rec["token_heads_per_s_cache_flushed"] = p.B * p.H * p.N / (statistics.median(fl) * 1e-3)
    log(f"[bench] config {name}: B{p.B} H{p.H} N{p.N} M{p.M} D{p.D} {p.dtype}: {med * 1e3:.1f} us/route "
        f"(mean {1e3 * rec['ms_per_step_mean']:.1f}), {rec['token_heads_per_s'] / 1e9:.3f} G token*heads/s, "
        f"{100 * rec['frac_of_compute_peak']:.1f}% of compute peak, {100 * rec['frac_of_hbm_peak']:.1f}% of HBM"
        + (f"; cache flushed {1e3 * rec['ms_per_step_cache_flushed']:.1f} us" if "ms_per_step_cache_flushed" in rec
           else "") + f"; graph replay {1e3 * rec['ms_per_step_graph']:.1f} us"
        + ("" if rec["replays_match_eager"] else " (REPLAYS DIFFER)") + f" ({time.perf_counter() - t0:.1f} s)")
    del r
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(p, n_sample: int) -> dict:
    """The oracle (one thread) on one head and the first n_sample tokens."""
    import oracle

    Kh = p.K[0:1, 0:1, :n_sample].copy()
    Vh = p.V[0:1, 0:1, :n_sample].copy()
    t0 = time.perf_counter()
    oracle.route(p.S, Kh, Vh, p.scale)
    dt = time.perf_counter() - t0
    rec = {
        "value": n_sample / dt,
        "unit": "token*heads/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"full three-stage route of 1 head x {n_sample} tokens of the {p.name} problem "
                  f"(M={p.M}, D={p.D}, bf16 inputs), fp64, {dt:.1f} s",
    }
    rec.update(host_cpu())
    return rec


def backward_record(fp, torch, r: Route, steps: int, route_ms: float) -> dict:
    """flarepp_route_backward on the same inputs (bf16, matrix cores) and on
    float32 copies of them (float32 vector path), with a seeded dY."""
    p = r.p
    dY = torch.randn(r.K.shape, generator=torch.Generator(device="cuda").manual_seed(7), device="cuda")
    th = p.B * p.H * p.N
    flops = 30.0 * p.M * p.D * th  # 3 stages x 10 M D (logits, dP, dV, dQ, dK)
    out = {"op": "flarepp_route_backward", "workload": f"{p.name} shapes, seeded dY", "steps": steps,
           "algorithmic_flops_per_step": flops}
    for label, cast in (("bf16", lambda t: t), ("f32", lambda t: t.float())):
        S, K, V = cast(r.S), cast(r.K), cast(r.V)
        dS = torch.empty(S.shape, dtype=torch.float32, device="cuda")
        dK = torch.empty(K.shape, dtype=torch.float32, device="cuda")
        dV = torch.empty(K.shape, dtype=torch.float32, device="cuda")
        bdesc = fp.desc_for(S, K, p.scale)
        bbytes = fp.flarepp_workspace_size(bdesc, fp.OP_ROUTE_BACKWARD)
        bws = torch.empty(max(bbytes, 1), dtype=torch.uint8, device="cuda")
        bptr = [t.data_ptr() for t in (S, K, V, dY, dS, dK, dV)]

        def bstep():
            st = fp.flarepp_route_backward(bdesc, *bptr, bws.data_ptr(), bbytes, r.stream)
            if st != 0:
                raise fp.FlareppError(st, "flarepp_route_backward")

        bstep()
        torch.cuda.synchronize()
        bms = statistics.median(time_steps(bstep, torch, r.stream, steps))
        btf = flops / (bms * 1e-3) / 1e12
        peak = BF16_PEAK_TFLOPS if label == "bf16" else FP32_VECTOR_PEAK_TFLOPS
        log(f"[bench] backward ({label}): {bms:.2f} ms/step, {btf:.2f} TFLOP/s algorithmic, "
            f"{bms / route_ms:.2f} x the forward route")
        out[label] = {
            "ms_per_step": bms, "value": th / (bms * 1e-3), "unit": "token*heads/s",
            "over_forward_route": round(bms / route_ms, 3),
            "roofline": {"bound": "mfma" if label == "bf16" else "alu", "achieved": round(btf, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(btf / peak, 4), "traffic": None},
        }
        del bws, dS, dK, dV
    # the training step with the forward kept for the backward: flarepp_route_save
    # (the route with the backward's forward stages, saving Qd, Z and the two
    # log-sum-exps), then flarepp_route_backward_saved (no recomputed forward)
    if p.dtype == "bf16" and p.M <= 256:
        bdesc = fp.desc_for(r.S, r.K, p.scale)
        bbytes = fp.flarepp_workspace_size(bdesc, fp.OP_ROUTE_BACKWARD)
        bws = torch.empty(max(bbytes, 1), dtype=torch.uint8, device="cuda")
        Y = torch.empty(r.K.shape, dtype=torch.float32, device="cuda")
        Qd = torch.empty((p.B, p.H, p.M, p.D), dtype=torch.float32, device="cuda")
        Z = torch.empty_like(Qd)
        lse = torch.empty(fp.saved_lse_count(bdesc), dtype=torch.float32, device="cuda")
        dS = torch.empty(r.S.shape, dtype=torch.float32, device="cuda")
        dK = torch.empty(r.K.shape, dtype=torch.float32, device="cuda")
        dV = torch.empty(r.K.shape, dtype=torch.float32, device="cuda")

        def fstep():
            st = fp.flarepp_route_save(bdesc, r.S.data_ptr(), r.K.data_ptr(), r.V.data_ptr(), Y.data_ptr(),
                                       Qd.data_ptr(), Z.data_ptr(), lse.data_ptr(), bws.data_ptr(), bbytes, r.stream)
            if st != 0:
                raise fp.FlareppError(st, "flarepp_route_save")

        def gstep():
            st = fp.flarepp_route_backward_saved(bdesc, r.S.data_ptr(), r.K.data_ptr(), r.V.data_ptr(),
                                                 Qd.data_ptr(), Z.data_ptr(), lse.data_ptr(), dY.data_ptr(),
                                                 dS.data_ptr(), dK.data_ptr(), dV.data_ptr(), bws.data_ptr(),
                                                 bbytes, r.stream)
            if st != 0:
                raise fp.FlareppError(st, "flarepp_route_backward_saved")

        fstep()
        gstep()
        torch.cuda.synchronize()
        fms = statistics.median(time_steps(fstep, torch, r.stream, steps))
        gms = statistics.median(time_steps(gstep, torch, r.stream, steps))
        gtf = flops / (gms * 1e-3) / 1e12
        log(f"[bench] saved forward {fms:.2f} ms + backward (bf16, saved) {gms:.2f} ms = {fms + gms:.2f} ms "
            f"per training step (route + recomputing backward: {route_ms + out['bf16']['ms_per_step']:.2f} ms); "
            f"backward {gms / route_ms:.2f} x the forward route")
        out["bf16_saved"] = {
            "ops": "flarepp_route_save + flarepp_route_backward_saved",
            "route_save_ms": fms, "backward_ms": gms, "training_step_ms": fms + gms,
            "over_forward_route": round(gms / route_ms, 3),
            "roofline": {"bound": "mfma", "achieved": round(gtf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(gtf / BF16_PEAK_TFLOPS, 4), "traffic": None},
        }
        del bws, Y, Qd, Z, lse, dS, dK, dV
    return out


def spectrum_record(fp, torch, r: Route, steps: int) -> dict:
    p = r.p
    eig = torch.empty((p.B, p.H, p.M), dtype=torch.float32, device="cuda")
    sbytes = fp.flarepp_workspace_size(r.desc, fp.OP_SPECTRUM)
    sws = torch.empty(max(sbytes, 1), dtype=torch.uint8, device="cuda")

    def sstep():
        st = fp.flarepp_spectrum(r.desc, r.ptrs[0], r.ptrs[1], r.ptrs[2], eig.data_ptr(), None, sws.data_ptr(),
                                 sbytes, r.stream)
        if st != 0:
            raise fp.FlareppError(st, "flarepp_spectrum")

    sstep()
    torch.cuda.synchronize()
    sms = statistics.median(time_steps(sstep, torch, r.stream, steps))
    sflops = 2.0 * p.M * p.M * p.B * p.H * p.N  # the M x M product F F^T over all tokens
    stf = sflops / (sms * 1e-3) / 1e12
    top = eig[:, :, :4].mean(dim=(0, 1)).tolist()
    log(f"[bench] spectrum: {sms:.2f} ms/step, Gram {stf:.2f} TFLOP/s; mean top eigenvalues {top}")
    return {"op": "flarepp_spectrum", "ms_per_step": sms, "steps": steps, "gram_tflops": round(stf, 2),
            "mean_top4_eigenvalues": [round(x, 6) for x in top]}


def shard_record(fp, torch, r: Route, shards: int, steps: int, route_ms: float) -> dict:
    """One GPU's share of the route sharded over `shards` equal token ranges
    (context parallelism): stage-1 encode of its shard to its record slot,
    merge of all slots, stage-2 encode, merge, decode of its shard.  The other
    shards' records are written once before timing and stay in place; the
    exchange of records between devices is not part of the timed work (its
    payload per stage is reported).  share_efficiency = (route time / shards)
    over this time: the fraction of linear speed-up one shard's work allows
    before any exchange."""
    p = r.p
    N = p.N
    bounds = [N * i // shards for i in range(shards + 1)]
    K = [r.K[:, :, b0:b1].contiguous() for b0, b1 in zip(bounds, bounds[1:])]
    V = [r.V[:, :, b0:b1].contiguous() for b0, b1 in zip(bounds, bounds[1:])]
    descs = [fp.desc_for(r.S, k, p.scale) for k in K]
    rec_bytes = fp.flarepp_shard_records_size(r.desc, shards)
    rec = torch.empty(rec_bytes // 4, dtype=torch.float32, device="cuda")
    Qd = torch.empty((p.B, p.H, p.M, p.D), dtype=torch.float32, device="cuda")
    Z = torch.empty_like(Qd)
    Y0 = torch.empty(K[0].shape, dtype=torch.float32, device="cuda")
    wsn = max(max(fp.flarepp_workspace_size(d, op) for op in (fp.OP_SEED_ENCODE, fp.OP_ENCODE, fp.OP_DECODE))
              for d in descs)
    ws = torch.empty(max(wsn, 1), dtype=torch.uint8, device="cuda")

    def ok(st, name):
        if st != 0:
            raise fp.FlareppError(st, name)

    def encode(stage, i):
        q = r.S if stage == 1 else Qd
        ok(fp.flarepp_encode_shard(descs[i], stage, q.data_ptr(), K[i].data_ptr(), V[i].data_ptr(),
                                   rec.data_ptr(), i, shards, ws.data_ptr(), wsn, r.stream), "flarepp_encode_shard")

    def merge(out):
        ok(fp.flarepp_merge_shards(r.desc, rec.data_ptr(), shards, out.data_ptr(), r.stream), "flarepp_merge_shards")

    for stage, out in ((1, Qd), (2, Z)):
        for i in range(shards):
            encode(stage, i)
        merge(out)

    def share_step():
        encode(1, 0)
        merge(Qd)
        encode(2, 0)
        merge(Z)
        ok(fp.flarepp_decode(descs[0], Qd.data_ptr(), Z.data_ptr(), K[0].data_ptr(), Y0.data_ptr(),
                             ws.data_ptr(), wsn, r.stream), "flarepp_decode")

    warm(share_step, torch, 4)
    sms = statistics.median(time_steps(share_step, torch, r.stream, steps))
    eff = route_ms / shards / sms
    log(f"[bench] token shards ({shards}): one shard's share {sms:.3f} ms, route/{shards} = "
        f"{route_ms / shards:.3f} ms, share efficiency {eff:.3f}; records {rec_bytes / 1e6:.2f} MB per stage")
    out = {"shards": shards, "tokens_per_shard": bounds[1], "ms_per_step": sms, "steps": steps,
           "share_efficiency": round(eff, 4), "record_bytes_per_stage": rec_bytes,
           "exchange": "not timed (one GPU)"}
    del K, V, rec, ws, Y0
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30,
                    help="warm-up steps at least (and at least 200 ms of continuous work)")
    ap.add_argument("--workload", default="million")
    ap.add_argument("--configs", default=",".join(OTHER_WORKLOADS),
                    help="other workloads to time after the headline one (comma list, or 'none')")
    ap.add_argument("--flare-steps", type=int, default=-1,
                    help="timed fixed-query FLARE steps (default: --steps; 0 = skip)")
    ap.add_argument("--kernel-steps", type=int, default=-1,
                    help="routes timed per kernel through flarepp_route_profiled (default: --steps)")
    ap.add_argument("--backward-steps", type=int, default=3,
                    help="timed calls of the float32 backward on the same shapes (0 = skip)")
    ap.add_argument("--spectrum-steps", type=int, default=2,
                    help="timed calls of the mixing-matrix spectrum on the same inputs (0 = skip)")
    ap.add_argument("--shards", type=int, default=4,
                    help="token shards for the one-GPU share of a context-parallel route (0 = skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the timed runs, copy MIB MiB device-to-device once (a kernel of known "
                         "traffic, for scaling hardware byte counters)")
    ap.add_argument("--cpu-sample", type=int, default=393216,
                    help="tokens of one head for the oracle baseline (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the exchange of "
              "token-shard records between GPUs is not built", file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        return 2
    flare_steps = args.steps if args.flare_steps < 0 else args.flare_steps
    kernel_steps = args.steps if args.kernel_steps < 0 else args.kernel_steps

    import torch
    from rank_latent_attention_seed_amd import flarepp as fp
    from rank_latent_attention_seed_amd import inputs

    fp.library()
    t0 = time.perf_counter()
    p = inputs.make_problem(args.workload)
    log(f"[bench] inputs {p.name}: B{p.B} H{p.H} N{p.N} M{p.M} D{p.D} {p.dtype} "
        f"({time.perf_counter() - t0:.1f} s to draw)")
    r = Route(fp, torch, p)

    nw = warm(r.step, torch, args.warmup)
    log(f"[bench] warm-up done ({nw} steps)")

    # ---- timed region: exactly K steps
    t_start = time.perf_counter()
    ms_steps = time_steps(r.step, torch, r.stream, args.steps)
    wall = time.perf_counter() - t_start
    ms = statistics.median(ms_steps)
    ms_mean = sum(ms_steps) / len(ms_steps)
    value = r.tokens_heads / (ms * 1e-3)
    flops = 12.0 * p.M * p.D * r.tokens_heads
    mfma_frac = flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
    log(f"[bench] {args.steps} steps: median {ms:.3f} ms/step, mean {ms_mean:.3f} (wall {wall:.2f} s), "
        f"{value / 1e9:.3f} G token*heads/s, {100 * mfma_frac:.1f}% of bf16 MFMA peak")

    # ---- fixed-query FLARE (Qd := S: one encode, one decode) on the same inputs
    flare = None
    if flare_steps > 0:
        fbytes = fp.flarepp_workspace_size(r.desc, fp.OP_FLARE)
        fws = torch.empty(max(fbytes, 1), dtype=torch.uint8, device="cuda")

        def flare_step():
            st = fp.flarepp_flare(r.desc, *r.ptrs, None, fws.data_ptr(), fbytes, r.stream)
            if st != 0:
                raise fp.FlareppError(st, "flarepp_flare")

        warm(flare_step, torch, args.warmup)
        flare_ms = statistics.median(time_steps(flare_step, torch, r.stream, flare_steps))
        del fws
        flare = {"ms_per_step": flare_ms, "route_over_flare": ms / flare_ms, "steps": flare_steps}
        log(f"[bench] fixed-query FLARE: {flare_ms:.3f} ms/step; route / FLARE = {ms / flare_ms:.3f}")

    # ---- per-kernel durations on the launch stream
    kstats = r.kernel_stats(max(kernel_steps, 1))
    for kind, st in sorted(kstats.items(), key=lambda kv: -kv[1]["ms_per_step"]):
        log(f"[bench]   {kind:12s} {st['launches_per_step']:3d} launches/step  avg {st['avg_us']:9.2f} us  "
            f"{st['ms_per_step']:.3f} ms/step")
    n_decode = kstats.get("decode", {}).get("launches_per_step", 1) or 1
    heads_per_launch = (p.B * p.H) // n_decode
    dom = max((k for k in kstats if per_token_bytes(k, p.D, r.elem) > 0), key=lambda k: kstats[k]["ms_per_step"])
    units = heads_per_launch * p.N
    alg_bytes = per_token_bytes(dom, p.D, r.elem) * units
    achieved = alg_bytes / (kstats[dom]["avg_us"] * 1e-6) / 1e9
    counters = counter_summary(p.name)
    ck = (counters or {}).get("kernels", {})
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": ck.get(dom, {}).get("hbm_bytes_per_launch"),
        "kernel": dom,
        "algorithmic_bytes_per_launch": alg_bytes,
        "avg_launch_us": round(kstats[dom]["avg_us"], 2),
        "mfma_busy_frac": ck.get(dom, {}).get("mfma_busy_frac"),
        "algorithmic_mfma_frac": round(4.0 * p.M * p.D * units / (kstats[dom]["avg_us"] * 1e-6)
                                       / (BF16_PEAK_TFLOPS * 1e12), 4),
    }
    counter_fields = None
    if counters:
        counter_fields = {"source_hash": counters["source_hash"], "summary": counters.get("summary_file"),
                          "kernels": {k: {f: v.get(f) for f in ("mfma_busy_frac", "mfma_valu_coexec_frac",
                                                                 "valu_busy_frac", "lds_bank_conflict_frac",
                                                                 "hbm_bytes_per_launch")}
                                      for k, v in ck.items()}}

    # ---- the other workloads (configs of the same line)
    configs = {}
    names = [] if args.configs in ("", "none") else [c for c in args.configs.split(",") if c and c != p.name]
    for name in names:
        configs[name] = config_record(fp, torch, inputs, name, args.steps, args.warmup)

    bwd = backward_record(fp, torch, r, args.backward_steps, ms) if args.backward_steps > 0 else None
    spec = spectrum_record(fp, torch, r, args.spectrum_steps) if args.spectrum_steps > 0 else None
    shard = shard_record(fp, torch, r, args.shards, max(args.steps // 2, 3), ms) if args.shards > 1 else None

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy} MiB done")
        del src, dst

    cpu = None
    if args.cpu_sample > 0:
        log(f"[bench] oracle baseline on {args.cpu_sample} tokens ...")
        cpu = cpu_baseline(p, min(args.cpu_sample, p.N))
        log(f"[bench] oracle: {cpu['value']:.0f} token*heads/s")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "token*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nw,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "B": p.B, "H": p.H, "N": p.N, "M": p.M, "D": p.D,
                   "scale": p.scale, "outputs": "fp32", "global_batch": p.B, "seq_len": p.N},
        "ms_per_step_mean": ms_mean,
        "mfma_frac_of_bf16_peak": mfma_frac,
        "kernels": kstats,
        "roofline": roofline,
        "counters": counter_fields,
        "configs": configs,
        "flare": flare,
        "backward": bwd,
        "spectrum": spec,
        "token_shards": shard,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
