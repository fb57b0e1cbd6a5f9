#!/usr/bin/env python3
"""Throughput of the fused FLARE++ route (libflarepp) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload million]

A step is one call of flarepp_route (seed encode -> encode -> decode for every
(b, h)) over the synthetic million-point problem (B1 H8 N2^20 M256 D32, bf16
inputs, float32 outputs), with inputs resident in HBM.  W untimed warm-up
steps are followed by exactly K timed steps bracketed by device
synchronisations; rank 0 prints one JSON line.  The line carries:

* value = routed token*heads per second (B*H*N / seconds per step), and the
  same work as a fraction of the bf16 matrix-core peak (12*M*D flops per
  token*head);
* roofline = the dominant kernel's algorithmic HBM bytes per launch over its
  average launch duration, from HIP events recorded around every kernel by
  flarepp_route_profiled over K further steps;
* backward = flarepp_route_backward (float32) on the same shapes: time per
  call and algorithmic TFLOP/s (30 M D flops per token*head: five D-length
  contractions per latent-token pair in each of the three stages) against
  the float32 vector peak;
* spectrum = flarepp_spectrum on the same inputs: time per call (forming the
  M x M matrix over all tokens and its Jacobi eigenvalues) and the mean of
  the four largest eigenvalues per head;
* route_over_flare = the route's time over fixed-query FLARE's (Qd := S: one
  encode and one decode) on the same inputs;
* cpu_baseline = the oracle (single-threaded C, fp64) on a bounded sample of
  the same problem (one head, the first 393216 tokens: ~13 s).

Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "rank_latent_attention_seed_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles through the HIP runtime (ctypes)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev
        self.n = n

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def per_token_bytes(kind: str, D: int) -> int:
    """Algorithmic HBM bytes per token*head of one kernel (bf16 in, fp32 out)."""
    if kind in ("seed_encode", "encode"):
        return 2 * D * 2          # K and V rows read once
    if kind == "decode":
        return D * 2 + D * 4      # K row read, Y row written
    return 0


def cpu_baseline(p, n_sample: int) -> dict:
    """The oracle (one thread) on one head and the first n_sample tokens."""
    import oracle

    Kh = p.K[0:1, 0:1, :n_sample].copy()
    Vh = p.V[0:1, 0:1, :n_sample].copy()
    t0 = time.perf_counter()
    oracle.route(p.S, Kh, Vh, p.scale)
    dt = time.perf_counter() - t0
    return {
        "value": n_sample / dt,
        "unit": "token*heads/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"full three-stage route of 1 head x {n_sample} tokens of the {p.name} problem "
                  f"(M={p.M}, D={p.D}, bf16 inputs), fp64, {dt:.1f} s",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clocks ramp up over the first tens of milliseconds of
    # continuous load: 30 warm-up steps (~45 ms) reach the steady state
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="million")
    ap.add_argument("--backward-steps", type=int, default=3,
                    help="timed calls of the float32 backward on the same shapes (0 = skip)")
    ap.add_argument("--spectrum-steps", type=int, default=2,
                    help="timed calls of the mixing-matrix spectrum on the same inputs (0 = skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the timed runs, copy MIB MiB device-to-device once (a kernel of known "
                         "traffic, for scaling hardware byte counters)")
    ap.add_argument("--cpu-sample", type=int, default=393216,
                    help="tokens of one head for the oracle baseline (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the route's "
              "multi-GPU token sharding is not built", file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        return 2

    import torch
    from rank_latent_attention_seed_amd import flarepp as fp
    from rank_latent_attention_seed_amd import inputs

    fp.library()
    t0 = time.perf_counter()
    p = inputs.make_problem(args.workload)
    log(f"[bench] inputs {p.name}: B{p.B} H{p.H} N{p.N} M{p.M} D{p.D} {p.dtype} "
        f"({time.perf_counter() - t0:.1f} s to draw)")

    def dev(x):
        import numpy as np

        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(x).to("cuda")

    S, K, V = dev(p.S), dev(p.K), dev(p.V)
    Y = torch.empty((p.B, p.H, p.N, p.D), dtype=torch.float32, device="cuda")
    desc = fp.desc_for(S, K, p.scale)
    nbytes = fp.flarepp_workspace_size(desc, fp.OP_ROUTE)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = (S.data_ptr(), K.data_ptr(), V.data_ptr(), Y.data_ptr())

    def step():
        st = fp.flarepp_route(desc, ptrs[0], ptrs[1], ptrs[2], ptrs[3], None, None, ws.data_ptr(),
                              nbytes, stream)
        if st != 0:
            raise fp.FlareppError(st, "flarepp_route")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warm-up done ({args.warmup} steps)")

    # ---- timed region: exactly K steps
    t_start = time.perf_counter()
    ev = HipEvents(2)
    ev.hip.hipEventRecord(ev.arr[0], stream)
    for _ in range(args.steps):
        step()
    ev.hip.hipEventRecord(ev.arr[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = ev.elapsed_ms(0, 1) / args.steps
    ev.close()
    tokens_heads = p.B * p.H * p.N
    value = tokens_heads / (ms * 1e-3)
    flops = 12.0 * p.M * p.D * tokens_heads
    mfma_frac = flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s), "
        f"{value / 1e9:.3f} G token*heads/s, {100 * mfma_frac:.1f}% of bf16 MFMA peak")

    # ---- fixed-query FLARE (Qd := S: one encode, one decode) on the same
    # inputs, K steps, for the route / FLARE time ratio
    fbytes = fp.flarepp_workspace_size(desc, fp.OP_FLARE)
    fws = torch.empty(max(fbytes, 1), dtype=torch.uint8, device="cuda")

    def flare_step():
        st = fp.flarepp_flare(desc, ptrs[0], ptrs[1], ptrs[2], ptrs[3], None, fws.data_ptr(), fbytes, stream)
        if st != 0:
            raise fp.FlareppError(st, "flarepp_flare")

    for _ in range(args.warmup):
        flare_step()
    torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.hip.hipEventRecord(ev.arr[0], stream)
    for _ in range(args.steps):
        flare_step()
    ev.hip.hipEventRecord(ev.arr[1], stream)
    torch.cuda.synchronize()
    flare_ms = ev.elapsed_ms(0, 1) / args.steps
    ev.close()
    del fws
    log(f"[bench] fixed-query FLARE: {flare_ms:.3f} ms/step; route / FLARE = {ms / flare_ms:.3f}")

    # ---- per-kernel durations: K more steps through flarepp_route_profiled
    max_l = 256
    kev = HipEvents(2 * max_l)
    kinds = (ctypes.c_int32 * max_l)()
    n_l = ctypes.c_int32(0)
    per_kind = {}
    for _ in range(args.steps):
        st = fp.flarepp_route_profiled(desc, ptrs[0], ptrs[1], ptrs[2], ptrs[3], None, None,
                                       ws.data_ptr(), nbytes, stream, kev.arr, kinds, max_l, n_l)
        if st != 0:
            raise fp.FlareppError(st, "flarepp_route_profiled")
        torch.cuda.synchronize()
        if n_l.value > max_l:
            raise RuntimeError("more launches than recorded events")
        for i in range(n_l.value):
            kind = fp.KERNEL_KINDS[kinds[i]]
            per_kind.setdefault(kind, []).append(kev.elapsed_ms(2 * i, 2 * i + 1))
    kev.close()
    launches_per_step = n_l.value
    G = max(1, launches_per_step and sum(1 for i in range(n_l.value) if kinds[i] == 4))
    heads_per_launch = (p.B * p.H) // G if G else p.B * p.H
    kstats = {}
    for kind, xs in per_kind.items():
        avg = sum(xs) / len(xs)
        kstats[kind] = {"launches_per_step": len(xs) // args.steps, "avg_us": 1e3 * avg,
                        "ms_per_step": sum(xs) / args.steps}
    for kind, st in sorted(kstats.items(), key=lambda kv: -kv[1]["ms_per_step"]):
        log(f"[bench]   {kind:12s} {st['launches_per_step']:3d} launches/step  avg {st['avg_us']:9.2f} us  "
            f"{st['ms_per_step']:.3f} ms/step")
    dom = max((k for k in kstats if per_token_bytes(k, p.D) > 0), key=lambda k: kstats[k]["ms_per_step"])
    units = heads_per_launch * p.N
    alg_bytes = per_token_bytes(dom, p.D) * units
    achieved = alg_bytes / (kstats[dom]["avg_us"] * 1e-6) / 1e9
    traffic = None
    tfile = os.path.join(PROFILES, f"traffic_{dom}_{p.name}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            rec = json.load(f)
        if rec.get("source_hash") == kernel_source_hash():
            traffic = rec.get("bytes_per_launch")
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": dom,
        "algorithmic_bytes_per_launch": alg_bytes,
        "avg_launch_us": round(kstats[dom]["avg_us"], 2),
    }

    # ---- backward of the route (float32): the same workload with float32
    # copies of the (bf16-valued) inputs and a seeded upstream dY
    bwd = None
    if args.backward_steps > 0:
        Sf, Kf, Vf = S.float(), K.float(), V.float()
        del Y
        dY = torch.randn(Kf.shape, generator=torch.Generator(device="cuda").manual_seed(7), device="cuda")
        dS, dK, dV = torch.empty_like(Sf), torch.empty_like(Kf), torch.empty_like(Vf)
        bdesc = fp.desc_for(Sf, Kf, p.scale)
        bbytes = fp.flarepp_workspace_size(bdesc, fp.OP_ROUTE_BACKWARD)
        bws = torch.empty(max(bbytes, 1), dtype=torch.uint8, device="cuda")
        bptr = [t.data_ptr() for t in (Sf, Kf, Vf, dY, dS, dK, dV)]

        def bstep():
            st = fp.flarepp_route_backward(bdesc, *bptr, bws.data_ptr(), bbytes, stream)
            if st != 0:
                raise fp.FlareppError(st, "flarepp_route_backward")

        bstep()
        torch.cuda.synchronize()
        ev = HipEvents(2)
        ev.hip.hipEventRecord(ev.arr[0], stream)
        for _ in range(args.backward_steps):
            bstep()
        ev.hip.hipEventRecord(ev.arr[1], stream)
        torch.cuda.synchronize()
        bms = ev.elapsed_ms(0, 1) / args.backward_steps
        ev.close()
        bflops = 30.0 * p.M * p.D * tokens_heads  # 3 stages x 10 M D (logits, dP, dV, dQ, dK)
        btf = bflops / (bms * 1e-3) / 1e12
        bwd = {
            "op": "flarepp_route_backward", "dtype": "f32",
            "workload": f"{p.name} shapes, float32 copies of the inputs, seeded dY",
            "steps": args.backward_steps, "ms_per_step": bms, "value": tokens_heads / (bms * 1e-3),
            "unit": "token*heads/s",
            "roofline": {"bound": "alu", "achieved": round(btf, 2), "peak": FP32_VECTOR_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(btf / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": None,
                         "algorithmic_flops_per_step": bflops},
        }
        log(f"[bench] backward (float32): {bms:.2f} ms/step, {btf:.2f} TFLOP/s algorithmic")
        del Sf, Kf, Vf, dY, dS, dK, dV, bws

    # ---- spectrum of every head's mixing matrix (bf16 inputs as the route)
    spec = None
    if args.spectrum_steps > 0:
        eig = torch.empty((p.B, p.H, p.M), dtype=torch.float32, device="cuda")
        sbytes = fp.flarepp_workspace_size(desc, fp.OP_SPECTRUM)
        sws = torch.empty(max(sbytes, 1), dtype=torch.uint8, device="cuda")

        def sstep():
            st = fp.flarepp_spectrum(desc, ptrs[0], ptrs[1], ptrs[2], eig.data_ptr(), None, sws.data_ptr(),
                                     sbytes, stream)
            if st != 0:
                raise fp.FlareppError(st, "flarepp_spectrum")

        sstep()
        torch.cuda.synchronize()
        ev = HipEvents(2)
        ev.hip.hipEventRecord(ev.arr[0], stream)
        for _ in range(args.spectrum_steps):
            sstep()
        ev.hip.hipEventRecord(ev.arr[1], stream)
        torch.cuda.synchronize()
        sms = ev.elapsed_ms(0, 1) / args.spectrum_steps
        ev.close()
        sflops = 2.0 * p.M * p.M * tokens_heads  # the M x M product F F^T over all tokens
        stf = sflops / (sms * 1e-3) / 1e12
        top = eig[:, :, :4].mean(dim=(0, 1)).tolist()
        spec = {"op": "flarepp_spectrum", "ms_per_step": sms, "steps": args.spectrum_steps,
                "gram_tflops": round(stf, 2), "fp32_vector_peak_tflops": FP32_VECTOR_PEAK_TFLOPS,
                "mean_top4_eigenvalues": [round(x, 6) for x in top]}
        log(f"[bench] spectrum: {sms:.2f} ms/step, Gram {stf:.2f} TFLOP/s; mean top eigenvalues {top}")
        del sws, eig

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
        "metric": "routed token*heads/s, fused route, N=1M M=256",
        "value": value,
        "unit": "token*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "B": p.B, "H": p.H, "N": p.N, "M": p.M, "D": p.D,
                   "scale": p.scale, "outputs": "fp32", "global_batch": p.B, "seq_len": p.N},
        "mfma_frac_of_bf16_peak": mfma_frac,
        "flare_fixed_query_ms_per_step": flare_ms,
        "route_over_flare": ms / flare_ms,
        "kernels": kstats,
        "roofline": roofline,
        "backward": bwd,
        "spectrum": spec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
