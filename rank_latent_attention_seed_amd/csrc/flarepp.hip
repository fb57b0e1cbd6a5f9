// libflarepp host side: argument validation, workspace planning and the
// launch sequences of the C ABI declared in include/flarepp.h.
//
// Launch sequence of the route for the bf16 path, per launch group of G
// (b, h) pairs (by default all of them: one launch per kernel, whose splits
// fill the GPU in one round):
//   encode  split-N seed encode (its query operands, c*S as bf16 hi/lo,
//           formed from S as it loads them), also records each split's max
//           key norm
//   merge   -> Qd (caller's copy, bf16 hi/lo operand, row norms, the bound for
//              the next encode)
//   encode  split-N encode with Qd
//   merge   -> Z (caller's copy, transposed bf16 operand)
//   decode  -> Y
// Everything is enqueued on the caller's stream; nothing synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "flarepp.h"
#include "common.h"
#include "decode_bf16.h"
#include "encode_bf16.h"
#include "f32_path.h"
#include "merge.h"
#include "backward_bf16.h"
#include "backward_f32.h"
#include "spectral.h"

using namespace flarepp;

namespace {

// Compute units the launch shapes target: those of the gfx950 products
// (MI350X, MI355X).  A constant rather than a device query, so that the split
// counts -- and with them the rounding of every result and the workspace
// size -- are a function of the descriptor alone, computable without a GPU.
constexpr int kComputeUnits = 256;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int64_t BH;
  int B, H, N, M, D, Mp;
  bool bf16;
  float c;          // scale * log2(e)
  float s;          // scale
  int G;            // heads per launch group
  int J, chunk;     // splits of N and tokens per split (encode)
  int nw, mbw;      // waves per workgroup and 16-latent blocks per wave (bf16 encode)
  int tpr;          // threads per latent row in the merge
  int dchunk;       // tokens per decode workgroup (bf16)
  bool dpair;       // paired decode (two waves per token block)
  // backward workspace regions
  size_t o_lse1, o_lse2, o_tlse, o_tdel, o_dz, o_dq3, o_dq, o_del;
  // bf16 backward: latent operands as bf16 (rows [G][Mp][D], transposed [.][D][Mt]),
  // Mt = M rounded up to 32, tokens per token-pass workgroup
  int Mt, tchunk;
  size_t o_zh, o_zl, o_dzr, o_dzl, o_dqr, o_dql, o_del1;
  // spectrum: Gram partials [G][Jg][M][M] over Jg token splits of gchunk, and the reduced [G][M][M]
  int Jg, gchunk;
  size_t o_gpart, o_mat;
  int nS;           // seed / fixed-query operand blocks (1 or H)
  // token-shard encodes: the stage's merge writes the shard's records here
  float* rec = nullptr;
  int rec_slot = 0, rec_nslots = 1;
  size_t o_shi, o_slo, o_sqn, o_part, o_knorm, o_qhi, o_qlo, o_qnorm, o_bias, o_zt, o_qf, o_zf, total;
};

// Tokens per decode workgroup at most: the workgroup's rows of Y (D <= 32
// float32) must fit a buffer resource's 32-bit byte count.
constexpr int64_t kMaxDecodeChunk = (int64_t(1) << 31) / (32 * 4) / 64 * 64;

flarepp_status check_desc(const flarepp_desc* d) {
  if (!d) return FLAREPP_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->N < 1 || d->M < 1 || d->D < 1) return FLAREPP_INVALID_ARG;
  if (!std::isfinite(d->scale)) return FLAREPP_INVALID_ARG;
  if (d->dtype != FLAREPP_F32 && d->dtype != FLAREPP_BF16) return FLAREPP_UNSUPPORTED;
  if (d->D != 16 && d->D != 32) return FLAREPP_UNSUPPORTED;
  if (d->M > FLAREPP_MAX_M) return FLAREPP_UNSUPPORTED;
  if (d->N >= FLAREPP_MAX_SLICE_ELEMS / d->D) return FLAREPP_UNSUPPORTED;
  if (d->B > (int64_t(1) << 31) / d->H) return FLAREPP_UNSUPPORTED;
  if (d->B * d->H > INT64_MAX / 8 / (d->N * d->D)) return FLAREPP_UNSUPPORTED;
  if (d->seed_head_stride != 0 && d->seed_head_stride != d->M * d->D) return FLAREPP_INVALID_ARG;
  return FLAREPP_OK;
}

flarepp_status check_tuning(const flarepp_tuning* t) {
  if (!t) return FLAREPP_OK;
  if (t->splits < 0 || t->head_group < 0 || t->decode_kernel < 0 || t->decode_wg_per_cu < 0)
    return FLAREPP_INVALID_ARG;
  if (t->decode_kernel > 2 || t->decode_wg_per_cu > 64) return FLAREPP_INVALID_ARG;
  return FLAREPP_OK;
}

// The launch plan and workspace layout of `op` for `d`; fields of `t` that are
// nonzero replace the library's choices (t may be null).
Plan make_plan(const flarepp_desc* d, int op, const flarepp_tuning* t = nullptr) {
  Plan p{};
  p.B = (int)d->B;
  p.H = (int)d->H;
  p.BH = d->B * d->H;
  p.N = (int)d->N;
  p.M = (int)d->M;
  p.D = (int)d->D;
  p.Mp = (int)cdiv(d->M, 16) * 16;
  p.bf16 = d->dtype == FLAREPP_BF16;
  p.c = d->scale * 1.4426950408889634f;
  p.s = d->scale;
  p.nS = d->seed_head_stride ? p.H : 1;

  // All heads in one launch group by default: larger launches have shorter
  // tails, and the split partials stay small because the split count per head
  // shrinks with the group (one round of encode workgroups per group).
  int64_t G = p.BH;
  if (t && t->head_group > 0) G = t->head_group;
  G = std::min<int64_t>(G, std::min<int64_t>(p.BH, 65535));
  p.G = (int)G;

  const int nMB = p.Mp / 16;
  // up to 128 latents: four waves; beyond: eight waves of two blocks each
  // (two blocks per wave keep a wave within the 128 registers of four
  // waves per SIMD)
  p.nw = nMB <= 8 ? 4 : 8;
  p.mbw = nMB <= 4 ? 1 : 2;
  // splits are whole encode tiles (8192 or 4096 bf16 of K per tile, by wave count)
  const int tile = p.bf16 ? (p.nw == 8 ? 8192 : 4096) / p.D : 64;
  // encode workgroups per head group: one round over the CUs, two
  // workgroups per CU (eight-wave ones: 64 KB of LDS and at most 128 VGPRs
  // per wave, four waves per SIMD)
  const int64_t target = (p.bf16 ? 2 : 4) * int64_t(kComputeUnits);
  int64_t J = std::max<int64_t>(1, cdiv(target, G));
  if (t && t->splits > 0) J = t->splits;
  J = std::min<int64_t>(J, cdiv(d->N, tile));
  const int64_t chunk = cdiv(cdiv(d->N, J), tile) * tile;
  p.chunk = (int)chunk;
  p.J = (int)cdiv(d->N, chunk);
  int tpr = 1;
  while (tpr < p.J && tpr < 64) tpr *= 2;
  p.tpr = tpr;
  // decode: beyond 8 latent blocks two waves share each token block (paired
  // kernel, eight 2-wave workgroups per CU); otherwise one 4-wave workgroup
  // per CU pair of SIMDs, 64-token rounds
  p.dpair = nMB > 8;
  if (t && t->decode_kernel > 0) p.dpair = nMB > 8 && t->decode_kernel == 1;
  if (p.dpair) {
    // eight 2-wave workgroups per CU: the fp16-logit form (<= 128 VGPRs)
    // holds them all at once, four waves per SIMD; the hi/lo form (three
    // waves per SIMD) takes them in one and a third rounds
    int per_cu = 8;
    if (t && t->decode_wg_per_cu > 0) per_cu = t->decode_wg_per_cu;
    const int64_t dwg = std::max<int64_t>(1, cdiv(per_cu * int64_t(kComputeUnits), G));
    p.dchunk = (int)std::min<int64_t>(cdiv(cdiv(d->N, dwg), 16) * 16, kMaxDecodeChunk);
  } else {
    const int64_t dwg = std::max<int64_t>(1, cdiv(2 * int64_t(kComputeUnits), G));
    p.dchunk = (int)std::min<int64_t>(cdiv(cdiv(d->N, dwg), 64) * 64, kMaxDecodeChunk);
  }

  // workspace layout
  const size_t G_ = (size_t)p.G, Mp = (size_t)p.Mp, D = (size_t)p.D;
  const size_t opnd = Mp * D * 2;  // one bf16 Mp x D block
  const bool route = op == FLAREPP_OP_ROUTE;
  const bool enc = op == FLAREPP_OP_ENCODE, dec = op == FLAREPP_OP_DECODE, flare = op == FLAREPP_OP_FLARE;
  const bool bwd = op == FLAREPP_OP_ROUTE_BACKWARD;
  const bool spec = op == FLAREPP_OP_SPECTRUM;
  {
    int64_t jg = std::max<int64_t>(1, cdiv(int64_t(kComputeUnits), G));
    jg = std::min<int64_t>(jg, cdiv(d->N, 32));
    p.gchunk = (int)(cdiv(cdiv(d->N, jg), 32) * 32);
    p.Jg = (int)cdiv(d->N, p.gchunk);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t none = SIZE_MAX;
  p.o_shi = p.o_slo = p.o_sqn = p.o_part = p.o_knorm = p.o_qhi = p.o_qlo = p.o_qnorm = p.o_bias =
      p.o_zt = p.o_qf = p.o_zf = none;
  p.o_lse1 = p.o_lse2 = p.o_tlse = p.o_tdel = p.o_dz = p.o_dq3 = p.o_dq = p.o_del = none;
  p.o_zh = p.o_zl = p.o_dzr = p.o_dzl = p.o_dqr = p.o_dql = p.o_del1 = none;
  p.Mt = (int)cdiv(d->M, 32) * 32;
  {
    // token passes of the bf16 backward: one workgroup per CU over the group
    const int64_t wgs = std::max<int64_t>(1, cdiv(int64_t(kComputeUnits), G));
    p.tchunk = (int)(cdiv(cdiv(d->N, wgs), 256) * 256);
  }
  p.o_gpart = p.o_mat = none;
  if (bwd && p.bf16) {
    p.o_shi = take(p.nS * opnd);
    p.o_slo = take(p.nS * opnd);
    p.o_part = take(G_ * p.J * Mp * std::max<size_t>(D + 4, 2 * D) * 4);
    p.o_knorm = take(G_ * p.J * 4);
    p.o_qhi = take(G_ * opnd);
    p.o_qlo = take(G_ * opnd);
    p.o_qnorm = take(G_ * Mp * 4);
    p.o_bias = take(G_ * Mp * 4);
    p.o_qf = take(G_ * p.M * D * 4);
    p.o_zf = take(G_ * p.M * D * 4);
    p.o_lse1 = take(G_ * Mp * 4);
    p.o_lse2 = take(G_ * Mp * 4);
    p.o_tlse = take(G_ * (size_t)cdiv(p.N, 4) * 16);
    p.o_tdel = take(G_ * (size_t)cdiv(p.N, 4) * 16);
    p.o_dz = take(G_ * p.M * D * 4);
    p.o_dq3 = take(G_ * p.M * D * 4);
    p.o_dq = take(G_ * p.M * D * 4);
    p.o_del = take(G_ * Mp * 4);
    p.o_zh = take(G_ * opnd);
    p.o_zl = take(G_ * opnd);
    p.o_del1 = take(G_ * Mp * 4);
    p.o_dzr = take(G_ * opnd);
    p.o_dzl = take(G_ * opnd);
    p.o_dqr = take(G_ * opnd);
    p.o_dql = take(G_ * opnd);
    p.o_zt = take(G_ * opnd);  // the decode of flarepp_route_save
  } else if (bwd) {
    p.o_part = take(G_ * p.J * Mp * std::max<size_t>(D + 4, 2 * D) * 4);
    p.o_qf = take(G_ * p.M * D * 4);
    p.o_zf = take(G_ * p.M * D * 4);
    p.o_lse1 = take(G_ * Mp * 4);
    p.o_lse2 = take(G_ * Mp * 4);
    p.o_tlse = take(G_ * (size_t)p.N * 4);
    p.o_tdel = take(G_ * (size_t)p.N * 4);
    p.o_dz = take(G_ * p.M * D * 4);
    p.o_dq3 = take(G_ * p.M * D * 4);
    p.o_dq = take(G_ * p.M * D * 4);
    p.o_del = take(G_ * Mp * 4);
  } else if (p.bf16) {
    if (flare) {
      p.o_shi = take(p.nS * opnd);
      p.o_slo = take(p.nS * opnd);
      p.o_sqn = take(p.nS * Mp * 4);
    }
    if (!dec) p.o_part = take(G_ * p.J * Mp * (D + 4) * 4);
    if (route || spec) p.o_knorm = take(G_ * p.J * 4);
    if (route || enc || dec || spec) {
      p.o_qhi = take(G_ * opnd);
      p.o_qlo = take(G_ * opnd);
    }
    if (route || dec || spec) p.o_qnorm = take(G_ * Mp * 4);
    if (route || spec) p.o_bias = take(G_ * Mp * 4);
    if (route || dec || flare) p.o_zt = take(G_ * opnd);
  } else {
    if (!dec) p.o_part = take(G_ * p.J * Mp * (D + 4) * 4);
    if (route) {
      p.o_qf = take(G_ * p.M * D * 4);
      p.o_zf = take(G_ * p.M * D * 4);
    }
    if (flare) p.o_zf = take(G_ * p.M * D * 4);
  }
  if (spec) {
    if (p.o_qf == none) p.o_qf = take(G_ * p.M * D * 4);
    p.o_lse2 = take(G_ * Mp * 4);
    if (!p.bf16) p.o_tlse = take(G_ * (size_t)p.N * 4);  // the bf16 path forms B_n in the Gram pass
    p.o_gpart = take(G_ * p.Jg * (size_t)p.M * p.M * 4);
    p.o_mat = take(G_ * (size_t)p.M * p.M * 4);
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return off == SIZE_MAX ? nullptr : reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

struct Range {
  uintptr_t lo, hi;
};
Range range(const void* p, size_t bytes) {
  return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Outputs must be disjoint from every input, from each other and from the
// workspace.  Null entries are skipped.
flarepp_status check_aliasing(const Range* outs, const void* const* outp, int nout, const Range* ins,
                              const void* const* inp, int nin) {
  for (int i = 0; i < nout; ++i) {
    if (!outp[i]) continue;
    for (int k = 0; k < nin; ++k)
      if (inp[k] && overlap(outs[i], ins[k])) return FLAREPP_ALIASING;
    for (int k = i + 1; k < nout; ++k)
      if (outp[k] && overlap(outs[i], outs[k])) return FLAREPP_ALIASING;
  }
  return FLAREPP_OK;
}

flarepp_status launched() {
  return hipGetLastError() == hipSuccess ? FLAREPP_OK : FLAREPP_HIP_ERROR;
}

// Optional per-launch event recording (flarepp_route_profiled); inert when
// `events` is null.
struct Recorder {
  void** events = nullptr;
  int32_t* kinds = nullptr;
  int32_t max = 0;
  int32_t n = 0;
  bool failed = false;
  void before(int kind, hipStream_t st) {
    if (events && n < max) {
      kinds[n] = kind;
      failed |= hipEventRecord(static_cast<hipEvent_t>(events[2 * n]), st) != hipSuccess;
    }
  }
  void after(hipStream_t st) {
    if (events && n < max) failed |= hipEventRecord(static_cast<hipEvent_t>(events[2 * n + 1]), st) != hipSuccess;
    ++n;
  }
};

#define FLAREPP_TRY(x)                          \
  do {                                          \
    const flarepp_status st_ = (x);             \
    if (st_ != FLAREPP_OK) return st_;          \
  } while (0)

// ------------------------------------------------------------- launchers --

template <int D>
flarepp_status run_prep(const Plan& p, const void* src, bool src_bf16, int64_t src_off, int64_t src_blk,
                        int nblk, __bf16* hi, __bf16* lo, __bf16* zt, float* qn, float c, hipStream_t st,
                        Recorder& rec) {
  PrepArgs a{src, src_bf16 ? 1 : 0, src_off, src_blk, nblk, p.M, p.Mp, hi, lo, zt, qn, c};
  const int64_t n = (int64_t)nblk * p.Mp * D;  // one thread per element
  rec.before(FLAREPP_KERNEL_PREP, st);
  prep_rows<D><<<dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st>>>(a);
  rec.after(st);
  return launched();
}

// EXQ: the query is the bf16 seeds themselves (a.q_seed set), an exact
// operand; otherwise the prepared hi/lo operand of c Qd (a.q_hi, a.q_lo).
template <int D, bool KNORM, bool BOUNDED, bool EXQ>
flarepp_status run_encode_bf16(const Plan& p, const EncodeArgs& a, int Gc, hipStream_t st, Recorder& rec,
                               int kind) {
  const dim3 grid((unsigned)p.J, (unsigned)Gc, (unsigned)cdiv(p.Mp / 16, p.nw * p.mbw));
  rec.before(kind, st);
  // the encodes that take a running max form P V in fp16 (see Pv)
  constexpr bool F16 = !BOUNDED;
  if (p.nw == 8)
    encode_split_bf16<D, 8, 2, KNORM, BOUNDED, F16, EXQ><<<grid, dim3(512), 0, st>>>(a);
  else if (p.mbw == 2)
    encode_split_bf16<D, 4, 2, KNORM, BOUNDED, F16, EXQ><<<grid, dim3(256), 0, st>>>(a);
  else
    encode_split_bf16<D, 4, 1, KNORM, BOUNDED, F16, EXQ><<<grid, dim3(256), 0, st>>>(a);
  rec.after(st);
  return launched();
}

template <int D>
flarepp_status run_encode_f32(const Plan& p, const EncodeF32Args& a, int Gc, hipStream_t st, Recorder& rec,
                              int kind) {
  const dim3 grid((unsigned)p.J, (unsigned)Gc, (unsigned)cdiv(p.M, 256));
  rec.before(kind, st);
  encode_split_f32<D><<<grid, dim3(256), 0, st>>>(a);
  rec.after(st);
  return launched();
}

template <int D>
flarepp_status run_merge(const Plan& p, const MergeArgs& a, int Gc, hipStream_t st, Recorder& rec) {
  rec.before(FLAREPP_KERNEL_MERGE, st);
  if (p.J > 64 && p.J <= 512) {  // one row per workgroup, records held in registers
    merge_rows256<D><<<dim3((unsigned)p.Mp, (unsigned)Gc), dim3(256), 0, st>>>(a);
    rec.after(st);
    return launched();
  }
  const int rpb = 256 / p.tpr;
  const dim3 grid((unsigned)cdiv(p.Mp, rpb), (unsigned)Gc);
  switch (p.tpr) {
    case 1: merge_partials<D, 1><<<grid, dim3(256), 0, st>>>(a); break;
    case 2: merge_partials<D, 2><<<grid, dim3(256), 0, st>>>(a); break;
    case 4: merge_partials<D, 4><<<grid, dim3(256), 0, st>>>(a); break;
    case 8: merge_partials<D, 8><<<grid, dim3(256), 0, st>>>(a); break;
    case 16: merge_partials<D, 16><<<grid, dim3(256), 0, st>>>(a); break;
    case 32: merge_partials<D, 32><<<grid, dim3(256), 0, st>>>(a); break;
    default: merge_partials<D, 64><<<grid, dim3(256), 0, st>>>(a); break;
  }
  rec.after(st);
  return launched();
}

template <int D, int MB>
void launch_decode_mb(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  decode_bf16<D, MB><<<grid, dim3(256), 0, st>>>(a);
}

template <int D, bool Q16>
void launch_decode_pair(int mbh, bool ragged, const DecodeArgs& a, dim3 grid, hipStream_t st) {
  if (!ragged) {
    switch (mbh) {
      case 5: decode_pair_bf16<D, 5, false, Q16><<<grid, dim3(128), 0, st>>>(a); break;
      case 6: decode_pair_bf16<D, 6, false, Q16><<<grid, dim3(128), 0, st>>>(a); break;
      case 7: decode_pair_bf16<D, 7, false, Q16><<<grid, dim3(128), 0, st>>>(a); break;
      default: decode_pair_bf16<D, 8, false, Q16><<<grid, dim3(128), 0, st>>>(a); break;
    }
  } else {
    switch (mbh) {
      case 5: decode_pair_bf16<D, 5, true, Q16><<<grid, dim3(128), 0, st>>>(a); break;
      case 6: decode_pair_bf16<D, 6, true, Q16><<<grid, dim3(128), 0, st>>>(a); break;
      case 7: decode_pair_bf16<D, 7, true, Q16><<<grid, dim3(128), 0, st>>>(a); break;
      default: decode_pair_bf16<D, 8, true, Q16><<<grid, dim3(128), 0, st>>>(a); break;
    }
  }
}

template <int D>
flarepp_status run_decode_bf16(const Plan& p, const DecodeArgs& a, int Gc, hipStream_t st, Recorder& rec) {
  const dim3 grid((unsigned)cdiv(p.N, p.dchunk), (unsigned)Gc);
  rec.before(FLAREPP_KERNEL_DECODE, st);
  if (p.dpair) {
    // the hi/lo form for heads outside the fp16 bound, then the fp16 form
    // (only the route passes the key norms that bound; without them every
    // head takes the hi/lo form)
    const int mbh = (p.Mp / 16 + 1) / 2;
    const bool ragged = p.M != 2 * mbh * 16;
    launch_decode_pair<D, false>(mbh, ragged, a, grid, st);
    if (a.knorm) launch_decode_pair<D, true>(mbh, ragged, a, grid, st);
    rec.after(st);
    return launched();
  }
  switch (p.Mp / 16) {
    case 1: launch_decode_mb<D, 1>(a, grid, st); break;
    case 2: launch_decode_mb<D, 2>(a, grid, st); break;
    case 3: launch_decode_mb<D, 3>(a, grid, st); break;
    case 4: launch_decode_mb<D, 4>(a, grid, st); break;
    case 5: launch_decode_mb<D, 5>(a, grid, st); break;
    case 6: launch_decode_mb<D, 6>(a, grid, st); break;
    case 7: launch_decode_mb<D, 7>(a, grid, st); break;
    case 8: launch_decode_mb<D, 8>(a, grid, st); break;
    case 9: launch_decode_mb<D, 9>(a, grid, st); break;
    case 10: launch_decode_mb<D, 10>(a, grid, st); break;
    case 11: launch_decode_mb<D, 11>(a, grid, st); break;
    case 12: launch_decode_mb<D, 12>(a, grid, st); break;
    case 13: launch_decode_mb<D, 13>(a, grid, st); break;
    case 14: launch_decode_mb<D, 14>(a, grid, st); break;
    case 15: launch_decode_mb<D, 15>(a, grid, st); break;
    default: launch_decode_mb<D, 16>(a, grid, st); break;
  }
  rec.after(st);
  return launched();
}

template <int D>
flarepp_status run_decode_f32(const Plan& p, const DecodeF32Args& a, int Gc, hipStream_t st, Recorder& rec) {
  const dim3 grid((unsigned)cdiv(p.N, 256), (unsigned)Gc);
  rec.before(FLAREPP_KERNEL_DECODE, st);
  decode_f32<D><<<grid, dim3(256), (size_t)2 * p.M * D * sizeof(float), st>>>(a);
  rec.after(st);
  return launched();
}

MergeArgs merge_args(const Plan& p, void* ws, int64_t g0) {
  MergeArgs m{};
  m.part = at<float>(ws, p.o_part);
  m.J = p.J;
  m.Mp = p.Mp;
  m.M = p.M;
  m.bh0 = g0;
  m.c = p.c;
  m.rec_out = p.rec;
  m.rec_slot = p.rec_slot;
  m.rec_nslots = p.rec_nslots;
  return m;
}

// The merge of an encode with fp16 weights recomputes any record whose sum
// overflowed (merge.h, refit_record): it needs that encode's operands.
void refit_from(MergeArgs& m, const EncodeArgs& e) {
  m.fq_hi = e.q_hi;
  m.fq_lo = e.q_lo;
  m.fq_seed = e.q_seed;
  m.fq_c = e.qc;
  m.fq_sb = e.q_sb;
  m.fq_sh = e.q_sh;
  m.fq_off = e.q_off;
  m.fK = e.K;
  m.fV = e.V;
  m.H = e.H;
  m.N = e.N;
  m.chunk = e.chunk;
}

EncodeArgs encode_args(const Plan& p, void* ws, const void* K, const void* V, int64_t g0) {
  EncodeArgs e{};
  e.K = static_cast<const __bf16*>(K);
  e.V = static_cast<const __bf16*>(V);
  e.part = at<float>(ws, p.o_part);
  e.H = p.H;
  e.N = p.N;
  e.Mp = p.Mp;
  e.J = p.J;
  e.chunk = p.chunk;
  e.bh0 = g0;
  return e;
}

// ---------------------------------------------------------------- stages --

enum Stage { kSeed, kEncode, kDecode, kRoute, kFlare, kSpectrum };

// Spectrum of one launch group (stages 1 and 2 already ran: Qd rows in the
// o_qf staging buffer and, for bf16 inputs, c * Qd as bf16 hi/lo in
// o_qhi / o_qlo; the encode's log-sum-exp in o_lse2).
template <int D, typename KT>
flarepp_status run_spectral(const Plan& p, const void* K, int64_t g0, int Gc, void* ws, float* eig, float* sym_out,
                            hipStream_t st) {
  float* gpart = at<float>(ws, p.o_gpart);
  float* mat = at<float>(ws, p.o_mat);
  const float* lse = at<float>(ws, p.o_lse2);
  if constexpr (std::is_same<KT, __bf16>::value) {
    SpecMfmaArgs g{at<__bf16>(ws, p.o_qhi), at<__bf16>(ws, p.o_qlo), static_cast<const __bf16*>(K), lse, gpart,
                   p.N, p.M, p.Mp, p.Jg, p.gchunk, g0};
    spectral_gram_mfma<D><<<dim3((unsigned)p.Jg, (unsigned)Gc), 512, 0, st>>>(g);
    FLAREPP_TRY(launched());
  } else {
    float* qf = at<float>(ws, p.o_qf);
    float* tlse = at<float>(ws, p.o_tlse);
    SpecTokArgs t{qf, K, tlse, p.H, p.N, p.M, g0, p.c};
    spectral_tokens<D, KT><<<dim3((unsigned)cdiv(p.N, 256), (unsigned)Gc), 256, 0, st>>>(t);
    FLAREPP_TRY(launched());
    SpecGramArgs g{qf, K, lse, tlse, gpart, p.H, p.N, p.M, p.Mp, p.Jg, p.gchunk, g0, p.c};
    spectral_gram<D, KT><<<dim3((unsigned)p.Jg, (unsigned)Gc), 1024, 0, st>>>(g);
    FLAREPP_TRY(launched());
  }
  SpecReduceArgs r{gpart, mat, sym_out, Gc, p.Jg, p.M, g0};
  spectral_reduce<<<(unsigned)cdiv((int64_t)Gc * p.M * p.M, 256), 256, 0, st>>>(r);
  FLAREPP_TRY(launched());
  EigArgs e{mat, eig, p.M, g0};
  tridiag_eigvals<<<(unsigned)Gc, 1024, 0, st>>>(e);
  return launched();
}

template <int D>
flarepp_status run(const Plan& p, Stage stage, const void* S, const float* Qd_in, const float* Z_in,
                   const void* K, const void* V, float* Y, float* Qd_out, float* Z_out, void* ws,
                   hipStream_t st, Recorder& rec) {
  const int64_t MD = (int64_t)p.M * D, MpD = (int64_t)p.Mp * D;
  const int64_t seed_h = p.nS > 1 ? MD : 0;
  if (p.bf16) {
    __bf16* shi = at<__bf16>(ws, p.o_shi);
    __bf16* slo = at<__bf16>(ws, p.o_slo);
    // FLARE's decode takes c S as its key operand; the other stages form the
    // seed encode's query operands from S inside the encode
    if (stage == kFlare)
      FLAREPP_TRY(run_prep<D>(p, S, true, 0, seed_h, p.nS, shi, slo, nullptr, at<float>(ws, p.o_sqn), p.c, st, rec));
    for (int64_t g0 = 0; g0 < p.BH; g0 += p.G) {
      const int Gc = (int)std::min<int64_t>(p.G, p.BH - g0);
      __bf16* qhi = at<__bf16>(ws, p.o_qhi);
      __bf16* qlo = at<__bf16>(ws, p.o_qlo);
      __bf16* zt = at<__bf16>(ws, p.o_zt);
      float* qnorm = at<float>(ws, p.o_qnorm);
      const bool routed = stage == kRoute || stage == kSpectrum;  // stages 1 and 2 as in the route
      if (stage == kSeed || routed || stage == kFlare) {
        EncodeArgs e = encode_args(p, ws, K, V, g0);
        // the seeds are the exact query operand, scaled by c in the encode
        e.q_seed = static_cast<const __bf16*>(S);
        e.qc = p.c;
        e.M = p.M;
        e.q_sb = 0;
        e.q_sh = seed_h;
        e.q_off = 0;
        e.knorm = at<float>(ws, p.o_knorm);
        if (routed)
          FLAREPP_TRY((run_encode_bf16<D, true, false, true>(p, e, Gc, st, rec, FLAREPP_KERNEL_SEED_ENCODE)));
        else
          FLAREPP_TRY((run_encode_bf16<D, false, false, true>(p, e, Gc, st, rec, FLAREPP_KERNEL_SEED_ENCODE)));
        MergeArgs m = merge_args(p, ws, g0);
        refit_from(m, e);  // an encode with fp16 weights (see run_encode_bf16)
        if (stage == kFlare) {
          m.out = Z_out;
          m.op_zt = zt;
        } else {
          m.out = Qd_out;
          if (stage == kSpectrum) m.outl = at<float>(ws, p.o_qf);
          if (routed) {
            m.op_hi = qhi;
            m.op_lo = qlo;
            m.qnorm = qnorm;
            m.knorm = e.knorm;
            m.Jk = p.J;
            m.bias = at<float>(ws, p.o_bias);
          }
        }
        FLAREPP_TRY(run_merge<D>(p, m, Gc, st, rec));
      }
      if (stage == kEncode)
        FLAREPP_TRY(run_prep<D>(p, Qd_in, false, g0 * MD, MD, Gc, qhi, qlo, nullptr, nullptr, p.c, st, rec));
      if (stage == kEncode || routed) {
        EncodeArgs e = encode_args(p, ws, K, V, g0);
        e.q_hi = qhi;
        e.q_lo = qlo;
        e.q_sb = (int64_t)p.H * MpD;
        e.q_sh = MpD;
        e.q_off = g0 * MpD;
        e.bias = routed ? at<float>(ws, p.o_bias) : nullptr;
        if (stage == kRoute) {  // the head's logit bound may pick fp16 logits (f16_logits)
          e.kin = at<float>(ws, p.o_knorm);
          e.Jk = p.J;
          e.qnorm = qnorm;
          e.qc = p.c;
        }
        if (routed)
          FLAREPP_TRY((run_encode_bf16<D, false, true, false>(p, e, Gc, st, rec, FLAREPP_KERNEL_ENCODE)));
        else
          FLAREPP_TRY((run_encode_bf16<D, false, false, false>(p, e, Gc, st, rec, FLAREPP_KERNEL_ENCODE)));
        MergeArgs m = merge_args(p, ws, g0);
        if (!routed) refit_from(m, e);  // the stand-alone encode has fp16 weights, the routed one bf16
        m.out = stage == kSpectrum ? nullptr : Z_out;  // (Z_out carries the spectrum's matrix output)
        if (stage == kRoute) m.op_zt = zt;
        if (stage == kSpectrum) m.lse = at<float>(ws, p.o_lse2);
        FLAREPP_TRY(run_merge<D>(p, m, Gc, st, rec));
      }
      if (stage == kSpectrum)  // Y carries the eigenvalue output, Z_out the optional matrix
        FLAREPP_TRY((run_spectral<D, __bf16>(p, K, g0, Gc, ws, Y, Z_out, st)));
      if (stage == kDecode) {
        FLAREPP_TRY(run_prep<D>(p, Qd_in, false, g0 * MD, MD, Gc, qhi, qlo, nullptr, qnorm, p.c, st, rec));
        FLAREPP_TRY(run_prep<D>(p, Z_in, false, g0 * MD, MD, Gc, nullptr, nullptr, zt, nullptr, p.c, st, rec));
      }
      if (stage == kDecode || stage == kRoute || stage == kFlare) {
        DecodeArgs dargs{};
        if (stage == kFlare) {
          dargs.q_hi = shi;
          dargs.q_lo = slo;
          dargs.q_sb = 0;
          dargs.q_sh = p.nS > 1 ? MpD : 0;
          dargs.q_off = 0;
          dargs.qnorm = at<float>(ws, p.o_sqn);
        } else {
          dargs.q_hi = qhi;
          dargs.q_lo = qlo;
          dargs.q_sb = (int64_t)p.H * MpD;
          dargs.q_sh = MpD;
          dargs.q_off = g0 * MpD;
          dargs.qnorm = qnorm;
          if (stage == kRoute) {  // split key norms of the seed encode
            dargs.knorm = at<float>(ws, p.o_knorm);
            dargs.Jk = p.J;
          }
        }
        dargs.zt = zt;
        dargs.K = static_cast<const __bf16*>(K);
        dargs.Y = Y;
        dargs.H = p.H;
        dargs.N = p.N;
        dargs.M = p.M;
        dargs.Mp = p.Mp;
        dargs.chunk = p.dchunk;
        dargs.bh0 = g0;
        dargs.c = p.c;
        FLAREPP_TRY(run_decode_bf16<D>(p, dargs, Gc, st, rec));
      }
    }
    return FLAREPP_OK;
  }

  // float32 path
  float* qf = at<float>(ws, p.o_qf);
  float* zf = at<float>(ws, p.o_zf);
  for (int64_t g0 = 0; g0 < p.BH; g0 += p.G) {
    const int Gc = (int)std::min<int64_t>(p.G, p.BH - g0);
    auto encode = [&](const float* q, int64_t sb, int64_t sh, int64_t off, float* out, float* outl, int kind,
                      float* lse = nullptr) {
      EncodeF32Args e{};
      e.q = q;
      e.q_sb = sb;
      e.q_sh = sh;
      e.q_off = off;
      e.K = static_cast<const float*>(K);
      e.V = static_cast<const float*>(V);
      e.part = at<float>(ws, p.o_part);
      e.H = p.H;
      e.N = p.N;
      e.M = p.M;
      e.Mp = p.Mp;
      e.J = p.J;
      e.chunk = p.chunk;
      e.bh0 = g0;
      e.c = p.c;
      FLAREPP_TRY(run_encode_f32<D>(p, e, Gc, st, rec, kind));
      MergeArgs m = merge_args(p, ws, g0);
      m.out = out;
      m.outl = outl;
      m.lse = lse;
      return run_merge<D>(p, m, Gc, st, rec);
    };
    auto decode = [&](const float* q, int64_t qsb, int64_t qsh, int64_t qoff, const float* z, int64_t zsb,
                      int64_t zsh, int64_t zoff) {
      DecodeF32Args d{q, qsb, qsh, qoff, z, zsb, zsh, zoff, static_cast<const float*>(K), Y,
                      p.H, p.N, p.M, g0, p.c};
      return run_decode_f32<D>(p, d, Gc, st, rec);
    };
    const float* Sf = static_cast<const float*>(S);
    const int64_t HMD = (int64_t)p.H * MD;
    switch (stage) {
      case kSeed:
        FLAREPP_TRY(encode(Sf, 0, seed_h, 0, Qd_out, nullptr, FLAREPP_KERNEL_SEED_ENCODE));
        break;
      case kEncode:
        FLAREPP_TRY(encode(Qd_in, HMD, MD, 0, Z_out, nullptr, FLAREPP_KERNEL_ENCODE));
        break;
      case kDecode:
        FLAREPP_TRY(decode(Qd_in, HMD, MD, 0, Z_in, HMD, MD, 0));
        break;
      case kRoute:
        FLAREPP_TRY(encode(Sf, 0, seed_h, 0, Qd_out, qf, FLAREPP_KERNEL_SEED_ENCODE));
        FLAREPP_TRY(encode(qf, HMD, MD, g0 * MD, Z_out, zf, FLAREPP_KERNEL_ENCODE));
        FLAREPP_TRY(decode(qf, HMD, MD, g0 * MD, zf, HMD, MD, g0 * MD));
        break;
      case kFlare:
        FLAREPP_TRY(encode(Sf, 0, seed_h, 0, Z_out, zf, FLAREPP_KERNEL_ENCODE));
        FLAREPP_TRY(decode(Sf, 0, seed_h, 0, zf, HMD, MD, g0 * MD));
        break;
      case kSpectrum:
        FLAREPP_TRY(encode(Sf, 0, seed_h, 0, nullptr, qf, FLAREPP_KERNEL_SEED_ENCODE));
        FLAREPP_TRY(encode(qf, HMD, MD, g0 * MD, nullptr, nullptr, FLAREPP_KERNEL_ENCODE,
                           at<float>(ws, p.o_lse2)));
        FLAREPP_TRY((run_spectral<D, float>(p, K, g0, Gc, ws, Y, Z_out, st)));
        break;
    }
  }
  return FLAREPP_OK;
}

// Backward of the route (float32): the forward's stages 1 and 2 with their
// log-sum-exp statistics, then per stage a token pass (dK, dV) and a latent
// pass (split partials of the latent gradients) with their reduction, in
// reverse order.
template <int D>
flarepp_status run_backward(const Plan& p, const float* S, const float* K, const float* V, const float* dY,
                            float* dS, float* dK, float* dV, void* ws, hipStream_t st) {
  Recorder rec;
  const int64_t MD = (int64_t)p.M * D, HMD = (int64_t)p.H * MD;
  const int64_t seed_h = p.nS > 1 ? MD : 0;
  const int nz = (int)cdiv((int64_t)p.nS * MD, 256);
  fill_zero<<<nz, 256, 0, st>>>(dS, (int64_t)p.nS * MD);
  FLAREPP_TRY(launched());
  float* qf = at<float>(ws, p.o_qf);
  float* zf = at<float>(ws, p.o_zf);
  float* part = at<float>(ws, p.o_part);
  float* dz = at<float>(ws, p.o_dz);
  float* dq3 = at<float>(ws, p.o_dq3);
  float* dq = at<float>(ws, p.o_dq);
  float* del = at<float>(ws, p.o_del);
  for (int64_t g0 = 0; g0 < p.BH; g0 += p.G) {
    const int Gc = (int)std::min<int64_t>(p.G, p.BH - g0);
    // ---- forward stages 1 and 2 with statistics
    auto encode = [&](const float* q, int64_t sb, int64_t sh, int64_t off, float* outl, float* lse) {
      EncodeF32Args e{};
      e.q = q;
      e.q_sb = sb;
      e.q_sh = sh;
      e.q_off = off;
      e.K = K;
      e.V = V;
      e.part = part;
      e.H = p.H;
      e.N = p.N;
      e.M = p.M;
      e.Mp = p.Mp;
      e.J = p.J;
      e.chunk = p.chunk;
      e.bh0 = g0;
      e.c = p.c;
      FLAREPP_TRY(run_encode_f32<D>(p, e, Gc, st, rec, FLAREPP_KERNEL_ENCODE));
      MergeArgs m = merge_args(p, ws, g0);
      m.outl = outl;
      m.lse = lse;
      return run_merge<D>(p, m, Gc, st, rec);
    };
    FLAREPP_TRY(encode(S, 0, seed_h, 0, qf, at<float>(ws, p.o_lse1)));
    FLAREPP_TRY(encode(qf, HMD, MD, g0 * MD, zf, at<float>(ws, p.o_lse2)));

    const dim3 tok_grid((unsigned)cdiv(p.N, 256), (unsigned)Gc);
    const dim3 lat_grid((unsigned)p.J, (unsigned)Gc, (unsigned)cdiv(p.M, 256));
    auto reduce = [&](int R, int field0, const float* add_to, float* out, const float* dot_with, float* delta,
                      int seed_blocks) {
      BwdReduceArgs r{part, p.J, R, field0, p.M, p.Mp, Gc, p.H, g0, add_to, out, dot_with, delta, seed_blocks};
      const int64_t rows = (int64_t)(seed_blocks ? seed_blocks : Gc) * p.M;
      bwd_reduce<D><<<(unsigned)cdiv(rows * D, 256), 256, 0, st>>>(r);
      return launched();
    };
    // ---- stage 3 (decode): queries K, keys Qd, values Z
    {
      BwdTokArgs t{};
      t.q = qf;
      t.q_sb = HMD;
      t.q_sh = MD;
      t.q_off = g0 * MD;
      t.lat2 = zf;
      t.K = K;
      t.dY = dY;
      t.dK = dK;
      t.tlse = at<float>(ws, p.o_tlse);
      t.tdelta = at<float>(ws, p.o_tdel);
      t.H = p.H;
      t.N = p.N;
      t.M = p.M;
      t.Mp = p.Mp;
      t.bh0 = g0;
      t.c = p.c;
      t.s = p.s;
      t.acc_dk = 0;
      t.acc_dv = 0;
      bwd_decode_tokens<D><<<tok_grid, 256, 0, st>>>(t);
      FLAREPP_TRY(launched());
      BwdLatArgs l{};
      l.q = qf;
      l.q_sb = HMD;
      l.q_sh = MD;
      l.q_off = g0 * MD;
      l.lat2 = zf;
      l.K = K;
      l.dY = dY;
      l.tlse = t.tlse;
      l.tdelta = t.tdelta;
      l.part = part;
      l.H = p.H;
      l.N = p.N;
      l.M = p.M;
      l.Mp = p.Mp;
      l.J = p.J;
      l.chunk = p.chunk;
      l.bh0 = g0;
      l.c = p.c;
      l.s = p.s;
      bwd_latents<D, true><<<lat_grid, 256, 0, st>>>(l);
      FLAREPP_TRY(launched());
      FLAREPP_TRY(reduce(2 * D, D, nullptr, dz, zf, del, 0));    // dZ, delta_2 = <dZ, Z>
      FLAREPP_TRY(reduce(2 * D, 0, nullptr, dq3, nullptr, nullptr, 0));  // dQd from the decode
    }
    // ---- stages 2 and 1 (encode, seed encode)
    auto enc_stage = [&](const float* q, int64_t sb, int64_t sh, int64_t off, const float* dO, const float* lse,
                         int accumulate_dv) {
      BwdTokArgs t{};
      t.q = q;
      t.q_sb = sb;
      t.q_sh = sh;
      t.q_off = off;
      t.lat2 = dO;
      t.lse = lse;
      t.delta = del;
      t.K = K;
      t.V = V;
      t.dK = dK;
      t.dV = dV;
      t.H = p.H;
      t.N = p.N;
      t.M = p.M;
      t.Mp = p.Mp;
      t.bh0 = g0;
      t.c = p.c;
      t.s = p.s;
      t.acc_dk = 1;  // the decode wrote dK first
      t.acc_dv = accumulate_dv;
      bwd_encode_tokens<D><<<tok_grid, 256, 0, st>>>(t);
      FLAREPP_TRY(launched());
      BwdLatArgs l{};
      l.q = q;
      l.q_sb = sb;
      l.q_sh = sh;
      l.q_off = off;
      l.lat2 = dO;
      l.lse = lse;
      l.delta = del;
      l.K = K;
      l.V = V;
      l.part = part;
      l.H = p.H;
      l.N = p.N;
      l.M = p.M;
      l.Mp = p.Mp;
      l.J = p.J;
      l.chunk = p.chunk;
      l.bh0 = g0;
      l.c = p.c;
      l.s = p.s;
      bwd_latents<D, false><<<lat_grid, 256, 0, st>>>(l);
      return launched();
    };
    FLAREPP_TRY(enc_stage(qf, HMD, MD, g0 * MD, dz, at<float>(ws, p.o_lse2), 0));
    FLAREPP_TRY(reduce(D, 0, dq3, dq, qf, del, 0));  // dQd = encode + decode parts, delta_1 = <dQd, Qd>
    FLAREPP_TRY(enc_stage(S, 0, seed_h, 0, dq, at<float>(ws, p.o_lse1), 1));
    FLAREPP_TRY(reduce(D, 0, nullptr, dS, nullptr, nullptr, p.nS));
  }
  return FLAREPP_OK;
}

// The forward stages 1 and 2 of the backward (and of flarepp_route_save) for
// one launch group: the seed encode with c S as the bf16 hi/lo operand that
// the backward's stage-1 passes also take, merge (Qd to qd_out, staged c Qd
// hi/lo operands, norms, bounds, stage 1's log-sum-exp), the encode with the
// hi/lo query (the backward's stage-2 logits), merge (Z to z_out, its
// log-sum-exp, and Z^T for a decode when zt is set).
template <int D>
flarepp_status forward_for_backward(const Plan& p, const void* K, const void* V, void* ws, int64_t g0, int Gc,
                                    float* qd_out, float* qd_stage, float* z_out, float* z_stage, float* lse1,
                                    float* lse2, __bf16* zt, hipStream_t st, Recorder& rec) {
  const int64_t MpD = (int64_t)p.Mp * D;
  EncodeArgs e = encode_args(p, ws, K, V, g0);
  e.q_hi = at<__bf16>(ws, p.o_shi);
  e.q_lo = at<__bf16>(ws, p.o_slo);
  e.q_sb = 0;
  e.q_sh = p.nS > 1 ? MpD : 0;
  e.q_off = 0;
  e.knorm = at<float>(ws, p.o_knorm);
  FLAREPP_TRY((run_encode_bf16<D, true, false, false>(p, e, Gc, st, rec, FLAREPP_KERNEL_SEED_ENCODE)));
  MergeArgs m = merge_args(p, ws, g0);
  refit_from(m, e);
  m.out = qd_out;
  m.outl = qd_stage;
  m.op_hi = at<__bf16>(ws, p.o_qhi);
  m.op_lo = at<__bf16>(ws, p.o_qlo);
  m.qnorm = at<float>(ws, p.o_qnorm);
  m.knorm = e.knorm;
  m.Jk = p.J;
  m.bias = at<float>(ws, p.o_bias);
  m.lse = lse1;
  FLAREPP_TRY(run_merge<D>(p, m, Gc, st, rec));
  EncodeArgs e2 = encode_args(p, ws, K, V, g0);
  e2.q_hi = m.op_hi;
  e2.q_lo = m.op_lo;
  e2.q_sb = (int64_t)p.H * MpD;
  e2.q_sh = MpD;
  e2.q_off = g0 * MpD;
  e2.bias = m.bias;
  FLAREPP_TRY((run_encode_bf16<D, false, true, false>(p, e2, Gc, st, rec, FLAREPP_KERNEL_ENCODE)));
  MergeArgs m2 = merge_args(p, ws, g0);
  m2.out = z_out;
  m2.outl = z_stage;
  m2.lse = lse2;
  m2.op_zt = zt;
  return run_merge<D>(p, m2, Gc, st, rec);
}

// Backward of the route (bf16 inputs, matrix cores): the forward's stages 1
// and 2 (forward_for_backward), keeping Qd, Z and the log-sum-exp of both
// encodes, or those of a saved forward; then per stage in reverse order the
// token pass (dK, dV), the latent pass (split partials) and their
// reduction, with the latent operands of each stage converted to bf16 rows
// and transposes first.
// saved (flarepp_route_backward_saved): Qd, Z and both log-sum-exps from
// flarepp_route_save instead of recomputing stages 1 and 2; null otherwise.
struct SavedForward {
  const float* Qd;   // [BH][M][D]
  const float* Z;    // [BH][M][D]
  const float* lse;  // [2][BH][Mp]
};

template <int D>
flarepp_status run_backward_bf16(const Plan& p, const void* S, const void* K, const void* V, const float* dY,
                                 float* dS, float* dK, float* dV, void* ws, hipStream_t st,
                                 const SavedForward* saved = nullptr) {
  Recorder rec;
  const int64_t MD = (int64_t)p.M * D, MpD = (int64_t)p.Mp * D;
  const int64_t seed_h = p.nS > 1 ? MD : 0;
  fill_zero<<<(unsigned)cdiv((int64_t)p.nS * MD, 256), 256, 0, st>>>(dS, (int64_t)p.nS * MD);
  FLAREPP_TRY(launched());
  __bf16* shi = at<__bf16>(ws, p.o_shi);
  __bf16* slo = at<__bf16>(ws, p.o_slo);
  __bf16* qhi = at<__bf16>(ws, p.o_qhi);
  __bf16* qlo = at<__bf16>(ws, p.o_qlo);
  float* part = at<float>(ws, p.o_part);
  float* dz = at<float>(ws, p.o_dz);
  float* dq3 = at<float>(ws, p.o_dq3);
  float* dq = at<float>(ws, p.o_dq);
  float* del = at<float>(ws, p.o_del);
  __bf16* zh = at<__bf16>(ws, p.o_zh);
  __bf16* zl = at<__bf16>(ws, p.o_zl);
  __bf16* dzr = at<__bf16>(ws, p.o_dzr);
  __bf16* dzl = at<__bf16>(ws, p.o_dzl);
  __bf16* dqr = at<__bf16>(ws, p.o_dqr);
  __bf16* dql = at<__bf16>(ws, p.o_dql);
  auto prep = [&](const void* src, bool src_bf16, int64_t src_blk, int nblk, bool center, float alpha, __bf16* hi,
                  __bf16* lo, __bf16* tr) {
    BwdPrepArgs a{src, src_bf16 ? 1 : 0, src_blk, p.M, p.Mp, p.Mt, center ? 1 : 0, alpha, hi, lo, tr};
    bwd_prep_bf16<D><<<(unsigned)nblk, 256, 0, st>>>(a);
    return launched();
  };
  // seed operands (c S as hi/lo for the forward, S^T for stage 1's dK)
  FLAREPP_TRY(run_prep<D>(p, S, true, 0, seed_h, p.nS, shi, slo, nullptr, nullptr, p.c, st, rec));
  for (int64_t g0 = 0; g0 < p.BH; g0 += p.G) {
    const int Gc = (int)std::min<int64_t>(p.G, p.BH - g0);
    // ---- forward stages 1 and 2 (recomputed, or from the saved forward)
    const float* qf;
    const float* zf;
    float* lse1;
    float* lse2;
    if (saved) {
      qf = saved->Qd + g0 * MD;
      zf = saved->Z + g0 * MD;
      lse1 = const_cast<float*>(saved->lse) + g0 * p.Mp;
      lse2 = const_cast<float*>(saved->lse) + (p.BH + g0) * p.Mp;
      FLAREPP_TRY(run_prep<D>(p, saved->Qd, false, g0 * MD, MD, Gc, qhi, qlo, nullptr, at<float>(ws, p.o_qnorm), p.c,
                              st, rec));
    } else {
      float* qs = at<float>(ws, p.o_qf);
      float* zs = at<float>(ws, p.o_zf);
      lse1 = at<float>(ws, p.o_lse1);
      lse2 = at<float>(ws, p.o_lse2);
      FLAREPP_TRY(forward_for_backward<D>(p, K, V, ws, g0, Gc, nullptr, qs, nullptr, zs, lse1, lse2, nullptr, st, rec));
      qf = qs;
      zf = zs;
    }
    auto reduce = [&](int R, int field0, const float* add_to, float* out, const float* dot_with, float* delta,
                      int seed_blocks) {
      BwdReduceArgs r{part, p.J, R, field0, p.M, p.Mp, Gc, p.H, g0, add_to, out, dot_with, delta, seed_blocks};
      const int64_t rows = (int64_t)(seed_blocks ? seed_blocks : Gc) * p.M;
      bwd_reduce<D><<<(unsigned)cdiv(rows * D, 256), 256, 0, st>>>(r);
      return launched();
    };
    const dim3 tok_grid((unsigned)cdiv(p.N, p.tchunk), (unsigned)Gc);
    const dim3 lat_grid((unsigned)p.J, (unsigned)Gc);
    // ---- stage 3 (decode): token pass (its dK part, per-token statistics), latent pass
    FLAREPP_TRY(prep(zf, false, MD, Gc, true, 1.0f, zh, zl, nullptr));
    const float kscale = p.c != 0.0f ? p.s / p.c : 0.0f;
    {
      BwdDecArgs d{};
      d.qhi = qhi;
      d.qlo = qlo;
      d.zh = zh;
      d.zl = zl;
      d.K = static_cast<const __bf16*>(K);
      d.dY = dY + g0 * (int64_t)p.N * D;
      d.qnorm = at<float>(ws, p.o_qnorm);
      d.c = p.c;
      d.dK = dK;
      d.tA = at<float>(ws, p.o_tlse);
      d.tD = at<float>(ws, p.o_tdel);
      d.tstride = cdiv(p.N, 4) * 4;
      d.part = part;
      d.J = p.J;
      d.chunk = p.chunk;
      d.tchunk = p.tchunk;
      d.N = p.N;
      d.M = p.M;
      d.Mp = p.Mp;
      d.Mt = p.Mt;
      d.bh0 = g0;
      d.s = p.s;
      d.kscale = kscale;
      bwd_dec_tok_bf16<D><<<tok_grid, 512, 0, st>>>(d);
      FLAREPP_TRY(launched());
      bwd_dec_lat_bf16<D><<<lat_grid, 512, 0, st>>>(d);
      FLAREPP_TRY(launched());
      FLAREPP_TRY(reduce(2 * D, D, nullptr, dz, zf, del, 0));            // dZ, delta_2 = <dZ, Z>
      FLAREPP_TRY(reduce(2 * D, 0, nullptr, dq3, nullptr, nullptr, 0));  // dQd from the decode
    }
    // ---- stages 2 and 1: latent passes, then one token pass for both
    BwdStageOps ops[2];
    ops[0] = BwdStageOps{qhi, qlo, (int64_t)p.H * MpD, MpD, g0 * MpD, dzr, dzl, lse2, nullptr};
    ops[1] = BwdStageOps{shi, slo, 0, p.nS > 1 ? MpD : 0, 0, dqr, dql, lse1, nullptr};
    auto enc_latent = [&](const BwdStageOps& o, const float* delta) {
      BwdEncArgs e{};
      e.qhi = o.qhi;
      e.qlo = o.qlo;
      e.q_sb = o.q_sb;
      e.q_sh = o.q_sh;
      e.q_off = o.q_off;
      e.dor = o.dor;
      e.dorl = o.dorl;
      e.lse = o.lse;
      e.delta = delta;
      e.K = static_cast<const __bf16*>(K);
      e.V = static_cast<const __bf16*>(V);
      e.part = part;
      e.J = p.J;
      e.chunk = p.chunk;
      e.H = p.H;
      e.N = p.N;
      e.M = p.M;
      e.Mp = p.Mp;
      e.bh0 = g0;
      e.s = p.s;
      bwd_enc_lat_bf16<D><<<lat_grid, 512, 0, st>>>(e);
      return launched();
    };
    float* del2 = del;
    float* del1 = at<float>(ws, p.o_del1);
    FLAREPP_TRY(prep(dz, false, MD, Gc, false, 1.0f, dzr, dzl, nullptr));
    FLAREPP_TRY(enc_latent(ops[0], del2));
    FLAREPP_TRY(reduce(D, 0, dq3, dq, qf, del1, 0));  // dQd = encode + decode parts, delta_1 = <dQd, Qd>
    FLAREPP_TRY(prep(dq, false, MD, Gc, false, 1.0f, dqr, dql, nullptr));
    FLAREPP_TRY(enc_latent(ops[1], del1));
    // dS: each head's split partials summed into dq3 (free again), then
    // the heads summed per seed block
    FLAREPP_TRY(reduce(D, 0, nullptr, dq3, nullptr, nullptr, 0));
    {
      BwdSeedSumArgs ss{dq3, dS, p.M, Gc, p.H, p.nS, g0};
      bwd_seed_sum<D><<<(unsigned)cdiv((int64_t)p.nS * MD, 256), 256, 0, st>>>(ss);
      FLAREPP_TRY(launched());
    }
    ops[0].delta = del2;
    ops[1].delta = del1;
    BwdEncTokArgs t{};
    t.st[0] = ops[0];
    t.st[1] = ops[1];
    t.K = static_cast<const __bf16*>(K);
    t.V = static_cast<const __bf16*>(V);
    t.dK = dK;
    t.dV = dV;
    t.tchunk = p.tchunk;
    t.H = p.H;
    t.N = p.N;
    t.M = p.M;
    t.Mp = p.Mp;
    t.Mt = p.Mt;
    t.bh0 = g0;
    t.kscale = kscale;
    bwd_enc_tok_bf16<D><<<tok_grid, 512, 0, st>>>(t);
    FLAREPP_TRY(launched());
  }
  return FLAREPP_OK;
}

// The route with the forward of the backward (flarepp_route_save): stages 1
// and 2 as forward_for_backward runs them (c S and c Qd as bf16 hi/lo
// operands, the logits the backward's passes take), Qd, Z and both
// log-sum-exps written for flarepp_route_backward_saved, then the route's
// decode.
template <int D>
flarepp_status run_route_save(const Plan& p, const void* S, const void* K, const void* V, float* Y, float* Qd_out,
                              float* Z_out, float* lse_out, void* ws, hipStream_t st) {
  Recorder rec;
  const int64_t MD = (int64_t)p.M * D, MpD = (int64_t)p.Mp * D;
  FLAREPP_TRY(run_prep<D>(p, S, true, 0, p.nS > 1 ? MD : 0, p.nS, at<__bf16>(ws, p.o_shi), at<__bf16>(ws, p.o_slo),
                          nullptr, nullptr, p.c, st, rec));
  for (int64_t g0 = 0; g0 < p.BH; g0 += p.G) {
    const int Gc = (int)std::min<int64_t>(p.G, p.BH - g0);
    __bf16* zt = at<__bf16>(ws, p.o_zt);
    FLAREPP_TRY(forward_for_backward<D>(p, K, V, ws, g0, Gc, Qd_out, nullptr, Z_out, nullptr, lse_out + g0 * p.Mp,
                                        lse_out + (p.BH + g0) * p.Mp, zt, st, rec));
    DecodeArgs d{};
    d.q_hi = at<__bf16>(ws, p.o_qhi);
    d.q_lo = at<__bf16>(ws, p.o_qlo);
    d.q_sb = (int64_t)p.H * MpD;
    d.q_sh = MpD;
    d.q_off = g0 * MpD;
    d.qnorm = at<float>(ws, p.o_qnorm);
    d.knorm = at<float>(ws, p.o_knorm);
    d.Jk = p.J;
    d.zt = zt;
    d.K = static_cast<const __bf16*>(K);
    d.Y = Y;
    d.H = p.H;
    d.N = p.N;
    d.M = p.M;
    d.Mp = p.Mp;
    d.chunk = p.dchunk;
    d.bh0 = g0;
    d.c = p.c;
    FLAREPP_TRY(run_decode_bf16<D>(p, d, Gc, st, rec));
  }
  return FLAREPP_OK;
}

flarepp_status dispatch(const Plan& p, Stage stage, const void* S, const float* Qd_in, const float* Z_in,
                        const void* K, const void* V, float* Y, float* Qd_out, float* Z_out, void* ws,
                        void* stream, Recorder* recorder = nullptr) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  Recorder inert;
  Recorder& rec = recorder ? *recorder : inert;
  if (p.D == 16) return run<16>(p, stage, S, Qd_in, Z_in, K, V, Y, Qd_out, Z_out, ws, st, rec);
  return run<32>(p, stage, S, Qd_in, Z_in, K, V, Y, Qd_out, Z_out, ws, st, rec);
}

// Shared argument checks of the compute calls: descriptor, pointers,
// alignment, workspace size and aliasing; all before any HIP call.
// ws_internal: the workspace is the library's own scratch (not checked here).
flarepp_status prologue(const flarepp_desc* d, int op, const void* const* in, const size_t* in_bytes, int nin,
                        const void* const* out, const size_t* out_bytes, const bool* out_required, int nout,
                        void* ws, size_t ws_bytes, Plan* plan, const flarepp_tuning* tuning = nullptr,
                        bool ws_internal = false) {
  FLAREPP_TRY(check_desc(d));
  FLAREPP_TRY(check_tuning(tuning));
  for (int i = 0; i < nin; ++i)
    if (!in[i] || misaligned(in[i])) return FLAREPP_INVALID_ARG;
  for (int i = 0; i < nout; ++i) {
    if (out_required[i] && !out[i]) return FLAREPP_INVALID_ARG;
    if (out[i] && misaligned(out[i])) return FLAREPP_INVALID_ARG;
  }
  *plan = make_plan(d, op, tuning);
  if (plan->total > 0 && !ws_internal) {
    if (!ws || misaligned(ws)) return FLAREPP_INVALID_ARG;
    if (ws_bytes < plan->total) return FLAREPP_WORKSPACE_TOO_SMALL;
  }
  Range ins[10], outs[6];
  const void* inp[10];
  const void* outp[6];
  if (nin > 9 || nout > 6) return FLAREPP_INVALID_ARG;
  int ni = 0;
  for (int i = 0; i < nin; ++i) {
    ins[ni] = range(in[i], in_bytes[i]);
    inp[ni++] = in[i];
  }
  if (plan->total > 0 && !ws_internal) {
    ins[ni] = range(ws, plan->total);
    inp[ni++] = ws;
  }
  for (int i = 0; i < nout; ++i) {
    outs[i] = range(out[i], out_bytes[i]);
    outp[i] = out[i];
  }
  return check_aliasing(outs, outp, nout, ins, inp, ni);
}

struct Sizes {
  size_t s, kv, md, y;
};
Sizes sizes(const flarepp_desc* d) {
  const size_t elem = d->dtype == FLAREPP_BF16 ? 2 : 4;
  Sizes z;
  z.s = (size_t)(d->seed_head_stride ? d->H : 1) * d->M * d->D * elem;
  z.kv = (size_t)d->B * d->H * d->N * d->D * elem;
  z.md = (size_t)d->B * d->H * d->M * d->D * 4;
  z.y = (size_t)d->B * d->H * d->N * d->D * 4;
  return z;
}

// ---- allocation-free route: the workspace is a file-scope device array.
// Every GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current and
// kept in g_scratch_ptr.  Calls on one GPU share the array, so calls that
// overlap in time on one GPU (different streams, or several host threads)
// race on it; nothing in it needs to start at zero (the route writes every
// workspace word it reads).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

flarepp_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLAREPP_HIP_ERROR;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FLAREPP_HIP_ERROR;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLAREPP_OK;
}

}  // namespace

extern "C" {

int flarepp_abi_version(void) { return FLAREPP_ABI_VERSION; }

const char* flarepp_status_string(flarepp_status s) {
  switch (s) {
    case FLAREPP_OK: return "ok";
    case FLAREPP_INVALID_ARG: return "invalid argument";
    case FLAREPP_UNSUPPORTED: return "unsupported shape or dtype";
    case FLAREPP_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FLAREPP_ALIASING: return "an output overlaps another buffer";
    case FLAREPP_HIP_ERROR: return "HIP launch error";
    case FLAREPP_SCRATCH_LIMIT: return "workspace needed exceeds the library's built-in scratch";
  }
  return "unknown status";
}

flarepp_status flarepp_workspace_size(const flarepp_desc* desc, int32_t op, size_t* bytes) {
  if (!bytes) return FLAREPP_INVALID_ARG;
  FLAREPP_TRY(check_desc(desc));
  if (op < FLAREPP_OP_SEED_ENCODE || op > FLAREPP_OP_SPECTRUM) return FLAREPP_INVALID_ARG;
  if (op == FLAREPP_OP_ROUTE_BACKWARD && desc->M > kBwdBf16MaxM) return FLAREPP_UNSUPPORTED;
  *bytes = make_plan(desc, op).total;
  return FLAREPP_OK;
}

flarepp_status flarepp_workspace_size_tuned(const flarepp_desc* desc, int32_t op, const flarepp_tuning* tuning,
                                            size_t* bytes) {
  if (!bytes) return FLAREPP_INVALID_ARG;
  FLAREPP_TRY(check_desc(desc));
  FLAREPP_TRY(check_tuning(tuning));
  if (op < FLAREPP_OP_SEED_ENCODE || op > FLAREPP_OP_SPECTRUM) return FLAREPP_INVALID_ARG;
  if (op == FLAREPP_OP_ROUTE_BACKWARD && desc->M > kBwdBf16MaxM) return FLAREPP_UNSUPPORTED;
  *bytes = make_plan(desc, op, tuning).total;
  return FLAREPP_OK;
}

flarepp_status flarepp_seed_encode(const flarepp_desc* desc, const void* S, const void* K, const void* V,
                                   float* Qd, void* ws, size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {S, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[1] = {Qd};
  const size_t outb[1] = {z.md};
  const bool req[1] = {true};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_SEED_ENCODE, in, inb, 3, out, outb, req, 1, ws, ws_bytes, &p));
  return dispatch(p, kSeed, S, nullptr, nullptr, K, V, nullptr, Qd, nullptr, ws, stream);
}

flarepp_status flarepp_encode(const flarepp_desc* desc, const float* Qd, const void* K, const void* V, float* Z,
                              void* ws, size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {Qd, K, V};
  const size_t inb[3] = {z.md, z.kv, z.kv};
  const void* out[1] = {Z};
  const size_t outb[1] = {z.md};
  const bool req[1] = {true};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ENCODE, in, inb, 3, out, outb, req, 1, ws, ws_bytes, &p));
  return dispatch(p, kEncode, nullptr, Qd, nullptr, K, V, nullptr, nullptr, Z, ws, stream);
}

flarepp_status flarepp_decode(const flarepp_desc* desc, const float* Qd, const float* Zin, const void* K, float* Y,
                              void* ws, size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {Qd, Zin, K};
  const size_t inb[3] = {z.md, z.md, z.kv};
  const void* out[1] = {Y};
  const size_t outb[1] = {z.y};
  const bool req[1] = {true};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_DECODE, in, inb, 3, out, outb, req, 1, ws, ws_bytes, &p));
  return dispatch(p, kDecode, nullptr, Qd, Zin, K, nullptr, Y, nullptr, nullptr, ws, stream);
}

flarepp_status flarepp_route(const flarepp_desc* desc, const void* S, const void* K, const void* V, float* Y,
                             float* Qd_out, float* Z_out, void* ws, size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {S, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[3] = {Y, Qd_out, Z_out};
  const size_t outb[3] = {z.y, z.md, z.md};
  const bool req[3] = {true, false, false};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ROUTE, in, inb, 3, out, outb, req, 3, ws, ws_bytes, &p));
  return dispatch(p, kRoute, S, nullptr, nullptr, K, V, Y, Qd_out, Z_out, ws, stream);
}

flarepp_status flarepp_route_tuned(const flarepp_desc* desc, const flarepp_tuning* tuning, const void* S,
                                   const void* K, const void* V, float* Y, float* Qd_out, float* Z_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {S, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[3] = {Y, Qd_out, Z_out};
  const size_t outb[3] = {z.y, z.md, z.md};
  const bool req[3] = {true, false, false};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ROUTE, in, inb, 3, out, outb, req, 3, ws, ws_bytes, &p, tuning));
  return dispatch(p, kRoute, S, nullptr, nullptr, K, V, Y, Qd_out, Z_out, ws, stream);
}

flarepp_status flarepp_route_noalloc(const flarepp_desc* desc, const void* S, const void* K, const void* V,
                                     float* Y, float* Qd_out, float* Z_out, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {S, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[3] = {Y, Qd_out, Z_out};
  const size_t outb[3] = {z.y, z.md, z.md};
  const bool req[3] = {true, false, false};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ROUTE, in, inb, 3, out, outb, req, 3, nullptr, 0, &p, nullptr, true));
  if (p.total > kScratchBytes) return FLAREPP_SCRATCH_LIMIT;
  void* ws = nullptr;
  FLAREPP_TRY(scratch_of_current_device(&ws));
  return dispatch(p, kRoute, S, nullptr, nullptr, K, V, Y, Qd_out, Z_out, ws, stream);
}

size_t flarepp_noalloc_scratch_bytes(void) { return kScratchBytes; }

flarepp_status flarepp_flare(const flarepp_desc* desc, const void* Q, const void* K, const void* V, float* Y,
                             float* Z_out, void* ws, size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {Q, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[2] = {Y, Z_out};
  const size_t outb[2] = {z.y, z.md};
  const bool req[2] = {true, false};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_FLARE, in, inb, 3, out, outb, req, 2, ws, ws_bytes, &p));
  return dispatch(p, kFlare, Q, nullptr, nullptr, K, V, Y, nullptr, Z_out, ws, stream);
}

flarepp_status flarepp_spectrum(const flarepp_desc* desc, const void* S, const void* K, const void* V, float* eig,
                                float* sym_out, void* ws, size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const size_t ne = (size_t)desc->B * desc->H * desc->M * 4;
  const void* in[3] = {S, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[2] = {eig, sym_out};
  const size_t outb[2] = {ne, ne * (size_t)desc->M};
  const bool req[2] = {true, false};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_SPECTRUM, in, inb, 3, out, outb, req, 2, ws, ws_bytes, &p));
  return dispatch(p, kSpectrum, S, nullptr, nullptr, K, V, eig, nullptr, sym_out, ws, stream);
}

flarepp_status flarepp_route_backward(const flarepp_desc* desc, const void* S, const void* K, const void* V,
                                      const float* dY, float* dS, float* dK, float* dV, void* ws, size_t ws_bytes,
                                      void* stream) {
  FLAREPP_TRY(check_desc(desc));
  if (desc->M > kBwdBf16MaxM) return FLAREPP_UNSUPPORTED;
  const Sizes z = sizes(desc);
  const void* in[4] = {S, K, V, dY};
  const size_t inb[4] = {z.s, z.kv, z.kv, z.y};
  const void* out[3] = {dS, dK, dV};
  const size_t outb[3] = {z.s, z.kv, z.kv};
  const bool req[3] = {true, true, true};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ROUTE_BACKWARD, in, inb, 4, out, outb, req, 3, ws, ws_bytes, &p));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.bf16) {
    if (p.D == 16) return run_backward_bf16<16>(p, S, K, V, dY, dS, dK, dV, ws, st);
    return run_backward_bf16<32>(p, S, K, V, dY, dS, dK, dV, ws, st);
  }
  const float *Sf = static_cast<const float*>(S), *Kf = static_cast<const float*>(K),
              *Vf = static_cast<const float*>(V);
  if (p.D == 16) return run_backward<16>(p, Sf, Kf, Vf, dY, dS, dK, dV, ws, st);
  return run_backward<32>(p, Sf, Kf, Vf, dY, dS, dK, dV, ws, st);
}

// Bytes of the saved log-sum-exps: [2][B H][Mp] float32.
static size_t saved_lse_bytes(const flarepp_desc* d) {
  return (size_t)2 * d->B * d->H * (size_t)(cdiv(d->M, 16) * 16) * 4;
}

flarepp_status flarepp_route_save(const flarepp_desc* desc, const void* S, const void* K, const void* V, float* Y,
                                  float* Qd_out, float* Z_out, float* lse_out, void* ws, size_t ws_bytes,
                                  void* stream) {
  FLAREPP_TRY(check_desc(desc));
  if (desc->dtype != FLAREPP_BF16 || desc->M > kBwdBf16MaxM) return FLAREPP_UNSUPPORTED;
  const Sizes z = sizes(desc);
  const void* in[3] = {S, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[4] = {Y, Qd_out, Z_out, lse_out};
  const size_t outb[4] = {z.y, z.md, z.md, saved_lse_bytes(desc)};
  const bool req[4] = {true, true, true, true};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ROUTE_BACKWARD, in, inb, 3, out, outb, req, 4, ws, ws_bytes, &p));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.D == 16) return run_route_save<16>(p, S, K, V, Y, Qd_out, Z_out, lse_out, ws, st);
  return run_route_save<32>(p, S, K, V, Y, Qd_out, Z_out, lse_out, ws, st);
}

flarepp_status flarepp_route_backward_saved(const flarepp_desc* desc, const void* S, const void* K, const void* V,
                                            const float* Qd, const float* Z, const float* lse, const float* dY,
                                            float* dS, float* dK, float* dV, void* ws, size_t ws_bytes,
                                            void* stream) {
  FLAREPP_TRY(check_desc(desc));
  if (desc->dtype != FLAREPP_BF16 || desc->M > kBwdBf16MaxM) return FLAREPP_UNSUPPORTED;
  const Sizes z = sizes(desc);
  const void* in[7] = {S, K, V, Qd, Z, lse, dY};
  const size_t inb[7] = {z.s, z.kv, z.kv, z.md, z.md, saved_lse_bytes(desc), z.y};
  const void* out[3] = {dS, dK, dV};
  const size_t outb[3] = {z.s, z.kv, z.kv};
  const bool req[3] = {true, true, true};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ROUTE_BACKWARD, in, inb, 7, out, outb, req, 3, ws, ws_bytes, &p));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const SavedForward saved{Qd, Z, lse};
  if (p.D == 16) return run_backward_bf16<16>(p, S, K, V, dY, dS, dK, dV, ws, st, &saved);
  return run_backward_bf16<32>(p, S, K, V, dY, dS, dK, dV, ws, st, &saved);
}

flarepp_status flarepp_route_profiled(const flarepp_desc* desc, const void* S, const void* K, const void* V,
                                      float* Y, float* Qd_out, float* Z_out, void* ws, size_t ws_bytes,
                                      void* stream, void** events, int32_t* kinds, int32_t max_launches,
                                      int32_t* n_launches) {
  if (!events || !kinds || !n_launches || max_launches < 0) return FLAREPP_INVALID_ARG;
  FLAREPP_TRY(check_desc(desc));
  const Sizes z = sizes(desc);
  const void* in[3] = {S, K, V};
  const size_t inb[3] = {z.s, z.kv, z.kv};
  const void* out[3] = {Y, Qd_out, Z_out};
  const size_t outb[3] = {z.y, z.md, z.md};
  const bool req[3] = {true, false, false};
  Plan p;
  FLAREPP_TRY(prologue(desc, FLAREPP_OP_ROUTE, in, inb, 3, out, outb, req, 3, ws, ws_bytes, &p));
  Recorder rec;
  rec.events = events;
  rec.kinds = kinds;
  rec.max = max_launches;
  const flarepp_status st = dispatch(p, kRoute, S, nullptr, nullptr, K, V, Y, Qd_out, Z_out, ws, stream, &rec);
  *n_launches = rec.n;
  if (st == FLAREPP_OK && rec.failed) return FLAREPP_HIP_ERROR;
  return st;
}

// ---- token shards (context parallelism): one shard's share of an encode
// stage as records, and the merge of the records of all shards.

flarepp_status flarepp_shard_records_size(const flarepp_desc* desc, int32_t nslots, size_t* bytes) {
  if (!bytes || nslots < 1) return FLAREPP_INVALID_ARG;
  FLAREPP_TRY(check_desc(desc));
  *bytes = (size_t)desc->B * desc->H * (size_t)cdiv(desc->M, 16) * 16 * (size_t)nslots * (desc->D + 4) * 4;
  return FLAREPP_OK;
}

flarepp_status flarepp_encode_shard(const flarepp_desc* desc, int32_t stage, const void* Q, const void* K,
                                    const void* V, float* rec, int32_t slot, int32_t nslots, void* ws,
                                    size_t ws_bytes, void* stream) {
  FLAREPP_TRY(check_desc(desc));
  if ((stage != 1 && stage != 2) || nslots < 1 || slot < 0 || slot >= nslots) return FLAREPP_INVALID_ARG;
  const Sizes z = sizes(desc);
  size_t recb = 0;
  FLAREPP_TRY(flarepp_shard_records_size(desc, nslots, &recb));
  const void* in[3] = {Q, K, V};
  const size_t inb[3] = {stage == 1 ? z.s : z.md, z.kv, z.kv};
  const void* out[1] = {rec};
  const size_t outb[1] = {recb};
  const bool req[1] = {true};
  Plan p;
  FLAREPP_TRY(prologue(desc, stage == 1 ? FLAREPP_OP_SEED_ENCODE : FLAREPP_OP_ENCODE, in, inb, 3, out, outb, req, 1,
                       ws, ws_bytes, &p));
  p.rec = rec;
  p.rec_slot = slot;
  p.rec_nslots = nslots;
  if (stage == 1) return dispatch(p, kSeed, Q, nullptr, nullptr, K, V, nullptr, nullptr, nullptr, ws, stream);
  return dispatch(p, kEncode, nullptr, static_cast<const float*>(Q), nullptr, K, V, nullptr, nullptr, nullptr, ws,
                  stream);
}

flarepp_status flarepp_merge_shards(const flarepp_desc* desc, const float* rec, int32_t nslots, float* out,
                                    void* stream) {
  FLAREPP_TRY(check_desc(desc));
  if (nslots < 1 || !rec || !out || misaligned(rec) || misaligned(out)) return FLAREPP_INVALID_ARG;
  size_t recb = 0;
  FLAREPP_TRY(flarepp_shard_records_size(desc, nslots, &recb));
  const Sizes z = sizes(desc);
  if (overlap(range(out, z.md), range(rec, recb))) return FLAREPP_ALIASING;
  Plan p = make_plan(desc, FLAREPP_OP_ROUTE);
  p.J = nslots;  // one record per shard and row
  int tpr = 1;
  while (tpr < p.J && tpr < 64) tpr *= 2;
  p.tpr = tpr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Recorder rcd;
  const int64_t PS = p.D + 4;
  for (int64_t g0 = 0; g0 < p.BH; g0 += p.G) {
    const int Gc = (int)std::min<int64_t>(p.G, p.BH - g0);
    MergeArgs m{};
    m.part = const_cast<float*>(rec) + g0 * p.Mp * (int64_t)nslots * PS;  // read only: no refit
    m.J = nslots;
    m.Mp = p.Mp;
    m.M = p.M;
    m.bh0 = g0;
    m.c = p.c;
    m.out = out;
    if (p.D == 16)
      FLAREPP_TRY(run_merge<16>(p, m, Gc, st, rcd));
    else
      FLAREPP_TRY(run_merge<32>(p, m, Gc, st, rcd));
  }
  return FLAREPP_OK;
}

}  // extern "C"
