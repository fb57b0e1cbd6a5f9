/*
 * flarepp.h -- C ABI of libflarepp, the FLARE++ routing forward pass on one
 * AMD Instinct MI355X (gfx950) GPU.
 *
 * The operation.  For every batch element b and head h, with token keys and
 * values K, V (N x D), learned latent seeds S (M x D) and a scale s:
 *
 *     Qd = SDPA(S,  K, V,  s)   seed encode: M input-conditioned queries
 *     Z  = SDPA(Qd, K, V,  s)   encode: the queries compress the tokens
 *     Y  = SDPA(K,  Qd, Z, s)   decode: every token reads the latents back
 *
 * where SDPA(Q, K, V, s)_i = sum_j softmax_j(s <Q_i, K_j>) V_j.  The first
 * line is the extra encode call driven by learned latent seeds that the
 * FLARE++ abstract introduces ("FLARE++: Low-rank attention with dynamic
 * attention routing", abstract; French technical summary, "Méthodologie",
 * "Synthèse de Requêtes Dynamiques"); the second and third are FLARE's
 * encode and decode with the synthesised queries in place of fixed ones
 * ("FLARE: Fast Low-rank Attention Routing Engine", section
 * "Основной механизм FLARE"; French summary, "Routage Encode-Décode").  The
 * encode softmaxes run over the N tokens and the decode softmax over the M
 * latents (FLARE summary, "Матрица коммуникации низкого ранга").  Nothing is
 * applied between the stages.  The N x N mixing matrix is never formed.
 *
 * Layouts.  Every tensor is dense, row-major, with D innermost:
 *     K, V         B x H x N x D   (dtype of the descriptor)
 *     S            M x D           (seed_head_stride == 0: shared by all
 *                                   (b, h)) or H x M x D (seed_head_stride
 *                                   == M*D: per-head seeds), descriptor dtype
 *     Qd, Z        B x H x M x D   float32
 *     Y            B x H x N x D   float32
 * Base pointers must be 16-byte aligned device pointers.
 *
 * Arithmetic.  FLAREPP_F32: float32 inputs, float32 arithmetic throughout.
 * FLAREPP_BF16: bf16 inputs; the contractions run on bf16 matrix cores with
 * float32 accumulation, softmax statistics are float32, and Qd is carried
 * into the later stages as a bf16 hi/lo pair; outputs are float32.
 *
 * Ownership and threading.  The caller owns every buffer.  The library never
 * allocates device memory, never synchronises, keeps no pointer after a call
 * returns and has no mutable global state; calls on different streams may
 * run concurrently if their output and workspace buffers are disjoint.  Work
 * is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 * Workspace contents are undefined on return.
 *
 * Errors.  Every call validates its arguments on the host before any GPU
 * call and returns a flarepp_status; no exception crosses the ABI.  A launch
 * failure is reported as FLAREPP_HIP_ERROR.  Faults inside kernels surface at
 * the caller's next synchronisation.  Results are bitwise repeatable for a
 * given descriptor: the split counts and launch shapes are a fixed function
 * of the descriptor alone (no environment variable, device query or global
 * state enters them) and no atomics are used.  flarepp_route_tuned lets a
 * caller override that choice explicitly.
 */
#ifndef FLAREPP_H
#define FLAREPP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLAREPP_ABI_VERSION 2

typedef enum flarepp_status {
    FLAREPP_OK = 0,
    FLAREPP_INVALID_ARG = 1,          /* null pointer, dims < 1, bad stride, non-finite scale, misaligned */
    FLAREPP_UNSUPPORTED = 2,          /* D not 16 or 32, dtype unknown, M or N*D beyond the limits below */
    FLAREPP_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below flarepp_workspace_size() */
    FLAREPP_ALIASING = 4,             /* an output overlaps an input, another output or the workspace */
    FLAREPP_HIP_ERROR = 5,            /* a kernel launch failed */
    FLAREPP_SCRATCH_LIMIT = 6         /* flarepp_route_noalloc: workspace beyond its built-in scratch */
} flarepp_status;

typedef enum flarepp_dtype {
    FLAREPP_F32 = 0,
    FLAREPP_BF16 = 1
} flarepp_dtype;

typedef enum flarepp_op {
    FLAREPP_OP_SEED_ENCODE = 0,
    FLAREPP_OP_ENCODE = 1,
    FLAREPP_OP_DECODE = 2,
    FLAREPP_OP_ROUTE = 3,
    FLAREPP_OP_FLARE = 4,
    FLAREPP_OP_ROUTE_BACKWARD = 5,
    FLAREPP_OP_SPECTRUM = 6
} flarepp_op;

/* Limits of this build. */
#define FLAREPP_MAX_M 256
#define FLAREPP_MAX_SLICE_ELEMS ((int64_t)1 << 31) /* N * D per (b, h) */

typedef struct flarepp_desc {
    int64_t B, H, N, M, D;    /* batch, heads, tokens, latents, head dim (16 or 32) */
    int32_t dtype;            /* flarepp_dtype of S, K, V */
    float scale;              /* s, used in all three stages */
    int64_t seed_head_stride; /* elements between heads' seed blocks: 0 or M*D */
} flarepp_desc;

/* FLAREPP_ABI_VERSION of the loaded library. */
int flarepp_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *flarepp_status_string(flarepp_status status);

/*
 * Bytes of device workspace that `op` needs for `desc` (the split-N partial
 * softmax statistics and the bf16 operand copies of Qd and Z).  Pure host
 * computation.  Returns INVALID_ARG / UNSUPPORTED for descriptors the
 * compute calls would reject.
 */
flarepp_status flarepp_workspace_size(const flarepp_desc *desc, int32_t op, size_t *bytes);

/*
 * Seed encode, Qd = SDPA(S, K, V, s) for every (b, h): the extra encode
 * call with learned latent seeds as queries (FLARE++ abstract; French
 * summary, "Synthèse de Requêtes Dynamiques").  S: M x D or H x M x D
 * (descriptor dtype); K, V: B x H x N x D; Qd (output): B x H x M x D fp32.
 */
flarepp_status flarepp_seed_encode(const flarepp_desc *desc, const void *S, const void *K,
                                   const void *V, float *Qd, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * Encode, Z = SDPA(Qd, K, V, s): FLARE's encode step with per-(b, h)
 * queries (FLARE summary, "Основной механизм FLARE", encode step).
 * Qd: B x H x M x D fp32; K, V: B x H x N x D; Z (output): B x H x M x D fp32.
 * Calling the stages one by one lets a caller transform Qd in between.
 */
flarepp_status flarepp_encode(const flarepp_desc *desc, const float *Qd, const void *K,
                              const void *V, float *Z, void *ws, size_t ws_bytes, void *stream);

/*
 * Decode, Y = SDPA(K, Qd, Z, s): every token attends over the M latents
 * (FLARE summary, "Основной механизм FLARE", decode step; softmax over the
 * latents, "Матрица коммуникации низкого ранга").  Qd, Z: B x H x M x D
 * fp32; K: B x H x N x D; Y (output): B x H x N x D fp32.
 */
flarepp_status flarepp_decode(const flarepp_desc *desc, const float *Qd, const float *Z,
                              const void *K, float *Y, void *ws, size_t ws_bytes, void *stream);

/*
 * The complete route, seed encode -> encode -> decode, enqueued on one
 * stream with no host synchronisation ("FLARE++" abstract: the complete
 * routing operation is scaled-dot-product attention calls alone).  Y is
 * required; Qd_out and Z_out may be NULL.
 */
flarepp_status flarepp_route(const flarepp_desc *desc, const void *S, const void *K,
                             const void *V, float *Y, float *Qd_out, float *Z_out, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * Fixed-query FLARE, the special case FLARE++ generalises: the latent
 * queries Q are parameters rather than synthesised, Z = SDPA(Q, K, V, s) and
 * Y = SDPA(K, Q, Z, s) ("FLARE: Fast Low-rank Attention Routing Engine",
 * section "Основной механизм FLARE"; the FLARE++ abstract's fixed learned
 * query templates).  Q: M x D or H x M x D (seed_head_stride), descriptor
 * dtype.  Y is required; Z_out may be NULL.
 */
flarepp_status flarepp_flare(const flarepp_desc *desc, const void *Q, const void *K,
                             const void *V, float *Y, float *Z_out, void *ws, size_t ws_bytes,
                             void *stream);

/*
 * Backward of the route: given dY (B x H x N x D fp32), the gradient of a
 * scalar loss with respect to Y = route(S, K, V), writes the gradients
 *     dS  (shape of S: M x D, or H x M x D with per-head seeds; a seed block
 *          shared by several (b, h) receives the sum of their gradients),
 *     dK, dV  (B x H x N x D),
 * all fp32.  The forward is recomputed inside the call (flarepp_route_save
 * and flarepp_route_backward_saved below split a training step so that it
 * is not).  It is the chain
 * rule through the three SDPA stages in reverse -- decode (queries K, keys
 * Qd, values Z), encode (queries Qd), seed encode (queries S) -- with Qd's
 * gradient collecting its two uses (encode query, decode key); for one SDPA
 * O = softmax(s Q K^T) V with upstream dO: dV = P^T dO, dL = P o (dO V^T -
 * rowsum(dO o O)), dQ = s dL K, dK = s dL^T Q.  The pages measure FLARE++
 * per training step (French technical summary, "Résultats"), i.e. forward
 * and this backward.  Both dtypes: S, K, V in the descriptor's dtype, dY and
 * the gradients fp32.  FLAREPP_F32: float32 vector arithmetic.  FLAREPP_BF16:
 * matrix-core products with float32 accumulation (logits from a bf16 hi/lo
 * query, gradient products from bf16 operands and weights) after the
 * route's own forward stages 1 and 2.  M <= 256.  Workspace:
 * flarepp_workspace_size with FLAREPP_OP_ROUTE_BACKWARD.  Inputs S, K, V, dY; outputs dS, dK, dV must
 * not overlap them, each other or the workspace.
 */
flarepp_status flarepp_route_backward(const flarepp_desc *desc, const void *S, const void *K,
                                      const void *V, const float *dY, float *dS, float *dK,
                                      float *dV, void *ws, size_t ws_bytes, void *stream);

/*
 * The training step without the recomputed forward: flarepp_route_save runs
 * the route with the backward's own forward stages 1 and 2 (c S and c Qd as
 * bf16 hi/lo operands, the logits the backward's passes take) and keeps
 * what the backward needs; flarepp_route_backward_saved takes those instead
 * of recomputing them.  The pair gives the gradients of
 * flarepp_route_backward up to the rounding of the latent norms (the saved
 * path recomputes ||Qd_m|| from the float32 Qd), and the forward's Y of
 * flarepp_route up to its query operands (hi/lo seeds here, exact seeds
 * there).  Chain rule and the pages' per-step cost: as flarepp_route_backward.
 *   Y, Qd_out, Z_out (outputs of flarepp_route_save): as flarepp_route's,
 *     all required.
 *   lse_out / lse: the log-sum-exp (log2 units) of the two encodes' softmax
 *     rows, float32 [2][B x H][Mp] with Mp = 16 * ceil(M / 16) (rows M ..
 *     Mp - 1 are written and read back as they are), 2 * B * H * Mp floats.
 * bf16 only (FLAREPP_F32: FLAREPP_UNSUPPORTED), M <= 256.  Workspace (both
 * calls): flarepp_workspace_size with FLAREPP_OP_ROUTE_BACKWARD; the saved
 * buffers are the caller's and pass nothing through the workspace.  Outputs
 * must not overlap the inputs, each other or the workspace.
 */
flarepp_status flarepp_route_save(const flarepp_desc *desc, const void *S, const void *K,
                                  const void *V, float *Y, float *Qd_out, float *Z_out,
                                  float *lse_out, void *ws, size_t ws_bytes, void *stream);
flarepp_status flarepp_route_backward_saved(const flarepp_desc *desc, const void *S,
                                            const void *K, const void *V, const float *Qd,
                                            const float *Z, const float *lse, const float *dY,
                                            float *dS, float *dK, float *dV, void *ws,
                                            size_t ws_bytes, void *stream);

/*
 * Spectrum of each head's mixing matrix W = W_dec W_enc (N x N, rank <= M):
 * its nonzero eigenvalues are those of the M x M product W_enc W_dec, where
 * W_enc = softmax over tokens of s Qd K^T (the encode weights) and W_dec =
 * softmax over latents of s K Qd^T (the decode weights), Qd the route's
 * synthesised queries -- the eigendecomposition in O(M^3 + M^2 N) of the
 * FLARE summary ("FLARE: Fast Low-rank Attention Routing Engine", section
 * "Спектральный анализ"; mixing matrix: "Матрица коммуникации низкого
 * ранга").  Because both factors are softmaxes of the same logits, W_enc
 * W_dec is similar to the symmetric positive semidefinite G = F F^T with
 * F_mn = sqrt(W_enc[m, n] W_dec[n, m]); its eigenvalues are real, in
 * [0, 1], the largest 1.  The library forms G on the GPU (O(M^2 N); for
 * bf16 inputs on the matrix cores with F rounded to fp16, for float32 inputs
 * in float32) and finds its eigenvalues by Householder reduction to
 * tridiagonal form and bisection (float32; each eigenvalue to about 2 ulp of
 * the largest).
 *   eig (output): B x H x M fp32, each head's eigenvalues by decreasing value.
 *   sym_out (optional output): B x H x M x M fp32, the matrix G.
 * Both dtypes; workspace: flarepp_workspace_size with FLAREPP_OP_SPECTRUM.
 */
flarepp_status flarepp_spectrum(const flarepp_desc *desc, const void *S, const void *K,
                                const void *V, float *eig, float *sym_out, void *ws,
                                size_t ws_bytes, void *stream);

/*
 * Explicit launch choices, for split-invariance tests and tuning sweeps.  A
 * zero field keeps the library's own choice, which depends on the descriptor
 * only.  The result is the same softmax up to rounding for every choice: the
 * token splits are combined exactly from their (max, sum, accumulator)
 * statistics, the combination the French technical summary gives for
 * token-sharded devices ("Contributions Clés", context parallelism).
 *   splits            token splits per (b, h) in the encodes (rounded so that
 *                     every split is a whole number of encode tiles; values
 *                     above the tile count are clamped to it)
 *   head_group        (b, h) pairs per launch (1 .. 65535; clamped to B*H)
 *   decode_kernel     1 = the paired two-wave decode (bf16, M > 128 only),
 *                     2 = the single-wave decode
 *   decode_wg_per_cu  paired decode: workgroups per compute unit that the
 *                     token chunking targets
 * Negative fields are INVALID_ARG.
 */
typedef struct flarepp_tuning {
    int32_t splits;
    int32_t head_group;
    int32_t decode_kernel;
    int32_t decode_wg_per_cu;
} flarepp_tuning;

/*
 * flarepp_workspace_size for the launch choices in `tuning` (NULL = the
 * library's own, identical to flarepp_workspace_size).
 */
flarepp_status flarepp_workspace_size_tuned(const flarepp_desc *desc, int32_t op,
                                            const flarepp_tuning *tuning, size_t *bytes);

/*
 * flarepp_route with the launch choices in `tuning` (NULL = the library's
 * own); the workspace must be sized by flarepp_workspace_size_tuned with the
 * same tuning and FLAREPP_OP_ROUTE.
 */
flarepp_status flarepp_route_tuned(const flarepp_desc *desc, const flarepp_tuning *tuning,
                                   const void *S, const void *K, const void *V, float *Y,
                                   float *Qd_out, float *Z_out, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * flarepp_route for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The caller passes the inputs and outputs only; the workspace is a device
 * array built into the library (flarepp_noalloc_scratch_bytes() bytes, 64
 * MiB; each GPU the library runs on holds its own copy until the process
 * ends).  The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first call on a device looks up that device's array address.
 * Returns FLAREPP_SCRATCH_LIMIT, before any GPU work, when the problem needs
 * more workspace than the array holds (flarepp_workspace_size with
 * FLAREPP_OP_ROUTE gives the need).  All calls on one GPU share the array:
 * calls whose work overlaps in time on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller.  Results are
 * bitwise those of flarepp_route.
 */
flarepp_status flarepp_route_noalloc(const flarepp_desc *desc, const void *S, const void *K,
                                     const void *V, float *Y, float *Qd_out, float *Z_out,
                                     void *stream);

/* Bytes of the built-in scratch of flarepp_route_noalloc. */
size_t flarepp_noalloc_scratch_bytes(void);

/*
 * Token shards (context parallelism; French technical summary, "Contributions
 * Clés": the tokens are split across devices and only the latent outputs and
 * the softmax statistics are exchanged).  A device holding tokens
 * [n0, n1) of every (b, h) runs an encode stage over them alone and emits,
 * per latent row, the shard's combined record (acc = sum of w V, lambda =
 * sum of w, mu = the shift, in log2 units, with w = 2^(c <q, k> - mu));
 * records of all shards, merged, give the stage's rows exactly as the
 * split-N merge does within one device.  The decode needs no exchange: run
 * flarepp_decode on each shard with the merged Qd and Z.
 *
 * Records: float32, [B*H][Mp][nslots][D + 4] with Mp = M rounded up to a
 * multiple of 16; element d < D of a record is acc_d, element D is lambda,
 * element D + 1 is mu (D + 2, D + 3 unused).  flarepp_shard_records_size
 * gives the bytes of a buffer for nslots shards.
 *
 * flarepp_encode_shard: desc describes this shard (N = its token count; B, H,
 * M, D, dtype, scale, seed_head_stride as for the whole problem); K and V
 * hold its tokens (B x H x N x D, desc dtype).  stage 1: Q = the seeds S (as
 * in flarepp_seed_encode), giving Qd's records; stage 2: Q = Qd (float32
 * rows B x H x M x D, the merged stage-1 result), giving Z's records.  The
 * call writes slot `slot` (0 <= slot < nslots) of every record of `rec` and
 * nothing else.  Workspace: flarepp_workspace_size with
 * FLAREPP_OP_SEED_ENCODE (stage 1) or FLAREPP_OP_ENCODE (stage 2) for this
 * desc.  INVALID_ARG for another stage or slot.
 *
 * flarepp_merge_shards: desc describes the whole problem (its N is not
 * used); out (B x H x M x D float32) receives the merged rows -- Qd after
 * stage 1, Z after stage 2.  No workspace.  Every slot of rec must have been
 * written.
 */
flarepp_status flarepp_shard_records_size(const flarepp_desc *desc, int32_t nslots, size_t *bytes);
flarepp_status flarepp_encode_shard(const flarepp_desc *desc, int32_t stage, const void *Q,
                                    const void *K, const void *V, float *rec, int32_t slot,
                                    int32_t nslots, void *ws, size_t ws_bytes, void *stream);
flarepp_status flarepp_merge_shards(const flarepp_desc *desc, const float *rec, int32_t nslots,
                                    float *out, void *stream);

/* Kernel kinds reported by flarepp_route_profiled. */
typedef enum flarepp_kernel_kind {
    FLAREPP_KERNEL_PREP = 0,        /* query / value operand preparation */
    FLAREPP_KERNEL_SEED_ENCODE = 1, /* split-N seed encode */
    FLAREPP_KERNEL_ENCODE = 2,      /* split-N encode */
    FLAREPP_KERNEL_MERGE = 3,       /* merge of split partials */
    FLAREPP_KERNEL_DECODE = 4       /* decode */
} flarepp_kernel_kind;

/*
 * Instrumented flarepp_route for measurement: identical work, plus events
 * recorded on `stream` around every kernel launch.  events: 2*max_launches
 * hipEvent_t handles created by the caller; launch i records events[2i]
 * before and events[2i+1] after it and stores its flarepp_kernel_kind in
 * kinds[i].  *n_launches receives the number of launches (which may exceed
 * max_launches; launches beyond it are not recorded).  A failed event
 * record is reported as FLAREPP_HIP_ERROR.
 */
flarepp_status flarepp_route_profiled(const flarepp_desc *desc, const void *S, const void *K,
                                      const void *V, float *Y, float *Qd_out, float *Z_out,
                                      void *ws, size_t ws_bytes, void *stream, void **events,
                                      int32_t *kinds, int32_t max_launches, int32_t *n_launches);

#ifdef __cplusplus
}
#endif

#endif /* FLAREPP_H */
