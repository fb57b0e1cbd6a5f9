/*
 * flarepp_oracle.c -- plain, slow, obviously correct CPU reference for the
 * FLARE++ routing forward pass.  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the benchmark's CPU-baseline leg may call it; the library
 * under rank_latent_attention_seed_amd/ never does, and the two share no
 * source, header, helper or table.
 *
 * Arithmetic: IEEE double throughout, one thread, no BLAS, no blocking, no
 * fusion.  Inputs are read as their exact stored values (fp32, bf16 bit
 * patterns, or fp64) and widened to double before any arithmetic.
 *
 * What it computes, per (batch b, head h):
 *
 *   SDPA(Q, K, V, s)_i = sum_j softmax_j( s * <Q_i, K_j> ) * V_j
 *       -- the scaled-dot-product-attention form that the FLARE summary
 *          ("FLARE: Fast Low-rank Attention Routing Engine", section
 *          "Основной механизм FLARE") uses for both of its steps; the
 *          softmax runs over the key index j (the rows of W_encode and
 *          W_decode are softmax-normalised, same page, section
 *          "Матрица коммуникации низкого ранга").
 *
 *   stage 1 (seed encode):  Qd = SDPA(S_h, K, V, s)      M x D
 *       -- "FLARE++: Low-rank attention with dynamic attention routing",
 *          abstract: learned latent seeds drive one extra encode call over
 *          the same N tokens; French technical summary, "Méthodologie",
 *          "Synthèse de Requêtes Dynamiques".
 *   stage 2 (encode):       Z  = SDPA(Qd, K, V, s)       M x D
 *   stage 3 (decode):       Y  = SDPA(K, Qd, Z, s)       N x D
 *       -- FLARE's encode/decode pair with the synthesised queries in place
 *          of the fixed ones (French summary, "Routage Encode-Décode"); no
 *          processing happens between the stages (same section: no separate
 *          latent-processing step).
 *
 * The softmax subtracts the row maximum before exponentiating (exact in real
 * arithmetic: softmax is invariant to a common shift), and uses exp() from
 * libm.  The pages give the scale as s = 1 for FLARE; here s is a parameter
 * and the same s is used in all three stages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to double. */
static double oracle_load(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORACLE_BF16) {
        /* a bf16 value is the top 16 bits of the fp32 with the same value */
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double *)base)[idx];
}

static size_t oracle_elem_size(int dtype)
{
    return dtype == ORACLE_F32 ? 4u : dtype == ORACLE_BF16 ? 2u : 8u;
}

static const void *oracle_offset(const void *base, int dtype, int64_t elems)
{
    return (const char *)base + (size_t)elems * oracle_elem_size(dtype);
}

/*
 * One SDPA application.  q: nq x d, k: nk x d, v: nk x dv (row-major),
 * out: nq x dv doubles.  Returns 0 on success, -1 on bad arguments or
 * allocation failure.
 */
int oracle_sdpa(const void *q, int q_dtype, int64_t nq,
                const void *k, int k_dtype,
                const void *v, int v_dtype, int64_t nk,
                int64_t d, int64_t dv, double s, double *out)
{
    if (nq < 0 || nk < 1 || d < 1 || dv < 1 || !out)
        return -1;
    if (nq == 0)
        return 0;
    if (!q || !k || !v)
        return -1;
    double *logit = (double *)malloc((size_t)nk * sizeof(double));
    if (!logit)
        return -1;
    for (int64_t i = 0; i < nq; ++i) {
        /* logits l_j = s * <q_i, k_j> */
        double lmax = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
            double dot = 0.0;
            for (int64_t e = 0; e < d; ++e)
                dot += oracle_load(q, q_dtype, i * d + e) *
                       oracle_load(k, k_dtype, j * d + e);
            logit[j] = s * dot;
            if (logit[j] > lmax)
                lmax = logit[j];
        }
        /* softmax over j, then the weighted sum of the value rows */
        double denom = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            logit[j] = exp(logit[j] - lmax);
            denom += logit[j];
        }
        for (int64_t e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int64_t j = 0; j < nk; ++j)
                acc += logit[j] * oracle_load(v, v_dtype, j * dv + e);
            out[i * dv + e] = acc / denom;
        }
    }
    free(logit);
    return 0;
}

static int oracle_check_dims(int64_t B, int64_t H, int64_t N, int64_t M,
                             int64_t D, int dtype, int64_t q_head_stride)
{
    if (B < 1 || H < 1 || N < 1 || M < 1 || D < 1)
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (q_head_stride != 0 && q_head_stride != M * D)
        return -1;
    return 0;
}

/*
 * The full route for every (b, h).  S: M x D (q_head_stride = 0, one seed
 * block shared by all heads) or H x M x D (q_head_stride = M*D).  K, V:
 * B x H x N x D.  Outputs Qd, Z: B x H x M x D doubles; Y: B x H x N x D
 * doubles.  Qd or Z may be NULL when the caller does not want them (Y is
 * required).
 */
int oracle_route(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                 int dtype, double s, int64_t q_head_stride,
                 const void *S, const void *K, const void *V,
                 double *Qd, double *Z, double *Y)
{
    if (oracle_check_dims(B, H, N, M, D, dtype, q_head_stride) || !S || !K ||
        !V || !Y)
        return -1;
    double *qd = (double *)malloc((size_t)(M * D) * sizeof(double));
    double *z = (double *)malloc((size_t)(M * D) * sizeof(double));
    if (!qd || !z) {
        free(qd);
        free(z);
        return -1;
    }
    int rc = 0;
    for (int64_t b = 0; b < B && rc == 0; ++b) {
        for (int64_t h = 0; h < H && rc == 0; ++h) {
            int64_t bh = b * H + h;
            const void *Sh = oracle_offset(S, dtype, h * q_head_stride);
            const void *Kbh = oracle_offset(K, dtype, bh * N * D);
            const void *Vbh = oracle_offset(V, dtype, bh * N * D);
            /* stage 1: seeds gather the tokens into M routing queries */
            rc |= oracle_sdpa(Sh, dtype, M, Kbh, dtype, Vbh, dtype, N, D, D, s, qd);
            /* stage 2: the routing queries compress the same tokens */
            rc |= oracle_sdpa(qd, ORACLE_F64, M, Kbh, dtype, Vbh, dtype, N, D, D, s, z);
            /* stage 3: each token reads the latents back, softmax over M */
            rc |= oracle_sdpa(Kbh, dtype, N, qd, ORACLE_F64, z, ORACLE_F64, M, D, D,
                              s, Y + bh * N * D);
            if (Qd)
                memcpy(Qd + bh * M * D, qd, (size_t)(M * D) * sizeof(double));
            if (Z)
                memcpy(Z + bh * M * D, z, (size_t)(M * D) * sizeof(double));
        }
    }
    free(qd);
    free(z);
    return rc ? -1 : 0;
}

/*
 * Fixed-query FLARE (the predecessor the FLARE++ abstract contrasts with):
 * the latent queries Q are parameters, Z = SDPA(Q, K, V, s) and
 * Y = SDPA(K, Q, Z, s).  Same layouts as oracle_route with Q in place of S.
 */
int oracle_flare(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                 int dtype, double s, int64_t q_head_stride,
                 const void *Q, const void *K, const void *V,
                 double *Z, double *Y)
{
    if (oracle_check_dims(B, H, N, M, D, dtype, q_head_stride) || !Q || !K ||
        !V || !Y)
        return -1;
    double *z = (double *)malloc((size_t)(M * D) * sizeof(double));
    if (!z)
        return -1;
    int rc = 0;
    for (int64_t b = 0; b < B && rc == 0; ++b) {
        for (int64_t h = 0; h < H && rc == 0; ++h) {
            int64_t bh = b * H + h;
            const void *Qh = oracle_offset(Q, dtype, h * q_head_stride);
            const void *Kbh = oracle_offset(K, dtype, bh * N * D);
            const void *Vbh = oracle_offset(V, dtype, bh * N * D);
            rc |= oracle_sdpa(Qh, dtype, M, Kbh, dtype, Vbh, dtype, N, D, D, s, z);
            rc |= oracle_sdpa(Kbh, dtype, N, Qh, dtype, z, ORACLE_F64, M, D, D, s,
                              Y + bh * N * D);
            if (Z)
                memcpy(Z + bh * M * D, z, (size_t)(M * D) * sizeof(double));
        }
    }
    free(z);
    return rc ? -1 : 0;
}
