/*
 * flarepp_oracle.c -- plain, slow, obviously correct CPU reference for the
 * FLARE++ routing forward pass and its backward (the gradients of a scalar
 * loss with respect to the seeds, keys and values, by the chain rule through
 * the same three stages; see oracle_route_backward at the end).  TEST
 * INFRASTRUCTURE ONLY: the tests, the
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

/*
 * Backward of one SDPA application out = SDPA(q, k, v, s), given the
 * gradient dout (nq x dv doubles) of a scalar loss with respect to out.
 * With P_ij = softmax_j(s <q_i, k_j>) recomputed from the inputs:
 *
 *   dv_j  += sum_i P_ij dout_i                          (out is linear in v)
 *   dP_ij  = <dout_i, v_j>
 *   dL_ij  = P_ij (dP_ij - sum_j' P_ij' dP_ij')         (softmax Jacobian)
 *   dq_i  += s sum_j dL_ij k_j                          (L_ij = s <q_i, k_j>)
 *   dk_j  += s sum_i dL_ij q_i
 *
 * -- the chain rule through the SDPA form of the FLARE summary ("Основной
 * механизм FLARE").  dq (nq x d), dk (nk x d) and dvv (nk x dv) are doubles
 * that this call adds into; any of them may be NULL.  Returns 0, or -1 on
 * bad arguments or allocation failure.
 */
int oracle_sdpa_backward(const void *q, int q_dtype, int64_t nq,
                         const void *k, int k_dtype,
                         const void *v, int v_dtype, int64_t nk,
                         int64_t d, int64_t dv, double s, const double *dout,
                         double *dq, double *dk, double *dvv)
{
    if (nq < 0 || nk < 1 || d < 1 || dv < 1 || !dout)
        return -1;
    if (nq == 0)
        return 0;
    if (!q || !k || !v)
        return -1;
    double *p = (double *)malloc((size_t)nk * sizeof(double));
    double *dp = (double *)malloc((size_t)nk * sizeof(double));
    if (!p || !dp) {
        free(p);
        free(dp);
        return -1;
    }
    for (int64_t i = 0; i < nq; ++i) {
        /* the softmax row P_i. */
        double lmax = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
            double dot = 0.0;
            for (int64_t e = 0; e < d; ++e)
                dot += oracle_load(q, q_dtype, i * d + e) *
                       oracle_load(k, k_dtype, j * d + e);
            p[j] = s * dot;
            if (p[j] > lmax)
                lmax = p[j];
        }
        double denom = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            p[j] = exp(p[j] - lmax);
            denom += p[j];
        }
        for (int64_t j = 0; j < nk; ++j)
            p[j] /= denom;
        /* value gradient and the gradient with respect to P_i. */
        double pdp = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            double dot = 0.0;
            for (int64_t e = 0; e < dv; ++e) {
                dot += dout[i * dv + e] * oracle_load(v, v_dtype, j * dv + e);
                if (dvv)
                    dvv[j * dv + e] += p[j] * dout[i * dv + e];
            }
            dp[j] = dot;
            pdp += p[j] * dot;
        }
        /* through the softmax to the logits, then to q and k */
        for (int64_t j = 0; j < nk; ++j) {
            double dl = p[j] * (dp[j] - pdp);
            for (int64_t e = 0; e < d; ++e) {
                if (dq)
                    dq[i * d + e] += s * dl * oracle_load(k, k_dtype, j * d + e);
                if (dk)
                    dk[j * d + e] += s * dl * oracle_load(q, q_dtype, i * d + e);
            }
        }
    }
    free(p);
    free(dp);
    return 0;
}

/*
 * Backward of the full route: given dY (B x H x N x D doubles), the
 * gradients dS (M x D when q_head_stride = 0 -- one seed block shared by
 * all (b, h), so its gradient sums over them -- or H x M x D), dK and dV
 * (B x H x N x D), all doubles, overwritten.  Per (b, h) the forward is
 * recomputed and the three stages are taken in reverse:
 *   stage 3  Y  = SDPA(K, Qd, Z):  dY -> dK, dQd, dZ
 *   stage 2  Z  = SDPA(Qd, K, V):  dZ -> dQd, dK, dV
 *   stage 1  Qd = SDPA(S, K, V):   dQd (both contributions) -> dS, dK, dV
 * Qd reaches the loss through stage 2 (as the query) and stage 3 (as the
 * key), so its gradient is the sum of both before stage 1 uses it.
 */
int oracle_route_backward(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                          int dtype, double s, int64_t q_head_stride,
                          const void *S, const void *K, const void *V,
                          const double *dY, double *dS, double *dK, double *dV)
{
    if (oracle_check_dims(B, H, N, M, D, dtype, q_head_stride) || !S || !K ||
        !V || !dY || !dS || !dK || !dV)
        return -1;
    const int64_t ns = q_head_stride ? H : 1;
    memset(dS, 0, (size_t)(ns * M * D) * sizeof(double));
    memset(dK, 0, (size_t)(B * H * N * D) * sizeof(double));
    memset(dV, 0, (size_t)(B * H * N * D) * sizeof(double));
    double *qd = (double *)malloc((size_t)(M * D) * sizeof(double));
    double *z = (double *)malloc((size_t)(M * D) * sizeof(double));
    double *dqd = (double *)malloc((size_t)(M * D) * sizeof(double));
    double *dz = (double *)malloc((size_t)(M * D) * sizeof(double));
    if (!qd || !z || !dqd || !dz) {
        free(qd);
        free(z);
        free(dqd);
        free(dz);
        return -1;
    }
    int rc = 0;
    for (int64_t b = 0; b < B && rc == 0; ++b) {
        for (int64_t h = 0; h < H && rc == 0; ++h) {
            int64_t bh = b * H + h;
            const void *Sh = oracle_offset(S, dtype, h * q_head_stride);
            const void *Kbh = oracle_offset(K, dtype, bh * N * D);
            const void *Vbh = oracle_offset(V, dtype, bh * N * D);
            double *dKbh = dK + bh * N * D, *dVbh = dV + bh * N * D;
            /* forward */
            rc |= oracle_sdpa(Sh, dtype, M, Kbh, dtype, Vbh, dtype, N, D, D, s, qd);
            rc |= oracle_sdpa(qd, ORACLE_F64, M, Kbh, dtype, Vbh, dtype, N, D, D, s, z);
            memset(dqd, 0, (size_t)(M * D) * sizeof(double));
            memset(dz, 0, (size_t)(M * D) * sizeof(double));
            /* stage 3: queries K, keys Qd, values Z */
            rc |= oracle_sdpa_backward(Kbh, dtype, N, qd, ORACLE_F64, z, ORACLE_F64, M, D, D,
                                       s, dY + bh * N * D, dKbh, dqd, dz);
            /* stage 2: queries Qd, keys K, values V */
            rc |= oracle_sdpa_backward(qd, ORACLE_F64, M, Kbh, dtype, Vbh, dtype, N, D, D,
                                       s, dz, dqd, dKbh, dVbh);
            /* stage 1: queries S, keys K, values V, upstream dQd */
            double *dSh = dS + (q_head_stride ? h * M * D : 0);
            rc |= oracle_sdpa_backward(Sh, dtype, M, Kbh, dtype, Vbh, dtype, N, D, D,
                                       s, dqd, dSh, dKbh, dVbh);
        }
    }
    free(qd);
    free(z);
    free(dqd);
    free(dz);
    return rc ? -1 : 0;
}
