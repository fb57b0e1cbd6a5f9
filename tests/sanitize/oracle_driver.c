/*
 * Drives the oracle's C entry points under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py builds and runs it):
 * every dtype, shared and per-head seeds, edge shapes (N = 1, M = 1, M > N,
 * D = 1) and the argument errors, with every returned value checked finite.
 * Test infrastructure only; it links the oracle's own source.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_sdpa(const void *q, int q_dtype, int64_t nq, const void *k, int k_dtype, const void *v, int v_dtype,
                int64_t nk, int64_t d, int64_t dv, double s, double *out);
int oracle_route(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, double s, int64_t q_head_stride,
                 const void *S, const void *K, const void *V, double *Qd, double *Z, double *Y);
int oracle_flare(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, double s, int64_t q_head_stride,
                 const void *Q, const void *K, const void *V, double *Z, double *Y);
int oracle_route_backward(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, double s,
                          int64_t q_head_stride, const void *S, const void *K, const void *V, const double *dY,
                          double *dS, double *dK, double *dV);

enum { F32 = 0, BF16 = 1, F64 = 2 };

static uint64_t rng = 88172645463325252ull;
static double uniform(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

/* n random values of the dtype, in a buffer of exactly that many elements */
static void *draw(int dtype, int64_t n) {
    size_t es = dtype == BF16 ? 2 : dtype == F32 ? 4 : 8;
    void *p = malloc((size_t)n * es);
    for (int64_t i = 0; i < n; ++i) {
        double x = 2.0 * uniform();
        if (dtype == F64) {
            ((double *)p)[i] = x;
        } else {
            float f = (float)x;
            if (dtype == F32) {
                ((float *)p)[i] = f;
            } else {
                uint32_t u;
                memcpy(&u, &f, 4);
                ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
            }
        }
    }
    return p;
}

static int failures = 0;
#define CHECK(cond, what)                                              \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static int finite_all(const double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i]))
            return 0;
    return 1;
}

static void one_case(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, double s, int per_head) {
    const int64_t ns = per_head ? H : 1, stride = per_head ? M * D : 0;
    void *S = draw(dtype, ns * M * D), *K = draw(dtype, B * H * N * D), *V = draw(dtype, B * H * N * D);
    double *Qd = malloc((size_t)(B * H * M * D) * 8), *Z = malloc((size_t)(B * H * M * D) * 8);
    double *Y = malloc((size_t)(B * H * N * D) * 8), *dY = malloc((size_t)(B * H * N * D) * 8);
    double *dS = malloc((size_t)(ns * M * D) * 8), *dK = malloc((size_t)(B * H * N * D) * 8);
    double *dV = malloc((size_t)(B * H * N * D) * 8);
    for (int64_t i = 0; i < B * H * N * D; ++i) dY[i] = uniform();
    CHECK(oracle_route(B, H, N, M, D, dtype, s, stride, S, K, V, Qd, Z, Y) == 0, "route");
    CHECK(finite_all(Qd, B * H * M * D) && finite_all(Z, B * H * M * D) && finite_all(Y, B * H * N * D),
          "route outputs finite");
    CHECK(oracle_route(B, H, N, M, D, dtype, s, stride, S, K, V, NULL, NULL, Y) == 0, "route, Y only");
    CHECK(oracle_flare(B, H, N, M, D, dtype, s, stride, S, K, V, Z, Y) == 0, "flare");
    CHECK(finite_all(Y, B * H * N * D), "flare outputs finite");
    CHECK(oracle_route_backward(B, H, N, M, D, dtype, s, stride, S, K, V, dY, dS, dK, dV) == 0, "backward");
    CHECK(finite_all(dS, ns * M * D) && finite_all(dK, B * H * N * D) && finite_all(dV, B * H * N * D),
          "backward outputs finite");
    free(S); free(K); free(V); free(Qd); free(Z); free(Y); free(dY); free(dS); free(dK); free(dV);
}

int main(void) {
    const int dtypes[3] = {F32, BF16, F64};
    for (int t = 0; t < 3; ++t) {
        one_case(1, 2, 37, 5, 8, dtypes[t], 0.35, 0);
        one_case(2, 1, 64, 16, 32, dtypes[t], 1.0, 0);
        one_case(1, 3, 20, 7, 16, dtypes[t], 0.25, 1);
        one_case(1, 1, 1, 1, 1, dtypes[t], 1.0, 0);     /* N = M = D = 1 */
        one_case(1, 2, 3, 9, 4, dtypes[t], -0.5, 1);    /* M > N, s < 0 */
        one_case(1, 1, 50, 4, 16, dtypes[t], 0.0, 0);   /* s = 0 */
    }
    /* argument errors return -1 without touching memory */
    double out[4];
    float q[4] = {0};
    CHECK(oracle_sdpa(q, F32, 1, q, F32, q, F32, 0, 4, 1, 1.0, out) == -1, "sdpa nk = 0");
    CHECK(oracle_sdpa(q, F32, 1, q, F32, q, F32, 1, 0, 1, 1.0, out) == -1, "sdpa d = 0");
    CHECK(oracle_sdpa(NULL, F32, 1, q, F32, q, F32, 1, 4, 1, 1.0, out) == -1, "sdpa null q");
    CHECK(oracle_sdpa(q, F32, 0, q, F32, q, F32, 1, 4, 1, 1.0, out) == 0, "sdpa nq = 0");
    CHECK(oracle_route(1, 1, 0, 1, 4, F32, 1.0, 0, q, q, q, NULL, NULL, out) == -1, "route N = 0");
    CHECK(oracle_route(1, 1, 1, 1, 4, 7, 1.0, 0, q, q, q, NULL, NULL, out) == -1, "route bad dtype");
    CHECK(oracle_route(1, 1, 1, 1, 4, F32, 1.0, 3, q, q, q, NULL, NULL, out) == -1, "route bad stride");
    CHECK(oracle_route(1, 1, 1, 1, 4, F32, 1.0, 0, q, q, q, NULL, NULL, NULL) == -1, "route null Y");
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
