// Drives libflarepp's host side -- descriptor and tuning checks, workspace
// planning, pointer, alignment and aliasing validation -- under
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py
// builds it with the library's source and runs it, without a GPU).  Every
// compute call here fails validation and returns before any HIP call.
#include <cstdint>
#include <cstdio>
#include <limits>

#include "flarepp.h"

static int failures = 0;
#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    const int got_ = (int)(call);                                                           \
    if (got_ != (int)(want)) {                                                              \
      std::fprintf(stderr, "FAILED line %d: %s -> %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

static void* addr(int i) { return reinterpret_cast<void*>((uintptr_t(1) << 40) + uintptr_t(i) * (uintptr_t(1) << 34)); }
static float* faddr(int i) { return static_cast<float*>(addr(i)); }

int main() {
  const flarepp_desc good = {2, 3, 1000, 64, 32, FLAREPP_BF16, 0.25f, 0};
  size_t n = 0;
  // workspace sizes over every op, dtype and a range of shapes
  const int64_t Ns[] = {1, 2, 31, 4097, 1 << 20};
  const int64_t Ms[] = {1, 16, 17, 128, 129, 256};
  for (int op = 0; op <= FLAREPP_OP_SPECTRUM; ++op)
    for (int dt = 0; dt < 2; ++dt)
      for (int64_t N : Ns)
        for (int64_t M : Ms) {
          flarepp_desc d = {1, 8, N, M, 32, dt, 0.2f, 0};
          const flarepp_status want = FLAREPP_OK;
          EXPECT(flarepp_workspace_size(&d, op, &n), want);
          for (int32_t sp : {1, 3, 1000000}) {
            flarepp_tuning t = {sp, 2, 0, 0};
            EXPECT(flarepp_workspace_size_tuned(&d, op, &t, &n), want);
          }
        }
  // descriptor errors
  flarepp_desc d = good;
  d.N = 0;
  EXPECT(flarepp_workspace_size(&d, FLAREPP_OP_ROUTE, &n), FLAREPP_INVALID_ARG);
  d = good; d.D = 24;
  EXPECT(flarepp_workspace_size(&d, FLAREPP_OP_ROUTE, &n), FLAREPP_UNSUPPORTED);
  d = good; d.M = 257;
  EXPECT(flarepp_workspace_size(&d, FLAREPP_OP_ROUTE, &n), FLAREPP_UNSUPPORTED);
  d = good; d.scale = std::numeric_limits<float>::infinity();
  EXPECT(flarepp_workspace_size(&d, FLAREPP_OP_ROUTE, &n), FLAREPP_INVALID_ARG);
  d = good; d.seed_head_stride = 7;
  EXPECT(flarepp_workspace_size(&d, FLAREPP_OP_ROUTE, &n), FLAREPP_INVALID_ARG);
  d = good; d.B = std::numeric_limits<int64_t>::max();
  EXPECT(flarepp_workspace_size(&d, FLAREPP_OP_ROUTE, &n), FLAREPP_UNSUPPORTED);
  d = good; d.N = std::numeric_limits<int64_t>::max() / 2;
  EXPECT(flarepp_workspace_size(&d, FLAREPP_OP_ROUTE, &n), FLAREPP_UNSUPPORTED);
  EXPECT(flarepp_workspace_size(nullptr, FLAREPP_OP_ROUTE, &n), FLAREPP_INVALID_ARG);
  EXPECT(flarepp_workspace_size(&good, 99, &n), FLAREPP_INVALID_ARG);
  EXPECT(flarepp_workspace_size(&good, FLAREPP_OP_ROUTE, nullptr), FLAREPP_INVALID_ARG);
  flarepp_tuning bad = {-1, 0, 0, 0};
  EXPECT(flarepp_workspace_size_tuned(&good, FLAREPP_OP_ROUTE, &bad, &n), FLAREPP_INVALID_ARG);

  // compute calls that fail validation
  size_t ws = 0;
  EXPECT(flarepp_workspace_size(&good, FLAREPP_OP_ROUTE, &ws), FLAREPP_OK);
  EXPECT(flarepp_route(&good, addr(0), addr(1), addr(2), faddr(3), nullptr, nullptr, addr(6), ws - 1, nullptr),
         FLAREPP_WORKSPACE_TOO_SMALL);
  EXPECT(flarepp_route(&good, addr(0), addr(1), addr(2), faddr(1), nullptr, nullptr, addr(6), ws, nullptr),
         FLAREPP_ALIASING);
  EXPECT(flarepp_route(&good, nullptr, addr(1), addr(2), faddr(3), nullptr, nullptr, addr(6), ws, nullptr),
         FLAREPP_INVALID_ARG);
  EXPECT(flarepp_route(&good, addr(0), static_cast<char*>(addr(1)) + 2, addr(2), faddr(3), nullptr, nullptr,
                       addr(6), ws, nullptr),
         FLAREPP_INVALID_ARG);
  flarepp_tuning t = {4, 0, 0, 0};
  EXPECT(flarepp_route_tuned(&good, &t, addr(0), addr(1), addr(2), faddr(3), faddr(4), faddr(4), addr(6),
                             size_t(1) << 40, nullptr),
         FLAREPP_ALIASING);
  EXPECT(flarepp_seed_encode(&good, addr(0), addr(1), addr(2), nullptr, addr(6), ws, nullptr), FLAREPP_INVALID_ARG);
  EXPECT(flarepp_encode(&good, faddr(0), addr(1), addr(2), faddr(0), addr(6), ws, nullptr), FLAREPP_ALIASING);
  EXPECT(flarepp_decode(&good, faddr(0), faddr(1), addr(2), faddr(3), addr(6), 0, nullptr),
         FLAREPP_WORKSPACE_TOO_SMALL);
  EXPECT(flarepp_flare(&good, addr(0), addr(1), nullptr, faddr(3), nullptr, addr(6), ws, nullptr),
         FLAREPP_INVALID_ARG);
  EXPECT(flarepp_spectrum(&good, addr(0), addr(1), addr(2), faddr(1), nullptr, addr(6), size_t(1) << 40, nullptr),
         FLAREPP_ALIASING);
  EXPECT(flarepp_route_backward(&good, addr(0), addr(1), addr(2), faddr(3), faddr(1), faddr(5), faddr(7), addr(6),
                                size_t(1) << 40, nullptr),
         FLAREPP_ALIASING);  // dS inside K
  // the saved-forward pair: seven inputs plus the workspace in one aliasing check
  EXPECT(flarepp_route_save(&good, addr(0), addr(1), addr(2), faddr(3), faddr(4), faddr(5), faddr(1), addr(6),
                            size_t(1) << 40, nullptr),
         FLAREPP_ALIASING);  // the log-sum-exps inside K
  EXPECT(flarepp_route_save(&good, addr(0), addr(1), addr(2), faddr(3), faddr(4), faddr(5), nullptr, addr(6),
                            size_t(1) << 40, nullptr),
         FLAREPP_INVALID_ARG);
  EXPECT(flarepp_route_backward_saved(&good, addr(0), addr(1), addr(2), faddr(3), faddr(4), faddr(5), faddr(8),
                                      faddr(9), faddr(10), faddr(4), addr(6), size_t(1) << 40, nullptr),
         FLAREPP_ALIASING);  // dV inside the saved Z
  EXPECT(flarepp_route_backward_saved(&good, addr(0), addr(1), addr(2), faddr(3), faddr(4), faddr(5), faddr(8),
                                      faddr(9), faddr(10), faddr(11), addr(6), 0, nullptr),
         FLAREPP_WORKSPACE_TOO_SMALL);
  size_t recb = 0;
  EXPECT(flarepp_shard_records_size(&good, 3, &recb), FLAREPP_OK);
  EXPECT(flarepp_shard_records_size(&good, 0, &recb), FLAREPP_INVALID_ARG);
  EXPECT(flarepp_encode_shard(&good, 1, addr(0), addr(1), addr(2), faddr(4), 3, 3, addr(6), size_t(1) << 40, nullptr),
         FLAREPP_INVALID_ARG);  // slot beyond the slots
  EXPECT(flarepp_encode_shard(&good, 2, faddr(0), addr(1), addr(2), faddr(1), 0, 2, addr(6), size_t(1) << 40,
                              nullptr),
         FLAREPP_ALIASING);  // records inside K
  EXPECT(flarepp_merge_shards(&good, faddr(4), 2, faddr(4), nullptr), FLAREPP_ALIASING);
  flarepp_desc big = {64, 64, 4096, 256, 32, FLAREPP_BF16, 0.2f, 0};
  EXPECT(flarepp_route_noalloc(&big, addr(0), addr(1), addr(2), faddr(3), nullptr, nullptr, nullptr),
         FLAREPP_SCRATCH_LIMIT);
  EXPECT(flarepp_route_noalloc(&good, addr(0), addr(1), addr(2), nullptr, nullptr, nullptr, nullptr),
         FLAREPP_INVALID_ARG);
  void* events[2] = {nullptr, nullptr};
  int32_t kinds[1];
  int32_t nl = 0;
  EXPECT(flarepp_route_profiled(&good, addr(0), addr(1), addr(2), faddr(3), nullptr, nullptr, addr(6), ws - 1,
                                nullptr, events, kinds, 1, &nl),
         FLAREPP_WORKSPACE_TOO_SMALL);
  for (int s = 0; s <= 7; ++s) (void)flarepp_status_string(static_cast<flarepp_status>(s));
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host driver: all checks passed\n");
  return 0;
}
