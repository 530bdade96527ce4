// Drives every entry point of include/ckda.h through its argument checks and,
// when no GPU is visible, on through the host side of its launches (which
// then fail with CKDA_ERR_HIP), for a build of the library's host code with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizer.py).
// Device pointers are fake addresses that the host code never dereferences.
// Exit status 0 means every call returned the expected status.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ckda.h"

static int failures = 0;
static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, got, want, ckda_last_error());
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static void* P(uintptr_t off) { return (void*)((uintptr_t)0x7F0000000000ull + off); }
static const uintptr_t MB = 1u << 20;

int main() {
  int ndev = 0;
  const bool gpu = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0;
  // accepted arguments launch: only where no GPU can run the fake pointers
  const int LAUNCH = CKDA_ERR_HIP;

  EXPECT(ckda_abi_version(), CKDA_ABI_VERSION);
  for (int s = -1; s < 10; ++s) (void)strlen(ckda_status_string(s));
  (void)strlen(ckda_last_error());

  // workspace sizes
  EXPECT(ckda_chunk_fwd_workspace_size(1, 1, 64, 128, 128, 64, 1) > 0, 1);
  EXPECT(ckda_chunk_fwd_workspace_size(-1, 1, 64, 128, 128, 64, 1) == 0, 1);
  EXPECT(ckda_chunk_fwd_workspace_size(1, 1, 64, 96, 128, 64, 1) == 0, 1);
  EXPECT(ckda_chunk_bwd_workspace_size(4, 16, 4096, 128, 128, 1) > 0, 1);
  EXPECT(ckda_chunk_bwd_ex_workspace_size(4, 16, 4096, 128, 128, 1, 15) > 0, 1);
  EXPECT(ckda_chunk_bwd_ex_workspace_size(4, 16, 4096, 128, 128, 1, 16) == 0, 1);
  EXPECT(ckda_deltaproduct2_bwd_workspace_size(1, 2, 64, 64, 64, 0) > 0, 1);
  EXPECT(ckda_deltaproduct2_bwd_workspace_size(1, 2, 1 << 30, 64, 64, 0) == 0, 1);

  // chunked forward: q k v alpha beta h0 o hT at 1 MB steps, workspace at 8 MB
  const int B = 1, H = 2, T = 100, dk = 64, dv = 64, C = 64;
  const size_t ws = ckda_chunk_fwd_workspace_size(B, H, T, dk, dv, C, 1);
  auto fwd = [&](void* q, void* o, void* w, size_t wsb, int dkk, int flags) {
    return ckda_chunk_fwd_ex(q, P(1 * MB), P(2 * MB), P(3 * MB), P(4 * MB), (const float*)P(5 * MB), o,
                             (float*)P(6 * MB), B, H, T, dkk, dv, C, 1, flags, w, wsb, nullptr);
  };
  EXPECT(fwd(nullptr, P(7 * MB), P(8 * MB), ws, dk, 0), CKDA_ERR_NULL);
  EXPECT(fwd(P(0), P(7 * MB), P(8 * MB), ws, 48, 0), CKDA_ERR_UNSUPPORTED);
  EXPECT(fwd(P(0), P(2 * MB + 64), P(8 * MB), ws, dk, 0), CKDA_ERR_ALIAS);
  EXPECT(fwd(P(0), P(7 * MB), P(8 * MB), 1024, dk, 0), CKDA_ERR_WORKSPACE);
  EXPECT(fwd(P(0), P(7 * MB), P(8 * MB + 16), ws, dk, 0), CKDA_ERR_WORKSPACE);
  EXPECT(fwd(P(0), P(7 * MB), P(8 * MB), ws, dk, 16), CKDA_ERR_FLAGS);
  EXPECT(fwd(P(8), P(7 * MB), P(8 * MB), ws, dk, 0), CKDA_ERR_DIM);
  EXPECT(ckda_chunk_fwd(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), nullptr, -1, H, T, dk, dv,
                        C, 1, P(8 * MB), ws, nullptr),
         CKDA_ERR_DIM);
  EXPECT(ckda_chunk_fwd(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), nullptr, 0, H, T, dk, dv,
                        C, 1, nullptr, 0, nullptr),
         CKDA_OK);
  EXPECT(ckda_chunk_fwd_gather(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), nullptr, B, H, T, 128,
                               nullptr, dk, dv, C, 1, 0, P(8 * MB), ws, nullptr),
         CKDA_ERR_NULL);
  EXPECT(ckda_deltaproduct2_fwd(P(0), P(MB), P(2 * MB), nullptr, P(4 * MB), nullptr, P(7 * MB), nullptr, B, H, T, dk,
                                dv, C, 1, 8, P(8 * MB), 1 << 30, nullptr),
         CKDA_ERR_FLAGS);
  EXPECT(ckda_chunk_fwd_noalloc(nullptr, P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), nullptr, B, H, T,
                                dk, dv, C, 1, nullptr),
         CKDA_ERR_NULL);
  // one head needing more records than the built-in scratch (buffers 32 MB apart)
  EXPECT(ckda_chunk_fwd_noalloc(P(0), P(32 * MB), P(64 * MB), P(96 * MB), P(128 * MB), nullptr, P(160 * MB), nullptr,
                                1, 1, 65536, 128, 128, 64, 1, nullptr),
         CKDA_ERR_WORKSPACE);

  // decode
  auto dec = [&](void* q, void* S, void* o, int flags) {
    return ckda_decode_step_ex(q, P(MB), P(2 * MB), P(3 * MB), P(4 * MB), (float*)S, o, 4, 2, 64, 64, 1, flags,
                               nullptr);
  };
  EXPECT(dec(nullptr, P(5 * MB), P(6 * MB), 0), CKDA_ERR_NULL);
  EXPECT(dec(P(0), P(5 * MB), P(5 * MB + 64), 0), CKDA_ERR_ALIAS);
  EXPECT(dec(P(0), P(5 * MB), P(6 * MB), 32), CKDA_ERR_FLAGS);
  EXPECT(ckda_deltaproduct2_decode_step(P(0), P(MB), P(2 * MB), nullptr, P(4 * MB), (float*)P(5 * MB), P(5 * MB + 64),
                                        4, 2, 64, 64, 1, 0, nullptr),
         CKDA_ERR_ALIAS);
  EXPECT(ckda_decode_step_gather(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), (float*)P(5 * MB), P(6 * MB), 4, 2,
                                 128, nullptr, 64, 64, 1, 0, nullptr),
         CKDA_ERR_NULL);

  // backward: inputs at 0..7 MB, outputs at 16.. MB, workspace at 64 MB
  const size_t bws = ckda_chunk_bwd_workspace_size(B, H, T, dk, dv, 1);
  auto bwd = [&](void* dq, void* w, size_t wsb, int flags) {
    return ckda_chunk_bwd_ex(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), (const float*)P(5 * MB), P(6 * MB),
                             (const float*)P(7 * MB), (float*)dq, (float*)P(17 * MB), (float*)P(18 * MB),
                             (float*)P(19 * MB), (float*)P(20 * MB), (float*)P(21 * MB), B, H, T, dk, dv, 1, flags, w,
                             wsb, nullptr);
  };
  EXPECT(bwd(nullptr, P(64 * MB), bws, 0), CKDA_ERR_NULL);
  EXPECT(bwd(P(MB + 64), P(64 * MB), bws, 0), CKDA_ERR_ALIAS);
  EXPECT(bwd(P(16 * MB), P(64 * MB), 256, 0), CKDA_ERR_WORKSPACE);
  EXPECT(bwd(P(16 * MB), P(64 * MB), bws, 64), CKDA_ERR_FLAGS);
  EXPECT(ckda_chunk_bwd(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(6 * MB), nullptr, (float*)P(16 * MB),
                        (float*)P(17 * MB), (float*)P(18 * MB), (float*)P(19 * MB), (float*)P(20 * MB), nullptr, B, H,
                        T, 96, dv, 1, P(64 * MB), bws, nullptr),
         CKDA_ERR_UNSUPPORTED);
  EXPECT(ckda_deltaproduct2_bwd(P(0), P(MB), P(2 * MB), nullptr, P(4 * MB), nullptr, P(6 * MB), nullptr,
                                (float*)P(16 * MB), (float*)P(17 * MB), (float*)P(18 * MB), nullptr, (float*)P(20 * MB),
                                nullptr, B, H, T, dk, dv, 1, nullptr, 0, nullptr),
         CKDA_ERR_WORKSPACE);

  if (!gpu) {
    // accepted arguments: the host side of every launch path, which then
    // fails for want of a device
    for (int flags : {0, 1, 2, 4, 7, 8, 15}) {
      EXPECT(fwd(P(0), P(7 * MB), P(8 * MB), ws, dk, flags), LAUNCH);
      EXPECT(dec(P(0), P(5 * MB), P(6 * MB), flags), LAUNCH);
      const size_t bx = ckda_chunk_bwd_ex_workspace_size(B, H, T, dk, dv, 1, flags);
      EXPECT(bwd(P(16 * MB), P(64 * MB), bx, flags), LAUNCH);
    }
    for (int d : {16, 32, 64, 128})
      for (int c : {16, 32, 64})
        EXPECT(ckda_chunk_fwd(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), (float*)P(6 * MB), B,
                              H, T, d, dv, c, 0, P(8 * MB), 64 * MB, nullptr),
               LAUNCH);
    EXPECT(ckda_chunk_fwd_timed(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), nullptr, B, H, T, dk,
                                dv, C, 1, P(8 * MB), ws, nullptr, nullptr, nullptr, nullptr),
           LAUNCH);
    EXPECT(ckda_chunk_fwd_gather(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), nullptr, B, H, T,
                                 128, (const int*)P(6 * MB), dk, dv, C, 1, 0, P(8 * MB), ws, nullptr),
           LAUNCH);
    EXPECT(ckda_deltaproduct2_fwd(P(0), P(MB), P(2 * MB), nullptr, P(4 * MB), nullptr, P(7 * MB), nullptr, B, H, T, dk,
                                  dv, C, 1, 0, P(8 * MB), 1 << 30, nullptr),
           LAUNCH);
    EXPECT(ckda_chunk_fwd_noalloc(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), nullptr, P(7 * MB), nullptr, B, H, T,
                                  dk, dv, C, 1, nullptr),
           LAUNCH);
    EXPECT(ckda_deltaproduct2_decode_step(P(0), P(MB), P(2 * MB), nullptr, P(4 * MB), (float*)P(5 * MB), P(6 * MB), 4,
                                          2, 64, 64, 1, 0, nullptr),
           LAUNCH);
    EXPECT(ckda_decode_step_gather(P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), (float*)P(5 * MB), P(6 * MB), 4, 2,
                                   128, (const int*)P(7 * MB), 64, 64, 1, 0, nullptr),
           LAUNCH);
    const size_t dws = ckda_deltaproduct2_bwd_workspace_size(B, H, T, dk, dv, 1);
    EXPECT(ckda_deltaproduct2_bwd(P(0), P(MB), P(2 * MB), nullptr, P(4 * MB), nullptr, P(6 * MB), nullptr,
                                  (float*)P(16 * MB), (float*)P(17 * MB), (float*)P(18 * MB), nullptr,
                                  (float*)P(20 * MB), nullptr, B, H, T, dk, dv, 1, P(64 * MB), dws, nullptr),
           LAUNCH);
  }
  printf("api driver (%s): %d failures\n", gpu ? "GPU visible: argument checks only" : "no GPU", failures);
  return failures ? 1 : 0;
}
