// ckda_api.cpp -- the C ABI declared in include/ckda.h: argument checking,
// aliasing and workspace checks, kernel dispatch and error reporting.
// Nothing here touches device memory; every check runs before a launch, so
// the whole argument contract can be exercised on a machine without a GPU.
#include "ckda.h"

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "ckda_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return CKDA_OK;
}

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }
bool supported_dtype(int t) { return t == CKDA_DTYPE_F32 || t == CKDA_DTYPE_BF16; }
size_t dtype_bytes(int t) { return t == CKDA_DTYPE_BF16 ? 2 : 4; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, size_t bytes) {
  uintptr_t a = (uintptr_t)p;
  return Range{name, a, a + bytes};
}

bool overlap(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

constexpr int kFuseAll = CKDA_FUSE_GATES | CKDA_FUSE_NORM_K | CKDA_FUSE_NORM_Q;
constexpr int kMaxDkIn = 65536;   // row width of gathered inputs

}  // namespace

extern "C" {

const char* ckda_status_string(int status) {
  switch (status) {
    case CKDA_OK: return "ok";
    case CKDA_ERR_NULL: return "a required pointer is NULL";
    case CKDA_ERR_DIM: return "invalid or inconsistent sizes";
    case CKDA_ERR_UNSUPPORTED: return "unsupported dtype, head dimension or chunk size";
    case CKDA_ERR_ALIAS: return "an output overlaps an input";
    case CKDA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case CKDA_ERR_HIP: return "HIP runtime error";
    case CKDA_ERR_FLAGS: return "unknown prologue flag bits";
  }
  return "unknown status";
}

const char* ckda_last_error(void) { return g_last_error.c_str(); }

int ckda_abi_version(void) { return CKDA_ABI_VERSION; }

size_t ckda_chunk_fwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  if (B < 0 || H < 0 || T < 0) return 0;
  if (!supported_dim(dk) || !supported_dim(dv) || !supported_chunk(chunk) || !supported_dtype(dtype))
    return 0;
  const size_t nchunks = (size_t)B * H * (((size_t)T + chunk - 1) / chunk);
  const ckda::ChunkRecord rec = ckda::chunk_record_layout(dk, chunk, dtype);
  const size_t bytes = nchunks * rec.bytes;
  return bytes == 0 ? 256 : bytes;  // never 0 for valid sizes: 0 means "invalid"
}

static int chunk_fwd_impl(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                          const float* h0, void* o, float* hT, int B, int H, int T, int dk, int dv, int chunk,
                          int dtype, int flags, void* workspace, size_t workspace_bytes, void* stream,
                          void* const ev[3], const int* gidx = nullptr, int dk_in = 0) {
  if ((flags & ~kFuseAll) != 0)
    return fail(CKDA_ERR_FLAGS, "ckda_chunk_fwd: flags 0x%x has bits outside CKDA_FUSE_* (0x%x)", flags, kFuseAll);
  if (!gidx) dk_in = dk;
  if (dk_in < 1 || dk_in > kMaxDkIn)
    return fail(CKDA_ERR_DIM, "ckda_chunk_fwd: dk_in=%d outside 1..%d", dk_in, kMaxDkIn);
  if (B < 0 || H < 0 || T < 0)
    return fail(CKDA_ERR_DIM, "ckda_chunk_fwd: negative size (B=%d H=%d T=%d)", B, H, T);
  if (!supported_dtype(dtype))
    return fail(CKDA_ERR_UNSUPPORTED, "ckda_chunk_fwd: dtype %d is not F32(0) or BF16(1)", dtype);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(CKDA_ERR_UNSUPPORTED, "ckda_chunk_fwd: dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  if (!supported_chunk(chunk))
    return fail(CKDA_ERR_UNSUPPORTED, "ckda_chunk_fwd: chunk=%d (supported: 16, 32, 64)", chunk);
  const size_t BH = (size_t)B * H;
  const size_t es = dtype_bytes(dtype);
  const size_t nk = BH * T * dk_in, nv = BH * T * dv, nb = BH * T, ns = BH * dk * dv;
  if (BH == 0) return ok();
  if (T > 0 && (!q || !k || !v || !alpha || !beta || !o))
    return fail(CKDA_ERR_NULL, "ckda_chunk_fwd: q, k, v, alpha, beta and o are required");
  if (T == 0 && !hT) return ok();
  const size_t need = ckda_chunk_fwd_workspace_size(B, H, T, dk, dv, chunk, dtype);
  const size_t nchunks = BH * (((size_t)T + chunk - 1) / chunk);
  if (nchunks > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "ckda_chunk_fwd: %zu chunks exceed the launch grid", nchunks);
  if (BH * ((size_t)dv / 16) > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "ckda_chunk_fwd: B*H too large");
  if (((size_t)T + 64) * dv * es > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "ckda_chunk_fwd: T=%d too long: one head's output must stay below 2 GiB", T);
  const size_t head_records = (((size_t)T + chunk - 1) / chunk) * ckda::chunk_record_layout(dk, chunk, dtype).bytes;
  if (head_records > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "ckda_chunk_fwd: T=%d too long: one head's chunk records must stay below 2 GiB", T);
  if (T > 0) {
    if (!workspace) return fail(CKDA_ERR_WORKSPACE, "ckda_chunk_fwd: workspace is NULL");
    if (workspace_bytes < need)
      return fail(CKDA_ERR_WORKSPACE, "ckda_chunk_fwd: workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(CKDA_ERR_WORKSPACE, "ckda_chunk_fwd: workspace not 256-byte aligned");
  }
  const void* ptrs[] = {q, k, v, alpha, beta, h0, o, hT, gidx};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "h0", "o", "hT", "idx"};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && misaligned(ptrs[i]))
      return fail(CKDA_ERR_DIM, "ckda_chunk_fwd: %s is not 16-byte aligned", names[i]);

  const Range in[] = {range("q", q, T ? nk * es : 0),     range("k", k, T ? nk * es : 0),
                      range("v", v, T ? nv * es : 0),     range("alpha", alpha, T ? nk * es : 0),
                      range("beta", beta, T ? nb * es : 0), range("h0", h0, h0 ? ns * 4 : 0),
                      range("idx", gidx, gidx ? (size_t)H * dk * 4 : 0)};
  const Range ro = range("o", o, T ? nv * es : 0);
  const Range rh = range("hT", hT, hT ? ns * 4 : 0);
  const Range rw = range("workspace", workspace, T ? need : 0);
  for (const Range& r : in) {
    if (overlap(ro, r)) return fail(CKDA_ERR_ALIAS, "ckda_chunk_fwd: o overlaps %s", r.name);
    if (overlap(rw, r)) return fail(CKDA_ERR_ALIAS, "ckda_chunk_fwd: workspace overlaps %s", r.name);
    const bool same_state = hT && h0 && (const void*)hT == (const void*)h0 && r.lo == (uintptr_t)h0;
    if (!same_state && overlap(rh, r)) return fail(CKDA_ERR_ALIAS, "ckda_chunk_fwd: hT overlaps %s", r.name);
  }
  if (overlap(ro, rh)) return fail(CKDA_ERR_ALIAS, "ckda_chunk_fwd: o overlaps hT");
  if (overlap(rw, ro) || overlap(rw, rh))
    return fail(CKDA_ERR_ALIAS, "ckda_chunk_fwd: workspace overlaps an output");

  ckda::ChunkArgs a{q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, flags, workspace,
                    (hipStream_t)stream, {(hipEvent_t)ev[0], (hipEvent_t)ev[1], (hipEvent_t)ev[2]}, gidx, dk_in};
  hipError_t e = ckda::launch_chunk_fwd(a);
  if (e != hipSuccess)
    return fail(CKDA_ERR_HIP, "ckda_chunk_fwd: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ckda_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha,
                   const void* beta, const float* h0, void* o, float* hT,
                   int B, int H, int T, int dk, int dv, int chunk, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream) {
  void* const none[3] = {nullptr, nullptr, nullptr};
  return chunk_fwd_impl(q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, 0, workspace,
                        workspace_bytes, stream, none);
}

int ckda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* alpha,
                      const void* beta, const float* h0, void* o, float* hT,
                      int B, int H, int T, int dk, int dv, int chunk, int dtype, int flags,
                      void* workspace, size_t workspace_bytes, void* stream) {
  void* const none[3] = {nullptr, nullptr, nullptr};
  return chunk_fwd_impl(q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, flags, workspace,
                        workspace_bytes, stream, none);
}

int ckda_chunk_fwd_gather(const void* q, const void* k, const void* v, const void* alpha,
                          const void* beta, const float* h0, void* o, float* hT,
                          int B, int H, int T, int dk_in, const int* idx, int dk, int dv, int chunk, int dtype,
                          int flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!idx && B > 0 && H > 0) return fail(CKDA_ERR_NULL, "ckda_chunk_fwd: idx is required");
  void* const none[3] = {nullptr, nullptr, nullptr};
  return chunk_fwd_impl(q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, flags, workspace,
                        workspace_bytes, stream, none, idx, dk_in);
}

int ckda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* alpha,
                         const void* beta, const float* h0, void* o, float* hT,
                         int B, int H, int T, int dk, int dv, int chunk, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream,
                         void* ev_start, void* ev_mid, void* ev_end) {
  void* const ev[3] = {ev_start, ev_mid, ev_end};
  return chunk_fwd_impl(q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, 0, workspace,
                        workspace_bytes, stream, ev);
}

static int decode_impl(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                       float* H_inout, void* o, int N, int H, int dk, int dv, int dtype, int flags, void* stream,
                       const int* gidx = nullptr, int dk_in = 0) {
  if ((flags & ~kFuseAll) != 0)
    return fail(CKDA_ERR_FLAGS, "ckda_decode_step: flags 0x%x has bits outside CKDA_FUSE_* (0x%x)", flags, kFuseAll);
  if (!gidx) dk_in = dk;
  if (dk_in < 1 || dk_in > kMaxDkIn)
    return fail(CKDA_ERR_DIM, "ckda_decode_step: dk_in=%d outside 1..%d", dk_in, kMaxDkIn);
  if (N < 0 || H < 0) return fail(CKDA_ERR_DIM, "ckda_decode_step: negative size (N=%d H=%d)", N, H);
  if (!supported_dtype(dtype))
    return fail(CKDA_ERR_UNSUPPORTED, "ckda_decode_step: dtype %d is not F32(0) or BF16(1)", dtype);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(CKDA_ERR_UNSUPPORTED, "ckda_decode_step: dk=%d dv=%d (supported: 16, 32, 64, 128)", dk, dv);
  const size_t NH = (size_t)N * H;
  if (NH == 0) return ok();
  if (NH > (size_t)INT32_MAX) return fail(CKDA_ERR_DIM, "ckda_decode_step: N*H exceeds the launch grid");
  if (!q || !k || !v || !alpha || !beta || !H_inout || !o)
    return fail(CKDA_ERR_NULL, "ckda_decode_step: every pointer is required");
  const void* ptrs[] = {q, k, v, alpha, beta, H_inout, o, gidx};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "H_inout", "o", "idx"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && misaligned(ptrs[i]))
      return fail(CKDA_ERR_DIM, "ckda_decode_step: %s is not 16-byte aligned", names[i]);
  const size_t es = dtype_bytes(dtype);
  const Range in[] = {range("q", q, NH * dk_in * es), range("k", k, NH * dk_in * es), range("v", v, NH * dv * es),
                      range("alpha", alpha, NH * dk_in * es), range("beta", beta, NH * es),
                      range("idx", gidx, gidx ? (size_t)H * dk * 4 : 0)};
  const Range rs = range("H_inout", H_inout, NH * dk * dv * 4);
  const Range ro = range("o", o, NH * dv * es);
  for (const Range& r : in) {
    if (overlap(ro, r)) return fail(CKDA_ERR_ALIAS, "ckda_decode_step: o overlaps %s", r.name);
    if (overlap(rs, r)) return fail(CKDA_ERR_ALIAS, "ckda_decode_step: H_inout overlaps %s", r.name);
  }
  if (overlap(ro, rs)) return fail(CKDA_ERR_ALIAS, "ckda_decode_step: o overlaps H_inout");

  ckda::DecodeArgs a{q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, flags, (hipStream_t)stream, gidx, dk_in};
  hipError_t e = ckda::launch_decode(a);
  if (e != hipSuccess)
    return fail(CKDA_ERR_HIP, "ckda_decode_step: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ckda_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                     const void* beta, float* H_inout, void* o,
                     int N, int H, int dk, int dv, int dtype, void* stream) {
  return decode_impl(q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, 0, stream);
}

int ckda_decode_step_gather(const void* q, const void* k, const void* v, const void* alpha,
                            const void* beta, float* H_inout, void* o,
                            int N, int H, int dk_in, const int* idx, int dk, int dv, int dtype, int flags,
                            void* stream) {
  if (!idx && N > 0 && H > 0) return fail(CKDA_ERR_NULL, "ckda_decode_step: idx is required");
  return decode_impl(q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, flags, stream, idx, dk_in);
}

int ckda_decode_step_ex(const void* q, const void* k, const void* v, const void* alpha,
                        const void* beta, float* H_inout, void* o,
                        int N, int H, int dk, int dv, int dtype, int flags, void* stream) {
  return decode_impl(q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, flags, stream);
}

}  // extern "C"
