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
constexpr int kFlagsAll = kFuseAll | CKDA_GATE_SCALAR;
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

// Shared checks and dispatch of the chunked forward entry points.  `flags`
// holds public bits only; prod2 selects DeltaProduct_2 (k, v, beta hold 2 T
// sub-steps, q, o and a scalar alpha T tokens; alpha may be NULL for no
// gate).  `fn` names the entry point in error messages.
static int chunk_fwd_impl(const char* fn, const void* q, const void* k, const void* v, const void* alpha,
                          const void* beta, const float* h0, void* o, float* hT, int B, int H, int T, int dk, int dv,
                          int chunk, int dtype, int flags, void* workspace, size_t workspace_bytes, void* stream,
                          void* const ev[3], const int* gidx = nullptr, int dk_in = 0, bool prod2 = false,
                          bool check_only = false) {
  if ((flags & ~kFlagsAll) != 0)
    return fail(CKDA_ERR_FLAGS, "%s: flags 0x%x has bits outside CKDA_FUSE_* and CKDA_GATE_SCALAR (0x%x)", fn, flags,
                kFlagsAll);
  const bool scalar = (flags & CKDA_GATE_SCALAR) != 0;
  if (gidx && scalar)
    return fail(CKDA_ERR_UNSUPPORTED, "%s: CKDA_GATE_SCALAR does not combine with a channel gather", fn);
  if (!gidx) dk_in = dk;
  if (dk_in < 1 || dk_in > kMaxDkIn)
    return fail(CKDA_ERR_DIM, "%s: dk_in=%d outside 1..%d", fn, dk_in, kMaxDkIn);
  if (B < 0 || H < 0 || T < 0 || (prod2 && T > INT32_MAX / 2))
    return fail(CKDA_ERR_DIM, "%s: negative or too large size (B=%d H=%d T=%d)", fn, B, H, T);
  if (!supported_dtype(dtype))
    return fail(CKDA_ERR_UNSUPPORTED, "%s: dtype %d is not F32(0) or BF16(1)", fn, dtype);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(CKDA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d (supported: 16, 32, 64, 128)", fn, dk, dv);
  if (!supported_chunk(chunk))
    return fail(CKDA_ERR_UNSUPPORTED, "%s: chunk=%d (supported: 16, 32, 64)", fn, chunk);
  const size_t BH = (size_t)B * H;
  const size_t es = dtype_bytes(dtype);
  const int rows = prod2 ? 2 * T : T;   // delta-rule steps per (batch, head)
  const size_t nq = BH * T * dk_in, nk = BH * rows * dk_in, nv = BH * rows * dv, nb = BH * rows;
  const size_t na = scalar ? BH * T : nk, no = BH * T * dv, ns = BH * dk * dv;
  if (BH == 0) return ok();
  if (T > 0 && (!q || !k || !v || !beta || !o || (!alpha && !prod2)))
    return fail(CKDA_ERR_NULL, "%s: q, k, v, %sbeta and o are required", fn, prod2 ? "" : "alpha, ");
  if (T == 0 && !hT) return ok();
  const size_t need = ckda_chunk_fwd_workspace_size(B, H, rows, dk, dv, chunk, dtype);
  const size_t nchunks = BH * (((size_t)rows + chunk - 1) / chunk);
  if (nchunks > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "%s: %zu chunks exceed the launch grid", fn, nchunks);
  if (BH * ((size_t)dv / 16) > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "%s: B*H too large", fn);
  if (((size_t)rows + 64) * dv * es > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "%s: T=%d too long: one head's values and outputs must stay below 2 GiB", fn, T);
  const size_t head_records = (((size_t)rows + chunk - 1) / chunk) * ckda::chunk_record_layout(dk, chunk, dtype).bytes;
  if (head_records > (size_t)INT32_MAX)
    return fail(CKDA_ERR_DIM, "%s: T=%d too long: one head's chunk records must stay below 2 GiB", fn, T);
  if (T > 0 && !check_only) {
    if (!workspace) return fail(CKDA_ERR_WORKSPACE, "%s: workspace is NULL", fn);
    if (workspace_bytes < need)
      return fail(CKDA_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(CKDA_ERR_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  }
  const void* ptrs[] = {q, k, v, alpha, beta, h0, o, hT, gidx};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "h0", "o", "hT", "idx"};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && misaligned(ptrs[i]))
      return fail(CKDA_ERR_DIM, "%s: %s is not 16-byte aligned", fn, names[i]);

  const Range in[] = {range("q", q, T ? nq * es : 0),     range("k", k, T ? nk * es : 0),
                      range("v", v, T ? nv * es : 0),     range("alpha", alpha, T && alpha ? na * es : 0),
                      range("beta", beta, T ? nb * es : 0), range("h0", h0, h0 ? ns * 4 : 0),
                      range("idx", gidx, gidx ? (size_t)H * dk * 4 : 0)};
  const Range ro = range("o", o, T ? no * es : 0);
  const Range rh = range("hT", hT, hT ? ns * 4 : 0);
  const Range rw = range("workspace", workspace, T && !check_only ? need : 0);
  for (const Range& r : in) {
    if (overlap(ro, r)) return fail(CKDA_ERR_ALIAS, "%s: o overlaps %s", fn, r.name);
    if (overlap(rw, r)) return fail(CKDA_ERR_ALIAS, "%s: workspace overlaps %s", fn, r.name);
    const bool same_state = hT && h0 && (const void*)hT == (const void*)h0 && r.lo == (uintptr_t)h0;
    if (!same_state && overlap(rh, r)) return fail(CKDA_ERR_ALIAS, "%s: hT overlaps %s", fn, r.name);
  }
  if (overlap(ro, rh)) return fail(CKDA_ERR_ALIAS, "%s: o overlaps hT", fn);
  if (overlap(rw, ro) || overlap(rw, rh))
    return fail(CKDA_ERR_ALIAS, "%s: workspace overlaps an output", fn);

  if (check_only) return ok();

  ckda::ChunkArgs a{q, k, v, alpha, beta, h0, o, hT, B, H, rows, dk, dv, chunk, dtype,
                    flags | (prod2 ? ckda::kProd2 : 0), workspace,
                    (hipStream_t)stream, {(hipEvent_t)ev[0], (hipEvent_t)ev[1], (hipEvent_t)ev[2]}, gidx, dk_in};
  hipError_t e = ckda::launch_chunk_fwd(a);
  if (e != hipSuccess)
    return fail(CKDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int ckda_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha,
                   const void* beta, const float* h0, void* o, float* hT,
                   int B, int H, int T, int dk, int dv, int chunk, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream) {
  void* const none[3] = {nullptr, nullptr, nullptr};
  return chunk_fwd_impl("ckda_chunk_fwd", q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, 0, workspace,
                        workspace_bytes, stream, none);
}

int ckda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                           const void* beta, const float* h0, void* o, float* hT,
                           int B, int H, int T, int dk, int dv, int chunk, int dtype, void* stream) {
  const char* fn = "ckda_chunk_fwd_noalloc";
  void* const none[3] = {nullptr, nullptr, nullptr};
  // every argument check of ckda_chunk_fwd, on the whole problem
  const int st = chunk_fwd_impl(fn, q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, 0, nullptr, 0,
                                stream, none, nullptr, 0, false, true);
  if (st != CKDA_OK) return st;
  const size_t BH = (size_t)B * H;
  if (BH == 0 || (T == 0 && !hT)) return ok();
  // one head's chunk records must fit the scratch; heads then run in batches
  // that fill it, one Gram + state-pass launch pair per batch, in order on
  // `stream` (records of one batch are consumed before the next overwrites them)
  const size_t per_head = ckda_chunk_fwd_workspace_size(1, 1, T, dk, dv, chunk, dtype);
  if (per_head > ckda::kNoallocScratchBytes)
    return fail(CKDA_ERR_WORKSPACE,
                "%s: T=%d needs %zu bytes of chunk records per head, more than the %zu-byte built-in scratch", fn, T,
                per_head, ckda::kNoallocScratchBytes);
  void* scr = nullptr;
  hipError_t e = ckda::noalloc_scratch(&scr);
  if (e != hipSuccess) return fail(CKDA_ERR_HIP, "%s: scratch lookup failed: %s", fn, hipGetErrorString(e));
  const size_t batch = ckda::kNoallocScratchBytes / per_head;
  const size_t es = dtype_bytes(dtype);
  const unsigned char *qb = (const unsigned char*)q, *kb = (const unsigned char*)k, *vb = (const unsigned char*)v,
                      *ab = (const unsigned char*)alpha, *bb = (const unsigned char*)beta;
  for (size_t f0 = 0; f0 < BH; f0 += batch) {
    const size_t nb = BH - f0 < batch ? BH - f0 : batch;
    const size_t rows = f0 * (size_t)T;   // first token row of the batch
    ckda::ChunkArgs a{T ? qb + rows * dk * es : nullptr, T ? kb + rows * dk * es : nullptr,
                      T ? vb + rows * dv * es : nullptr, T ? ab + rows * dk * es : nullptr,
                      T ? bb + rows * es : nullptr, h0 ? h0 + f0 * dk * dv : nullptr,
                      T ? (unsigned char*)o + rows * dv * es : nullptr, hT ? hT + f0 * dk * dv : nullptr,
                      1, (int)nb, T, dk, dv, chunk, dtype, 0, scr, (hipStream_t)stream, {nullptr, nullptr, nullptr}};
    e = ckda::launch_chunk_fwd(a);
    if (e != hipSuccess) return fail(CKDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

int ckda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* alpha,
                      const void* beta, const float* h0, void* o, float* hT,
                      int B, int H, int T, int dk, int dv, int chunk, int dtype, int flags,
                      void* workspace, size_t workspace_bytes, void* stream) {
  void* const none[3] = {nullptr, nullptr, nullptr};
  return chunk_fwd_impl("ckda_chunk_fwd", q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, flags, workspace,
                        workspace_bytes, stream, none);
}

int ckda_chunk_fwd_gather(const void* q, const void* k, const void* v, const void* alpha,
                          const void* beta, const float* h0, void* o, float* hT,
                          int B, int H, int T, int dk_in, const int* idx, int dk, int dv, int chunk, int dtype,
                          int flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!idx && B > 0 && H > 0) return fail(CKDA_ERR_NULL, "ckda_chunk_fwd: idx is required");
  void* const none[3] = {nullptr, nullptr, nullptr};
  return chunk_fwd_impl("ckda_chunk_fwd", q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, flags, workspace,
                        workspace_bytes, stream, none, idx, dk_in);
}

int ckda_deltaproduct2_fwd(const void* q, const void* k, const void* v, const void* alpha,
                           const void* beta, const float* h0, void* o, float* hT,
                           int B, int H, int T, int dk, int dv, int chunk, int dtype, int flags,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if ((flags & ~kFuseAll) != 0)
    return fail(CKDA_ERR_FLAGS, "ckda_deltaproduct2_fwd: flags 0x%x has bits outside CKDA_FUSE_* (0x%x)", flags,
                kFuseAll);
  void* const none[3] = {nullptr, nullptr, nullptr};
  const int f = flags | (alpha ? CKDA_GATE_SCALAR : 0);
  return chunk_fwd_impl("ckda_deltaproduct2_fwd", q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, f,
                        workspace, workspace_bytes, stream, none, nullptr, 0, true);
}

size_t ckda_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int dtype) {
  if (B < 0 || H < 0 || T < 0) return 0;
  if (!supported_dim(dk) || !supported_dim(dv) || !supported_dtype(dtype)) return 0;
  const size_t bytes = ckda::chunk_bwd_workspace_floats(B, H, T, dk, dv) * 4;
  return bytes == 0 ? 256 : bytes;
}

size_t ckda_chunk_bwd_ex_workspace_size(int B, int H, int T, int dk, int dv, int dtype, int flags) {
  if ((flags & ~kFlagsAll) != 0) return 0;
  if (flags == 0) return ckda_chunk_bwd_workspace_size(B, H, T, dk, dv, dtype);
  if (B < 0 || H < 0 || T < 0) return 0;
  if (!supported_dim(dk) || !supported_dim(dv) || !supported_dtype(dtype)) return 0;
  const size_t bytes = ckda::prologue_bwd_workspace_floats(B, H, T, dk, dv, flags) * 4;
  return bytes == 0 ? 256 : bytes;
}

// Shared checks and dispatch of the backward entry points; flags as
// ckda_chunk_bwd_ex (0 for ckda_chunk_bwd).
static int chunk_bwd_impl(const char* fn, const void* q, const void* k, const void* v, const void* alpha,
                          const void* beta, const float* h0, const void* dout, const float* dhT, float* dq,
                          float* dk_out, float* dv_out, float* dalpha, float* dbeta, float* dh0, int B, int H, int T,
                          int dk, int dv, int dtype, int flags, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if ((flags & ~kFlagsAll) != 0)
    return fail(CKDA_ERR_FLAGS, "%s: flags 0x%x has bits outside CKDA_FUSE_* and CKDA_GATE_SCALAR (0x%x)", fn, flags,
                kFlagsAll);
  if (B < 0 || H < 0 || T < 0) return fail(CKDA_ERR_DIM, "%s: negative size (B=%d H=%d T=%d)", fn, B, H, T);
  if (!supported_dtype(dtype)) return fail(CKDA_ERR_UNSUPPORTED, "%s: dtype %d is not F32(0) or BF16(1)", fn, dtype);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(CKDA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d (supported: 16, 32, 64, 128)", fn, dk, dv);
  const size_t BH = (size_t)B * H;
  if (BH == 0) return ok();
  const bool scalar = (flags & CKDA_GATE_SCALAR) != 0;
  const size_t es = dtype_bytes(dtype);
  const size_t nk = BH * T * dk, nv = BH * T * dv, nb = BH * T, ns = BH * dk * dv;
  const size_t na = scalar ? nb : nk;   // gates (and their gradient)
  if (T > 0 && (!q || !k || !v || !alpha || !beta || !dout || !dq || !dk_out || !dv_out || !dalpha || !dbeta))
    return fail(CKDA_ERR_NULL, "%s: inputs, do and every per-token gradient are required", fn);
  const size_t nch = BH * (((size_t)T + 31) / 32);
  if (nch > (size_t)INT32_MAX || BH * (size_t)(dv / 16) > (size_t)INT32_MAX || (flags && (nb + 3) / 4 > INT32_MAX))
    return fail(CKDA_ERR_DIM, "%s: sizes exceed the launch grid", fn);
  const size_t need = ckda_chunk_bwd_ex_workspace_size(B, H, T, dk, dv, dtype, flags);
  if (!workspace) return fail(CKDA_ERR_WORKSPACE, "%s: workspace is NULL", fn);
  if (workspace_bytes < need)
    return fail(CKDA_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(CKDA_ERR_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  const void* ptrs[] = {q, k, v, alpha, beta, h0, dout, dhT, dq, dk_out, dv_out, dalpha, dbeta, dh0};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "h0", "do", "dhT", "dq", "dk", "dv", "dalpha", "dbeta", "dh0"};
  for (int i = 0; i < 14; ++i)
    if (ptrs[i] && misaligned(ptrs[i])) return fail(CKDA_ERR_DIM, "%s: %s is not 16-byte aligned", fn, names[i]);
  const Range in[] = {range("q", q, T ? nk * es : 0),       range("k", k, T ? nk * es : 0),
                      range("v", v, T ? nv * es : 0),       range("alpha", alpha, T ? na * es : 0),
                      range("beta", beta, T ? nb * es : 0), range("h0", h0, h0 ? ns * 4 : 0),
                      range("do", dout, T ? nv * es : 0),   range("dhT", dhT, dhT ? ns * 4 : 0),
                      range("workspace", workspace, need)};
  const Range out[] = {range("dq", dq, T ? nk * 4 : 0),         range("dk", dk_out, T ? nk * 4 : 0),
                       range("dv", dv_out, T ? nv * 4 : 0),     range("dalpha", dalpha, T ? na * 4 : 0),
                       range("dbeta", dbeta, T ? nb * 4 : 0),   range("dh0", dh0, dh0 ? ns * 4 : 0)};
  for (const Range& o : out) {
    for (const Range& r : in)
      if (overlap(o, r)) return fail(CKDA_ERR_ALIAS, "%s: %s overlaps %s", fn, o.name, r.name);
    for (const Range& o2 : out)
      if (&o2 != &o && overlap(o, o2)) return fail(CKDA_ERR_ALIAS, "%s: %s overlaps %s", fn, o.name, o2.name);
  }
  ckda::BwdArgs a{q, k, v, alpha, beta, h0, dout, dhT, dq, dk_out, dv_out, dalpha, dbeta, dh0,
                  B, H, T, dk, dv, dtype, workspace, (hipStream_t)stream};
  hipError_t e = flags ? ckda::launch_prologue_bwd(a, flags) : ckda::launch_chunk_bwd(a);
  if (e != hipSuccess) return fail(CKDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int ckda_chunk_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                   const float* h0, const void* dout, const float* dhT, float* dq, float* dk_out, float* dv_out,
                   float* dalpha, float* dbeta, float* dh0, int B, int H, int T, int dk, int dv, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("ckda_chunk_bwd", q, k, v, alpha, beta, h0, dout, dhT, dq, dk_out, dv_out, dalpha, dbeta, dh0,
                        B, H, T, dk, dv, dtype, 0, workspace, workspace_bytes, stream);
}

int ckda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                      const float* h0, const void* dout, const float* dhT, float* dq, float* dk_out, float* dv_out,
                      float* dalpha, float* dbeta, float* dh0, int B, int H, int T, int dk, int dv, int dtype,
                      int flags, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("ckda_chunk_bwd_ex", q, k, v, alpha, beta, h0, dout, dhT, dq, dk_out, dv_out, dalpha, dbeta,
                        dh0, B, H, T, dk, dv, dtype, flags, workspace, workspace_bytes, stream);
}

size_t ckda_deltaproduct2_bwd_workspace_size(int B, int H, int T, int dk, int dv, int dtype) {
  if (B < 0 || H < 0 || T < 0 || T > INT32_MAX / 2) return 0;
  if (!supported_dim(dk) || !supported_dim(dv) || !supported_dtype(dtype)) return 0;
  const size_t bytes = ckda::dp2_bwd_workspace_bytes(B, H, T, dk, dv, dtype);
  return bytes == 0 ? 256 : bytes;
}

int ckda_deltaproduct2_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                           const float* h0, const void* dout, const float* dhT, float* dq, float* dk_out,
                           float* dv_out, float* dalpha, float* dbeta, float* dh0, int B, int H, int T, int dk,
                           int dv, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "ckda_deltaproduct2_bwd";
  if (B < 0 || H < 0 || T < 0 || T > INT32_MAX / 2)
    return fail(CKDA_ERR_DIM, "%s: negative or too large size (B=%d H=%d T=%d)", fn, B, H, T);
  if (!supported_dtype(dtype)) return fail(CKDA_ERR_UNSUPPORTED, "%s: dtype %d is not F32(0) or BF16(1)", fn, dtype);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(CKDA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d (supported: 16, 32, 64, 128)", fn, dk, dv);
  const size_t BH = (size_t)B * H;
  if (BH == 0) return ok();
  const size_t es = dtype_bytes(dtype);
  const size_t nq = BH * T * dk, nk = 2 * nq, nv = 2 * BH * T * dv, no = BH * T * dv, nt = BH * T, ns = BH * dk * dv;
  if (T > 0 && (!q || !k || !v || !beta || !dout || !dq || !dk_out || !dv_out || !dbeta || (alpha && !dalpha)))
    return fail(CKDA_ERR_NULL, "%s: inputs, do and every per-token gradient (dalpha with alpha) are required", fn);
  const size_t nch = BH * ((2 * (size_t)T + 31) / 32);
  if (nch > (size_t)INT32_MAX || BH * (size_t)(dv / 16) > (size_t)INT32_MAX || (2 * nt + 3) / 4 > INT32_MAX)
    return fail(CKDA_ERR_DIM, "%s: sizes exceed the launch grid", fn);
  const size_t need = ckda_deltaproduct2_bwd_workspace_size(B, H, T, dk, dv, dtype);
  if (!workspace) return fail(CKDA_ERR_WORKSPACE, "%s: workspace is NULL", fn);
  if (workspace_bytes < need)
    return fail(CKDA_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(CKDA_ERR_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  const void* ptrs[] = {q, k, v, alpha, beta, h0, dout, dhT, dq, dk_out, dv_out, dalpha, dbeta, dh0};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "h0", "do", "dhT", "dq", "dk", "dv", "dalpha", "dbeta", "dh0"};
  for (int i = 0; i < 14; ++i)
    if (ptrs[i] && misaligned(ptrs[i])) return fail(CKDA_ERR_DIM, "%s: %s is not 16-byte aligned", fn, names[i]);
  const bool gated = alpha != nullptr;
  const Range in[] = {range("q", q, T ? nq * es : 0),       range("k", k, T ? nk * es : 0),
                      range("v", v, T ? nv * es : 0),       range("alpha", alpha, T && gated ? nt * es : 0),
                      range("beta", beta, T ? 2 * nt * es : 0), range("h0", h0, h0 ? ns * 4 : 0),
                      range("do", dout, T ? no * es : 0),   range("dhT", dhT, dhT ? ns * 4 : 0),
                      range("workspace", workspace, need)};
  const Range out[] = {range("dq", dq, T ? nq * 4 : 0),         range("dk", dk_out, T ? nk * 4 : 0),
                       range("dv", dv_out, T ? nv * 4 : 0),     range("dalpha", dalpha, T && gated ? nt * 4 : 0),
                       range("dbeta", dbeta, T ? 2 * nt * 4 : 0), range("dh0", dh0, dh0 ? ns * 4 : 0)};
  for (const Range& o : out) {
    for (const Range& r : in)
      if (overlap(o, r)) return fail(CKDA_ERR_ALIAS, "%s: %s overlaps %s", fn, o.name, r.name);
    for (const Range& o2 : out)
      if (&o2 != &o && overlap(o, o2)) return fail(CKDA_ERR_ALIAS, "%s: %s overlaps %s", fn, o.name, o2.name);
  }
  ckda::BwdArgs a{q, k, v, alpha, beta, h0, dout, dhT, dq, dk_out, dv_out, gated ? dalpha : nullptr, dbeta, dh0,
                  B, H, T, dk, dv, dtype, workspace, (hipStream_t)stream};
  hipError_t e = ckda::launch_dp2_bwd(a);
  if (e != hipSuccess) return fail(CKDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int ckda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* alpha,
                         const void* beta, const float* h0, void* o, float* hT,
                         int B, int H, int T, int dk, int dv, int chunk, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream,
                         void* ev_start, void* ev_mid, void* ev_end) {
  void* const ev[3] = {ev_start, ev_mid, ev_end};
  return chunk_fwd_impl("ckda_chunk_fwd", q, k, v, alpha, beta, h0, o, hT, B, H, T, dk, dv, chunk, dtype, 0, workspace,
                        workspace_bytes, stream, ev);
}

static int decode_impl(const char* fn, const void* q, const void* k, const void* v, const void* alpha,
                       const void* beta, float* H_inout, void* o, int N, int H, int dk, int dv, int dtype, int flags,
                       void* stream, const int* gidx = nullptr, int dk_in = 0, bool prod2 = false) {
  if ((flags & ~kFlagsAll) != 0)
    return fail(CKDA_ERR_FLAGS, "%s: flags 0x%x has bits outside CKDA_FUSE_* and CKDA_GATE_SCALAR (0x%x)", fn, flags,
                kFlagsAll);
  const bool scalar = (flags & CKDA_GATE_SCALAR) != 0;
  if (gidx && scalar)
    return fail(CKDA_ERR_UNSUPPORTED, "%s: CKDA_GATE_SCALAR does not combine with a channel gather", fn);
  if (!gidx) dk_in = dk;
  if (dk_in < 1 || dk_in > kMaxDkIn)
    return fail(CKDA_ERR_DIM, "%s: dk_in=%d outside 1..%d", fn, dk_in, kMaxDkIn);
  if (N < 0 || H < 0) return fail(CKDA_ERR_DIM, "%s: negative size (N=%d H=%d)", fn, N, H);
  if (!supported_dtype(dtype))
    return fail(CKDA_ERR_UNSUPPORTED, "%s: dtype %d is not F32(0) or BF16(1)", fn, dtype);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(CKDA_ERR_UNSUPPORTED, "%s: dk=%d dv=%d (supported: 16, 32, 64, 128)", fn, dk, dv);
  const size_t NH = (size_t)N * H;
  if (NH == 0) return ok();
  if (NH > (size_t)INT32_MAX) return fail(CKDA_ERR_DIM, "%s: N*H exceeds the launch grid", fn);
  if (!q || !k || !v || (!alpha && !prod2) || !beta || !H_inout || !o)
    return fail(CKDA_ERR_NULL, "%s: every pointer%s is required", fn, prod2 ? " but alpha" : "");
  const void* ptrs[] = {q, k, v, alpha, beta, H_inout, o, gidx};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "H_inout", "o", "idx"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && misaligned(ptrs[i]))
      return fail(CKDA_ERR_DIM, "%s: %s is not 16-byte aligned", fn, names[i]);
  const size_t es = dtype_bytes(dtype);
  const size_t sub = prod2 ? 2 : 1;   // delta sub-steps per token
  const Range in[] = {range("q", q, NH * dk_in * es), range("k", k, sub * NH * dk_in * es),
                      range("v", v, sub * NH * dv * es),
                      range("alpha", alpha, alpha ? (scalar ? NH : NH * dk_in) * es : 0), range("beta", beta, sub * NH * es),
                      range("idx", gidx, gidx ? (size_t)H * dk * 4 : 0)};
  const Range rs = range("H_inout", H_inout, NH * dk * dv * 4);
  const Range ro = range("o", o, NH * dv * es);
  for (const Range& r : in) {
    if (overlap(ro, r)) return fail(CKDA_ERR_ALIAS, "%s: o overlaps %s", fn, r.name);
    if (overlap(rs, r)) return fail(CKDA_ERR_ALIAS, "%s: H_inout overlaps %s", fn, r.name);
  }
  if (overlap(ro, rs)) return fail(CKDA_ERR_ALIAS, "%s: o overlaps H_inout", fn);

  ckda::DecodeArgs a{q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, flags | (prod2 ? ckda::kProd2 : 0),
                     (hipStream_t)stream, gidx, dk_in};
  hipError_t e = ckda::launch_decode(a);
  if (e != hipSuccess)
    return fail(CKDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int ckda_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                     const void* beta, float* H_inout, void* o,
                     int N, int H, int dk, int dv, int dtype, void* stream) {
  return decode_impl("ckda_decode_step", q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, 0, stream);
}

int ckda_deltaproduct2_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                                   const void* beta, float* H_inout, void* o,
                                   int N, int H, int dk, int dv, int dtype, int flags, void* stream) {
  if ((flags & ~kFuseAll) != 0)
    return fail(CKDA_ERR_FLAGS, "ckda_deltaproduct2_decode_step: flags 0x%x has bits outside CKDA_FUSE_* (0x%x)",
                flags, kFuseAll);
  const int f = flags | (alpha ? CKDA_GATE_SCALAR : 0);
  return decode_impl("ckda_deltaproduct2_decode_step", q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, f,
                     stream, nullptr, 0, true);
}

int ckda_decode_step_gather(const void* q, const void* k, const void* v, const void* alpha,
                            const void* beta, float* H_inout, void* o,
                            int N, int H, int dk_in, const int* idx, int dk, int dv, int dtype, int flags,
                            void* stream) {
  if (!idx && N > 0 && H > 0) return fail(CKDA_ERR_NULL, "ckda_decode_step: idx is required");
  return decode_impl("ckda_decode_step", q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, flags, stream, idx, dk_in);
}

int ckda_decode_step_ex(const void* q, const void* k, const void* v, const void* alpha,
                        const void* beta, float* H_inout, void* o,
                        int N, int H, int dk, int dv, int dtype, int flags, void* stream) {
  return decode_impl("ckda_decode_step", q, k, v, alpha, beta, H_inout, o, N, H, dk, dv, dtype, flags, stream);
}

}  // extern "C"
