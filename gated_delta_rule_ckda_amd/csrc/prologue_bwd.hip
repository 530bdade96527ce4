// prologue_bwd.hip -- the backward through the per-token prologue
// (ckda_chunk_bwd_ex): gradients with respect to the gate and beta logits and
// the raw keys and queries.
//
// The prologue is the practical parameterisation of the "Complex KDA"
// discussion slides (frame "Backup: practical gates differ from exact
// theoretical endpoints"): alpha = s [eps + (1 - eps) |r|], r = tanh(a / 2),
// s the sign of r (+1 at 0), beta = 2 sigma(b), and unit-norm keys (and
// queries) y = x (sum x^2 + 1e-6)^-1/2.  The same frame fixes the backward
// convention: s is held constant and |r| takes the zero subgradient at r = 0.
//
// The path runs in three steps on the caller's stream:
//   1. prologue_fwd_kernel writes the prologue's outputs (and v, do) in fp32;
//   2. the fp32 backward of the recurrence (chunk_bwd.hip) on them, writing
//      the gradients with respect to alpha, beta, k^, q^ (and v, h0);
//   3. prologue_bwd_kernel maps those back through the prologue, in place:
//        da = dalpha (1 - eps)(1 - r^2) / 2  (a != 0; 0 at a = 0),
//        db = dbeta 2 sigma(b)(1 - sigma(b)),
//        dx = n (dy - y (y . dy)),  y = x n   (normalised rows),
//      and with one gate per token the per-channel gate gradients summed.
// One wave per token row: lane l holds channels 4 l .. 4 l + 3 (d <= 128,
// 16-byte fp32 and 8-byte bf16 accesses).
#include "ckda_device.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int kRowsPerBlock = 4;   // one wave per row, four waves per workgroup

// this lane's four channels of row `row` (rows of d elements), widened; zero
// past the row's end
template <typename T>
__device__ __forceinline__ f32x4 row_quad(const T* x, long long row, int d, int lane) {
  if (4 * lane >= d) return zero4();
  if constexpr (sizeof(T) == 2) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(x + row * d + 4 * lane);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xFFFF0000u)};
  } else {
    return *reinterpret_cast<const f32x4*>(x + row * d + 4 * lane);
  }
}

__device__ __forceinline__ void put_quad(float* y, long long row, int d, int lane, f32x4 v) {
  if (4 * lane < d) *reinterpret_cast<f32x4*>(y + row * d + 4 * lane) = v;
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
  return __builtin_fmaf(a[0], b[0], __builtin_fmaf(a[1], b[1], __builtin_fmaf(a[2], b[2], a[3] * b[3])));
}

template <typename T>
__global__ __launch_bounds__(64 * kRowsPerBlock) void prologue_fwd_kernel(
    const T* q, const T* k, const T* v, const T* alpha, const T* beta, const T* dout, float* qf, float* kf, float* vf,
    float* af, float* bf, float* of, long long ntok, int dk, int dv, int flags) {
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / 64;
  if (row >= ntok) return;   // the whole wave
  const int lane = threadIdx.x & 63;
  auto unit = [&](const T* x, float* y, bool on) __attribute__((always_inline)) {
    f32x4 e = row_quad(x, row, dk, lane);
    if (on) e *= __builtin_amdgcn_rsqf(wave_sum(dot4(e, e)) + kUnitGuard);
    put_quad(y, row, dk, lane, e);
  };
  unit(k, kf, flags & kFuseNormK);
  unit(q, qf, flags & kFuseNormQ);
  const bool gates = flags & kFuseGates;
  if (flags & kScalarGate) {
    const float a = to_f32(alpha[row]);
    const float g = gates ? practical_gate(a) : a;
    put_quad(af, row, dk, lane, f32x4{g, g, g, g});
  } else {
    f32x4 a = row_quad(alpha, row, dk, lane);
    if (gates) {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = practical_gate(a[e]);
    }
    put_quad(af, row, dk, lane, a);
  }
  if (lane == 0) {
    const float b = to_f32(beta[row]);
    bf[row] = gates ? practical_beta(b) : b;
  }
  put_quad(vf, row, dv, lane, row_quad(v, row, dv, lane));
  put_quad(of, row, dv, lane, row_quad(dout, row, dv, lane));
}

// dq, dk hold the gradients with respect to q^, k^ on entry and those with
// respect to the raw q, k on return; dalpha, dbeta likewise (with one gate
// per token, galpha_ch holds the per-channel gate gradients and dalpha gets
// their sum through the slope).
template <typename T>
__global__ __launch_bounds__(64 * kRowsPerBlock) void prologue_bwd_kernel(
    const T* q, const T* k, const T* alpha, const T* beta, float* dq, float* dk, float* dalpha, float* dbeta,
    const float* galpha_ch, long long ntok, int d, int flags) {
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / 64;
  if (row >= ntok) return;   // the whole wave
  const int lane = threadIdx.x & 63;
  auto unit_bwd = [&](const T* x, float* g) __attribute__((always_inline)) {
    const f32x4 e = row_quad(x, row, d, lane);
    const f32x4 dy = row_quad(g, row, d, lane);
    const float n = __builtin_amdgcn_rsqf(wave_sum(dot4(e, e)) + kUnitGuard);
    const f32x4 y = e * n;
    const float ydy = wave_sum(dot4(y, dy));
    put_quad(g, row, d, lane, (dy - y * ydy) * n);
  };
  if (flags & kFuseNormK) unit_bwd(k, dk);
  if (flags & kFuseNormQ) unit_bwd(q, dq);
  const bool gates = flags & kFuseGates;
  if (flags & kScalarGate) {
    const f32x4 gch = row_quad(galpha_ch, row, d, lane);
    const float sum = wave_sum((gch[0] + gch[1]) + (gch[2] + gch[3]));
    if (lane == 0) dalpha[row] = gates ? sum * practical_gate_slope(to_f32(alpha[row])) : sum;
  } else if (gates) {
    const f32x4 a = row_quad(alpha, row, d, lane);
    f32x4 ga = row_quad(dalpha, row, d, lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) ga[e] *= practical_gate_slope(a[e]);
    put_quad(dalpha, row, d, lane, ga);
  }
  if (gates && lane == 0) dbeta[row] *= practical_beta_slope(to_f32(beta[row]));
}

// fp32 elements of each workspace part, rounded up to 256 bytes
static size_t part(size_t n) { return (n + 63) / 64 * 64; }

size_t prologue_bwd_workspace_floats(int B, int H, int T, int dk, int dv, int flags) {
  const size_t ntok = (size_t)B * H * T;
  size_t n = 3 * part(ntok * dk) + 2 * part(ntok * dv) + part(ntok);
  if (flags & kScalarGate) n += part(ntok * dk);
  return n + chunk_bwd_workspace_floats(B, H, T, dk, dv);
}

template <typename T>
static hipError_t launch_t(const BwdArgs& a, int flags) {
  const long long ntok = (long long)a.B * a.H * a.T;
  float* w = (float*)a.workspace;
  auto take = [&](size_t n) {
    float* p = w;
    w += part(n);
    return p;
  };
  float* qf = take((size_t)ntok * a.dk);
  float* kf = take((size_t)ntok * a.dk);
  float* af = take((size_t)ntok * a.dk);
  float* vf = take((size_t)ntok * a.dv);
  float* of = take((size_t)ntok * a.dv);
  float* bf = take((size_t)ntok);
  float* gach = (flags & kScalarGate) ? take((size_t)ntok * a.dk) : nullptr;
  const unsigned blocks = (unsigned)((ntok + kRowsPerBlock - 1) / kRowsPerBlock);
  if (ntok > 0) {
    hipLaunchKernelGGL((prologue_fwd_kernel<T>), dim3(blocks), dim3(64 * kRowsPerBlock), 0, a.stream, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, (const T*)a.alpha, (const T*)a.beta, (const T*)a.dout, qf, kf,
                       vf, af, bf, of, ntok, a.dk, a.dv, flags);
  }
  BwdArgs f = a;
  f.q = qf;
  f.k = kf;
  f.v = vf;
  f.alpha = af;
  f.beta = bf;
  f.dout = of;
  f.galpha = gach ? gach : a.galpha;
  f.dtype = 0;
  f.workspace = w;
  hipError_t e = launch_chunk_bwd(f);
  if (e != hipSuccess || ntok == 0) return e;
  hipLaunchKernelGGL((prologue_bwd_kernel<T>), dim3(blocks), dim3(64 * kRowsPerBlock), 0, a.stream, (const T*)a.q,
                     (const T*)a.k, (const T*)a.alpha, (const T*)a.beta, a.gq, a.gk, a.galpha, a.gbeta, gach, ntok,
                     a.dk, flags);
  return hipGetLastError();
}

hipError_t launch_prologue_bwd(const BwdArgs& a, int flags) {
  if ((long long)a.B * a.H == 0) return hipSuccess;
  return a.dtype == 1 ? launch_t<bf16_t>(a, flags) : launch_t<float>(a, flags);
}

}  // namespace ckda
