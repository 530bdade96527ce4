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
// One wave per token row: lane l holds channels l and l + 64 (d <= 128).
#include "ckda_device.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int kRowsPerBlock = 4;   // one wave per row, four waves per workgroup

template <typename T>
__device__ __forceinline__ void row_pair(const T* x, long long row, int d, int lane, float& e0, float& e1) {
  e0 = lane < d ? to_f32(x[row * d + lane]) : 0.f;
  e1 = lane + 64 < d ? to_f32(x[row * d + lane + 64]) : 0.f;
}

__device__ __forceinline__ void put_pair(float* y, long long row, int d, int lane, float e0, float e1) {
  if (lane < d) y[row * d + lane] = e0;
  if (lane + 64 < d) y[row * d + lane + 64] = e1;
}

template <typename T>
__global__ __launch_bounds__(64 * kRowsPerBlock) void prologue_fwd_kernel(
    const T* q, const T* k, const T* v, const T* alpha, const T* beta, const T* dout, float* qf, float* kf, float* vf,
    float* af, float* bf, float* of, long long ntok, int dk, int dv, int flags) {
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / 64;
  if (row >= ntok) return;   // the whole wave
  const int lane = threadIdx.x & 63;
  auto unit = [&](const T* x, float* y, bool on) __attribute__((always_inline)) {
    float e0, e1;
    row_pair(x, row, dk, lane, e0, e1);
    if (on) {
      const float n = __builtin_amdgcn_rsqf(wave_sum(__builtin_fmaf(e0, e0, e1 * e1)) + kUnitGuard);
      e0 *= n;
      e1 *= n;
    }
    put_pair(y, row, dk, lane, e0, e1);
  };
  unit(k, kf, flags & kFuseNormK);
  unit(q, qf, flags & kFuseNormQ);
  const bool gates = flags & kFuseGates;
  if (flags & kScalarGate) {
    const float a = to_f32(alpha[row]);
    const float g = gates ? practical_gate(a) : a;
    put_pair(af, row, dk, lane, g, g);
  } else {
    float a0, a1;
    row_pair(alpha, row, dk, lane, a0, a1);
    put_pair(af, row, dk, lane, gates ? practical_gate(a0) : a0, gates ? practical_gate(a1) : a1);
  }
  if (lane == 0) {
    const float b = to_f32(beta[row]);
    bf[row] = gates ? practical_beta(b) : b;
  }
  float v0, v1;
  row_pair(v, row, dv, lane, v0, v1);
  put_pair(vf, row, dv, lane, v0, v1);
  row_pair(dout, row, dv, lane, v0, v1);
  put_pair(of, row, dv, lane, v0, v1);
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
    float e0, e1, g0, g1;
    row_pair(x, row, d, lane, e0, e1);
    g0 = lane < d ? g[row * d + lane] : 0.f;
    g1 = lane + 64 < d ? g[row * d + lane + 64] : 0.f;
    const float n = __builtin_amdgcn_rsqf(wave_sum(__builtin_fmaf(e0, e0, e1 * e1)) + kUnitGuard);
    const float y0 = e0 * n, y1 = e1 * n;
    const float ydy = wave_sum(__builtin_fmaf(y0, g0, y1 * g1));
    put_pair(g, row, d, lane, n * __builtin_fmaf(-y0, ydy, g0), n * __builtin_fmaf(-y1, ydy, g1));
  };
  if (flags & kFuseNormK) unit_bwd(k, dk);
  if (flags & kFuseNormQ) unit_bwd(q, dq);
  const bool gates = flags & kFuseGates;
  if (flags & kScalarGate) {
    float g0 = lane < d ? galpha_ch[row * d + lane] : 0.f;
    float g1 = lane + 64 < d ? galpha_ch[row * d + lane + 64] : 0.f;
    const float sum = wave_sum(g0 + g1);
    if (lane == 0) dalpha[row] = gates ? sum * practical_gate_slope(to_f32(alpha[row])) : sum;
  } else if (gates) {
    float a0, a1;
    row_pair(alpha, row, d, lane, a0, a1);
    if (lane < d) dalpha[row * d + lane] *= practical_gate_slope(a0);
    if (lane + 64 < d) dalpha[row * d + lane + 64] *= practical_gate_slope(a1);
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
