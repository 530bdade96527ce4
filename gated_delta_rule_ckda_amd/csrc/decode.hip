// decode.hip -- single-token CKDA/KDA step with the fp32 state updated in place.
//
// One workgroup per (sequence, head) state.  The state is read from HBM once
// into registers (16-byte vector loads, each wave covering whole contiguous
// rows), the two column reductions s = H^T (alpha . k) and r = H^T (alpha . q)
// are formed from those registers, and the updated state
// H' = Diag(alpha) H + k u^T with u = beta (v - s) is written back once.
// The read-out uses o = H'^T q = r + (k^T q) u, so H' never has to be read
// again.  This is the read-compare-correct step of the KDA course lesson
// (session 17, "Mechanism map"), queried after the update as in the paper's
// Eq. (1); the diagonal-plus-rank-one transition keeps it at O(dk dv) work
// per token (discussion slides, "The transition remains non-expansive and
// inexpensive").  The kernel is HBM-bound: 2 * dk * dv * 4 bytes of state
// traffic per state and step, against a few flops per byte.  The state's
// loads are issued before anything else, and the updated state is written
// with nontemporal (streaming) stores, which lifts the step from about 5.3 to
// about 6.9 TB/s on MI355X.
//
// PRO instantiation: the per-token prologue (ckda.h, CKDA_FUSE_*) runs on the
// loaded token before the step: gates and beta from their logits, keys and
// queries scaled to unit norm (one wave reduces each vector).  It also
// gathers each head's retained key channels from rows of dk_in when gidx is
// set.
#include "ckda_device.hpp"
#include "ckda_internal.hpp"

namespace ckda {

static_assert(kFuseGates == CKDA_FUSE_GATES && kFuseNormK == CKDA_FUSE_NORM_K && kFuseNormQ == CKDA_FUSE_NORM_Q &&
                  kScalarGate == CKDA_GATE_SCALAR && (kProd2 & 0xFF) == 0,
              "prologue flags");

constexpr int kDecodeThreads = 256;

template <typename T, int DK, int DV, bool PRO>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ alpha, const T* __restrict__ beta, float* __restrict__ H,
    T* __restrict__ o, int flags, const int* __restrict__ gidx, int dk_in, int nheads) {
  constexpr int TPR = DV / 4;                    // threads per state row (4 columns each)
  constexpr int RPI = kDecodeThreads / TPR;      // rows covered per pass
  constexpr int ITER = (DK + RPI - 1) / RPI;     // passes over the rows
  static_assert(DV % 4 == 0 && kDecodeThreads % TPR == 0, "decode tiling");

  __shared__ float s_a[DK], s_ak[DK], s_aq[DK], s_k[DK], s_q[DK];
  __shared__ f32x4 s_ps[RPI][TPR], s_pr[RPI][TPR];
  __shared__ float s_kq, s_inv[2];

  const long long st = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % TPR, rg = tid / TPR;

  // the state first: its loads are the long ones
  float* Hs = H + st * (long long)DK * DV;
  f32x4 h[ITER];
#pragma unroll
  for (int j = 0; j < ITER; ++j) {
    const int row = rg + j * RPI;
    if (row < DK) h[j] = *reinterpret_cast<const f32x4*>(Hs + row * DV + 4 * cg);
  }
  if constexpr (PRO) {
    for (int i = tid; i < DK; i += kDecodeThreads) {
      // channel gather: element i of the retained set (index clamped into the row)
      const long long e = gidx ? st * (long long)dk_in + min(max(gidx[(st % nheads) * DK + i], 0), dk_in - 1)
                               : st * DK + i;
      const float a = to_f32(alpha[(flags & kScalarGate) ? st : e]);   // scalar gate: one per state
      s_a[i] = (flags & kFuseGates) ? practical_gate(a) : a;
      s_k[i] = to_f32(k[e]);
      s_q[i] = to_f32(q[e]);
    }
    __syncthreads();
    const int w = tid >> 6;
    if (w < 2) {   // wave 0: |k|, wave 1: |q|
      const float* x = w == 0 ? s_k : s_q;
      float ss = 0.f;
      for (int i = tid & 63; i < DK; i += 64) ss += x[i] * x[i];
      ss = wave_sum(ss);
      const bool on = (flags & (w == 0 ? kFuseNormK : kFuseNormQ)) != 0;
      if ((tid & 63) == 0) s_inv[w] = on ? 1.f / sqrtf(ss + kUnitGuard) : 1.f;
    }
    __syncthreads();
    for (int i = tid; i < DK; i += kDecodeThreads) {
      const float a = s_a[i], kk = s_k[i] * s_inv[0], qq = s_q[i] * s_inv[1];
      s_k[i] = kk;
      s_q[i] = qq;
      s_ak[i] = a * kk;
      s_aq[i] = a * qq;
    }
  } else {
    for (int i = tid; i < DK; i += kDecodeThreads) {
      float a = to_f32(alpha[st * DK + i]), kk = to_f32(k[st * DK + i]), qq = to_f32(q[st * DK + i]);
      s_a[i] = a;
      s_k[i] = kk;
      s_q[i] = qq;
      s_ak[i] = a * kk;
      s_aq[i] = a * qq;
    }
  }
  __syncthreads();

  if (tid < 64) {
    float p = 0.f;
    for (int i = tid; i < DK; i += 64) p += s_k[i] * s_q[i];
    p = wave_sum(p);
    if (tid == 0) s_kq = p;
  }

  f32x4 ps = zero4(), pr = zero4();
#pragma unroll
  for (int j = 0; j < ITER; ++j) {
    const int row = rg + j * RPI;
    if (row < DK) {
      ps += s_ak[row] * h[j];
      pr += s_aq[row] * h[j];
    }
  }
  s_ps[rg][cg] = ps;
  s_pr[rg][cg] = pr;
  __syncthreads();

  f32x4 sc = zero4(), rc = zero4();
#pragma unroll 8
  for (int g = 0; g < RPI; ++g) {
    sc += s_ps[g][cg];
    rc += s_pr[g][cg];
  }
  float b = to_f32(beta[st]);
  if (PRO && (flags & kFuseGates)) b = practical_beta(b);
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = to_f32(v[st * DV + 4 * cg + e]);
  const f32x4 u = b * (vv - sc);

  if (rg == 0) {
    const f32x4 oc = rc + s_kq * u;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[st * DV + 4 * cg + e] = from_f32<T>(oc[e]);
  }

#pragma unroll
  for (int j = 0; j < ITER; ++j) {
    const int row = rg + j * RPI;
    if (row < DK) {
      const f32x4 hn = s_a[row] * h[j] + s_k[row] * u;
      // streaming store: the state is not read again in this step
      __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(Hs + row * DV + 4 * cg));
    }
  }
}

// DeltaProduct_2 step (two delta-rule sub-steps per token, then the read-out;
// a scalar gate, if any, acts before the first), in one read and one write
// of H.  With Hb = alpha H and the three column reductions s1 = Hb^T k1,
// s2 = Hb^T k2, r = Hb^T q of the gated state:
//   u1 = beta1 (v1 - s1),   u2 = beta2 (v2 - s2 - (k1^T k2) u1),
//   o = r + (k1^T q) u1 + (k2^T q) u2,   H <- Hb + k1 u1^T + k2 u2^T,
// since the state after the first sub-step is Hb + k1 u1^T.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kDecodeThreads) void decode_prod2_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ alpha, const T* __restrict__ beta, float* __restrict__ H,
    T* __restrict__ o, int flags) {
  constexpr int TPR = DV / 4;
  constexpr int RPI = kDecodeThreads / TPR;
  constexpr int ITER = (DK + RPI - 1) / RPI;
  __shared__ float s_k1[DK], s_k2[DK], s_q[DK];
  __shared__ f32x4 s_p1[RPI][TPR], s_p2[RPI][TPR], s_pr[RPI][TPR];
  __shared__ float s_inv[3], s_dot[3];

  const long long st = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % TPR, rg = tid / TPR;
  float* Hs = H + st * (long long)DK * DV;
  f32x4 h[ITER];
#pragma unroll
  for (int j = 0; j < ITER; ++j) {
    const int row = rg + j * RPI;
    if (row < DK) h[j] = *reinterpret_cast<const f32x4*>(Hs + row * DV + 4 * cg);
  }
  for (int i = tid; i < DK; i += kDecodeThreads) {
    s_k1[i] = to_f32(k[(2 * st) * DK + i]);
    s_k2[i] = to_f32(k[(2 * st + 1) * DK + i]);
    s_q[i] = to_f32(q[st * DK + i]);
  }
  __syncthreads();
  const int w = tid >> 6;
  if (w < 3) {   // wave 0: |k1|, wave 1: |k2|, wave 2: |q|
    const float* x = w == 0 ? s_k1 : (w == 1 ? s_k2 : s_q);
    float ss = 0.f;
    for (int i = tid & 63; i < DK; i += 64) ss += x[i] * x[i];
    ss = wave_sum(ss);
    const bool on = (flags & (w < 2 ? kFuseNormK : kFuseNormQ)) != 0;
    if ((tid & 63) == 0) s_inv[w] = on ? 1.f / sqrtf(ss + kUnitGuard) : 1.f;
  }
  __syncthreads();
  for (int i = tid; i < DK; i += kDecodeThreads) {
    s_k1[i] *= s_inv[0];
    s_k2[i] *= s_inv[1];
    s_q[i] *= s_inv[2];
  }
  __syncthreads();
  if (w < 3) {   // k1.k2, k1.q, k2.q
    const float* x = w == 2 ? s_k2 : s_k1;
    const float* y = w == 0 ? s_k2 : s_q;
    float p = 0.f;
    for (int i = tid & 63; i < DK; i += 64) p += x[i] * y[i];
    p = wave_sum(p);
    if ((tid & 63) == 0) s_dot[w] = p;
  }
  float a = 1.f;
  if (alpha) {
    a = to_f32(alpha[st]);
    if (flags & kFuseGates) a = practical_gate(a);
  }
  f32x4 p1 = zero4(), p2 = zero4(), pr = zero4();
#pragma unroll
  for (int j = 0; j < ITER; ++j) {
    const int row = rg + j * RPI;
    if (row < DK) {
      h[j] = a * h[j];
      p1 += s_k1[row] * h[j];
      p2 += s_k2[row] * h[j];
      pr += s_q[row] * h[j];
    }
  }
  s_p1[rg][cg] = p1;
  s_p2[rg][cg] = p2;
  s_pr[rg][cg] = pr;
  __syncthreads();
  f32x4 s1 = zero4(), s2 = zero4(), rc = zero4();
#pragma unroll 8
  for (int g = 0; g < RPI; ++g) {
    s1 += s_p1[g][cg];
    s2 += s_p2[g][cg];
    rc += s_pr[g][cg];
  }
  float b1 = to_f32(beta[2 * st]), b2 = to_f32(beta[2 * st + 1]);
  if (flags & kFuseGates) {
    b1 = practical_beta(b1);
    b2 = practical_beta(b2);
  }
  f32x4 v1, v2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v1[e] = to_f32(v[(2 * st) * DV + 4 * cg + e]);
    v2[e] = to_f32(v[(2 * st + 1) * DV + 4 * cg + e]);
  }
  const f32x4 u1 = b1 * (v1 - s1);
  const f32x4 u2 = b2 * (v2 - s2 - s_dot[0] * u1);
  if (rg == 0) {
    const f32x4 oc = rc + s_dot[1] * u1 + s_dot[2] * u2;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[st * DV + 4 * cg + e] = from_f32<T>(oc[e]);
  }
#pragma unroll
  for (int j = 0; j < ITER; ++j) {
    const int row = rg + j * RPI;
    if (row < DK) {
      const f32x4 hn = h[j] + s_k1[row] * u1 + s_k2[row] * u2;
      __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(Hs + row * DV + 4 * cg));
    }
  }
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const long long states = (long long)a.N * a.H;
  if (states == 0) return hipSuccess;
  if (a.flags & kProd2) {
    hipLaunchKernelGGL((decode_prod2_kernel<T, DK, DV>), dim3((unsigned)states), dim3(kDecodeThreads), 0, a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.alpha, (const T*)a.beta, a.H_inout,
                       (T*)a.o, a.flags);
    return hipGetLastError();
  }
  if (a.flags != 0 || a.gidx)
    hipLaunchKernelGGL((decode_kernel<T, DK, DV, true>), dim3((unsigned)states), dim3(kDecodeThreads), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.alpha,
                       (const T*)a.beta, a.H_inout, (T*)a.o, a.flags, a.gidx, a.gidx ? a.dk_in : DK, a.H);
  else
    hipLaunchKernelGGL((decode_kernel<T, DK, DV, false>), dim3((unsigned)states), dim3(kDecodeThreads), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.alpha,
                       (const T*)a.beta, a.H_inout, (T*)a.o, 0, nullptr, DK, 1);
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t dispatch_dv(const DecodeArgs& a) {
  switch (a.dv) {
    case 16: return launch_decode_t<T, DK, 16>(a);
    case 32: return launch_decode_t<T, DK, 32>(a);
    case 64: return launch_decode_t<T, DK, 64>(a);
    case 128: return launch_decode_t<T, DK, 128>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dispatch_dk(const DecodeArgs& a) {
  switch (a.dk) {
    case 16: return dispatch_dv<T, 16>(a);
    case 32: return dispatch_dv<T, 32>(a);
    case 64: return dispatch_dv<T, 64>(a);
    case 128: return dispatch_dv<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.dtype == 1 ? dispatch_dk<bf16_t>(a) : dispatch_dk<float>(a);
}

}  // namespace ckda
