// dp2_bwd.hip -- backward of the DeltaProduct_2 comparator
// (ckda_deltaproduct2_bwd).
//
// DeltaProduct_2 makes two delta-rule updates per token ("Complex KDA" paper,
// Fig. 5 and Sec. 6; the gated form scales the state by the token's scalar
// gate first, App. C).  As the forward does, the backward treats it as the
// delta rule over 2 T sub-steps: sub-step 2 t gated by alpha_t on every key
// channel, sub-step 2 t + 1 ungated, only odd sub-steps read out (with q_t).
// k, v and beta, stored [B, H, T, 2, .], already are that sequence; so:
//   1. dp2_expand_kernel writes, in the input dtype (exact copies), the
//      sub-step queries (q_t twice), gates ([alpha_t, 1] on every channel, or
//      1 when ungated) and upstream gradients ([0, do_t]);
//   2. the chunked backward (chunk_bwd.hip) runs on the 2 T sub-steps, writing
//      dk, dv, dbeta and dh0 straight to the caller's outputs;
//   3. dp2_fold_kernel sums each token's two sub-step query gradients and its
//      gate sub-step's channel gate gradients.
// One wave per sub-step row (expand) or token row (fold); lane l holds
// channels 4 l .. 4 l + 3 (d <= 128).
#include "ckda_device.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int kDp2Rows = 4;   // rows per workgroup, one wave each

// four elements of the storage type, moved as one unit
template <typename T> struct Four;
template <> struct Four<float> {
  typedef f32x4 raw;
  static __device__ __forceinline__ raw splat(float x) { return raw{x, x, x, x}; }
};
template <> struct Four<bf16_t> {
  typedef u32x2 raw;
  static __device__ __forceinline__ raw splat(float x) {
    const uint32_t h = (uint32_t)from_f32<bf16_t>(x).bits;
    return raw{h | (h << 16), h | (h << 16)};
  }
};

template <typename T>
__global__ __launch_bounds__(64 * kDp2Rows) void dp2_expand_kernel(const T* q, const T* alpha, const T* dout, T* q2,
                                                                  T* a2, T* do2, long long nsub, int dk, int dv) {
  const long long s = (long long)blockIdx.x * kDp2Rows + threadIdx.x / 64;   // sub-step row
  if (s >= nsub) return;
  const int lane = threadIdx.x & 63;
  const long long t = s >> 1;   // its token
  const bool first = (s & 1) == 0;
  typedef typename Four<T>::raw R4;
  const int c = 4 * lane;
  if (c < dk) {
    *reinterpret_cast<R4*>(q2 + s * dk + c) = *reinterpret_cast<const R4*>(q + t * dk + c);
    *reinterpret_cast<R4*>(a2 + s * dk + c) = Four<T>::splat((first && alpha) ? to_f32(alpha[t]) : 1.f);
  }
  if (c < dv)
    *reinterpret_cast<R4*>(do2 + s * dv + c) =
        first ? Four<T>::splat(0.f) : *reinterpret_cast<const R4*>(dout + t * dv + c);
}

__global__ __launch_bounds__(64 * kDp2Rows) void dp2_fold_kernel(const float* gq2, const float* ga2, float* dq,
                                                                float* dalpha, long long ntok, int dk) {
  const long long t = (long long)blockIdx.x * kDp2Rows + threadIdx.x / 64;
  if (t >= ntok) return;   // the whole wave
  const int lane = threadIdx.x & 63;
  float gsum = 0.f;
  const int c = 4 * lane;
  if (c < dk) {
    *reinterpret_cast<f32x4*>(dq + t * dk + c) = *reinterpret_cast<const f32x4*>(gq2 + 2 * t * dk + c) +
                                                 *reinterpret_cast<const f32x4*>(gq2 + (2 * t + 1) * dk + c);
    if (dalpha) {
      const f32x4 g = *reinterpret_cast<const f32x4*>(ga2 + 2 * t * dk + c);
      gsum = (g[0] + g[1]) + (g[2] + g[3]);
    }
  }
  if (dalpha) {
    gsum = wave_sum(gsum);
    if (lane == 0) dalpha[t] = gsum;
  }
}

static size_t part_bytes(size_t n) { return (n + 255) / 256 * 256; }

size_t dp2_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
  const size_t nsub = 2 * (size_t)B * H * T, es = dtype == 1 ? 2 : 4;
  return 2 * part_bytes(nsub * dk * es) + part_bytes(nsub * dv * es) + 2 * part_bytes(nsub * dk * 4) +
         chunk_bwd_workspace_floats(B, H, 2 * T, dk, dv) * 4;
}

template <typename T>
static hipError_t launch_t(const BwdArgs& a) {
  const long long ntok = (long long)a.B * a.H * a.T, nsub = 2 * ntok;
  unsigned char* w = (unsigned char*)a.workspace;
  auto take = [&](size_t bytes) {
    unsigned char* p = w;
    w += part_bytes(bytes);
    return p;
  };
  T* q2 = (T*)take((size_t)nsub * a.dk * sizeof(T));
  T* a2 = (T*)take((size_t)nsub * a.dk * sizeof(T));
  T* do2 = (T*)take((size_t)nsub * a.dv * sizeof(T));
  float* gq2 = (float*)take((size_t)nsub * a.dk * 4);
  float* ga2 = (float*)take((size_t)nsub * a.dk * 4);
  if (nsub > 0) {
    hipLaunchKernelGGL((dp2_expand_kernel<T>), dim3((unsigned)((nsub + kDp2Rows - 1) / kDp2Rows)),
                       dim3(64 * kDp2Rows), 0, a.stream, (const T*)a.q, (const T*)a.alpha, (const T*)a.dout, q2, a2,
                       do2, nsub, a.dk, a.dv);
  }
  BwdArgs s = a;
  s.q = q2;
  s.alpha = a2;
  s.dout = do2;
  s.gq = gq2;
  s.galpha = ga2;
  s.T = 2 * a.T;
  s.workspace = w;
  hipError_t e = launch_chunk_bwd(s);
  if (e != hipSuccess || ntok == 0) return e;
  hipLaunchKernelGGL(dp2_fold_kernel, dim3((unsigned)((ntok + kDp2Rows - 1) / kDp2Rows)), dim3(64 * kDp2Rows), 0,
                     a.stream, gq2, ga2, a.gq, a.alpha ? a.galpha : nullptr, ntok, a.dk);
  return hipGetLastError();
}

hipError_t launch_dp2_bwd(const BwdArgs& a) {
  if ((long long)a.B * a.H == 0) return hipSuccess;
  return a.dtype == 1 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace ckda
