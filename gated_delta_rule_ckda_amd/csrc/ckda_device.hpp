// ckda_device.hpp -- gfx950 device building blocks shared by the CKDA kernels:
// element conversion, 16-byte MFMA operand fragments and the matrix-core
// products built on them.
//
// Fragment convention.  Every matrix-core product here produces 16x16 fp32
// tiles in the MFMA accumulator layout: lane l (g = l / 16, r = l % 16) holds
// rows 4g .. 4g+3 of column r.  Operands are moved as 16-byte fragments, one
// per lane, covering a 16-row tile of a row-major operand over one "K block"
// of its contraction index:
//   bf16 : K block of 32; lane (g, r) holds 8 values at k = kappa(g, e),
//          kappa(g, e) = 4g + e for e < 4 and 16 + 4g + (e - 4) for e >= 4;
//          consumed by one v_mfma_f32_16x16x32_bf16.
//   fp32 : K block of 16; lane (g, r) holds 4 values at k = 4g + e;
//          consumed by four v_mfma_f32_16x16x4_f32 (sub-step e uses value e).
// With this K order the accumulator registers of the 16x16 tiles covering a
// K block are, converted element-wise, exactly the B-operand fragment of that
// K block (bf16: two tiles, rows 0-15 then 16-31; fp32: one tile), so a
// product's result feeds the next product without a shuffle.  Any operand
// that meets it on the other side must be laid out in the same K order, which
// the Gram kernel does when it writes the chunk records.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- elements

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, h);
  return r;
}

// ---------------------------------------------------------------- prologue
// The per-token prologue the fused entry points apply (ckda.h, CKDA_FUSE_*):
// the practical gate parameterisation of the "Complex KDA" discussion slides
// (frame "Backup: practical gates differ from exact theoretical endpoints")
// and unit-norm keys and queries.
constexpr int kFuseGates = 1, kFuseNormK = 2, kFuseNormQ = 4;   // as CKDA_FUSE_GATES, _NORM_K, _NORM_Q
constexpr int kScalarGate = 8;   // as CKDA_GATE_SCALAR: one gate per token and head
constexpr float kUnitGuard = 1e-6f;                 // x / sqrt(sum x^2 + guard)
constexpr float kGateFloor = 0.006737946999085467f;  // e^-5: log|alpha| >= -5

// alpha = sign(a) (eps + (1 - eps) |tanh(a / 2)|), sign(0) = +1, in a few
// VALU operations.  With x = |a| / 2:
//   x < 5/16: the Maclaurin series of tanh, x - x^3/3 + 2x^5/15 - 17x^7/315
//             + 62x^9/2835 - 1382x^11/155925 (next term below 2^-27 x);
//   else:     (1 - e) / (1 + e), e = e^-2x by v_exp_f32 and v_rcp_f32
//             (1 - e > 0.46, no cancellation).
// Both branches are evaluated and selected (no divergence); a few ulp.
__device__ __forceinline__ float tanh_half_abs(float a) {   // |tanh(a / 2)|
  const float x = 0.5f * fabsf(a);
  const float z = x * x;
  float p = -1382.f / 155925.f;
  p = __builtin_fmaf(p, z, 62.f / 2835.f);
  p = __builtin_fmaf(p, z, -17.f / 315.f);
  p = __builtin_fmaf(p, z, 2.f / 15.f);
  p = __builtin_fmaf(p, z, -1.f / 3.f);
  const float small = __builtin_fmaf(p * z, x, x);
  const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * x);   // 2 log2(e) = 2.88539...
  const float large = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
  return x < 0.3125f ? small : large;
}
__device__ __forceinline__ float practical_gate(float a) {
  const float g = __builtin_fmaf(1.f - kGateFloor, tanh_half_abs(a), kGateFloor);
  return a >= 0.f ? g : -g;
}
// d alpha / d a with the sign held constant: s (1 - eps) d|r|/da = (1 - eps)
// (1 - r^2) / 2, and the zero subgradient of |r| at r = 0 (a = 0).
__device__ __forceinline__ float practical_gate_slope(float a) {
  const float r = tanh_half_abs(a);
  return a == 0.f ? 0.f : 0.5f * (1.f - kGateFloor) * __builtin_fmaf(-r, r, 1.f);
}

// beta = 2 sigma(b) in [0, 2].
__device__ __forceinline__ float practical_beta(float b) { return 2.f / (1.f + expf(-b)); }
// d beta / d b = 2 sigma(b) (1 - sigma(b)).
__device__ __forceinline__ float practical_beta_slope(float b) {
  const float sg = 1.f / (1.f + expf(-b));
  return 2.f * sg * (1.f - sg);
}

// Two floats -> packed bf16 pair (low = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- fragments

// A 16-byte operand fragment held by one lane.
struct Frag {
  u32x4 w;
};

template <typename T> struct FragTraits;
template <> struct FragTraits<bf16_t> {
  static constexpr int KB = 32;  // contraction length covered by one fragment
  static constexpr int EPL = 8;  // elements per lane
};
template <> struct FragTraits<float> {
  static constexpr int KB = 16;
  static constexpr int EPL = 4;
};

// K offset of element e held by lane group g within a K block.
template <typename T> __host__ __device__ constexpr int kappa(int g, int e);
template <> __host__ __device__ constexpr int kappa<bf16_t>(int g, int e) {
  return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
}
template <> __host__ __device__ constexpr int kappa<float>(int g, int e) { return 4 * g + e; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// acc += A_frag * B_frag over one K block.
template <typename T> __device__ __forceinline__ f32x4 mma(f32x4 acc, Frag a, Frag b);

template <> __device__ __forceinline__ f32x4 mma<bf16_t>(f32x4 acc, Frag a, Frag b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.w),
                                                 __builtin_bit_cast(bf16x8, b.w), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mma<float>(f32x4 acc, Frag a, Frag b) {
  f32x4 fa = __builtin_bit_cast(f32x4, a.w), fb = __builtin_bit_cast(f32x4, b.w);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], acc, 0, 0, 0);
  return acc;
}

// Accumulator tiles -> B fragment of the K block they cover.
// bf16: lo = tile of K rows 0-15, hi = tile of K rows 16-31 (may be zero).
__device__ __forceinline__ Frag frag_from_acc_bf16(f32x4 lo, f32x4 hi) {
  Frag f;
  f.w[0] = pack_bf16x2(lo[0], lo[1]);
  f.w[1] = pack_bf16x2(lo[2], lo[3]);
  f.w[2] = pack_bf16x2(hi[0], hi[1]);
  f.w[3] = pack_bf16x2(hi[2], hi[3]);
  return f;
}
// Split bf16 operands.  A value x is carried as hi = bf16(x) and
// lo = bf16(x - hi) (x - hi is exact in fp32), about 16 significant bits in
// all; a product then takes the partial products hi.hi, hi.lo and lo.hi,
// whose sum differs from the fp32 product by about 2^-16 relative.
__device__ __forceinline__ float bf16_lo_half(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_half(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// The lo fragment of 8 values v whose hi fragment (same K order) is `hi`.
__device__ __forceinline__ Frag frag_residual_bf16(const float* v, Frag hi) {
  Frag f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.w[i] = pack_bf16x2(v[2 * i] - bf16_lo_half(hi.w[i]), v[2 * i + 1] - bf16_hi_half(hi.w[i]));
  return f;
}
// hi and lo of the pair (a, b), packed.  The empty asm hides the packed hi
// word from the optimiser, which would otherwise convert a again on its own
// to get the low half back (one conversion more per pair).
__device__ __forceinline__ void split_pair_bf16(float a, float b, uint32_t& h, uint32_t& l) {
  uint32_t w = pack_bf16x2(a, b);
  asm("" : "+v"(w));
  h = w;
  l = pack_bf16x2(a - bf16_lo_half(w), b - bf16_hi_half(w));
}
// hi and lo B fragments of the K block covered by accumulator tiles lo, hi.
__device__ __forceinline__ void frags_from_acc_bf16_split(f32x4 lo, f32x4 hi, Frag& fh, Frag& fl) {
  const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a, b;
    split_pair_bf16(v[2 * i], v[2 * i + 1], a, b);
    fh.w[i] = a;
    fl.w[i] = b;
  }
}
__device__ __forceinline__ Frag frag_from_acc_f32(f32x4 t) {
  Frag f;
  f.w = __builtin_bit_cast(u32x4, t);
  return f;
}

__device__ __forceinline__ Frag load_frag(const void* p) {
  Frag f;
  f.w = *reinterpret_cast<const u32x4*>(p);
  return f;
}
__device__ __forceinline__ void store_frag(void* p, Frag f) { *reinterpret_cast<u32x4*>(p) = f.w; }
// global memory, nontemporal (streaming) store
__device__ __forceinline__ void store_frag_stream(void* p, Frag f) {
  __builtin_nontemporal_store(f.w, reinterpret_cast<u32x4*>(p));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads and stores (on gfx9-family GPUs the vector memory
// counter covers both), so prefetches and output stores stay in flight across
// it.  Use it only where the waves exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- register-level helpers
// Ties a value to this point of the program: the compiler may not move its
// uses above it, so a widening of prefetched bits cannot be hoisted into an
// earlier phase (which would make that phase wait for the prefetch).
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(u32x2& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(f32x4& x) { asm volatile("" : "+v"(x)); }

// ---- range-checked buffer access
// A raw buffer resource over `bytes` bytes from `base` (stride 0, so an access
// at byte offset >= bytes is out of range: stores are dropped, loads read 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// four consecutive elements from LDS, widened
template <typename T> __device__ __forceinline__ f32x4 load_vals4(const unsigned char* p);
template <> __device__ __forceinline__ f32x4 load_vals4<float>(const unsigned char* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <> __device__ __forceinline__ f32x4 load_vals4<bf16_t>(const unsigned char* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u), __uint_as_float(w[1] << 16),
               __uint_as_float(w[1] & 0xFFFF0000u)};
}

// four consecutive elements to global memory in the storage type
template <typename T> __device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 x);
template <> __device__ __forceinline__ void store4<float>(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, byte_off, 0, 0);
}
template <> __device__ __forceinline__ void store4<bf16_t>(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])}, r, byte_off, 0, 0);
}

// Sum over aligned groups of N lanes (N = 2 .. 64), every lane of a group
// receiving its group's sum; all lanes of the wave must be active.  Within a
// 16-lane row the steps are DPP moves (swap neighbours, swap pairs, mirror
// each half row, mirror the row: after the sums so far, each mirror partner
// lies in the other half); across rows, DPP row broadcasts accumulate the
// group's sum in its last lane, which v_readlane hands to the group.
template <int CTRL> __device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "group size");
  x = dpp_add<0xB1>(x);                            // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x = dpp_add<0x4E>(x);      // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x = dpp_add<0x141>(x);     // row_half_mirror
  if constexpr (N >= 16) x = dpp_add<0x140>(x);    // row_mirror
  if constexpr (N >= 32) {
    // row_bcast:15 into rows 1 and 3: they now hold the sums of rows 0-1, 2-3
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false));
    if constexpr (N == 32) {
      const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
      const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
      x = (threadIdx.x & 32) ? hi : lo;
    } else {
      // row_bcast:31 into rows 2 and 3: row 3 now holds the wave's sum
      x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false));
      x = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
    }
  }
  return x;
}

// Wave-wide sum (wave64) via cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace ckda
