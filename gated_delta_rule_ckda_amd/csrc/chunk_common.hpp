// chunk_common.hpp -- compile-time geometry of the chunkwise forward, shared by
// the Gram kernel (writer of the per-chunk records) and the state-pass kernel
// (their reader).
//
// Per chunk of C positions of one (batch, head), the record holds the
// matrix-core A operands of the state pass as 1 KB fragments (64 lanes x 16
// bytes, K order of ckda_device.hpp), each operand indexed [row tile][K block]:
//   TB  [C x C]  = (I + Diag(beta) A)^-1 Diag(beta)    the UT/WY triangular solve
//   TBL [C x C]  = TB - bf16(TB), rounded to bf16      (bf16 records only: TB as
//                  a hi + lo pair, about 16 significant bits, for the state pass's
//                  U = TB X, which sits on the state's chunk-to-chunk chain)
//   M   [C x C]  = causal (incl. diagonal) decayed query-key products
//   W   [C x DK] = -(K . gamma)      gamma_t: signed gate product from the chunk start to t
//   Q   [C x DK] =   Q . gamma
//   KR  [DK x C] = (K . G(C, .))^T   G(C, t): signed gate product after t to the chunk end
// followed by d = gamma at the last position (DK floats, fp32), padded to a
// whole fragment so that the record is a sequence of 1 KB blocks.

// Padded fragments.  Operands that are assembled in LDS by threads that own a
// pair of channels over a run of rows use a padded fragment: lane (g, r)'s
// 16-byte slot sits at g * kFragGroupBytes + r * 16 (272-byte group stride
// instead of 256).  A wave that stores one row of all channel pairs then hits
// 64 distinct LDS banks, and a wave that reads the fragment (16 lanes of one
// group at a time) hits 64 distinct banks as well.
#pragma once

#include "ckda_device.hpp"

namespace ckda {

constexpr int kFragGroupBytes = 16 * 16 + 16;        // 272
constexpr int kFragPadBytes = 4 * kFragGroupBytes;   // 1088

template <typename T, int DK, int C>
struct ChunkGeom {
  static constexpr int KB = FragTraits<T>::KB;
  static constexpr int EPL = FragTraits<T>::EPL;
  static constexpr int E = sizeof(T);
  static constexpr int RT = C / 16;                 // row tiles of a chunk
  static constexpr int RH = DK / 16;                // row tiles of the state
  static constexpr int KBN = (DK + KB - 1) / KB;    // K blocks over channels
  static constexpr int KBC = (C + KB - 1) / KB;     // K blocks over positions
  static constexpr size_t FRAG = 1024;
  // TB and M are lower triangular (j <= t): of their (row tile, K block)
  // fragments only those reaching the diagonal are stored, row tile by row
  // tile; blocks entirely above it hold zeros and are neither stored nor read
  static constexpr bool tri_live(int pt, int kb) { return kb * KB < 16 * (pt + 1); }
  static constexpr int tri_index(int pt, int kb) {
    int n = 0;
    for (int p = 0; p < pt; ++p)
      for (int b = 0; b < KBC; ++b) n += tri_live(p, b) ? 1 : 0;
    return n + kb;
  }
  static constexpr int NF_T = tri_index(RT, 0);     // stored fragments of TB (and of M)
  static constexpr bool SPLIT = sizeof(T) == 2;     // TB kept as hi + lo (bf16 records)
  static constexpr int NF_TL = SPLIT ? NF_T : 0;    // fragments of TBL
  static constexpr int NF_W = RT * KBN;             // fragments of W (and of Q)
  static constexpr int NF_KR = RH * KBC;            // fragments of KR
  static constexpr int NF_D = (DK * 4 + 1023) / 1024;
  static constexpr int NFR = 2 * NF_T + NF_TL + 2 * NF_W + NF_KR + NF_D;
  static constexpr size_t T_OFF = 0;
  static constexpr size_t TL_OFF = T_OFF + NF_T * FRAG;
  static constexpr size_t M_OFF = TL_OFF + NF_TL * FRAG;
  static constexpr size_t W_OFF = M_OFF + NF_T * FRAG;
  static constexpr size_t Q_OFF = W_OFF + NF_W * FRAG;
  static constexpr size_t KR_OFF = Q_OFF + NF_W * FRAG;
  static constexpr size_t D_OFF = KR_OFF + NF_KR * FRAG;
  static constexpr size_t BYTES = NFR * FRAG;
};

// Position of K index `kk` (0 <= kk < DK or C) in a padded fragment row:
// byte offset of its element relative to the start of row 0 of the fragment
// block for K block 0, i.e. kb * kFragPadBytes + g * kFragGroupBytes + e * sizeof(T).
template <typename T>
__host__ __device__ constexpr int padded_col_offset(int kk) {
  const int kb = kk / FragTraits<T>::KB, o = kk % FragTraits<T>::KB;
  const int g = (sizeof(T) == 2 && o >= 16) ? (o - 16) / 4 : o / 4;
  const int e = (sizeof(T) == 2 && o >= 16) ? 4 + (o - 16) % 4 : o % 4;
  return kb * kFragPadBytes + g * kFragGroupBytes + e * (int)sizeof(T);
}

// Lane `lane`'s slot of padded fragment `f` of a buffer.
__device__ __forceinline__ int padded_slot(int f, int lane) {
  return f * kFragPadBytes + (lane >> 4) * kFragGroupBytes + (lane & 15) * 16;
}

// ---- raw element pairs: two adjacent channels of one row, loaded as one unit
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
  typedef uint32_t raw;
  static __device__ __forceinline__ raw load(const bf16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
  static __device__ __forceinline__ float lo(raw w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(raw w) { return __uint_as_float(w & 0xFFFF0000u); }
  static __device__ __forceinline__ raw ones() { return 0x3F803F80u; }
  static __device__ __forceinline__ raw zeros() { return 0u; }
  static __device__ __forceinline__ raw pack(bf16_t a, bf16_t b) { return (uint32_t)a.bits | ((uint32_t)b.bits << 16); }
  // store two values (channels c, c + 1) of one padded-fragment row
  static __device__ __forceinline__ void put(unsigned char* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
  }
};
template <> struct Pair<float> {
  typedef float __attribute__((ext_vector_type(2))) raw;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const raw*>(p); }
  static __device__ __forceinline__ float lo(raw w) { return w[0]; }
  static __device__ __forceinline__ float hi(raw w) { return w[1]; }
  static __device__ __forceinline__ raw ones() { return raw{1.f, 1.f}; }
  static __device__ __forceinline__ raw zeros() { return raw{0.f, 0.f}; }
  static __device__ __forceinline__ raw pack(float a, float b) { return raw{a, b}; }
  static __device__ __forceinline__ void put(unsigned char* p, float a, float b) {
    *reinterpret_cast<raw*>(p) = raw{a, b};
  }
};

// ---- four adjacent channels of one row, loaded as one unit
template <typename T> struct Quad;
template <> struct Quad<bf16_t> {
  u32x2 w;
  static __device__ __forceinline__ Quad load(const bf16_t* p) {
    Quad x;
    x.w = *reinterpret_cast<const u32x2*>(p);
    return x;
  }
  static __device__ __forceinline__ Quad load(__amdgpu_buffer_rsrc_t r, int byte_off) {
    Quad x;
    x.w = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
    return x;
  }
  __device__ __forceinline__ float get(int j) const {
    const uint32_t x = w[j >> 1];
    return __uint_as_float((j & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
  __device__ __forceinline__ void pin() { ckda::pin(w); }
  static __device__ __forceinline__ Quad ones() { return Quad{u32x2{0x3F803F80u, 0x3F803F80u}}; }
  static __device__ __forceinline__ Quad zeros() { return Quad{u32x2{0u, 0u}}; }
  // store four values as consecutive elements
  static __device__ __forceinline__ void put(unsigned char* p, const float* v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};
template <> struct Quad<float> {
  f32x4 w;
  static __device__ __forceinline__ Quad load(const float* p) {
    Quad x;
    x.w = *reinterpret_cast<const f32x4*>(p);
    return x;
  }
  static __device__ __forceinline__ Quad load(__amdgpu_buffer_rsrc_t r, int byte_off) {
    Quad x;
    x.w = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
    return x;
  }
  __device__ __forceinline__ float get(int j) const { return w[j]; }
  __device__ __forceinline__ void pin() { ckda::pin(w); }
  static __device__ __forceinline__ Quad ones() { return Quad{f32x4{1.f, 1.f, 1.f, 1.f}}; }
  static __device__ __forceinline__ Quad zeros() { return Quad{f32x4{0.f, 0.f, 0.f, 0.f}}; }
  static __device__ __forceinline__ void put(unsigned char* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
};

}  // namespace ckda
