// chunk_common.hpp -- compile-time geometry of the chunkwise forward, shared by
// the preparation kernel (writer of the per-chunk operand records) and the
// state-pass kernel (their reader).
//
// Per chunk of C positions of one (batch, head), with d_k = DK channels, the
// record holds five matrix-core A operands, each as 1 KB fragments (64 lanes x
// 16 bytes, K order of ckda_device.hpp) indexed [row tile][K block]:
//   W   [C  x DK] = -(K~ . gamma)     keys with signs absorbed, decayed to their position
//   Q   [C  x DK] =   Q~ . gamma      queries likewise
//   KR  [DK x C ] = P_C (K~ . gamma_C / gamma)^T   keys decayed to the chunk end
//   TB  [C  x C ] = (I + A)^-1 Diag(beta)          the UT/WY triangular solve
//   M   [C  x C ] = causal (incl. diagonal) decayed query-key products
// followed by DK floats d = P_C gamma_C (the signed decay of the whole chunk).
#pragma once

#include "ckda_device.hpp"

namespace ckda {

template <typename T, int DK, int C>
struct ChunkGeom {
  static constexpr int KB = FragTraits<T>::KB;
  static constexpr int EPL = FragTraits<T>::EPL;
  static constexpr int E = sizeof(T);
  static constexpr int HALVES = KB / 16;            // 16-row accumulator tiles per K block
  static constexpr int RT = C / 16;                 // row tiles of a chunk
  static constexpr int RH = DK / 16;                // row tiles of the state
  static constexpr int KBN = (DK + KB - 1) / KB;    // K blocks over channels
  static constexpr int KBC = (C + KB - 1) / KB;     // K blocks over positions
  static constexpr size_t FRAG = 1024;
  static constexpr size_t W_OFF = 0;
  static constexpr size_t Q_OFF = W_OFF + (size_t)RT * KBN * FRAG;
  static constexpr size_t KR_OFF = Q_OFF + (size_t)RT * KBN * FRAG;
  static constexpr size_t T_OFF = KR_OFF + (size_t)RH * KBC * FRAG;
  static constexpr size_t M_OFF = T_OFF + (size_t)RT * KBC * FRAG;
  static constexpr size_t D_OFF = M_OFF + (size_t)RT * KBC * FRAG;
  static constexpr size_t BYTES = (D_OFF + (size_t)DK * 4 + 255) / 256 * 256;
};

// Byte offset of lane `lane`'s 16-byte slot in fragment (tile, kblock) of an
// operand with `nkb` K blocks.
__host__ __device__ constexpr size_t frag_slot(int tile, int kblock, int nkb, int lane) {
  return (((size_t)tile * nkb + kblock) * 64 + lane) * 16;
}

}  // namespace ckda
