// chunk_state.hip -- chunk-to-chunk state pass and output of the chunkwise
// CKDA forward.
//
// Per chunk, with gamma_t the signed product of the gates from the chunk start
// to t and G(C, t) the product after t to the chunk end (chunk form of the
// recurrence of the "Complex KDA" paper, Eq. (1), as in chunk_gram.hip):
//   X = V + W H            W  = -(K . gamma)               [C x DK]
//   U = TB X               TB from the chunk's record
//   O = Q~ H + M U         Q~ = Q . gamma, M from the record
//   H <- d . H + KR^T U    KR = K . G(C, .)  [C x DK],  d = gamma_C
//
// One workgroup per (batch, head, slice of 16 NMW value columns).  The columns
// of the state evolve independently once keys, gates and beta are fixed, so
// each "matrix wave" owns 16 columns and runs the whole recurrence in its own
// registers: its fp32 state slice H (DK x 16) stays in accumulators, and with
// the K order of ckda_device.hpp the accumulator tiles of one product are,
// converted element-wise, the B operand of the next (H for X and O, X for U,
// U for O and H), so the matrix waves exchange nothing.  The decay of H is
// applied element-wise in fp32; the state itself is never rounded.
//
// Four "build waves" assemble the operands of the next chunk in LDS while
// the matrix waves work on the current one: W, Q~ and KR^T from the chunk's
// keys, queries and gates, d, a copy of TB and M from the record, and the
// slice's values V.  So the matrix waves issue no global loads, only the
// output stores: with loads and stores in flight together, every wait for a
// load would also wait for all stores.  Build
// thread (tile bb, channel quad cq, half hf) owns channels 4 cq .. 4 cq + 3
// over rows 16 bb + 8 hf .. + 7: the gate products along the rows are running
// products inside the thread, the two halves of a tile meet through a DPP
// swap, and whole-tile products go through LDS one chunk ahead.  Every factor
// is a product of gates of modulus at most 1: no floor or reciprocal here.
//
// Operand sets are double-buffered (one copy when two do not fit in LDS), so
// one workgroup barrier per chunk separates "build chunk c + 1" from "use
// chunk c".
#include <type_traits>

#include "chunk_common.hpp"
#include "ckda_internal.hpp"

namespace ckda {

template <typename T, int DK, int C, int NMW>
struct StateCfg : ChunkGeom<T, DK, C> {
  using G = ChunkGeom<T, DK, C>;
  static constexpr int NTHREADS = (NMW + 4) * 64;
  static constexpr int NTM = 2 * G::RT * G::KBC;            // TB and M fragments of a record
  // one operand set: padded fragments of W, Q~ [RT][KBN], KR^T [RH][KBC];
  // TB and M as stored in the record; d
  static constexpr int W_OFF = 0;
  static constexpr int Q_OFF = W_OFF + G::RT * G::KBN * kFragPadBytes;
  static constexpr int KR_OFF = Q_OFF + G::RT * G::KBN * kFragPadBytes;
  static constexpr int TM_OFF = KR_OFF + G::RH * G::KBC * kFragPadBytes;
  static constexpr int D_OFF = TM_OFF + NTM * 1024;
  // V of the slice in accumulator order: [matrix wave][row tile][lane][4]
  static constexpr int V_OFF = D_OFF + DK * 4;
  static constexpr int V_BYTES = NMW * G::RT * 64 * 4 * (int)sizeof(T);
  static constexpr int SET_BYTES = V_OFF + V_BYTES;
  static constexpr int TOT_BYTES = 2 * G::RT * DK * 4;      // tile products of two chunks
  static constexpr int NBUF = 2 * SET_BYTES + TOT_BYTES <= 160 * 1024 ? 2 : 1;
  static constexpr int LDS_BYTES = NBUF * SET_BYTES + TOT_BYTES;
};

// Calls f(c, integral_constant<c % NPF>) for c = 0 .. n-1.  Whole groups of
// NPF chunks run in a loop whose body has no conditional part, so that the
// compiler sees the same outstanding prefetches on every path through it and
// waits for exactly the loads a chunk needs; the remainder follows the loop.
template <int NPF, typename F>
__device__ __forceinline__ void run_chunks(int n, F&& f) {
  int cb = 0;
  for (; cb + NPF <= n; cb += NPF) {
    f(cb, std::integral_constant<int, 0>{});
    if constexpr (NPF > 1) f(cb + 1, std::integral_constant<int, (NPF > 1 ? 1 : 0)>{});
    if constexpr (NPF > 2) f(cb + 2, std::integral_constant<int, (NPF > 2 ? 2 : 0)>{});
  }
  if constexpr (NPF > 1) {
    if (cb < n) f(cb, std::integral_constant<int, 0>{});
  }
  if constexpr (NPF > 2) {
    if (cb + 1 < n) f(cb + 1, std::integral_constant<int, (NPF > 2 ? 1 : 0)>{});
  }
}

// Calls f(integral_constant<c % NPF>) for a chunk index known only at run time.
template <int NPF, typename F>
__device__ __forceinline__ void with_slot(int c, F&& f) {
  const int j = c % NPF;
  if (j == 0) f(std::integral_constant<int, 0>{});
  if constexpr (NPF > 1) {
    if (j == 1) f(std::integral_constant<int, (NPF > 1 ? 1 : 0)>{});
  }
  if constexpr (NPF > 2) {
    if (j == 2) f(std::integral_constant<int, (NPF > 2 ? 2 : 0)>{});
  }
}

template <typename T, int DK, int C, int NMW>
__global__ __launch_bounds__((StateCfg<T, DK, C, NMW>::NTHREADS)) void chunk_state_kernel(
    const T* q, const T* k, const T* alpha, const T* v, const float* __restrict__ h0, T* o,
    float* __restrict__ hT, const unsigned char* rec, int T_len, int nchunks, int dv, int slices,
    int xcd_map) {
  using S = StateCfg<T, DK, C, NMW>;
  constexpr int RT = S::RT, RH = S::RH, KBN = S::KBN, KBC = S::KBC, NBUF = S::NBUF, NTM = S::NTM;
  constexpr int E = (int)sizeof(T);
  constexpr bool BF = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) unsigned char lds[S::LDS_BYTES];
  unsigned char* const sets = lds;
  float* const s_tot = reinterpret_cast<float*>(lds + NBUF * S::SET_BYTES);   // [2][RT][DK]

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane / 16, r = lane % 16;
  const bool matrix = wave < NMW;

  // workgroup -> (head, slice); with xcd_map the slices of one head get ids
  // that are equal modulo 8 so that they share an XCD's L2 (workgroups are
  // dispatched to the 8 XCDs round-robin)
  int bh, slice;
  {
    const int id = blockIdx.x;
    if (xcd_map) {
      const int xcd = id % 8, k8 = id / 8;
      bh = (k8 / slices) * 8 + xcd;
      slice = k8 % slices;
    } else {
      bh = id / slices;
      slice = id % slices;
    }
  }

  // zero the operand sets once: fragment slots that no thread writes
  // (channels or positions past DK or C inside a K block) must read as zero
  for (int i = tid; i < NBUF * S::SET_BYTES / 16; i += S::NTHREADS)
    reinterpret_cast<u32x4*>(sets)[i] = u32x4{0u, 0u, 0u, 0u};
  lds_barrier();

  const long long rowbase = (long long)bh * T_len;   // first input row of this (batch, head)
  const __amdgpu_buffer_rsrc_t rrsrc =
      make_rsrc(rec + (size_t)bh * nchunks * S::BYTES, (uint32_t)((size_t)nchunks * S::BYTES));
  auto set_of = [&](int c) __attribute__((always_inline)) { return sets + (NBUF == 2 ? (c & 1) : 0) * S::SET_BYTES; };

  if (matrix) {
    // ============================================================ matrix waves
    // This head's output rows as a range-checked buffer: stores to rows past
    // the end of the sequence are dropped.
    const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(o + rowbase * dv, (uint32_t)((size_t)T_len * dv * E));
    const int col = slice * 16 * NMW + 16 * wave + r;       // this lane's value column
    const long long sbase = (long long)bh * DK * dv;
    f32x4 hacc[RH];
#pragma unroll
    for (int j = 0; j < RH; ++j) {
      hacc[j] = zero4();
      if (h0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hacc[j][i] = h0[sbase + (long long)(16 * j + 4 * g + i) * dv + col];
      }
    }
    // B operand of K block kb from accumulator tiles (bf16: two tiles)
    auto bfrag = [&](const f32x4* acc, int kb, int ntiles) __attribute__((always_inline)) {
      if constexpr (BF) return frag_from_acc_bf16(acc[2 * kb], 2 * kb + 1 < ntiles ? acc[2 * kb + 1] : zero4());
      else return frag_from_acc_f32(acc[kb]);
    };
    lds_barrier();   // the build waves prepare chunk 0
    lds_barrier();

    auto iter = [&](int c, auto) __attribute__((always_inline)) {
      const unsigned char* set = set_of(c);
      // Operand fragments are read from LDS one group ahead of the products
      // that use them; the scheduling barriers keep each group of reads
      // together so that their latencies overlap.  (fp32 fragments are twice
      // as many: no read-ahead there, to stay within the register file.)
      constexpr int DB = BF ? 2 : 1;
      Frag wf[DB][KBN], qf[DB][KBN], tf[RT][KBC], mf[RT][KBC];
      auto ld_wq = [&](int pt) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
          wf[pt % DB][kb] = load_frag(set + S::W_OFF + padded_slot(pt * KBN + kb, lane));
          qf[pt % DB][kb] = load_frag(set + S::Q_OFF + padded_slot(pt * KBN + kb, lane));
        }
      };
      auto ld_tm = [&](Frag (*dst)[KBC], int which) __attribute__((always_inline)) {
#pragma unroll
        for (int pt = 0; pt < RT; ++pt)
#pragma unroll
          for (int kb = 0; kb < KBC; ++kb)
            dst[pt][kb] = load_frag(set + S::TM_OFF + (((which * RT + pt) * KBC + kb) * 64 + lane) * 16);
      };
      constexpr int RHG = RH < 2 ? RH : 2;   // state row tiles per group of reads
      constexpr int NG = RH / RHG;
      Frag kf[2][RHG][KBC];
      f32x4 dd[2][RHG];
      auto ld_kr = [&](int grp) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < RHG; ++j) {
          const int rh = grp * RHG + j;
          dd[grp & 1][j] = *reinterpret_cast<const f32x4*>(set + S::D_OFF + (16 * rh + 4 * g) * 4);
#pragma unroll
          for (int kb = 0; kb < KBC; ++kb)
            kf[grp & 1][j][kb] = load_frag(set + S::KR_OFF + padded_slot(rh * KBC + kb, lane));
        }
      };

      Frag hb[KBN];
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) hb[kb] = bfrag(hacc, kb, RH);
      // X = V + W H, O = Q~ H
      f32x4 xacc[RT], oacc[RT];
      if constexpr (DB == 2) ld_wq(0);
#pragma unroll
      for (int pt = 0; pt < RT; ++pt) {
        if constexpr (DB == 2) {
          if (pt + 1 < RT) ld_wq(pt + 1);
          else ld_tm(tf, 0);
        } else {
          ld_wq(pt);
        }
        __builtin_amdgcn_sched_barrier(0);
        xacc[pt] = load_vals4<T>(set + S::V_OFF + ((wave * RT + pt) * 64 + lane) * 4 * E);
        oacc[pt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
          xacc[pt] = mma<T>(xacc[pt], wf[pt % DB][kb], hb[kb]);
          oacc[pt] = mma<T>(oacc[pt], qf[pt % DB][kb], hb[kb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (DB == 1) ld_tm(tf, 0);
      if constexpr (DB == 2) ld_tm(mf, 1);
      __builtin_amdgcn_sched_barrier(0);
      // U = TB X
      Frag xb[KBC];
#pragma unroll
      for (int kb = 0; kb < KBC; ++kb) xb[kb] = bfrag(xacc, kb, RT);
      f32x4 uacc[RT];
#pragma unroll
      for (int pt = 0; pt < RT; ++pt) {
        uacc[pt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) uacc[pt] = mma<T>(uacc[pt], tf[pt][kb], xb[kb]);
      }
      if constexpr (DB == 1) ld_tm(mf, 1);
      ld_kr(0);
      __builtin_amdgcn_sched_barrier(0);
      Frag ub[KBC];
#pragma unroll
      for (int kb = 0; kb < KBC; ++kb) ub[kb] = bfrag(uacc, kb, RT);
      // O += M U
      const int t0 = c * C;
#pragma unroll
      for (int pt = 0; pt < RT; ++pt) {
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) oacc[pt] = mma<T>(oacc[pt], mf[pt][kb], ub[kb]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_elem<T>(orsrc, ((t0 + 16 * pt + 4 * g + i) * dv + col) * E, oacc[pt][i]);
      }
      // H <- d . H + KR^T U
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) {
        if (grp + 1 < NG) ld_kr(grp + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < RHG; ++j) {
          const int rh = grp * RHG + j;
          f32x4 hh = dd[grp & 1][j] * hacc[rh];
#pragma unroll
          for (int kb = 0; kb < KBC; ++kb) hh = mma<T>(hh, kf[grp & 1][j][kb], ub[kb]);
          hacc[rh] = hh;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      lds_barrier();
      if constexpr (NBUF == 1) {
        lds_barrier();   // the build waves rewrite the one set
      }
    };
    run_chunks<1>(nchunks, iter);

    if (hT) {
#pragma unroll
      for (int j = 0; j < RH; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) hT[sbase + (long long)(16 * j + 4 * g + i) * dv + col] = hacc[j][i];
    }
  } else {
    // ============================================================ build waves
    constexpr int NCQ = DK / 4;
    constexpr int BPF = 2;                       // input slots: chunk x lives in slot x % 2
    constexpr int NTMW = (NTM + 3) / 4;          // record fragments copied per build wave
    const int bw = wave - NMW;                   // build wave 0..3
    const int bt = tid - NMW * 64;
    const int hf = bt & 1, cq = (bt >> 1) % NCQ, bb = bt / (2 * NCQ);
    // every build thread is busy when the tiles fill the 256 build threads
    const bool bact = 2 * NCQ * RT >= 256 || bb < RT;
    const int bc0 = 4 * cq, brow0 = 16 * bb + 8 * hf;
    const uint32_t in_bytes = (uint32_t)((size_t)T_len * DK * E);
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(alpha + rowbase * DK, in_bytes);
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(k + rowbase * DK, in_bytes);
    const __amdgpu_buffer_rsrc_t qrsrc = make_rsrc(q + rowbase * DK, in_bytes);
    const int in_voff = (brow0 * DK + bc0) * E;
    // bf16 inputs are prefetched whole; for fp32 (twice the registers) keys
    // and queries are loaded when the build needs them
    constexpr bool KQ_AHEAD = BF;
    // values of the slice: thread vt reads 8 consecutive columns of one row
    constexpr int VCG = 2 * NMW;                     // 8-column groups per row
    const int vrow = bt / VCG, vcg = bt % VCG;
    const bool vact = bt < C * VCG;
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(v + rowbase * dv, (uint32_t)((size_t)T_len * dv * E));
    const int v_voff = (vrow * dv + slice * 16 * NMW + 8 * vcg) * E;
    struct BRaw {
      Quad<T> a[8], k[KQ_AHEAD ? 8 : 1], q[KQ_AHEAD ? 8 : 1];
    };
    BRaw br[BPF];
    // TB and M fragments and 8 values on their way to LDS (loaded at the start
    // of an iteration, stored at its end)
    Frag tm[NTMW];
    Quad<T> vv[2];
    // products of the other half of the tile before / after this half, from
    // btotals of a chunk to its bbuild one iteration later
    float pre[4], suf[4];
    Quad<T> kq_k[8], kq_q[8];                    // fp32: keys and queries of the chunk being built
    // the record's TB and M fragments and the slice's values, moved by every
    // build wave whatever its share of the channel work
    auto tmload = [&](int c) __attribute__((always_inline)) {
      c = min(c, nchunks - 1);
#pragma unroll
      for (int j = 0; j < NTMW; ++j) {
        const int f = min(bw + 4 * j, NTM - 1);
        tm[j].w = __builtin_amdgcn_raw_buffer_load_b128(rrsrc, c * (int)S::BYTES + (f * 64 + lane) * 16, 0, 0);
      }
      const int ofs = v_voff + c * C * dv * E;
      vv[0] = Quad<T>::load(vrsrc, ofs);
      vv[1] = Quad<T>::load(vrsrc, ofs + 4 * E);
    };
    auto tmstore = [&](int c) __attribute__((always_inline)) {
      unsigned char* set = set_of(c);
#pragma unroll
      for (int j = 0; j < NTMW; ++j) {
        const int f = bw + 4 * j;
        if (f < NTM) store_frag(set + S::TM_OFF + (f * 64 + lane) * 16, tm[j]);
      }
      if (vact) {
        // element (row vrow, column 8 vcg + e) -> matrix wave mw, lane (g, r), slot i
        const int pt = vrow / 16, vg = (vrow % 16) / 4, vi = vrow % 4;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cc = 8 * vcg + e, mw = cc / 16, rr = cc % 16;
          vv[e >> 2].store_raw(set + S::V_OFF + (((mw * RT + pt) * 64 + vg * 16 + rr) * 4 + vi) * E, e & 3);
        }
      }
    };
    // inputs of chunk c (clamped to the last chunk); rows past the end read 0
    auto bload = [&](BRaw& x, int c) __attribute__((always_inline)) {
      c = min(c, nchunks - 1);
      const int ofs = in_voff + c * C * DK * E;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x.a[i] = Quad<T>::load(arsrc, ofs + i * DK * E);
        if constexpr (KQ_AHEAD) {
          x.k[i] = Quad<T>::load(krsrc, ofs + i * DK * E);
          x.q[i] = Quad<T>::load(qrsrc, ofs + i * DK * E);
        }
      }
    };
    // ragged last chunk: rows past the end are identity steps (gate 1; their
    // keys and queries already read as zero)
    auto bfix = [&](BRaw& x, int c) __attribute__((always_inline)) {
      const int cv = T_len - c * C;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (brow0 + i >= cv) x.a[i] = Quad<T>::ones();
    };
    // products of this tile's gates -> s_tot[c % 2]
    auto btotals = [&](BRaw& x, int c) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x.a[i].pin();
      float tot[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p *= x.a[i].get(j);
        const float other = dpp<kDppQuad1032>(p);
        pre[j] = hf ? other : 1.f;
        suf[j] = hf ? 1.f : other;
        tot[j] = hf ? other * p : p * other;   // lower half first in both lanes
      }
      if (hf == 0)
        *reinterpret_cast<f32x4*>(&s_tot[((c & 1) * RT + bb) * DK + bc0]) = f32x4{tot[0], tot[1], tot[2], tot[3]};
    };
    // the operand set of chunk c (tile products already in s_tot[c % 2])
    auto bbuild = [&](BRaw& x, int c) __attribute__((always_inline)) {
      unsigned char* set = set_of(c);
      Quad<T>* kk = kq_k;
      Quad<T>* qq = kq_q;
      if constexpr (KQ_AHEAD) {
        kk = x.k;
        qq = x.q;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x.k[i].pin();
          x.q[i].pin();
        }
      } else {
        const int ofs = in_voff + min(c, nchunks - 1) * C * DK * E;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          kq_k[i] = Quad<T>::load(krsrc, ofs + i * DK * E);
          kq_q[i] = Quad<T>::load(qrsrc, ofs + i * DK * E);
        }
      }
      // products over the tiles before and after this one
      float before[4] = {1.f, 1.f, 1.f, 1.f}, after[4] = {1.f, 1.f, 1.f, 1.f};
      const float* tot = s_tot + (c & 1) * RT * DK;
#pragma unroll
      for (int J = 0; J < RT; ++J) {
        const f32x4 tj = *reinterpret_cast<const f32x4*>(&tot[J * DK + bc0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (J < bb) before[j] *= tj[j];
          if (J > bb) after[j] *= tj[j];
        }
      }
      // W = -(K . gamma), Q~ = Q . gamma (rows of tile bb)
      const int wq = bb * KBN * kFragPadBytes + padded_col_offset<T>(bc0);
      float gm[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) gm[j] = before[j] * pre[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float w[4], qv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          gm[j] *= x.a[i].get(j);
          w[j] = -kk[i].get(j) * gm[j];
          qv[j] = qq[i].get(j) * gm[j];
        }
        const int rr = (8 * hf + i) * 16;
        Quad<T>::put(set + S::W_OFF + wq + rr, w);
        Quad<T>::put(set + S::Q_OFF + wq + rr, qv);
      }
      // d: the whole chunk's decay
      if (bb == 0 && hf == 0)
        *reinterpret_cast<f32x4*>(set + S::D_OFF + bc0 * 4) =
            f32x4{gm[0] * suf[0] * after[0], gm[1] * suf[1] * after[1], gm[2] * suf[2] * after[2],
                  gm[3] * suf[3] * after[3]};
      // KR^T = (K . G(C, .))^T: rows = channels, K = positions brow0 .. brow0 + 7,
      // written four positions at a time
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = suf[j] * after[j];
#pragma unroll
      for (int hq = 1; hq >= 0; --hq) {
        float kr[4][4];
#pragma unroll
        for (int i = 3; i >= 0; --i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kr[j][i] = kk[4 * hq + i].get(j) * e[j];
            e[j] *= x.a[4 * hq + i].get(j);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ch = bc0 + j;
          Quad<T>::put(set + S::KR_OFF + (ch >> 4) * KBC * kFragPadBytes + (ch & 15) * 16 +
                           padded_col_offset<T>(brow0 + 4 * hq),
                       kr[j]);
        }
      }
    };

    // The last chunk is ragged when T is not a multiple of C; only its tile
    // products need the gate fix (done in place, before the build uses them).
    const bool ragged = nchunks > 0 && T_len - (nchunks - 1) * C < C;
    // ---- chunks 0 and 1 in flight; products of chunk 0; build chunk 0, products of chunk 1
    if (nchunks > 0) {
      tmload(0);
      if (bact) {
        bload(br[0], 0);
        bload(br[1], 1);
        if (ragged && nchunks == 1) bfix(br[0], 0);
        btotals(br[0], 0);
      }
    }
    lds_barrier();
    if (nchunks > 0) {
      tmstore(0);
      if (bact) {
        bbuild(br[0], 0);
        if (ragged && nchunks == 2) bfix(br[1], 1);
        btotals(br[1], 1);
        bload(br[0], 2);
      }
    }
    lds_barrier();

    // ---- while the matrix waves run chunk c: build chunk c + 1 (slot
    // (c + 1) % 2), products of chunk c + 2 (slot c % 2), refill slot (c + 1) % 2
    // with chunk c + 3.  Past the last chunk this repeats work on a copy of it
    // that nobody reads, so the work stays unconditional.
    auto iter = [&](int c, auto jconst, bool fix) __attribute__((always_inline)) {
      constexpr int J = decltype(jconst)::value;
      constexpr int JA = (J + 1) % BPF;
      if constexpr (NBUF == 1) {
        lds_barrier();   // the matrix waves are done with the one set
      }
      tmload(c + 1);
      if (bact) {
        bbuild(br[JA], c + 1);
        if (fix) bfix(br[J], c + 2);
        btotals(br[J], c + 2);
        bload(br[JA], c + 3);
      }
      tmstore(c + 1);
      lds_barrier();
    };
    // chunk c + 2 is the ragged last one in iteration nchunks - 3
    const int cend = ragged && nchunks >= 3 ? nchunks - 3 : nchunks;
    run_chunks<BPF>(cend, [&](int c, auto jc) __attribute__((always_inline)) { iter(c, jc, false); });
    for (int c = cend; c < nchunks; ++c)
      with_slot<BPF>(c, [&](auto jc) __attribute__((always_inline)) { iter(c, jc, c + 2 == nchunks - 1); });
  }
}

template <typename T, int DK, int C, int NMW>
hipError_t launch_state_nmw(const ChunkArgs& a, int nchunks) {
  using S = StateCfg<T, DK, C, NMW>;
  const int BH = a.B * a.H;
  const int slices = a.dv / (16 * NMW);
  const long long wgs = (long long)BH * slices;
  const int xcd_map = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((chunk_state_kernel<T, DK, C, NMW>), dim3((unsigned)wgs), dim3(S::NTHREADS), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.alpha, (const T*)a.v, a.h0, (T*)a.o, a.hT,
                     (const unsigned char*)a.workspace, a.T, nchunks, a.dv, slices, xcd_map);
  return hipGetLastError();
}

template <typename T, int DK, int C>
hipError_t launch_state_t(const ChunkArgs& a, int nchunks) {
  // two matrix waves (32 value columns) per workgroup when dv allows
  return a.dv >= 32 ? launch_state_nmw<T, DK, C, 2>(a, nchunks) : launch_state_nmw<T, DK, C, 1>(a, nchunks);
}

template <typename T, int DK>
hipError_t state_chunk_dispatch(const ChunkArgs& a, int nch) {
  switch (a.chunk) {
    case 16: return launch_state_t<T, DK, 16>(a, nch);
    case 32: return launch_state_t<T, DK, 32>(a, nch);
    case 64: return launch_state_t<T, DK, 64>(a, nch);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t state_dk_dispatch(const ChunkArgs& a, int nch) {
  switch (a.dk) {
    case 16: return state_chunk_dispatch<T, 16>(a, nch);
    case 32: return state_chunk_dispatch<T, 32>(a, nch);
    case 64: return state_chunk_dispatch<T, 64>(a, nch);
    case 128: return state_chunk_dispatch<T, 128>(a, nch);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_gram(const ChunkArgs& a, long long total_chunks, int nchunks);

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  const int nchunks = (a.T + a.chunk - 1) / a.chunk;
  const long long BH = (long long)a.B * a.H;
  hipError_t e = launch_chunk_gram(a, BH * nchunks, nchunks);
  if (e != hipSuccess) return e;
  return a.dtype == 1 ? state_dk_dispatch<bf16_t>(a, nchunks) : state_dk_dispatch<float>(a, nchunks);
}

}  // namespace ckda
