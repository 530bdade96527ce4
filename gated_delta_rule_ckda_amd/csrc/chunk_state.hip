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
// applied element-wise in fp32; the state itself is never rounded.  With bf16
// operands the products that carry the state from chunk to chunk (W H, TB X,
// KR^T U) multiply split bf16 pairs for H, X, U and TB (hi + lo, about 16
// significant bits), so that the state keeps close to fp32 accuracy over long
// runs of undamped steps; the read-out products take the hi parts only.
//
// Every operand of a chunk but the values is state-independent and sits in
// the chunk's record (chunk_gram.hip).  Four "copy waves" move the records and
// the slice's values V (gathered into accumulator order) into a double-
// buffered operand set in LDS, staging them in registers: a chunk's loads are
// issued two (or three) chunks before it is placed, which keeps enough bytes in flight
// per CU to cover the memory latency.  So the matrix waves issue no global
// loads, only the output stores, and the copy waves only loads: with loads
// and stores in flight together, every wait for a load would also wait for
// all stores.  One workgroup barrier per chunk hands a filled set to the
// matrix waves.
#include <type_traits>

#include "chunk_common.hpp"
#include "ckda_internal.hpp"

namespace ckda {

template <typename T, int DK, int C, int NMW>
struct StateCfg : ChunkGeom<T, DK, C> {
  using G = ChunkGeom<T, DK, C>;
  static constexpr int NCW = 4;                              // copy waves
  static constexpr int NTHREADS = (NMW + NCW) * 64;
  // one operand set: the chunk's record as stored, then the slice's values in
  // accumulator order: for matrix wave w and row tile pt, lane (g, r) finds
  // rows 16 pt + 4 g .. + 3 of its column 16 w + r as four consecutive
  // elements at ((w RT + pt) 64 + lane) 4 E, one 8- or 16-byte read
  static constexpr int V_OFF = (int)G::BYTES;
  static constexpr int VRB = NMW * 16 * (int)sizeof(T);   // bytes of one value row of the slice
  static constexpr int V_BYTES = C * VRB;
  static constexpr int SET_BYTES = V_OFF + V_BYTES;
  static constexpr int NSET = 2 * SET_BYTES <= 160 * 1024 ? 2 : 1;
  static constexpr int LDS_BYTES = NSET * SET_BYTES;
  // per copy lane and chunk: record fragments and 16-byte pieces of value rows
  static constexpr int NFL = (G::NFR + NCW - 1) / NCW;
  static constexpr int NVP = C * VRB / 16;
  static constexpr int NVI = (NVP + NCW * 64 - 1) / (NCW * 64);
  // register sets: a chunk's loads are issued NR iterations before they are
  // placed in LDS (two when they fit beside the loop's other registers)
  static constexpr int NR = 3 * 4 * (NFL + NVI) <= 160 ? 3 : 2 * 4 * (NFL + NVI) <= 144 ? 2 : 1;
};

template <typename T, int DK, int C, int NMW>
__global__ __launch_bounds__((StateCfg<T, DK, C, NMW>::NTHREADS)) void chunk_state_kernel(
    const T* v, const float* __restrict__ h0, T* o, float* __restrict__ hT, const unsigned char* rec, int T_len,
    int nchunks, int dv, int slices, int xcd_map, int prod2) {
  using S = StateCfg<T, DK, C, NMW>;
  constexpr int RT = S::RT, RH = S::RH, KBN = S::KBN, KBC = S::KBC, NSET = S::NSET;
  constexpr int E = (int)sizeof(T);
  constexpr bool BF = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) unsigned char lds[S::LDS_BYTES];

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
  const long long rowbase = (long long)bh * T_len;   // first row of this (batch, head)
  auto set_of = [&](int c) __attribute__((always_inline)) { return lds + (c % NSET) * S::SET_BYTES; };

  if (matrix) {
    // ============================================================ matrix waves
    // This head's output rows as a range-checked buffer: stores to rows past
    // the end of the sequence are dropped.  With two sub-steps per token
    // (prod2 = 1) row r is sub-step r of the head and only odd rows are
    // outputs, of token r / 2; even rows are dropped the same way.
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(o + (rowbase >> prod2) * dv, (uint32_t)((size_t)(T_len >> prod2) * dv * E));
    const int col = slice * 16 * NMW + 16 * wave + r;       // this lane's value column
    const int ocol = slice * 16 * NMW + 16 * wave + 4 * g;  // first of its four output columns
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
    lds_barrier();   // the copy waves fill the first set(s)

    for (int c = 0; c < nchunks; ++c) {
      const unsigned char* set = set_of(c);
      auto frag = [&](size_t off, int f) __attribute__((always_inline)) {
        return load_frag(set + off + (f * 64 + lane) * 16);
      };
      // Operand fragments are read from LDS one group ahead of the products
      // that use them; the scheduling barriers keep each group of reads
      // together so that their latencies overlap.  (fp32 fragments are twice
      // as many: no read-ahead there, to stay within the register file.)
      constexpr int DB = BF ? 2 : 1;
      Frag wf[DB][KBN], qf[DB][KBN], tf[RT][KBC], mf[RT][KBC];
      Frag tl[BF ? RT : 1][KBC];   // TB lo parts (bf16)
      auto ld_wq = [&](int pt) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
          wf[pt % DB][kb] = frag(S::W_OFF, pt * KBN + kb);
          qf[pt % DB][kb] = frag(S::Q_OFF, pt * KBN + kb);
        }
      };
      // K blocks of TB and M entirely above the diagonal are zero: the record
      // does not hold them and they are not multiplied
      auto upper = [](int pt, int kb) constexpr { return !S::tri_live(pt, kb); };
      auto ld_tm = [&](Frag (*dst)[KBC], size_t off) __attribute__((always_inline)) {
#pragma unroll
        for (int pt = 0; pt < RT; ++pt)
#pragma unroll
          for (int kb = 0; kb < KBC; ++kb)
            if (!upper(pt, kb)) dst[pt][kb] = frag(off, S::tri_index(pt, kb));
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
          for (int kb = 0; kb < KBC; ++kb) kf[grp & 1][j][kb] = frag(S::KR_OFF, rh * KBC + kb);
        }
      };

      // this lane's value rows (X starts from V), read first with bf16 operands:
      // reads complete in order, so the products then wait only for what they
      // need (fp32 reads them per row tile, to stay within the register file)
      f32x4 xacc[RT], oacc[RT];
      auto ld_v = [&](int pt) __attribute__((always_inline)) {
        xacc[pt] = load_vals4<T>(set + S::V_OFF + ((wave * RT + pt) * 64 + lane) * 4 * E);
      };
      if constexpr (DB == 2) {
#pragma unroll
        for (int pt = 0; pt < RT; ++pt) ld_v(pt);
      }
      // The products on the state's chain from chunk to chunk (W H, TB X and
      // KR^T U) take their state-dependent B operands H, X and U, and TB, as
      // split bf16 pairs (hi + lo, ckda_device.hpp): with plain bf16 operands
      // each of these roundings alone left errors near 2e-2 after 64 chunks of
      // orthogonal steps (beta = 2, alpha = +-1), where nothing damps them.
      // W, KR and the read-out operands Q~ and M stay single bf16.
      Frag hb[KBN], hl[BF ? KBN : 1];
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) {
        if constexpr (BF) frags_from_acc_bf16_split(hacc[2 * kb], 2 * kb + 1 < RH ? hacc[2 * kb + 1] : zero4(), hb[kb], hl[kb]);
        else hb[kb] = bfrag(hacc, kb, RH);
      }
      // X = V + W H, O = Q~ H
      if constexpr (DB == 2) ld_wq(0);
#pragma unroll
      for (int pt = 0; pt < RT; ++pt) {
        if constexpr (DB == 2) {
          if (pt + 1 < RT) ld_wq(pt + 1);
          else {
            ld_tm(tf, S::T_OFF);
            if constexpr (BF) ld_tm(tl, S::TL_OFF);
          }
        } else {
          ld_wq(pt);
          ld_v(pt);
        }
        __builtin_amdgcn_sched_barrier(0);
        oacc[pt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
          xacc[pt] = mma<T>(xacc[pt], wf[pt % DB][kb], hb[kb]);
          if constexpr (BF) xacc[pt] = mma<T>(xacc[pt], wf[pt % DB][kb], hl[kb]);
          oacc[pt] = mma<T>(oacc[pt], hb[kb], qf[pt % DB][kb]);   // O^T: H^T Q~^T
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (DB == 1) ld_tm(tf, S::T_OFF);
      if constexpr (DB == 2) ld_tm(mf, S::M_OFF);
      __builtin_amdgcn_sched_barrier(0);
      // U = TB X
      Frag xb[KBC], xl[BF ? KBC : 1];
#pragma unroll
      for (int kb = 0; kb < KBC; ++kb) {
        if constexpr (BF) frags_from_acc_bf16_split(xacc[2 * kb], 2 * kb + 1 < RT ? xacc[2 * kb + 1] : zero4(), xb[kb], xl[kb]);
        else xb[kb] = bfrag(xacc, kb, RT);
      }
      f32x4 uacc[RT];
#pragma unroll
      for (int pt = 0; pt < RT; ++pt) {
        uacc[pt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb)
          if (!upper(pt, kb)) {
            uacc[pt] = mma<T>(uacc[pt], tf[pt][kb], xb[kb]);
            if constexpr (BF) {
              uacc[pt] = mma<T>(uacc[pt], tf[pt][kb], xl[kb]);
              uacc[pt] = mma<T>(uacc[pt], tl[pt][kb], xb[kb]);
            }
          }
      }
      if constexpr (DB == 1) ld_tm(mf, S::M_OFF);
      ld_kr(0);
      __builtin_amdgcn_sched_barrier(0);
      Frag ub[KBC], ul[BF ? KBC : 1];
#pragma unroll
      for (int kb = 0; kb < KBC; ++kb) {
        if constexpr (BF) frags_from_acc_bf16_split(uacc[2 * kb], 2 * kb + 1 < RT ? uacc[2 * kb + 1] : zero4(), ub[kb], ul[kb]);
        else ub[kb] = bfrag(uacc, kb, RT);
      }
      // lane (g, r) holds O^T rows 4 g .. 4 g + 3 of column r: four consecutive
      // value columns of output row 16 pt + r.  With bf16 operands the outputs
      // are stored last, when their products have long completed (fp32 stores
      // them at once, to stay within the register file).
      auto store_o = [&](int pt) __attribute__((always_inline)) {
        const int orow = c * C + 16 * pt + r;
        const int prow = prod2 ? orow >> 1 : orow;
        const bool keep = !prod2 || (orow & 1);
        store4<T>(orsrc, keep ? (prow * dv + ocol) * E : 0x7FFFFFF0, oacc[pt]);
      };
      // O += M U
#pragma unroll
      for (int pt = 0; pt < RT; ++pt) {
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb)
          if (!upper(pt, kb)) oacc[pt] = mma<T>(oacc[pt], ub[kb], mf[pt][kb]);   // + U^T M^T
        if constexpr (DB == 1) store_o(pt);
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
          for (int kb = 0; kb < KBC; ++kb) {
            hh = mma<T>(hh, kf[grp & 1][j][kb], ub[kb]);
            if constexpr (BF) hh = mma<T>(hh, kf[grp & 1][j][kb], ul[kb]);
          }
          hacc[rh] = hh;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (DB == 2) {
#pragma unroll
        for (int pt = 0; pt < RT; ++pt) store_o(pt);
      }
      lds_barrier();
      if constexpr (NSET == 1) {
        lds_barrier();   // the copy waves refill the one set
      }
    }

    if (hT) {
#pragma unroll
      for (int j = 0; j < RH; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) hT[sbase + (long long)(16 * j + 4 * g + i) * dv + col] = hacc[j][i];
    }
  } else {
    // ============================================================ copy waves
    constexpr int NFL = S::NFL, NVI = S::NVI, NR = S::NR, NCT = S::NCW * 64;
    const int cw = wave - NMW;   // copy wave 0 .. NCW-1
    const int ct = tid - NMW * 64;
    const __amdgpu_buffer_rsrc_t rrsrc =
        make_rsrc(rec + (size_t)bh * nchunks * S::BYTES, (uint32_t)((size_t)nchunks * S::BYTES));
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(v + rowbase * dv, (uint32_t)((size_t)T_len * dv * E));
    // value pieces: piece it = row it / (VRB / 16), 16 bytes at (it % (VRB / 16)) 16
    // of the slice's columns (rows past the end read as zero); its element e
    // (column 16 w + cr of the slice) goes to the accumulator-order slot of
    // lane (g, cr) = ((row % 16) / 4, cr) at position row % 4
    constexpr int PPR = S::VRB / 16, EPP = 16 / E;
    int v_goff[NVI], v_loff[NVI];
    bool v_act[NVI];
#pragma unroll
    for (int j = 0; j < NVI; ++j) {
      const int it = ct + NCT * j;
      v_act[j] = it < S::NVP;
      const int row = min(it, S::NVP - 1) / PPR, piece = it % PPR;
      const int col0 = piece * EPP, w = col0 / 16;
      v_goff[j] = (row * dv + slice * 16 * NMW) * E + piece * 16;
      v_loff[j] = S::V_OFF + ((w * S::RT + row / 16) * 64 + ((row % 16) / 4) * 16 + col0 % 16) * 4 * E + (row % 4) * E;
    }
    auto put_vals = [&](unsigned char* set, int j, const Frag& x) __attribute__((always_inline)) {
      unsigned char* p = set + v_loff[j];
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        if constexpr (E == 2) {
          *reinterpret_cast<uint16_t*>(p + e * 4 * E) = (uint16_t)(x.w[e / 2] >> (16 * (e % 2)));
        } else {
          *reinterpret_cast<uint32_t*>(p + e * 4 * E) = x.w[e];
        }
      }
    };
    struct Regs {
      Frag f[NFL];
      Frag v[NVI];
    };
    Regs rr[NR];
    // Register set d holds chunk xs: place it in its operand set, each
    // register refilled with the same piece of chunk xl (clamped to the last
    // chunk) right after its store, so that LDS writes and global loads
    // overlap.
    // The slices of one head read the same record at about the same time;
    // each starts at a different fragment so that their requests spread over
    // the L2 channels instead of queueing on one.
    const int rot = slice * S::NFR / slices;
    int fr[NFL];
#pragma unroll
    for (int j = 0; j < NFL; ++j) {
      const int q = cw + S::NCW * j;
      fr[j] = q < S::NFR ? (q + rot) % S::NFR : -1;   // -1: a spare register (load repeated, not stored)
    }
    auto swap = [&](Regs& d, int xs, int xl, bool store) __attribute__((always_inline)) {
      unsigned char* set = set_of(xs);
      const int cc = min(xl, nchunks - 1);
#pragma unroll
      for (int j = 0; j < NFL; ++j) {
        const int f = fr[j];
        // every copy wave has a real fragment in the first NFR / NCW registers
        // (stated for bf16 only: the fp32 copy loop then runs out of registers)
        if (store && ((BF && j < S::NFR / S::NCW) || f >= 0)) store_frag(set + (f * 64 + lane) * 16, d.f[j]);
        d.f[j].w = __builtin_amdgcn_raw_buffer_load_b128(rrsrc, cc * (int)S::BYTES + (max(f, 0) * 64 + lane) * 16, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < NVI; ++j) {
        if (store && (S::NVP % NCT == 0 || v_act[j])) put_vals(set, j, d.v[j]);
        d.v[j].w = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, cc * C * dv * E + v_goff[j], 0, 0);
      }
    };

    // Chunk x is loaded into register set x % NR in iteration x - NR - 1 (the
    // prologue for the first ones) and placed in LDS in iteration x - 1.
    // Prologue: chunks 0 .. NR-1 requested, chunk 0 placed, chunk NR
    // requested: the loads in flight are then those one loop pass leaves.
#pragma unroll
    for (int j = 0; j < NR; ++j) swap(rr[j], 0, j, false);
    swap(rr[0], 0, NR, true);
    lds_barrier();
    // Chunk c in use by the matrix waves: place chunk c + 1, then reuse its
    // registers for chunk c + 1 + NR.  Past the last chunk this repeats the
    // last chunk's loads into sets nobody reads.
    auto iter = [&](int c, auto jconst) __attribute__((always_inline)) {
      constexpr int J = decltype(jconst)::value;   // (c + 1) % NR
      if constexpr (NSET == 1) {
        lds_barrier();   // the matrix waves are done with the one set
      }
      swap(rr[J], c + 1, c + 1 + NR, true);
      lds_barrier();
    };
    // the register set is a compile-time index: whole groups of NR chunks per
    // loop pass, so that every pass sees the same loads in flight
    int c = 0;
    for (; c + NR <= nchunks; c += NR) {
      iter(c, std::integral_constant<int, 1 % NR>{});
      if constexpr (NR > 1) iter(c + 1, std::integral_constant<int, 2 % NR>{});
      if constexpr (NR > 2) iter(c + 2, std::integral_constant<int, 3 % NR>{});
    }
    if constexpr (NR > 1) {
      if (c < nchunks) iter(c, std::integral_constant<int, 1 % NR>{});
    }
    if constexpr (NR > 2) {
      if (c + 1 < nchunks) iter(c + 1, std::integral_constant<int, 2 % NR>{});
    }
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
                     (const T*)a.v, a.h0, (T*)a.o, a.hT, (const unsigned char*)a.workspace, a.T, nchunks, a.dv,
                     slices, xcd_map, (a.flags & kProd2) ? 1 : 0);
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
  hipError_t e;
  if (a.ev[0] && (e = hipEventRecord(a.ev[0], a.stream)) != hipSuccess) return e;
  if ((e = launch_chunk_gram(a, BH * nchunks, nchunks)) != hipSuccess) return e;
  if (a.ev[1] && (e = hipEventRecord(a.ev[1], a.stream)) != hipSuccess) return e;
  e = a.dtype == 1 ? state_dk_dispatch<bf16_t>(a, nchunks) : state_dk_dispatch<float>(a, nchunks);
  if (e != hipSuccess) return e;
  if (a.ev[2] && (e = hipEventRecord(a.ev[2], a.stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace ckda
