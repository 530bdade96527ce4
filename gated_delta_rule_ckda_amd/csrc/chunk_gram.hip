// chunk_gram.hip -- the state-independent part of the chunkwise CKDA forward:
// for every chunk of every (batch, head) at once, the decayed Gram matrices on
// the matrix cores and the unit lower-triangular (UT/WY) solve, written as the
// chunk's record (TB, M, W, Q~, KR and d, chunk_common.hpp).
//
// Chunk form (derived from the recurrence of the "Complex KDA" paper, Eq. (1);
// the pages do not print it).  For a chunk with local positions t and the
// signed segment products of the gates
//     G(t, j) = alpha_{j+1} ... alpha_t      (per channel, element-wise; 1 if t = j),
//     A[t, j] = beta_t sum_c k_tc k_jc G_c(t, j)        (j < t)
//     M[t, j] =        sum_c q_tc k_jc G_c(t, j)        (j <= t)
//     TB = (I + A)^-1 Diag(beta).
// Keeping the signs inside the products is the sign absorption of the
// discussion slides ("Absorb cumulative signs into keys and queries"): the
// parities P_t P_j of the absorbed keys are exactly the sign of G(t, j).
//
// Factorisation.  A decay G(t, j) enters a matrix-core product as x_t * y_j,
// a row factor times a column factor around a reference point s, j <= s <= t.
// With p_t the product of the gates of t's 16-row tile from its first row up
// to t, s_j the product after j up to the end of j's tile, and P_b the product
// over all of tile b, the lower triangle is covered by:
//   * tile pairs (I, J), I > J: x_t = p_t, y_j = s_j, except that x carries
//     P_2 when I = 3 and J <= 1 and y carries P_1 when J = 0 and I >= 2 --
//     reference points at the tile boundary for adjacent tiles and between
//     rows 31 and 32 for the lower-left 32 x 32 block of a 64-row chunk;
//   * rows 8-15 x 0-7 of each diagonal tile ("LL" quadrant): s at row 8;
//   * the two diagonal 8 x 8 quadrants of each tile: s at the quadrant's
//     midpoint, the far-side factor being the reciprocal of a product of at
//     most 4 gate magnitudes.
// All factors but the last kind are products of gates, of modulus at most 1.
// Gate magnitudes are floored at 2^-31 (sign kept), so the reciprocals stay
// below 2^124; a power-of-two scale of 2^16 on one side centres the quadrant
// factors in 2^-109 .. 2^109, keeping the bf16 operands (keys are unit
// vectors) clear of the subnormal range.  Entries on the wrong side of the
// diagonal, where the factors may overflow, are discarded by selection, never
// by multiplication.  The floor changes a decay only where the true value is
// below 2^-31 already.
//
// Thread layout.  Thread (tile b, pair u) owns channels 2u, 2u + 1 over the
// 16 rows of row tile b: every product along the rows is a running product
// inside the thread, and one load of a channel pair per row reads a whole row
// per wave.  The factors are multiplied into keys and queries and stored, one
// row at a time, into padded fragment buffers in LDS, from which the waves
// feed the matrix cores.  Three stages (diagonal quadrants, LL quadrants, tile
// pairs) reuse one LDS area; the tile products P_b go through LDS.
#include <type_traits>

#include "chunk_common.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

constexpr float kQuadScale = 65536.f;           // 2^16
constexpr float kQuadScaleInv = 1.f / 65536.f;

// Floor gate magnitudes at 2^-31 on raw element bits, keeping the sign
// (exponent field below that of 2^-31, zero and subnormals included, becomes
// exactly +-2^-31).  NaN and infinity pass through.
template <typename T> __device__ __forceinline__ typename Pair<T>::raw floor_gates(typename Pair<T>::raw w);
template <>
__device__ __forceinline__ uint32_t floor_gates<bf16_t>(uint32_t w) {
  const uint32_t elo = w & 0x7F80u, ehi = w & 0x7F800000u;   // 2^-31: biased exponent 96
  w = elo < 0x3000u ? ((w & 0xFFFF8000u) | 0x3000u) : w;
  w = ehi < 0x30000000u ? ((w & 0x8000FFFFu) | 0x30000000u) : w;
  return w;
}
template <>
__device__ __forceinline__ Pair<float>::raw floor_gates<float>(Pair<float>::raw w) {
  Pair<float>::raw out;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t b = __float_as_uint(w[i]);
    out[i] = __uint_as_float((b & 0x7F800000u) < 0x30000000u ? ((b & 0x80000000u) | 0x30000000u) : b);
  }
  return out;
}

template <typename T, int DK, int C>
struct GramCfg : ChunkGeom<T, DK, C> {
  using G = ChunkGeom<T, DK, C>;
  static constexpr int RT = G::RT;
  static constexpr int NU = DK / 2;               // channel pairs
  static constexpr int NTH = (NU * RT + 63) / 64 * 64;
  static constexpr int NW = NTH / 64;
  static constexpr int TOPB = G::KBN * kFragPadBytes;   // one 16-row operand tile
  // operand tiles of the tile-pair stage: key / query prefixes of tiles 1..RT-1,
  // key suffixes of tiles 0..RT-2, and for RT = 4 the rescaled tile-3 rows and
  // tile-0 columns of the 32 x 32 block
  static constexpr int NSLOT_P = 3 * (RT - 1) + (RT == 4 ? 3 : 0);
  static constexpr int NSLOT_C = 3 * RT;                // per tile: XDk, XDq, YD
  static constexpr int NSLOT_D = 2 * RT;                // per tile: LLk, LLq
  static constexpr int NSLOT = cmax(NSLOT_P, cmax(NSLOT_C, NSLOT_D));
  // row stride of the fp32 scratch: 272 bytes like a padded-fragment group,
  // so that every layout of the area leaves bytes 256..271 of each 272-byte
  // group unused (see pad_float)
  // A, M (then T in M's place) in fp32: only the 16x16 blocks on and below
  // the diagonal, each in a padded fragment slot (four 272-byte groups of four
  // 64-byte rows), which leaves bytes 256..271 of every group unused
  static constexpr int NBT = RT * (RT + 1) / 2;
  static constexpr int SCR_BYTES = 2 * NBT * kFragPadBytes;
  // phase 0: padded fragments of W, Q~ and KR, in record order
  static constexpr int NF3 = 2 * G::NF_W + G::NF_KR;
  static constexpr int KR_AREA = 2 * G::NF_W * kFragPadBytes;
  static constexpr int AREA = cmax(cmax(NSLOT * TOPB, SCR_BYTES), NF3 * kFragPadBytes);
  // The tile products [RT][DK] and beta [C] live in those unused 16-byte
  // pads: no LDS beyond the area, which lets three workgroups share a CU.
  static constexpr int TOT_F = 0;
  static constexpr int BETA_F = RT * DK;
  static constexpr int NPADF = RT * DK + C;
  static_assert(AREA % kFragGroupBytes == 0 && NPADF <= AREA / kFragGroupBytes * 4, "pad space");
  static constexpr int LDS_BYTES = AREA;
  // products (A and M of each block) per stage, and per wave
  static constexpr int NBLK = RT * (RT - 1) / 2;
  static constexpr int NPP = 2 * NBLK;
  static constexpr int NPC = 2 * RT;                    // diagonal stages alike
  static constexpr int PP = cmax((NPP + NW - 1) / NW, 1);
  static constexpr int PC = cmax((NPC + NW - 1) / NW, 1);
  // slots of the tile-pair stage
  static constexpr __device__ int pk(int b) { return b - 1; }
  static constexpr __device__ int pq(int b) { return RT - 1 + b - 1; }
  static constexpr __device__ int sk(int b) { return 2 * (RT - 1) + b; }
  static constexpr int X32K = 3 * (RT - 1), X32Q = X32K + 1, Y32 = X32K + 2;
};

// Tile pair n of the tile-pair stage: (I, J) and the operand slots of its key
// rows, query rows and columns.
template <typename P>
__device__ __forceinline__ void tile_pair(int n, int& I, int& J, int& xk, int& xq, int& ys) {
  if (n < P::RT - 1) {            // adjacent tiles, reference at their boundary
    J = n;
    I = n + 1;
    xk = P::pk(I);
    xq = P::pq(I);
    ys = P::sk(J);
  } else {                        // the 32 x 32 block of a 64-row chunk: (2,0), (3,1), (3,0)
    const int m = n - (P::RT - 1);
    I = m == 0 ? 2 : 3;
    J = m == 1 ? 1 : 0;
    xk = I == 2 ? P::pk(2) : P::X32K;
    xq = I == 2 ? P::pq(2) : P::X32Q;
    ys = J == 1 ? P::sk(1) : P::Y32;
  }
}

// PRO: the per-token prologue of ckda.h (flags CKDA_FUSE_*) runs on the loads:
// gates from their logits, beta from its logit, unit-norm keys and queries.
// The gates are then kept in fp32 (a rounded computed gate would compound
// over the chunk's products).  The same instantiation gathers each head's
// retained key channels when gidx is set (q, k, alpha rows of dk_in channels;
// gidx [nheads][DK] channel indices).
// Waves per SIMD the compiler is asked to leave room for: three for bf16 at
// dk 64, chunk 64 (two-wave workgroups, 26 KB of LDS: the registers, at 190,
// would otherwise hold them to two), one (no bound) elsewhere.
template <typename T, int DK, int C>
constexpr int kGramMinWaves = (std::is_same<T, bf16_t>::value && DK == 64 && C == 64) ? 3 : 1;

template <typename T, int DK, int C, bool PRO>
__global__ __launch_bounds__((GramCfg<T, DK, C>::NTH), (kGramMinWaves<T, DK, C>)) void chunk_gram_kernel(
    const T* q, const T* k, const T* alpha, const T* beta, unsigned char* __restrict__ ws, int T_len,
    int nchunks, int flags, const int* __restrict__ gidx, int dk_in, int nheads) {
  using P = GramCfg<T, DK, C>;
  using PR = Pair<T>;
  typedef typename PR::raw raw;
  using GR = Pair<typename std::conditional<PRO, float, T>::type>;   // storage of the gates
  typedef typename GR::raw graw;
  constexpr int NU = P::NU, NW = P::NW, NTH = P::NTH, RT = P::RT, KBN = P::KBN, KBC = P::KBC,
                TOPB = P::TOPB, EPL = P::EPL, KB = P::KB;
  __shared__ __attribute__((aligned(16))) unsigned char lds[P::LDS_BYTES];
  unsigned char* area = lds;
  // float i of the pad space: 4 floats in the last 16 bytes of each 272-byte group
  auto pad_float = [&](int i) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(area + (i >> 2) * kFragGroupBytes + 256 + (i & 3) * 4);
  };
  auto s_tot = [&](int i) __attribute__((always_inline)) { return pad_float(P::TOT_F + i); };
  auto s_beta = [&](int i) __attribute__((always_inline)) { return pad_float(P::BETA_F + i); };

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  // Workgroups run chunk-major from the last chunk back: the records the
  // state pass reads first are written last (most likely still cached), and
  // when the number of (batch, head) pairs is a multiple of 8 a head's chunks
  // run on the XCD its state pass will use (ids equal modulo 8).
  const long long nbh = gridDim.x / nchunks;
  const long long bh = blockIdx.x % nbh;
  const int c = nchunks - 1 - (int)(blockIdx.x / nbh);
  const long long chunk_id = bh * nchunks + c;
  const int t0 = c * C;
  const int cv = min(C, T_len - t0);
  const long long row0 = bh * (long long)T_len + t0;

  if (tid < C) {
    float bt = tid < cv ? to_f32(beta[row0 + tid]) : 0.f;
    if (PRO && (flags & kFuseGates) && tid < cv) bt = practical_beta(bt);
    *s_beta(tid) = bt;
  }

  const int b = tid / NU, u = tid % NU;
  const bool act = b < RT;
  const int c0 = 2 * u;
  const int colofs = padded_col_offset<T>(c0);

  // ---- this thread's rows: signed gates (floored), keys, queries
  raw rl[16], rk[16], rq[16];   // gates (or, with the prologue, their logits) as loaded
  // lda / ldk / ldq (i): this thread's channel pair of row 16 b + i
  auto load_rows = [&](auto lda, auto ldk, auto ldq) __attribute__((always_inline)) {
    if (cv == C) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        rl[i] = lda(i);
        rk[i] = ldk(i);
        rq[i] = ldq(i);
      }
    } else {
      // ragged last chunk: rows past the end act as identity steps (gate 1, no key)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 16 * b + i;
        const int ii = min(t, cv - 1) - 16 * b;
        const raw a = lda(ii), kk = ldk(ii), qq = ldq(ii);
        rl[i] = PR::ones();
        rk[i] = PR::zeros();
        rq[i] = PR::zeros();
        if (t < cv) {
          rl[i] = a;
          rk[i] = kk;
          rq[i] = qq;
        }
      }
    }
  };
  const long long grow = row0 + 16 * b;   // global row of this thread's first row
  auto pairs = [&](const T* x) __attribute__((always_inline)) {
    const size_t base = (size_t)grow * DK + c0;
    return [=](int i) __attribute__((always_inline)) { return PR::load(x + base + (size_t)i * DK); };
  };
  if (act) {
    if constexpr (PRO) {
      // one uniform branch per load mode, outside the row loops
      if (gidx) {
        // channel gather: rows of dk_in channels, this head's retained index
        // set picks channels 2u and 2u + 1 (indices clamped into the row)
        const int* hidx = gidx + (bh % nheads) * DK;
        const int g0 = min(max(hidx[c0], 0), dk_in - 1), g1 = min(max(hidx[c0 + 1], 0), dk_in - 1);
        const size_t rb = (size_t)grow * dk_in;
        auto gat = [&](const T* x) __attribute__((always_inline)) {
          return [=](int i) __attribute__((always_inline)) {
            const T* r = x + rb + (size_t)i * dk_in;
            return PR::pack(r[g0], r[g1]);
          };
        };
        load_rows(gat(alpha), gat(k), gat(q));
      } else if (flags & kProd2) {
        // two sub-steps per token: rows 2 tau and 2 tau + 1 share query tau;
        // the token's scalar gate (if any) acts on its first sub-step
        const size_t qbase = (size_t)(grow >> 1) * DK + c0;
        auto ldq = [=](int i) __attribute__((always_inline)) {
          return PR::load(q + qbase + (size_t)(((grow & 1) + i) >> 1) * DK);
        };
        if (flags & kScalarGate) {
          auto lda = [=](int i) __attribute__((always_inline)) {
            const T g = alpha[(grow + i) >> 1];
            return ((grow + i) & 1) ? PR::ones() : PR::pack(g, g);
          };
          load_rows(lda, pairs(k), ldq);
        } else {
          load_rows([](int) { return PR::ones(); }, pairs(k), ldq);
        }
      } else if (flags & kScalarGate) {
        // one gate per token and head, the same on every channel
        auto lda = [=](int i) __attribute__((always_inline)) {
          const T g = alpha[grow + i];
          return PR::pack(g, g);
        };
        load_rows(lda, pairs(k), pairs(q));
      } else {
        load_rows(pairs(alpha), pairs(k), pairs(q));
      }
    } else {
      load_rows(pairs(alpha), pairs(k), pairs(q));
    }
  }
  // Prologue gates: transformed after all loads are in flight, under one
  // branch (a branch per row would split the loads into separate blocks,
  // each waiting for its own).  Ragged rows stay identity steps.
  graw ra[16];
  if constexpr (PRO) {
#pragma unroll
    for (int i = 0; i < 16; ++i) ra[i] = graw{PR::lo(rl[i]), PR::hi(rl[i])};
    if (flags & kFuseGates) {
      // rows that are identity steps keep gate 1: past a ragged end, and with
      // two sub-steps per token the second one (or both, ungated)
      const bool ones2 = (flags & kProd2) && !(flags & kScalarGate);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool keep = 16 * b + i >= cv || ((flags & kProd2) && (ones2 || ((grow + i) & 1)));
        ra[i] = graw{keep ? 1.f : practical_gate(ra[i][0]), keep ? 1.f : practical_gate(ra[i][1])};
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) ra[i] = rl[i];
  }

  // keys and queries widened to fp32 once: every operand below multiplies
  // them (the gates stay packed: widened as well they would cost the third
  // workgroup per CU its registers)
  // (In the bf16 prologue instantiation the queries stay packed and are
  // widened at each use, behind an opaque copy so that the widened values
  // are not kept: the fp32 gates take those registers, which keeps the third
  // workgroup per CU.)
  constexpr bool QPACK = PRO && std::is_same<T, bf16_t>::value;
  float kl[16], kh[16], ql[16], qh[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    kl[i] = PR::lo(rk[i]);
    kh[i] = PR::hi(rk[i]);
    if constexpr (!QPACK) {
      ql[i] = PR::lo(rq[i]);
      qh[i] = PR::hi(rq[i]);
    }
  }
  auto qraw = [&](int i) __attribute__((always_inline)) {
    raw t = rq[i];
    if constexpr (QPACK) pin(t);
    return t;
  };
#define QL(i) (QPACK ? PR::lo(qraw(i)) : ql[i])
#define QH(i) (QPACK ? PR::hi(qraw(i)) : qh[i])
  if constexpr (PRO) {
    // unit rows: the NU lanes holding one row (an aligned lane group) sum
    // their squares; v_rsq_f32 gives the inverse norm
    auto unit_rows = [&](float* lo, float* hi) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float ss = group_sum<NU>(__builtin_fmaf(lo[i], lo[i], hi[i] * hi[i]));
        const float inv = __builtin_amdgcn_rsqf(ss + kUnitGuard);
        lo[i] *= inv;
        hi[i] *= inv;
      }
    };
    if (flags & kFuseNormK) unit_rows(kl, kh);
    if (flags & kFuseNormQ) {
      if constexpr (QPACK) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float l = PR::lo(rq[i]), h = PR::hi(rq[i]);
          const float inv = __builtin_amdgcn_rsqf(group_sum<NU>(__builtin_fmaf(l, l, h * h)) + kUnitGuard);
          rq[i] = pack_bf16x2(l * inv, h * inv);
        }
      } else {
        unit_rows(ql, qh);
      }
    }
  }

  // K blocks only partly covered (bf16: channels when DK = 16, positions of
  // KR when C = 16): the uncovered half of every fragment must read as zero
  // (the pads, 16-byte unit 16 of every 17, hold beta and the tile products)
  auto zero_area = [&]() {
    for (int i = tid; i < P::AREA / 16; i += NTH)
      if (i % 17 != 16) reinterpret_cast<u32x4*>(area)[i] = u32x4{0u, 0u, 0u, 0u};
  };
  if constexpr (DK % KB != 0 || C % KB != 0) {
    zero_area();
    lds_barrier();
  }

  // store the value pair of tile row i into operand tile `slot`
  auto put = [&](int slot, int i, float v0, float v1) {
    PR::put(area + slot * TOPB + colofs + i * 16, v0, v1);
  };
#define LO(x) GR::lo(x)
#define HI(x) GR::hi(x)

  // ---- phase 0: the gate-product operands of the state pass.  Only products
  // of gates occur (modulus at most 1), so the gates are used as given.
  //   W = -(K . gamma), Q~ = Q . gamma, KR = (K . G(C, .))^T, d = gamma_{C-1},
  // gamma_t being the product from the chunk start to t and G(C, t) the
  // product after t to the chunk end; rows past a ragged end have gate 1 and
  // zero key and query.
  // (records are written with streaming stores: nothing reads them before
  // the state pass, and keeping them out of the caches speeds this kernel up)
  unsigned char* rec = ws + (size_t)chunk_id * P::BYTES;
  {
    if (act) {
      float p0 = 1.f, p1 = 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p0 *= LO(ra[i]);
        p1 *= HI(ra[i]);
      }
      *reinterpret_cast<float2*>(s_tot(b * DK + c0)) = make_float2(p0, p1);
    }
    lds_barrier();
    if (act) {
      float bf0 = 1.f, bf1 = 1.f, af0 = 1.f, af1 = 1.f;   // tiles before / after this one
#pragma unroll
      for (int J = 0; J < RT; ++J) {
        const float2 tt = *reinterpret_cast<const float2*>(s_tot(J * DK + c0));
        if (J < b) {
          bf0 *= tt.x;
          bf1 *= tt.y;
        }
        if (J > b) {
          af0 *= tt.x;
          af1 *= tt.y;
        }
      }
      float g0 = bf0, g1 = bf1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        g0 *= LO(ra[i]);
        g1 *= HI(ra[i]);
        put(b, i, -kl[i] * g0, -kh[i] * g1);
        put(RT + b, i, QL(i) * g0, QH(i) * g1);
      }
      if (b == RT - 1) *reinterpret_cast<float2*>(rec + P::D_OFF + c0 * 4) = make_float2(g0, g1);
      // KR^T: rows = channels c0, c0 + 1; K = positions, four at a time
      float e0 = af0, e1 = af1;
#pragma unroll
      for (int m = 3; m >= 0; --m) {
        float kr0[4], kr1[4];
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          kr0[i] = kl[4 * m + i] * e0;
          kr1[i] = kh[4 * m + i] * e1;
          e0 *= LO(ra[4 * m + i]);
          e1 *= HI(ra[4 * m + i]);
        }
        unsigned char* base = area + P::KR_AREA + padded_col_offset<T>(16 * b + 4 * m);
        Quad<T>::put(base + (c0 >> 4) * KBC * kFragPadBytes + (c0 & 15) * 16, kr0);
        Quad<T>::put(base + ((c0 + 1) >> 4) * KBC * kFragPadBytes + ((c0 + 1) & 15) * 16, kr1);
      }
    }
    lds_barrier();
    // padded fragments [W][Q~][KR] -> the record, unpadded, same order
    {
      // unrolled, so that all of a wave's LDS reads are in flight together
      constexpr int NPW = (P::NF3 + NW - 1) / NW;
      Frag fr[NPW];
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        const int f = wave + NW * j;
        if (f < P::NF3) fr[j] = load_frag(area + padded_slot(f, lane));
      }
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        const int f = wave + NW * j;
        if (f < P::NF3) store_frag_stream(rec + P::W_OFF + (size_t)f * 1024 + lane * 16, fr[j]);
      }
    }
    lds_barrier();
    if constexpr (DK % KB != 0) {
      zero_area();
      lds_barrier();
    }
  }

  // Gate magnitudes floored for the Gram stages (see the file comment)
  if (act) {
#pragma unroll
    for (int i = 0; i < 16; ++i) ra[i] = floor_gates<typename std::conditional<PRO, float, T>::type>(ra[i]);
  }
  // acc += X[xs] Y[ys]^T over all channels
  auto gram = [&](f32x4 acc, int xs, int ys) {
#pragma unroll
    for (int kb = 0; kb < KBN; ++kb)
      acc = mma<T>(acc, load_frag(area + xs * TOPB + padded_slot(kb, lane)),
                   load_frag(area + ys * TOPB + padded_slot(kb, lane)));
    return acc;
  };

  // ---- stage 1: the diagonal 8 x 8 quadrants, reference at their midpoints;
  // tile products to LDS
  f32x4 accC[P::PC];
  {
    if (act) {
#pragma unroll
      for (int q0 = 0; q0 < 16; q0 += 8) {
        float p0 = kQuadScale, p1 = kQuadScale;
#pragma unroll
        for (int i = q0 + 4; i < q0 + 8; ++i) {   // am = scale x prefix from the midpoint, bm = 1 / am
          p0 *= LO(ra[i]);
          p1 *= HI(ra[i]);
          const float b0 = __builtin_amdgcn_rcpf(p0), b1 = __builtin_amdgcn_rcpf(p1);
          put(3 * b, i, kl[i] * p0, kh[i] * p1);
          put(3 * b + 1, i, QL(i) * p0, QH(i) * p1);
          put(3 * b + 2, i, kl[i] * b0, kh[i] * b1);
        }
        float s0 = kQuadScaleInv, s1 = kQuadScaleInv;
#pragma unroll
        for (int i = q0 + 3; i >= q0; --i) {      // bm = suffix up to the midpoint / scale, am = 1 / bm
          const float a0 = __builtin_amdgcn_rcpf(s0), a1 = __builtin_amdgcn_rcpf(s1);
          put(3 * b, i, kl[i] * a0, kh[i] * a1);
          put(3 * b + 1, i, QL(i) * a0, QH(i) * a1);
          put(3 * b + 2, i, kl[i] * s0, kh[i] * s1);
          s0 *= LO(ra[i]);
          s1 *= HI(ra[i]);
        }
      }
      if constexpr (RT == 4) {
        float p0 = 1.f, p1 = 1.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p0 *= LO(ra[i]);
          p1 *= HI(ra[i]);
        }
        *reinterpret_cast<float2*>(s_tot(b * DK + c0)) = make_float2(p0, p1);
      }
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < P::PC; ++j) {
      const int p = wave + NW * j;
      accC[j] = zero4();
      if (p < P::NPC) accC[j] = gram(accC[j], 3 * (p >> 1) + (p & 1), 3 * (p >> 1) + 2);
    }
    lds_barrier();
  }

  // ---- stage 2: rows 8-15 x 0-7 of each tile, reference at row 8.  LLk holds
  // the column operand in rows 0-7 and the key row operand in rows 8-15, so
  // LLk LLk^T and LLq LLk^T carry the block in their lower-left quadrant.
  f32x4 accD[P::PC];
  {
    if (act) {
      float x0 = 1.f, x1 = 1.f;
#pragma unroll
      for (int i = 8; i < 16; ++i) {
        x0 *= LO(ra[i]);
        x1 *= HI(ra[i]);
        put(2 * b, i, kl[i] * x0, kh[i] * x1);
        put(2 * b + 1, i, QL(i) * x0, QH(i) * x1);
      }
      float y0 = 1.f, y1 = 1.f;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        put(2 * b, i, kl[i] * y0, kh[i] * y1);
        y0 *= LO(ra[i]);
        y1 *= HI(ra[i]);
      }
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < P::PC; ++j) {
      const int p = wave + NW * j;
      accD[j] = zero4();
      if (p < P::NPC) accD[j] = gram(accD[j], 2 * (p >> 1) + (p & 1), 2 * (p >> 1));
    }
    lds_barrier();
  }

  // ---- stage 3: tile pairs below the diagonal
  f32x4 accP[P::PP];
  if constexpr (P::NPP > 0) {
    if (act) {
      // products over the tiles between: P_2 for tile-3 rows, P_1 for tile-0 columns
      float m0 = 1.f, m1 = 1.f;
      if (RT == 4 && (b == 3 || b == 0)) {
        const float2 tt = *reinterpret_cast<const float2*>(s_tot((b == 3 ? 2 : 1) * DK + c0));
        m0 = tt.x;
        m1 = tt.y;
      }
      if (b >= 1) {                // row operands: prefix inside the tile
        float x0 = 1.f, x1 = 1.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          x0 *= LO(ra[i]);
          x1 *= HI(ra[i]);
          put(P::pk(b), i, kl[i] * x0, kh[i] * x1);
          put(P::pq(b), i, QL(i) * x0, QH(i) * x1);
          if (RT == 4 && b == 3) {
            const float z0 = x0 * m0, z1 = x1 * m1;
            put(P::X32K, i, kl[i] * z0, kh[i] * z1);
            put(P::X32Q, i, QL(i) * z0, QH(i) * z1);
          }
        }
      }
      if (b <= RT - 2) {           // column operands: suffix inside the tile
        float y0 = 1.f, y1 = 1.f;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
          put(P::sk(b), i, kl[i] * y0, kh[i] * y1);
          if (RT == 4 && b == 0) put(P::Y32, i, kl[i] * (y0 * m0), kh[i] * (y1 * m1));
          y0 *= LO(ra[i]);
          y1 *= HI(ra[i]);
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < P::PP; ++j) {
      const int p = wave + NW * j;
      accP[j] = zero4();
      if (p < P::NPP) {
        int I, J, xk, xq, ys;
        tile_pair<P>(p >> 1, I, J, xk, xq, ys);
        accP[j] = gram(accP[j], (p & 1) ? xq : xk, ys);
      }
    }
    lds_barrier();
  }
#undef LO
#undef HI
#undef QL
#undef QH

  // ---- A (rows scaled by beta, strictly lower) and M (lower incl.) to LDS,
  // fp32, blocks on and below the diagonal only (GramCfg::SCR_BYTES); M goes
  // to the record before the solve, which then keeps T in M's blocks
  constexpr int NBT = P::NBT, MA = 0, MM = 1, MT = 1;
  auto sc = [&](int m, int row, int col) __attribute__((always_inline)) {
    const int I = row >> 4, J = col >> 4;
    return reinterpret_cast<float*>(area + (m * NBT + I * (I + 1) / 2 + J) * kFragPadBytes +
                                    ((row & 15) >> 2) * kFragGroupBytes + (row & 3) * 64 + (col & 15) * 4);
  };
  auto put_tile = [&](int I, int J, int kind, f32x4 acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * I + 4 * g + i, col = 16 * J + r;
      if (kind == 0) *sc(MA, row, col) = acc[i] * *s_beta(row);
      else *sc(MM, row, col) = acc[i];
    }
  };
  if constexpr (P::NPP > 0) {
#pragma unroll
    for (int j = 0; j < P::PP; ++j) {
      const int p = wave + NW * j;
      if (p < P::NPP) {
        int I, J, xk, xq, ys;
        tile_pair<P>(p >> 1, I, J, xk, xq, ys);
        put_tile(I, J, p & 1, accP[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < P::PC; ++j) {
    const int p = wave + NW * j;
    if (p < P::NPC) {
      const int tt = p >> 1, kind = p & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = 4 * g + i, row = 16 * tt + lr, col = 16 * tt + r;
        const bool diagq = (lr >> 3) == (r >> 3);
        const bool ll = lr >= 8 && r < 8;
        if (kind == 0) {
          const float a = diagq ? (r < lr ? accC[j][i] : 0.f) : (ll ? accD[j][i] : 0.f);
          *sc(MA, row, col) = a * *s_beta(row);
        } else {
          *sc(MM, row, col) = diagq ? (r <= lr ? accC[j][i] : 0.f) : (ll ? accD[j][i] : 0.f);
        }
      }
    }
  }
  lds_barrier();

  // ---- record fragments of a C x C lower-triangular matrix (set 0: T Diag(beta),
  // 1: M, 2: the lo part of T Diag(beta), bf16 only); blocks above the diagonal
  // are all zero and not stored
  constexpr int NF = RT * KBC;
  auto emit = [&](int set, int ff) __attribute__((always_inline)) {
    const bool isT = set != 1;
    const int rt = ff / KBC, kb = ff % KBC;
    if (!P::tri_live(rt, kb)) return;
    float vals[8];
    // K order: elements 0-3 are 4 consecutive columns, so are 4-7 (bf16)
#pragma unroll
    for (int hh = 0; hh < EPL / 4; ++hh) {
      const int col = kb * KB + kappa<T>(g, 4 * hh);
      f32x4 x = zero4();
      if (col < C && col / 16 <= rt) {
        x = *reinterpret_cast<const f32x4*>(sc(isT ? MT : MM, 16 * rt + r, col));
        if (isT) x *= *reinterpret_cast<const f32x4*>(s_beta(col));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) vals[4 * hh + e] = x[e];
    }
    Frag out;
    if constexpr (sizeof(T) == 2) {
      out.w = u32x4{pack_bf16x2(vals[0], vals[1]), pack_bf16x2(vals[2], vals[3]), pack_bf16x2(vals[4], vals[5]),
                    pack_bf16x2(vals[6], vals[7])};
      if (set == 2) out = frag_residual_bf16(vals, out);   // TB - bf16(TB), rounded
    } else {
      out.w = __builtin_bit_cast(u32x4, f32x4{vals[0], vals[1], vals[2], vals[3]});
    }
    const size_t off = set == 0 ? P::T_OFF : set == 1 ? P::M_OFF : P::TL_OFF;
    store_frag_stream(rec + off + ((size_t)P::tri_index(rt, kb) * 64 + lane) * 16, out);
  };
  // M first: T takes its blocks
#pragma unroll
  for (int j = 0; j < (NF + NW - 1) / NW; ++j) {
    const int f = wave + NW * j;
    if (f < NF) emit(1, f);
  }
  lds_barrier();

  // ---- T = (I + A)^-1: diagonal 16x16 blocks by forward substitution
  if (tid < 16 * RT) {
    const int blk = tid >> 4, jc = tid & 15, o = 16 * blk;
    float tcol[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jc) ? 1.f : 0.f;
#pragma unroll
      for (int k4 = 0; k4 < i; k4 += 4) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(sc(MA, o + i, o + k4));
#pragma unroll
        for (int uu = 0; uu < 4; ++uu)
          if (k4 + uu < i) s -= av[uu] * tcol[k4 + uu];
      }
      tcol[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) *sc(MT, o + i, o + jc) = tcol[i];
  }
  lds_barrier();

  // ---- off-diagonal blocks by distance on fp32 matrix cores:
  //      T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
  for (int d = 1; d < RT; ++d) {
    for (int J = wave; J + d < RT; J += NW) {
      const int I = J + d;
      f32x4 s = zero4();
      for (int K = J; K < I; ++K) {
        Frag fa, fb;
        fa.w = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4*>(sc(MA, 16 * I + r, 16 * K + 4 * g)));
        fb.w = __builtin_bit_cast(u32x4, f32x4{*sc(MT, 16 * K + 4 * g + 0, 16 * J + r), *sc(MT, 16 * K + 4 * g + 1, 16 * J + r),
                                               *sc(MT, 16 * K + 4 * g + 2, 16 * J + r), *sc(MT, 16 * K + 4 * g + 3, 16 * J + r)});
        s = mma<float>(s, fa, fb);
      }
      Frag fa;
      fa.w = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4*>(sc(MT, 16 * I + r, 16 * I + 4 * g)));
      const f32x4 tij = mma<float>(zero4(), fa, frag_from_acc_f32(s));
#pragma unroll
      for (int i = 0; i < 4; ++i) *sc(MT, 16 * I + 4 * g + i, 16 * J + r) = -tij[i];
    }
    lds_barrier();
  }

  // ---- record: T Diag(beta) (bf16: as hi and lo parts)
  constexpr int NTS = P::SPLIT ? 2 : 1;
#pragma unroll
  for (int j = 0; j < (NTS * NF + NW - 1) / NW; ++j) {
    const int f = wave + NW * j;
    if (f < NTS * NF) emit(f < NF ? 0 : 2, f < NF ? f : f - NF);
  }
}

template <typename T, int DK, int C>
hipError_t launch_gram_t(const ChunkArgs& a, long long total_chunks, int nchunks) {
  using P = GramCfg<T, DK, C>;
  if (a.flags != 0 || a.gidx)
    hipLaunchKernelGGL((chunk_gram_kernel<T, DK, C, true>), dim3((unsigned)total_chunks), dim3(P::NTH), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.alpha, (const T*)a.beta,
                       (unsigned char*)a.workspace, a.T, nchunks, a.flags, a.gidx, a.gidx ? a.dk_in : DK, a.H);
  else
    hipLaunchKernelGGL((chunk_gram_kernel<T, DK, C, false>), dim3((unsigned)total_chunks), dim3(P::NTH), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.alpha, (const T*)a.beta,
                       (unsigned char*)a.workspace, a.T, nchunks, 0, nullptr, DK, 1);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t gram_chunk_dispatch(const ChunkArgs& a, long long total, int nch) {
  switch (a.chunk) {
    case 16: return launch_gram_t<T, DK, 16>(a, total, nch);
    case 32: return launch_gram_t<T, DK, 32>(a, total, nch);
    case 64: return launch_gram_t<T, DK, 64>(a, total, nch);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t gram_dk_dispatch(const ChunkArgs& a, long long total, int nch) {
  switch (a.dk) {
    case 16: return gram_chunk_dispatch<T, 16>(a, total, nch);
    case 32: return gram_chunk_dispatch<T, 32>(a, total, nch);
    case 64: return gram_chunk_dispatch<T, 64>(a, total, nch);
    case 128: return gram_chunk_dispatch<T, 128>(a, total, nch);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_gram(const ChunkArgs& a, long long total_chunks, int nchunks) {
  if (total_chunks == 0) return hipSuccess;
  return a.dtype == 1 ? gram_dk_dispatch<bf16_t>(a, total_chunks, nchunks)
                      : gram_dk_dispatch<float>(a, total_chunks, nchunks);
}

template <typename T, int DK>
static ChunkRecord record_c(int chunk) {
  switch (chunk) {
    case 16: return {ChunkGeom<T, DK, 16>::T_OFF, ChunkGeom<T, DK, 16>::M_OFF, ChunkGeom<T, DK, 16>::BYTES};
    case 32: return {ChunkGeom<T, DK, 32>::T_OFF, ChunkGeom<T, DK, 32>::M_OFF, ChunkGeom<T, DK, 32>::BYTES};
    case 64: return {ChunkGeom<T, DK, 64>::T_OFF, ChunkGeom<T, DK, 64>::M_OFF, ChunkGeom<T, DK, 64>::BYTES};
  }
  return {0, 0, 0};
}

template <typename T>
static ChunkRecord record_t(int dk, int chunk) {
  switch (dk) {
    case 16: return record_c<T, 16>(chunk);
    case 32: return record_c<T, 32>(chunk);
    case 64: return record_c<T, 64>(chunk);
    case 128: return record_c<T, 128>(chunk);
  }
  return {0, 0, 0};
}

ChunkRecord chunk_record_layout(int dk, int chunk, int dtype) {
  return dtype == 1 ? record_t<bf16_t>(dk, chunk) : record_t<float>(dk, chunk);
}

}  // namespace ckda
