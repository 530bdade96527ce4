// prologue.hpp -- the state-independent part of one chunk of the chunkwise
// CKDA forward, computed by four waves of a workgroup: signed cumulative gate
// products, the decayed Gram matrices, the unit lower-triangular (UT/WY)
// solve, and the operand record the state pass consumes (chunk_common.hpp).
//
// Chunk form (derived from the recurrence of the "Complex KDA" paper, Eq. (1);
// the pages do not print it).  For a chunk with incoming state H0 and local
// positions t = 1..C, with the signed segment products
//     G(t, j) = alpha_{j+1} ... alpha_t      (per channel, element-wise; 1 if t = j)
// and gamma_t = G(t, 0):
//     A[t, j] = beta_t sum_c k_tc k_jc G_c(t, j)        (j < t)
//     M[t, j] =        sum_c q_tc k_jc G_c(t, j)        (j <= t)
//     T = (I + A)^-1,  U = T Diag(beta) (V - (K . gamma) H0),
//     O = (Q . gamma) H0 + M U,   H_C = Diag(gamma_C) H0 + (K . G(C, .))^T U.
// Keeping the signs inside the products is the sign absorption of the
// discussion slides ("Absorb cumulative signs into keys and queries"): the
// parities P_t P_j of the absorbed keys are exactly the sign of G(t, j).
//
// Layout.  Wave I owns rows 16 I .. 16 I + 15 of the chunk; lane (g, r) owns
// row r and, in every K block of the channels, the channels kappa(g, e) --
// i.e. each lane holds exactly its slot of the matrix-core fragments of its
// row tile, so the Gram operands are built in registers.  Products along the
// rows (prefix / suffix products inside 4-, 8- and 16-row segments) use DPP
// lane permutations inside each 16-lane row; the products over whole tiles
// are exchanged through LDS.
//
// Overflow.  A decay factor G(t, j) is applied as a product x_t * y_j of a
// row factor and a column factor around a reference point between j and t:
//   * tiles below the diagonal: split at tile boundaries -- a prefix inside
//     t's tile, whole tiles in between, a suffix inside j's tile (all <= 1);
//   * the lower-left 8x8 quadrant of a diagonal tile: split at the quadrant
//     boundary (prefix / suffix inside 8-row halves, <= 1);
//   * the two diagonal 8x8 quadrants: split at their midpoint; the factor on
//     the far side is the reciprocal of a product of at most 4 magnitudes.
// Magnitudes are floored at 2^-31 (sign kept; a zero gate counts as +), so
// that reciprocal is at most 2^124 and finite in fp32 and bf16.  Entries
// above the diagonal, where such factors may overflow, are discarded by
// selection, never by multiplication.
#pragma once

#include "chunk_common.hpp"

namespace ckda {

constexpr float kGateFloor = 4.656612873077393e-10f;  // 2^-31

// ---- DPP helpers (16-lane rows of a wave64)
enum : int {
  kDppQuad0012 = 0 | (0 << 2) | (1 << 4) | (2 << 6),
  kDppQuad0001 = 0 | (0 << 2) | (0 << 4) | (1 << 6),
  kDppQuad1233 = 1 | (2 << 2) | (3 << 4) | (3 << 6),
  kDppQuad2333 = 2 | (3 << 2) | (3 << 4) | (3 << 6),
  kDppQuad3333 = 3 | (3 << 2) | (3 << 4) | (3 << 6),
  kDppRowMirror = 0x140,
  kDppRowHalfMirror = 0x141,
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Segment products of the signed gates a along the 16 rows of a lane row
// (r = row inside the tile, 0..15).
struct RowScan {
  float p4, s4, p8, s8, p16, s16, tot;  // inclusive prefix / exclusive suffix in 4-, 8-, 16-row segments
};

__device__ __forceinline__ RowScan row_scan(float a, int r) {
  const int q = r & 3;
  RowScan s;
  // inclusive prefix inside the aligned 4-row quarter
  float p = a;
  {
    const float x1 = dpp<kDppQuad0012>(p);
    p = q >= 1 ? p * x1 : p;
    const float x2 = dpp<kDppQuad0001>(p);
    p = q >= 2 ? p * x2 : p;
  }
  // exclusive suffix inside the quarter
  float b = dpp<kDppQuad1233>(a);
  b = q == 3 ? 1.f : b;
  {
    const float y1 = dpp<kDppQuad1233>(b);
    b = q <= 2 ? b * y1 : b;
    const float y2 = dpp<kDppQuad2333>(b);
    b = q <= 1 ? b * y2 : b;
  }
  // quarter totals: own, and the other quarter of the same 8-row half
  const float qt = dpp<kDppQuad3333>(p);
  const float oqt = dpp<kDppRowHalfMirror>(qt);
  const bool upper4 = (r & 4) != 0;
  s.p4 = p;
  s.s4 = b;
  s.p8 = upper4 ? p * oqt : p;
  s.s8 = upper4 ? b : b * oqt;
  // half totals: own (qt * oqt, in a fixed order), and the other half's
  const float ht = upper4 ? oqt * qt : qt * oqt;
  const float oht = dpp<kDppRowMirror>(ht);
  const bool upper8 = r >= 8;
  s.p16 = upper8 ? s.p8 * oht : s.p8;
  s.s16 = upper8 ? s.s8 : s.s8 * oht;
  s.tot = upper8 ? oht * ht : ht * oht;   // lower half first: identical bits in every lane
  return s;
}

// Tile product only (the first pass needs nothing else).
__device__ __forceinline__ float row_total(float a, int r) {
  const int q = r & 3;
  float p = a;
  const float x1 = dpp<kDppQuad0012>(p);
  p = q >= 1 ? p * x1 : p;
  const float x2 = dpp<kDppQuad0001>(p);
  p = q >= 2 ? p * x2 : p;
  const float qt = dpp<kDppQuad3333>(p);
  const float oqt = dpp<kDppRowHalfMirror>(qt);
  const bool upper4 = (r & 4) != 0;
  const float ht = upper4 ? oqt * qt : qt * oqt;
  const float oht = dpp<kDppRowMirror>(ht);
  return r >= 8 ? oht * ht : ht * oht;
}

__device__ __forceinline__ float floor_gate(float a) {
  return fabsf(a) < kGateFloor ? kGateFloor : a;  // keeps the sign; NaN passes through
}

template <typename T, int DK, int C>
struct ProCfg : ChunkGeom<T, DK, C> {
  using G = ChunkGeom<T, DK, C>;
  static constexpr int NSB = C / 16;                  // row tiles (one per wave)
  static constexpr int NPAIR = NSB * (NSB - 1) / 2;   // tile pairs below the diagonal
  // LDS layout (bytes)
  static constexpr int TOT_OFF = 0;                                     // [NSB][DK] fp32 tile products
  static constexpr int BETA_OFF = TOT_OFF + NSB * DK * 4;               // [C] fp32
  static constexpr int KRS_OFF = BETA_OFF + C * 4;                      // [C][DK] keys decayed to chunk end
  static constexpr int KRS_BYTES = C * DK * (int)sizeof(T);
  static constexpr int MAIN_OFF = (KRS_OFF + KRS_BYTES + 15) / 16 * 16;
  // phase 1 of MAIN: Gram operand fragments
  static constexpr int XP_OFF = 0;                                      // [2][NSB-1][KBN] fragments
  static constexpr int Y_OFF = XP_OFF + 2 * (NSB - 1) * G::KBN * 1024;  // [NPAIR][KBN]
  static constexpr int OPER_BYTES = Y_OFF + NPAIR * G::KBN * 1024;
  // phase 2 of MAIN: fp32 C x C matrices A, M, T
  static constexpr int SCR_BYTES = 3 * C * C * 4;
  static constexpr int MAIN_BYTES = OPER_BYTES > SCR_BYTES ? OPER_BYTES : SCR_BYTES;
  static constexpr int LDS_BYTES = MAIN_OFF + MAIN_BYTES;
  static constexpr int NCHAIN = 2 * NPAIR;            // off-diagonal Gram tiles (A and M)
  static constexpr int CPW = NCHAIN > 4 ? (NCHAIN + 3) / 4 : 1;   // per wave (at least 1)
};

// Raw bits of one lane's EPL consecutive-in-kappa elements.
template <typename T> struct Raw;
template <> struct Raw<bf16_t> { u32x4 w; };   // 8 bf16
template <> struct Raw<float> { f32x4 w; };    // 4 fp32

template <typename T>
__device__ __forceinline__ float raw_get(const Raw<T>& x, int e);
template <>
__device__ __forceinline__ float raw_get<bf16_t>(const Raw<bf16_t>& x, int e) {
  const uint32_t w = x.w[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float raw_get<float>(const Raw<float>& x, int e) { return x.w[e]; }

// Load lane's fragment slot of one K block of a row-major [rows][DK] input.
template <typename T, int DK>
__device__ __forceinline__ Raw<T> load_row_frag(const T* rowp, int kb, int g) {
  Raw<T> x;
  if constexpr (sizeof(T) == 2) {
    const int c0 = kb * 32 + 4 * g;
    u32x2 lo{0u, 0u}, hi{0u, 0u};
    if (c0 < DK) lo = *reinterpret_cast<const u32x2*>(rowp + c0);
    if (c0 + 16 < DK) hi = *reinterpret_cast<const u32x2*>(rowp + c0 + 16);
    x.w = u32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    x.w = *reinterpret_cast<const f32x4*>(rowp + kb * 16 + 4 * g);
  }
  return x;
}

// Set elements e, e + 1 (e even) of a fragment.
template <typename T>
__device__ __forceinline__ void put2(Frag& f, int e, float v0, float v1) {
  if constexpr (sizeof(T) == 2) {
    f.w[e >> 1] = pack_bf16x2(v0, v1);
  } else {
    f.w[e] = __float_as_uint(v0);
    f.w[e + 1] = __float_as_uint(v1);
  }
}

template <typename T>
__device__ __forceinline__ Frag pack_frag(const float* v);
template <>
__device__ __forceinline__ Frag pack_frag<bf16_t>(const float* v) {
  Frag f;
  f.w = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  return f;
}
template <>
__device__ __forceinline__ Frag pack_frag<float>(const float* v) {
  Frag f;
  f.w = __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]});
  return f;
}

// Channel of element e of lane group g in K block kb.
template <typename T>
__device__ __forceinline__ int chan(int kb, int g, int e) {
  return kb * FragTraits<T>::KB + kappa<T>(g, e);
}

// The prologue of one chunk.  Called by all threads of a workgroup whose
// first four waves (256 threads) take part; `lds` has P::LDS_BYTES bytes.
//   q, k, alpha, beta : the chunk's first row of each input (row stride DK, beta stride 1)
//   cv                : valid positions in the chunk (the rest act as identity steps)
//   rec               : the chunk's record (ChunkGeom layout)
// `sync` is the workgroup barrier used between phases.
template <typename T, int DK, int C, typename Sync>
__device__ void chunk_prologue(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ alpha,
                               const T* __restrict__ beta, int cv, unsigned char* __restrict__ rec,
                               unsigned char* lds, int tid, Sync sync) {
  using P = ProCfg<T, DK, C>;
  constexpr int NSB = P::NSB, KBN = P::KBN, KBC = P::KBC, EPL = P::EPL, KB = P::KB;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
  float* s_tot = reinterpret_cast<float*>(lds + P::TOT_OFF);
  float* s_beta = reinterpret_cast<float*>(lds + P::BETA_OFF);
  T* s_krs = reinterpret_cast<T*>(lds + P::KRS_OFF);
  unsigned char* s_main = lds + P::MAIN_OFF;
  const bool active = wave < NSB && tid < 256;        // owns row tile `wave`
  const int t = 16 * wave + r;                       // chunk row of this lane
  const bool valid = active && t < cv;
  const int tl = min(t, cv - 1);                     // row index kept in range

  if (tid < C) {
    const float b = to_f32(beta[min(tid, cv - 1)]);
    s_beta[tid] = tid < cv ? b : 0.f;
  }

  // ---- pass 1: load this lane's slots, signed gates, tile products
  Raw<T> ra[KBN], rk[KBN], rq[KBN];
  if (active) {
#pragma unroll
    for (int kb = 0; kb < KBN; ++kb) {
      ra[kb] = load_row_frag<T, DK>(alpha + (size_t)tl * DK, kb, g);
      rk[kb] = load_row_frag<T, DK>(k + (size_t)tl * DK, kb, g);
      rq[kb] = load_row_frag<T, DK>(q + (size_t)tl * DK, kb, g);
    }
#pragma unroll
    for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int c = chan<T>(kb, g, e);
        const float a = (valid && c < DK) ? floor_gate(raw_get<T>(ra[kb], e)) : 1.f;
        const float tot = row_total(a, r);
        if (r == 15 && c < DK) s_tot[wave * DK + c] = tot;
      }
  }
  sync();

  // ---- pass 2: scans, record operands, Gram operands, diagonal tiles
  f32x4 accAD = zero4(), accMD = zero4(), accAL = zero4(), accML = zero4();
  if (active) {
    const bool lo4 = (r & 4) == 0;     // first quarter of an 8-row half
    const bool up8 = r >= 8;
#pragma unroll
    for (int kb = 0; kb < KBN; ++kb) {
      Frag fw, fq, fxkp, fxqp, fxkd, fxqd, fyd, fxkl, fxql, fyl;
      Frag fy[NSB];
#pragma unroll
      for (int e = 0; e < EPL; e += 2) {
        float v[2][13];
        float yv[2][NSB];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = chan<T>(kb, g, e + h);
          const bool live = valid && c < DK;
          const float a = live ? floor_gate(raw_get<T>(ra[kb], e + h)) : 1.f;
          const float kk = live ? raw_get<T>(rk[kb], e + h) : 0.f;
          const float qq = live ? raw_get<T>(rq[kb], e + h) : 0.f;
          const RowScan sc = row_scan(a, r);
          // products over whole tiles: before, after, and between this and later tiles
          const int cc = c < DK ? c : 0;
          float before = 1.f, after = 1.f, all = 1.f, run = 1.f;
          float mid[NSB];
#pragma unroll
          for (int J = 0; J < NSB; ++J) {
            const float tj = s_tot[J * DK + cc];
            all *= tj;
            if (J < wave) before *= tj;
            if (J > wave) after *= tj;
            mid[J] = run;                      // product of tiles wave+1 .. J-1
            if (J > wave) run *= tj;
          }
          const float gam = before * sc.p16;   // signed prefix from the chunk start (inclusive)
          const float gend = sc.s16 * after;   // signed product after this row to the chunk end
          v[h][0] = -kk * gam;                 // W
          v[h][1] = qq * gam;                  // Q
          v[h][2] = all;                       // d
          if (c < DK) s_krs[t * DK + c] = from_f32<T>(kk * gend);
          v[h][3] = kk * sc.p16;               // X (keys) of tile pairs below the diagonal
          v[h][4] = qq * sc.p16;               // X (queries)
          const float ky = kk * sc.s16;
#pragma unroll
          for (int I = 0; I < NSB; ++I) yv[h][I] = ky * mid[I];   // Y of pair (I, wave), I > wave
          // diagonal quadrants: split at the quadrant midpoint
          const float sel = lo4 ? sc.s4 : sc.p4;
          const float rc = __builtin_amdgcn_rcpf(sel);
          const float am = lo4 ? rc : sc.p4;
          const float bm = lo4 ? sc.s4 : rc;
          v[h][5] = kk * am;
          v[h][6] = qq * am;
          v[h][7] = kk * bm;
          // lower-left quadrant: split at the quadrant boundary
          v[h][8] = up8 ? kk * sc.p8 : 0.f;
          v[h][9] = up8 ? qq * sc.p8 : 0.f;
          v[h][10] = up8 ? 0.f : kk * sc.s8;
          if (r == 0 && c < DK) reinterpret_cast<float*>(rec + P::D_OFF)[c] = all;
        }
        put2<T>(fw, e, v[0][0], v[1][0]);
        put2<T>(fq, e, v[0][1], v[1][1]);
        put2<T>(fxkp, e, v[0][3], v[1][3]);
        put2<T>(fxqp, e, v[0][4], v[1][4]);
        put2<T>(fxkd, e, v[0][5], v[1][5]);
        put2<T>(fxqd, e, v[0][6], v[1][6]);
        put2<T>(fyd, e, v[0][7], v[1][7]);
        put2<T>(fxkl, e, v[0][8], v[1][8]);
        put2<T>(fxql, e, v[0][9], v[1][9]);
        put2<T>(fyl, e, v[0][10], v[1][10]);
#pragma unroll
        for (int I = 0; I < NSB; ++I) put2<T>(fy[I], e, yv[0][I], yv[1][I]);
      }
      // record: W and Q fragments of row tile `wave`, K block kb
      store_frag(rec + P::W_OFF + frag_slot(wave, kb, KBN, lane), fw);
      store_frag(rec + P::Q_OFF + frag_slot(wave, kb, KBN, lane), fq);
      // Gram operands other waves need
      Frag* xp = reinterpret_cast<Frag*>(s_main + P::XP_OFF);
      Frag* yp = reinterpret_cast<Frag*>(s_main + P::Y_OFF);
      if (wave >= 1) {
        xp[((0 * (NSB - 1) + wave - 1) * KBN + kb) * 64 + lane] = fxkp;
        xp[((1 * (NSB - 1) + wave - 1) * KBN + kb) * 64 + lane] = fxqp;
      }
      int pbase = 0;                          // pairs (., J) with J < wave come first
      for (int j = 0; j < wave; ++j) pbase += NSB - 1 - j;
#pragma unroll
      for (int I = 1; I < NSB; ++I)
        if (I > wave) yp[((pbase + I - wave - 1) * KBN + kb) * 64 + lane] = fy[I];
      // this wave's diagonal tile
      accAD = mma<T>(accAD, fxkd, fyd);
      accMD = mma<T>(accMD, fxqd, fyd);
      accAL = mma<T>(accAL, fxkl, fyl);
      accML = mma<T>(accML, fxql, fyl);
    }
  }
  sync();

  // ---- pass 3: Gram tiles below the diagonal; chain -> (kind, pair)
  f32x4 acc[P::CPW];
  int chain_I[P::CPW], chain_J[P::CPW], chain_kind[P::CPW];
#pragma unroll
  for (int j = 0; j < P::CPW; ++j) {
    acc[j] = zero4();
    chain_I[j] = chain_J[j] = chain_kind[j] = -1;
    const int ch = wave + 4 * j;
    if (tid < 256 && ch < P::NCHAIN) {
      const int kind = ch & 1, pr = ch >> 1;
      int J = 0, rem = pr;
      while (rem >= NSB - 1 - J) { rem -= NSB - 1 - J; ++J; }
      const int I = J + 1 + rem;
      chain_I[j] = I; chain_J[j] = J; chain_kind[j] = kind;
      const Frag* xp = reinterpret_cast<const Frag*>(s_main + P::XP_OFF) + ((kind * (NSB - 1) + I - 1) * KBN) * 64;
      const Frag* yp = reinterpret_cast<const Frag*>(s_main + P::Y_OFF) + (pr * KBN) * 64;
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) acc[j] = mma<T>(acc[j], xp[kb * 64 + lane], yp[kb * 64 + lane]);
    }
  }
  sync();

  // ---- A (rows scaled by beta, strictly lower) and M (lower incl.) to LDS, fp32
  float* As = reinterpret_cast<float*>(s_main);
  float* Ms = As + C * C;
  float* Ts = Ms + C * C;
  // upper tiles are zero; T starts as zero
  for (int i = tid; i < C * C; i += (int)blockDim.x) {
    const int row = i / C, col = i % C;
    if (col / 16 > row / 16) { As[i] = 0.f; Ms[i] = 0.f; }
    Ts[i] = 0.f;
  }
  if (active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 4 * g + i, row = 16 * wave + lr, col = 16 * wave + r;
      const bool diagq = (lr >> 3) == (r >> 3);
      const bool ll = lr >= 8 && r < 8;
      const float a = diagq ? (r < lr ? accAD[i] : 0.f) : (ll ? accAL[i] : 0.f);
      const float m = diagq ? (r <= lr ? accMD[i] : 0.f) : (ll ? accML[i] : 0.f);
      As[row * C + col] = a * s_beta[row];
      Ms[row * C + col] = m;
    }
  }
#pragma unroll
  for (int j = 0; j < P::CPW; ++j) {
    if (chain_kind[j] >= 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * chain_I[j] + 4 * g + i, col = 16 * chain_J[j] + r;
        if (chain_kind[j] == 0) As[row * C + col] = acc[j][i] * s_beta[row];
        else Ms[row * C + col] = acc[j][i];
      }
    }
  }
  sync();

  // ---- T = (I + A)^-1: diagonal 16x16 blocks by forward substitution
  if (tid < 16 * NSB) {
    const int blk = tid >> 4, jc = tid & 15, o = 16 * blk;
    float tcol[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jc) ? 1.f : 0.f;
      const float* arow = As + (o + i) * C + o;
#pragma unroll
      for (int k4 = 0; k4 < i; k4 += 4) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(arow + k4);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (k4 + u < i) s -= av[u] * tcol[k4 + u];
      }
      tcol[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Ts[(o + i) * C + o + jc] = tcol[i];
  }
  sync();

  // ---- off-diagonal blocks by distance on fp32 matrix cores:
  //      T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
  for (int d = 1; d < NSB; ++d) {
    const int J = wave, I = J + d;
    if (tid < 256 && I < NSB) {
      f32x4 s = zero4();
      for (int K = J; K < I; ++K) {
        // A-operand: rows of A_IK (4 consecutive floats); B-operand: T_KJ column slots
        const float* arow = As + (16 * I + r) * C + 16 * K;
        const float* tb = Ts + (16 * K) * C + 16 * J + r;
        Frag fa, fb;
        fa.w = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4*>(arow + 4 * g));
        fb.w = __builtin_bit_cast(u32x4, f32x4{tb[(4 * g + 0) * C], tb[(4 * g + 1) * C], tb[(4 * g + 2) * C],
                                               tb[(4 * g + 3) * C]});
        s = mma<float>(s, fa, fb);
      }
      // T_II (A-operand rows) times S (its accumulator registers are its B fragment)
      const float* trow = Ts + (16 * I + r) * C + 16 * I;
      Frag fa;
      fa.w = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4*>(trow + 4 * g));
      const f32x4 tij = mma<float>(zero4(), fa, frag_from_acc_f32(s));
#pragma unroll
      for (int i = 0; i < 4; ++i) Ts[(16 * I + 4 * g + i) * C + 16 * J + r] = -tij[i];
    }
    sync();
  }

  // ---- record: T Diag(beta) and M fragments, and KR (keys decayed to the chunk end)
  constexpr int NF = P::RT * KBC;
  constexpr int NKR = P::RH * KBC;
  for (int f = wave; tid < 256 && f < 2 * NF + NKR; f += 4) {
    Frag out;
    float vals[8];
    if (f < 2 * NF) {
      const bool isT = f < NF;
      const int ff = isT ? f : f - NF;
      const int rt = ff / KBC, kb = ff % KBC;
      const float* src = (isT ? Ts : Ms) + (16 * rt + r) * C;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int col = kb * KB + kappa<T>(g, e);
        float v = 0.f;
        if (col < C) v = isT ? src[col] * s_beta[col] : src[col];
        vals[e] = v;
      }
      out = pack_frag<T>(vals);
      store_frag(rec + (isT ? P::T_OFF : P::M_OFF) + frag_slot(rt, kb, KBC, lane), out);
    } else {
      const int ff = f - 2 * NF;
      const int rt = ff / KBC, kb = ff % KBC;   // channel tile, position block
      const int c = 16 * rt + r;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int pos = kb * KB + kappa<T>(g, e);
        vals[e] = pos < C ? to_f32(s_krs[pos * DK + c]) : 0.f;
      }
      out = pack_frag<T>(vals);
      store_frag(rec + P::KR_OFF + frag_slot(rt, kb, KBC, lane), out);
    }
  }
}

}  // namespace ckda
