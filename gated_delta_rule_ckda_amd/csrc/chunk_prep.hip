// chunk_prep.hip -- per-chunk preparation of the chunkwise CKDA forward.
//
// One workgroup (4 waves) per chunk of one (batch, head); every chunk of every
// head is independent, so the grid covers them all at once.  For its chunk
// the workgroup
//   (a) splits each gate into a sign bit and a magnitude (paper Prop. 2,
//       sign(0) = +1), forms the chunk-local cumulative sign parity P_t and
//       absorbs it into keys and queries (discussion slides, "Absorb
//       cumulative signs into keys and queries"); magnitudes are combined as
//       products over position segments in fp32 -- never logarithms, so zero
//       and negative gates need no special case beyond the magnitude floor;
//   (b) builds the decayed Gram matrices on the matrix cores
//         A[t,j] = beta_t sum_c k~_tc k~_jc r_c(t,j)   (j < t)
//         M[t,j] =        sum_c q~_tc k~_jc r_c(t,j)   (j <= t)
//       with r_c(t,j) = prod_{s=j+1..t} |alpha_sc|, and solves the unit lower
//       triangular system T = (I + A)^-1 in fp32 (16x16 diagonal blocks by
//       forward substitution, off-diagonal blocks by block recursion);
//   (c) writes the record of operands the state pass consumes (layout in
//       chunk_common.hpp), in matrix-core fragment order.
//
// Decay factors never overflow: r(t,j) is split at sub-block boundaries into
// a prefix inside t's 16-row sub-block, whole sub-blocks in between and a
// suffix inside j's sub-block, each a product of magnitudes <= 1.  A 16x16
// diagonal tile is split into 8x8 quadrants: the lower-left one splits r at
// the quadrant boundary (again two products <= 1); each diagonal quadrant
// splits it at its midpoint, where the factor on the far side is the
// reciprocal of at most 4 magnitudes.  Magnitudes are floored at 2^-31 so
// that this reciprocal stays finite in fp32 and bf16 (a product of 4 floored
// magnitudes is >= 2^-124); the floor changes a gate by at most 2^-31.
//
// The chunk form itself is derived from the recurrence (paper Eq. (1)): for
// incoming state H0, U = T Diag(beta) (V - (K~ . gamma) H0),
// O = (Q~ . gamma) H0 + M U, H_C = P_C [gamma_C . H0 + (K~ . gamma_C/gamma)^T U].
#include "chunk_common.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int kPrepThreads = 512;
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr float kGateFloor = 4.656612873077393e-10f;  // 2^-31

template <typename T, int DK, int C>
struct PrepCfg : ChunkGeom<T, DK, C> {
  using G = ChunkGeom<T, DK, C>;
  static constexpr int NSB = C / 16;                              // 16-row sub-blocks
  static constexpr int NHB = C / 8;                               // 8-row half blocks
  static constexpr int CG = DK < kPrepThreads / NHB ? DK : kPrepThreads / NHB;  // channels per group
  static constexpr int NG = DK / CG;                              // channel groups
  static constexpr int CGP = CG > G::KB ? CG : G::KB;             // padded row length
  static constexpr int RS = CGP * G::E + (G::E == 2 ? 8 : 16);    // LDS row stride (bytes)
  static constexpr int NPAIR = NSB * (NSB - 1) / 2;
  static constexpr int R_XK = 0;                                  // rows of sub-blocks 1..NSB-1
  static constexpr int R_XQ = R_XK + (NSB - 1) * 16;
  static constexpr int R_Y = R_XQ + (NSB - 1) * 16;               // one 16-row block per pair
  static constexpr int R_XKD = R_Y + NPAIR * 16;
  static constexpr int R_XQD = R_XKD + C;
  static constexpr int R_YD = R_XQD + C;
  static constexpr int R_X2K = R_YD + C;                          // rows 8-15 of each sub-block
  static constexpr int R_X2Q = R_X2K + C / 2;
  static constexpr int R_Y2 = R_X2Q + C / 2;                      // rows 0-7 of each sub-block
  static constexpr int ROWS = R_Y2 + C / 2;
  static constexpr int OPER_BYTES = ROWS * RS;
  static constexpr int SCR_BYTES = 3 * C * C * 4 + kPrepWaves * 16 * 16 * 4;
  static constexpr int MAIN_BYTES = OPER_BYTES > SCR_BYTES ? OPER_BYTES : SCR_BYTES;
  static constexpr int NT1 = NSB * (NSB + 1);                     // A and M tiles (I >= J)
  static constexpr int NTILE = NT1 + 2 * NSB;                     // + lower-left diagonal quadrants
  static constexpr int TPW = (NTILE + kPrepWaves - 1) / kPrepWaves;
};

// Pair index of sub-blocks (I, J), I > J, in J-major order.
__device__ __forceinline__ int pair_index(int I, int J, int nsb) {
  int p = 0;
  for (int j = 0; j < J; ++j) p += nsb - 1 - j;
  return p + (I - J - 1);
}

// Byte offset, inside an A-operand region with `nkb` K blocks, of element
// (row m, contraction index k).
template <typename T>
__host__ __device__ constexpr size_t a_elem_offset(int m, int k, int nkb) {
  constexpr int KB = FragTraits<T>::KB;
  return frag_slot(m / 16, k / KB, nkb, ((k % KB) % 16) / 4 * 16 + (m % 16)) +
         (size_t)(((k % KB) / 16) * 4 + (k % KB) % 4) * sizeof(T);
}

template <typename T>
__device__ __forceinline__ void st_elem(unsigned char* p, float x) {
  *reinterpret_cast<T*>(p) = from_f32<T>(x);
}

// Row fragment from an LDS operand array: lane (g, r) gets row r0 + r at the
// K-block kb columns of the fragment K order.
template <typename T>
__device__ __forceinline__ Frag lds_row_frag(const unsigned char* lds, int rs, int r0, int kb, int lane) {
  const int g = lane / 16, r = lane % 16;
  const unsigned char* row = lds + (r0 + r) * rs;
  Frag f;
  if constexpr (sizeof(T) == 2) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(row + (kb * 32 + 4 * g) * 2);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(row + (kb * 32 + 16 + 4 * g) * 2);
    f.w = u32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    f.w = *reinterpret_cast<const u32x4*>(row + (kb * 16 + 4 * g) * 4);
  }
  return f;
}

// As lds_row_frag for an operand that exists on half of the 16 rows only:
// upper = true -> lanes r >= 8 read row r0 + r - 8 and lanes r < 8 get zeros;
// upper = false -> lanes r < 8 read row r0 + r and lanes r >= 8 get zeros.
template <typename T>
__device__ __forceinline__ Frag lds_half_frag(const unsigned char* lds, int rs, int r0, int kb, int lane,
                                              bool upper) {
  const int r = lane % 16;
  const bool live = upper ? r >= 8 : r < 8;
  const int rr = upper ? r0 - 8 : r0;
  Frag f;
  f.w = u32x4{0u, 0u, 0u, 0u};
  if (live) f = lds_row_frag<T>(lds, rs, rr, kb, lane);
  return f;
}

// out[rr][cc..cc+3] += sum_k X[rr][k] * Y[k][cc..cc+3] for 16x16 fp32 blocks in
// LDS (row strides in floats); lane l owns rr = l / 4, cc = 4 (l % 4).
__device__ __forceinline__ f32x4 block_mac(f32x4 acc, const float* X, int xs, const float* Y, int ys,
                                           int lane) {
  const int rr = lane / 4, cc = 4 * (lane % 4);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float x = X[rr * xs + k];
    const f32x4 y = *reinterpret_cast<const f32x4*>(Y + k * ys + cc);
    acc += x * y;
  }
  return acc;
}

template <typename T, int DK, int C>
__global__ __launch_bounds__(kPrepThreads, 4) void chunk_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ alpha,
    const T* __restrict__ beta, unsigned char* __restrict__ ws, int T_len, int nchunks) {
  using P = PrepCfg<T, DK, C>;
  constexpr int NSB = P::NSB, NHB = P::NHB, CG = P::CG, RS = P::RS, E = P::E, KB = P::KB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[P::MAIN_BYTES];
  __shared__ float s_beta[C];
  __shared__ float s_hp[NHB][CG];
  __shared__ unsigned s_hpar[NHB][CG];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane / 16, r = lane % 16;
  const long long chunk_id = blockIdx.x;
  const long long bh = chunk_id / nchunks;
  const int c_idx = (int)(chunk_id % nchunks);
  const int t_begin = c_idx * C;
  const int cv = min(C, T_len - t_begin);            // valid positions in this chunk
  const long long row0 = bh * (long long)T_len + t_begin;
  unsigned char* rec = ws + (size_t)chunk_id * P::BYTES;

  for (int t = tid; t < C; t += kPrepThreads) {
    const float b = to_f32(beta[row0 + min(t, cv - 1)]);   // index kept in range
    s_beta[t] = t < cv ? b : 0.f;
  }
  if constexpr (P::CGP > CG) {  // zero the padding columns once (bf16 with DK = 16)
    for (int i = tid; i < P::OPER_BYTES / 4; i += kPrepThreads) reinterpret_cast<unsigned*>(smem)[i] = 0u;
    lds_barrier();
  }

  f32x4 acc[P::TPW];
#pragma unroll
  for (int j = 0; j < P::TPW; ++j) acc[j] = zero4();

  // gate task of this thread: channel cl of the group, 8-row half block hb
  const bool has_task = tid < CG * NHB;
  const int cl = tid % CG, hb = tid / CG;
  const int sb = hb / 2, hh = hb % 2;                 // 16-row sub-block, half inside it

  for (int grp = 0; grp < P::NG; ++grp) {
    const int c = grp * CG + cl;
    float m[8], kk[8], qq[8];
    unsigned sg = 0;
    if (has_task) {
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        const int t = hb * 8 + l;
        const bool valid = t < cv;
        const long long ix = (row0 + min(t, cv - 1)) * DK + c;   // index kept in range
        const float a0 = to_f32(alpha[ix]), k0 = to_f32(k[ix]), q0 = to_f32(q[ix]);
        const float a = valid ? a0 : 1.f;
        kk[l] = valid ? k0 : 0.f;
        qq[l] = valid ? q0 : 0.f;
        sg |= (a < 0.f ? 1u : 0u) << l;
        const float mag = fabsf(a);
        m[l] = mag < kGateFloor ? kGateFloor : mag;   // NaN propagates
      }
      float hp = 1.f;
#pragma unroll
      for (int l = 0; l < 8; ++l) hp *= m[l];
      s_hp[hb][cl] = hp;
      s_hpar[hb][cl] = __builtin_popcount(sg) & 1u;
    }
    lds_barrier();

    if (has_task) {
      // products of the half blocks before / after this one, of the other half
      // of this sub-block, of the whole chunk, and of the sub-blocks strictly
      // between this one and each later sub-block I
      float before = 1.f, after = 1.f, gC = 1.f, other = 1.f;
      unsigned pbefore = 0, pC = 0;
      float hps[NHB];
#pragma unroll
      for (int h = 0; h < NHB; ++h) {
        hps[h] = s_hp[h][cl];
        const unsigned pp = s_hpar[h][cl];
        gC *= hps[h];
        pC ^= pp;
        if (h < hb) { before *= hps[h]; pbefore ^= pp; }
        if (h > hb) after *= hps[h];
      }
      other = hps[hb ^ 1];
      float mid[NSB];
      {
        float run = 1.f;
#pragma unroll
        for (int I = 0; I < NSB; ++I) {
          mid[I] = run;                              // prod of sub-blocks sb+1 .. I-1
          if (I > sb) run *= hps[2 * I] * hps[2 * I + 1];
        }
      }
      // within-half prefix (inclusive) and suffix (exclusive) products, and
      // the split factors around the half's midpoint (between rows 3 and 4)
      float wpre[8], wsuf[8], am[8], bm[8];
      wpre[0] = m[0];
#pragma unroll
      for (int l = 1; l < 8; ++l) wpre[l] = wpre[l - 1] * m[l];
      wsuf[7] = 1.f;
#pragma unroll
      for (int l = 6; l >= 0; --l) wsuf[l] = wsuf[l + 1] * m[l + 1];
      bm[3] = 1.f;
#pragma unroll
      for (int l = 2; l >= 0; --l) bm[l] = bm[l + 1] * m[l + 1];
      am[4] = m[4];
#pragma unroll
      for (int l = 5; l < 8; ++l) am[l] = am[l - 1] * m[l];
#pragma unroll
      for (int l = 0; l < 4; ++l) am[l] = __builtin_amdgcn_rcpf(bm[l]);
#pragma unroll
      for (int l = 4; l < 8; ++l) bm[l] = __builtin_amdgcn_rcpf(am[l]);

      // per-thread bases of the record elements this thread writes; the row
      // inside the half block only adds a constant to them
      unsigned char* w_base = rec + P::W_OFF + a_elem_offset<T>(hb * 8, c, P::KBN);
      unsigned char* q_base = rec + P::Q_OFF + a_elem_offset<T>(hb * 8, c, P::KBN);
      unsigned char* kr_base = rec + P::KR_OFF + a_elem_offset<T>(c, hb * 8, P::KBC);
      unsigned char* lrow = smem + cl * E + (8 * hh) * RS;
      unsigned char* y_base[NSB];
#pragma unroll
      for (int I = 0; I < NSB; ++I)
        y_base[I] = smem + cl * E + (P::R_Y + (I > sb ? pair_index(I, sb, NSB) : 0) * 16 + 8 * hh) * RS;

      unsigned par = pbefore;
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        par ^= (sg >> l) & 1u;
        const float kt = par ? -kk[l] : kk[l];
        const float qt = par ? -qq[l] : qq[l];
        const float gam = before * wpre[l];                  // gamma_t
        const float pre = (hh ? other : 1.f) * wpre[l];      // prefix inside the sub-block
        const float suf = wsuf[l] * (hh ? 1.f : other);      // suffix inside the sub-block
        const float kr = wsuf[l] * after;                    // gamma_C / gamma_t
        st_elem<T>(w_base + l * 16, -kt * gam);
        st_elem<T>(q_base + l * 16, qt * gam);
        st_elem<T>(kr_base + (l / 4) * 256 + (l % 4) * E, (pC ^ par) ? -kk[l] * kr : kk[l] * kr);
        if constexpr (C < KB)  // zero the K padding of the positions operand
          st_elem<T>(kr_base + (l / 4) * 256 + (l % 4) * E + 4 * E, 0.f);
        if constexpr (DK < KB) {  // zero the K padding of the channel operands
          st_elem<T>(w_base + l * 16 + 4 * E, 0.f);
          st_elem<T>(q_base + l * 16 + 4 * E, 0.f);
        }
        // Gram operands for this channel group
        unsigned char* rowp = lrow + l * RS;
        if (sb >= 1) {
          st_elem<T>(rowp + (P::R_XK + (sb - 1) * 16) * RS, kt * pre);
          st_elem<T>(rowp + (P::R_XQ + (sb - 1) * 16) * RS, qt * pre);
        }
#pragma unroll
        for (int I = 0; I < NSB; ++I)
          if (I > sb) st_elem<T>(y_base[I] + l * RS, kt * suf * mid[I]);
        st_elem<T>(rowp + (P::R_XKD + sb * 16) * RS, kt * am[l]);
        st_elem<T>(rowp + (P::R_XQD + sb * 16) * RS, qt * am[l]);
        st_elem<T>(rowp + (P::R_YD + sb * 16) * RS, kt * bm[l]);
        if (hh) {   // rows 8-15: prefix from row 8
          st_elem<T>(rowp + (P::R_X2K + sb * 8 - 8) * RS, kt * wpre[l]);
          st_elem<T>(rowp + (P::R_X2Q + sb * 8 - 8) * RS, qt * wpre[l]);
        } else {    // rows 0-7: suffix up to row 7
          st_elem<T>(rowp + (P::R_Y2 + sb * 8) * RS, kt * wsuf[l]);
        }
      }
      if (hb == 0) reinterpret_cast<float*>(rec + P::D_OFF)[c] = pC ? -gC : gC;
    }
    lds_barrier();

    // Gram tiles: tile index tau -> (kind, I, J), kind 0 = A (keys), 1 = M
    // (queries); tau >= NT1 are the lower-left quadrants of diagonal tiles
#pragma unroll
    for (int j = 0; j < P::TPW; ++j) {
      const int tau = wave + kPrepWaves * j;
      if (tau < P::NT1) {
        const int kind = tau & 1, pr = tau >> 1;
        int I = 0, J = pr;
        while (J > I) { J -= I + 1; ++I; }
        int xr, yr;
        if (I > J) {
          xr = (kind ? P::R_XQ : P::R_XK) + (I - 1) * 16;
          yr = P::R_Y + pair_index(I, J, NSB) * 16;
        } else {
          xr = (kind ? P::R_XQD : P::R_XKD) + I * 16;
          yr = P::R_YD + J * 16;
        }
#pragma unroll
        for (int kb = 0; kb < P::CGP / KB; ++kb)
          acc[j] = mma<T>(acc[j], lds_row_frag<T>(smem, RS, xr, kb, lane), lds_row_frag<T>(smem, RS, yr, kb, lane));
      } else if (tau < P::NTILE) {
        const int kind = (tau - P::NT1) & 1, I = (tau - P::NT1) >> 1;
        const int xr = (kind ? P::R_X2Q : P::R_X2K) + I * 8, yr = P::R_Y2 + I * 8;
#pragma unroll
        for (int kb = 0; kb < P::CGP / KB; ++kb)
          acc[j] = mma<T>(acc[j], lds_half_frag<T>(smem, RS, xr, kb, lane, true),
                          lds_half_frag<T>(smem, RS, yr, kb, lane, false));
      }
    }
    lds_barrier();
  }

  // ---- A and M to LDS (fp32), then the triangular solve
  float* As = reinterpret_cast<float*>(smem);
  float* Ms = As + C * C;
  float* Ts = Ms + C * C;
  float* Ss = Ts + C * C;  // per-wave 16x16 scratch
  for (int i = tid; i < 3 * C * C; i += kPrepThreads) As[i] = 0.f;
  lds_barrier();
  // masked write: off-diagonal tiles whole, diagonal tiles only inside their
  // two diagonal quadrants (elsewhere the midpoint factors are not valid)
#pragma unroll
  for (int j = 0; j < P::TPW; ++j) {
    const int tau = wave + kPrepWaves * j;
    if (tau < P::NT1) {
      const int kind = tau & 1, pr = tau >> 1;
      int I = 0, J = pr;
      while (J > I) { J -= I + 1; ++I; }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = 4 * g + i, row = 16 * I + lr, col = 16 * J + r;
        const bool keep = I > J || (lr / 8 == r / 8 && (kind == 0 ? r < lr : r <= lr));
        const float v = acc[j][i];
        if (kind == 0) As[row * C + col] = keep ? v * s_beta[row] : 0.f;
        else Ms[row * C + col] = keep ? v : 0.f;
      }
    }
  }
  lds_barrier();
  // add the lower-left quadrants of the diagonal tiles
#pragma unroll
  for (int j = 0; j < P::TPW; ++j) {
    const int tau = wave + kPrepWaves * j;
    if (tau >= P::NT1 && tau < P::NTILE) {
      const int kind = (tau - P::NT1) & 1, I = (tau - P::NT1) >> 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = 4 * g + i, row = 16 * I + lr, col = 16 * I + r;
        if (lr >= 8 && r < 8) {
          if (kind == 0) As[row * C + col] += acc[j][i] * s_beta[row];
          else Ms[row * C + col] += acc[j][i];
        }
      }
    }
  }
  lds_barrier();

  // diagonal 16x16 blocks of T by forward substitution: lane (blk, jcol)
  if (wave == 0 && lane < 16 * NSB) {
    const int blk = lane / 16, jc = lane % 16, o = 16 * blk;
    float tcol[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jc) ? 1.f : 0.f;
#pragma unroll
      for (int kx = 0; kx < i; ++kx) s -= As[(o + i) * C + o + kx] * tcol[kx];
      tcol[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Ts[(o + i) * C + o + jc] = tcol[i];
  }
  lds_barrier();

  // off-diagonal blocks by distance: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
  for (int d = 1; d < NSB; ++d) {
    for (int J = wave; J + d < NSB; J += kPrepWaves) {
      const int I = J + d;
      f32x4 s = zero4();
      for (int K = J; K < I; ++K)
        s = block_mac(s, As + (16 * I) * C + 16 * K, C, Ts + (16 * K) * C + 16 * J, C, lane);
      float* S = Ss + wave * 256;
      const int rr = lane / 4, cc = 4 * (lane % 4);
      *reinterpret_cast<f32x4*>(S + rr * 16 + cc) = s;
      lds_wave_fence();
      f32x4 t = block_mac(zero4(), Ts + (16 * I) * C + 16 * I, C, S, 16, lane);
      *reinterpret_cast<f32x4*>(Ts + (16 * I + rr) * C + 16 * J + cc) = -t;
      lds_wave_fence();
    }
    lds_barrier();
  }

  // ---- emit T Diag(beta) and M as A-operand fragments (K order of the positions)
  constexpr int NF = P::RT * P::KBC;
  for (int f = wave; f < 2 * NF; f += kPrepWaves) {
    const bool isT = f < NF;
    const int ff = isT ? f : f - NF;
    const int rt = ff / P::KBC, kb = ff % P::KBC;
    const float* src = isT ? Ts : Ms;
    const int row = 16 * rt + r;
    float vals[8];
#pragma unroll
    for (int e = 0; e < P::EPL; ++e) {
      const int col = kb * KB + kappa<T>(g, e);
      float v = 0.f;
      if (col < C) {
        v = src[row * C + col];
        if (isT) v *= s_beta[col];
      }
      vals[e] = v;
    }
    Frag out;
    if constexpr (sizeof(T) == 2) {
      out.w = u32x4{pack_bf16x2(vals[0], vals[1]), pack_bf16x2(vals[2], vals[3]),
                    pack_bf16x2(vals[4], vals[5]), pack_bf16x2(vals[6], vals[7])};
    } else {
      out.w = __builtin_bit_cast(u32x4, f32x4{vals[0], vals[1], vals[2], vals[3]});
    }
    store_frag(rec + (isT ? P::T_OFF : P::M_OFF) + frag_slot(rt, kb, P::KBC, lane), out);
  }
}

template <typename T, int DK, int C>
hipError_t launch_prep_t(const ChunkArgs& a, long long total_chunks, int nchunks) {
  hipLaunchKernelGGL((chunk_prep_kernel<T, DK, C>), dim3((unsigned)total_chunks), dim3(kPrepThreads), 0,
                     a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.alpha, (const T*)a.beta,
                     (unsigned char*)a.workspace, a.T, nchunks);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t prep_chunk_dispatch(const ChunkArgs& a, long long total, int nch) {
  switch (a.chunk) {
    case 16: return launch_prep_t<T, DK, 16>(a, total, nch);
    case 32: return launch_prep_t<T, DK, 32>(a, total, nch);
    case 64: return launch_prep_t<T, DK, 64>(a, total, nch);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t prep_dk_dispatch(const ChunkArgs& a, long long total, int nch) {
  switch (a.dk) {
    case 16: return prep_chunk_dispatch<T, 16>(a, total, nch);
    case 32: return prep_chunk_dispatch<T, 32>(a, total, nch);
    case 64: return prep_chunk_dispatch<T, 64>(a, total, nch);
    case 128: return prep_chunk_dispatch<T, 128>(a, total, nch);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_prep(const ChunkArgs& a, long long total_chunks, int nchunks) {
  if (total_chunks == 0) return hipSuccess;
  return a.dtype == 1 ? prep_dk_dispatch<bf16_t>(a, total_chunks, nchunks)
                      : prep_dk_dispatch<float>(a, total_chunks, nchunks);
}

template <typename T, int DK>
static size_t record_bytes_c(int chunk) {
  switch (chunk) {
    case 16: return ChunkGeom<T, DK, 16>::BYTES;
    case 32: return ChunkGeom<T, DK, 32>::BYTES;
    case 64: return ChunkGeom<T, DK, 64>::BYTES;
  }
  return 0;
}

template <typename T>
static size_t record_bytes_t(int dk, int chunk) {
  switch (dk) {
    case 16: return record_bytes_c<T, 16>(chunk);
    case 32: return record_bytes_c<T, 32>(chunk);
    case 64: return record_bytes_c<T, 64>(chunk);
    case 128: return record_bytes_c<T, 128>(chunk);
  }
  return 0;
}

ChunkRecord chunk_record_layout(int dk, int chunk, int dtype) {
  ChunkRecord rr{};
  rr.bytes = dtype == 1 ? record_bytes_t<bf16_t>(dk, chunk) : record_bytes_t<float>(dk, chunk);
  return rr;
}

}  // namespace ckda
