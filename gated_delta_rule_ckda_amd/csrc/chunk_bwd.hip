// chunk_bwd.hip -- chunkwise backward of the CKDA / KDA recurrence: given
// dL/do and dL/dH_T, the gradients of q, k, v, alpha, beta and h0.
//
// The recurrence (paper Eq. (1)) per chunk of C positions with incoming
// state H, signed gate products G(t, j) = alpha_{j+1} ... alpha_t per channel,
// Gamma_t = G(t, -1):
//   KG = K . Gamma, QG = Q . Gamma, KR_j = k_j . G(C-1, j),
//   S[t, j] = sum_c k_tc k_jc G_c(t, j) (j < t), M[t, j] = sum_c q_tc k_jc G_c(t, j) (j <= t),
//   T = (I + Diag(beta) S)^-1, TB = T Diag(beta),
//   X = V - KG H, U = TB X, O = QG H + M U, H' = Gamma_C . H + KR^T U,
// and its reverse-mode derivative
//   dU = M^T dO + KR dH',  dX = TB^T dU (= dV),  dH = Gamma_C . dH' + QG^T dO - KG^T dX,
//   dQG = dO H^T, dKG = -dX H^T, dKR = U dH'^T, dGamma_C = rowsum(H . dH'),
//   dM = tril(dO U^T), dTB = tril(dU X^T), dbeta = colsum(T . dTB) + rowsum(dA . S),
//   dA = -T^T dTB Diag(beta) T^T (strictly lower), dS = Diag(beta) dA,
// followed by the decayed-Gram derivatives and every gate derivative.
//
// Four kernels, fp32 arithmetic (with bf16 inputs at dk >= 64 the products of
// the sequential passes and of grad's value-slice loop take split bf16 pairs,
// about 16 bits, on bf16 matrix cores):
//   prep    (resident workgroups looping over chunks) S, M by recursive
//           halving (every level's rescaled rows written at once, each
//           level's cross blocks as 16 x 16 fp32 matrix-core tiles), T by
//           forward substitution, TB, KG, KR, QG, Gamma_C -> a per-chunk
//           record (with the transposes the sequential kernels contract
//           along);
//   states  (sequential, per head and 16-column value slice; two slices per
//           wave with split products once one per wave would put two
//           workgroups on every CU) chunk-start states;
//   dstates (sequential, reverse; at dk 128 with split products and such
//           grids, four waves of two slices per workgroup) the state gradient
//           entering each chunk from its end, and dh0;
//   grad    (one workgroup per chunk)   all per-token gradients.
//
// No gate is ever divided by.  Recursive halving: for a block of positions
// split into halves L (keys, j) and R (queries, t) at m = last of L,
// G(t, j) = G(t, m) G(m, j), both factors products of gates (modulus <= 1),
// so the cross terms are plain products of operands rescaled by them, and the
// derivative for the gate at s collects the pairs j < s <= t with its own
// factor left out, G(t, s) G(s - 1, j), by scans inside the halves.  Exact
// zero gates need no special case.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "ckda_device.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int kBC = 32;          // positions per backward chunk
constexpr int kBThreads = 256;
constexpr int kBDS = 16;         // value columns per slice

// per-chunk fp32 record of the prep kernel (offsets in floats): M^T, TB,
// TB^T, T, S (C x C); KG, KG^T, KR, KR^T, QG^T (C x DK or DK x C); Gamma_C
// (DK).  T and S are row-major; the others, the matrix-core A operands of the
// sequential kernels (the states kernel KG, TB, KR^T; the dstates kernel
// M^T, KR, TB^T, QG^T, KG^T), are in fragment order (frag_off), so that a
// wave reads one operand fragment as 1 KB in one piece.
// Fragment order of an fp32 A operand with R rows and KD columns (K, the
// contraction): 16 x 16 tiles (row tile, K tile) in row-major order, 256
// floats each, lane 16 g + r holding row r, columns 4 g .. 4 g + 3 of its tile.
__host__ __device__ constexpr int frag_off(int row, int k, int KD) {
  return ((row / 16) * (KD / 16) + k / 16) * 256 + ((((k % 16) / 4) * 16 + row % 16) * 4) + k % 4;
}
// the inverse: row and column of the element at offset e
__device__ __forceinline__ void frag_pos(int e, int KD, int& row, int& k) {
  const int f = e / 256, w = e % 256, ln = w / 4;
  row = 16 * (f / (KD / 16)) + ln % 16;
  k = 16 * (f % (KD / 16)) + 4 * (ln / 16) + w % 4;
}

// Split record (bf16 inputs, dk >= 64, d_v a multiple of 32: every consumer
// multiplies split bf16 pairs).  The matrix-core A operands (KG, KG^T, KR,
// KR^T, QG^T, M^T, TB, TB^T) are stored as the pairs themselves, in the same
// bytes: the two fp32 tiles (row tile, 2 kb) and (row tile, 2 kb + 1) of K
// block kb (32 wide) hold the hi and the lo bf16 fragments of that block,
// lane 16 g + r's 16 bytes being row r, K = 32 kb + kappa(g, e), e = 0..7
// (hi = bf16(x), lo = bf16(x - hi), as split_frag forms them from fp32).
// T, S and Gamma_C stay fp32.  In a split record the place of KG^T (which
// only dstates reads) holds -K~G^T, K~G = TB KG, which takes one dependent
// product off the dstates pass:  dH = Gamma_C . dH' + QG^T dO - K~G^T dU
// (= ... - KG^T TB^T dU, without forming dX); TB^T, then unread, is not
// written.
template <int DK>
struct BwdRec {
  static constexpr int C = kBC;
  static constexpr int MT_OFF = 0, TB_OFF = C * C, TBT_OFF = 2 * C * C, T_OFF = 3 * C * C, S_OFF = 4 * C * C;
  static constexpr int KG_OFF = 5 * C * C, KGT_OFF = KG_OFF + C * DK, KR_OFF = KGT_OFF + C * DK;
  static constexpr int KRT_OFF = KR_OFF + C * DK, QGT_OFF = KRT_OFF + C * DK;
  static constexpr int GC_OFF = QGT_OFF + C * DK;
  static constexpr int FLOATS = (GC_OFF + DK + 63) / 64 * 64;
};

// ---------------------------------------------------------------- fp32 MFMA on LDS operands
// v_mfma_f32_16x16x4_f32: lane (g, r) supplies A(r, g) and B(g, r) of one
// 4-wide K step and holds D(4 g + v, r), v = 0..3, of the 16 x 16 result.
// Operands are read from LDS through strides, so a transposed operand is only
// a different pair of strides:  A(i, k) = a[i * ai + k * ak],
// B(k, j) = b[k * bk + j * bj].
// (K is a compile-time constant so that every operand load of the product
// is issued before the chain of matrix-core steps.)
template <int K>
__device__ __forceinline__ f32x4 mfma_lds(f32x4 acc, const float* a, int ai, int ak, const float* b, int bk, int bj) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  float av[K / 4], bv[K / 4];
#pragma unroll
  for (int s = 0; s < K / 4; ++s) {
    av[s] = a[r * ai + (4 * s + g) * ak];
    bv[s] = b[(4 * s + g) * bk + r * bj];
  }
#pragma unroll
  for (int s = 0; s < K / 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
  return acc;
}

// D (Mr x Nc, multiples of 16) = scale * A B  (ACC: D += scale * A B), the
// 16 x 16 tiles spread over the waves; D(i, j) = d[i * di + j].
// W0: the wave that takes the first tile (two products of one phase can so
// run on different waves).
template <bool ACC, int K, int W0 = 0, int NW = kBThreads / 64>
__device__ __forceinline__ void gemm_lds(float* d, int di, const float* a, int ai, int ak, const float* b, int bk,
                                         int bj, int Mr, int Nc, float scale) {
  const int wave = ((threadIdx.x >> 6) + NW - W0) % NW, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int tn = Nc / 16, tiles = (Mr / 16) * tn;
  for (int ti = wave; ti < tiles; ti += NW) {
    const int i0 = (ti / tn) * 16, j0 = (ti % tn) * 16;
    const f32x4 acc = mfma_lds<K>(zero4(), a + i0 * ai, ai, ak, b + j0 * bj, bk, bj);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float* p = d + (i0 + 4 * g + v) * di + j0 + r;
      *p = ACC ? *p + scale * acc[v] : scale * acc[v];
    }
  }
}


// Workgroup -> (batch-head, value slice) of the two sequential kernels.  With
// xcd_map the nsl slices of one head get ids that are equal modulo 8, so they
// run on one XCD (workgroups are dispatched to the 8 XCDs round-robin) and
// share its L2: each chunk's record then comes from HBM once per head rather
// than once per slice.
__device__ __forceinline__ void head_slice(int id, int nsl, int xcd_map, long long& bh, int& slice) {
  if (xcd_map) {
    const int xcd = id % 8, k8 = id / 8;
    bh = (long long)(k8 / nsl) * 8 + xcd;
    slice = k8 % nsl;
  } else {
    bh = id / nsl;
    slice = id % nsl;
  }
}

// Split bf16 products for the sequential passes with bf16 inputs and
// dk >= 64: each operand x (fp32) enters as hi = bf16(x), lo = bf16(x - hi),
// and acc + A B takes lo.hi + hi.lo + hi.hi on bf16 matrix cores (about
// 2^-16 relative per product, against 2^-24 for fp32 matrix cores, at 3 bf16
// steps of 32 K each instead of 8 fp32 steps of 4).  The operands are given
// as two f32x4 in the K order of an fp32 fragment (K 0-15 and 16-31 of the
// block), which is the bf16 fragment's K order (kappa) once packed.
template <typename T, int DK>
constexpr bool kSplitSeq = std::is_same<T, bf16_t>::value && DK >= 64;

struct SplitFrag {
  Frag h, l;
};
__device__ __forceinline__ SplitFrag split_frag(f32x4 k0, f32x4 k1) {
  SplitFrag f;
  frags_from_acc_bf16_split(k0, k1, f.h, f.l);
  return f;
}
__device__ __forceinline__ f32x4 mma_split(f32x4 acc, SplitFrag a, SplitFrag b) {
  acc = mma<bf16_t>(acc, a.l, b.h);
  acc = mma<bf16_t>(acc, a.h, b.l);
  return mma<bf16_t>(acc, a.h, b.h);
}
// B exact in bf16 (an input): lo.B + hi.B
__device__ __forceinline__ f32x4 mma_split_exact(f32x4 acc, SplitFrag a, Frag b) {
  acc = mma<bf16_t>(acc, a.l, b);
  return mma<bf16_t>(acc, a.h, b);
}

// hi and lo of 8 values as two bf16 fragments, the values in the fragment's
// element order (hi = bf16(x), lo = bf16(x - hi), as split_frag forms them)
__device__ __forceinline__ void split8(const float* x, u32x4& h, u32x4& l) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t a, b;
    split_pair_bf16(x[2 * p], x[2 * p + 1], a, b);
    h[p] = a;
    l[p] = b;
  }
}
// A operand `a` as a split pair read from a split record: the two tiles' 16
// bytes are the hi and lo fragments
__device__ __forceinline__ SplitFrag rec_pair(f32x4 hi, f32x4 lo) {
  return SplitFrag{Frag{__builtin_bit_cast(u32x4, hi)}, Frag{__builtin_bit_cast(u32x4, lo)}};
}

// ============================================================ prep
// threads of the prep kernel (its LDS keeps one workgroup per CU at dk = 128:
// two waves per SIMD hide part of each one's latencies)
constexpr int kPThreads = 512;

template <typename T, int DK, bool RS>
__global__ __launch_bounds__(kPThreads) void chunk_bwd_prep_kernel(const T* q, const T* k, const T* alpha,
                                                                   const T* beta, float* __restrict__ rec, int T_len,
                                                                   int nchunks, long long total) {
  constexpr int C = kBC, CP = C + 1;
  using R = BwdRec<DK>;
  // One buffer holds, in turn, the staged q, k and alpha, then (split record)
  // QG and KR, then the rescaled rows of the five halving levels (per level
  // 16 x, 16 query and 16 y rows), then B21 T11, all in rows of XP floats,
  // 16-byte aligned for 4-channel accesses: the staged rows are read once,
  // into the channel threads' registers and the diagonal of M, before
  // anything else is written there.
  constexpr int XP = DK + 4;
  static_assert(C == 32, "five halving levels of 16-row tiles");
  static_assert(3 * C <= 5 * 3 * 16, "the staged rows fit the level rows' buffer");
  __shared__ __align__(16) float slev[5 * 3 * 16 * XP];
  float* const sq = slev;
  float* const sk = slev + C * XP;
  float* const sa = slev + 2 * C * XP;
  float* const sqg = slev;
  float* const skr = slev + C * XP;
  // (split record) KG, kept for K~G = TB KG
  __shared__ __align__(16) float skg[RS ? C * XP : 1];
  // S in 16-byte aligned rows (the block solve reads them four at a time)
  constexpr int SP = C + 4;
  __shared__ __align__(16) float sS[C * SP], sb[C];
  __shared__ float sM[C * CP], sT[C * CP];

  const int tid = threadIdx.x;
  // A persistent loop over chunks blockIdx.x, + gridDim.x, ...: each chunk's
  // inputs are fetched, as stored and at in-bounds addresses, while the
  // previous chunk is computed, and the barriers wait for LDS traffic only
  // (the kernel reads no global memory that it writes), so the fetch and the
  // record stores stay in flight across them.
  // Thread tid fetches the 8 consecutive channels 8 tid ... of row 8 tid / DK
  // of q, k and alpha (16 bytes each in bf16) and beta of row tid.
  static_assert(C * DK <= 8 * kPThreads && DK % 8 == 0, "one group of 8 channels per thread");
  struct alignas(16) G8 {
    T v[8];
  };
  G8 xq, xk, xa;   // the fetched chunk's q, k and alpha
  T xb;            // and beta
  auto fetch = [&](long long chunk) __attribute__((always_inline)) {
    const long long bh = chunk / nchunks;
    const int c = (int)(chunk % nchunks), t0 = c * C, cv = min(C, T_len - t0);
    const long long row0 = bh * (long long)T_len + t0;
    const int t = 8 * tid / DK, ch = 8 * tid % DK;
    const size_t gi = 8 * tid < C * DK && t < cv ? (size_t)(row0 + t) * DK + ch : 0;
    xq = *reinterpret_cast<const G8*>(q + gi);
    xk = *reinterpret_cast<const G8*>(k + gi);
    xa = *reinterpret_cast<const G8*>(alpha + gi);
    xb = beta[row0 + (tid < cv ? tid : 0)];
  };
  if (blockIdx.x < total) fetch(blockIdx.x);
  for (long long chunk = blockIdx.x; chunk < total; chunk += gridDim.x) {
    // (the thread index, hidden from the optimiser per chunk: its many derived
    // offsets are recomputed in each chunk rather than held across the loop)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int cv = min(C, T_len - (int)(chunk % nchunks) * C);
    // rows past a ragged end are identity steps: gate 1, no key, query or beta
    if (8 * tid < C * DK) {
      const int t = 8 * tid / DK, o = t * XP + 8 * tid % DK;
      const bool ok = t < cv;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 vq, vk, va;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vq[e] = ok ? to_f32(xq.v[4 * hf + e]) : 0.f;
          vk[e] = ok ? to_f32(xk.v[4 * hf + e]) : 0.f;
          va[e] = ok ? to_f32(xa.v[4 * hf + e]) : 1.f;
        }
        *reinterpret_cast<f32x4*>(sq + o + 4 * hf) = vq;
        *reinterpret_cast<f32x4*>(sk + o + 4 * hf) = vk;
        *reinterpret_cast<f32x4*>(sa + o + 4 * hf) = va;
      }
    }
    if (tid < C) sb[tid] = tid < cv ? to_f32(xb) : 0.f;
    for (int e = tid; e < C * SP; e += kPThreads) {
      sS[e] = 0.f;
      if (e < C * CP) sM[e] = 0.f;
    }
    lds_barrier();
    if (chunk + gridDim.x < total) fetch(chunk + gridDim.x);   // the next chunk's inputs, under this one's work

    float* rc = rec + (size_t)chunk * R::FLOATS;
    // this thread's channel (tid < DK): its gate, key and query columns in
    // registers for the sequential products below (the staged rows' only read
    // besides the diagonal of M)
    float ca[C], ck[C], cq[C];
    if (tid < DK) {
#pragma unroll
      for (int t = 0; t < C; ++t) {
        ca[t] = sa[t * XP + tid];
        ck[t] = sk[t * XP + tid];
        cq[t] = sq[t * XP + tid];
      }
    }
    {   // diagonal of M (G = 1): kPThreads / C threads per row
      constexpr int TPE = kPThreads / C;
      static_assert(TPE <= 64 && DK % TPE == 0, "row groups within a wave");
      const int t = tid / TPE, sub = tid % TPE;
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < DK / TPE; ++i) d += sq[t * XP + sub + i * TPE] * sk[t * XP + sub + i * TPE];
      d = group_sum<TPE>(d);
      if (sub == 0) sM[t * CP + t] = d;
    }
    lds_barrier();   // the staged rows are read: their buffer is rewritten below
    if (tid < DK) {   // per channel: Gamma, KG, QG, Gamma_C; G(C-1, j), KR
      const int ch = tid;
      float gm = 1.f, kg[4], qg[4];
#pragma unroll
      for (int t = 0; t < C; ++t) {
        gm *= ca[t];
        kg[t % 4] = ck[t] * gm;
        qg[t % 4] = cq[t] * gm;
        if constexpr (RS) {   // to LDS; all threads write the split record below
          skg[t * XP + ch] = kg[t % 4];
          sqg[t * XP + ch] = qg[t % 4];
        } else {
          rc[R::KG_OFF + frag_off(t, ch, DK)] = kg[t % 4];
          if (t % 4 == 3) {   // KG^T, QG^T: this channel's rows, 16 bytes at a time
            *reinterpret_cast<f32x4*>(rc + R::KGT_OFF + frag_off(ch, t - 3, C)) = f32x4{kg[0], kg[1], kg[2], kg[3]};
            *reinterpret_cast<f32x4*>(rc + R::QGT_OFF + frag_off(ch, t - 3, C)) = f32x4{qg[0], qg[1], qg[2], qg[3]};
          }
        }
      }
      rc[R::GC_OFF + ch] = gm;
      float ge = 1.f, kr[4];
#pragma unroll
      for (int t = C - 1; t >= 0; --t) {
        kr[t % 4] = ck[t] * ge;
        ge *= ca[t];
        if constexpr (RS) {
          skr[t * XP + ch] = kr[t % 4];
        } else {
          rc[R::KR_OFF + frag_off(t, ch, DK)] = kr[t % 4];
          if (t % 4 == 0)   // KR^T: this channel's row
            *reinterpret_cast<f32x4*>(rc + R::KRT_OFF + frag_off(ch, t, C)) = f32x4{kr[0], kr[1], kr[2], kr[3]};
        }
      }
    }
    // S and M below the diagonal by recursive halving.  Level h (16, 8, 4, 2,
    // 1) splits the chunk into blocks of 2h positions around their midpoints
    // m: entry (t, j) with t in the upper and j in the lower half of one block
    // is sum over channels of (x_t G(t, m)) (y_j G(m, j)), every factor a
    // product of at most h gates.  The channel threads write each level's
    // rescaled rows; each level is then two 16 x 16 products over the channels
    // (rows u = block * h + offset in the half: S from the x rows, M from the
    // query rows, both against the y rows), on fp32 matrix cores, of which the
    // blocks' h x h diagonal quadrants are the level's entries.  Levels 4, 2
    // and 1 sit past QG and KR in the shared buffer: their rows are written
    // while the other waves write the split record, and their products run
    // while the rows of levels 16 and 8 are written over QG and KR.
    {
      constexpr int CW = (DK + 63) / 64;   // the waves that hold channel threads
      static_assert(kPThreads / 64 - CW >= 6, "six whole waves beside the channel threads");
      const int wv = tid >> 6, ln = tid & 63, rr = ln & 15, gg = ln >> 4;
      auto rescale = [&](auto ll) __attribute__((always_inline)) {   // level ll's rows (channel threads)
        constexpr int L = decltype(ll)::value, h = (C / 2) >> L;
        const int ch = tid;
        float* X = slev + L * 3 * 16 * XP;
#pragma unroll
        for (int lo = 0; lo < C; lo += 2 * h) {
          const int m = lo + h - 1, u0 = lo / 2;
          float f = 1.f;
#pragma unroll
          for (int t = m + 1; t <= m + h; ++t) {   // x_t G(t, m)
            f *= ca[t];
            X[(u0 + t - m - 1) * XP + ch] = ck[t] * f;
            X[(16 + u0 + t - m - 1) * XP + ch] = cq[t] * f;
          }
          float e = 1.f;
#pragma unroll
          for (int j = m; j >= lo; --j) {          // y_j G(m, j)
            X[(32 + u0 + j - lo) * XP + ch] = ck[j] * e;
            e *= ca[j];
          }
        }
      };
      // tile tt (level tt / 2; S for even tt, M for odd) by one whole wave:
      // lane (g, r) takes the 16-byte channel groups 16 s + 4 g of row r of
      // both operands, K step e of group s being channel 16 s + 4 g + e
      auto tile = [&](int tt) __attribute__((always_inline)) {
        const int L = tt >> 1, h = (C / 2) >> L;
        const float* A = slev + (L * 3 + (tt & 1)) * 16 * XP + rr * XP + 4 * gg;
        const float* B = slev + (L * 3 + 2) * 16 * XP + rr * XP + 4 * gg;
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < DK / 16; ++s) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(A + 16 * s);
          const f32x4 b = *reinterpret_cast<const f32x4*>(B + 16 * s);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
        }
        // lane (g, r) holds entries (4 g + e, r): x row 4 g + e against y row r
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ut = 4 * gg + e, blk = ut / h;
          if (blk == rr / h) {
            const int lo = 2 * h * blk, t = lo + h + ut % h, j = lo + rr % h;
            if (tt & 1) sM[t * CP + j] = acc[e];
            else sS[t * SP + j] = acc[e];
          }
        }
      };
      if constexpr (RS) lds_barrier();   // KG, QG and KR are in LDS
      if (tid < DK) {
        rescale(std::integral_constant<int, 2>{});
        rescale(std::integral_constant<int, 3>{});
        rescale(std::integral_constant<int, 4>{});
      } else if constexpr (RS) {
        // KG, KR (C x DK) and QG^T, KR^T (DK x C) as split fragment pairs,
        // the threads past the channel waves writing whole 16-byte hi and lo
        // fragments: a task is one lane of one pair (row tile rt, K block kb)
        // of one field.  (Barriers for the LDS data only: the record stores
        // drain meanwhile.)
        constexpr int NT = 4 * DK;   // tasks per field: 64 lanes x (2 (DK / 32) pairs, or DK / 16)
        constexpr int NWT = kPThreads - 64 * CW;
        static_assert(NT % 64 == 0 && NWT % 64 == 0, "whole waves per field");
        const int wt = tid - 64 * CW;
#pragma unroll
        for (int i = 0; i < (4 * NT + NWT - 1) / NWT; ++i) {
          const int task0 = wt + i * NWT, f0 = task0 / NT;
          // fields 0 KG, 1 KR, 3 QG^T, 4 KR^T (2, KG^T, is replaced by -K~G^T below)
          const int field = f0 < 2 ? f0 : f0 + 1, task = task0 + (f0 < 2 ? 0 : NT);
          const int pair = (task % NT) / 64, ln = task % 64;
          if (task0 >= 4 * NT) break;
          const int gg = ln >> 4, rr = ln & 15;
          float v8[8];
          int off, kd, rt, kb;
          // (one LDS array per call: a pointer chosen at run time would be a flat access)
          auto rows = [&](const float* src) __attribute__((always_inline)) {   // row t, K = channels
            const float* row = src + (16 * rt + rr) * XP + 32 * kb;
            const f32x4 a = *reinterpret_cast<const f32x4*>(row + 4 * gg), b = *reinterpret_cast<const f32x4*>(row + 16 + 4 * gg);
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              v8[e] = a[e];
              v8[4 + e] = b[e];
            }
          };
          auto cols = [&](const float* src) __attribute__((always_inline)) {   // row = channel, K = positions
  #pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = src[kappa<bf16_t>(gg, e) * XP + 16 * rt + rr];
          };
          if (field < 2) {   // KG, KR
            rt = pair / (DK / 32);
            kb = pair % (DK / 32);
            off = field == 0 ? R::KG_OFF : R::KR_OFF;
            kd = DK;
            if (field == 0) rows(skg);
            else rows(skr);
          } else {           // KG^T, QG^T, KR^T
            rt = pair;
            kb = 0;
            off = field == 2 ? R::KGT_OFF : field == 3 ? R::QGT_OFF : R::KRT_OFF;
            kd = C;
            if (field == 3) cols(sqg);
            else cols(skr);
          }
          u32x4 h, l;
          split8(v8, h, l);
          float* tile = rc + off + (rt * (kd / 16) + 2 * kb) * 256 + 4 * ln;
          *reinterpret_cast<u32x4*>(tile) = h;
          *reinterpret_cast<u32x4*>(tile + 256) = l;
        }
      }
      lds_barrier();   // the rows of levels 4, 2 and 1 are written; QG and KR are read
      if (tid < DK) {
        rescale(std::integral_constant<int, 0>{});
        rescale(std::integral_constant<int, 1>{});
      } else if (wv >= CW && wv < CW + 6) {
        tile(4 + wv - CW);
      }
      lds_barrier();
      if (wv < 4) tile(wv);   // levels 16 and 8
      lds_barrier();
    }
    // T = (I + B)^-1, B = Diag(beta) S strictly lower, unit lower triangular,
    // by 16 x 16 blocks: the diagonal blocks T11 = (I + B11)^-1 and
    // T22 = (I + B22)^-1 by forward substitution, one column per thread held in
    // registers (T[i][j] = -beta_i sum_{l < i} S[i][l] T[l][j] for i > j; each
    // row of S is read as the solve reaches it, 16 bytes at a time and the
    // same by every lane), then T21 = -T22 (B21 T11) as two 16 x 16 products,
    // one entry per thread.  Meanwhile the waves past the first store S and
    // M^T, which are final, to the record.
    constexpr int HB = C / 2;
    static_assert(HB % 4 == 0, "whole 16-byte groups per block row");
    if (tid < C) {
      const int o = (tid / HB) * HB, j = tid % HB;   // the block's first row, the column in it
      f32x4 bq[HB / 4];
#pragma unroll
      for (int v = 0; v < HB / 4; ++v) bq[v] = *reinterpret_cast<const f32x4*>(sb + o + 4 * v);
      float tc[HB];
#pragma unroll
      for (int i = 0; i < HB; ++i) {
        f32x4 srow[HB / 4];   // S(o + i, o + 4 v ...), v <= (i - 1) / 4
#pragma unroll
        for (int v = 0; v < (i + 3) / 4; ++v) srow[v] = *reinterpret_cast<const f32x4*>(sS + (o + i) * SP + o + 4 * v);
        float acc = 0.f;
#pragma unroll
        for (int l = 0; l < i; ++l) acc += srow[l / 4][l % 4] * tc[l];
        tc[i] = i > j ? -bq[i / 4][i % 4] * acc : (i == j ? 1.f : 0.f);
      }
#pragma unroll
      for (int i = 0; i < HB; ++i) sT[(o + i) * CP + o + j] = tc[i];
      if (o == 0)
#pragma unroll
        for (int i = 0; i < HB; ++i) sT[i * CP + HB + j] = 0.f;   // T12
    } else if (tid >= 64) {
      if constexpr (RS) {
        if (tid < 3 * 64) {   // M^T as split pairs: 2 row tiles x 64 lanes
          const int rt = tid / 64 - 1, ln = tid % 64, gg = ln >> 4, i = 16 * rt + (ln & 15);
          float v8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = sM[kappa<bf16_t>(gg, e) * CP + i];
          u32x4 h, l;
          split8(v8, h, l);
          float* tile = rc + R::MT_OFF + (rt * (C / 16)) * 256 + 4 * ln;
          *reinterpret_cast<u32x4*>(tile) = h;
          *reinterpret_cast<u32x4*>(tile + 256) = l;
        } else {
          for (int e = tid - 3 * 64; e < C * C; e += kPThreads - 3 * 64) rc[R::S_OFF + e] = sS[(e / C) * SP + e % C];
        }
      } else {
        for (int e = tid - 64; e < C * C; e += kPThreads - 64) {
          const int i = e / C, j = e % C;
          rc[R::MT_OFF + frag_off(i, j, C)] = sM[j * CP + i];
          rc[R::S_OFF + e] = sS[i * SP + j];
        }
      }
    }
    lds_barrier();
    float* sW = slev;   // B21 T11 (the level rows are consumed)
    if (tid < HB * HB) {
      const int i = tid / HB, j = tid % HB;
      float acc = 0.f;
#pragma unroll
      for (int l = 0; l < HB; ++l) acc += sS[(HB + i) * SP + l] * sT[l * CP + j];
      sW[i * HB + j] = sb[HB + i] * acc;
    }
    lds_barrier();
    if (tid < HB * HB) {
      const int i = tid / HB, j = tid % HB;
      float acc = 0.f;
#pragma unroll
      for (int l = 0; l < HB; ++l) acc += sT[(HB + i) * CP + HB + l] * sW[l * HB + j];
      sT[(HB + i) * CP + j] = -acc;
    }
    lds_barrier();
    if constexpr (RS) {
      // -K~G^T, K~G = TB KG, on fp32 matrix cores straight from T, beta and KG
      // in LDS: the accumulator tiles of positions 0-15 and 16-31 of channel
      // tile ct are, element by element, the fragment of row tile ct of K~G^T
      // (K = positions in kappa order), split and stored as a pair
      const int wv = tid >> 6, ln = tid & 63, rr = ln & 15, gg = ln >> 4;
      for (int ct = wv; ct < DK / 16; ct += kPThreads / 64) {
        f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
        for (int st = 0; st < C / 4; ++st) {
          const int kk = 4 * st + gg;   // lane (g, r) supplies A(r, k) and B(k, r) of K step k = 4 st + g
          const float bk = skg[kk * XP + 16 * ct + rr], bt = sb[kk];
#pragma unroll
          for (int pt = 0; pt < 2; ++pt)
            acc[pt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * pt + rr) * CP + kk] * bt, bk, acc[pt], 0, 0, 0);
        }
        float v8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v8[e] = -acc[0][e];
          v8[4 + e] = -acc[1][e];
        }
        u32x4 h, l;
        split8(v8, h, l);
        float* tile = rc + R::KGT_OFF + (ct * (C / 16)) * 256 + 4 * ln;
        *reinterpret_cast<u32x4*>(tile) = h;
        *reinterpret_cast<u32x4*>(tile + 256) = l;
      }
    }
    for (int e = tid; e < C * C; e += kPThreads) {
      const int i = e / C, j = e % C;
      if constexpr (!RS) {
        const int fo = frag_off(i, j, C);
        rc[R::TB_OFF + fo] = sT[i * CP + j] * sb[j];
        rc[R::TBT_OFF + fo] = sT[j * CP + i] * sb[i];
      }
      rc[R::T_OFF + e] = sT[i * CP + j];
    }
    if constexpr (RS) {   // TB as split pairs: 2 row tiles, one K block, 64 lanes each
      if (tid < 2 * 64) {
        // the rounded product T beta is split: its lo part is not the exact
        // product's, which fusing it into the split's subtraction would give
#pragma clang fp contract(off)
        const int rt = tid / 64, ln = tid % 64, gg = ln >> 4, i = 16 * rt + (ln & 15);
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = kappa<bf16_t>(gg, e);
          v8[e] = sT[i * CP + j] * sb[j];
        }
        u32x4 h, l;
        split8(v8, h, l);
        float* tile = rc + R::TB_OFF + (rt * (C / 16)) * 256 + 4 * ln;
        *reinterpret_cast<u32x4*>(tile) = h;
        *reinterpret_cast<u32x4*>(tile + 256) = l;
      }
    }
    lds_barrier();   // the next chunk's staging rewrites the LDS operands
  }
}

// ============================================================ states (forward, sequential)
// float offset, within a chunk's dk x dv state block, of element (i, j) as the
// states kernel writes it (value slices of 16 columns, each in accumulator
// order)
template <int DK>
__device__ __forceinline__ int hc_slot(int i, int j) {
  return (j / 16) * (DK * 16) + ((i / 16) * 64 + ((i % 16) / 4) * 16 + j % 16) * 4 + i % 4;
}

// 16 bytes at a wave-uniform float address plus a per-lane byte offset: the
// address form with a scalar base and a 32-bit lane offset, so that no 64-bit
// address arithmetic is done per lane
__device__ __forceinline__ f32x4 ld16(const float* base, uint32_t boff) {
  return *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(base) + boff);
}
__device__ __forceinline__ void st16(float* base, uint32_t boff, f32x4 x) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(base) + boff) = x;
}

// One wave per head and NS 16-column value slices (NS = 1 or 2), each
// slice's state (dk x 16) in its accumulator registers, as the forward's state
// pass keeps it: per chunk
//   X = V - KG H,  U = TB X,  H <- Gamma_C . H + KR^T U
// on matrix cores, the accumulator tiles of one product being (with the K
// order 4 g + e of an fp32 fragment) the B operand of the next.  The A
// operands come straight from the chunk record (the slices of a head share it
// through their XCD's L2), every fragment one 16-byte load of a KG, TB or
// KR^T row, and serve all NS slices: the kernel moves its record through each
// CU's vector memory path, whose throughput for L2 hits bounds it once two
// workgroups share a CU, so two slices per wave halve those bytes (and the
// two slices' independent chains fill each other's latency; the launcher
// takes two with split products only).  Each operand is
// loaded for the next chunk as soon as the current chunk has used it (KR^T and
// Gamma_C, used last, at the top of their own chunk), so the loads run under
// the matrix-core work without a second register set; the next chunk's loads
// are unconditional (the last chunk reloads itself), which keeps them in one
// basic block.  No LDS and no barrier.
//
// The chunk-start states go out in accumulator order: per chunk and slice a
// dk x 16 block, the f32x4 of lane l of row tile rh at float (64 rh + l) 4,
// holding rows 16 rh + 4 (l / 16) + i, column l % 16 (hc_slot).
template <typename T, int DK, bool RS, int NS>
__global__ __launch_bounds__(64) void chunk_bwd_states_kernel(const T* v, const float* __restrict__ h0,
                                                              const float* __restrict__ rec, float* __restrict__ hc,
                                                              int T_len, int nchunks, int dv, int xcd_map) {
  constexpr int C = kBC, RH = DK / 16, RT = C / 16;
  constexpr bool SPLIT = kSplitSeq<T, DK>;
  static_assert(RT == 2, "one 32-position K block per chunk");
  static_assert(NS == 1 || NS == 2, "one or two slices per wave");
  using R = BwdRec<DK>;
  const int lane = threadIdx.x, g = lane >> 4, r = lane & 15;
  long long bh;
  int sg;
  head_slice(blockIdx.x, dv / (16 * NS), xcd_map, bh, sg);
  const int slice0 = sg * NS;         // the wave's first slice
  const int col0 = slice0 * 16 + r;   // this lane's value column in it (slice s: + 16 s)
  f32x4 hacc[NS][RH];   // H rows 16 rh + 4 g + i, column col0 + 16 s
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int rh = 0; rh < RH; ++rh)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hacc[s][rh][i] = h0 ? h0[(bh * DK + 16 * rh + 4 * g + i) * (long long)dv + col0 + 16 * s] : 0.f;
  f32x4 kg[RT][RH];   // KG rows 16 rt + r, channels 16 kb + 4 g .. + 3
  f32x4 kr[RH][RT];   // KR^T rows 16 rh + r (channels), positions 16 kb + 4 g .. + 3
  f32x4 tb[RT][RT];   // TB rows 16 rt + r, positions 16 kb + 4 g .. + 3 (kb <= rt)
  f32x4 gc[RH];       // Gamma_C at channels 16 rh + 4 g .. + 3
  T vv[NS][RT][4];    // V rows 16 rt + 4 g .. + 3, column col0 + 16 s, as stored (rows past the end: 0 or any row)
  const uint32_t v_boff = (uint32_t)((4 * g * dv + col0) * sizeof(T));
  const uint32_t lboff = 16u * lane;   // this lane's 16 bytes of a fragment tile
  auto recp = [&](int c) { return rec + (size_t)(bh * nchunks + c) * R::FLOATS; };
  auto load_kg = [&](int c) __attribute__((always_inline)) {
    const float* rc = recp(c);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kb = 0; kb < RH; ++kb)
        kg[rt][kb] = ld16(rc + R::KG_OFF + (rt * (DK / 16) + kb) * 256, lboff);
  };
  auto load_tb_v = [&](int c) __attribute__((always_inline)) {
    const float* rc = recp(c);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kb = 0; kb < (RS ? RT : rt + 1); ++kb)   // (a split record: both halves of every pair)
        tb[rt][kb] = ld16(rc + R::TB_OFF + (rt * RT + kb) * 256, lboff);
    // V rows kept as stored, so that nothing waits for them before the next
    // chunk.  With split products: row 16 rt + i of the chunk at a uniform base
    // plus this lane's byte offset (rows 4 g and its column), rows past the end
    // (last chunk only) read as 0; with fp32 products that form came out slower
    // (389 -> 474 us at the bench shape), and every row's address is formed
    // per element, a row past the end reading the chunk's first row and masked
    // where it is used.
    const int t0 = c * C, cv = min(C, T_len - t0);
    const T* vc = v + ((size_t)bh * T_len + t0) * dv;
    if constexpr (!SPLIT) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * rt + 4 * g + i;
            vv[s][rt][i] = v[(size_t)(bh * T_len + t0 + (t < cv ? t : 0)) * dv + col0 + 16 * s];
          }
    } else if (cv == C) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vv[s][rt][i] = *reinterpret_cast<const T*>(reinterpret_cast<const char*>(vc + (size_t)(16 * rt + i) * dv) +
                                                       v_boff + 16 * s * sizeof(T));
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vv[s][rt][i] = 16 * rt + 4 * g + i < cv ? vc[(size_t)(16 * rt + 4 * g + i) * dv + col0 + 16 * s] : T{};
    }
  };
  auto load_kr_gc = [&](int c) __attribute__((always_inline)) {
    const float* rc = recp(c);
#pragma unroll
    for (int rh = 0; rh < RH; ++rh)
#pragma unroll
      for (int kb = 0; kb < RT; ++kb)
        kr[rh][kb] = ld16(rc + R::KRT_OFF + (rh * RT + kb) * 256, lboff);
#pragma unroll
    for (int rh = 0; rh < RH; ++rh) gc[rh] = ld16(rc + R::GC_OFF + 16 * rh, 16u * g);
  };
  if (nchunks > 0) {
    load_kg(0);
    load_tb_v(0);
  }
  for (int c = 0; c < nchunks; ++c) {
    const long long chunk = bh * nchunks + c;
    const int cn = min(c + 1, nchunks - 1);
    // KR^T and Gamma_C, then the chunk-start state (the vector memory counter
    // drains in issue order: loads issued after the stores would make the
    // update's wait for them a wait for the stores too)
    load_kr_gc(c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int rh = 0; rh < RH; ++rh)   // (hc_slot order)
        st16(hc + (size_t)chunk * DK * dv + (slice0 + s) * (DK * 16) + rh * 256, lboff, hacc[s][rh]);
    // (scheduling barriers keep each group of loads where it is written: the
    // scheduler would otherwise sink them toward their uses)
    __builtin_amdgcn_sched_barrier(0);
    // X = V - KG H
    f32x4 xacc[NS][RT];
    SplitFrag hs[NS][SPLIT ? RH / 2 : 1];
    if constexpr (SPLIT)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < RH / 2; ++j) hs[s][j] = split_frag(hacc[s][2 * j], hacc[s][2 * j + 1]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 p[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) p[s] = zero4();
      if constexpr (SPLIT) {
#pragma unroll
        for (int j = 0; j < RH / 2; ++j) {
          const SplitFrag a = RS ? rec_pair(kg[rt][2 * j], kg[rt][2 * j + 1]) : split_frag(kg[rt][2 * j], kg[rt][2 * j + 1]);
#pragma unroll
          for (int s = 0; s < NS; ++s) p[s] = mma_split(p[s], a, hs[s][j]);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < RH; ++kb)
#pragma unroll
          for (int s = 0; s < NS; ++s)
            p[s] = mma<float>(p[s], Frag{__builtin_bit_cast(u32x4, kg[rt][kb])}, frag_from_acc_f32(hacc[s][kb]));
      }
      // (rows past the end: V read as 0 or masked here, and no key, so X is 0)
      const int cvx = min(C, T_len - c * C);
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xacc[s][rt][i] = (SPLIT || 16 * rt + 4 * g + i < cvx ? to_f32(vv[s][rt][i]) : 0.f) - p[s][i];
    }
    __builtin_amdgcn_sched_barrier(0);
    load_kg(cn);
    __builtin_amdgcn_sched_barrier(0);
    // U = TB X
    f32x4 uacc[NS][RT];
    if constexpr (SPLIT) {
      SplitFrag xs[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) xs[s] = split_frag(xacc[s][0], xacc[s][1]);
      // TB is lower triangular
      const SplitFrag t0 = RS ? rec_pair(tb[0][0], tb[0][1]) : split_frag(tb[0][0], zero4());
      const SplitFrag t1 = RS ? rec_pair(tb[1][0], tb[1][1]) : split_frag(tb[1][0], tb[1][1]);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        uacc[s][0] = mma_split(zero4(), t0, xs[s]);
        uacc[s][1] = mma_split(zero4(), t1, xs[s]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          uacc[s][rt] = zero4();
#pragma unroll
          for (int kb = 0; kb <= rt; ++kb)
            uacc[s][rt] =
                mma<float>(uacc[s][rt], Frag{__builtin_bit_cast(u32x4, tb[rt][kb])}, frag_from_acc_f32(xacc[s][kb]));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_tb_v(cn);
    __builtin_amdgcn_sched_barrier(0);
    // H <- Gamma_C . H + KR^T U
    SplitFrag us[NS];
    if constexpr (SPLIT)
#pragma unroll
      for (int s = 0; s < NS; ++s) us[s] = split_frag(uacc[s][0], uacc[s][1]);
#pragma unroll
    for (int rh = 0; rh < RH; ++rh) {
      if constexpr (SPLIT) {
        const SplitFrag a = RS ? rec_pair(kr[rh][0], kr[rh][1]) : split_frag(kr[rh][0], kr[rh][1]);
#pragma unroll
        for (int s = 0; s < NS; ++s) hacc[s][rh] = mma_split(gc[rh] * hacc[s][rh], a, us[s]);
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          f32x4 hh = gc[rh] * hacc[s][rh];
#pragma unroll
          for (int kb = 0; kb < RT; ++kb)
            hh = mma<float>(hh, Frag{__builtin_bit_cast(u32x4, kr[rh][kb])}, frag_from_acc_f32(uacc[s][kb]));
          hacc[s][rh] = hh;
        }
      }
    }
  }
}

// ============================================================ dstates (reverse, sequential)
// One workgroup per head and NS 16-column value slices (NS = 1 or 2), its NW
// waves splitting the key channels: each holds dk / NW rows of the state
// gradient (x 16 columns, per slice) in accumulator registers.  Per chunk,
// from the last:
//   dU = M^T dO + KR dH',  dX = TB^T dU,  dH = Gamma_C . dH' + QG^T dO - KG^T dX
// on matrix cores, accumulator tiles feeding the next product as B operands.
// Each wave's KR dH' covers its own channels; the waves' partial dU are
// summed through LDS (one barrier per chunk, the exchange buffer alternating
// between chunks), in the same order in every wave, so all waves hold the
// same dU (with two waves, a + b = b + a).  Every A fragment is one 16-byte
// load of a record row and serves all NS slices; dO's fragments are four
// loads of the input each, kept as stored until used.  Operands are reloaded
// for the next chunk as soon as the current one has used them (KR, M^T and
// dO, needed first, into the other of two sets).  The state gradient entering
// each chunk from its end (dH') is stored in accumulator order (hc_slot), dh0
// at the end.  The kernel moves its record through each CU's vector memory
// path, which bounds it at two workgroups per CU; at the bench shape four
// waves of two slices each make one workgroup per CU with each wave's work
// unchanged.
template <int DK>
constexpr int kDsWaves = DK >= 32 ? 2 : 1;

template <typename T, int DK, bool RS, int NW, int NS>
__global__ __launch_bounds__(64 * NW) void chunk_bwd_dstates_kernel(const T* dout, const float* __restrict__ dhT,
                                                                   const float* __restrict__ rec,
                                                                   float* __restrict__ dhn, float* __restrict__ dh0,
                                                                   int T_len, int nchunks, int dv, int xcd_map) {
  constexpr int C = kBC, RHW = DK / 16 / NW, RT = C / 16;
  constexpr bool SPLIT = kSplitSeq<T, DK>;
  static_assert(RT == 2 && RHW >= 1 && (!SPLIT || RHW % 2 == 0), "32-position K blocks; whole 32-channel blocks per wave");
  static_assert(NS == 1 || NS == 2, "one or two slices per workgroup");
  using R = BwdRec<DK>;
  __shared__ f32x4 xb[2][NW][NS][RT][64];   // partial dU of each wave, by chunk parity
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  long long bh;
  int sg;
  head_slice(blockIdx.x, dv / (16 * NS), xcd_map, bh, sg);
  const int slice0 = sg * NS;         // the first slice
  const int col0 = slice0 * 16 + r;   // this lane's value column in it (slice s: + 16 s)
  const int rb = wave * RHW;          // the wave's first row tile
  f32x4 dacc[NS][RHW];                // dH rows 16 (rb + rh) + 4 g + i, column col0 + 16 s
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int rh = 0; rh < RHW; ++rh)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dacc[s][rh][i] = dhT ? dhT[(bh * DK + 16 * (rb + rh) + 4 * g + i) * (long long)dv + col0 + 16 * s] : 0.f;
  struct First {          // needed first in a chunk
    f32x4 kr[RT][RHW];    // KR rows 16 rt + r, channels 16 (rb + kb) + 4 g .. + 3
    f32x4 mt[RT][RT];     // M^T rows 16 rt + r, positions 16 kb + 4 g .. + 3 (kb >= rt)
    T dov[NS][RT][4];     // dO rows 16 kb + 4 g + e, column col0 + 16 s, as stored (rows past the end: any row)
  };
  f32x4 tbt[RT][RT];    // TB^T rows 16 rt + r, positions 16 kb + 4 g .. + 3 (kb >= rt)
  f32x4 qgt[RHW][RT];   // QG^T rows 16 (rb + rh) + r, positions 16 kb + 4 g .. + 3
  f32x4 kgt[RHW][RT];   // KG^T likewise
  f32x4 gc[RHW];        // Gamma_C at channels 16 (rb + rh) + 4 g .. + 3
  auto recp = [&](int c) { return rec + (size_t)(bh * nchunks + c) * R::FLOATS; };
  auto load_first = [&](First& o, int c) __attribute__((always_inline)) {
    const float* rc = recp(c);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kb = 0; kb < RHW; ++kb)
        o.kr[rt][kb] = *reinterpret_cast<const f32x4*>(rc + R::KR_OFF + (rt * (DK / 16) + rb + kb) * 256 + 4 * lane);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kb = RS ? 0 : rt; kb < RT; ++kb)   // (a split record: both halves of every pair)
        o.mt[rt][kb] = *reinterpret_cast<const f32x4*>(rc + R::MT_OFF + (rt * RT + kb) * 256 + 4 * lane);
    const int t0 = c * C, cv = min(C, T_len - t0);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < RT; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * kb + 4 * g + e;
          o.dov[s][kb][e] = dout[(size_t)(bh * T_len + t0 + (t < cv ? t : 0)) * dv + col0 + 16 * s];
        }
  };
  auto load_tbt = [&](int c) __attribute__((always_inline)) {
    if constexpr (RS) return;   // TB^T is not read (and not written) with a split record
    const float* rc = recp(c);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kb = RS ? 0 : rt; kb < RT; ++kb)
        tbt[rt][kb] = *reinterpret_cast<const f32x4*>(rc + R::TBT_OFF + (rt * RT + kb) * 256 + 4 * lane);
  };
  auto load_last = [&](int c) __attribute__((always_inline)) {
    const float* rc = recp(c);
#pragma unroll
    for (int rh = 0; rh < RHW; ++rh)
#pragma unroll
      for (int kb = 0; kb < RT; ++kb) {
        qgt[rh][kb] = *reinterpret_cast<const f32x4*>(rc + R::QGT_OFF + ((rb + rh) * RT + kb) * 256 + 4 * lane);
        kgt[rh][kb] = *reinterpret_cast<const f32x4*>(rc + R::KGT_OFF + ((rb + rh) * RT + kb) * 256 + 4 * lane);
      }
#pragma unroll
    for (int rh = 0; rh < RHW; ++rh)
      gc[rh] = *reinterpret_cast<const f32x4*>(rc + R::GC_OFF + 16 * (rb + rh) + 4 * g);
  };
  // chunk c with the first-needed operands in `cur`, loading chunk c - 1's
  // into `nxt`; a step with live == false (past the first chunk) computes on
  // chunk 0 again and changes nothing
  auto step = [&](First& cur, First& nxt, int c, bool live) __attribute__((always_inline)) {
    // exchange buffer by the parity of the UNCLAMPED chunk index: the dead
    // step (c = -1) then writes buffer 1, last read before the live chunk-0
    // step's barrier, never buffer 0, which the other waves may still be
    // reading for chunk 0
    const int par = c & 1;
    c = max(c, 0);
    const long long chunk = bh * nchunks + c;
    const int cn = max(c - 1, 0);   // the next chunk processed (the first reloads itself)
    if (live)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rh = 0; rh < RHW; ++rh)   // dH'
          *reinterpret_cast<f32x4*>(dhn + (size_t)chunk * DK * dv +
                                    hc_slot<DK>(16 * (rb + rh) + 4 * g, col0 + 16 * s)) = dacc[s][rh];
    // (scheduling barriers keep each group of loads where it is written: the
    // scheduler would otherwise sink them toward their uses)
    __builtin_amdgcn_sched_barrier(0);
    load_first(nxt, cn);
    __builtin_amdgcn_sched_barrier(0);
    const int cv = min(C, T_len - c * C);
    f32x4 dof[NS][RT];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < RT; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dof[s][kb][e] = 16 * kb + 4 * g + e < cv ? to_f32(cur.dov[s][kb][e]) : 0.f;
    // dU = M^T dO (first wave) + KR dH' (each wave its channels), summed over the waves
    f32x4 du[NS][RT];
    Frag dob[NS];   // dO as bf16 (exact: the input)
    SplitFrag dhs[NS][SPLIT ? RHW / 2 : 1];
    if constexpr (SPLIT) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        dob[s] = frag_from_acc_bf16(dof[s][0], dof[s][1]);
#pragma unroll
        for (int j = 0; j < RHW / 2; ++j) dhs[s][j] = split_frag(dacc[s][2 * j], dacc[s][2 * j + 1]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (SPLIT) {   // M^T is upper triangular
        const SplitFrag am = RS ? rec_pair(cur.mt[rt][0], cur.mt[rt][1])
                                : split_frag(rt == 0 ? cur.mt[0][0] : zero4(), cur.mt[rt][1]);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f32x4 m = mma_split_exact(zero4(), am, dob[s]);
          du[s][rt] = wave == 0 ? m : zero4();
        }
#pragma unroll
        for (int j = 0; j < RHW / 2; ++j) {
          const SplitFrag ak = RS ? rec_pair(cur.kr[rt][2 * j], cur.kr[rt][2 * j + 1])
                                  : split_frag(cur.kr[rt][2 * j], cur.kr[rt][2 * j + 1]);
#pragma unroll
          for (int s = 0; s < NS; ++s) du[s][rt] = mma_split(du[s][rt], ak, dhs[s][j]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          f32x4 m = zero4();
#pragma unroll
          for (int kb = rt; kb < RT; ++kb)
            m = mma<float>(m, Frag{__builtin_bit_cast(u32x4, cur.mt[rt][kb])}, frag_from_acc_f32(dof[s][kb]));
          du[s][rt] = wave == 0 ? m : zero4();
#pragma unroll
          for (int kb = 0; kb < RHW; ++kb)
            du[s][rt] =
                mma<float>(du[s][rt], Frag{__builtin_bit_cast(u32x4, cur.kr[rt][kb])}, frag_from_acc_f32(dacc[s][kb]));
        }
      }
    }
    // the part of dH that does not wait for dX: Gamma_C . dH' + QG^T dO, issued
    // before the exchange so that it runs while the waves meet
    f32x4 hp[NS][RHW];
#pragma unroll
    for (int rh = 0; rh < RHW; ++rh) {
      if constexpr (SPLIT) {
        const SplitFrag aq = RS ? rec_pair(qgt[rh][0], qgt[rh][1]) : split_frag(qgt[rh][0], qgt[rh][1]);
#pragma unroll
        for (int s = 0; s < NS; ++s) hp[s][rh] = mma_split_exact(gc[rh] * dacc[s][rh], aq, dob[s]);
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          hp[s][rh] = gc[rh] * dacc[s][rh];
#pragma unroll
          for (int kb = 0; kb < RT; ++kb)
            hp[s][rh] = mma<float>(hp[s][rh], Frag{__builtin_bit_cast(u32x4, qgt[rh][kb])}, frag_from_acc_f32(dof[s][kb]));
        }
      }
    }
    if constexpr (NW > 1) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) xb[par][wave][s][rt][lane] = du[s][rt];
      __syncthreads();
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if constexpr (NW == 2) {
            du[s][rt] += xb[par][1 - wave][s][rt][lane];
          } else {   // the waves' parts in wave order, the same sum in every wave
            f32x4 a = xb[par][0][s][rt][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) a += xb[par][w][s][rt][lane];
            du[s][rt] = a;
          }
        }
    }
    if constexpr (RS) {
      // dH = Gamma_C . dH' + QG^T dO + (-K~G^T) dU: no dX on the chain
      SplitFrag dus[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) dus[s] = split_frag(du[s][0], du[s][1]);
#pragma unroll
      for (int rh = 0; rh < RHW; ++rh) {
        const SplitFrag ak = rec_pair(kgt[rh][0], kgt[rh][1]);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f32x4 h = mma_split(hp[s][rh], ak, dus[s]);
#pragma unroll
          for (int i = 0; i < 4; ++i) dacc[s][rh][i] = live ? h[i] : dacc[s][rh][i];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_last(cn);
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    // dX = TB^T dU, negated for the update below
    f32x4 ndx[NS][RT];
    if constexpr (SPLIT) {   // TB^T is upper triangular
      const SplitFrag t0 = split_frag(tbt[0][0], tbt[0][1]), t1 = split_frag(zero4(), tbt[1][1]);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const SplitFrag dus = split_frag(du[s][0], du[s][1]);
        ndx[s][0] = -mma_split(zero4(), t0, dus);
        ndx[s][1] = -mma_split(zero4(), t1, dus);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4 x = zero4();
#pragma unroll
          for (int kb = rt; kb < RT; ++kb)
            x = mma<float>(x, Frag{__builtin_bit_cast(u32x4, tbt[rt][kb])}, frag_from_acc_f32(du[s][kb]));
          ndx[s][rt] = -x;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_tbt(cn);
    __builtin_amdgcn_sched_barrier(0);
    // dH = Gamma_C . dH' + QG^T dO - KG^T dX
    SplitFrag ndxs[NS];
    if constexpr (SPLIT)
#pragma unroll
      for (int s = 0; s < NS; ++s) ndxs[s] = split_frag(ndx[s][0], ndx[s][1]);
#pragma unroll
    for (int rh = 0; rh < RHW; ++rh) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        f32x4 h = hp[s][rh];
        if constexpr (SPLIT) {
          h = mma_split(h, split_frag(kgt[rh][0], kgt[rh][1]), ndxs[s]);
        } else {
#pragma unroll
          for (int kb = 0; kb < RT; ++kb)
            h = mma<float>(h, Frag{__builtin_bit_cast(u32x4, kgt[rh][kb])}, frag_from_acc_f32(ndx[s][kb]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dacc[s][rh][i] = live ? h[i] : dacc[s][rh][i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_last(cn);
    __builtin_amdgcn_sched_barrier(0);
  };
  // two first-needed sets trading roles, so that no register copy waits for
  // loads just issued
  First s0, s1;
  if (nchunks > 0) {
    load_first(s0, nchunks - 1);
    load_tbt(nchunks - 1);
    load_last(nchunks - 1);
  }
  for (int c = nchunks - 1; c >= 0; c -= 2) {
    step(s0, s1, c, true);
    step(s1, s0, c - 1, c >= 1);
  }
  if (dh0)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int rh = 0; rh < RHW; ++rh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dh0[(bh * DK + 16 * (rb + rh) + 4 * g + i) * (long long)dv + col0 + 16 * s] = dacc[s][rh][i];
}

// ============================================================ grad (per chunk)
// Split bf16 operands of the grad kernel's value-slice loop, kept in LDS as
// bf16 bit patterns (hi = bf16(x), lo = bf16(x - hi)).  Along the contracted
// index K, each 32-wide block is stored in the K order of a bf16 fragment
// (kappa), so that a lane's 8 values of a row are one 16-byte read; a
// fragment along the other index ("column" fragment) is 8 two-byte reads.
__device__ __forceinline__ int kperm(int k) {   // storage position of K index k within its 32-block
  return (k & ~31) + ((k & 31) < 16 ? 8 * ((k & 15) >> 2) + (k & 3) : 8 * ((k & 15) >> 2) + 4 + (k & 3));
}
__device__ __forceinline__ void split_bits(float x, unsigned short& h, unsigned short& l) {
  const uint32_t hw = pack_bf16x2(x, 0.f) & 0xFFFFu;
  h = (unsigned short)hw;
  l = (unsigned short)(pack_bf16x2(x - __uint_as_float(hw << 16), 0.f) & 0xFFFFu);
}
__device__ __forceinline__ float bits_f32(unsigned short b) { return __uint_as_float((uint32_t)b << 16); }
// lane (r, g): row `row`, the 8 K values of block kb (16-byte read)
__device__ __forceinline__ Frag row_frag(const unsigned short* m, int stride, int row, int kb, int g) {
  return load_frag(m + row * stride + 32 * kb + 8 * g);
}
// lane (r, g): column position `cpos` = kperm(16 b + r) of a 16-column block
// b (the same b for the whole wave), rows 32 kb + kappa(g, e), as two
// transposing LDS reads (ds_read_b64_tr_b16).  Within each 16-lane group, that
// read gives lane i, as its element j, element i % 4 of the 8 bytes that lane
// 4 j + i / 4 of the group addresses; so lane (g, s) addresses row 4 g + s / 4
// (16 rows further for the second read) at column position 8 (s % 4) + 4 b,
// the first of the 4 consecutive positions kperm gives lanes 4 (s % 4) .. + 3.
__device__ __forceinline__ Frag col_frag(const unsigned short* m, int stride, int cpos, int kb, int g) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int s = threadIdx.x & 15;
  const unsigned short* p = m + (32 * kb + 4 * g + (s >> 2)) * stride + 8 * (s & 3) + (cpos & 4);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 16 * stride));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  Frag f;
  f.w = u32x4{a[0], a[1], b[0], b[1]};
  return f;
}
struct SFrag {
  Frag h, l;
};
__device__ __forceinline__ SFrag srow(const unsigned short* mh, const unsigned short* ml, int stride, int row, int kb,
                                      int g) {
  return SFrag{row_frag(mh, stride, row, kb, g), row_frag(ml, stride, row, kb, g)};
}
__device__ __forceinline__ SFrag scol(const unsigned short* mh, const unsigned short* ml, int stride, int cpos, int kb,
                                      int g) {
  return SFrag{col_frag(mh, stride, cpos, kb, g), col_frag(ml, stride, cpos, kb, g)};
}
__device__ __forceinline__ f32x4 mma3(f32x4 acc, SFrag a, SFrag b) {
  acc = mma<bf16_t>(acc, a.l, b.h);
  acc = mma<bf16_t>(acc, a.h, b.l);
  return mma<bf16_t>(acc, a.h, b.h);
}
__device__ __forceinline__ f32x4 mma2a(f32x4 acc, Frag a, SFrag b) {   // A exact in bf16
  acc = mma<bf16_t>(acc, a, b.l);
  return mma<bf16_t>(acc, a, b.h);
}
__device__ __forceinline__ f32x4 mma2b(f32x4 acc, SFrag a, Frag b) {   // B exact in bf16
  acc = mma<bf16_t>(acc, a.l, b);
  return mma<bf16_t>(acc, a.h, b);
}

// threads of the grad kernel: two waves per SIMD, so that one wave's LDS and
// matrix-core latencies overlap the other's (its LDS keeps one workgroup per
// CU at dk = 128)
constexpr int kGThreads = 512;

template <typename T, int DK, int DS, bool RS>
__global__ __launch_bounds__(kGThreads) void chunk_bwd_grad_kernel(
    const T* q, const T* k, const T* v, const T* alpha, const T* beta, const T* dout, const float* __restrict__ rec,
    const float* __restrict__ hc, const float* __restrict__ dhn, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dvo, float* __restrict__ dal, float* __restrict__ dbe, int T_len, int nchunks, int dv) {
  constexpr int C = kBC, DKP = DK + 1, CP = C + 1, DSP = DS + 1;
  constexpr int NW = kGThreads / 64;
  static_assert(DS == 16 || DS == 32, "value slices are one or two 16-column blocks");
  using R = BwdRec<DK>;
  // SG: bf16 inputs with 32-column slices: the value-slice loop on split bf16
  // operands (bf16 matrix cores, 3 steps of 32 K where fp32 takes 8 of 4)
  constexpr bool SG = std::is_same<T, bf16_t>::value && DS == 32 && DK >= 32;
  static_assert(!RS || SG, "a split record is read by the split-bf16 value-slice loop");
  // split-bf16 areas (in 2-byte units): per chunk KG, KR (hi, lo; rows of
  // KP), M^T, TB (hi, lo; rows of CP2); per slice H, dH' (hi, lo; DK rows of
  // SP), dO (bf16, C rows of SP), V (as stored, C x DS), X, U, dU, dX (hi, lo;
  // C rows of SP).  Row strides are multiples of 16 bytes.
  constexpr int KP = DK + 8, SP = DS + 8, CP2 = C + 8;
  constexpr int SG_U16 = 4 * C * KP + 4 * C * CP2 + 4 * DK * SP + C * SP + C * DS + 8 * C * SP;
  // after the loop: dQG, dKG, dKR, the per-channel scratch, (SG) the halving's
  // scan inputs and the slots' H . dH' partial sums
  constexpr int POST = 3 * C * DKP + C * DK + (SG ? C * DK + DK * DS : 0);
  // big area: KG, KR and the slice buffers during the value-slice loop (SG:
  // the split areas), the accumulated dQG, dKG, dKR and the per-channel
  // scratch columns afterwards
  constexpr int SLICE = 2 * DK * DSP + 5 * C * DSP;
  constexpr int LOOP = SG ? (SG_U16 + 1) / 2 : 2 * C * DKP + SLICE;
  constexpr int BIG = LOOP > POST ? LOOP : POST;
  // q, k and alpha in their input type (bf16 inputs are kept exactly)
  __shared__ T sq[C * DKP], sk[C * DKP], sa[C * DKP];
  __shared__ __align__(16) float big[BIG];
  // C x C matrices: (not SG) M and TB for the loop; dM, dTB; T, S and P, which
  // are consumed before the halving's scalar passes keep data there
  constexpr int NCC = SG ? 5 : 7;
  __shared__ float sCC[NCC * C * CP];
  float* sM = SG ? nullptr : sCC;
  float* sdM = sCC + (SG ? 0 : 1) * C * CP;
  float* sdTB = sCC + (SG ? 1 : 2) * C * CP;
  float* sTB = SG ? nullptr : sCC + 3 * C * CP;
  float* sT = sCC + (SG ? 2 : 4) * C * CP;
  float* sS = sCC + (SG ? 3 : 5) * C * CP;
  float* sP = sCC + (SG ? 4 : 6) * C * CP;
  using u16 = unsigned short;
  u16* KGh = reinterpret_cast<u16*>(big);
  u16* KGl = KGh + C * KP;
  u16* KRh = KGl + C * KP;
  u16* KRl = KRh + C * KP;
  u16* MTh = KRl + C * KP;
  u16* MTl = MTh + C * CP2;
  u16* TBh = MTl + C * CP2;
  u16* TBl = TBh + C * CP2;
  u16* Hh = TBl + C * CP2;
  u16* Hl = Hh + DK * SP;
  u16* dHh = Hl + DK * SP;
  u16* dHl = dHh + DK * SP;
  u16* dOb = dHl + DK * SP;
  u16* Vb = dOb + C * SP;
  u16* Xh = Vb + C * DS;
  u16* Xl = Xh + C * SP;
  u16* Uh = Xl + C * SP;
  u16* Ul = Uh + C * SP;
  u16* dUh = Ul + C * SP;
  u16* dUl = dUh + C * SP;
  u16* dXh = dUl + C * SP;
  u16* dXl = dXh + C * SP;
  __shared__ float sb[C], sdb[C], sGC[DK];
  float* sKG = big;
  float* sKR = big + C * DKP;
  float* sH = big + 2 * C * DKP;
  float* sdH = sH + DK * DSP;
  float* sdO = sdH + DK * DSP;
  float* sX = sdO + C * DSP;
  float* sU = sX + C * DSP;
  float* sdU = sU + C * DSP;
  float* sdX = sdU + C * DSP;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const long long chunk = blockIdx.x;
  const long long bh = chunk / nchunks;
  const int c = (int)(chunk % nchunks);
  const int t0 = c * C, cv = min(C, T_len - t0);
  const long long row0 = bh * (long long)T_len + t0;
  const float* rc = rec + (size_t)chunk * R::FLOATS;
  const float* hcc = hc + (size_t)chunk * DK * dv;
  const float* dhc = dhn + (size_t)chunk * DK * dv;
  // one value slice's operands, fetched into registers a slice ahead (V and
  // dO as stored, at in-bounds addresses: the mask for rows past the end is
  // applied when they are staged, so that nothing waits for them early)
  constexpr int NH = (DK * DS + kGThreads - 1) / kGThreads, NV = (C * DS + kGThreads - 1) / kGThreads;
  float rH[NH], rdH[NH];
  T rV[NV], rO[NV];
  auto fetch = [&](int col0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int e = tid + i * kGThreads, ee = e < DK * DS ? e : 0;
      rH[i] = hcc[(size_t)col0 * DK + ee];   // the slice's blocks, in slot order (hc_slot)
      rdH[i] = dhc[(size_t)col0 * DK + ee];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + i * kGThreads, t = e / DS, j = e % DS;
      const size_t gi = e < C * DS && t < cv ? (size_t)(row0 + t) * dv + col0 + j : 0;
      rV[i] = v[gi];
      rO[i] = dout[gi];
    }
  };
  auto v_ok = [&](int e) { return e < C * DS && e / DS < cv; };   // a staged V / dO element inside the chunk
  // beta as stored, fetched with the chunk's operands
  const T braw = beta[row0 + (tid < C && tid < cv ? tid : 0)];

  {   // all of the chunk's operand loads, and the first value slice's, issued before any is stored
    constexpr int NK = (C * DK + kGThreads - 1) / kGThreads, NC = (C * C + kGThreads - 1) / kGThreads;
    // (q, k and alpha as stored, at in-bounds addresses: rows past the end
    // are masked when staged, so that nothing waits for them early)
    T r0[NK], r1[NK], r2[NK];
    float r3[NK], r4[NK], m0[NC], m1[NC], m2[NC], m3[NC];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = tid + i * kGThreads, t = e / DK, ch = e % DK;
      const bool in = e < C * DK, ok = in && t < cv;
      const size_t gi = ok ? (size_t)(row0 + t) * DK + ch : 0;
      r0[i] = q[gi];
      r1[i] = k[gi];
      r2[i] = alpha[gi];
      if constexpr (!RS) {
        r3[i] = rc[R::KG_OFF + (in ? e : 0)];
        r4[i] = rc[R::KR_OFF + (in ? e : 0)];
      }
    }
    // a split record: KG, KR, M^T and TB as hi and lo fragments, copied as
    // they are (task = one lane of one pair: row tile rt, K block kb)
    constexpr int NPK = 2 * (DK / 32) * 64, NPS = 2 * NPK + 2 * 2 * 64;
    constexpr int NRS = RS ? (NPS + kGThreads - 1) / kGThreads : 0;
    u32x4 ph[NRS > 0 ? NRS : 1], pl[NRS > 0 ? NRS : 1];
    // (the LDS destinations as offsets from KGh, so that the stores stay LDS
    // stores: KGh, KGl, KRh, KRl of C x KP, then MTh, MTl, TBh, TBl of C x CP2)
    constexpr int KBS = DK >= 32 ? DK / 32 : 1;
    auto rs_task = [&](int task, int& off, int& kd, int& rt, int& kb, int& stride, int& dh, int& dl)
                       __attribute__((always_inline)) {
      const int field = task < NPK ? 0 : task < 2 * NPK ? 1 : task < 2 * NPK + 128 ? 2 : 3;
      const int pair = field < 2 ? (task - field * NPK) / 64 : (task - 2 * NPK - (field - 2) * 128) / 64;
      kd = field < 2 ? DK : C;
      rt = field < 2 ? pair / KBS : pair;
      kb = field < 2 ? pair % KBS : 0;
      off = field == 0 ? R::KG_OFF : field == 1 ? R::KR_OFF : field == 2 ? R::MT_OFF : R::TB_OFF;
      stride = field < 2 ? KP : CP2;
      dh = field < 2 ? 2 * field * C * KP : 4 * C * KP + 2 * (field - 2) * C * CP2;
      dl = dh + (field < 2 ? C * KP : C * CP2);
    };
    if constexpr (RS) {
#pragma unroll
      for (int i = 0; i < NRS; ++i) {
        const int task = tid + i * kGThreads;
        if (task < NPS) {
          int off, kd, rt, kb, stride, dh, dl;
          rs_task(task, off, kd, rt, kb, stride, dh, dl);
          const float* tile = rc + off + (rt * (kd / 16) + 2 * kb) * 256 + 4 * (task % 64);
          ph[i] = *reinterpret_cast<const u32x4*>(tile);
          pl[i] = *reinterpret_cast<const u32x4*>(tile + 256);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int e = tid + i * kGThreads;
      const bool in = e < C * C;
      if constexpr (!RS) {
        m0[i] = rc[R::MT_OFF + (in ? e : 0)];
        m1[i] = rc[R::TB_OFF + (in ? e : 0)];
      }
      m2[i] = rc[R::T_OFF + (in ? e : 0)];
      m3[i] = rc[R::S_OFF + (in ? e : 0)];
    }
    fetch(0);
    if constexpr (RS) {
#pragma unroll
      for (int i = 0; i < NRS; ++i) {
        const int task = tid + i * kGThreads;
        if (task < NPS) {
          int off, kd, rt, kb, stride, dh, dl;
          rs_task(task, off, kd, rt, kb, stride, dh, dl);
          const int ln = task % 64, o = (16 * rt + (ln & 15)) * stride + 32 * kb + 8 * (ln >> 4);
          *reinterpret_cast<u32x4*>(KGh + dh + o) = ph[i];
          *reinterpret_cast<u32x4*>(KGh + dl + o) = pl[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = tid + i * kGThreads;
      if (e < C * DK) {
        const int o = (e / DK) * DKP + e % DK;
        const bool ok = e / DK < cv;   // rows past a ragged end: no query or key, gate 1
        sq[o] = ok ? r0[i] : T{};
        sk[o] = ok ? r1[i] : T{};
        sa[o] = ok ? r2[i] : from_f32<T>(1.f);
        int tt, cc;   // KG and KR are in fragment order
        frag_pos(e, DK, tt, cc);
        if constexpr (RS) {
        } else if constexpr (SG) {
          const int os = tt * KP + kperm(cc);
          split_bits(r3[i], KGh[os], KGl[os]);
          split_bits(r4[i], KRh[os], KRl[os]);
        } else {
          sKG[tt * DKP + cc] = r3[i];
          sKR[tt * DKP + cc] = r4[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int e = tid + i * kGThreads;
      if (e < C * C) {
        const int o = (e / C) * CP + e % C;
        int ii, jj;   // M^T and TB are in fragment order, T and S row-major
        frag_pos(e, C, ii, jj);
        if constexpr (RS) {
        } else if constexpr (SG) {   // the record holds M^T, the A operand of M^T dO
          const int os = ii * CP2 + kperm(jj);
          split_bits(m0[i], MTh[os], MTl[os]);
          split_bits(m1[i], TBh[os], TBl[os]);
        } else {
          sM[jj * CP + ii] = m0[i];   // the record holds M^T
          sTB[ii * CP + jj] = m1[i];
        }
        sT[o] = m2[i];
        sS[o] = m3[i];
      }
    }
  }
  if (tid < C) sb[tid] = tid < cv ? to_f32(braw) : 0.f;
  if (tid < DK) sGC[tid] = 0.f;

  // ---- value slices: dV, and the dv contractions accumulated on the matrix cores
  constexpr int TQ = (C / 16) * (DK / 16);          // tiles of a C x DK matrix
  constexpr int TPW = (TQ + NW - 1) / NW;           // per wave
  constexpr int TM = (C / 16) * (C / 16);           // tiles of a C x C matrix
  constexpr int TMW = (TM + NW - 1) / NW;
  f32x4 aqg[TPW], akg[TPW], akr[TPW], am[TMW], atb[TMW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) aqg[i] = akg[i] = akr[i] = zero4();
#pragma unroll
  for (int i = 0; i < TMW; ++i) am[i] = atb[i] = zero4();
  if constexpr (SG) {
    // per slot, H . dH' summed over the slices (the slot's row is the same in
    // every slice), reduced per channel after the loop in a fixed order
    float gcp[NH];
#pragma unroll
    for (int i = 0; i < NH; ++i) gcp[i] = 0.f;
    const int tq = wave & 3, prt = tq >> 1, pct = tq & 1;   // a wave's tile of the C x DS products
    const int cpos = kperm(16 * pct + r);                     // its column's storage position
    for (int col0 = 0; col0 < dv; col0 += DS) {
      __syncthreads();   // previous slice fully consumed (and, first time, the loads above)
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int e = tid + i * kGThreads;
        if (e < DK * DS) {
          // slot e of 16-column block b = e / (16 dk) holds, with l = e % (16 dk),
          // row 16 (l / 256) + 4 ((l / 64) % 4) + l % 4, column 16 b + (l / 4) % 16
          const int b = e / (16 * DK), l = e % (16 * DK);
          const int o = (16 * (l / 256) + 4 * ((l / 64) % 4) + l % 4) * SP + kperm(16 * b + (l / 4) % 16);
          split_bits(rH[i], Hh[o], Hl[o]);
          split_bits(rdH[i], dHh[o], dHl[o]);
          gcp[i] += rH[i] * rdH[i];
        }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = tid + i * kGThreads;
        if (e < C * DS) {   // exact in bf16 (the inputs)
          Vb[e] = v_ok(e) ? rV[i].bits : (u16)0;
          dOb[(e / DS) * SP + kperm(e % DS)] = v_ok(e) ? rO[i].bits : (u16)0;
        }
      }
      __syncthreads();
      if (col0 + DS < dv) fetch(col0 + DS);
      // waves 0-3: X = V - KG H; waves 4-7: dU = M^T dO + KR dH'  (tile prt, pct)
      {
        f32x4 acc = zero4();
        if (wave < 4) {
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb)
            acc = mma3(acc, srow(KGh, KGl, KP, 16 * prt + r, kb, g), scol(Hh, Hl, SP, cpos, kb, g));
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const int t = 16 * prt + 4 * g + vv;
            split_bits(bits_f32(Vb[t * DS + 16 * pct + r]) - acc[vv], Xh[t * SP + cpos], Xl[t * SP + cpos]);
          }
        } else {
          acc = mma2b(acc, srow(MTh, MTl, CP2, 16 * prt + r, 0, g), col_frag(dOb, SP, cpos, 0, g));
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb)
            acc = mma3(acc, srow(KRh, KRl, KP, 16 * prt + r, kb, g), scol(dHh, dHl, SP, cpos, kb, g));
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const int t = 16 * prt + 4 * g + vv;
            split_bits(acc[vv], dUh[t * SP + cpos], dUl[t * SP + cpos]);
          }
        }
      }
      __syncthreads();
      // waves 0-3: U = TB X; waves 4-7: dX = TB^T dU (= dv, stored)
      {
        f32x4 acc = zero4();
        if (wave < 4) {
          acc = mma3(acc, srow(TBh, TBl, CP2, 16 * prt + r, 0, g), scol(Xh, Xl, SP, cpos, 0, g));
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const int t = 16 * prt + 4 * g + vv;
            split_bits(acc[vv], Uh[t * SP + cpos], Ul[t * SP + cpos]);
          }
        } else {
          // TB^T's row t is TB's column t: a column fragment of TB
          acc = mma3(acc, scol(TBh, TBl, CP2, kperm(16 * prt + r), 0, g), scol(dUh, dUl, SP, cpos, 0, g));
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const int t = 16 * prt + 4 * g + vv;
            split_bits(acc[vv], dXh[t * SP + cpos], dXl[t * SP + cpos]);
            if (t < cv) dvo[(size_t)(row0 + t) * dv + col0 + 16 * pct + r] = acc[vv];
          }
        }
      }
      __syncthreads();
      // dQG += dO H^T, dKG += dX H^T (negated when stored), dKR += U dH'^T  (C x DK, K = DS)
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int ti = wave + NW * i;
        if (ti < TQ) {
          const int i0 = (ti / (DK / 16)) * 16, j0 = (ti % (DK / 16)) * 16;
          const SFrag bh = srow(Hh, Hl, SP, j0 + r, 0, g);
          aqg[i] = mma2a(aqg[i], row_frag(dOb, SP, i0 + r, 0, g), bh);
          akg[i] = mma3(akg[i], srow(dXh, dXl, SP, i0 + r, 0, g), bh);
          akr[i] = mma3(akr[i], srow(Uh, Ul, SP, i0 + r, 0, g), srow(dHh, dHl, SP, j0 + r, 0, g));
        }
      }
      // waves 0-3: dM += dO U^T; waves 4-7: dTB += dU X^T  (C x C, K = DS)
      if (wave < 4) am[0] = mma2a(am[0], row_frag(dOb, SP, 16 * prt + r, 0, g), srow(Uh, Ul, SP, 16 * pct + r, 0, g));
      else atb[0] = mma3(atb[0], srow(dUh, dUl, SP, 16 * prt + r, 0, g), srow(Xh, Xl, SP, 16 * pct + r, 0, g));
    }
    __syncthreads();
    // H . dH' per channel: the channel's 16 DS / 16 slots, in a fixed order
    float* gpart = big + 3 * C * DKP + 2 * C * DK;   // [slot]
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int e = tid + i * kGThreads;
      if (e < DK * DS) gpart[e] = gcp[i];
    }
    __syncthreads();
    if (tid < DK) {
      const int ch = tid;
      float acc = 0.f;
      for (int b = 0; b < DS / 16; ++b)
        for (int m = 0; m < 16; ++m) acc += gpart[b * 16 * DK + 256 * (ch / 16) + 64 * ((ch % 16) / 4) + 4 * m + ch % 4];
      sGC[ch] = acc;
    }
  } else
  for (int col0 = 0; col0 < dv; col0 += DS) {
    __syncthreads();   // previous slice fully consumed (and, first time, the loads above)
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int e = tid + i * kGThreads;
      if (e < DK * DS) {
        // slot e of 16-column block b = e / (16 dk) holds, with l = e % (16 dk),
        // row 16 (l / 256) + 4 ((l / 64) % 4) + l % 4, column 16 b + (l / 4) % 16
        const int b = e / (16 * DK), l = e % (16 * DK);
        const int o = (16 * (l / 256) + 4 * ((l / 64) % 4) + l % 4) * DSP + 16 * b + (l / 4) % 16;
        sH[o] = rH[i];
        sdH[o] = rdH[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + i * kGThreads;
      if (e < C * DS) {
        const int o = (e / DS) * DSP + e % DS;
        sX[o] = v_ok(e) ? to_f32(rV[i]) : 0.f;
        sdO[o] = v_ok(e) ? to_f32(rO[i]) : 0.f;
      }
    }
    __syncthreads();
    if (col0 + DS < dv) fetch(col0 + DS);
    // X and dU on different waves
    gemm_lds<true, DK, 0, NW>(sX, DSP, sKG, DKP, 1, sH, DSP, 1, C, DS, -1.f);           // X = V - KG H
    gemm_lds<false, C, NW / 2, NW>(sdU, DSP, sM, 1, CP, sdO, DSP, 1, C, DS, 1.f);         // dU = M^T dO + KR dH'
    gemm_lds<true, DK, NW / 2, NW>(sdU, DSP, sKR, DKP, 1, sdH, DSP, 1, C, DS, 1.f);
    __syncthreads();
    gemm_lds<false, C, 0, NW>(sU, DSP, sTB, CP, 1, sX, DSP, 1, C, DS, 1.f);             // U = TB X
    gemm_lds<false, C, NW / 2, NW>(sdX, DSP, sTB, 1, CP, sdU, DSP, 1, C, DS, 1.f);        // dX = TB^T dU
    if (tid < DK) {
      float acc = 0.f;
      for (int j = 0; j < DS; ++j) acc += sH[tid * DSP + j] * sdH[tid * DSP + j];
      sGC[tid] += acc;
    }
    __syncthreads();
    for (int e = tid; e < C * DS; e += kGThreads) {
      const int t = e / DS, j = e % DS;
      if (t < cv) dvo[(size_t)(row0 + t) * dv + col0 + j] = sdX[t * DSP + j];
    }
    // dQG += dO H^T, dKG -= dX H^T, dKR += U dH'^T   (C x DK, K = DS)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ti = wave + NW * i;
      if (ti < TQ) {
        const int i0 = (ti / (DK / 16)) * 16, j0 = (ti % (DK / 16)) * 16;
        aqg[i] = mfma_lds<DS>(aqg[i], sdO + i0 * DSP, DSP, 1, sH + j0 * DSP, 1, DSP);
        akg[i] = mfma_lds<DS>(akg[i], sdX + i0 * DSP, DSP, 1, sH + j0 * DSP, 1, DSP);
        akr[i] = mfma_lds<DS>(akr[i], sU + i0 * DSP, DSP, 1, sdH + j0 * DSP, 1, DSP);
      }
    }
    // dM += dO U^T, dTB += dU X^T   (C x C, K = DS)
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
      const int ti = wave + NW * i;
      if (ti < TM) {
        const int i0 = (ti / (C / 16)) * 16, j0 = (ti % (C / 16)) * 16;
        am[i] = mfma_lds<DS>(am[i], sdO + i0 * DSP, DSP, 1, sU + j0 * DSP, 1, DSP);
        atb[i] = mfma_lds<DS>(atb[i], sdU + i0 * DSP, DSP, 1, sX + j0 * DSP, 1, DSP);
      }
    }
  }
  __syncthreads();
  // accumulators to LDS (the big area is free now); dKG is stored negated
  float* sdQG = big;
  float* sdKG = big + C * DKP;
  float* sdKR = big + 2 * C * DKP;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int ti = wave + NW * i;
    if (ti < TQ) {
      const int i0 = (ti / (DK / 16)) * 16, j0 = (ti % (DK / 16)) * 16;
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int o = (i0 + 4 * g + vv) * DKP + j0 + r;
        sdQG[o] = aqg[i][vv];
        sdKG[o] = -akg[i][vv];
        sdKR[o] = akr[i][vv];
      }
    }
  }
  if constexpr (SG) {   // dM on waves 0-3, dTB on waves 4-7, tile wave % 4
    const int tq = wave & 3, i0 = (tq >> 1) * 16, j0 = (tq & 1) * 16;
    float* dst = wave < 4 ? sdM : sdTB;
    const f32x4 a = wave < 4 ? am[0] : atb[0];
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      const int row = i0 + 4 * g + vv, col = j0 + r;
      dst[row * CP + col] = col <= row ? a[vv] : 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
      const int ti = wave + NW * i;
      if (ti < TM) {
        const int i0 = (ti / (C / 16)) * 16, j0 = (ti % (C / 16)) * 16;
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int row = i0 + 4 * g + vv, col = j0 + r;
          sdM[row * CP + col] = col <= row ? am[i][vv] : 0.f;
          sdTB[row * CP + col] = col <= row ? atb[i][vv] : 0.f;
        }
      }
    }
  }
  __syncthreads();
  // ---- through the solve: TB = T Diag(beta), T = (I + A)^-1, A = Diag(beta) S.
  // Row and column sums below take TPC threads per row (column), summed by DPP.
  constexpr int TPC = kGThreads / C;
  static_assert(TPC <= 64 && C % TPC == 0, "row groups within a wave");
  {   // dbeta from TB = T Diag(beta): colsum(T . dTB)
    const int col = tid / TPC, sub = tid % TPC;
    float acc = 0.f;
#pragma unroll
    for (int i = sub; i < C; i += TPC) acc += sT[i * CP + col] * sdTB[i * CP + col];
    acc = group_sum<TPC>(acc);
    if (sub == 0) sdb[col] = acc;
  }
  __syncthreads();
  for (int e = tid; e < C * C; e += kGThreads) sdTB[(e / C) * CP + e % C] *= sb[e % C];   // dT = dTB Diag(beta)
  __syncthreads();
  gemm_lds<false, C, 0, NW>(sP, CP, sdTB, CP, 1, sT, 1, CP, C, C, 1.f);                         // P = dT T^T
  __syncthreads();
  gemm_lds<false, C, 0, NW>(sdTB, CP, sT, 1, CP, sP, CP, 1, C, C, -1.f);                        // dA = -T^T P
  __syncthreads();
  {   // strictly lower part: dbeta += rowsum(dA . S), dS = Diag(beta) dA
    const int t = tid / TPC, sub = tid % TPC;
    float acc = 0.f;
#pragma unroll
    for (int j = sub; j < C; j += TPC) {
      const float da = j < t ? sdTB[t * CP + j] : 0.f;
      acc += da * sS[t * CP + j];
      sdTB[t * CP + j] = sb[t] * da;
    }
    acc = group_sum<TPC>(acc);
    if (sub == 0) sdb[t] += acc;
  }
  __syncthreads();
  float* sdS = sdTB;

  // ---- per channel: direct terms, gate scans, recursive halving of S and M.
  // The accumulators live in each channel's column of the (now consumed)
  // dQG / dKG / dKR arrays: gq, gk, ga; sg is a per-channel scratch column.
  {
    const int ch = tid % DK, part = tid / DK;   // P threads per channel in the halving's scalar passes
    auto Q = [&](int t) { return to_f32(sq[t * DKP + ch]); };
    auto K = [&](int t) { return to_f32(sk[t * DKP + ch]); };
    auto A = [&](int t) { return to_f32(sa[t * DKP + ch]); };
    float* gq = sdQG + ch;   // element t at gq[t * DKP]
    float* gk = sdKG + ch;
    float* ga = sdKR + ch;
    float* sg = big + 3 * C * DKP + ch;   // element t at sg[t * DK]
    constexpr int P = kGThreads / DK;
    // Direct terms, the KR scan (pairs with the chunk end), the Gamma_C term
    // and the Gamma_t terms (pairs with the chunk start), per channel:
    //   dq_t = dM_tt k_t + dQG_t pre_{t+1},  dk_t = dM_tt q_t + dKG_t pre_{t+1} + dKR_t se_t,
    //   dalpha_t = se_t f_t + gc pre_t se_t + pre_t b_t,
    // with pre_t = Gamma_{t-1} (alpha_0 ... alpha_{t-1}), se_t = G(C-1, t),
    // f_0 = 0, f_{t+1} = alpha_t f_t + dKR_t k_t, and b_t = R_t + alpha_{t+1} b_{t+1}
    // (b_{C-1} = R_{C-1}), R_t = dQG_t q_t + dKG_t k_t, gc = rowsum(H . dH').
    // NS threads per channel take NS segments of SL positions: each forms its
    // segment's part of every product and scan with nothing carried in, the
    // carries (segment products, f at the segment end, b at its start and its
    // gate product) go through LDS, and each then completes its positions.
    constexpr int NS = 4, SL = C / NS;
    static_assert(P >= NS, "a thread per channel and segment");
    // [4][NS][DK] carries, in C x C arrays consumed by now (T, S, P and, not SG, TB)
    float* xs = SG ? sT : sCC + 3 * C * CP;
    static_assert(4 * NS * DK <= 3 * C * CP, "carries fit in the consumed C x C arrays");
    const bool segon = part < NS;
    const int t0s = part * SL;
    float av[SL], pl[SL + 1], sl[SL], fl[SL], bl[SL], ml[SL];
    if (segon) {
      pl[0] = 1.f;
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        av[i] = A(t0s + i);
        pl[i + 1] = pl[i] * av[i];
      }
      xs[(0 * NS + part) * DK + ch] = pl[SL];
    }
    __syncthreads();
    float pre_in = 1.f;
    if (segon) {
      float suf_in = 1.f;
#pragma unroll
      for (int p = 0; p < NS; ++p) {
        const float lp = xs[(0 * NS + p) * DK + ch];
        if (p < part) pre_in *= lp;
        if (p > part) suf_in *= lp;
      }
      float e = suf_in;   // se of the segment's positions
#pragma unroll
      for (int i = SL - 1; i >= 0; --i) {
        sl[i] = e;
        e *= av[i];
      }
      float f = 0.f, rv[SL];
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int t = t0s + i;
        const float dqg = gq[t * DKP], dkg = gk[t * DKP], dkr = ga[t * DKP], dmd = sdM[t * CP + t];
        const float pr1 = pre_in * pl[i + 1];
        gq[t * DKP] = dmd * K(t) + dqg * pr1;
        gk[t * DKP] = dmd * Q(t) + dkg * pr1 + dkr * sl[i];
        fl[i] = f;
        f = av[i] * f + dkr * K(t);
        rv[i] = dqg * Q(t) + dkg * K(t);
      }
      xs[(1 * NS + part) * DK + ch] = f;
      // b inside the segment with nothing from the right, and the gate product
      // ml_t = alpha_{t+1} ... alpha_{t0s+SL} that carries the right part in
      const float anext = part + 1 < NS ? A(t0s + SL) : 0.f;
      float bb = 0.f, mm = 1.f;
#pragma unroll
      for (int i = SL - 1; i >= 0; --i) {
        const float a1 = i + 1 < SL ? av[i + 1] : anext;
        bb = rv[i] + a1 * bb;
        mm = a1 * mm;
        bl[i] = bb;
        ml[i] = mm;
      }
      xs[(2 * NS + part) * DK + ch] = bl[0];
      xs[(3 * NS + part) * DK + ch] = ml[0];
    }
    __syncthreads();
    if (segon) {
      float fin = 0.f, bin = 0.f;   // f at the segment's start, b at the next segment's start
#pragma unroll
      for (int p = 0; p < NS; ++p)
        if (p < part) fin = xs[(0 * NS + p) * DK + ch] * fin + xs[(1 * NS + p) * DK + ch];
#pragma unroll
      for (int p = NS - 1; p >= 0; --p)
        if (p > part) bin = xs[(2 * NS + p) * DK + ch] + xs[(3 * NS + p) * DK + ch] * bin;
      const float gc = sGC[ch];
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int t = t0s + i;
        const float pr = pre_in * pl[i];
        ga[t * DKP] = sl[i] * (fl[i] + pl[i] * fin) + gc * pr * sl[i] + pr * (bl[i] + ml[i] * bin);
      }
    }
    __syncthreads();
    // recursive halving: blocks [lo, lo + 2h), L = [lo, m], R = [m + 1, lo + 2h - 1];
    // sg holds G(m, j) on L and G(t, m) on R.  h is a compile-time constant per
    // level so that the loops unroll.
    auto factors = [&](int lo, auto hh, bool left) __attribute__((always_inline)) {
      constexpr int h = decltype(hh)::value;
      if (left) {
        float e = 1.f;
#pragma unroll
        for (int i = h - 1; i >= 0; --i) {
          sg[(lo + i) * DK] = e;
          e *= A(lo + i);
        }
      } else {
        float f = 1.f;
#pragma unroll
        for (int i = 0; i < h; ++i) {
          f *= A(lo + h + i);
          sg[(lo + h + i) * DK] = f;
        }
      }
    };
    // The first level (one block: L = 0..15, R = 16..31, all 16 x 16 pairs)
    // has its cross terms on the matrix cores for all channels at once: with
    // k~_j = k_j G(15, j) on L and q~_t = q_t G(t, 15), k~_t = k_t G(t, 15) on R,
    //   zm = dM[R, L] k~_L,  zs = dS[R, L] k~_L  (rows of R),
    //   zl = dM[R, L]^T q~_R + dS[R, L]^T k~_R    (rows of L);
    // then dq_t += G(t, 15) zm_t, dk_t += G(t, 15) zs_t, dk_j += G(15, j) zl_j,
    // and the scans take Z_t = q_t zm_t + k_t zs_t on R and Z_j = k_j zl_j on L:
    // on R, s from last to first, b_s = Z_s + alpha_{s+1} b_{s+1} and dalpha_s
    // += G(s - 1, 15) b_s (1 at s = 16); on L, j from first to last, dalpha_j +=
    // G(15, j) f and f = alpha_j f + Z_j.
    // [t][channel]: (not SG) in TB, T, S and P, consumed by now; (SG) after the
    // scratch columns in the big area
    float* Z = SG ? big + 3 * C * DKP + C * DK : sCC + 3 * C * CP;
    static_assert(SG || C * DK <= 4 * C * CP, "scan inputs fit in the consumed C x C arrays");
    const float* sgall = big + 3 * C * DKP;
    auto level16 = [&]() __attribute__((always_inline)) {
      constexpr int h = C / 2;
      const auto hh = std::integral_constant<int, h>{};
      if (part < 2) factors(0, hh, part == 1);
      __syncthreads();
      constexpr int TJ = DK / 16;
      for (int ti = wave; ti < 2 * TJ; ti += NW) {   // ti / TJ is uniform in a wave
        const int J = ti % TJ, c = 16 * J + r;
        f32x4 z0 = zero4(), z1 = zero4();
        if (ti >= TJ) {   // rows t = 16 + r of R, contraction over L
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int t = h + r, j = 4 * st + g;
            const float kt = to_f32(sk[j * DKP + c]) * sgall[j * DK + c];
            z0 = __builtin_amdgcn_mfma_f32_16x16x4f32(sdM[t * CP + j], kt, z0, 0, 0, 0);
            z1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sdS[t * CP + j], kt, z1, 0, 0, 0);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int tr = h + 4 * g + v;
            const float fac = sgall[tr * DK + c];
            sdQG[tr * DKP + c] += fac * z0[v];
            sdKG[tr * DKP + c] += fac * z1[v];
            Z[tr * DK + c] = to_f32(sq[tr * DKP + c]) * z0[v] + to_f32(sk[tr * DKP + c]) * z1[v];
          }
        } else {   // rows j = r of L, contraction over R
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int j = r, t = h + 4 * st + g;
            const float fac = sgall[t * DK + c];
            const float qt = to_f32(sq[t * DKP + c]) * fac, kt = to_f32(sk[t * DKP + c]) * fac;
            z0 = __builtin_amdgcn_mfma_f32_16x16x4f32(sdM[t * CP + j], qt, z0, 0, 0, 0);
            z0 = __builtin_amdgcn_mfma_f32_16x16x4f32(sdS[t * CP + j], kt, z0, 0, 0, 0);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int jr = 4 * g + v;
            sdKG[jr * DKP + c] += sgall[jr * DK + c] * z0[v];
            Z[jr * DK + c] = to_f32(sk[jr * DKP + c]) * z0[v];
          }
        }
      }
      __syncthreads();
      if (part == 1) {
        float f = 0.f;
#pragma unroll
        for (int j = 0; j < h; ++j) {
          ga[j * DKP] += sg[j * DK] * f;
          f = A(j) * f + Z[j * DK + ch];
        }
      } else if (part == 0) {
        float bsum = 0.f;
#pragma unroll
        for (int t = C - 1; t >= h; --t) {
          bsum = Z[t * DK + ch] + (t + 1 < C ? A(t + 1) * bsum : 0.f);
          ga[t * DKP] += (t > h ? sg[(t - 1) * DK] : 1.f) * bsum;
        }
      }
      __syncthreads();
    };
    static_assert(C == 32, "halving levels below assume 32-position chunks");
    level16();
    // The levels below the first (h = 8, 4, 2, 1) by position segments: the
    // thread of segment p (positions 8p .. 8p + 7 of its channel) keeps their
    // q, k, alpha and the three accumulators in registers and takes every
    // (block, side) of a level whose positions lie in its segment: at h = 8
    // one side of a 16-position block (the other side's operands come from
    // LDS), below it both sides of every block of the segment.  Right-side
    // rows t, last to first: the cross terms with L (zm = sum_j dM[t, j] k~_j,
    // zs likewise with dS; dq_t += G(t, m) zm, dk_t += G(t, m) zs) and the
    // scan for the gates s in R, G(s - 1, m) sum_{t >= s} (q_t zm_t + k_t zs_t)
    // G(t, s).  Left-side rows j, first to last: the cross terms with R
    // (zl = sum_t dM[t, j] q~_t + dS[t, j] k~_t; dk_j += G(m, j) zl) and the
    // scan for the gates s in L, G(m, s) sum_{j < s} k_j zl_j G(s - 1, j).
    static_assert(SL == 8 && NS == 4, "8-position segments");
    float rq[SL], rk[SL], ra[SL], aq[SL], ak[SL], aa[SL], sgv[SL];
    if (segon) {
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int t = t0s + i;
        rq[i] = Q(t);
        rk[i] = K(t);
        ra[i] = av[i];
        aq[i] = gq[t * DKP];
        ak[i] = gk[t * DKP];
        aa[i] = ga[t * DKP];
      }
    }
    // factors of one side, positions o .. o + h - 1 of the segment: G(t, m) on
    // the right side (m = o - 1), G(m, j) on the left (m = o + h - 1)
    // (written to LDS too when another segment's thread reads them: h = 8)
    auto seg_factors = [&](auto oo, auto hh, bool right) __attribute__((always_inline)) {
      constexpr int o = decltype(oo)::value, h = decltype(hh)::value;
      constexpr bool publish = h == SL;
      if (right) {
        float f = 1.f;
#pragma unroll
        for (int i = 0; i < h; ++i) {
          f *= ra[o + i];
          sgv[o + i] = f;
          if (publish) sg[(t0s + o + i) * DK] = f;
        }
      } else {
        float e = 1.f;
#pragma unroll
        for (int i = h - 1; i >= 0; --i) {
          sgv[o + i] = e;
          if (publish) sg[(t0s + o + i) * DK] = e;
          e *= ra[o + i];
        }
      }
    };
    // right side at segment offset o (positions t0s + o ..), its left side at
    // lo (absolute); the left side's k~ from registers (same segment) or LDS
    auto seg_right = [&](auto oo, auto hh, int lo, bool left_here) __attribute__((always_inline)) {
      constexpr int o = decltype(oo)::value, h = decltype(hh)::value;
      float ky[h];
#pragma unroll
      for (int jj = 0; jj < h; ++jj)
        ky[jj] = left_here ? rk[o - h + jj] * sgv[o - h + jj] : K(lo + jj) * sg[(lo + jj) * DK];
      float bs = 0.f;
#pragma unroll
      for (int i = h - 1; i >= 0; --i) {
        const int t = t0s + o + i;
        float zm = 0.f, zs = 0.f;
#pragma unroll
        for (int jj = 0; jj < h; ++jj) {
          zm += sdM[t * CP + lo + jj] * ky[jj];
          zs += sdS[t * CP + lo + jj] * ky[jj];
        }
        const float gr = sgv[o + i];
        aq[o + i] += gr * zm;
        ak[o + i] += gr * zs;
        bs = rq[o + i] * zm + rk[o + i] * zs + (i + 1 < h ? ra[o + i + 1] * bs : 0.f);
        aa[o + i] += (i > 0 ? sgv[o + i - 1] : 1.f) * bs;
      }
    };
    // left side at segment offset o, its right side starting at rlo (absolute)
    auto seg_left = [&](auto oo, auto hh, int rlo, bool right_here) __attribute__((always_inline)) {
      constexpr int o = decltype(oo)::value, h = decltype(hh)::value;
      float qr[h], kr[h];
#pragma unroll
      for (int i = 0; i < h; ++i) {
        if (right_here) {
          qr[i] = rq[o + h + i] * sgv[o + h + i];
          kr[i] = rk[o + h + i] * sgv[o + h + i];
        } else {
          const float gr = sg[(rlo + i) * DK];
          qr[i] = Q(rlo + i) * gr;
          kr[i] = K(rlo + i) * gr;
        }
      }
      float f = 0.f;
#pragma unroll
      for (int jj = 0; jj < h; ++jj) {
        const int j = t0s + o + jj;
        float zl = 0.f;
#pragma unroll
        for (int i = 0; i < h; ++i) zl += sdM[(rlo + i) * CP + j] * qr[i] + sdS[(rlo + i) * CP + j] * kr[i];
        const float gl = sgv[o + jj];
        ak[o + jj] += gl * zl;
        aa[o + jj] += gl * f;
        f = ra[o + jj] * f + rk[o + jj] * zl;
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I8 = std::integral_constant<int, 8>;
    // h = 8: blocks of 16 positions, segment 2b is the left side of block b, 2b + 1 its right
    const bool odd = part & 1;
    if (segon) seg_factors(I0{}, I8{}, odd);
    __syncthreads();
    if (segon) {
      if (odd) seg_right(I0{}, I8{}, t0s - SL, false);
      else seg_left(I0{}, I8{}, t0s + SL, false);
    }
    // h = 4, 2, 1: every block inside the segment, both sides, from this
    // thread's registers only (no barrier)
    auto seg_block = [&](auto bb, auto hh) __attribute__((always_inline)) {
      constexpr int b = decltype(bb)::value, h = decltype(hh)::value;
      using OL = std::integral_constant<int, 2 * h * b>;
      using OR = std::integral_constant<int, 2 * h * b + h>;
      seg_factors(OL{}, hh, false);
      seg_factors(OR{}, hh, true);
      seg_right(OR{}, hh, t0s + 2 * h * b, true);
      seg_left(OL{}, hh, t0s + 2 * h * b + h, true);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    if (segon) {
      seg_block(I0{}, I4{});
      seg_block(I0{}, I2{});
      seg_block(I1{}, I2{});
      seg_block(I0{}, I1{});
      seg_block(I1{}, I1{});
      seg_block(I2{}, I1{});
      seg_block(I3{}, I1{});
    }
    if (segon)
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int t = t0s + i;
        if (t < cv) {
          const size_t o = (size_t)(row0 + t) * DK + ch;
          dq[o] = aq[i];
          dk[o] = ak[i];
          dal[o] = aa[i];
        }
      }
  }
  if (tid < cv) dbe[row0 + tid] = sdb[tid];
}

// ============================================================ launch
// compute units of the current device, cached per device
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// workgroups of `kernel` resident per CU at `threads` threads (its LDS and
// registers decide), cached per kernel and device (kernels past the cache's
// slots are asked each time); at least 1
template <typename K>
static int resident_per_cu(K kernel, int threads) {
  constexpr int kSlots = 16;
  static std::atomic<int> cache[kSlots][64];   // [kernel slot][device]
  static std::atomic<const void*> which[kSlots];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const void* f = reinterpret_cast<const void*>(kernel);
  int slot = -1;
  for (int i = 0; i < kSlots && slot < 0; ++i) {
    const void* w = which[i].load(std::memory_order_relaxed);
    if (w == f) slot = i;
    else if (w == nullptr) {
      const void* expected = nullptr;
      if (which[i].compare_exchange_strong(expected, f) || expected == f) slot = i;
    }
  }
  int n = slot >= 0 ? cache[slot][dev].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
    if (slot >= 0) cache[slot][dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename T, int DK>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  using R = BwdRec<DK>;
  const int nch = (a.T + kBC - 1) / kBC;
  const long long BH = (long long)a.B * a.H, total = BH * nch;
  float* rec = (float*)a.workspace;
  float* hc = rec + (size_t)total * R::FLOATS;
  float* dhn = hc + (size_t)total * DK * a.dv;
  const unsigned nsl = (unsigned)(a.dv / kBDS);
  const int xcd_map = (BH % 8 == 0) ? 1 : 0;
  // bf16 inputs free enough LDS for 32-column value slices (half the slice
  // steps); fp32 inputs, and dv = 16, take 16 columns.  With bf16 inputs,
  // dk >= 64 and 32-column slices every consumer of the record multiplies
  // split pairs, and the record holds them (BwdRec).
  auto prep = chunk_bwd_prep_kernel<T, DK, false>;
  auto states = chunk_bwd_states_kernel<T, DK, false, 1>;
  auto dstates = chunk_bwd_dstates_kernel<T, DK, false, kDsWaves<DK>, 1>;
  auto grad = chunk_bwd_grad_kernel<T, DK, 16, false>;
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (a.dv % 32 == 0) grad = chunk_bwd_grad_kernel<T, DK, 32, false>;
    if constexpr (kSplitSeq<T, DK>) {
      if (a.dv % 32 == 0) {
        prep = chunk_bwd_prep_kernel<T, DK, true>;
        states = chunk_bwd_states_kernel<T, DK, true, 1>;
        dstates = chunk_bwd_dstates_kernel<T, DK, true, kDsWaves<DK>, 1>;
        grad = chunk_bwd_grad_kernel<T, DK, 32, true>;
      }
    }
  }
  if (total > 0) {
    // prep loops over chunks: as many workgroups as are resident at once
    const long long nprep = std::min<long long>(total, (long long)resident_per_cu(prep, kPThreads) * device_cus());
    hipLaunchKernelGGL(prep, dim3((unsigned)nprep), dim3(kPThreads), 0, a.stream, (const T*)a.q, (const T*)a.k,
                       (const T*)a.alpha, (const T*)a.beta, rec, a.T, nch, total);
    // with split products, two value slices per wave once one per wave would
    // put two or more workgroups on every compute unit (they would share its
    // memory path); the fp32 matrix-core chain is bound by its own issue, and
    // one slice per wave is faster there
    bool two = false;
    if constexpr (kSplitSeq<T, DK>)
      if (states == chunk_bwd_states_kernel<T, DK, true, 1> && BH * nsl >= 2LL * device_cus()) {
        two = true;
        states = chunk_bwd_states_kernel<T, DK, true, 2>;
      }
    hipLaunchKernelGGL(states, dim3((unsigned)(BH * nsl / (two ? 2 : 1))), dim3(64), 0, a.stream, (const T*)a.v, a.h0,
                       rec, hc, a.T, nch, a.dv, xcd_map);
  }
  // the reverse pass likewise halves its workgroups (four waves of two slices
  // each) once one slice per workgroup would put two or more on every CU
  bool two_ds = false;
  int ds_waves = kDsWaves<DK>;
  if constexpr (kSplitSeq<T, DK> && DK == 128)
    if (dstates == chunk_bwd_dstates_kernel<T, DK, true, kDsWaves<DK>, 1> && BH * nsl >= 2LL * device_cus()) {
      two_ds = true;
      ds_waves = 4;
      dstates = chunk_bwd_dstates_kernel<T, DK, true, 4, 2>;
    }
  hipLaunchKernelGGL(dstates, dim3((unsigned)(BH * nsl / (two_ds ? 2 : 1))), dim3(64 * ds_waves), 0, a.stream,
                     (const T*)a.dout, a.dhT, rec, dhn, a.gh0, a.T, nch, a.dv, xcd_map);
  if (total > 0)
    hipLaunchKernelGGL(grad, dim3((unsigned)total), dim3(kGThreads), 0, a.stream, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.alpha, (const T*)a.beta, (const T*)a.dout, rec, hc, dhn, a.gq, a.gk,
                       a.gv, a.galpha, a.gbeta, a.T, nch, a.dv);
  return hipGetLastError();
}

template <typename T>
static hipError_t bwd_dk_dispatch(const BwdArgs& a) {
  switch (a.dk) {
    case 16: return launch_bwd_t<T, 16>(a);
    case 32: return launch_bwd_t<T, 32>(a);
    case 64: return launch_bwd_t<T, 64>(a);
    case 128: return launch_bwd_t<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
  if ((long long)a.B * a.H == 0) return hipSuccess;
  return a.dtype == 1 ? bwd_dk_dispatch<bf16_t>(a) : bwd_dk_dispatch<float>(a);
}

size_t chunk_bwd_workspace_floats(int B, int H, int T, int dk, int dv) {
  size_t per = 0;
  switch (dk) {
    case 16: per = BwdRec<16>::FLOATS; break;
    case 32: per = BwdRec<32>::FLOATS; break;
    case 64: per = BwdRec<64>::FLOATS; break;
    case 128: per = BwdRec<128>::FLOATS; break;
    default: return 0;
  }
  const size_t total = (size_t)B * H * (((size_t)T + kBC - 1) / kBC);
  return total * (per + 2 * (size_t)dk * dv);
}

}  // namespace ckda
