// chunk_state.hip -- chunk-to-chunk state pass and output of the chunkwise
// CKDA forward.
//
// One workgroup (4 waves) per (batch, head, slice of 16 * NCT value columns).
// The columns of the state evolve independently once the keys, gates and
// beta are fixed (the value v_t only enters column j through v_t[j]), so the
// slices of one head need no communication.  The fp32 state slice H stays in
// accumulator registers for the whole sequence; per chunk, with the operand
// record written by the preparation kernel (layout in chunk_common.hpp):
//   X = V + W H             (W = -(K~ . gamma))
//   U = TB X                (TB = (I + A)^-1 Diag(beta): the UT/WY solve)
//   O = Q H + M U           (output of every position, from the state at
//                            chunk start and the chunk's own writes)
//   H <- d . H + KR U       (d = P_C gamma_C, KR = P_C (K~ . gamma_C/gamma)^T)
// All five products run on the matrix cores (bf16 x bf16 -> fp32 for bf16
// inputs, fp32 for fp32 inputs).  H, X and U are exchanged between the waves
// through LDS in the B-operand fragment layout; the decay of H is applied
// element-wise in fp32, so the state itself is never rounded.
#include "chunk_common.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int kStateThreads = 256;

template <typename T, int DK, int C, int NCT>
__global__ __launch_bounds__(kStateThreads) void chunk_state_kernel(
    const T* __restrict__ v, const float* __restrict__ h0, T* o, float* __restrict__ hT,
    const unsigned char* ws, int T_len, int nchunks, int dv, int slices, int xcd_map) {
  using G = ChunkGeom<T, DK, C>;
  constexpr int RT = G::RT, RH = G::RH, KBN = G::KBN, KBC = G::KBC, HALVES = G::HALVES;
  constexpr int NRH = (RH + 3) / 4;  // state row tiles per wave (row tile rh = wave + 4 j)
  __shared__ __attribute__((aligned(16))) Frag s_h[KBN][NCT][64];
  __shared__ __attribute__((aligned(16))) Frag s_x[KBC][NCT][64];
  __shared__ __attribute__((aligned(16))) Frag s_u[KBC][NCT][64];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane / 16, r = lane % 16;

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
  const int col0 = slice * 16 * NCT;

  // zero the exchange buffers once: K-block halves that no tile ever writes
  // (DK or C smaller than a K block) must read as zero
  for (int i = tid; i < (int)(sizeof(s_h) + sizeof(s_x) + sizeof(s_u)) / 16; i += kStateThreads) {
    Frag z;
    z.w = u32x4{0u, 0u, 0u, 0u};
    if (i < (int)sizeof(s_h) / 16) (&s_h[0][0][0])[i] = z;
    else if (i < (int)(sizeof(s_h) + sizeof(s_x)) / 16) (&s_x[0][0][0])[i - sizeof(s_h) / 16] = z;
    else (&s_u[0][0][0])[i - (sizeof(s_h) + sizeof(s_x)) / 16] = z;
  }
  lds_barrier();

  // write one accumulator tile (row tile rt) into a B-fragment exchange slot
  auto put = [&](Frag* base, int rt, int ct, f32x4 t) {
    Frag* slot = base + ((rt / HALVES) * NCT + ct) * 64 + lane;
    if constexpr (sizeof(T) == 2) {
      u32x2 p{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
      reinterpret_cast<u32x2*>(slot)[rt % 2] = p;
    } else {
      *slot = frag_from_acc_f32(t);
    }
  };

  // initial state
  const long long sbase = (long long)bh * DK * dv;
  f32x4 hacc[NRH][NCT];
#pragma unroll
  for (int j = 0; j < NRH; ++j) {
    const int rh = wave + 4 * j;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      hacc[j][ct] = zero4();
      if (rh < RH) {
        if (h0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            hacc[j][ct][i] = h0[sbase + (long long)(16 * rh + 4 * g + i) * dv + col0 + 16 * ct + r];
        }
        put(&s_h[0][0][0], rh, ct, hacc[j][ct]);
      }
    }
  }

  // operands of one chunk that this wave needs, loaded one chunk ahead
  struct Ops {
    Frag w[KBN], q[KBN], t[KBC], m[KBC], kr[NRH][KBC];
    f32x4 d[NRH];
    T v[NCT][4];     // raw values; masked and widened when used
  };
  const long long vbase = (long long)bh * T_len;
  // waves that own a row tile of X, U and O (all of them when C = 64), and
  // whether every wave's state row tiles exist (DK >= 64): compile-time where
  // possible, so that the prefetch below is straight-line code
  const bool xrow = RT >= 4 || wave < RT;
  constexpr bool all_rh = RH % 4 == 0;
  auto fetch = [&](Ops& x, int c) {
    const unsigned char* rec = ws + ((size_t)bh * nchunks + c) * G::BYTES;
    const int t0 = c * C, cv = min(C, T_len - t0);
    if (xrow) {
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) {
        x.w[kb] = load_frag(rec + G::W_OFF + frag_slot(wave, kb, KBN, lane));
        x.q[kb] = load_frag(rec + G::Q_OFF + frag_slot(wave, kb, KBN, lane));
      }
#pragma unroll
      for (int kb = 0; kb < KBC; ++kb) {
        x.t[kb] = load_frag(rec + G::T_OFF + frag_slot(wave, kb, KBC, lane));
        x.m[kb] = load_frag(rec + G::M_OFF + frag_slot(wave, kb, KBC, lane));
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * wave + 4 * g + i;
          x.v[ct][i] = v[(vbase + t0 + min(t, cv - 1)) * dv + col0 + 16 * ct + r];
        }
    }
#pragma unroll
    for (int j = 0; j < NRH; ++j) {
      const int rh = wave + 4 * j;
      if (all_rh || rh < RH) {
        x.d[j] = *reinterpret_cast<const f32x4*>(rec + G::D_OFF + (16 * rh + 4 * g) * 4);
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) x.kr[j][kb] = load_frag(rec + G::KR_OFF + frag_slot(rh, kb, KBC, lane));
      }
    }
  };

  // one chunk: consume `cur`, prefetch chunk c + 1 into `nxt`
  auto step = [&](Ops& cur, Ops& nxt, int c) {
    fetch(nxt, min(c + 1, nchunks - 1));   // the last step re-reads its own chunk (unused)
    const int t0 = c * C;
    const int cv = min(C, T_len - t0);
    f32x4 oacc[NCT];
    if (xrow) {
      f32x4 xacc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xacc[ct][i] = 16 * wave + 4 * g + i < cv ? to_f32(cur.v[ct][i]) : 0.f;
        oacc[ct] = zero4();
      }
#pragma unroll
      for (int kb = 0; kb < KBN; ++kb) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const Frag hb = s_h[kb][ct][lane];
          xacc[ct] = mma<T>(xacc[ct], cur.w[kb], hb);
          oacc[ct] = mma<T>(oacc[ct], cur.q[kb], hb);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) put(&s_x[0][0][0], wave, ct, xacc[ct]);
    }
    lds_barrier();

    if (xrow) {
      f32x4 uacc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) uacc[ct] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBC; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) uacc[ct] = mma<T>(uacc[ct], cur.t[kb], s_x[kb][ct][lane]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) put(&s_u[0][0][0], wave, ct, uacc[ct]);
    }
    lds_barrier();

    Frag ub[KBC][NCT];
#pragma unroll
    for (int kb = 0; kb < KBC; ++kb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) ub[kb][ct] = s_u[kb][ct][lane];
#pragma unroll
    for (int j = 0; j < NRH; ++j) {
      const int rh = wave + 4 * j;
      if (all_rh || rh < RH) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          f32x4 h = cur.d[j] * hacc[j][ct];
#pragma unroll
          for (int kb = 0; kb < KBC; ++kb) h = mma<T>(h, cur.kr[j][kb], ub[kb][ct]);
          hacc[j][ct] = h;
          put(&s_h[0][0][0], rh, ct, h);
        }
      }
    }
    if (xrow) {
#pragma unroll
      for (int kb = 0; kb < KBC; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) oacc[ct] = mma<T>(oacc[ct], cur.m[kb], ub[kb][ct]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * wave + 4 * g + i;
          if (t < cv) o[(vbase + t0 + t) * dv + col0 + 16 * ct + r] = from_f32<T>(oacc[ct][i]);
        }
      }
    }
    lds_barrier();
  };

  // two operand buffers used in turn, so prefetched registers are never copied
  Ops bufA, bufB;
  if (nchunks > 0) fetch(bufA, 0);
  lds_barrier();
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(bufA, bufB, c);
    step(bufB, bufA, c + 1);
  }
  if (c < nchunks) step(bufA, bufB, c);

  if (hT) {
#pragma unroll
    for (int j = 0; j < NRH; ++j) {
      const int rh = wave + 4 * j;
      if (rh < RH) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            hT[sbase + (long long)(16 * rh + 4 * g + i) * dv + col0 + 16 * ct + r] = hacc[j][ct][i];
      }
    }
  }
}

template <typename T, int DK, int C>
hipError_t launch_state_t(const ChunkArgs& a, int nchunks) {
  const int BH = a.B * a.H;
  const int nct = a.dv >= 32 ? 2 : 1;
  const int slices = a.dv / (16 * nct);
  const long long wgs = (long long)BH * slices;
  const int xcd_map = (BH % 8 == 0) ? 1 : 0;
  if (nct == 2)
    hipLaunchKernelGGL((chunk_state_kernel<T, DK, C, 2>), dim3((unsigned)wgs), dim3(kStateThreads), 0, a.stream,
                       (const T*)a.v, a.h0, (T*)a.o, a.hT, (const unsigned char*)a.workspace, a.T, nchunks,
                       a.dv, slices, xcd_map);
  else
    hipLaunchKernelGGL((chunk_state_kernel<T, DK, C, 1>), dim3((unsigned)wgs), dim3(kStateThreads), 0, a.stream,
                       (const T*)a.v, a.h0, (T*)a.o, a.hT, (const unsigned char*)a.workspace, a.T, nchunks,
                       a.dv, slices, xcd_map);
  return hipGetLastError();
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

hipError_t launch_chunk_prep(const ChunkArgs& a, long long total_chunks, int nchunks);

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  const int nchunks = (a.T + a.chunk - 1) / a.chunk;
  const long long BH = (long long)a.B * a.H;
  hipError_t e = launch_chunk_prep(a, BH * nchunks, nchunks);
  if (e != hipSuccess) return e;
  return a.dtype == 1 ? state_dk_dispatch<bf16_t>(a, nchunks) : state_dk_dispatch<float>(a, nchunks);
}

}  // namespace ckda
