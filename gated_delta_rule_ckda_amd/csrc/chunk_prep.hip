// chunk_prep.hip -- per-chunk preparation kernel of the chunkwise CKDA
// forward: one workgroup (4 waves) per chunk of one (batch, head), every chunk
// of every head at once.  The work itself is chunk_prologue (prologue.hpp):
// signed segment products of the gates, the decayed Gram matrices on the
// matrix cores, the UT/WY triangular solve, and the operand record that the
// state-pass kernel (chunk_state.hip) consumes, written to the workspace.
#include "prologue.hpp"
#include "ckda_internal.hpp"

namespace ckda {

constexpr int kPrepThreads = 256;

template <typename T, int DK, int C>
__global__ __launch_bounds__(kPrepThreads) void chunk_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ alpha,
    const T* __restrict__ beta, unsigned char* __restrict__ ws, int T_len, int nchunks) {
  using P = ProCfg<T, DK, C>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[P::LDS_BYTES];
  const long long chunk_id = blockIdx.x;
  const long long bh = chunk_id / nchunks;
  const int t0 = (int)(chunk_id % nchunks) * C;
  const long long row0 = bh * (long long)T_len + t0;
  chunk_prologue<T, DK, C>(q + row0 * DK, k + row0 * DK, alpha + row0 * DK, beta + row0, min(C, T_len - t0),
                           ws + (size_t)chunk_id * P::BYTES, lds, (int)threadIdx.x, [] { lds_barrier(); });
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
