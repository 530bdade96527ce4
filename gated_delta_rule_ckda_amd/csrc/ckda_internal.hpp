// ckda_internal.hpp -- host-side launch descriptors shared between the C ABI
// layer (argument checking, dispatch) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "ckda.h"

namespace ckda {

// Launch flag beside the public CKDA_FUSE_* / CKDA_GATE_SCALAR bits: two
// delta-rule sub-steps per token (DeltaProduct_2; rows of k, v, beta are
// sub-steps, rows of q, o and of a scalar alpha are tokens).
constexpr int kProd2 = 1 << 16;

struct DecodeArgs {
  const void *q, *k, *v, *alpha, *beta;
  float* H_inout;
  void* o;
  int N, H, dk, dv, dtype;
  int flags;   // CKDA_FUSE_* prologue steps (0: inputs used as given)
  hipStream_t stream;
  const int* gidx = nullptr;   // [H][dk] retained channel indices into rows of dk_in (NULL: no gather)
  int dk_in = 0;
};

struct ChunkArgs {
  const void *q, *k, *v, *alpha, *beta;
  const float* h0;
  void* o;
  float* hT;
  int B, H, T, dk, dv, chunk, dtype;
  int flags;   // CKDA_FUSE_* prologue steps (0: inputs used as given)
  void* workspace;
  hipStream_t stream;
  hipEvent_t ev[3];   // recorded before the Gram kernel, between the kernels, after the state kernel (if set)
  const int* gidx = nullptr;   // [H][dk] retained channel indices into rows of dk_in (NULL: no gather)
  int dk_in = 0;
};

// Layout of the per-chunk records the Gram kernel writes and the state-pass
// kernel reads (byte offsets inside one chunk's record).
struct ChunkRecord {
  size_t t_off, m_off, bytes;
};
ChunkRecord chunk_record_layout(int dk, int chunk, int dtype);

struct BwdArgs {
  const void *q, *k, *v, *alpha, *beta;
  const float* h0;
  const void* dout;
  const float* dhT;
  float *gq, *gk, *gv, *galpha, *gbeta, *gh0;   // gradients of q, k, v, alpha, beta, h0
  int B, H, T, dk, dv, dtype;
  void* workspace;
  hipStream_t stream;
};
// floats of backward workspace (per-chunk records, chunk-start states and
// state gradients), 0 for an unsupported dk
size_t chunk_bwd_workspace_floats(int B, int H, int T, int dk, int dv);
hipError_t launch_chunk_bwd(const BwdArgs& a);
// the backward through the per-token prologue (prologue_bwd.hip); flags as
// CKDA_FUSE_* | CKDA_GATE_SCALAR, nonzero
size_t prologue_bwd_workspace_floats(int B, int H, int T, int dk, int dv, int flags);
hipError_t launch_prologue_bwd(const BwdArgs& a, int flags);
// the DeltaProduct_2 backward (dp2_bwd.hip): k, v, beta, dk, dv, dbeta hold 2 T
// sub-steps; alpha (or NULL: ungated) and dalpha are [B, H, T]
size_t dp2_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype);
hipError_t launch_dp2_bwd(const BwdArgs& a);

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_chunk_fwd(const ChunkArgs& a);

// Size of the fixed device scratch of ckda_chunk_fwd_noalloc (noalloc.hip),
// and its device address on the current device (looked up on first use).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace ckda
