// Inter-layer retrieval reuse: the layer takes the previous layer's selected block
// indices and counts unchanged (tutorial page "Accelerate Speculative Decoding with
// Sparse Computation in Verification", section "Core technique 1"; sciencestack
// abstract of arXiv 2512.21911). One small grid-stride copy kernel, so the step
// stays a kernel node when the caller captures the layer loop in a graph.
#include "internal.h"

namespace sv {
namespace {

__global__ __launch_bounds__(256) void reuse_kernel(ReuseParams p) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < p.n_idx + p.n_cnt; i += stride) {
    if (i < p.n_idx)
      p.idx[i] = p.prev_idx[i];
    else
      p.cnt[i - p.n_idx] = p.prev_cnt[i - p.n_idx];
  }
}

}  // namespace

hipError_t launch_reuse(const ReuseParams& p, hipStream_t stream) {
  const int64_t n = p.n_idx + p.n_cnt;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(reuse_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
