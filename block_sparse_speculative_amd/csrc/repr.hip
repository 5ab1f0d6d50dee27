// KV append fused with the block-representative update.
//
// The representative of a KV block is the mean of its keys (the pages name a
// per-block "representative value" -- sciencestack page of arXiv 2512.21911,
// Figure 1 caption -- without defining it; the mean is the reading taken here).
// One workgroup per (sequence, touched logical block, KV head); thread d owns
// head dimension d. New tokens are scattered into the pool through the block
// table, then the float32 sum over ALL valid slots of the block is taken in slot
// order (old slots read from the pool, new ones from the input), so the result
// is the same whether the block was filled at once or token by token.
#include "internal.h"

namespace sv {
namespace {

template <typename E>
__device__ __forceinline__ float to_f32(E x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <typename E>
__global__ void block_repr_kernel(ReprParams p) {
  const int d = threadIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  int n = p.n_new[b];
  if (n > p.n_new_max) n = p.n_new_max;
  const int c0 = p.ctx_before[b];
  if (n <= 0 || c0 < 0) return;
  const int c1 = c0 + n;
  const int j = c0 / p.bs + static_cast<int>(blockIdx.x);
  const int blk_lo = j * p.bs;
  if (blk_lo >= c1 || j >= p.NB) return;
  const int phys = p.block_table[static_cast<int64_t>(b) * p.NB + j];
  if (phys < 0 || phys >= p.P) return;

  const int new_lo = (c0 > blk_lo ? c0 : blk_lo) - blk_lo;      // first new slot
  const int hi = c1 < blk_lo + p.bs ? c1 : blk_lo + p.bs;
  const int n_valid = hi - blk_lo;                                // valid slots after append

  const E* kn = static_cast<const E*>(p.k_new);
  const E* vn = static_cast<const E*>(p.v_new);
  E* kp = static_cast<E*>(p.k_pool);
  E* vp = static_cast<E*>(p.v_pool);
  const int64_t blk = static_cast<int64_t>(phys) * p.Hkv + g;
  E* kblk = kp + blk * p.bs * p.D;          // [bs, D]
  E* vblk = vp + blk * p.D * p.bs;          // [D, bs]

  float sum = 0.0f;
  for (int slot = 0; slot < n_valid; ++slot) {
    E kv;
    if (slot >= new_lo) {
      const int tok = blk_lo + slot - c0;
      const int64_t src = ((static_cast<int64_t>(b) * p.n_new_max + tok) * p.Hkv + g) * p.D + d;
      kv = kn[src];
      kblk[static_cast<int64_t>(slot) * p.D + d] = kv;
      vblk[static_cast<int64_t>(d) * p.bs + slot] = vn[src];
    } else {
      kv = kblk[static_cast<int64_t>(slot) * p.D + d];
    }
    sum += to_f32<E>(kv);
  }
  p.repr_pool[blk * p.D + d] = sum / static_cast<float>(n_valid);
}

}  // namespace

hipError_t launch_block_repr(const ReprParams& p, bool bf16, hipStream_t stream) {
  if (p.B == 0 || p.n_new_max == 0) return hipSuccess;
  const int max_touch = (p.n_new_max + p.bs - 1) / p.bs + 1;
  dim3 grid(max_touch, p.Hkv, p.B);
  dim3 block(p.D);
  if (bf16)
    hipLaunchKernelGGL(block_repr_kernel<uint16_t>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(block_repr_kernel<float>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
