// KV append (or in-place refresh) fused with the block-representative update.
//
// The representative of a KV block is the mean of its keys (the pages name a
// per-block "representative value" -- sciencestack page of arXiv 2512.21911,
// Figure 1 caption -- without defining it; the mean is the reading taken here).
//
// One workgroup of 256 threads per (sequence, touched logical block, KV head). A
// token row of K or V is D * ES bytes = NCH 16-byte chunks; thread t owns chunk
// t % NCH of the slots t / NCH, t / NCH + SG, ... (SG = 256 / NCH slot groups), so
// every load and store is a 16-byte access and the threads of a slot group cover one
// token row contiguously (K and V are both token-major in the pool). New tokens are
// copied from the input into the pool; every valid slot of the block (new ones from
// the input, the others from the pool) is summed in float32: first per slot group in
// slot order, then over the slot groups in order. That order depends only on the
// block's valid-slot count, so the representative is the same whether the block was
// filled at once, token by token, or partly rewritten.
#include "internal.h"

namespace sv {
namespace {

constexpr int kReprThreads = 256;

template <int ES>
__device__ __forceinline__ void add_chunk(float* acc, uint4 x) {
  if constexpr (ES == 2) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    acc[0] += __uint_as_float(x.x);
    acc[1] += __uint_as_float(x.y);
    acc[2] += __uint_as_float(x.z);
    acc[3] += __uint_as_float(x.w);
  }
}

template <int ES, int D>
__global__ __launch_bounds__(kReprThreads) void block_repr_kernel(ReprParams p) {
  constexpr int NCH = D * ES / 16;          // 16-byte chunks per token row
  constexpr int SG = kReprThreads / NCH;    // slot groups
  constexpr int EPC = 16 / ES;              // elements per chunk
  __shared__ float part[SG * D];

  const int t = threadIdx.x;
  const int ch = t % NCH;
  const int sg = t / NCH;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  int n = p.n_new[b];
  if (n > p.n_new_max) n = p.n_new_max;
  const int c0 = p.ctx_before[b];
  if (n <= 0 || c0 < 0) return;
  const int c1 = c0 + n;
  // Valid tokens of the sequence after the call: the end of the new tokens (append),
  // or the caller's ctx_after when it rewrites tokens inside the context.
  int end = p.ctx_after ? p.ctx_after[b] : c1;
  if (end < c1) end = c1;
  const int cap = p.NB * p.bs;
  if (end > cap) end = cap;
  const int j = c0 / p.bs + static_cast<int>(blockIdx.x);
  const int blk_lo = j * p.bs;
  if (blk_lo >= c1 || j >= p.NB) return;
  const int phys = p.block_table[static_cast<int64_t>(b) * p.NB + j];
  if (phys < 0 || phys >= p.P) return;

  const int new_lo = (c0 > blk_lo ? c0 : blk_lo) - blk_lo;               // first new slot
  const int new_hi = (c1 < blk_lo + p.bs ? c1 : blk_lo + p.bs) - blk_lo;  // past the last
  const int n_valid = (end < blk_lo + p.bs ? end : blk_lo + p.bs) - blk_lo;

  const int64_t row_bytes = static_cast<int64_t>(D) * ES;
  const int64_t blk = static_cast<int64_t>(phys) * p.Hkv + g;
  char* kblk = static_cast<char*>(p.k_pool) + blk * p.bs * row_bytes;
  char* vblk = static_cast<char*>(p.v_pool) + blk * p.bs * row_bytes;
  const char* kn = static_cast<const char*>(p.k_new);
  const char* vn = static_cast<const char*>(p.v_new);

  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
  for (int s = sg; s < n_valid; s += SG) {
    uint4 kv;
    if (s >= new_lo && s < new_hi) {
      const int tok = blk_lo + s - c0;
      const int64_t src = ((static_cast<int64_t>(b) * p.n_new_max + tok) * p.Hkv + g) * row_bytes;
      kv = *reinterpret_cast<const uint4*>(kn + src + ch * 16);
      const uint4 vv = *reinterpret_cast<const uint4*>(vn + src + ch * 16);
      *reinterpret_cast<uint4*>(kblk + s * row_bytes + ch * 16) = kv;
      *reinterpret_cast<uint4*>(vblk + s * row_bytes + ch * 16) = vv;
    } else {
      kv = *reinterpret_cast<const uint4*>(kblk + s * row_bytes + ch * 16);
    }
    add_chunk<ES>(acc, kv);
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[sg * D + ch * EPC + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < SG; ++q) sum += part[q * D + t];
    p.repr_pool[blk * D + t] = sum / static_cast<float>(n_valid);
  }
}

template <int ES>
hipError_t launch_es(const ReprParams& p, dim3 grid, hipStream_t stream) {
  if (p.D == 128)
    hipLaunchKernelGGL((block_repr_kernel<ES, 128>), grid, dim3(kReprThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((block_repr_kernel<ES, 64>), grid, dim3(kReprThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_repr(const ReprParams& p, bool bf16, hipStream_t stream) {
  if (p.B == 0 || p.n_new_max == 0) return hipSuccess;
  const int max_touch = (p.n_new_max + p.bs - 1) / p.bs + 1;
  dim3 grid(max_touch, p.Hkv, p.B);
  return bf16 ? launch_es<2>(p, grid, stream) : launch_es<4>(p, grid, stream);
}

}  // namespace sv
