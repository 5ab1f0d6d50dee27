// Block selection: GQA-batched scoring of block representatives by the first draft
// token's query, piecewise budget, and top-k with lowest-index tie-break
// (tutorial page "Accelerate Speculative Decoding with Sparse Computation in
// Verification", section "Core technique 1"; sciencestack page of arXiv 2512.21911,
// Figure 1 caption).
//
// Two launches.
//  score_kernel  grid = (ceil(NB / C) chunks, Hkv, B), C = 128 blocks (32 when that
//                grid would give a CU at most one workgroup): workgroup (c, g, b) scores
//                blocks [Cc, Cc+C) of sequence b for KV head g, streaming the
//                float32 representatives through the block table (one 16-byte load
//                per lane, D/4 lanes per block, DPP reduction in a fixed order).
//                Sequences that keep every block (budget capped at k_max >= nb)
//                are skipped unless the caller asked for the scores.
//  top-k         grid = (Hkv, B): budget, then
//                 - NB <= 1024: the keys spread over the registers of four
//                   wavefronts, LDS radix select with a single-register finish and
//                   ballot compaction (topk_wg.h);
//                 - larger NB: an LDS radix select on the same order-preserving
//                   keys and an ascending compaction with block-wide scans.
#include "internal.h"
#include "topk_wg.h"

namespace sv {
namespace {

constexpr int NT = kSelectThreads;
constexpr int NWAVE = NT / 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// x moved across lanes by the DPP control CTRL on the rows in ROW_MASK; lanes whose
// source lies outside their row, and rows outside the mask, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

// Block-wide exclusive scan of one int per thread; returns the prefix and sets
// *total. Uses `scratch` (NWAVE ints of LDS). Must be called by all threads.
__device__ int block_exclusive_scan(int v, int* total, int* scratch) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    const int t = scratch[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + x - v;
}

__device__ __forceinline__ int budget_of(const SelectParams& p, int ctx, int nb) {
  return budget_blocks_dev(ctx, nb, p.dense_ctx, p.min_blocks, p.frac_per_mille);
}

template <typename E, int D, int CHUNK>
__global__ __launch_bounds__(NT) void score_kernel(SelectParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Linear workgroup id -> (unit, chunk); with xcd_group the workgroups of unit u
  // have linear ids congruent to u mod 8, the XCD its attention workgroups use.
  const int nchunk = (p.NB + CHUNK - 1) / CHUNK;
  int unit, chunk;
  {
    const int lin = blockIdx.x;
    if (p.xcd_group) {
      const int slot = lin >> 3;
      unit = (slot / nchunk) * 8 + (lin & 7);
      chunk = slot - (slot / nchunk) * nchunk;
    } else {
      unit = lin / nchunk;
      chunk = lin - unit * nchunk;
    }
  }
  const int b = unit / p.Hkv;
  const int g = unit - b * p.Hkv;
  int ctx = p.ctx_lens[b];
  if (ctx < 0) ctx = 0;
  int nb = (ctx + p.bs - 1) / p.bs;
  if (nb > p.NB) nb = p.NB;
  float* sc = p.scores + static_cast<int64_t>(unit) * p.NB;
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.NB;

  // ------------------------------------------------------------ scoring
  constexpr int LPB = D / 4;                   // lanes per block (one float4 each)
  constexpr int BPW = 64 / LPB;                // blocks per wave per pass
  constexpr int PASSES = CHUNK / (NWAVE * BPW);
  static_assert(PASSES >= 1 && CHUNK % (NWAVE * BPW) == 0, "chunk must fill the passes");
  const int sub = lane / LPB;
  const int li = lane % LPB;
  const int j0 = chunk * CHUNK;
  // A sequence that keeps every block needs no scores: its budget, capped at k_max
  // as the top-k caps it, reaches nb.
  int kcap = budget_of(p, ctx, nb);
  if (kcap > p.k_max) kcap = p.k_max;
  const bool dense = kcap >= nb;
  if (j0 < nb && (!dense || p.scores_requested)) {
    const E* q = static_cast<const E*>(p.q) + static_cast<int64_t>(b) * p.T * p.Hq * D;
    // Block-table loads first, then the query loads, then all representative loads
    // (a bad entry re-reads block 0), then the dot products: no load waits for an
    // unrelated one.
    float4 r[PASSES];
    int jj[PASSES], ph[PASSES];
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      const int j = j0 + (u * NWAVE + wave) * BPW + sub;
      jj[u] = j;
      ph[u] = bt[j < nb ? j : 0];
    }
    // Sum of the group's first-draft query vectors, 8 heads per batch of loads. The
    // loads are unconditional (a head index past the group re-reads the last head)
    // and masked afterwards, so none waits for another.
    float qs[4] = {0.f, 0.f, 0.f, 0.f};
    for (int h0 = 0; h0 < p.G; h0 += 8) {
      float v[8][4];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int hl = h0 + k < p.G ? h0 + k : p.G - 1;
        const E* qh = q + static_cast<int64_t>(g * p.G + hl) * D + 4 * li;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (sizeof(E) == 2) v[k][e] = bf16_to_f32(qh[e]); else v[k][e] = qh[e];
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) qs[e] += h0 + k < p.G ? v[k][e] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      const bool ok = jj[u] < nb && ph[u] >= 0 && ph[u] < p.P;
      r[u] = *reinterpret_cast<const float4*>(
          p.repr_pool + (static_cast<int64_t>(ok ? ph[u] : 0) * p.Hkv + g) * D + 4 * li);
    }
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      float d = qs[0] * r[u].x;
      d = __builtin_fmaf(qs[1], r[u].y, d);
      d = __builtin_fmaf(qs[2], r[u].z, d);
      d = __builtin_fmaf(qs[3], r[u].w, d);
      // Sum over the block's LPB lanes with DPP (no LDS round trip): prefix sums
      // within each 16-lane row leave the row's total in its last lane; when a block
      // spans two rows, the second row then adds the first row's total.
      d += dpp_f32<0x111, 0xF>(d);   // row_shr:1
      d += dpp_f32<0x112, 0xF>(d);   // row_shr:2
      d += dpp_f32<0x114, 0xF>(d);   // row_shr:4
      d += dpp_f32<0x118, 0xF>(d);   // row_shr:8
      if constexpr (LPB == 32) d += dpp_f32<0x142, 0xA>(d);   // row_bcast:15 into rows 1, 3
      const bool ok = ph[u] >= 0 && ph[u] < p.P;
      d = ok ? d : 0.0f;
      if (li == LPB - 1 && jj[u] < nb) sc[jj[u]] = d;
    }
  }

}

// One workgroup of kTopkWaves wavefronts per unit (NB <= 1024).
constexpr int kTopkWaves = 4;
__global__ __launch_bounds__(kTopkWaves * 64) void topk_wg_kernel(SelectParams p) {
  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int unit = b * p.Hkv + g;
  __shared__ __attribute__((aligned(16))) char lds[kTopkLdsBytes];
  float s[kWaveTopkMax / (64 * kTopkWaves)];
  wg_topk_load<kTopkWaves>(p.scores + static_cast<int64_t>(unit) * p.NB, p.NB, s);
  int ctx = p.ctx_lens[b];
  if (ctx < 0) ctx = 0;
  int nb = (ctx + p.bs - 1) / p.bs;
  if (nb > p.NB) nb = p.NB;
  int k = budget_of(p, ctx, nb);
  if (k > p.k_max) k = p.k_max;
  int32_t* out = p.idx + static_cast<int64_t>(unit) * p.k_max;
  int total = wg_topk_select<kTopkWaves>(s, nb, k, p.keep_first, p.keep_last, lds,
                                         [&](int j, int pos) {
                                           if (pos < p.k_max) out[pos] = j;
                                         });
  if (total > p.k_max) total = p.k_max;
  for (int pos = total + tid; pos < p.k_max; pos += kTopkWaves * 64) out[pos] = -1;
  if (tid == 0) p.cnt[unit] = total;
}

// One workgroup per unit, keys in LDS (any NB).
__global__ __launch_bounds__(NT) void topk_kernel(SelectParams p) {
  extern __shared__ uint32_t keys[];           // [NB]
  __shared__ int hist[256];
  __shared__ int scan_scratch[NWAVE];
  __shared__ int bcast[4];

  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int unit = b * p.Hkv + g;
  int ctx = p.ctx_lens[b];
  if (ctx < 0) ctx = 0;
  int nb = (ctx + p.bs - 1) / p.bs;
  if (nb > p.NB) nb = p.NB;
  const float* sc = p.scores + static_cast<int64_t>(unit) * p.NB;

  // ------------------------------------------------------------ budget + top-k
  int k = budget_of(p, ctx, nb);
  if (k > p.k_max) k = p.k_max;
  int32_t* out = p.idx + static_cast<int64_t>(unit) * p.k_max;
  if (k >= nb) {
    if (tid == 0) p.cnt[unit] = nb < p.k_max ? nb : p.k_max;
    for (int pos = tid; pos < p.k_max; pos += NT) out[pos] = pos < nb ? pos : -1;
    return;
  }
  const int f0 = p.keep_first ? 0 : -1;
  const int f1 = p.keep_last ? nb - 1 : -1;
  const int nforced = (f0 >= 0) + (f1 >= 0 && f1 != f0);
  int want = k - nforced;                     // candidates to pick
  if (want < 0) want = 0;                     // k_max below the forced count: forced only

  const int E_PER = (nb + NT - 1) / NT;       // contiguous keys owned by each thread
  const int my_lo = tid * E_PER;
  const int my_hi = my_lo + E_PER < nb ? my_lo + E_PER : nb;
  for (int j = tid; j < nb; j += NT) {
    const bool forced = (j == f0) || (j == f1);
    keys[j] = forced ? 0u : score_key(sc[j]);
  }
  __syncthreads();

  // Radix select of the want-th largest key: after 4 passes `prefix` is the
  // threshold key and `want` the number of keys equal to it that are taken.
  uint32_t prefix = 0u, mask = 0u;
  if (want == 0) {
    prefix = 0xFFFFFFFFu;                     // nothing beats it, no ties taken
  } else {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int j = my_lo; j < my_hi; ++j) {
        const uint32_t key = keys[j];
        if (key != 0u && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      const int v = hist[255 - tid];
      int tot;
      const int cum = block_exclusive_scan(v, &tot, scan_scratch) + v;   // count of digits >= 255-tid
      if (cum >= want && cum - v < want) {
        bcast[1] = 255 - tid;
        bcast[2] = want - (cum - v);
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(bcast[1]) << shift;
      mask |= 255u << shift;
      want = bcast[2];
      __syncthreads();
    }
  }

  // Ties at the threshold go to the lowest indices: rank equal keys in index order.
  int n_eq = 0;
  for (int j = my_lo; j < my_hi; ++j) n_eq += (keys[j] == prefix);
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, &tot, scan_scratch);
  int n_sel = 0;
  {
    int e = eq_before;
    for (int j = my_lo; j < my_hi; ++j) {
      const uint32_t key = keys[j];
      const bool take = (j == f0) || (j == f1) || (key != 0u && key > prefix) ||
                        (key == prefix && e < want);
      e += (key == prefix);
      n_sel += take;
    }
  }
  int total_sel;
  const int sel_before = block_exclusive_scan(n_sel, &total_sel, scan_scratch);
  {
    int e = eq_before;
    int pos = sel_before;
    for (int j = my_lo; j < my_hi; ++j) {
      const uint32_t key = keys[j];
      const bool take = (j == f0) || (j == f1) || (key != 0u && key > prefix) ||
                        (key == prefix && e < want);
      e += (key == prefix);
      if (take) {
        if (pos < p.k_max) out[pos] = j;
        ++pos;
      }
    }
  }
  if (total_sel > p.k_max) total_sel = p.k_max;
  if (tid == 0) p.cnt[unit] = total_sel;
  for (int pos = total_sel + tid; pos < p.k_max; pos += NT) out[pos] = -1;
}

}  // namespace

template <int CHUNK>
void launch_score_chunk(const SelectParams& p, bool bf16, hipStream_t stream) {
  dim3 grid((p.NB + CHUNK - 1) / CHUNK * p.Hkv * p.B);
  if (bf16) {
    if (p.D == 128)
      hipLaunchKernelGGL((score_kernel<uint16_t, 128, CHUNK>), grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((score_kernel<uint16_t, 64, CHUNK>), grid, dim3(NT), 0, stream, p);
  } else {
    if (p.D == 128)
      hipLaunchKernelGGL((score_kernel<float, 128, CHUNK>), grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((score_kernel<float, 64, CHUNK>), grid, dim3(NT), 0, stream, p);
  }
}

hipError_t launch_score(const SelectParams& p, bool bf16, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  // Blocks per workgroup: kSelectChunk, or a quarter of it when kSelectChunk would
  // give a CU at most one workgroup (8 units over 1024 blocks leave most CUs idle;
  // 32 units give each CU one workgroup, whose two dependent round trips then move
  // only 64 KB: four smaller workgroups per CU keep more loads in flight).
  const int64_t units = static_cast<int64_t>(p.B) * p.Hkv;
  if (units * ((p.NB + kSelectChunk - 1) / kSelectChunk) <= kAttnCUs)
    launch_score_chunk<kSelectChunk / 4>(p, bf16, stream);
  else
    launch_score_chunk<kSelectChunk>(p, bf16, stream);
  return hipGetLastError();
}

hipError_t launch_topk(const SelectParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  static_assert(kWaveTopkMax == kWaveTopkMaxBlocks, "one workgroup holds a whole row");
  if (p.NB <= kWaveTopkMax) {
    hipLaunchKernelGGL(topk_wg_kernel, dim3(p.Hkv, p.B), dim3(kTopkWaves * 64), 0, stream, p);
  } else {
    const size_t lds = static_cast<size_t>(p.NB) * sizeof(uint32_t);
    hipLaunchKernelGGL(topk_kernel, dim3(p.Hkv, p.B), dim3(NT), lds, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, bool bf16, hipStream_t stream) {
  const hipError_t e = launch_score(p, bf16, stream);
  return e != hipSuccess ? e : launch_topk(p, stream);
}

}  // namespace sv
