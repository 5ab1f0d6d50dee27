// Split-K multi-draft verification attention over gathered KV blocks, with a
// log-sum-exp merge (sciencestack page of arXiv 2512.21911, Figure 1 caption: all
// draft tokens attend over the one shared set of selected blocks; abstract: the
// draft tokens are verified in one parallel pass).
//
// Work unit = (sequence b, KV head g). Its rows are the T x G (draft token, query
// head of the group) pairs, padded to RP in {16, 32, 64, 128}; its keys are the
// valid tokens of the selected blocks plus the T draft tokens (draft t sees drafts
// 0..t of a chain, or itself and its ancestors in a draft tree: SpecPV page,
// introduction, on tree-shaped candidates). Keys are cut into tiles of TT tokens (a
// tile never spans two blocks). The
// k_max * (bs / TT) tile slots of a unit are cut into S balanced contiguous ranges
// fixed by k_max alone, so a split knows which selected positions it owns before
// the selected count arrives; slots at or past the count are skipped. One more
// workgroup per unit takes the draft tile alone (with S == 1 the single split
// takes it first).
//
// Prologue: the block-table row, the split's block indices (or, in the fused
// select mode, the unit's block scores), the context length and the query
// fragments are requested together, so one round trip precedes the first tile.
// In the fused select mode every context-split workgroup runs the exact budget +
// top-k of the unit from the scores (topk_wg.h: the keys spread over all its
// wavefronts) and keeps the positions its split owns; split 0 also writes the unit's
// indices and count.
//
// Data movement: tiles stream HBM -> LDS through 16-byte LDS-DMA loads
// (global_load_lds_dwordx4) into a ring of NBUF buffers, so NBUF - 1 tiles are in
// flight while one is computed (a 64 KB ring when two workgroups share a CU, else
// 128 KB). The DMA is issued from inline assembly (from a wave-uniform base in SGPRs
// plus a 32-bit per-lane offset) and waited for with explicit vmcnt counts: every
// tile is exactly LPW loads per lane. Any other vector memory access in the loop
// (the register reloads of the fp32 128-row variants) only makes such a wait
// stricter, never looser, since loads complete in issue order. LDS rows are
// XOR-swizzled in 16-byte chunks so the MFMA operand reads (16 lanes, 16 rows, one
// chunk) hit distinct banks.
//
// Compute, per wave (16 rows, a subset of a tile's 32-token groups):
//   S^T = K Q^T      (MFMA, M = tokens, N = rows, K = head dim)
//   online softmax in log2 units: the scale folds into one FMA per score, rows live
//   on lanes, so max / denominator / rescale are lane-local after a 4-lane swap
//   reduction, and the accumulators are rescaled only when some row max moved
//   O^T += V^T P^T   (MFMA, M = head dim, N = rows, K = tokens)
// Token order inside a 32-token group is permuted so the S^T accumulator a lane
// holds is exactly the P^T operand it feeds. V tiles stay token-major in LDS, as in
// the pool, and the matching V^T operand comes from two transposing LDS reads
// (ds_read_b64_tr_b16, 8 bf16 tokens of one head dim per lane). Full context tiles take a path
// with no per-token masking. bf16 uses v_mfma_f32_16x16x32_bf16, fp32
// v_mfma_f32_16x16x4_f32; accumulation is fp32.
//
// Merge of the partials of a unit:  O = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s.
//  - S == 1: the workgroup normalises and writes the output itself.
//  - in the launch (at most 32 workgroups per unit): every workgroup stores its
//    partial with device-scope stores and counts itself in the unit's arrival word.
//    When the whole grid can be resident at once, each workgroup waits (bounded in
//    time) until all siblings have arrived and merges its own slice of the unit's
//    rows; a workgroup whose wait runs out hands its slice to the last arriver. When
//    the grid cannot be resident, the last arriver merges every row at once. No
//    workgroup ever waits for a sibling without a time bound.
//  - otherwise merge_kernel combines the partials in a second launch.
//
// XCD placement: workgroups are dispatched to the 8 XCDs round-robin by linear id.
// When the unit count is a multiple of 8, every kernel of the path (scoring,
// attention, merge) maps unit u to linear ids congruent to u mod 8, so a unit's
// scores, partials and indices are produced and consumed inside one XCD's L2 (a
// handoff between kernels then costs no memory round trip). This is placement for
// speed only; kernel boundaries keep the results coherent wherever a workgroup runs.
#include "gfx950_mem.h"
#include "internal.h"
#include "topk_wg.h"

#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "attn.hip is written for gfx950: its transposing LDS reads, LDS-DMA and cache-policy bits"
#endif

namespace sv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kBtStageMax = 1024;    // block-table rows up to this length are staged in LDS
static_assert(kWaveTopkMaxBlocks <= kBtStageMax, "the fused select mode reads the staged row");

// Workgroup barrier that orders LDS accesses but leaves the LDS-DMA prefetch in
// flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Reductions over the 4 lanes l, l^16, l^32, l^48 (the lanes holding one row) with
// the gfx950 cross-row lane swaps (VALU, no LDS round trip).
__device__ __forceinline__ float max_over_row_lanes(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float sum_over_row_lanes(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Buffer resource over `bytes` bytes at `base` (raw, untyped); accesses past the
// end return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Cache-policy bits of buffer accesses: kDeviceScope (sc1) makes a store or load
// coherent across the XCDs without a cache writeback fence.
constexpr int kDeviceScope = 16;
typedef unsigned int u32x4v __attribute__((__vector_size__(16)));
typedef unsigned int u32x2v __attribute__((__vector_size__(8)));
template <int AUX>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), r, off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ f32x4 load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t r, int off, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2v, v), r, off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ float2 load2(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
}

// Combines the NP partials of one (unit, row) for the 4 head dims at `dim`:
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, sixteen partials per batch of
// loads (unconditional, masked afterwards, so a batch is in flight together; a
// running max rescales across batches). Returns out; *lse2 = M + log2(L).
template <int AUX>
__device__ __forceinline__ f32x4 combine_partials(__amdgpu_buffer_rsrc_t po,
                                                  __amdgpu_buffer_rsrc_t pml, int NP, int R,
                                                  int D, int row, int dim, float* lse2) {
  constexpr int BATCH = 16;
  float mrun = -__builtin_inff(), l = 0.0f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < NP; s0 += BATCH) {
    float2 ml[BATCH];
    f32x4 os[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int sk = s0 + k < NP ? s0 + k : NP - 1;
      ml[k] = load2<AUX>(pml, (sk * R + row) * 8);
      os[k] = load4<AUX>(po, ((sk * R + row) * D + dim) * 4);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch issues before any use
    float mb = mrun;
#pragma unroll
    for (int k = 0; k < BATCH; ++k)
      if (s0 + k < NP) mb = fmaxf(mb, ml[k].x);
    const float msafe = mb == -__builtin_inff() ? 0.0f : mb;
    const float a = __builtin_amdgcn_exp2f(mrun - msafe);
    l *= a;
    o *= a;
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const float w = s0 + k < NP ? __builtin_amdgcn_exp2f(ml[k].x - msafe) : 0.0f;
      l += w * ml[k].y;
      o += w * os[k];
    }
    mrun = mb;
  }
  *lse2 = mrun + __builtin_log2f(l);
  return o * (1.0f / l);
}

template <bool BF16>
__device__ __forceinline__ void store_out4(void* out, int64_t off, f32x4 v) {
  if constexpr (BF16) {
    bf16x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = static_cast<__bf16>(v[e]);
    *reinterpret_cast<bf16x4_t*>(static_cast<char*>(out) + off * 2) = w;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + off) = v;
  }
}

template <bool BF16_, int D_, int TT_, int RP_, int RING_KB_>
struct Cfg {
  static constexpr bool BF16 = BF16_;
  static constexpr int D = D_;
  static constexpr int TT = TT_;           // tokens per tile
  static constexpr int RP = RP_;           // padded rows
  static constexpr int ES = BF16 ? 2 : 4;  // element bytes
  static constexpr int RW = 16;                   // rows per wave (one MFMA N-tile)
  static constexpr int NRG = RP / RW;             // row groups
  static constexpr int NGRP = TT / 32;            // 32-token groups per tile
  static constexpr int NTG = NRG >= 4 ? 1 : NGRP; // waves sharing a row group
  static constexpr int NWAVE = NRG * NTG;
  static constexpr int NT = 64 * NWAVE;
  static constexpr int NN = RW / 16;              // 16-row MFMA tiles per wave
  static constexpr int NMD = D / 16;              // 16-dim MFMA tiles of O^T
  static constexpr int NCHK = D * ES / 16;        // 16-byte chunks per K or V row (a token)
  static constexpr int KCH = TT * NCHK;           // chunks of the K half of a tile (V: as many)
  static constexpr int TILE_CH = 2 * KCH;
  static constexpr int TILE_BYTES = TILE_CH * 16;
  static constexpr int LPW = TILE_CH / NT;        // LDS-DMA loads per lane per tile
  // Ring depth: RING_KB of tiles (64 when two workgroups share a CU, 128 when one
  // has it alone); vmcnt holds at most 63 outstanding loads.
  static constexpr int RING_KB = RING_KB_;
  // Workgroups per CU: two with a 64 KB ring (bf16; fp32 needs the registers of one).
  // The second __launch_bounds__ argument is the minimum number of waves per SIMD (EU):
  // two workgroups of NWAVE waves on the CU's four SIMDs need ceil(2 * NWAVE / 4); a
  // workgroup that has the CU alone asks for no more than one.
  static constexpr int WG_PER_CU = (RING_KB <= 64 && BF16) ? 2 : 1;
  static constexpr int MIN_WAVES_PER_EU = WG_PER_CU == 2 ? (2 * NWAVE + 3) / 4 : 1;
  static constexpr int NBUF_VM = 1 + 63 / LPW;
  static constexpr int NBUF_LDS = RING_KB * 1024 / TILE_BYTES;
  static constexpr int NBUF_CAP = 8;
  static constexpr int NBUF = NBUF_VM < NBUF_LDS ? (NBUF_VM < NBUF_CAP ? NBUF_VM : NBUF_CAP)
                                                 : (NBUF_LDS < NBUF_CAP ? NBUF_LDS : NBUF_CAP);
  static constexpr int KFC = NCHK / 4;            // K chunks per lane (a quarter row)
  static constexpr int MERGE_BYTES = ((NTG - 1) * RP * D + 2 * NTG * RP) * 4;
  static constexpr int RING_BYTES =
      NBUF * TILE_BYTES > MERGE_BYTES ? NBUF * TILE_BYTES : MERGE_BYTES;
  static constexpr int DESC_OFF = RING_BYTES;                            // int2 per block
  static constexpr int BT_OFF = DESC_OFF + kAttnMaxBlocksPerSplit * 8;   // staged table row
  static constexpr int FLAG_OFF = BT_OFF + kBtStageMax * 4;
  static constexpr int LDS_BYTES = FLAG_OFF + 16;
  static constexpr int BT_PER = (kBtStageMax + NT - 1) / NT;
  static_assert(NBUF >= 2, "need at least double buffering");
  static_assert(RING_BYTES >= kTopkLdsBytes, "the top-k scratch lives in the ring");
  static_assert(TILE_CH % NT == 0, "tile must split evenly over the lanes");
  static_assert(KCH % 64 == 0, "a wave load must not straddle K and V");
  static_assert((NBUF - 1) * LPW < 64, "vmcnt range");
  static_assert(NCHK >= 8 && NCHK <= 32, "swizzle cases");
};

template <int NCH>
__device__ __forceinline__ int swz_k(int r) {
  // The 16 rows one K-operand read touches are tau(mt, 0..15) + 32*grp; mu maps
  // them to 0..15.
  const int mu = (r & 3) | (((r >> 3) & 3) << 2);
  return NCH >= 16 ? mu : (mu >> 1);
}

// V rows (tokens) of a tile, XOR-swizzled in 16-byte chunks for the V^T operand reads.
// bf16: a transposing read (ds_read_b64_tr_b16) makes each 16-lane group fetch 4 token
// rows x 32 bytes (one pair of chunks), and the wave's four groups take rows 8*g4 + 4h
// + 0..3 of a 32-token group. XOR-ing the pair index with a 3-bit function of the row
// (2 bits for 128-byte rows, together with the row's parity) puts the 8 rows that
// lanes 0-31 fetch, and those of lanes 32-63, on 8 distinct 32-byte bank windows, and
// every 16-lane group's 4 rows on 4. fp32: one 4-byte read per lane; the 16 lanes of a
// group read 64 bytes of row 8*g4 + jj, and XOR-ing the 64-byte window with g4 gives
// the four groups distinct banks.
template <class C>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (C::BF16) {
    const int f = C::NCHK >= 16 ? ((r & 3) | (((r >> 3) & 1) << 2))
                                : (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
    return 2 * f;
  } else {
    return 4 * ((r >> 3) & 3);
  }
}

// Token (within a 32-token group) held by MFMA M-row m of M-tile mt, chosen so that
// lane l of the S^T result holds tokens 8*(l/16) .. 8*(l/16)+7.
__device__ __forceinline__ int tau(int mt, int m) { return 8 * (m >> 2) + 4 * mt + (m & 3); }

__device__ __forceinline__ uint4 lds_read16(const char* base, int chunk) {
  return *reinterpret_cast<const uint4*>(base + chunk * 16);
}

// Waits until the tile that has n_after (0 .. NBUF-2) younger tiles in flight has
// landed: at most n_after * LPW DMA loads may still be outstanding.
template <class C, int N = C::NBUF - 2>
__device__ __forceinline__ void wait_for_tile(int n_after) {
  if constexpr (N <= 0) {
    gmem::wait_vmcnt<0>();
  } else {
    if (n_after >= N) {
      gmem::wait_vmcnt<N * C::LPW>();
      return;
    }
    wait_for_tile<C, N - 1>(n_after);
  }
}

// Running softmax state of one wave: O^T accumulators, row max (log2 units, scaled)
// and the lane-partial denominators.
template <class C>
struct WaveState {
  f32x4 o[C::NMD][C::NN];
  float m[C::NN];
  float l[C::NN];
};

// 4 x 16-bit elements per lane from LDS through the gfx950 transposing read: within
// each 16-lane group, lane i receives element i % 4 of the 8 bytes fetched by lanes
// i/4, i/4 + 4, i/4 + 8 and i/4 + 12 of the group (in that order).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(
          (__attribute__((address_space(3))) char*)(const_cast<char*>(p))));
}

// One 32-token group of one tile for one wave. MASKED: tokens >= nvalid (and, for
// the draft tile, drafts the row's draft does not see: bit u of tvis) are excluded.
// K and V are token-major in LDS ([TT][D], K rows swizzled by swz_k, V rows by swz_v).
template <class C, bool MASKED, bool DRAFT>
__device__ __forceinline__ void attend_group(WaveState<C>& st, const char* kbase,
                                             const char* vbase, int grp, int nvalid,
                                             const uint4 (&qf)[C::NN][C::KFC],
                                             const uint32_t (&tvis)[C::NN], float c, int l16,
                                             int g4) {
  const int tok0 = grp * 32 + 8 * g4;   // the lane's 8 tokens: tok0 .. tok0 + 7
  // The group's K fragments are requested together; the V fragments are requested
  // once the S^T MFMAs are issued (they overlap the MFMAs and the softmax, and reuse
  // the K fragments' registers).
  uint4 kf[2][C::KFC];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = grp * 32 + tau(mt, l16);
#pragma unroll
    for (int kc = 0; kc < C::KFC; ++kc)
      kf[mt][kc] = lds_read16(kbase, r * C::NCHK + ((C::KFC * g4 + kc) ^ swz_k<C::NCHK>(r)));
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- S^T = K Q^T
  f32x4 sacc[2][C::NN];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < C::KFC; ++kc) {
        if constexpr (C::BF16) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[mt][kc]),
                                                        __builtin_bit_cast(bf16x8_t, qf[nt][kc]),
                                                        acc, 0, 0, 0);
        } else {
          const f32x4 ka = __builtin_bit_cast(f32x4, kf[mt][kc]);
          const f32x4 qa = __builtin_bit_cast(f32x4, qf[nt][kc]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], qa[e], acc, 0, 0, 0);
        }
      }
      sacc[mt][nt] = acc;
    }
  }

  // ---- V^T fragments: lane (g4, l16) needs head dim md*16 + l16 of tokens tok0..+7.
  // bf16: two transposing reads per md (h = 0, 1); lane j of the 16-lane group g4
  // fetches token row tok0 + 4h + j/4 at head dims md*16 + 4*(j%4) .. +3, so lane i of
  // the group receives head dim md*16 + i of those 4 rows, in token order. fp32: one
  // 4-byte read per (md, token).
  constexpr int NV = C::BF16 ? 1 : 2;   // 16-byte registers per md
  uint4 vf[C::NMD][NV];
#pragma unroll
  for (int md = 0; md < C::NMD; ++md) {
    if constexpr (C::BF16) {
      s16x4 half[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = tok0 + 4 * h + (l16 >> 2);
        const int ch = 2 * md + ((l16 & 3) >> 1);
        half[h] = lds_read_tr16(vbase + (r * C::NCHK + (ch ^ swz_v<C>(r))) * 16 + 8 * (l16 & 1));
      }
      vf[md][0] = __builtin_bit_cast(uint4, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3,
                                                                   4, 5, 6, 7));
    } else {
      float v[8];
      const int ch = md * 4 + (l16 >> 2);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = tok0 + jj;
        v[jj] = *reinterpret_cast<const float*>(vbase + (r * C::NCHK + (ch ^ swz_v<C>(r))) * 16 +
                                                4 * (l16 & 3));
      }
      vf[md][0] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                             __float_as_uint(v[3]));
      vf[md][NV - 1] = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]),
                                  __float_as_uint(v[6]), __float_as_uint(v[7]));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- online softmax; the lane holds tokens tok0 + 0..7 of row l16. Scores are
  // raw dot products; c = scale * log2(e) > 0 commutes with the max.
  float pv[C::NN][8];
#pragma unroll
  for (int nt = 0; nt < C::NN; ++nt) {
    float s[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float x = sacc[jj >> 2][nt][jj & 3];
      if constexpr (MASKED) {
        const int tok = tok0 + jj;
        const bool vis = tok < nvalid && (!DRAFT || ((tvis[nt] >> (tok & 31)) & 1u));
        s[jj] = vis ? x : -__builtin_inff();
      } else {
        s[jj] = x;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                     fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = max_over_row_lanes(mx);
    const float mnew = fmaxf(st.m[nt], mx * c);
    const float msafe = mnew == -__builtin_inff() ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(st.m[nt] - msafe);
    float ls = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      pv[nt][jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jj], c, -msafe));
      ls += pv[nt][jj];
    }
    st.l[nt] = st.l[nt] * alpha + ls;
    st.m[nt] = mnew;
    // Rescale the accumulators only if some row's max moved (exact skip).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int md = 0; md < C::NMD; ++md) st.o[md][nt] *= alpha;
    }
  }

  // ---- O^T += V^T P^T
  if constexpr (C::BF16) {
    bf16x8_t pf[C::NN];
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pf[nt][jj] = static_cast<__bf16>(pv[nt][jj]);
#pragma unroll
    for (int md = 0; md < C::NMD; ++md)
#pragma unroll
      for (int nt = 0; nt < C::NN; ++nt)
        st.o[md][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, vf[md][0]), pf[nt], st.o[md][nt], 0, 0, 0);
  } else {
#pragma unroll
    for (int md = 0; md < C::NMD; ++md) {
      const f32x4 v0 = __builtin_bit_cast(f32x4, vf[md][0]);
      const f32x4 v1 = __builtin_bit_cast(f32x4, vf[md][NV - 1]);
#pragma unroll
      for (int nt = 0; nt < C::NN; ++nt) {
        f32x4 acc = st.o[md][nt];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v0[e], pv[nt][e], acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v1[e], pv[nt][4 + e], acc, 0, 0, 0);
        st.o[md][nt] = acc;
      }
    }
  }
}

template <class C, bool TOPK>
__global__ __launch_bounds__(C::NT, C::MIN_WAVES_PER_EU) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  constexpr int ES = C::ES;
  constexpr int D = C::D;
  constexpr int TT = C::TT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave / C::NTG;
  const int tg = wave % C::NTG;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int S = p.S;                  // context splits
  const int NP = S > 1 ? S + 1 : 1;   // workgroups per unit (+1: the draft-only split)
  // Linear workgroup id -> (unit, split); with xcd_group all workgroups of unit u
  // have linear ids congruent to u mod 8 (same XCD).
  int unit, split;
  {
    const int lin = blockIdx.x;
    if (p.xcd_group) {
      const int slot = lin >> 3;
      unit = (slot / NP) * 8 + (lin & 7);
      split = slot - (slot / NP) * NP;
    } else {
      unit = lin / NP;
      split = lin - unit * NP;
    }
  }
  const int b = unit / p.Hkv;
  const int g = unit - b * p.Hkv;
  const bool draft_split = S > 1 && split == S;
  const int tpb = p.bs / TT;

  // Tile slots [s_begin, s_end) of this split, from k_max alone (balanced), and the
  // selected positions q0 .. q0+nblk-1 they fall in.
  const int n_slots = p.k_max * tpb;
  int s_begin = 0, s_end = 0;
  if (!draft_split) {
    s_begin = static_cast<int>(static_cast<int64_t>(split) * n_slots / S);
    s_end = static_cast<int>(static_cast<int64_t>(split + 1) * n_slots / S);
  }
  const int q0 = s_begin / tpb;
  int nblk = s_end > s_begin ? (s_end - 1) / tpb - q0 + 1 : 0;
  if (nblk > kAttnMaxBlocksPerSplit) nblk = kAttnMaxBlocksPerSplit;   // never for valid S

  // ---------------------------------------------------------------- prologue
  // Every request below is independent of the others: scalar context length (and
  // selected count), the block-table row (staged in LDS when short enough), the
  // split's block indices or the unit's scores, and the query fragments.
  const cint_ptr s_ctx = (cint_ptr)(p.ctx_lens);
  int ctx = s_ctx[b];
  // In-launch merge: the unit's launch epoch (its parity picks the arrival word).
  uint32_t epoch = 0u;
  if (p.merge == kMergeWait || p.merge == kMergeLast)
    epoch = __hip_atomic_load(p.tickets + static_cast<int64_t>(unit) * kTicketStride + kEpochWord,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int nsel_in = 0;
  if constexpr (!TOPK) {
    const cint_ptr s_cnt = (cint_ptr)(p.cnt);
    nsel_in = s_cnt[unit];
  }

  const int32_t* gbt = p.block_table + static_cast<int64_t>(b) * p.NB;
  int* bt_lds = reinterpret_cast<int*>(smem + C::BT_OFF);
  const bool bt_staged = p.NB <= kBtStageMax;
  int btv[C::BT_PER];
  if (bt_staged) {
#pragma unroll
    for (int u = 0; u < C::BT_PER; ++u) {
      const int i = tid + u * C::NT;
      btv[u] = i < p.NB ? gbt[i] : 0;
    }
  }

  int jv = -1;
  const int32_t* gidx = TOPK ? nullptr : p.idx + static_cast<int64_t>(unit) * p.k_max + q0;
  float sc[kWaveTopkMax / C::NT];
  const bool selector = TOPK && !draft_split;   // the whole workgroup selects
  if constexpr (TOPK) {
    if (selector)
      wg_topk_load<C::NWAVE>(p.scores + static_cast<int64_t>(unit) * p.NB,
                             p.NB < kWaveTopkMax ? p.NB : kWaveTopkMax, sc);
  } else {
    if (tid < nblk) jv = gidx[tid];
  }

  // Row r of this wave's N-tile nt: (draft t, head hl) = (row / G, row % G). tvis:
  // the drafts draft t sees, as bits: 0..t (a chain), or the caller's draft_mask row
  // (a tree: t's ancestors), t itself always. Padding rows see every draft.
  const int row0 = rg * C::RW;
  uint4 qf[C::NN][C::KFC];
  uint32_t tvis[C::NN];
  {
    const char* qbase = static_cast<const char*>(p.q);
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt) {
      const int row = row0 + nt * 16 + l16;
      const int t = row / p.G;
      const bool ok = row < p.R;
      if (p.draft_mask)
        tvis[nt] = ok ? (static_cast<uint32_t>(p.draft_mask[b * p.T + t]) | (1u << t)) : ~0u;
      else
        tvis[nt] = ok ? (2u << t) - 1u : ~0u;
      const int h = g * p.G + (row - t * p.G);
      const char* src = qbase + ((static_cast<int64_t>(b) * p.T + t) * p.Hq + h) * D * ES;
#pragma unroll
      for (int kc = 0; kc < C::KFC; ++kc)
        qf[nt][kc] = ok ? *reinterpret_cast<const uint4*>(src + (C::KFC * g4 + kc) * 16)
                        : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  if (ctx < 0) ctx = 0;
  int nb = (ctx + p.bs - 1) / p.bs;
  if (nb > p.NB) nb = p.NB;
  if (bt_staged) {
#pragma unroll
    for (int u = 0; u < C::BT_PER; ++u) {
      const int i = tid + u * C::NT;
      if (i < p.NB) bt_lds[i] = btv[u];
    }
  }
  gmem::wait_vmcnt<0>();
  lds_barrier();

  // Block descriptors of this split: desc[q] = (physical block, valid tokens of the
  // block) for selected position q0 + q, or (0, -1) for an index outside [0, nb) or
  // a bad table entry.
  int2* desc = reinterpret_cast<int2*>(smem + C::DESC_OFF);
  // The table row is read from LDS when staged; the two sources stay in separate
  // code paths so each compiles to its own instruction (a pointer chosen at run
  // time between them would become a generic access that waits for all memory).
  auto desc_of = [&](int j, int pb) {
    const bool ok = j >= 0 && j < nb && pb >= 0 && pb < p.P;
    return ok ? make_int2(pb, ctx - j * p.bs) : make_int2(0, -1);
  };
  auto clamp_j = [&](int j) { return (j >= 0 && j < nb) ? j : 0; };
  int nsel;
  if constexpr (TOPK) {
    // Budget + exact top-k of the unit (the whole workgroup); this split keeps the
    // positions it owns, split 0 publishes the indices and the count.
    nsel = 0;
    if (selector) {
      int k = budget_blocks_dev(ctx, nb, p.dense_ctx, p.min_blocks, p.frac_per_mille);
      if (k > p.k_max) k = p.k_max;
      int32_t* idx_out = p.idx_out + static_cast<int64_t>(unit) * p.k_max;
      const bool publish = split == 0;
      // The table row is staged (the fused mode requires NB <= kBtStageMax); the LDS
      // scratch is the start of the tile ring (no DMA is in flight yet).
      int total = wg_topk_select<C::NWAVE>(
          sc, nb, k, p.keep_first, p.keep_last, smem, [&](int j, int pos) {
            if (pos >= q0 && pos < q0 + nblk) desc[pos - q0] = desc_of(j, bt_lds[clamp_j(j)]);
            if (publish && pos < p.k_max) idx_out[pos] = j;
          });
      total = __builtin_amdgcn_readfirstlane(total);
      if (total > p.k_max) total = p.k_max;
      if (publish) {
        for (int pos = total + tid; pos < p.k_max; pos += C::NT) idx_out[pos] = -1;
        if (tid == 0) p.cnt_out[unit] = total;
      }
      nsel = total;
    }
    lds_barrier();
  } else {
    if (bt_staged) {
      for (int i = tid; i < nblk; i += C::NT) {
        const int j = i == tid ? jv : gidx[i];
        desc[i] = desc_of(j, bt_lds[clamp_j(j)]);
      }
    } else {
      for (int i = tid; i < nblk; i += C::NT) {
        const int j = i == tid ? jv : gidx[i];
        desc[i] = desc_of(j, gbt[clamp_j(j)]);
      }
    }
    nsel = nsel_in;
    gmem::wait_vmcnt<0>();   // nothing but the DMA stream is outstanding from here on
    lds_barrier();
  }
  if (nsel > p.k_max) nsel = p.k_max;
  if (nsel < 0) nsel = 0;
  const int nt_ctx = nsel * tpb;
  const int t_begin = s_begin < nt_ctx ? s_begin : nt_ctx;
  const int t_end = s_end < nt_ctx ? s_end : nt_ctx;
  // The draft tile: its own split when S > 1, else the single split's first tile.
  const int has_draft = (S == 1 || draft_split) ? 1 : 0;
  const int ntiles = (t_end - t_begin) + has_draft;

  const char* kpool = static_cast<const char*>(p.k_pool);
  const char* vpool = static_cast<const char*>(p.v_pool);
  const char* kdraft = static_cast<const char*>(p.k_draft) +
                       (static_cast<int64_t>(b) * p.T * p.Hkv + g) * D * ES;
  const char* vdraft = static_cast<const char*>(p.v_draft) +
                       (static_cast<int64_t>(b) * p.T * p.Hkv + g) * D * ES;
  const int64_t draft_row = static_cast<int64_t>(p.Hkv) * D * ES;   // bytes between drafts
  const uint32_t smem_base = gmem::lds_address(smem);

  // Tile i of this split: the draft tile first (if owned), then context tiles.
  // Context tile -> physical block, token offset inside it, valid tokens (0 for a
  // bad block index; such a tile still moves LPW loads from block 0 so the vmcnt
  // accounting stays uniform, and is not computed).
  auto ctx_tile = [&](int i, int& phys, int& tt0, int& nvalid) {
    const int ti = t_begin + i - has_draft;
    const int q = ti / tpb;
    tt0 = (ti - q * tpb) * TT;
    int qi = q - q0;
    if (qi >= kAttnMaxBlocksPerSplit) qi = kAttnMaxBlocksPerSplit - 1;   // never for valid S
    const int2 d = desc[qi];
    phys = __builtin_amdgcn_readfirstlane(d.x);
    const int avail = __builtin_amdgcn_readfirstlane(d.y);
    const int n = avail - tt0;
    nvalid = avail < 0 ? 0 : (n < 0 ? 0 : (n > TT ? TT : n));
  };

  // Per-lane source offsets of the LPW context-tile loads: the same for every tile
  // (only the block base changes), so they are computed once, as 32-bit offsets from
  // the wave-uniform block base.
  uint32_t dma_off[C::LPW];
#pragma unroll
  for (int u = 0; u < C::LPW; ++u) {
    const int cbase = (u * C::NWAVE + wave) * 64;
    const int ch = cbase + lane;
    const bool is_k = cbase < C::KCH;
    const int q = is_k ? ch : ch - C::KCH;
    const int r = q / C::NCHK;
    dma_off[u] = r * (D * ES) + ((q % C::NCHK) ^ (is_k ? swz_k<C::NCHK>(r) : swz_v<C>(r))) * 16;
  }

  auto issue = [&](int i, int buf) {
    const uint32_t lbase = smem_base + buf * C::TILE_BYTES;
    if (has_draft && i == 0) {
      // Draft tile: rows are draft tokens, laid out as a context tile; rows >= T
      // re-read draft 0 (finite data, masked out of the softmax).
#pragma unroll
      for (int u = 0; u < C::LPW; ++u) {
        const int cbase = (u * C::NWAVE + wave) * 64;
        const int ch = cbase + lane;
        const bool is_k = cbase < C::KCH;
        const int q = is_k ? ch : ch - C::KCH;
        const int r = q / C::NCHK;
        const int cc = (q % C::NCHK) ^ (is_k ? swz_k<C::NCHK>(r) : swz_v<C>(r));
        const char* base = is_k ? kdraft : vdraft;
        gmem::dma16(base, static_cast<uint32_t>((r < p.T ? r : 0) * draft_row + cc * 16),
               lbase + cbase * 16);
      }
    } else {
      int phys, tt0, nv;
      ctx_tile(i, phys, tt0, nv);
      const int64_t blk = static_cast<int64_t>(phys) * p.Hkv + g;
      const char* kb = kpool + (blk * p.bs + tt0) * D * ES;
      const char* vb = vpool + (blk * p.bs + tt0) * D * ES;
#pragma unroll
      for (int u = 0; u < C::LPW; ++u) {
        const int cbase = (u * C::NWAVE + wave) * 64;
        gmem::dma16(cbase < C::KCH ? kb : vb, dma_off[u], lbase + cbase * 16);
      }
    }
  };

  // Zero the V rows of tokens >= nvalid in buffer buf (partly filled last block): the
  // pool holds arbitrary bits there and P = 0 must not meet a NaN.
  auto zero_tail = [&](int buf, int nvalid) {
    char* vbase = smem + buf * C::TILE_BYTES + C::KCH * 16;
    for (int e = nvalid * C::NCHK + tid; e < TT * C::NCHK; e += C::NT)
      *reinterpret_cast<uint4*>(vbase + e * 16) = make_uint4(0u, 0u, 0u, 0u);
  };

  WaveState<C> st;
#pragma unroll
  for (int nt = 0; nt < C::NN; ++nt) {
    st.m[nt] = -__builtin_inff();
    st.l[nt] = 0.0f;
#pragma unroll
    for (int md = 0; md < C::NMD; ++md) st.o[md][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c = p.scale_log2;

  // ---------------------------------------------------------------- tile loop
#pragma unroll
  for (int i = 0; i < C::NBUF - 1; ++i)
    if (i < ntiles) issue(i, i);

  for (int it = 0; it < ntiles; ++it) {
    int last_issued = it + C::NBUF - 2;
    if (last_issued > ntiles - 1) last_issued = ntiles - 1;
    wait_for_tile<C>(last_issued - it);
    lds_barrier();                      // tile `it` landed for all waves; it-1 done
    const int nxt = it + C::NBUF - 1;
    if (nxt < ntiles) issue(nxt, nxt % C::NBUF);

    const int buf = it % C::NBUF;
    const char* kbase = smem + buf * C::TILE_BYTES;
    const char* vbase = kbase + C::KCH * 16;
    if (has_draft && it == 0) {
#pragma unroll 1
      for (int grp = tg; grp < C::NGRP; grp += C::NTG) {
        if (grp * 32 >= p.T) break;
        attend_group<C, true, true>(st, kbase, vbase, grp, p.T, qf, tvis, c, l16, g4);
      }
      continue;
    }
    int phys, tt0, nvalid;
    ctx_tile(it, phys, tt0, nvalid);
    if (nvalid == TT) {
#pragma unroll 1
      for (int grp = tg; grp < C::NGRP; grp += C::NTG)
        attend_group<C, false, false>(st, kbase, vbase, grp, TT, qf, tvis, c, l16, g4);
    } else if (nvalid > 0) {
      zero_tail(buf, nvalid);
      lds_barrier();
#pragma unroll 1
      for (int grp = tg; grp < C::NGRP; grp += C::NTG) {
        if (grp * 32 >= nvalid) break;
        attend_group<C, true, false>(st, kbase, vbase, grp, nvalid, qf, tvis, c, l16, g4);
      }
    }
  }
  lds_barrier();   // every wave is done with the tile buffers

  // ---------------------------------------------------------------- finish
#pragma unroll
  for (int nt = 0; nt < C::NN; ++nt) st.l[nt] = sum_over_row_lanes(st.l[nt]);

  if constexpr (C::NTG > 1) {
    // Combine the waves that share a row group: stats[tg][row][2], then the O^T
    // accumulators of waves tg > 0 as [tg-1][row][D].
    float* stats = reinterpret_cast<float*>(smem);
    float* olds = stats + 2 * C::NTG * C::RP;
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt) {
      const int row = row0 + nt * 16 + l16;
      if (g4 == 0) {
        stats[(tg * C::RP + row) * 2 + 0] = st.m[nt];
        stats[(tg * C::RP + row) * 2 + 1] = st.l[nt];
      }
      if (tg > 0) {
#pragma unroll
        for (int md = 0; md < C::NMD; ++md)
          *reinterpret_cast<f32x4*>(olds + (static_cast<int64_t>(tg - 1) * C::RP + row) * D +
                                    md * 16 + 4 * g4) = st.o[md][nt];
      }
    }
    lds_barrier();
    if (tg == 0) {
#pragma unroll
      for (int nt = 0; nt < C::NN; ++nt) {
        const int row = row0 + nt * 16 + l16;
        float mmax = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < C::NTG; ++w) mmax = fmaxf(mmax, stats[(w * C::RP + row) * 2]);
        const float msafe = mmax == -__builtin_inff() ? 0.0f : mmax;
        const float a0 = __builtin_amdgcn_exp2f(st.m[nt] - msafe);
        float l = st.l[nt] * a0;
#pragma unroll
        for (int md = 0; md < C::NMD; ++md) st.o[md][nt] *= a0;
#pragma unroll
        for (int w = 1; w < C::NTG; ++w) {
          const float aw = __builtin_amdgcn_exp2f(stats[(w * C::RP + row) * 2] - msafe);
          l += stats[(w * C::RP + row) * 2 + 1] * aw;
#pragma unroll
          for (int md = 0; md < C::NMD; ++md)
            st.o[md][nt] += aw * *reinterpret_cast<const f32x4*>(
                                     olds + (static_cast<int64_t>(w - 1) * C::RP + row) * D +
                                     md * 16 + 4 * g4);
        }
        st.m[nt] = mmax;
        st.l[nt] = l;
      }
    }
  }

  // ---------------------------------------------------------------- write
  const bool writer = tg == 0;
  if (S == 1) {
    if (!writer) return;
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt) {
      const int row = row0 + nt * 16 + l16;
      if (row >= p.R) continue;
      const int t = row / p.G;
      const int h = g * p.G + (row - t * p.G);
      const float inv = 1.0f / st.l[nt];
      const int64_t o = ((static_cast<int64_t>(b) * p.T + t) * p.Hq + h) * D;
#pragma unroll
      for (int md = 0; md < C::NMD; ++md) {
        const f32x4 v = st.o[md][nt] * inv;
        if constexpr (C::BF16) {
          bf16x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = static_cast<__bf16>(v[e]);
          *reinterpret_cast<bf16x4_t*>(static_cast<char*>(p.out) + (o + md * 16 + 4 * g4) * 2) = w;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o + md * 16 + 4 * g4) = v;
        }
      }
      if (p.lse && g4 == 0)
        p.lse[(static_cast<int64_t>(b) * p.T + t) * p.Hq + h] =
            (st.m[nt] + __builtin_log2f(st.l[nt])) * kLn2;
    }
    return;
  }

  // Partial of this split: O (unnormalised), running max (log2 units), denominator.
  // kMergeKernel: plain stores for merge_kernel (with XCD grouping its workgroups for
  // the unit run on the same XCD and find them in its L2). kMergeWait / kMergeLast:
  // device-scope stores, then the in-launch merge below.
  const bool ink = p.merge == kMergeWait || p.merge == kMergeLast;
  const int part_bytes = NP * p.R * D * 4;
  const __amdgpu_buffer_rsrc_t po =
      make_rsrc(p.part_o + static_cast<int64_t>(unit) * NP * p.R * D, part_bytes);
  const __amdgpu_buffer_rsrc_t pml =
      make_rsrc(p.part_ml + static_cast<int64_t>(unit) * NP * p.R * 2, NP * p.R * 8);
  if (writer) {
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt) {
      const int row = row0 + nt * 16 + l16;
      if (row >= p.R) continue;
      const int prow = split * p.R + row;
#pragma unroll
      for (int md = 0; md < C::NMD; ++md) {
        const int off = (prow * D + md * 16 + 4 * g4) * 4;
        if (ink) store4<kDeviceScope>(po, off, st.o[md][nt]);
        else     store4<0>(po, off, st.o[md][nt]);
      }
      if (g4 == 0) {
        const float2 ml = make_float2(st.m[nt], st.l[nt]);
        if (ink) store2<kDeviceScope>(pml, prow * 8, ml);
        else     store2<0>(pml, prow * 8, ml);
      }
    }
  }
  if (!ink) return;

  // ---------------------------------------------------------------- in-launch merge
  // Memory ordering. Partials cross workgroups (and XCDs) only through device-scope
  // accesses: they are stored with sc1 buffer stores, which write through this XCD's
  // L2, and the workgroup waits for those stores to complete (vmcnt(0)) before its
  // arrival atomic; they are read back with sc1 buffer loads, which do not hit a
  // stale line in the reader's L1 or L2. Together this stands in for a release
  // (arrival) / acquire (seeing the arrival) pair at agent scope: since both sides
  // carry the device scope themselves, no L2 writeback (buffer_wbl2) or invalidate
  // (buffer_inv) is needed. The control words are agent-scope atomics.
  //
  // Protocol. Arrival word A = line[kArriveWord0 + 2 * (epoch & 1)]: low 32 bits count
  // the unit's workgroups whose partials are stored, high 32 bits mark slices handed
  // to the last arriver. Each workgroup adds 1 to A. The one that brings the count to
  // NP is the last arriver: every partial is stored, and it merges its own slice plus
  // every slice marked in the value it replaced. In kMergeWait every other workgroup
  // polls A until the count reaches NP and then merges its own slice; if that takes
  // longer than merge_wait_ticks (a sibling is not running: the grid is not resident,
  // for instance because other kernels hold CUs), it marks its slice in A with a
  // compare-and-swap and leaves, unless the count reached NP first. A mark can only
  // precede the last arrival, so every slice is merged exactly once and no wait is
  // unbounded. In kMergeLast the others leave at once and the last arriver merges all.
  // The last arriver then clears the other arrival word (no workgroup of this launch
  // uses it; every sibling read this launch's epoch before arriving) and advances the
  // epoch, which the next launch on this workspace reads.
  gmem::wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_barrier();
  uint32_t* line = p.tickets + static_cast<int64_t>(unit) * kTicketStride;
  const uint32_t ep = __builtin_amdgcn_readfirstlane(epoch);
  uint64_t* arrive = reinterpret_cast<uint64_t*>(line + kArriveWord0) + (ep & 1u);
  int* flag = reinterpret_cast<int*>(smem + C::FLAG_OFF);
  // flag[0]: 0 = leave, 1 = merge the own slice, 2 = last arriver; flag[1]: handed slices.
  if (tid == 0) {
    const uint64_t old =
        __hip_atomic_fetch_add(arrive, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int mode = 1;
    uint32_t handed = 0u;
    if (static_cast<uint32_t>(old) + 1u == static_cast<uint32_t>(NP)) {
      mode = 2;
      handed = static_cast<uint32_t>(old >> 32);
    } else if (p.merge == kMergeLast) {
      mode = 0;
    } else {
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + p.merge_wait_ticks;
      for (;;) {
        uint64_t cur = __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (static_cast<uint32_t>(cur) == static_cast<uint32_t>(NP)) break;
        if (__builtin_amdgcn_s_memrealtime() > t_end) {
          // Hand the slice over, unless the last sibling arrives first. A failed
          // exchange means another workgroup changed A (an arrival or a hand-over, at
          // most 2 * NP of them), so this loop ends.
          while (static_cast<uint32_t>(cur) != static_cast<uint32_t>(NP)) {
            const uint64_t want = cur | (1ull << (32 + split));
            if (__hip_atomic_compare_exchange_strong(arrive, &cur, want, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
              mode = 0;
              break;
            }
          }
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
    }
    flag[0] = mode;
    flag[1] = static_cast<int>(handed);
  }
  lds_barrier();
  const int mode = __builtin_amdgcn_readfirstlane(flag[0]);
  const uint32_t handed = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(flag[1]));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (mode == 0) return;

  // Rows of slice s: [s * rpw, s * rpw + rpw) (kMergeLast: the last arriver takes all).
  const int rpw = p.merge == kMergeLast ? p.R : (p.R + NP - 1) / NP;
  auto merge_rows = [&](int rb, int re) {
    for (int i4 = tid; i4 < (re - rb) * (D / 4); i4 += C::NT) {
      const int row = rb + i4 / (D / 4);
      const int dim = (i4 - (row - rb) * (D / 4)) * 4;
      float lse2;
      const f32x4 v = combine_partials<kDeviceScope>(po, pml, NP, p.R, D, row, dim, &lse2);
      const int t = row / p.G;
      const int h = g * p.G + (row - t * p.G);
      const int64_t ob = (static_cast<int64_t>(b) * p.T + t) * p.Hq + h;
      store_out4<C::BF16>(p.out, ob * D + dim, v);
      if (p.lse && dim == 0) p.lse[ob] = lse2 * kLn2;
    }
  };
  auto slice = [&](int s_) {
    const int rb = p.merge == kMergeLast ? 0 : s_ * rpw;
    const int re = rb + rpw < p.R ? rb + rpw : p.R;
    if (rb < re) merge_rows(rb, re);
  };
  slice(split);
  if (mode == 2) {
    if (p.merge == kMergeWait) {
      for (uint32_t m = handed; m != 0u; m &= m - 1u) slice(__builtin_ctz(m));
    }
    if (tid == 0) {
      __hip_atomic_store(reinterpret_cast<uint64_t*>(line + kArriveWord0) + ((ep + 1u) & 1u), 0ull,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(line + kEpochWord, ep + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Combine the S partials of every (unit, row) in one pass over the splits, sixteen
// splits per batch of loads (a running max rescales the accumulated sum across
// batches). One thread per 4 head dims.
constexpr int kMergeThreads = 64;

template <bool BF16>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnParams p) {
  const int D = p.D;
  const int per_unit = (p.R * D / 4 + kMergeThreads - 1) / kMergeThreads;   // workgroups
  int unit, blk;
  {
    const int lin = blockIdx.x;
    if (p.xcd_group) {
      const int slot = lin >> 3;
      unit = (slot / per_unit) * 8 + (lin & 7);
      blk = slot - (slot / per_unit) * per_unit;
    } else {
      unit = lin / per_unit;
      blk = lin - unit * per_unit;
    }
  }
  const int i4 = blk * kMergeThreads + threadIdx.x;
  if (i4 * 4 >= p.R * D) return;
  const int row = (i4 * 4) / D;
  const int dim = i4 * 4 - row * D;
  const int NP = p.S + 1;   // context splits plus the draft split
  const __amdgpu_buffer_rsrc_t po =
      make_rsrc(p.part_o + static_cast<int64_t>(unit) * NP * p.R * D, NP * p.R * D * 4);
  const __amdgpu_buffer_rsrc_t pml =
      make_rsrc(p.part_ml + static_cast<int64_t>(unit) * NP * p.R * 2, NP * p.R * 8);
  float lse2;
  const f32x4 v = combine_partials<0>(po, pml, NP, p.R, D, row, dim, &lse2);
  const int b = unit / p.Hkv;
  const int g = unit - b * p.Hkv;
  const int t = row / p.G;
  const int h = g * p.G + (row - t * p.G);
  const int64_t ob = (static_cast<int64_t>(b) * p.T + t) * p.Hq + h;
  store_out4<BF16>(p.out, ob * D + dim, v);
  if (p.lse && dim == 0) p.lse[ob] = lse2 * kLn2;
}

template <class C>
hipError_t launch_cfg(const AttnParams& p, hipStream_t stream) {
  dim3 grid((p.S > 1 ? p.S + 1 : 1) * p.B * p.Hkv);
  if (p.scores)
    hipLaunchKernelGGL((attn_kernel<C, true>), grid, dim3(C::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_kernel<C, false>), grid, dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16, int D, int TT, int RP>
hipError_t launch_ring(const AttnParams& p, hipStream_t stream) {
  if (attn_ring_kb(p.S, p.B * p.Hkv, p.R, BF16) == 128)
    return launch_cfg<Cfg<BF16, D, TT, RP, 128>>(p, stream);
  return launch_cfg<Cfg<BF16, D, TT, RP, 64>>(p, stream);
}

template <bool BF16, int D, int TT>
hipError_t launch_rows(const AttnParams& p, hipStream_t stream) {
  switch (attn_padded_rows(p.R)) {
    case 16: return launch_ring<BF16, D, TT, 16>(p, stream);
    case 32: return launch_ring<BF16, D, TT, 32>(p, stream);
    case 64: return launch_ring<BF16, D, TT, 64>(p, stream);
    default: return launch_cfg<Cfg<BF16, D, TT, 128, 128>>(p, stream);   // always one per CU
  }
}

template <bool BF16>
hipError_t launch_dtype(const AttnParams& p, hipStream_t stream) {
  if constexpr (BF16) {
    const int tt = attn_tile_tokens(p.bs, true, p.R);
    if (tt == 128) {   // 128-row units only: one workgroup per CU, 128 KB ring of 2 tiles
      if (p.D == 128) return launch_cfg<Cfg<true, 128, 128, 128, 128>>(p, stream);
      return launch_cfg<Cfg<true, 64, 128, 128, 128>>(p, stream);
    }
    const bool t64 = tt == 64;
    if (p.D == 128)
      return t64 ? launch_rows<true, 128, 64>(p, stream) : launch_rows<true, 128, 32>(p, stream);
    return t64 ? launch_rows<true, 64, 64>(p, stream) : launch_rows<true, 64, 32>(p, stream);
  } else {
    return p.D == 128 ? launch_rows<false, 128, 32>(p, stream) : launch_rows<false, 64, 32>(p, stream);
  }
}

}  // namespace

int attn_merge_mode(int splits, int units, int rows, bool bf16, int cus) {
  if (splits <= 1) return kMergeNone;
  if (splits + 1 > kMaxInKernelParts) return kMergeKernel;   // one hand-over bit per workgroup
  // workgroups the launch keeps resident per CU: two with the 64 KB ring (bf16), else one
  const int per_cu = (attn_ring_kb(splits, units, rows, bf16) == 64 && bf16) ? 2 : 1;
  const int64_t grid = static_cast<int64_t>(splits + 1) * units;
  return grid <= static_cast<int64_t>(cus) * per_cu ? kMergeWait : kMergeLast;
}

hipError_t launch_attn(const AttnParams& p, bool bf16, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  hipError_t e = bf16 ? launch_dtype<true>(p, stream) : launch_dtype<false>(p, stream);
  if (e != hipSuccess || p.merge != kMergeKernel) return e;
  dim3 grid((p.R * p.D / 4 + kMergeThreads - 1) / kMergeThreads * p.B * p.Hkv);
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(kMergeThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
