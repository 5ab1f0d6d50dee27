// Split-K multi-draft verification attention over gathered KV blocks, with a
// log-sum-exp merge (sciencestack page of arXiv 2512.21911, Figure 1 caption: all
// draft tokens attend over the one shared set of selected blocks; abstract: the
// draft tokens are verified in one parallel pass).
//
// Work unit = (sequence b, KV head g). Its rows are the T x G (draft token, query
// head of the group) pairs, padded to RP in {16, 32, 64, 128}; its keys are the
// valid tokens of the selected blocks followed by the T draft tokens (draft t sees
// drafts 0..t). The keys of a unit are cut into tiles of TT tokens (one tile never
// spans two blocks); split s of S takes a contiguous range of context tiles, and
// the last split also takes the draft tile.
//
// Per workgroup: tiles stream HBM -> LDS with 16-byte LDS-DMA loads
// (global_load_lds_dwordx4), double-buffered, so the next tile is in flight while
// the current one is computed. LDS rows are XOR-swizzled in 16-byte chunks so the
// MFMA operand reads (16 lanes, 16 different rows, same chunk) hit distinct banks.
// Each wave owns RW rows and a subset of the tile's 32-token groups and computes
//   S^T = K Q^T      (MFMA, M = tokens, N = rows, K = head dim)
//   online softmax in log2 units per row (rows live on lanes, so the running max,
//   denominator and rescale factor are lane-local after a 4-lane reduction)
//   O^T += V^T P^T   (MFMA, M = head dim, N = rows, K = tokens)
// The token order inside a 32-token group is permuted so that the S^T accumulator
// a lane holds is exactly the P^T operand it must feed, and V^T (the pool keeps V
// dim-major inside a block) gives the matching operand as one 16-byte LDS read.
// bf16 uses v_mfma_f32_16x16x32_bf16, fp32 uses v_mfma_f32_16x16x4_f32; both
// accumulate in fp32.
//
// With S == 1 the workgroup normalises and writes the output; otherwise it writes
// an unnormalised partial (O, running max, denominator) and merge_kernel combines
// the S partials of a row:  O = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s.
#include "internal.h"

namespace sv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

#define SV_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr float kLn2 = 0.69314718055994530942f;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt in bits [3:0] and [15:14]; expcnt (bits [6:4]) and lgkmcnt (bits [11:8])
  // left at their maximum so they do not wait.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses but leaves outstanding global loads
// (the LDS-DMA prefetch) in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool BF16_, int D_, int TT_, int RP_>
struct Cfg {
  static constexpr bool BF16 = BF16_;
  static constexpr int D = D_;
  static constexpr int TT = TT_;           // tokens per tile
  static constexpr int RP = RP_;           // padded rows
  static constexpr int ES = BF16 ? 2 : 4;  // element bytes
  static constexpr int RW = RP < 32 ? RP : 32;   // rows per wave
  static constexpr int NRG = RP / RW;             // row groups
  static constexpr int NGRP = TT / 32;            // 32-token groups per tile
  static constexpr int NTG = NRG >= 4 ? 1 : NGRP; // waves sharing a row group
  static constexpr int NWAVE = NRG * NTG;
  static constexpr int NT = 64 * NWAVE;
  static constexpr int NN = RW / 16;              // 16-row MFMA tiles per wave
  static constexpr int NMD = D / 16;              // 16-dim MFMA tiles of O^T
  static constexpr int NCHK = D * ES / 16;        // 16-byte chunks per K row
  static constexpr int NCHV = TT * ES / 16;       // 16-byte chunks per V^T row
  static constexpr int KCH = TT * NCHK;
  static constexpr int VCH = D * NCHV;
  static constexpr int TILE_CH = KCH + VCH;
  static constexpr int TILE_BYTES = TILE_CH * 16;
  static constexpr int LPW = TILE_CH / NT;        // LDS-DMA loads per lane per tile
  static constexpr int NBUF = 2;
  static constexpr int KFC = NCHK / 4;            // K chunks per lane (a quarter row)
  static constexpr int MERGE_BYTES = ((NTG - 1) * RP * D + 2 * NTG * RP) * 4;
  static constexpr int LDS_BYTES =
      NBUF * TILE_BYTES > MERGE_BYTES ? NBUF * TILE_BYTES : MERGE_BYTES;
  static_assert(TILE_CH % NT == 0, "tile must split evenly over the lanes");
  static_assert(KCH % 64 == 0, "a wave load must not straddle K and V");
  static_assert((NBUF - 1) * LPW < 64, "vmcnt range");
  static_assert(NCHK >= 8 && NCHV >= 4 && NCHV <= 16, "swizzle cases");
};

template <int NCH>
__device__ __forceinline__ int swz_k(int r) {
  // The 16 rows one K-operand read touches are tau(mt, 0..15) + 32*grp; mu maps
  // them to 0..15.
  const int mu = (r & 3) | (((r >> 3) & 3) << 2);
  return NCH >= 16 ? mu : (mu >> 1);
}

template <int NCH>
__device__ __forceinline__ int swz_v(int r) {
  return NCH == 16 ? (r & 15) : NCH == 8 ? ((r & 15) >> 1) : ((r & 15) >> 2);
}

// Token (within a 32-token group) held by MFMA M-row m of M-tile mt. Chosen so
// that lane l of the S^T result holds tokens 8*(l/16) .. 8*(l/16)+7.
__device__ __forceinline__ int tau(int mt, int m) { return 8 * (m >> 2) + 4 * mt + (m & 3); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

__device__ __forceinline__ uint4 lds_read16(const char* base, int chunk) {
  return *reinterpret_cast<const uint4*>(base + chunk * 16);
}

template <class C>
__global__ __launch_bounds__(C::NT) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = wave / C::NTG;
  const int tg = wave % C::NTG;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / p.Hkv;
  const int g = unit - b * p.Hkv;
  const int S = p.S;

  int ctx = p.ctx_lens[b];
  if (ctx < 0) ctx = 0;
  int nb = (ctx + p.bs - 1) / p.bs;
  if (nb > p.NB) nb = p.NB;
  int nsel = p.cnt[unit];
  if (nsel > p.k_max) nsel = p.k_max;
  if (nsel < 0) nsel = 0;
  const int tpb = p.bs / C::TT;
  const int nt_ctx = nsel * tpb;
  const int tps = (nt_ctx + S - 1) / S;
  int t_begin = split * tps;
  if (t_begin > nt_ctx) t_begin = nt_ctx;
  int t_end = t_begin + tps;
  if (t_end > nt_ctx) t_end = nt_ctx;
  const int n_ctx_tiles = t_end - t_begin;
  const bool has_draft = (split == S - 1);
  const int ntiles = n_ctx_tiles + (has_draft ? 1 : 0);

  const int32_t* sel_idx = p.idx + static_cast<int64_t>(unit) * p.k_max;
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.NB;
  const char* kpool = static_cast<const char*>(p.k_pool);
  const char* vpool = static_cast<const char*>(p.v_pool);
  constexpr int ES = C::ES;
  constexpr int D = C::D;
  constexpr int TT = C::TT;

  // Context tile i of this split -> physical block, token offset, valid tokens.
  auto tile_info = [&](int i, int& phys, int& tt0, int& nvalid) {
    const int ti = t_begin + i;
    const int j = sel_idx[ti / tpb];
    tt0 = (ti - (ti / tpb) * tpb) * TT;
    phys = 0;
    nvalid = 0;
    if (j >= 0 && j < nb) {
      const int pb = bt[j];
      if (pb >= 0 && pb < p.P) {
        phys = pb;
        int n = ctx - j * p.bs - tt0;
        nvalid = n < 0 ? 0 : (n > TT ? TT : n);
      }
    }
  };

  // Asynchronous HBM -> LDS copy of context tile i into buffer buf (LPW loads per
  // lane). Tiles with no valid token still issue their loads (from block 0) so that
  // every context tile accounts for exactly LPW outstanding loads.
  auto issue_tile = [&](int i, int buf) {
    int phys, tt0, nv;
    tile_info(i, phys, tt0, nv);
    const int64_t blk = static_cast<int64_t>(phys) * p.Hkv + g;
    const char* kb = kpool + (blk * p.bs + tt0) * D * ES;
    const char* vb = vpool + blk * D * p.bs * ES + tt0 * ES;
    char* lbase = smem + buf * C::TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
      const int cbase = (u * C::NWAVE + wave) * 64;
      const int ch = cbase + lane;
      const char* src;
      if (cbase < C::KCH) {
        const int r = ch / C::NCHK;
        const int c = (ch % C::NCHK) ^ swz_k<C::NCHK>(r);
        src = kb + r * (D * ES) + c * 16;
      } else {
        const int q = ch - C::KCH;
        const int r = q / C::NCHV;
        const int c = (q % C::NCHV) ^ swz_v<C::NCHV>(r);
        src = vb + static_cast<int64_t>(r) * p.bs * ES + c * 16;
      }
      __builtin_amdgcn_global_load_lds(src, SV_LDS(lbase + cbase * 16), 16, 0, 0);
    }
  };

  // Synchronous load of the draft tile (T <= 16 tokens, natural [t][d] layout)
  // into buffer buf, transposing V; slots past T are zero.
  auto load_draft = [&](int buf) {
    char* lbase = smem + buf * C::TILE_BYTES;
    const char* kd = static_cast<const char*>(p.k_draft);
    const char* vd = static_cast<const char*>(p.v_draft);
    for (int ch = tid; ch < C::KCH; ch += C::NT) {
      const int r = ch / C::NCHK;
      const int c = ch % C::NCHK;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < p.T)
        v = *reinterpret_cast<const uint4*>(
            kd + ((static_cast<int64_t>(b) * p.T + r) * p.Hkv + g) * D * ES + c * 16);
      *reinterpret_cast<uint4*>(lbase + (r * C::NCHK + (c ^ swz_k<C::NCHK>(r))) * 16) = v;
    }
    char* vbase = lbase + C::KCH * 16;
    constexpr int EPC = 16 / ES;    // elements per chunk
    for (int ch = tid; ch < C::VCH; ch += C::NT) {
      const int r = ch / C::NCHV;   // head dim
      const int c = ch % C::NCHV;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int t = c * EPC + e;
        if (t < p.T) {
          const char* src = vd + (((static_cast<int64_t>(b) * p.T + t) * p.Hkv + g) * D + r) * ES;
          if constexpr (ES == 2) {
            const uint32_t x = *reinterpret_cast<const uint16_t*>(src);
            w[e >> 1] |= x << (16 * (e & 1));
          } else {
            w[e] = *reinterpret_cast<const uint32_t*>(src);
          }
        }
      }
      *reinterpret_cast<uint4*>(vbase + (r * C::NCHV + (c ^ swz_v<C::NCHV>(r))) * 16) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  // Zero V^T columns of tokens >= nvalid in buffer buf (partly filled last block).
  auto zero_tail = [&](int buf, int nvalid) {
    char* vbase = smem + buf * C::TILE_BYTES + C::KCH * 16;
    const int ntail = TT - nvalid;
    for (int e = tid; e < D * ntail; e += C::NT) {
      const int r = e / ntail;
      const int t = nvalid + (e - r * ntail);
      const int c = (t * ES) >> 4;
      char* dst = vbase + (r * C::NCHV + (c ^ swz_v<C::NCHV>(r))) * 16 + ((t * ES) & 15);
      if constexpr (ES == 2)
        *reinterpret_cast<uint16_t*>(dst) = 0;
      else
        *reinterpret_cast<uint32_t*>(dst) = 0u;
    }
  };

  // ---------------------------------------------------------------- Q fragments
  // Row r of this wave's N-tile nt: (draft t, head hl) = (row / G, row % G).
  const int row0 = rg * C::RW;
  const char* qbase = static_cast<const char*>(p.q);
  uint4 qf[C::NN][C::KFC];
  int trow[C::NN];
#pragma unroll
  for (int nt = 0; nt < C::NN; ++nt) {
    const int row = row0 + nt * 16 + l16;
    const int t = row / p.G;
    trow[nt] = t;
    const bool ok = row < p.R;
    const int h = g * p.G + (row - t * p.G);
    const char* src = qbase + ((static_cast<int64_t>(b) * p.T + t) * p.Hq + h) * D * ES;
#pragma unroll
    for (int kc = 0; kc < C::KFC; ++kc)
      qf[nt][kc] = ok ? *reinterpret_cast<const uint4*>(src + (C::KFC * g4 + kc) * 16)
                      : make_uint4(0u, 0u, 0u, 0u);
  }

  f32x4 oacc[C::NMD][C::NN];
  float mrow[C::NN], lrow[C::NN];
#pragma unroll
  for (int nt = 0; nt < C::NN; ++nt) {
    mrow[nt] = -__builtin_inff();
    lrow[nt] = 0.0f;
#pragma unroll
    for (int md = 0; md < C::NMD; ++md) oacc[md][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---------------------------------------------------------------- tile loop
  auto issue_any = [&](int i) {
    const int buf = i % C::NBUF;
    if (i < n_ctx_tiles) issue_tile(i, buf); else load_draft(buf);
  };
#pragma unroll
  for (int i = 0; i < C::NBUF - 1; ++i)
    if (i < ntiles) issue_any(i);

  for (int it = 0; it < ntiles; ++it) {
    const int nxt = it + C::NBUF - 1;
    if (nxt < ntiles) issue_any(nxt);
    int n_after = (n_ctx_tiles - 1 < nxt ? n_ctx_tiles - 1 : nxt) - it;
    if (n_after > 0) wait_vmcnt<C::LPW>(); else wait_vmcnt<0>();
    lds_barrier();

    const bool is_draft = it >= n_ctx_tiles;
    int nvalid;
    if (is_draft) {
      nvalid = p.T;
    } else {
      int phys, tt0;
      tile_info(it, phys, tt0, nvalid);
      if (nvalid > 0 && nvalid < TT) {
        zero_tail(it % C::NBUF, nvalid);
        lds_barrier();
      }
    }
    const char* kbase = smem + (it % C::NBUF) * C::TILE_BYTES;
    const char* vbase = kbase + C::KCH * 16;

    for (int grp = tg; grp < C::NGRP; grp += C::NTG) {
      if (grp * 32 >= nvalid) break;
      // ---- S^T = K Q^T for the 32 tokens of this group
      f32x4 sacc[2][C::NN];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = grp * 32 + tau(mt, l16);
        uint4 kf[C::KFC];
#pragma unroll
        for (int kc = 0; kc < C::KFC; ++kc)
          kf[kc] = lds_read16(kbase, r * C::NCHK + ((C::KFC * g4 + kc) ^ swz_k<C::NCHK>(r)));
#pragma unroll
        for (int nt = 0; nt < C::NN; ++nt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < C::KFC; ++kc) {
            if constexpr (C::BF16) {
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, kf[kc]), __builtin_bit_cast(bf16x8_t, qf[nt][kc]),
                  acc, 0, 0, 0);
            } else {
              const f32x4 ka = __builtin_bit_cast(f32x4, kf[kc]);
              const f32x4 qa = __builtin_bit_cast(f32x4, qf[nt][kc]);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], qa[e], acc, 0, 0, 0);
            }
          }
          sacc[mt][nt] = acc;
        }
      }
      // ---- online softmax (log2 units); lane holds tokens tok0 + 0..7 of row l16
      const int tok0 = grp * 32 + 8 * g4;
      float pv[C::NN][8];
#pragma unroll
      for (int nt = 0; nt < C::NN; ++nt) {
        float s[8];
        float mx = -__builtin_inff();
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int tok = tok0 + jj;
          const bool vis = tok < nvalid && (!is_draft || tok <= trow[nt]);
          const float x = sacc[jj >> 2][nt][jj & 3] * p.scale_log2;
          s[jj] = vis ? x : -__builtin_inff();
          mx = fmaxf(mx, s[jj]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(mrow[nt], mx);
        const float msafe = mnew == -__builtin_inff() ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrow[nt] - msafe);
        float ls = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          pv[nt][jj] = __builtin_amdgcn_exp2f(s[jj] - msafe);
          ls += pv[nt][jj];
        }
        lrow[nt] = lrow[nt] * alpha + ls;
        mrow[nt] = mnew;
#pragma unroll
        for (int md = 0; md < C::NMD; ++md) oacc[md][nt] *= alpha;
      }
      // ---- O^T += V^T P^T
      if constexpr (C::BF16) {
        bf16x8_t pf[C::NN];
#pragma unroll
        for (int nt = 0; nt < C::NN; ++nt)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) pf[nt][jj] = static_cast<__bf16>(pv[nt][jj]);
        const int vc = (tok0 * ES) >> 4;
#pragma unroll
        for (int md = 0; md < C::NMD; ++md) {
          const int r = md * 16 + l16;
          const uint4 vf = lds_read16(vbase, r * C::NCHV + (vc ^ swz_v<C::NCHV>(r)));
#pragma unroll
          for (int nt = 0; nt < C::NN; ++nt)
            oacc[md][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, vf), pf[nt], oacc[md][nt], 0, 0, 0);
        }
      } else {
        const int vc = (tok0 * ES) >> 4;
#pragma unroll
        for (int md = 0; md < C::NMD; ++md) {
          const int r = md * 16 + l16;
          const f32x4 v0 = __builtin_bit_cast(
              f32x4, lds_read16(vbase, r * C::NCHV + (vc ^ swz_v<C::NCHV>(r))));
          const f32x4 v1 = __builtin_bit_cast(
              f32x4, lds_read16(vbase, r * C::NCHV + ((vc + 1) ^ swz_v<C::NCHV>(r))));
#pragma unroll
          for (int nt = 0; nt < C::NN; ++nt) {
            f32x4 acc = oacc[md][nt];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v0[e], pv[nt][e], acc, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v1[e], pv[nt][4 + e], acc, 0, 0, 0);
            oacc[md][nt] = acc;
          }
        }
      }
    }
    lds_barrier();
  }

  // ---------------------------------------------------------------- finish
#pragma unroll
  for (int nt = 0; nt < C::NN; ++nt) {
    lrow[nt] += __shfl_xor(lrow[nt], 16, 64);
    lrow[nt] += __shfl_xor(lrow[nt], 32, 64);
  }

  if constexpr (C::NTG > 1) {
    // Combine the waves that share a row group: stats[tg][row][2], then the O^T
    // accumulators of waves tg > 0 as [tg-1][row][D].
    float* stats = reinterpret_cast<float*>(smem);
    float* olds = stats + 2 * C::NTG * C::RP;
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt) {
      const int row = row0 + nt * 16 + l16;
      if (g4 == 0) {
        stats[(tg * C::RP + row) * 2 + 0] = mrow[nt];
        stats[(tg * C::RP + row) * 2 + 1] = lrow[nt];
      }
      if (tg > 0) {
#pragma unroll
        for (int md = 0; md < C::NMD; ++md)
          *reinterpret_cast<f32x4*>(olds + (static_cast<int64_t>(tg - 1) * C::RP + row) * D +
                                    md * 16 + 4 * g4) = oacc[md][nt];
      }
    }
    lds_barrier();
    if (tg > 0) return;
#pragma unroll
    for (int nt = 0; nt < C::NN; ++nt) {
      const int row = row0 + nt * 16 + l16;
      float mmax = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < C::NTG; ++w) mmax = fmaxf(mmax, stats[(w * C::RP + row) * 2]);
      const float msafe = mmax == -__builtin_inff() ? 0.0f : mmax;
      const float a0 = __builtin_amdgcn_exp2f(mrow[nt] - msafe);
      float l = lrow[nt] * a0;
#pragma unroll
      for (int md = 0; md < C::NMD; ++md) oacc[md][nt] *= a0;
#pragma unroll
      for (int w = 1; w < C::NTG; ++w) {
        const float aw = __builtin_amdgcn_exp2f(stats[(w * C::RP + row) * 2] - msafe);
        l += stats[(w * C::RP + row) * 2 + 1] * aw;
#pragma unroll
        for (int md = 0; md < C::NMD; ++md)
          oacc[md][nt] += aw * *reinterpret_cast<const f32x4*>(
                                   olds + (static_cast<int64_t>(w - 1) * C::RP + row) * D +
                                   md * 16 + 4 * g4);
      }
      mrow[nt] = mmax;
      lrow[nt] = l;
    }
  }

  // ---------------------------------------------------------------- write
#pragma unroll
  for (int nt = 0; nt < C::NN; ++nt) {
    const int row = row0 + nt * 16 + l16;
    if (row >= p.R) continue;
    const int t = row / p.G;
    const int h = g * p.G + (row - t * p.G);
    if (S == 1) {
      const float inv = 1.0f / lrow[nt];
      const int64_t o = ((static_cast<int64_t>(b) * p.T + t) * p.Hq + h) * D;
#pragma unroll
      for (int md = 0; md < C::NMD; ++md) {
        const f32x4 v = oacc[md][nt] * inv;
        if constexpr (C::BF16) {
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
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
            (mrow[nt] + __builtin_log2f(lrow[nt])) * kLn2;
    } else {
      const int64_t prow = (static_cast<int64_t>(unit) * S + split) * p.R + row;
#pragma unroll
      for (int md = 0; md < C::NMD; ++md)
        *reinterpret_cast<f32x4*>(p.part_o + prow * D + md * 16 + 4 * g4) = oacc[md][nt];
      if (g4 == 0) {
        p.part_ml[prow * 2 + 0] = mrow[nt];
        p.part_ml[prow * 2 + 1] = lrow[nt];
      }
    }
  }
}

// Combine the S partials of every (unit, row): one thread per 4 head dims.
template <bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  const int unit = blockIdx.y;
  const int i4 = blockIdx.x * 256 + threadIdx.x;
  const int D = p.D;
  if (i4 * 4 >= p.R * D) return;
  const int row = (i4 * 4) / D;
  const int dim = i4 * 4 - row * D;
  const int S = p.S;
  const int64_t base = static_cast<int64_t>(unit) * S * p.R + row;
  float mmax = -__builtin_inff();
  for (int s = 0; s < S; ++s) mmax = fmaxf(mmax, p.part_ml[(base + static_cast<int64_t>(s) * p.R) * 2]);
  const float msafe = mmax == -__builtin_inff() ? 0.0f : mmax;
  float l = 0.0f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const int64_t pr = base + static_cast<int64_t>(s) * p.R;
    const float a = __builtin_amdgcn_exp2f(p.part_ml[pr * 2] - msafe);
    l += a * p.part_ml[pr * 2 + 1];
    o += a * *reinterpret_cast<const f32x4*>(p.part_o + pr * D + dim);
  }
  const int b = unit / p.Hkv;
  const int g = unit - b * p.Hkv;
  const int t = row / p.G;
  const int h = g * p.G + (row - t * p.G);
  const int64_t off = ((static_cast<int64_t>(b) * p.T + t) * p.Hq + h) * D + dim;
  const f32x4 v = o * (1.0f / l);
  if constexpr (BF16) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = static_cast<__bf16>(v[e]);
    *reinterpret_cast<bf16x4_t*>(static_cast<char*>(p.out) + off * 2) = w;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + off) = v;
  }
  if (p.lse && dim == 0)
    p.lse[(static_cast<int64_t>(b) * p.T + t) * p.Hq + h] = (mmax + __builtin_log2f(l)) * kLn2;
}

template <class C>
hipError_t launch_cfg(const AttnParams& p, hipStream_t stream) {
  dim3 grid(p.S, p.B * p.Hkv);
  hipLaunchKernelGGL(attn_kernel<C>, grid, dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16, int D, int TT>
hipError_t launch_rows(const AttnParams& p, hipStream_t stream) {
  switch (attn_padded_rows(p.R)) {
    case 16: return launch_cfg<Cfg<BF16, D, TT, 16>>(p, stream);
    case 32: return launch_cfg<Cfg<BF16, D, TT, 32>>(p, stream);
    case 64: return launch_cfg<Cfg<BF16, D, TT, 64>>(p, stream);
    default: return launch_cfg<Cfg<BF16, D, TT, 128>>(p, stream);
  }
}

template <bool BF16>
hipError_t launch_dtype(const AttnParams& p, hipStream_t stream) {
  const int tt = attn_tile_tokens(p.bs);
  if (p.D == 128) {
    return tt == 64 ? launch_rows<BF16, 128, 64>(p, stream) : launch_rows<BF16, 128, 32>(p, stream);
  }
  return tt == 64 ? launch_rows<BF16, 64, 64>(p, stream) : launch_rows<BF16, 64, 32>(p, stream);
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, bool bf16, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  hipError_t e = bf16 ? launch_dtype<true>(p, stream) : launch_dtype<false>(p, stream);
  if (e != hipSuccess || p.S == 1) return e;
  dim3 grid((p.R * p.D / 4 + 255) / 256, p.B * p.Hkv);
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
