// Budget and exact top-k pieces shared by the selection kernel and the fused
// select-and-attend kernel (tutorial page "Accelerate Speculative Decoding with
// Sparse Computation in Verification", section "Core technique 1": piecewise
// budget, top-k blocks by representative score).
//
// The top-k here runs in one workgroup of NW wavefronts over at most 1024 scores,
// held in registers: wave w, lane l, slot i holds block j = (w*PER + i)*64 + l
// (PER = 1024 / (64*NW)), so ascending block order is (w, i, l) order. Spreading
// the keys over every wave keeps each wave's instruction chain short, which is
// what bounds a selection this small.
//  1. keys: order-preserving 32-bit images of the scores; forced and absent blocks
//     get key 0 (never a candidate).
//  2. threshold: the want-th largest key, by radix select over the key bits from
//     the top (digits of 11, 11 and 10 bits): each pass builds an LDS histogram of
//     the digit over the keys still in play (one atomic add per key), scans it from
//     the top with DPP prefix sums and one cross-wave exchange, and keeps the bin
//     holding the want-th key. As soon as that bin holds at most 64 keys they are
//     gathered, in index order, into one register per lane of wave 0, whose
//     remaining low bits are searched bit by bit (compare + ballot + popcount),
//     stopping early once exactly the needed number of keys clear the candidate.
//  3. compaction in ascending block order: per-wave counts of keys above the
//     threshold and equal to it are exchanged once; keys equal to the threshold are
//     taken in index order (lowest index wins a tie); ballot + mbcnt give each
//     taken block its output position.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWaveTopkMax = 1024;          // scores one workgroup can select from
constexpr int kTopkBins = 2048;             // largest radix digit: 11 bits
// LDS scratch of wg_topk_select: histogram, gathered keys, exchange slots.
constexpr int kTopkLdsBytes = kTopkBins * 4 + 64 * 4 + 64 * 4;

// Order-preserving map of a float score to an unsigned key: a larger score gives a
// larger key. -0 and +0 share a key; NaN takes the key of -inf (lowest rank, tied
// with -inf). Key 0 is never produced (reserved for "not a candidate").
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) s = -__builtin_inff();
  if (s == 0.0f) s = 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Piecewise budget for a sequence of ctx tokens in nb blocks (formula of
// sv_budget in sv.h).
__device__ __forceinline__ int budget_blocks_dev(int ctx, int nb, int dense_ctx, int min_blocks,
                                                 int frac_per_mille) {
  if (ctx <= dense_ctx) return nb;
  int k = (frac_per_mille * nb + 999) / 1000;
  if (k < min_blocks) k = min_blocks;
  return k < nb ? k : nb;
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Inclusive prefix sum over the 64 lanes in lane order (DPP row shifts within rows
// of 16, then the row totals carried across rows).
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  const int row = (threadIdx.x & 63) >> 4;
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Largest t with #{lanes: v >= t} >= want over one register (v = 0 never counts;
// 1 <= want <= #{v != 0}; every v < 2^(top_bit+1)). *exact: exactly `want` lanes
// hold v >= t (then t need not be one of the values).
__device__ __forceinline__ uint32_t wave_kth_one(uint32_t v, int want, int top_bit, bool* exact) {
  uint32_t tau = 0u;
  *exact = false;
#pragma unroll 1
  for (int bit = top_bit; bit >= 0; --bit) {
    const uint32_t c = __builtin_amdgcn_readfirstlane(tau | (1u << bit));
    const int n = __builtin_popcountll(__builtin_amdgcn_ballot_w64(v >= c));
    if (n >= want) {
      tau = c;
      if (n == want) {
        *exact = true;
        break;
      }
    }
  }
  return tau;
}

// Workgroup barrier ordering LDS accesses (global loads and stores may stay in
// flight).
__device__ __forceinline__ void topk_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Loads this thread's scores of a row: slot i <- row[(w*PER + i)*64 + lane] for
// blocks below n_load (else 0).
template <int NW>
__device__ __forceinline__ void wg_topk_load(const float* row, int n_load,
                                             float (&s)[kWaveTopkMax / (64 * NW)]) {
  constexpr int PER = kWaveTopkMax / (64 * NW);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (w * PER + i) * 64 + lane;
    s[i] = j < n_load ? row[j] : 0.0f;
  }
}

// Selects, from blocks 0..nb-1 (nb <= 1024) with scores s (wg_topk_load layout),
// the budget k (already clamped by the caller): every block if k >= nb, else the
// forced blocks plus the best k - |forced| others. Calls emit(j, pos) once per
// selected block, on the thread holding it, with pos its position in ascending
// block order; returns the number selected. Called by all NW*64 threads of the
// workgroup (it contains barriers); `lds` is kTopkLdsBytes of 16-byte aligned LDS
// that nothing else uses meanwhile.
template <int NW, class Emit>
__device__ __forceinline__ int wg_topk_select(const float (&s)[kWaveTopkMax / (64 * NW)], int nb,
                                              int k, int keep_first, int keep_last, char* lds,
                                              Emit emit) {
  static_assert(NW >= 1 && NW <= 8 && kWaveTopkMax % (64 * NW) == 0, "wave count");
  constexpr int PER = kWaveTopkMax / (64 * NW);
  constexpr int NT = NW * 64;
  // exchange slots (ints): scan totals, bin broadcast, gather counts, threshold
  // broadcast, compaction counts
  constexpr int XS = 0, XB = 8, XG = 12, XL = 20, XC = 24;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto block_of = [&](int i) { return (w * PER + i) * 64 + lane; };
  if (k >= nb) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = block_of(i);
      if (j < nb) emit(j, j);
    }
    return nb;
  }
  const int f0 = keep_first ? 0 : -1;
  const int f1 = keep_last ? nb - 1 : -1;
  const int nforced = (f0 >= 0) + (f1 >= 0 && f1 != f0);
  int want = k - nforced;
  if (want < 0) want = 0;

  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = block_of(i);
    key[i] = (j < nb && j != f0 && j != f1) ? score_key(s[i]) : 0u;
  }

  int* hist = reinterpret_cast<int*>(lds);
  uint32_t* cand = reinterpret_cast<uint32_t*>(lds + kTopkBins * 4);
  int* xch = reinterpret_cast<int*>(lds + kTopkBins * 4 + 64 * 4);

  // Threshold `lo` and the number of keys equal to it that are taken (lowest
  // indices first): the taken set is {key > lo} plus the first eq_take keys == lo.
  uint32_t lo = 0xFFFFFFFFu;   // want == 0: nothing clears it
  int eq_take = 0;
  if (want > 0) {
    uint32_t prefix = 0u;      // high key bits fixed so far
    int shift = 32;            // number of key bits below them
    int rem = want;            // keys still to take among those matching prefix
    bool gathered = false;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int width = pass < 2 ? 11 : 10;
      const int nbins = 1 << width;
      const uint32_t hi_mask = shift >= 32 ? 0u : ~0u << shift;
      shift -= width;
      for (int x = tid; x < nbins / 4; x += NT)
        reinterpret_cast<int4*>(hist)[x] = make_int4(0, 0, 0, 0);
      topk_barrier();
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (key[i] != 0u && (key[i] & hi_mask) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & (nbins - 1)], 1);
      topk_barrier();
      // thread t sums bins [nbins - bpt(t+1), nbins - bpt t): thread 0 the top ones
      const int bpt = nbins / NT;
      const int b_lo = nbins - bpt * (tid + 1);
      int lsum = 0;
      for (int x = 0; x < bpt; ++x) lsum += hist[b_lo + x];
      const int incl_w = wave_incl_sum(lsum);
      if (lane == 63) xch[XS + w] = incl_w;
      topk_barrier();
      int before = 0;
      for (int v = 0; v < w; ++v) before += xch[XS + v];
      const int incl = before + incl_w;
      if (incl >= rem && incl - lsum < rem) {
        // this thread's bins hold the rem-th key: walk them from the top
        int acc = incl - lsum;
        for (int x = bpt - 1; x >= 0; --x) {
          const int h = hist[b_lo + x];
          if (acc + h >= rem) {
            xch[XB] = b_lo + x;
            xch[XB + 1] = acc;
            xch[XB + 2] = h;
            break;
          }
          acc += h;
        }
      }
      topk_barrier();
      const uint32_t bin = static_cast<uint32_t>(xch[XB]);
      const int above = xch[XB + 1];
      const int n_bin = xch[XB + 2];
      prefix |= bin << shift;
      rem -= above;
      if (shift == 0) break;   // every bit fixed: prefix is the threshold key
      if (n_bin <= 64) {
        gathered = true;
        // the bin's keys, in ascending block order, into cand[0 .. n_bin)
        const uint32_t m2 = ~0u << shift;
        int cnt_w = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i)
          cnt_w += __builtin_popcountll(
              __builtin_amdgcn_ballot_w64(key[i] != 0u && (key[i] & m2) == prefix));
        if (lane == 0) xch[XG + w] = cnt_w;
        topk_barrier();
        int base = 0;
        for (int v = 0; v < w; ++v) base += xch[XG + v];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const bool in = key[i] != 0u && (key[i] & m2) == prefix;
          const uint64_t mk = __builtin_amdgcn_ballot_w64(in);
          if (in) cand[base + lanes_below(mk)] = key[i];
          base += __builtin_popcountll(mk);
        }
        topk_barrier();
        if (w == 0) {
          const uint32_t low = (1u << shift) - 1u;
          const uint32_t v = lane < n_bin ? (cand[lane] & low) + 1u : 0u;   // +1: never 0
          bool exact;
          const uint32_t t = wave_kth_one(v, rem, shift, &exact);
          const uint32_t kth = prefix | (t - 1u);
          if (lane == 0) {
            // exact: the keys >= kth are exactly the wanted ones, none taken by tie
            xch[XL] = static_cast<int>(exact ? kth - 1u : kth);
            xch[XL + 1] = exact ? 0 : rem - __builtin_popcountll(__builtin_amdgcn_ballot_w64(v > t));
          }
        }
        topk_barrier();
        lo = static_cast<uint32_t>(xch[XL]);
        eq_take = xch[XL + 1];
        break;
      }
    }
    if (!gathered) {
      lo = prefix;             // the want-th largest key
      eq_take = rem;           // how many keys equal to it are taken
    }
  }

  // Compaction: per-wave counts of keys taken outright (forced, or above lo) and of
  // keys equal to lo, exchanged once; equal keys are taken in index order.
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = block_of(i);
    const bool gt = j == f0 || j == f1 || (key[i] != 0u && key[i] > lo);
    const bool eq = key[i] != 0u && key[i] == lo;
    n_gt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(gt));
    n_eq += __builtin_popcountll(__builtin_amdgcn_ballot_w64(eq));
  }
  if (lane == 0) {
    xch[XC + 2 * w] = n_gt;
    xch[XC + 2 * w + 1] = n_eq;
  }
  topk_barrier();
  int pos = 0, eq_before = 0, total = 0, eq_cum = 0;
  for (int v = 0; v < NW; ++v) {
    const int g_v = xch[XC + 2 * v];
    const int e_v = xch[XC + 2 * v + 1];
    int take_e = eq_take - eq_cum;          // equal keys taken from wave v
    take_e = take_e < 0 ? 0 : (take_e > e_v ? e_v : take_e);
    if (v < w) {
      pos += g_v + take_e;
      eq_before += e_v;
    }
    total += g_v + take_e;
    eq_cum += e_v;
  }
  int eq_seen = eq_before;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = block_of(i);
    const bool eq = key[i] != 0u && key[i] == lo;
    const uint64_t eqm = __builtin_amdgcn_ballot_w64(eq);
    const int eq_rank = eq_seen + lanes_below(eqm);
    const bool take = j == f0 || j == f1 || (key[i] != 0u && key[i] > lo) ||
                      (eq && eq_rank < eq_take);
    const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
    if (take) emit(j, pos + lanes_below(tm));
    pos += __builtin_popcountll(tm);
    eq_seen += __builtin_popcountll(eqm);
  }
  return total;
}

}  // namespace sv
