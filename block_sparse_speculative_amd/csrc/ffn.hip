// Threshold-pruned (sparse) gated FFN of the verification pass (tutorial page
// "Accelerate Speculative Decoding with Sparse Computation in Verification", section
// "Core technique 2"; sciencestack page of arXiv 2512.21911, Figure 1 caption: the
// pruned channels are set by the activation function's output and a threshold).
//
//   a[t, c] = SiLU(x[t] . w_gate[c]);  token t keeps channel c iff |a[t, c]| >= tau
//   h[t, c] = kept ? a[t, c] * (x[t] . w_up[c]) : 0
//   y[t]    = sum_c h[t, c] * w_down_t[c]
//
// The tokens are the draft tokens of one verification pass (at most 16), so every
// projection is a skinny, HBM-bound stream of weight rows. What the pruning saves is HBM
// traffic: the up- and down-projection rows of a channel are read only if some token
// keeps it.
//
// Kernels:
//  - ffn_gate_up_kernel: 16 channels per workgroup, the model dimension split over 8
//    waves. The gate and up products are MFMA contractions (16 channels x 16 padded
//    tokens x 32 dims per instruction) over weight rows loaded straight from HBM and x
//    staged in LDS; MFMA is used so that the per-byte issue cost stays small (4
//    accumulator registers, one instruction per 1 KB of weights), leaving the registers
//    to loads in flight. The gate totals give a and the keep bits; then only the kept
//    rows of w_up are read, giving h.
//  - ffn_down_kernel: one workgroup per (range of channels, 256 model dims). The kept
//    channels of the range are compacted (ballot) and streamed 32 at a time through an
//    LDS-DMA ring, W_down rows and their h together; the products are MFMAs whose W^T
//    operand comes from the gfx950 transposing LDS read and whose h^T operand is h split
//    into two bf16 parts. Each workgroup writes the partial y of its range.
//  - ffn_reduce_kernel: y = the range partials summed in range order (deterministic),
//    rounded to bf16.
#include "gfx950_mem.h"
#include "internal.h"

namespace sv {
namespace {

constexpr int kFfnReduceThreads = 64;

// ---- gate and up projections (MFMA) ----------------------------------------------------
//
// One workgroup = 16 channels (the MFMA's M) x all tokens (N, padded to 16) x the whole
// model dimension, split over kGuWaves waves (each wave a contiguous Dm / kGuWaves slice,
// in 32-dim MFMA blocks); the slices' partial sums are added in LDS in wave order.
// Operands of v_mfma_f32_16x16x32_bf16 for lane l (r = l % 16, q = l / 16):
//   A: weight row c0 + r, dims 32 kb + 8 q .. + 7 (one 16-byte load; 16 rows x 64 bytes
//      per instruction)
//   B: x of token r at the same dims (from LDS; zero for tokens r >= N)
//   D: channel c0 + 4 q + e (e = 0..3), token r.
// x is staged in LDS by LDS-DMA in fragment order: fragment (kb, q, t) at
// ((kb * 4 + q) * NP + t) * 16, so the B reads of a wave are consecutive 16-byte pieces
// (no bank conflicts).
constexpr int kGuWaves = 8;
constexpr int kGuThreads = kGuWaves * 64;
constexpr int kGuBatch = 16;   // 16-byte weight loads (MFMA blocks) in flight per lane

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Sum over the wave's nmf MFMA blocks starting at block kf0 of row `row` (not read unless
// row_ok) times x, for the lane's (channel, token) slots; B is zero for tokens >= N.
// X_PENDING: x is still arriving by LDS-DMA; the first batch of weight loads is issued
// before the wave waits for it (and for the rest of the workgroup) at a barrier.
template <int NP, bool X_PENDING>
__device__ __forceinline__ f32x4 gu_phase(const char* w, int64_t row, bool row_ok, int Dm,
                                          int kf0, int nmf, const char* xs, int q, int r,
                                          int N) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const char* wrow = w + row * Dm * 2 + q * 16;
  for (int b = 0; b < nmf; b += kGuBatch) {
    uint4 wr[kGuBatch];
#pragma unroll
    for (int j = 0; j < kGuBatch; ++j)
      wr[j] = (row_ok && b + j < nmf)
                  ? *reinterpret_cast<const uint4*>(wrow + static_cast<int64_t>(kf0 + b + j) * 64)
                  : make_uint4(0u, 0u, 0u, 0u);
    if (X_PENDING && b == 0) {
      gmem::wait_vmcnt<0>();   // this wave's x pieces (and its first weight batch) landed
      __syncthreads();         // every wave's pieces landed
    }
#pragma unroll
    for (int j = 0; j < kGuBatch; ++j) {
      if (b + j < nmf) {   // wave-uniform
        const uint4 xb = r < N ? *reinterpret_cast<const uint4*>(
                                     xs + (((kf0 + b + j) * 4 + q) * NP + r) * 16)
                               : make_uint4(0u, 0u, 0u, 0u);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wr[j]),
                                                      __builtin_bit_cast(bf16x8_t, xb), acc, 0,
                                                      0, 0);
      }
    }
  }
  return acc;
}

template <int NP>
__global__ __launch_bounds__(kGuThreads) void ffn_gate_up_kernel(FfnParams p) {
  extern __shared__ __attribute__((aligned(16))) char xs[];   // NP x Dm bf16, fragment order
  __shared__ f32x4 red[kGuWaves][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;
  const int r = lane & 15;
  const int Dm = p.Dm;
  // Stage x by LDS-DMA, one fragment per lane and instruction (the pieces of tokens >= N
  // repeat token 0 and are never read: their B operand is zero). Waited for inside the
  // gate phase, after its first weight batch is in flight.
  {
    const uint32_t xs_lds = gmem::lds_address(xs);
    const int frags = NP * Dm / 8;   // a multiple of kGuThreads (Dm is a multiple of 512)
    for (int base = wave * 64; base < frags; base += kGuThreads) {
      const int i = base + lane;
      const int t = i % NP;
      const int rest = i / NP;   // kb * 4 + q
      const int d = (rest >> 2) * 32 + (rest & 3) * 8;
      gmem::dma16(p.x, static_cast<uint32_t>(((t < p.N ? t : 0) * Dm + d) * 2),
                  xs_lds + static_cast<uint32_t>(base) * 16);
    }
  }

  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int nmf = Dm / kGuWaves / 32;   // MFMA blocks per wave (Dm is a multiple of 512)
  const int kf0 = wave * nmf;
  const int64_t row = c0 + r;
  // Gate: every wave forms the same total (partials added in wave order).
  red[wave][lane] = gu_phase<NP, true>(static_cast<const char*>(p.w_gate), row, row < p.F, Dm,
                                       kf0, nmf, xs, q, r, p.N);
  __syncthreads();
  f32x4 g = red[0][lane];
#pragma unroll
  for (int w = 1; w < kGuWaves; ++w) g += red[w][lane];
  __syncthreads();   // red is written again below
  // Lane slots: channel c0 + 4 q + e, token r.
  float a[4];
  bool keep[4];
  uint64_t kb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = g[e] / (1.0f + expf(-g[e]));
    keep[e] = r < p.N && c0 + 4 * q + e < p.F && fabsf(a[e]) >= p.tau;
    kb[e] = __builtin_amdgcn_ballot_w64(keep[e]);
  }
  // Tokens keeping channel c0 + 4 qq + e: bits 16 qq .. 16 qq + 15 of kb[e]. The up row a
  // lane loads is c0 + r, read only if some token keeps it.
  const uint64_t kbr = (r & 3) == 0 ? kb[0] : (r & 3) == 1 ? kb[1] : (r & 3) == 2 ? kb[2] : kb[3];
  const uint32_t row_bits = static_cast<uint32_t>((kbr >> (16 * (r >> 2))) & 0xffffu);
  red[wave][lane] = gu_phase<NP, false>(static_cast<const char*>(p.w_up), row, row_bits != 0u,
                                        Dm, kf0, nmf, xs, q, r, p.N);
  __syncthreads();
  if (wave != 0) return;   // no barrier follows
  f32x4 u = red[0][lane];
#pragma unroll
  for (int w = 1; w < kGuWaves; ++w) u += red[w][lane];
  // h channel-major, 16 token slots per channel (zero for tokens >= N, whose keep bits
  // are never set): the down projection streams a channel's 64 bytes with its row.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t c = c0 + 4 * q + e;
    if (c < p.F) p.h[c * 16 + r] = keep[e] ? a[e] * u[e] : 0.0f;
  }
  if (lane < 16 && c0 + lane < p.F) {
    p.mask[c0 + lane] = row_bits;
    if (p.keep_out) p.keep_out[c0 + lane] = row_bits;
  }
}

// ---- down projection (MFMA over W_down tiles read transposed from LDS) ---------------
//
// Workgroup (channel range rg, model-dim group dg): the kept channels of its range (a
// ballot compaction of the keep mask, ascending) are consumed 32 at a time, one MFMA K
// step each: y^T[256 dims x 16 tokens] += W^T[256 dims x 32 channels] . h^T[32 x 16].
// W_down_t rows are contiguous along the model dimension, so each tile (32 kept rows x
// 512 bytes of this dim group, plus the 32 channels' h, 64 bytes each) is staged by
// LDS-DMA into a 3-deep ring and the A operand is read with the gfx950 transposing LDS
// read (ds_read_b64_tr_b16: lane (g4, i) receives dim i of 4 consecutive rows; two reads
// give the 8 channels 8 g4 .. 8 g4 + 7 the MFMA wants per lane). Rows are XOR-swizzled
// in 32-byte pairs (the swizzle is applied on the global side of the DMA, which keeps
// every DMA instruction's LDS writes contiguous) so that the 16 rows a read touches fall
// on distinct banks. h is fp32; the B operand is its split h = hi + lo into two bf16
// parts (|h - hi - lo| <= 2^-16 |h|), one MFMA each. Each wave owns 64 of the 256 dims,
// so no cross-wave reduction is needed; the partial of the range is written per token.
// Pad rows of the last tile re-read the last kept row (already in cache) and take h = 0,
// so every tile is the same number of DMA instructions and the vmcnt waits are exact.
constexpr int kDnWaves = 4;
constexpr int kDnThreads = kDnWaves * 64;
constexpr int kDnDims = 256;                        // model dims per workgroup
constexpr int kDnRows = 32;                         // channels per tile (one MFMA K step)
constexpr int kDnRowBytes = kDnDims * 2;            // 512
constexpr int kDnWBytes = kDnRows * kDnRowBytes;    // 16 KB of W per tile
constexpr int kDnHBytes = kDnRows * 64;             // 2 KB of h per tile
constexpr int kDnTileBytes = kDnWBytes + kDnHBytes;
constexpr int kDnBuf = 3;                           // ring depth (two tiles in flight)
constexpr int kDnMaxRange = 512;                    // channels per range at most
constexpr int kDnWLoads = kDnWBytes / 1024 / kDnWaves;   // W DMA instructions per wave: 4
static_assert(kDnWLoads == 4 && kDnHBytes == 2048, "tile layout");

// XOR applied to the 16-byte chunk index of row r (0..31): a 3-bit function of the row
// on the pair index, distinct for the 8 rows each half-wave's transposing read touches.
__device__ __forceinline__ int dn_swz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4_t lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(
          (__attribute__((address_space(3))) char*)(const_cast<char*>(p))));
}

// bf16 (round to nearest even) bits of a finite float.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int NP>
__global__ __launch_bounds__(kDnThreads, 2) void ffn_down_kernel(FfnParams p) {
  __shared__ __attribute__((aligned(16))) char ring[kDnBuf * kDnTileBytes];
  __shared__ int list[kDnMaxRange];
  __shared__ int nk_s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int Dm = p.Dm;
  const int rg = blockIdx.x;
  const int dg = blockIdx.y;
  const int c0 = rg * p.dn_range;
  const int cn = p.F - c0 < p.dn_range ? p.F - c0 : p.dn_range;

  // Kept channels of the range, ascending (wave 0; every mask load issued first).
  if (wave == 0) {
    constexpr int kSub = kDnMaxRange / 64;
    bool kk[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const int c = s * 64 + lane;
      kk[s] = c < cn && p.mask[c0 + c] != 0u;
    }
    int nk = 0;
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const uint64_t b = __builtin_amdgcn_ballot_w64(kk[s]);
      if (kk[s]) list[nk + __builtin_popcountll(b & ((uint64_t{1} << lane) - 1))] = c0 + s * 64 + lane;
      nk += __builtin_popcountll(b);
    }
    if (lane == 0) nk_s = nk;
  }
  __syncthreads();
  const int nk = nk_s;
  const int steps = (nk + kDnRows - 1) / kDnRows;

  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (steps > 0) {   // workgroup-uniform
    const uint32_t ring_lds = gmem::lds_address(ring);
    // Tile s into buffer s % kDnBuf: wave w DMAs W rows 8w .. 8w + 7 (two rows of 512
    // bytes per instruction) and, waves 0 and 1, the h of channels 16w .. 16w + 15.
    auto issue = [&](int s) {
      const uint32_t tb = ring_lds + static_cast<uint32_t>((s % kDnBuf) * kDnTileBytes);
#pragma unroll
      for (int j = 0; j < kDnWLoads; ++j) {
        const int row = 8 * wave + 2 * j + (lane >> 5);
        const int k = s * kDnRows + row;
        const int ch = list[k < nk ? k : nk - 1];
        const int gch = (lane & 31) ^ dn_swz(row);
        gmem::dma16(p.w_down_t,
                    (static_cast<uint32_t>(ch) * static_cast<uint32_t>(Dm) + dg * kDnDims + gch * 8) *
                        2u,
                    tb + static_cast<uint32_t>((8 * wave + 2 * j) * kDnRowBytes));
      }
      if (wave < 2) {
        const int k = s * kDnRows + 16 * wave + (lane >> 2);
        const int ch = list[k < nk ? k : nk - 1];
        gmem::dma16(p.h, static_cast<uint32_t>(ch) * 64u + (lane & 3) * 16u,
                    tb + kDnWBytes + static_cast<uint32_t>(wave * 1024));
      }
    };
    static_assert(kDnBuf == 3, "the waits below assume at most one younger tile in flight");
    for (int s = 0; s < kDnBuf - 1 && s < steps; ++s) issue(s);
    const int md0 = wave * 4;   // this wave's first 16-dim M tile of the group
    for (int s = 0; s < steps; ++s) {
      // Tile s landed, with the younger tile already issued (if any) still in flight:
      // waves 0 and 1 issue kDnWLoads + 1 DMA instructions per tile, the others kDnWLoads.
      const int younger = steps - 1 - s < kDnBuf - 2 ? steps - 1 - s : kDnBuf - 2;
      if (younger == 1) {
        if (wave < 2) gmem::wait_vmcnt<kDnWLoads + 1>();
        else gmem::wait_vmcnt<kDnWLoads>();
      } else {
        gmem::wait_vmcnt<0>();
      }
      __syncthreads();   // also: every wave is done with tile s - 1's buffer
      if (s + kDnBuf - 1 < steps) issue(s + kDnBuf - 1);
      const char* tb = ring + (s % kDnBuf) * kDnTileBytes;
      // B operand: channels 8 g4 .. 8 g4 + 7 of the tile, token l16, as hi / lo bf16.
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint32_t ph = 0u, pl = 0u;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int kk = 8 * g4 + 2 * jj + e;
          const bool ok = s * kDnRows + kk < nk && l16 < NP;
          const float h = ok ? *reinterpret_cast<const float*>(tb + kDnWBytes + kk * 64 + l16 * 4)
                             : 0.0f;
          const uint32_t bh = bf16_bits(h);
          const uint32_t bl = bf16_bits(h - __uint_as_float(bh << 16));
          ph |= bh << (16 * e);
          pl |= bl << (16 * e);
        }
        hi[jj] = ph;
        lo[jj] = pl;
      }
      const bf16x8_t bhi = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
      const bf16x8_t blo = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int md = md0 + m;
        s16x4_t half[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = 8 * g4 + 4 * hh + (l16 >> 2);
          const int ch = 2 * md + ((l16 & 3) >> 1);
          half[hh] = lds_tr16(tb + row * kDnRowBytes + ((ch ^ dn_swz(row)) * 16) + 8 * (l16 & 1));
        }
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo, acc[m], 0, 0, 0);
      }
    }
  }
  // Partial of the range: lane (g4, l16) holds dims 16 md + 4 g4 .. + 3 of token l16.
  if (l16 < p.N) {
    float* dst = p.part + (static_cast<int64_t>(rg) * NP + l16) * Dm + dg * kDnDims;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<float4*>(dst + (wave * 4 + m) * 16 + 4 * g4) =
          make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
  }
}

template <int NP>
__global__ __launch_bounds__(kFfnReduceThreads) void ffn_reduce_kernel(FfnParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kFfnReduceThreads + threadIdx.x;   // 4 dims
  const int64_t per_t = p.Dm / 4;
  if (i >= static_cast<int64_t>(p.N) * per_t) return;
  const int t = static_cast<int>(i / per_t);
  const int d = static_cast<int>(i - t * per_t) * 4;
  const int ranges = p.dn_ranges;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int B = 8;   // range loads in flight
  for (int k0 = 0; k0 < ranges; k0 += B) {
    float4 v[B];
#pragma unroll
    for (int k = 0; k < B; ++k)
      v[k] = k0 + k < ranges ? *reinterpret_cast<const float4*>(
                                   p.part + (static_cast<int64_t>(k0 + k) * NP + t) * p.Dm + d)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < B; ++k) {   // range order
      s.x += v[k].x;
      s.y += v[k].y;
      s.z += v[k].z;
      s.w += v[k].w;
    }
  }
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 o;
  o[0] = static_cast<__bf16>(s.x);
  o[1] = static_cast<__bf16>(s.y);
  o[2] = static_cast<__bf16>(s.z);
  o[3] = static_cast<__bf16>(s.w);
  *reinterpret_cast<bf16x4*>(static_cast<char*>(p.y) + (static_cast<int64_t>(t) * p.Dm + d) * 2) = o;
}

template <int NP>
hipError_t launch_np(const FfnParams& p, hipStream_t stream) {
  const int gu_blocks = (p.F + 15) / 16;
  const size_t lds = static_cast<size_t>(NP) * p.Dm * 2;
  hipError_t e = hipSuccess;
  if (lds + sizeof(float) * 4 * 64 * kGuWaves > 64 * 1024) {   // beyond the default allowance
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_gate_up_kernel<NP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ffn_gate_up_kernel<NP>, dim3(gu_blocks), dim3(kGuThreads), lds, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ffn_down_kernel<NP>, dim3(p.dn_ranges, p.Dm / kDnDims), dim3(kDnThreads), 0,
                     stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n4 = static_cast<int64_t>(p.N) * p.Dm / 4;
  hipLaunchKernelGGL(ffn_reduce_kernel<NP>,
                     dim3(static_cast<uint32_t>((n4 + kFfnReduceThreads - 1) / kFfnReduceThreads)),
                     dim3(kFfnReduceThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int ffn_padded_tokens(int n) { return n <= 8 ? 8 : 16; }
// Channels per range of the down projection: about 2 workgroups per CU of a 256-CU GPU
// over the (range, 256-dim group) grid, a multiple of 64, between 64 and 512.
int ffn_range(int f, int dm) {
  const int64_t groups = dm / kDnDims;
  int64_t r = (static_cast<int64_t>(f) * groups + 511) / 512;
  r = (r + 63) / 64 * 64;
  return static_cast<int>(r < 64 ? 64 : r > kDnMaxRange ? kDnMaxRange : r);
}
int ffn_ranges(int f, int dm) {
  const int r = ffn_range(f, dm);
  return (f + r - 1) / r;
}

hipError_t launch_ffn(const FfnParams& p, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  return ffn_padded_tokens(p.N) == 8 ? launch_np<8>(p, stream) : launch_np<16>(p, stream);
}

}  // namespace sv
