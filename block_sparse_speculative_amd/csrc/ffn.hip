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
//  - ffn_down_kernel: channel chunks of 256 x model-dim groups of 512. Each wave gathers
//    the kept channels of its quarter of the chunk (ballot compaction) and streams those
//    w_down_t rows, 8 dims per lane, h broadcast from LDS (fp32 FMAs: the rows are
//    contiguous along the model dimension, not along the summed channels); the four
//    waves' sums are added in LDS and written as the chunk's partial y.
//  - ffn_reduce_kernel: y = the chunk partials summed in chunk order (deterministic),
//    rounded to bf16.
#include "gfx950_mem.h"
#include "internal.h"

namespace sv {
namespace {

constexpr int kFfnThreads = 256;
constexpr int kFfnReduceThreads = 64;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- gate and up projections (MFMA) ----------------------------------------------------
//
// One workgroup = 16 channels (the MFMA's M) x all tokens (N, padded to 16) x the whole
// model dimension, split over kGuWaves waves (each wave a contiguous Dm / kGuWaves slice,
// in 32-dim MFMA blocks); the slices' partial sums are added in LDS in wave order.
// Operands of v_mfma_f32_16x16x32_bf16 for lane l (r = l % 16, q = l / 16):
//   A: weight row c0 + r, dims 32 kb + 8 q .. + 7 (one 16-byte load; 16 rows x 64 bytes
//      per instruction)
//   B: x of token r at the same dims (from LDS; zero for r >= NP)
//   D: channel c0 + 4 q + e (e = 0..3), token r.
// x is staged in LDS in fragment order: fragment (kb, q, t) at ((kb * 4 + q) * NP + t) * 16,
// so the B reads of a wave are consecutive 16-byte pieces (no bank conflicts).
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
  if (r < p.N) {
    float* hrow = p.h + static_cast<int64_t>(r) * p.F;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = c0 + 4 * q + e;
      if (c < p.F) hrow[c] = keep[e] ? a[e] * u[e] : 0.0f;
    }
  }
  if (lane < 16 && c0 + lane < p.F) {
    p.mask[c0 + lane] = row_bits;
    if (p.keep_out) p.keep_out[c0 + lane] = row_bits;
  }
}

constexpr int kFfnChunk = 256;          // channels per down-projection chunk
constexpr int kFfnDimGroup = 64 * 8;    // model dims per down-projection workgroup

template <int NP>
__global__ __launch_bounds__(kFfnThreads) void ffn_down_kernel(FfnParams p) {
  __shared__ float hs[NP][kFfnChunk];
  __shared__ int list[4][kFfnChunk / 4];
  __shared__ float red[3][NP][kFfnDimGroup];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int Dm = p.Dm;
  const int64_t cbase = static_cast<int64_t>(blockIdx.x) * kFfnChunk;
  const int d0 = blockIdx.y * kFfnDimGroup + lane * 8;
  // h of the chunk (zero past F and for tokens >= N), every load issued before the stores.
  {
    constexpr int L = NP * kFfnChunk / kFfnThreads;
    float v[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const int i = tid + k * kFfnThreads;
      const int t = i / kFfnChunk;
      const int64_t c = cbase + (i - t * kFfnChunk);
      v[k] = (t < p.N && c < p.F) ? p.h[static_cast<int64_t>(t) * p.F + c] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const int i = tid + k * kFfnThreads;
      hs[i / kFfnChunk][i % kFfnChunk] = v[k];
    }
  }
  // The kept channels of this wave's quarter of the chunk (ascending), by ballot.
  int nk = 0;
  {
    constexpr int Q = kFfnChunk / 4 / 64;
    bool kk[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int64_t c = cbase + wave * (kFfnChunk / 4) + q * 64 + lane;
      kk[q] = c < p.F && p.mask[c] != 0u;
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int j = wave * (kFfnChunk / 4) + q * 64 + lane;
      const uint64_t b = __builtin_amdgcn_ballot_w64(kk[q]);
      if (kk[q]) list[wave][nk + __builtin_popcountll(b & ((uint64_t{1} << lane) - 1))] = j;
      nk += __builtin_popcountll(b);
    }
  }
  __syncthreads();
  float acc[NP][8];
#pragma unroll
  for (int t = 0; t < NP; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.0f;
  const char* wd = static_cast<const char*>(p.w_down_t);
  constexpr int U = 16;   // rows in flight per lane
  for (int i0 = 0; i0 < nk; i0 += U) {
    uint4 wr[U];
    int jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      jj[u] = i0 + u < nk ? list[wave][i0 + u] : -1;
      wr[u] = jj[u] >= 0 ? *reinterpret_cast<const uint4*>(wd + ((cbase + jj[u]) * Dm + d0) * 2)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (jj[u] < 0) continue;
      const float w[8] = {bf16lo(wr[u].x), bf16hi(wr[u].x), bf16lo(wr[u].y), bf16hi(wr[u].y),
                          bf16lo(wr[u].z), bf16hi(wr[u].z), bf16lo(wr[u].w), bf16hi(wr[u].w)};
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        const float hv = hs[t][jj[u]];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = __builtin_fmaf(hv, w[e], acc[t][e]);
      }
    }
  }
  // Waves 1..3 hand their sums to wave 0, which writes the chunk's partial.
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < NP; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave - 1][t][lane * 8 + e] = acc[t][e];
  }
  __syncthreads();
  if (wave == 0) {
    float* part = p.part + (static_cast<int64_t>(blockIdx.x) * NP) * Dm;
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = ((acc[t][e] + red[0][t][lane * 8 + e]) + red[1][t][lane * 8 + e]) +
               red[2][t][lane * 8 + e];
      float4* dst = reinterpret_cast<float4*>(part + static_cast<int64_t>(t) * Dm + d0);
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

template <int NP>
__global__ __launch_bounds__(kFfnReduceThreads) void ffn_reduce_kernel(FfnParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kFfnReduceThreads + threadIdx.x;   // 4 dims
  const int64_t per_t = p.Dm / 4;
  if (i >= static_cast<int64_t>(p.N) * per_t) return;
  const int t = static_cast<int>(i / per_t);
  const int d = static_cast<int>(i - t * per_t) * 4;
  const int chunks = (p.F + kFfnChunk - 1) / kFfnChunk;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int B = 8;   // chunk loads in flight
  for (int k0 = 0; k0 < chunks; k0 += B) {
    float4 v[B];
#pragma unroll
    for (int k = 0; k < B; ++k)
      v[k] = k0 + k < chunks ? *reinterpret_cast<const float4*>(
                                   p.part + (static_cast<int64_t>(k0 + k) * NP + t) * p.Dm + d)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < B; ++k) {   // chunk order
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
  const int chunks = (p.F + kFfnChunk - 1) / kFfnChunk;
  hipLaunchKernelGGL(ffn_down_kernel<NP>, dim3(chunks, p.Dm / kFfnDimGroup), dim3(kFfnThreads), 0,
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
int ffn_chunks(int f) { return (f + kFfnChunk - 1) / kFfnChunk; }

hipError_t launch_ffn(const FfnParams& p, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  return ffn_padded_tokens(p.N) == 8 ? launch_np<8>(p, stream) : launch_np<16>(p, stream);
}

}  // namespace sv
