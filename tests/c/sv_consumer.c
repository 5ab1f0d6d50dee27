/*
 * A C99 consumer of libsv.so: the C ABI used from plain C, with no Python and no C++.
 *
 *   sv_consumer host         argument checks, queries and error reporting (no GPU)
 *   sv_consumer gpu OUTDIR   one verification layer on a small paged problem:
 *                            append with representatives (sv_block_repr), selection
 *                            (sv_select_blocks), attention on the selection
 *                            (sv_sparse_verify_attn), the fused call
 *                            (sv_select_and_attend) and its allocation-free form
 *                            (sv_select_and_attend_static, whose results must equal the
 *                            fused call's bit for bit), reuse (sv_reuse_indices) and a
 *                            threshold-pruned FFN (sv_sparse_ffn). Inputs and outputs
 *                            are written to OUTDIR as raw little-endian arrays, with
 *                            their sizes in OUTDIR/meta.txt, for a check against the
 *                            oracle.
 *
 * Exit status 0 when every call returned as expected.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sv.h"

#define CHECK_SV(call)                                                                   \
  do {                                                                                   \
    sv_status st_ = (call);                                                              \
    if (st_ != SV_OK) {                                                                  \
      fprintf(stderr, "%s:%d: %s -> %s: %s\n", __FILE__, __LINE__, #call,                \
              sv_status_str(st_), sv_last_error());                                      \
      return 1;                                                                          \
    }                                                                                    \
  } while (0)

#define CHECK_HIP(call)                                                                  \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess) {                                                              \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call,                    \
              hipGetErrorString(e_));                                                    \
      return 1;                                                                          \
    }                                                                                    \
  } while (0)

#define EXPECT(cond)                                                                     \
  do {                                                                                   \
    if (!(cond)) {                                                                       \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond);                \
      return 1;                                                                          \
    }                                                                                    \
  } while (0)

static sv_shape make_shape(int32_t b, int32_t hq, int32_t hkv, int32_t d, int32_t bs, int32_t nb,
                           int32_t p, int32_t t) {
  sv_shape s;
  s.num_seqs = b;
  s.num_q_heads = hq;
  s.num_kv_heads = hkv;
  s.head_dim = d;
  s.block_size = bs;
  s.max_blocks_per_seq = nb;
  s.num_phys_blocks = p;
  s.num_draft = t;
  s.dtype = SV_BF16;
  return s;
}

/* ------------------------------------------------------------------ host checks */

static int host_checks(void) {
  const sv_budget budget = {4096, 64, 50, 1, 1};
  const sv_budget bad = {4096, 1, 50, 1, 1};  /* min_blocks < keep_first + keep_last */
  sv_shape s = make_shape(2, 32, 8, 128, 64, 1024, 2048, 8);
  sv_attn_plan plan;
  sv_ffn_shape fs = {8, 4096, 14336, SV_BF16};
  int32_t i;
  size_t n_sel, n_attn, n_fused;

  EXPECT(sv_abi_version() == SV_ABI_VERSION);
  for (i = 0; i <= SV_ERR_HIP; ++i) EXPECT(sv_status_str(i) != NULL);
  EXPECT(strcmp(sv_status_str(SV_ERR_NULL_ARG), sv_status_str(SV_ERR_BAD_SHAPE)) != 0);

  /* the budget formula: dense up to 4096 tokens, else max(64, 5% of the blocks) */
  EXPECT(sv_budget_blocks(&budget, 4096, 64) == 64);
  EXPECT(sv_budget_blocks(&budget, 32768, 64) == 64);
  EXPECT(sv_budget_blocks(&budget, 131072, 64) == 103);
  EXPECT(sv_budget_blocks(&bad, 32768, 64) == -1);
  EXPECT(sv_budget_blocks(NULL, 32768, 64) == -1);

  n_sel = sv_select_workspace_bytes(&s, 64);
  n_attn = sv_attn_workspace_bytes(&s, 64, 0);
  n_fused = sv_select_and_attend_workspace_bytes(&s, 64, 0);
  EXPECT(n_sel > 0 && n_fused >= n_attn);
  EXPECT(sv_attn_num_splits(&s, 64, 0) >= 1);
  CHECK_SV(sv_attn_plan_query(&s, 64, 0, &plan));
  EXPECT(plan.num_splits == sv_attn_num_splits(&s, 64, 0));
  EXPECT(plan.padded_rows >= 32 && plan.workgroups > 0);
  EXPECT(sv_sparse_ffn_workspace_bytes(&fs) > 0);

  /* rejections, before anything is launched */
  EXPECT(sv_sparse_verify_attn(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                               64, 0.1f, 0, NULL, NULL, NULL, 0, NULL) == SV_ERR_NULL_ARG);
  EXPECT(strlen(sv_last_error()) > 0);
  {
    sv_shape odd = s;
    odd.head_dim = 96;
    EXPECT(sv_attn_plan_query(&odd, 64, 0, &plan) == SV_ERR_UNSUPPORTED);
  }
  {
    /* distinct, 256-byte aligned stand-in addresses; q 8 bytes off its alignment */
    char* base = (char*)(uintptr_t)0x10000000;
    const int32_t* i32 = (const int32_t*)(base + 0x6000000);
    EXPECT(sv_sparse_verify_attn(&s, base + 0x1000008, base + 0x2000000, base + 0x3000000, NULL,
                                 base + 0x4000000, base + 0x5000000, i32, i32 + 0x400000,
                                 i32 + 0x800000, i32 + 0xC00000, 64, 0.1f, 0, base + 0xA000000,
                                 NULL, base + 0xB000000, (size_t)1 << 30,
                                 NULL) == SV_ERR_UNSUPPORTED);
    EXPECT(strstr(sv_last_error(), "q is not 16-byte aligned") != NULL);
  }
  fs.num_tokens = 17;
  EXPECT(sv_sparse_ffn_workspace_bytes(&fs) == 0);
  printf("host ok\n");
  return 0;
}

/* ------------------------------------------------------------------ GPU run */

/* xorshift64* stream */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  uint64_t x = rng_state;
  x ^= x >> 12;
  x ^= x << 25;
  x ^= x >> 27;
  rng_state = x;
  return x * 0x2545F4914F6CDD1Dull;
}

/* uniform draw in [-1, 1) */
static float uniform(void) {
  return (float)((double)(next_u64() >> 11) * (2.0 / 9007199254740992.0) - 1.0);
}

/* round to nearest even bf16 bits of a finite float */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static void fill_bf16(uint16_t* dst, size_t n, float scale) {
  size_t i;
  for (i = 0; i < n; ++i) dst[i] = to_bf16(scale * uniform());
}

static int save(const char* dir, const char* name, const void* host, size_t bytes) {
  char path[1024];
  FILE* f;
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    if (f) fclose(f);
    return 1;
  }
  fclose(f);
  return 0;
}

/* device copy of a host array (NULL for zero bytes) */
static int upload(void** dev, const void* host, size_t bytes) {
  *dev = NULL;
  if (bytes == 0) return 0;
  if (hipMalloc(dev, bytes) != hipSuccess) return 1;
  if (host && hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return 1;
  if (!host && hipMemset(*dev, 0, bytes) != hipSuccess) return 1;
  return 0;
}

static int download_save(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes);
  int rc;
  if (!host || hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    free(host);
    return 1;
  }
  rc = save(dir, name, host, bytes);
  free(host);
  return rc;
}

/* 1 when two device arrays hold the same bytes */
static int same_on_device(const void* a, const void* b, size_t bytes) {
  unsigned char* ha = malloc(bytes);
  unsigned char* hb = malloc(bytes);
  int same = ha && hb && hipMemcpy(ha, a, bytes, hipMemcpyDeviceToHost) == hipSuccess &&
             hipMemcpy(hb, b, bytes, hipMemcpyDeviceToHost) == hipSuccess &&
             memcmp(ha, hb, bytes) == 0;
  free(ha);
  free(hb);
  return same;
}

enum { B = 2, HQ = 8, HKV = 2, D = 128, BS = 64, T = 4, KMAX = 8 };
static const int32_t CTX[B] = {1000, 2500};

static int gpu_run(const char* dir) {
  const int32_t nb0 = (CTX[0] + BS - 1) / BS, nb1 = (CTX[1] + BS - 1) / BS;
  const int32_t NB = nb1 > nb0 ? nb1 : nb0;
  const int32_t P = nb0 + nb1 + 4; /* four physical blocks no sequence maps */
  const int32_t NMAX = CTX[1] > CTX[0] ? CTX[1] : CTX[0];
  const sv_budget budget = {0, KMAX, 0, 1, 1}; /* k = min(nb, 8), first and last kept */
  const float scale = 1.0f / sqrtf((float)D);
  const sv_shape s = make_shape(B, HQ, HKV, D, BS, NB, P, T);
  const size_t n_new_el = (size_t)B * NMAX * HKV * D, n_q = (size_t)B * T * HQ * D,
               n_draft = (size_t)B * T * HKV * D, n_pool = (size_t)P * HKV * BS * D,
               n_reps = (size_t)P * HKV * D, n_idx = (size_t)B * HKV * KMAX,
               n_cnt = (size_t)B * HKV, n_scores = (size_t)B * HKV * NB,
               n_lse = (size_t)B * T * HQ;
  const sv_ffn_shape fs = {4, 512, 600, SV_BF16};
  const float tau = 0.3f;
  const size_t n_x = (size_t)fs.num_tokens * fs.d_model, n_w = (size_t)fs.d_ffn * fs.d_model;
  uint16_t *k_new, *v_new, *q, *kd, *vd, *x, *wg, *wu, *wd;
  int32_t* table;
  int32_t perm[256], n_new[B], ctx_before[B] = {0, 0}, ctx_after[B];
  void *d_knew, *d_vnew, *d_q, *d_kd, *d_vd, *d_kpool, *d_vpool, *d_reps, *d_table, *d_ctx,
      *d_nnew, *d_cbefore, *d_cafter, *d_idx, *d_cnt, *d_scores, *d_out, *d_lse, *d_idx2,
      *d_cnt2, *d_out2, *d_lse2, *d_idx3, *d_cnt3, *d_wsel, *d_wattn, *d_wfused, *d_x, *d_wg,
      *d_wu, *d_wd, *d_y, *d_keep, *d_wffn, *d_idx4, *d_cnt4, *d_out4, *d_lse4;
  size_t n_wsel, n_wattn, n_wfused, n_wffn;
  int32_t i, j;
  FILE* meta;
  char path[1024];

  if (P > 256) return 1;
  /* inputs: keys and values of every context token, queries and drafts (bf16) */
  k_new = malloc(n_new_el * 2);
  v_new = malloc(n_new_el * 2);
  q = malloc(n_q * 2);
  kd = malloc(n_draft * 2);
  vd = malloc(n_draft * 2);
  table = malloc((size_t)B * NB * 4);
  x = malloc(n_x * 2);
  wg = malloc(n_w * 2);
  wu = malloc(n_w * 2);
  wd = malloc(n_w * 2);
  if (!k_new || !v_new || !q || !kd || !vd || !table || !x || !wg || !wu || !wd) return 1;
  fill_bf16(k_new, n_new_el, 1.7f);
  fill_bf16(v_new, n_new_el, 1.7f);
  fill_bf16(q, n_q, 1.7f);
  fill_bf16(kd, n_draft, 1.7f);
  fill_bf16(vd, n_draft, 1.7f);
  fill_bf16(x, n_x, 1.7f);
  fill_bf16(wg, n_w, 1.7f / sqrtf((float)fs.d_model));
  fill_bf16(wu, n_w, 1.7f / sqrtf((float)fs.d_model));
  fill_bf16(wd, n_w, 1.7f / sqrtf((float)fs.d_ffn));
  /* a paged table: a seeded permutation of the physical blocks */
  for (i = 0; i < P; ++i) perm[i] = i;
  for (i = P - 1; i > 0; --i) {
    j = (int32_t)(next_u64() % (uint64_t)(i + 1));
    { int32_t t_ = perm[i]; perm[i] = perm[j]; perm[j] = t_; }
  }
  for (i = 0; i < B * NB; ++i) table[i] = 0;
  for (j = 0; j < nb0; ++j) table[0 * NB + j] = perm[j];
  for (j = 0; j < nb1; ++j) table[1 * NB + j] = perm[nb0 + j];
  for (i = 0; i < B; ++i) {
    n_new[i] = CTX[i];
    ctx_after[i] = CTX[i];
  }

  n_wsel = sv_select_workspace_bytes(&s, KMAX);
  n_wattn = sv_attn_workspace_bytes(&s, KMAX, 0);
  n_wfused = sv_select_and_attend_workspace_bytes(&s, KMAX, 0);
  n_wffn = sv_sparse_ffn_workspace_bytes(&fs);
  EXPECT(n_wsel > 0 && n_wfused > 0 && n_wffn > 0);

  /* device buffers; outputs and workspaces zero-filled at allocation */
  if (upload(&d_knew, k_new, n_new_el * 2) || upload(&d_vnew, v_new, n_new_el * 2) ||
      upload(&d_q, q, n_q * 2) || upload(&d_kd, kd, n_draft * 2) ||
      upload(&d_vd, vd, n_draft * 2) || upload(&d_kpool, NULL, n_pool * 2) ||
      upload(&d_vpool, NULL, n_pool * 2) || upload(&d_reps, NULL, n_reps * 4) ||
      upload(&d_table, table, (size_t)B * NB * 4) || upload(&d_ctx, CTX, B * 4) ||
      upload(&d_nnew, n_new, B * 4) || upload(&d_cbefore, ctx_before, B * 4) ||
      upload(&d_cafter, ctx_after, B * 4) || upload(&d_idx, NULL, n_idx * 4) ||
      upload(&d_cnt, NULL, n_cnt * 4) || upload(&d_scores, NULL, n_scores * 4) ||
      upload(&d_out, NULL, n_q * 2) || upload(&d_lse, NULL, n_lse * 4) ||
      upload(&d_idx2, NULL, n_idx * 4) || upload(&d_cnt2, NULL, n_cnt * 4) ||
      upload(&d_out2, NULL, n_q * 2) || upload(&d_lse2, NULL, n_lse * 4) ||
      upload(&d_idx3, NULL, n_idx * 4) || upload(&d_cnt3, NULL, n_cnt * 4) ||
      upload(&d_wsel, NULL, n_wsel) || upload(&d_wattn, NULL, n_wattn) ||
      upload(&d_wfused, NULL, n_wfused) || upload(&d_x, x, n_x * 2) ||
      upload(&d_wg, wg, n_w * 2) || upload(&d_wu, wu, n_w * 2) || upload(&d_wd, wd, n_w * 2) ||
      upload(&d_y, NULL, n_x * 2) || upload(&d_keep, NULL, (size_t)fs.d_ffn * 4) ||
      upload(&d_wffn, NULL, n_wffn) || upload(&d_idx4, NULL, n_idx * 4) ||
      upload(&d_cnt4, NULL, n_cnt * 4) || upload(&d_out4, NULL, n_q * 2) ||
      upload(&d_lse4, NULL, n_lse * 4)) {
    fprintf(stderr, "device allocation or copy failed\n");
    return 1;
  }

  /* one layer, all on the default stream */
  CHECK_SV(sv_block_repr(&s, d_knew, d_vnew, NMAX, d_nnew, d_cbefore, d_cafter, d_table, d_kpool,
                         d_vpool, d_reps, NULL));
  CHECK_SV(sv_select_blocks(&s, &budget, d_q, d_reps, d_table, d_ctx, KMAX, d_idx, d_cnt,
                            d_scores, d_wsel, n_wsel, NULL));
  CHECK_SV(sv_sparse_verify_attn(&s, d_q, d_kd, d_vd, NULL, d_kpool, d_vpool, d_table, d_ctx,
                                 d_idx, d_cnt, KMAX, scale, 0, d_out, d_lse, d_wattn, n_wattn,
                                 NULL));
  CHECK_SV(sv_select_and_attend(&s, &budget, d_q, d_reps, d_kd, d_vd, NULL, d_kpool, d_vpool,
                                d_table, d_ctx, KMAX, scale, 0, d_idx2, d_cnt2, d_out2, d_lse2,
                                d_wfused, n_wfused, NULL));
  CHECK_SV(sv_select_and_attend_static(&s, &budget, d_q, d_reps, d_kd, d_vd, NULL, d_kpool,
                                       d_vpool, d_table, d_ctx, KMAX, scale, 0, d_idx4, d_cnt4,
                                       d_out4, d_lse4, NULL));
  CHECK_SV(sv_reuse_indices(&s, KMAX, d_idx, d_cnt, d_idx3, d_cnt3, NULL));
  CHECK_SV(sv_sparse_ffn(&fs, d_x, d_wg, d_wu, d_wd, tau, d_y, d_keep, d_wffn, n_wffn, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  EXPECT(same_on_device(d_idx4, d_idx2, n_idx * 4) && same_on_device(d_cnt4, d_cnt2, n_cnt * 4));
  EXPECT(same_on_device(d_out4, d_out2, n_q * 2) && same_on_device(d_lse4, d_lse2, n_lse * 4));

  snprintf(path, sizeof path, "%s/meta.txt", dir);
  meta = fopen(path, "w");
  if (!meta) return 1;
  fprintf(meta, "B %d\nHQ %d\nHKV %d\nD %d\nBS %d\nT %d\nNB %d\nP %d\nNMAX %d\nKMAX %d\n"
                "CTX0 %d\nCTX1 %d\nSCALE %.9g\nDENSE %d\nMIN %d\nFRAC %d\nKF %d\nKL %d\n"
                "FN %d\nFDM %d\nFF %d\nTAU %.9g\n",
          B, HQ, HKV, D, BS, T, NB, P, NMAX, KMAX, CTX[0], CTX[1], scale,
          budget.dense_ctx_tokens, budget.min_blocks, budget.frac_per_mille, budget.keep_first,
          budget.keep_last, fs.num_tokens, fs.d_model, fs.d_ffn, tau);
  fclose(meta);
  if (save(dir, "k_new.bin", k_new, n_new_el * 2) ||
      save(dir, "v_new.bin", v_new, n_new_el * 2) || save(dir, "q.bin", q, n_q * 2) ||
      save(dir, "k_draft.bin", kd, n_draft * 2) || save(dir, "v_draft.bin", vd, n_draft * 2) ||
      save(dir, "table.bin", table, (size_t)B * NB * 4) ||
      save(dir, "x.bin", x, n_x * 2) || save(dir, "w_gate.bin", wg, n_w * 2) ||
      save(dir, "w_up.bin", wu, n_w * 2) || save(dir, "w_down_t.bin", wd, n_w * 2) ||
      download_save(dir, "k_pool.bin", d_kpool, n_pool * 2) ||
      download_save(dir, "v_pool.bin", d_vpool, n_pool * 2) ||
      download_save(dir, "reps.bin", d_reps, n_reps * 4) ||
      download_save(dir, "idx.bin", d_idx, n_idx * 4) ||
      download_save(dir, "cnt.bin", d_cnt, n_cnt * 4) ||
      download_save(dir, "scores.bin", d_scores, n_scores * 4) ||
      download_save(dir, "out.bin", d_out, n_q * 2) ||
      download_save(dir, "lse.bin", d_lse, n_lse * 4) ||
      download_save(dir, "idx2.bin", d_idx2, n_idx * 4) ||
      download_save(dir, "cnt2.bin", d_cnt2, n_cnt * 4) ||
      download_save(dir, "out2.bin", d_out2, n_q * 2) ||
      download_save(dir, "lse2.bin", d_lse2, n_lse * 4) ||
      download_save(dir, "idx3.bin", d_idx3, n_idx * 4) ||
      download_save(dir, "cnt3.bin", d_cnt3, n_cnt * 4) ||
      download_save(dir, "y.bin", d_y, n_x * 2) ||
      download_save(dir, "keep.bin", d_keep, (size_t)fs.d_ffn * 4))
    return 1;
  printf("gpu ok: %d sequences, %d KV heads, %d of %d / %d blocks selected\n", B, HKV, KMAX,
         nb0, nb1);
  return 0; /* the process exit frees the device buffers */
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc >= 3 && strcmp(argv[1], "gpu") == 0) return gpu_run(argv[2]);
  fprintf(stderr, "usage: %s host | gpu OUTDIR\n", argv[0]);
  return 2;
}
