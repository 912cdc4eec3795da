/* A standalone C user of libqsa: builds a small paged batch on the host, copies it to the
 * device with the HIP runtime, runs qsa_decode and then qsa_decode_multi (TD = 3 new tokens per
 * request, the last three positions of each context) on the null stream and writes inputs
 * and results as raw little-endian files into the directory given as argv[1]:
 *   meta.txt    B Hq Hkv P NP max_pages max_blocks k, then the B lengths
 *   q.bin (bf16 bits), q_idx.bin, idx_cache.bin, k_cache.bin, v_cache.bin (bf16 bits),
 *   page_table.bin, scores.bin, sel.bin, sel_count.bin, partial_out.bin, partial_lse.bin,
 *   out.bin, out_lse.bin; for the multi-token call m_q.bin, m_q_idx.bin, m_scores.bin,
 *   m_sel.bin, m_sel_count.bin, m_out.bin (rows b*TD + t)
 * Rows of a request's last page past its length hold NaN K/V and indexer keys of 127. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qsa.h"

#define B 3
#define HQ 16
#define HKV 2
#define P 3
#define D 128
#define PAGE 64
#define KMAX 512
#define TD 3

static const int lens[B] = {9000, 700, 2049};

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static uint16_t to_bf16(float f) { /* round to nearest even; finite inputs */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float uniform(void) { return (float)next_u32() / 4294967296.0f * 2.0f - 1.0f; }
static int8_t int8v(void) { return (int8_t)((int)(next_u32() % 255u) - 127); }

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static int dump(const char* dir, const char* name, const void* p, size_t n) {
  char path[1024];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, n, f) != n) return 1;
  fclose(f);
  return 0;
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  int npages[B], NP = 0, max_pages = 0;
  for (int b = 0; b < B; ++b) {
    npages[b] = (lens[b] + PAGE - 1) / PAGE;
    NP += npages[b];
    if (npages[b] > max_pages) max_pages = npages[b];
  }
  const int max_blocks = max_pages * PAGE / 4;
  /* page table: a fixed permutation of the physical pages, -1 in unused slots */
  int32_t* perm = malloc(sizeof(int32_t) * NP);
  for (int i = 0; i < NP; ++i) perm[i] = i;
  for (int i = NP - 1; i > 0; --i) {
    const int j = (int)(next_u32() % (uint32_t)(i + 1));
    const int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  int32_t* pt = malloc(sizeof(int32_t) * B * max_pages);
  for (int i = 0; i < B * max_pages; ++i) pt[i] = -1;
  for (int b = 0, off = 0; b < B; off += npages[b], ++b)
    for (int p = 0; p < npages[b]; ++p) pt[b * max_pages + p] = perm[off + p];

  const size_t nq = (size_t)B * HQ * D, nqi = (size_t)B * 256, nidx = (size_t)NP * PAGE * 256,
               nkv = (size_t)NP * PAGE * HKV * D;
  uint16_t* q = malloc(2 * nq);
  int8_t* qi = malloc(nqi);
  int8_t* idx = malloc(nidx);
  uint16_t* kc = malloc(2 * nkv);
  uint16_t* vc = malloc(2 * nkv);
  for (size_t i = 0; i < nq; ++i) q[i] = to_bf16(uniform());
  for (size_t i = 0; i < nqi; ++i) qi[i] = int8v();
  for (size_t i = 0; i < nidx; ++i) idx[i] = int8v();
  for (size_t i = 0; i < nkv; ++i) kc[i] = to_bf16(uniform());
  for (size_t i = 0; i < nkv; ++i) vc[i] = to_bf16(uniform());
  for (int b = 0; b < B; ++b) /* poison past the length */
    for (int t = lens[b]; t < npages[b] * PAGE; ++t) {
      const size_t row = (size_t)pt[b * max_pages + t / PAGE] * PAGE + t % PAGE;
      memset(idx + row * 256, 127, 256);
      for (int e = 0; e < HKV * D; ++e) kc[row * HKV * D + e] = vc[row * HKV * D + e] = 0x7FC0;
    }

  void *d_q, *d_qi, *d_idx, *d_k, *d_v, *d_pt, *d_len, *d_scores, *d_sel, *d_cnt, *d_po, *d_pl, *d_out, *d_lse,
      *d_ws = NULL;
  const size_t ws = qsa_decode_workspace_size(B, HQ, HKV, max_blocks, KMAX, P);
  HIP_OK(hipMalloc(&d_q, 2 * nq));
  HIP_OK(hipMalloc(&d_qi, nqi));
  HIP_OK(hipMalloc(&d_idx, nidx));
  HIP_OK(hipMalloc(&d_k, 2 * nkv));
  HIP_OK(hipMalloc(&d_v, 2 * nkv));
  HIP_OK(hipMalloc(&d_pt, 4 * (size_t)B * max_pages));
  HIP_OK(hipMalloc(&d_len, 4 * B));
  HIP_OK(hipMalloc(&d_scores, 4 * (size_t)B * max_blocks));
  HIP_OK(hipMalloc(&d_sel, 4 * (size_t)B * KMAX));
  HIP_OK(hipMalloc(&d_cnt, 4 * B));
  HIP_OK(hipMalloc(&d_po, 4 * (size_t)B * P * HQ * D));
  HIP_OK(hipMalloc(&d_pl, 4 * (size_t)B * P * HQ));
  HIP_OK(hipMalloc(&d_out, 4 * (size_t)B * HQ * D));
  HIP_OK(hipMalloc(&d_lse, 4 * (size_t)B * HQ));
  if (ws) HIP_OK(hipMalloc(&d_ws, ws));
  HIP_OK(hipMemcpy(d_q, q, 2 * nq, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_qi, qi, nqi, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_idx, idx, nidx, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_k, kc, 2 * nkv, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_v, vc, 2 * nkv, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_pt, pt, 4 * (size_t)B * max_pages, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_len, lens, 4 * B, hipMemcpyHostToDevice));

  const float scale = 1.0f / sqrtf((float)D);
  qsa_status_t st = qsa_decode(d_q, d_qi, d_idx, d_k, d_v, d_pt, d_len, B, HQ, HKV, D, 4, 64, PAGE, max_pages,
                               max_blocks, KMAX, P, scale, d_scores, d_sel, d_cnt, d_po, d_pl, d_out, d_lse, d_ws,
                               ws, NULL);
  if (st != QSA_OK) {
    fprintf(stderr, "qsa_decode: %s (hip %d)\n", qsa_status_string(st), qsa_last_hip_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());

  int32_t* scores = malloc(4 * (size_t)B * max_blocks);
  int32_t* sel = malloc(4 * (size_t)B * KMAX);
  int32_t cnt[B];
  float* po = malloc(4 * (size_t)B * P * HQ * D);
  float* pl = malloc(4 * (size_t)B * P * HQ);
  float* out = malloc(4 * (size_t)B * HQ * D);
  float* lse = malloc(4 * (size_t)B * HQ);
  HIP_OK(hipMemcpy(scores, d_scores, 4 * (size_t)B * max_blocks, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(sel, d_sel, 4 * (size_t)B * KMAX, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(cnt, d_cnt, 4 * B, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(po, d_po, 4 * (size_t)B * P * HQ * D, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(pl, d_pl, 4 * (size_t)B * P * HQ, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, d_out, 4 * (size_t)B * HQ * D, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, d_lse, 4 * (size_t)B * HQ, hipMemcpyDeviceToHost));

  const char* dir = argv[1];
  char meta[256];
  snprintf(meta, sizeof meta, "%d %d %d %d %d %d %d %d %d %d %d %d\n", B, HQ, HKV, P, NP, max_pages, max_blocks, KMAX,
           TD, lens[0], lens[1], lens[2]);
  if (dump(dir, "meta.txt", meta, strlen(meta)) || dump(dir, "q.bin", q, 2 * nq) || dump(dir, "q_idx.bin", qi, nqi) ||
      dump(dir, "idx_cache.bin", idx, nidx) || dump(dir, "k_cache.bin", kc, 2 * nkv) ||
      dump(dir, "v_cache.bin", vc, 2 * nkv) || dump(dir, "page_table.bin", pt, 4 * (size_t)B * max_pages) ||
      dump(dir, "scores.bin", scores, 4 * (size_t)B * max_blocks) || dump(dir, "sel.bin", sel, 4 * (size_t)B * KMAX) ||
      dump(dir, "sel_count.bin", cnt, 4 * B) || dump(dir, "partial_out.bin", po, 4 * (size_t)B * P * HQ * D) ||
      dump(dir, "partial_lse.bin", pl, 4 * (size_t)B * P * HQ) || dump(dir, "out.bin", out, 4 * (size_t)B * HQ * D) ||
      dump(dir, "out_lse.bin", lse, 4 * (size_t)B * HQ))
    return 3;
  /* multi-token decode: TD new tokens per request, its own queries, workspace and outputs */
  const size_t mq = (size_t)B * TD * HQ * D, mqi = (size_t)B * TD * 256, BT = (size_t)B * TD;
  uint16_t* q2 = malloc(2 * mq);
  int8_t* qi2 = malloc(mqi);
  for (size_t i = 0; i < mq; ++i) q2[i] = to_bf16(uniform());
  for (size_t i = 0; i < mqi; ++i) qi2[i] = int8v();
  void *d_q2, *d_qi2, *d_s2, *d_sel2, *d_cnt2, *d_po2, *d_pl2, *d_out2, *d_ws2 = NULL;
  const size_t ws2 = qsa_decode_multi_workspace_size(B, TD, HQ, HKV, max_blocks, KMAX, P);
  HIP_OK(hipMalloc(&d_q2, 2 * mq));
  HIP_OK(hipMalloc(&d_qi2, mqi));
  HIP_OK(hipMalloc(&d_s2, 4 * BT * max_blocks));
  HIP_OK(hipMalloc(&d_sel2, 4 * BT * KMAX));
  HIP_OK(hipMalloc(&d_cnt2, 4 * BT));
  HIP_OK(hipMalloc(&d_po2, 4 * BT * P * HQ * D));
  HIP_OK(hipMalloc(&d_pl2, 4 * BT * P * HQ));
  HIP_OK(hipMalloc(&d_out2, 4 * BT * HQ * D));
  if (ws2) HIP_OK(hipMalloc(&d_ws2, ws2));
  HIP_OK(hipMemcpy(d_q2, q2, 2 * mq, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_qi2, qi2, mqi, hipMemcpyHostToDevice));
  st = qsa_decode_multi(d_q2, d_qi2, d_idx, d_k, d_v, d_pt, d_len, B, TD, HQ, HKV, D, 4, 64, PAGE, max_pages,
                        max_blocks, KMAX, P, scale, d_s2, d_sel2, d_cnt2, d_po2, d_pl2, d_out2, NULL, d_ws2, ws2,
                        NULL);
  if (st != QSA_OK) {
    fprintf(stderr, "qsa_decode_multi: %s (hip %d)\n", qsa_status_string(st), qsa_last_hip_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  int32_t* s2 = malloc(4 * BT * max_blocks);
  int32_t* sel2 = malloc(4 * BT * KMAX);
  int32_t* cnt2 = malloc(4 * BT);
  float* out2 = malloc(4 * BT * HQ * D);
  HIP_OK(hipMemcpy(s2, d_s2, 4 * BT * max_blocks, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(sel2, d_sel2, 4 * BT * KMAX, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(cnt2, d_cnt2, 4 * BT, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out2, d_out2, 4 * BT * HQ * D, hipMemcpyDeviceToHost));
  if (dump(dir, "m_q.bin", q2, 2 * mq) || dump(dir, "m_q_idx.bin", qi2, mqi) ||
      dump(dir, "m_scores.bin", s2, 4 * BT * max_blocks) || dump(dir, "m_sel.bin", sel2, 4 * BT * KMAX) ||
      dump(dir, "m_sel_count.bin", cnt2, 4 * BT) || dump(dir, "m_out.bin", out2, 4 * BT * HQ * D))
    return 3;
  printf("ok %s\n", qsa_status_string(st));
  return 0;
}
