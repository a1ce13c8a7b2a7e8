/* Host (CPU) side of the seeded synthetic-input generator.
 *
 * Fills buffers with the same values as the device kernels in synth_dev.hip;
 * the per-element arithmetic is in synth_core.h. Work is split over POSIX
 * threads by element range; each element depends only on (seed, tid, index),
 * so the result does not depend on the thread count.
 *
 * Built with gcc -O2 -ffp-contract=off (no FMA contraction, IEEE binary32).
 */
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define SYN_FN static inline
#include "synth_core.h"

typedef struct {
  int kind;
  uint64_t seed;
  uint32_t tid;
  uint64_t start, n;
  float a, b;
  const float* q;
  void* out;
  /* bank quantisers */
  int64_t e0, ne, rows, cols;
  void* out2;
  uint64_t lo, hi; /* work range for this thread */
} syn_job;

enum { K_WORDS = 0, K_NORMAL_F32, K_NORMAL_BF16, K_UNIFORM_F32, K_FP8_BANK, K_MXFP4_BANK,
       K_INT8_BANK };

/* A 128 x 128 block of an E4M3 (scale amax/448) or INT8 (scale amax/127) bank. */
static void run_fp8_block(const syn_job* j, uint64_t blk) {
  /* block index over (expert, row block, col block) of 128 x 128 */
  int64_t nrb = j->rows / 128, ncb = j->cols / 128;
  int64_t e = (int64_t)(blk / (uint64_t)(nrb * ncb));
  int64_t rem = (int64_t)(blk % (uint64_t)(nrb * ncb));
  int64_t rb = rem / ncb, cb = rem % ncb;
  int64_t ge = j->e0 + e;
  float vals[128 * 128];
  float amax = 0.0f;
  for (int r = 0; r < 128; ++r) {
    /* cols is a multiple of 128, so base is a multiple of 4: whole Philox blocks */
    uint64_t base = (uint64_t)((ge * j->rows + rb * 128 + r) * j->cols + cb * 128);
    for (int c = 0; c < 128; c += 4) {
      syn_normal4(j->seed, j->tid, (base + (uint64_t)c) >> 2, j->a, j->q, &vals[r * 128 + c]);
      for (int i = 0; i < 4; ++i) {
        float v = vals[r * 128 + c + i];
        float av = v < 0.0f ? -v : v;
        if (av > amax) amax = av;
      }
    }
  }
  const int i8 = j->kind == K_INT8_BANK;
  float s = (amax == 0.0f) ? 1.0f : amax / (i8 ? 127.0f : 448.0f);
  uint8_t* codes = (uint8_t*)j->out;
  for (int r = 0; r < 128; ++r) {
    size_t o = (size_t)((e * j->rows + rb * 128 + r) * j->cols + cb * 128);
    for (int c = 0; c < 128; ++c) {
      const float v = vals[r * 128 + c] / s;
      codes[o + c] = i8 ? (uint8_t)syn_int8_rne_sat(v) : syn_e4m3_rne_sat(v);
    }
  }
  ((float*)j->out2)[blk] = s;
}

static void run_mxfp4_block(const syn_job* j, uint64_t blk) {
  /* block index over (expert, row, 32-column block) */
  int64_t ncb = j->cols / 32;
  int64_t er = (int64_t)(blk / (uint64_t)ncb);     /* e * rows + row */
  int64_t cb = (int64_t)(blk % (uint64_t)ncb);
  int64_t e = er / j->rows, r = er % j->rows;
  uint64_t base = (uint64_t)(((j->e0 + e) * j->rows + r) * j->cols + cb * 32);
  float vals[32];
  float amax = 0.0f;
  /* cols is a multiple of 32, so base is a multiple of 4: whole Philox blocks */
  for (int c = 0; c < 32; c += 4) syn_normal4(j->seed, j->tid, (base + (uint64_t)c) >> 2, j->a, j->q, &vals[c]);
  for (int c = 0; c < 32; ++c) {
    float av = vals[c] < 0.0f ? -vals[c] : vals[c];
    if (av > amax) amax = av;
  }
  uint8_t sc = syn_mx_scale_code(amax);
  uint8_t* packed = (uint8_t*)j->out;
  size_t o = (size_t)((e * j->rows + r) * j->cols + cb * 32) / 2;
  for (int c = 0; c < 32; c += 2) {
    uint8_t lo = syn_e2m1_rne_sat(syn_scale_pow2(vals[c], 254 - sc));
    uint8_t hi = syn_e2m1_rne_sat(syn_scale_pow2(vals[c + 1], 254 - sc));
    packed[o + (size_t)(c / 2)] = (uint8_t)(lo | (hi << 4));
  }
  ((uint8_t*)j->out2)[blk] = sc;
}

/* Normal fills: elements start+i for i in [lo, hi), whole Philox blocks where the element
 * index is a multiple of 4 and single elements at the ragged ends. */
static void run_normal(const syn_job* j, int bf16) {
  uint64_t i = j->lo;
  float v4[4];
  for (; i < j->hi && ((j->start + i) & 3u); ++i) {
    float v = syn_normal(j->seed, j->tid, j->start + i, j->a, j->q);
    if (bf16) ((uint16_t*)j->out)[i] = syn_bf16_rne(v); else ((float*)j->out)[i] = v;
  }
  for (; i + 4 <= j->hi; i += 4) {
    syn_normal4(j->seed, j->tid, (j->start + i) >> 2, j->a, j->q, v4);
    for (int t = 0; t < 4; ++t) {
      if (bf16) ((uint16_t*)j->out)[i + t] = syn_bf16_rne(v4[t]); else ((float*)j->out)[i + t] = v4[t];
    }
  }
  for (; i < j->hi; ++i) {
    float v = syn_normal(j->seed, j->tid, j->start + i, j->a, j->q);
    if (bf16) ((uint16_t*)j->out)[i] = syn_bf16_rne(v); else ((float*)j->out)[i] = v;
  }
}

static void* worker(void* arg) {
  const syn_job* j = (const syn_job*)arg;
  if (j->kind == K_NORMAL_F32 || j->kind == K_NORMAL_BF16) {
    run_normal(j, j->kind == K_NORMAL_BF16);
    return NULL;
  }
  for (uint64_t i = j->lo; i < j->hi; ++i) {
    switch (j->kind) {
      case K_WORDS:
        ((uint32_t*)j->out)[i] = syn_word(j->seed, j->tid, j->start + i);
        break;
      case K_NORMAL_F32:
        ((float*)j->out)[i] = syn_normal(j->seed, j->tid, j->start + i, j->a, j->q);
        break;
      case K_NORMAL_BF16:
        ((uint16_t*)j->out)[i] = syn_bf16_rne(syn_normal(j->seed, j->tid, j->start + i, j->a, j->q));
        break;
      case K_UNIFORM_F32:
        ((float*)j->out)[i] = syn_uniform(j->seed, j->tid, j->start + i, j->a, j->b);
        break;
      case K_FP8_BANK:
      case K_INT8_BANK:
        run_fp8_block(j, i);
        break;
      case K_MXFP4_BANK:
        run_mxfp4_block(j, i);
        break;
    }
  }
  return NULL;
}

#define SYN_MAX_THREADS 64

static void run(syn_job proto, uint64_t count, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > SYN_MAX_THREADS) nthreads = SYN_MAX_THREADS;
  if ((uint64_t)nthreads > count) nthreads = count ? (int)count : 1;
  pthread_t th[SYN_MAX_THREADS];
  syn_job jobs[SYN_MAX_THREADS];
  uint64_t per = (count + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].lo = (uint64_t)t * per;
    jobs[t].hi = jobs[t].lo + per > count ? count : jobs[t].lo + per;
    if (jobs[t].lo >= jobs[t].hi) break;
    if (t == nthreads - 1 || pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) {
      worker(&jobs[t]);           /* last range (or a failed spawn) runs inline */
      th[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
}

void synth_host_words(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, uint32_t* out,
                      int nthreads) {
  syn_job j; memset(&j, 0, sizeof j);
  j.kind = K_WORDS; j.seed = seed; j.tid = tid; j.start = start; j.out = out;
  run(j, n, nthreads);
}

void synth_host_normal_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float std,
                           const float* q, float* out, int nthreads) {
  syn_job j; memset(&j, 0, sizeof j);
  j.kind = K_NORMAL_F32; j.seed = seed; j.tid = tid; j.start = start; j.a = std; j.q = q; j.out = out;
  run(j, n, nthreads);
}

void synth_host_normal_bf16(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float std,
                            const float* q, uint16_t* out, int nthreads) {
  syn_job j; memset(&j, 0, sizeof j);
  j.kind = K_NORMAL_BF16; j.seed = seed; j.tid = tid; j.start = start; j.a = std; j.q = q; j.out = out;
  run(j, n, nthreads);
}

void synth_host_uniform_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float lo,
                            float span, float* out, int nthreads) {
  syn_job j; memset(&j, 0, sizeof j);
  j.kind = K_UNIFORM_F32; j.seed = seed; j.tid = tid; j.start = start; j.a = lo; j.b = span; j.out = out;
  run(j, n, nthreads);
}

/* Experts [e0, e0+ne) of a bank of [rows, cols] matrices, N(0, std^2) values
 * quantised per 128x128 block: codes [ne, rows, cols] E4M3FN, scales
 * [ne, rows/128, cols/128] fp32 with scale = amax/448 (1 for an all-zero block). */
void synth_host_fp8_bank(uint64_t seed, uint32_t tid, int64_t e0, int64_t ne, int64_t rows,
                         int64_t cols, float std, const float* q, uint8_t* codes, float* scales,
                         int nthreads) {
  syn_job j; memset(&j, 0, sizeof j);
  j.kind = K_FP8_BANK; j.seed = seed; j.tid = tid; j.a = std; j.q = q; j.out = codes; j.out2 = scales;
  j.e0 = e0; j.ne = ne; j.rows = rows; j.cols = cols;
  run(j, (uint64_t)(ne * (rows / 128) * (cols / 128)), nthreads);
}

/* The same as symmetric INT8 codes (two's complement bytes) with fp32 scales amax/127. */
void synth_host_int8_bank(uint64_t seed, uint32_t tid, int64_t e0, int64_t ne, int64_t rows,
                          int64_t cols, float std, const float* q, int8_t* codes, float* scales,
                          int nthreads) {
  syn_job j; memset(&j, 0, sizeof j);
  j.kind = K_INT8_BANK; j.seed = seed; j.tid = tid; j.a = std; j.q = q; j.out = codes; j.out2 = scales;
  j.e0 = e0; j.ne = ne; j.rows = rows; j.cols = cols;
  run(j, (uint64_t)(ne * (rows / 128) * (cols / 128)), nthreads);
}

/* Experts [e0, e0+ne) of a bank of [rows, cols] matrices, N(0, std^2) values in
 * OCP MXFP4: packed [ne, rows, cols/2] (element 2i in the low nibble of byte i),
 * e8m0 scale codes [ne, rows, cols/32]. */
void synth_host_mxfp4_bank(uint64_t seed, uint32_t tid, int64_t e0, int64_t ne, int64_t rows,
                           int64_t cols, float std, const float* q, uint8_t* packed, uint8_t* scales,
                           int nthreads) {
  syn_job j; memset(&j, 0, sizeof j);
  j.kind = K_MXFP4_BANK; j.seed = seed; j.tid = tid; j.a = std; j.q = q; j.out = packed; j.out2 = scales;
  j.e0 = e0; j.ne = ne; j.rows = rows; j.cols = cols;
  run(j, (uint64_t)(ne * rows * (cols / 32)), nthreads);
}

/* One raw Philox4x32-10 block, for known-answer tests of the generator. */
void synth_host_philox_block(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  syn_u32x4 r = syn_philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int i = 0; i < 4; ++i) out[i] = r.v[i];
}
