// Device (HIP, gfx950) side of the seeded synthetic-input generator.
//
// Fills device buffers with exactly the values synth_host.c writes on the host
// for the same (seed, tensor id, element index); the per-element arithmetic is
// in synth_core.h. Built with -ffp-contract=off so that every fp32 step is one
// IEEE-rounded operation, as on the host.
//
// These kernels make test and benchmark inputs only; they are no part of the
// MoE layer library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYN_FN __host__ __device__ static inline
#include "synth_core.h"

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) k_words(uint64_t seed, uint32_t tid, uint64_t start,
                                                    uint64_t n, uint32_t* out) {
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * kThreads)
    out[i] = syn_word(seed, tid, start + i);
}

__global__ void __launch_bounds__(kThreads) k_normal_bf16(uint64_t seed, uint32_t tid, uint64_t n,
                                                          float std, const float* q, uint16_t* out) {
  // one Philox call per 4 consecutive elements
  uint64_t nb = (n + 3) / 4;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < nb;
       b += (uint64_t)gridDim.x * kThreads) {
    syn_u32x4 r = syn_philox4x32_10((uint32_t)b, (uint32_t)(b >> 32), tid, 0u, (uint32_t)seed,
                                    (uint32_t)(seed >> 32));
    for (int w = 0; w < 4; ++w) {
      uint64_t i = b * 4 + (uint64_t)w;
      if (i < n) out[i] = syn_bf16_rne(syn_std_normal(r.v[w], q) * std);
    }
  }
}

__global__ void __launch_bounds__(kThreads) k_normal_f32(uint64_t seed, uint32_t tid, uint64_t n,
                                                         float std, const float* q, float* out) {
  uint64_t nb = (n + 3) / 4;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < nb;
       b += (uint64_t)gridDim.x * kThreads) {
    syn_u32x4 r = syn_philox4x32_10((uint32_t)b, (uint32_t)(b >> 32), tid, 0u, (uint32_t)seed,
                                    (uint32_t)(seed >> 32));
    for (int w = 0; w < 4; ++w) {
      uint64_t i = b * 4 + (uint64_t)w;
      if (i < n) out[i] = syn_std_normal(r.v[w], q) * std;
    }
  }
}

// One workgroup per 128 x 128 block; 64 elements per thread. kI8: symmetric INT8 codes with
// scale amax/127, else E4M3 codes with scale amax/448.
template <bool kI8>
__global__ void __launch_bounds__(kThreads) k_fp8_bank(uint64_t seed, uint32_t tid, int64_t e0,
                                                       int64_t rows, int64_t cols, float std,
                                                       const float* q, uint8_t* codes,
                                                       float* scales) {
  __shared__ float red[kThreads];
  int64_t nrb = rows / 128, ncb = cols / 128;
  int64_t blk = blockIdx.x;
  int64_t e = blk / (nrb * ncb);
  int64_t rem = blk % (nrb * ncb);
  int64_t rb = rem / ncb, cb = rem % ncb;
  int t = threadIdx.x;
  int r = t / 2;                 // row inside the block
  int c0 = (t % 2) * 64;         // first of 64 columns
  uint64_t base = (uint64_t)(((e0 + e) * rows + rb * 128 + r) * cols + cb * 128 + c0);
  float v[64];
  float amax = 0.0f;
  for (int c = 0; c < 64; ++c) {
    v[c] = syn_normal(seed, tid, base + (uint64_t)c, std, q);
    amax = fmaxf(amax, fabsf(v[c]));
  }
  red[t] = amax;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  amax = red[0];
  float sc = (amax == 0.0f) ? 1.0f : __fdiv_rn(amax, kI8 ? 127.0f : 448.0f);
  size_t o = (size_t)((e * rows + rb * 128 + r) * cols + cb * 128 + c0);
  for (int c = 0; c < 64; ++c) {
    const float x = __fdiv_rn(v[c], sc);
    codes[o + c] = kI8 ? (uint8_t)syn_int8_rne_sat(x) : syn_e4m3_rne_sat(x);
  }
  if (t == 0) scales[blk] = sc;
}

// One thread per (expert, row, 32-column block).
__global__ void __launch_bounds__(kThreads) k_mxfp4_bank(uint64_t seed, uint32_t tid, int64_t e0,
                                                         int64_t rows, int64_t cols, float std,
                                                         const float* q, uint8_t* packed,
                                                         uint8_t* scales, int64_t nblk) {
  int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= nblk) return;
  int64_t ncb = cols / 32;
  int64_t er = blk / ncb, cb = blk % ncb;
  int64_t e = er / rows, r = er % rows;
  uint64_t base = (uint64_t)(((e0 + e) * rows + r) * cols + cb * 32);
  float v[32];
  float amax = 0.0f;
  for (int c = 0; c < 32; ++c) {
    v[c] = syn_normal(seed, tid, base + (uint64_t)c, std, q);
    amax = fmaxf(amax, fabsf(v[c]));
  }
  uint8_t sc = syn_mx_scale_code(amax);
  size_t o = (size_t)((e * rows + r) * cols + cb * 32) / 2;
  for (int c = 0; c < 32; c += 2) {
    uint8_t lo = syn_e2m1_rne_sat(syn_scale_pow2(v[c], 254 - sc));
    uint8_t hi = syn_e2m1_rne_sat(syn_scale_pow2(v[c + 1], 254 - sc));
    packed[o + c / 2] = (uint8_t)(lo | (hi << 4));
  }
  scales[blk] = sc;
}

int grid_for(uint64_t work) {
  uint64_t g = (work + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

// All pointers are device pointers except `stream` (a hipStream_t). Return 0 on
// success, else the hipError_t of the launch.
int synth_dev_words(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, uint32_t* out,
                    void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_words, dim3(grid_for(n)), dim3(kThreads), 0, (hipStream_t)stream, seed,
                     tid, start, n, out);
  return (int)hipGetLastError();
}

int synth_dev_normal_bf16(uint64_t seed, uint32_t tid, uint64_t n, float std, const float* q,
                          uint16_t* out, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_normal_bf16, dim3(grid_for((n + 3) / 4)), dim3(kThreads), 0,
                     (hipStream_t)stream, seed, tid, n, std, q, out);
  return (int)hipGetLastError();
}

int synth_dev_normal_f32(uint64_t seed, uint32_t tid, uint64_t n, float std, const float* q,
                         float* out, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_normal_f32, dim3(grid_for((n + 3) / 4)), dim3(kThreads), 0,
                     (hipStream_t)stream, seed, tid, n, std, q, out);
  return (int)hipGetLastError();
}

int synth_dev_fp8_bank(uint64_t seed, uint32_t tid, int64_t e0, int64_t ne, int64_t rows,
                       int64_t cols, float std, const float* q, uint8_t* codes, float* scales,
                       void* stream) {
  if (rows % 128 || cols % 128) return -1;
  int64_t nblk = ne * (rows / 128) * (cols / 128);
  if (nblk == 0) return 0;
  if (nblk > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(k_fp8_bank<false>, dim3((unsigned)nblk), dim3(kThreads), 0, (hipStream_t)stream,
                     seed, tid, e0, rows, cols, std, q, codes, scales);
  return (int)hipGetLastError();
}

int synth_dev_int8_bank(uint64_t seed, uint32_t tid, int64_t e0, int64_t ne, int64_t rows,
                        int64_t cols, float std, const float* q, int8_t* codes, float* scales,
                        void* stream) {
  if (rows % 128 || cols % 128) return -1;
  int64_t nblk = ne * (rows / 128) * (cols / 128);
  if (nblk == 0) return 0;
  if (nblk > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(k_fp8_bank<true>, dim3((unsigned)nblk), dim3(kThreads), 0, (hipStream_t)stream,
                     seed, tid, e0, rows, cols, std, q, reinterpret_cast<uint8_t*>(codes), scales);
  return (int)hipGetLastError();
}

int synth_dev_mxfp4_bank(uint64_t seed, uint32_t tid, int64_t e0, int64_t ne, int64_t rows,
                         int64_t cols, float std, const float* q, uint8_t* packed, uint8_t* scales,
                         void* stream) {
  if (cols % 32) return -1;
  int64_t nblk = ne * rows * (cols / 32);
  if (nblk == 0) return 0;
  int64_t g = (nblk + kThreads - 1) / kThreads;
  if (g > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(k_mxfp4_bank, dim3((unsigned)g), dim3(kThreads), 0, (hipStream_t)stream, seed,
                     tid, e0, rows, cols, std, q, packed, scales, nblk);
  return (int)hipGetLastError();
}

}  // extern "C"
