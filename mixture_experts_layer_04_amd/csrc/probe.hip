// Measurement probes: the HBM read rate and the dense MFMA rate the device sustains, so
// that a benchmark can state each kernel's fraction of a measured peak beside the
// datasheet one. Not part of the layer; nothing here touches the layer's buffers.
//
// k_probe_read  streams a buffer once with non-temporal 16-B loads, each wavefront reading
//               its own contiguous chunk 1 KB per instruction, sixteen in flight per lane.
// k_probe_mfma  four wavefronts a SIMD on every CU, each issuing rounds of eight
//               independent MFMAs on register operands: the matrix cores' rate at the clock
//               the chip holds under that load, with no memory traffic.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kSinkMark = 0x9E3779B9u;  // the sink is written only for this value

// Each wavefront reads its own contiguous chunk of the buffer, 1 KB per instruction, 16
// instructions in flight (measured on MI355X: 7.0-7.1 TB/s at two 256-thread workgroups a
// CU, against 6.4-6.5 TB/s for a grid-stride order in which neighbouring wavefronts read
// neighbouring kilobytes); the words past the last whole chunk are read grid-stride.
constexpr int kReadU = 16;
__global__ void __launch_bounds__(256) k_probe_read(const u32x4v* __restrict__ buf, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int64_t per = n16 / waves / (64 * kReadU) * (64 * kReadU);  // words a wavefront
  const u32x4v* p = buf + w * per + l;
  uint32_t acc = 0;
  for (int64_t i = 0; i < per; i += 64 * kReadU) {
    u32x4v v[kReadU];
#pragma unroll
    for (int u = 0; u < kReadU; ++u) v[u] = __builtin_nontemporal_load(p + i + 64 * u);
#pragma unroll
    for (int u = 0; u < kReadU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (int64_t i = waves * per + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256) {
    const u32x4v v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == kSinkMark) sink[0] = acc;  // keeps every load; practically never stores
}

// kKind: 0 bf16 (v_mfma_f32_16x16x32_bf16), 1 fp8 E4M3 (v_mfma_scale_f32_16x16x128_f8f6f4
// with unit scales), 2 INT8 (v_mfma_i32_16x16x64_i8), 3 FP4 E2M1 (the scaled 16x16x128 form
// with both operands E2M1). Each chain has its own A operand, the accumulators stay in place
// in VGPRs (with the occupancy bound below; without it the compiler kept them in AGPRs and
// copied them around every round), and the loop is nothing but the eight MFMAs.
template <int kKind>
__global__ void __launch_bounds__(256, 4) k_probe_mfma(int iters, uint32_t* __restrict__ sink) {
  const uint32_t l = threadIdx.x;
  // operands from the lane index (small finite values in every format), so nothing folds
  const uint32_t wa = 0x3C003C00u + (l & 7), wb = 0x3C003C00u + ((l >> 3) & 7);
  uint32_t sum = 0;
  if constexpr (kKind == 0 || kKind == 2) {
    typedef typename std::conditional<kKind == 0, f32x4, i32x4>::type Acc;
    u32x4v a[8];
    Acc c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = kKind == 0 ? u32x4v{wa + j, wa + 1, wa + 2, wa + 3} : u32x4v{(l & 7) + j, 1, 2, 3};
      c[j] = Acc{0, 0, 0, 0};
    }
    const u32x4v b = kKind == 0 ? u32x4v{wb, wb + 1, wb + 2, wb + 3} : u32x4v{(l >> 3) & 7, 1, 2, 3};
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (kKind == 0)
          c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                         __builtin_bit_cast(bf16x8, b), c[j], 0, 0, 0);
        else
          c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a[j]),
                                                       __builtin_bit_cast(i32x4, b), c[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (kKind == 0) sum ^= __float_as_uint(c[j][0]) ^ __float_as_uint(c[j][3]);
      else sum ^= (uint32_t)c[j][0] ^ (uint32_t)c[j][3];
    }
  } else {
    // fp8: E4M3 codes near 1.0 in every byte; FP4: E2M1 codes 1.0 in the slot's first 16 B
    const int base = kKind == 1 ? 0x38383838 : 0x22222222;
    i32x8 a[8];
    f32x4 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = base + (int)(l & 7) + j;
      a[j] = kKind == 1 ? i32x8{v, v, v, v, v, v, v, v} : i32x8{v, v, v, v, 0, 0, 0, 0};
      c[j] = f32x4{0, 0, 0, 0};
    }
    const int w = base + (int)((l >> 3) & 7);
    const i32x8 b = kKind == 1 ? i32x8{w, w, w, w, w, w, w, w} : i32x8{w, w, w, w, 0, 0, 0, 0};
    constexpr int kFmt = kKind == 1 ? 0 : 4;
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j], b, c[j], kFmt, kFmt, 0, 127, 0, 127);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sum ^= __float_as_uint(c[j][0]) ^ __float_as_uint(c[j][3]);
  }
  if (sum == kSinkMark) sink[0] = sum;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int blocks = device_cus() * 2;  // two 256-thread workgroups a CU
  hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const u32x4v*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(moe_dtype dt, int64_t iters64, uint32_t* sink, double* flops,
                             hipStream_t s) {
  const int iters = (int)iters64;  // at most 2^30, checked by the caller
  const int blocks = device_cus() * 4;  // four 256-thread workgroups a CU: 4 wavefronts a SIMD
  const double waves = (double)blocks * 4;
  const double per_mfma = dt == MOE_BF16 ? 2.0 * 16 * 16 * 32
                          : dt == MOE_INT8 ? 2.0 * 16 * 16 * 64
                                           : 2.0 * 16 * 16 * 128;  // fp8, FP4
  *flops = waves * (double)iters * 8 * per_mfma;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(k_probe_mfma<0>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else if (dt == MOE_FP8_E4M3)
    hipLaunchKernelGGL(k_probe_mfma<1>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else if (dt == MOE_MXFP4_A4)
    hipLaunchKernelGGL(k_probe_mfma<3>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(k_probe_mfma<2>, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace moe
