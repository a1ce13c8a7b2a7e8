// Selection-bias update of auxiliary-loss-free balancing ("Chapter 7: Serving Mega-MoE at
// Scale", roadmap: auxiliary-loss-free bias routing). The pages give the technique's name
// and purpose, not its rule; the rule implemented is
//     b_e <- b_e + u * sign(mean load - load_e),   loads = tokens routed to each expert,
// so under-loaded experts become more likely to be selected and over-loaded ones less.
//
// The sign is decided in exact integer arithmetic: mean - load_e has the sign of
// sum(counts) - E * counts[e] (int64, no rounding). The bias then moves by one fp32 add of
// u * sign (exact), so the result is fully determined: no reduction order enters.
#include "moe_internal.h"

namespace moe {
namespace {

// One workgroup; thread e owns expert e (E <= 1024). The block sums all counts, then each
// thread updates its own bias entry in place.
__global__ __launch_bounds__(1024) void k_bias_update(const int32_t* __restrict__ counts,
                                                      int32_t E, float u,
                                                      float* __restrict__ bias) {
  __shared__ long long wave_sum[1024 / kWave];
  const int e = threadIdx.x;
  const long long c = e < E ? (long long)counts[e] : 0;
  long long v = c;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if ((e & (kWave - 1)) == 0) wave_sum[e / kWave] = v;
  __syncthreads();
  long long total = 0;
  const int waves = blockDim.x / kWave;
  for (int w = 0; w < waves; ++w) total += wave_sum[w];
  if (e < E) {
    const long long d = total - (long long)E * c;   // E * (mean - load_e)
    const float sgn = d > 0 ? 1.0f : (d < 0 ? -1.0f : 0.0f);
    bias[e] = bias[e] + u * sgn;   // u * sgn is exact; at the mean this is b + (+-0)
  }
}

}  // namespace

hipError_t launch_bias_update(const int32_t* counts, int32_t E, float u, float* bias,
                              hipStream_t s) {
  const int threads = (E + kWave - 1) / kWave * kWave;
  k_bias_update<<<1, threads, 0, s>>>(counts, E, u, bias);
  return hipGetLastError();
}

}  // namespace moe
