// Stage 1, routing index: per-token top-k with softmax over the selected
// logits (HPC-Ops page, FusedMoE stage 1).  One wave64 per token.
#include "route_token.hpp"

namespace moe355 {

namespace {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias,
                                                    const uint8_t* __restrict__ bias_rows, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<VPL>(logits, bias, bias_rows, t, E, k, ids, w);
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, const uint8_t* bias_rows, int64_t T,
                        int E, int k, int32_t* ids, float* w, hipStream_t s) {
  const int waves = 4;
  dim3 grid((unsigned)((T + waves - 1) / waves)), block(64 * waves);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)
    route_kernel<1><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else if (vpl <= 2)
    route_kernel<2><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else if (vpl <= 4)
    route_kernel<4><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else if (vpl <= 8)
    route_kernel<8><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe355
