// Stage 5, top-k weighted combine (HPC-Ops page, FusedMoE stage 5):
//   out[t] = sum_j w[t,j] * y[pair_slot[t*k+j]] + shared * y[P+t]
// in a fixed order (j ascending, then the shared expert) in fp32, one
// round-to-nearest-even to bf16.  No atomics: one workgroup owns a token.
#include "common.hpp"

namespace moe355 {

namespace {

constexpr int kThreads = 256;

template <int YBF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ yv,
                                                           const int32_t* __restrict__ pair_slot,
                                                           const float* __restrict__ w, int64_t T, int k,
                                                           int H, int has_shared,
                                                           uint16_t* __restrict__ out) {
  __shared__ int32_t slot[33];
  __shared__ float wt[33];
  const int64_t t = blockIdx.x;
  const int64_t P = T * k;
  if (threadIdx.x < k) {
    slot[threadIdx.x] = pair_slot[t * k + threadIdx.x];
    wt[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int nterm = k + (has_shared ? 1 : 0);
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < nterm; ++j) {
      const bool sh = j == k;
      const int64_t s = sh ? P + t : (int64_t)slot[j];
      const float a = sh ? 1.0f : wt[j];
      float v[8];
      if (YBF16) {
        const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(yv) + s * H + c);
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_to_f32(u[i] & 0xFFFFu);
          v[2 * i + 1] = bf16_to_f32(u[i] >> 16);
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(yv) + s * H + c);
        const float4 a0 = p[0], a1 = p[1];
        v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
        v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
      }
      if (sh) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(a, v[i], acc[i]);
      }
    }
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
    o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
    o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
    o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + t * H + c) = o;
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dtype, const int32_t* pair_slot, const float* w, int64_t T,
                          int k, int H, int has_shared, uint16_t* out, hipStream_t s) {
  if (y_dtype == 1)
    combine_kernel<1><<<(unsigned)T, kThreads, 0, s>>>(y, pair_slot, w, T, k, H, has_shared, out);
  else
    combine_kernel<0><<<(unsigned)T, kThreads, 0, s>>>(y, pair_slot, w, T, k, H, has_shared, out);
  return hipGetLastError();
}

}  // namespace moe355
