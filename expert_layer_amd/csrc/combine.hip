// Stage 5, top-k weighted combine (HPC-Ops page, FusedMoE stage 5):
//   out[t] = sum_j w[t,j] * y[pair_slot[t*k+j]] + shared * y[P+t]
// in a fixed order (j ascending, then the shared expert) in fp32, one
// round-to-nearest-even to bf16.  No atomics: one workgroup owns a token.
//
// combine_rmsnorm_kernel adds the residual stream and applies RMSNorm in the
// same pass, the single-GPU half of the fused AllReduce+Norm of the HPC-Ops
// page (technical principles: RMSNorm(AllReduce(x) + residual, weight)):
//   s = combine(t) + residual[t]   (fp32, the combine sum unrounded)
//   res_out[t] = bf16(s)           (optional; may be residual itself)
//   out[t] = bf16(s * 1/sqrt(mean(s^2) + eps) * weight)
// The row of s stays in LDS between the reduction and the scaling.
#include "combine8.hpp"

namespace moe355 {

namespace {

constexpr int kThreads = 256;
// Small batches (T < 2048, latency-bound): 8 y terms are loaded before they
// are summed (decode combine 10.7 -> 8.5 us).  Large batches load 4 at a time
// (1, 2 and 4 measured the same there; the RMSNorm variant keeps 1).  All
// sum in the same order.
constexpr int64_t kBatchBelowT = 2048;

template <int YBF16, int BATCH>
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
    combine8<YBF16, BATCH>(yv, slot, wt, nterm, k, P, t, H, c, acc);
    *reinterpret_cast<uint4*>(out + t * H + c) = pack_bf16x8(acc);
  }
}

template <int YBF16, int BATCH>
__global__ __launch_bounds__(kThreads) void combine_rmsnorm_kernel(
    const void* __restrict__ yv, const int32_t* __restrict__ pair_slot, const float* __restrict__ w, int64_t T,
    int k, int H, int has_shared, const uint16_t* residual, const uint16_t* __restrict__ weight, float eps,
    uint16_t* __restrict__ out, uint16_t* res_out) {
  extern __shared__ float srow[];   // H floats: the row of s
  __shared__ int32_t slot[33];
  __shared__ float wt[33];
  __shared__ float part[kThreads / 64];
  const int64_t t = blockIdx.x;
  const int64_t P = T * k;
  if (threadIdx.x < k) {
    slot[threadIdx.x] = pair_slot[t * k + threadIdx.x];
    wt[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int nterm = k + (has_shared ? 1 : 0);
  float ssq = 0.0f;
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float acc[8];
    combine8<YBF16, BATCH>(yv, slot, wt, nterm, k, P, t, H, c, acc);
    // residual read before res_out is written (same thread, same columns), so
    // res_out may be residual itself
    const uint4 raw = *reinterpret_cast<const uint4*>(residual + t * H + c);
    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(u[i] & 0xFFFFu);
      acc[2 * i + 1] += bf16_to_f32(u[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      srow[c + i] = acc[i];
      ssq = __builtin_fmaf(acc[i], acc[i], ssq);
    }
    if (res_out) *reinterpret_cast<uint4*>(res_out + t * H + c) = pack_bf16x8(acc);
  }
  // fixed-order reduction: within each wave, then over the waves
  for (int off = 32; off >= 1; off >>= 1) ssq += __shfl_xor(ssq, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ssq;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) tot += part[i];
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(tot, (float)H) + eps));
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(weight + c);
    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
    float o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = srow[c + 2 * i] * inv * bf16_to_f32(u[i] & 0xFFFFu);
      o[2 * i + 1] = srow[c + 2 * i + 1] * inv * bf16_to_f32(u[i] >> 16);
    }
    *reinterpret_cast<uint4*>(out + t * H + c) = pack_bf16x8(o);
  }
}

}  // namespace

hipError_t launch_combine_rmsnorm(const void* y, int y_dtype, const int32_t* pair_slot, const float* w, int64_t T,
                                  int k, int H, int has_shared, const uint16_t* residual, const uint16_t* weight,
                                  float eps, uint16_t* out, uint16_t* res_out, hipStream_t s) {
  const size_t lds = (size_t)H * sizeof(float);
  const bool small = T < kBatchBelowT;
  auto go = [&](auto kern) {
    kern<<<(unsigned)T, kThreads, lds, s>>>(y, pair_slot, w, T, k, H, has_shared, residual, weight, eps, out,
                                            res_out);
  };
  if (y_dtype == 1) {
    if (small) go(combine_rmsnorm_kernel<1, 8>); else go(combine_rmsnorm_kernel<1, 1>);
  } else {
    if (small) go(combine_rmsnorm_kernel<0, 8>); else go(combine_rmsnorm_kernel<0, 1>);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, int y_dtype, const int32_t* pair_slot, const float* w, int64_t T,
                          int k, int H, int has_shared, uint16_t* out, hipStream_t s) {
  const bool small = T < kBatchBelowT;
  auto go = [&](auto kern) { kern<<<(unsigned)T, kThreads, 0, s>>>(y, pair_slot, w, T, k, H, has_shared, out); };
  if (y_dtype == 1) {
    if (small) go(combine_kernel<1, 8>); else go(combine_kernel<1, 4>);
  } else {
    if (small) go(combine_kernel<0, 8>); else go(combine_kernel<0, 4>);
  }
  return hipGetLastError();
}

}  // namespace moe355
