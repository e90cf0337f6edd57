// Fixed-order top-k weighted sum of one token's expert outputs, 8 columns
// at a time (HPC-Ops page, FusedMoE stage 5): j ascending with fp32 fma,
// then the shared expert added, no atomics.  Shared by the combine kernels
// and the persistent chain.
#pragma once

#include "common.hpp"

namespace moe355 {

// One y term: 8 columns of slot s as fp32.  Every y element is read exactly
// once, so the loads are non-temporal (combine 12 % faster at T = 8192 and
// 10 % at T = 16384 than with ordinary loads).
template <int YBF16>
__device__ __forceinline__ void load_y8(const void* __restrict__ yv, int64_t s, int H, int c, float v[8]) {
  if (YBF16) {
    const i32x4_t raw =
        __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(static_cast<const uint16_t*>(yv) + s * H + c));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = (uint32_t)raw[i];
      v[2 * i] = bf16_to_f32(u & 0xFFFFu);
      v[2 * i + 1] = bf16_to_f32(u >> 16);
    }
  } else {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(yv) + s * H + c);
    const f32x4_t a0 = __builtin_nontemporal_load(p), a1 = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a0[i];
      v[4 + i] = a1[i];
    }
  }
}

// y terms of one token for 8 columns starting at c, summed in fixed order
// (fma for j = 0..k-1 ascending, then + the shared term).  BATCH terms are
// loaded before they are summed, so BATCH loads per lane are in flight; the
// order of the sum, and so every result bit, does not depend on BATCH.
template <int YBF16, int BATCH = 1>
__device__ __forceinline__ void combine8(const void* __restrict__ yv, const int32_t* slot, const float* wt,
                                         int nterm, int k, int64_t P, int64_t t, int H, int c, float acc[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int j0 = 0; j0 < nterm; j0 += BATCH) {
    float v[BATCH][8];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int j = j0 + u;
      if (j < nterm) load_y8<YBF16>(yv, j == k ? P + t : (int64_t)slot[j], H, c, v[u]);
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int j = j0 + u;
      if (j < nterm) {
        if (j == k) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += v[u][i];
        } else {
          const float a = wt[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(a, v[u][i], acc[i]);
        }
      }
    }
  }
}

__device__ __forceinline__ uint4 pack_bf16x8(const float v[8]) {
  uint4 o;
  o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  o.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
  o.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
  return o;
}

}  // namespace moe355
