// Split-BF16 router GEMM (HPC-Ops page, "Router GEMM" under main functions
// and technical principles): fp32 router weights are split offline into a
// high bf16 part and a residual bf16 part with scale 1/256; the logits are two
// bf16 matrix-core products that share one read of the activations, kept in
// two register accumulators and combined by a single FMA in the epilogue:
//     logits = fma(x.w_lo^T, 1/256, x.w_hi^T).
#include "common.hpp"

namespace moe355 {

namespace {

__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w,
                                                           uint16_t* __restrict__ hi,
                                                           uint16_t* __restrict__ lo, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = w[i];
  const uint32_t h = f32_to_bf16(v);
  const float resid = v - bf16_to_f32(h);  // exact
  hi[i] = (uint16_t)h;
  lo[i] = (uint16_t)f32_to_bf16(resid * 256.0f);
}

__device__ __forceinline__ bf16x8_t ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// A wave computes a 32-token x 64-expert tile: 2 x 4 MFMA tiles for each of
// the hi and lo parts.  Rows past T and experts past E are masked.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ whi,
                                                          const uint16_t* __restrict__ wlo,
                                                          float* __restrict__ logits, int64_t T, int H,
                                                          int E) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int ntile_e = (E + 63) / 64;
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tt = wave_id / ntile_e;
  const int e0 = (int)(wave_id % ntile_e) * 64;
  const int64_t t0 = tt * 32;
  if (t0 >= T) return;
  const bf16x8_t zero = {};
  const uint16_t* ap[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int64_t t = t0 + m * 16 + lr;
    ap[m] = t < T ? x + t * H + lq * 8 : nullptr;
  }
  const uint16_t* bh[4];
  const uint16_t* bl[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + n * 16 + lr;
    bh[n] = e < E ? whi + (int64_t)e * H + lq * 8 : nullptr;
    bl[n] = e < E ? wlo + (int64_t)e * H + lq * 8 : nullptr;
  }
  f32x4_t ah[2][4], al[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      ah[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      al[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  for (int k0 = 0; k0 < H; k0 += 32) {
    bf16x8_t a[2], b1[4], b2[4];
#pragma unroll
    for (int m = 0; m < 2; ++m) a[m] = ap[m] ? ld8(ap[m] + k0) : zero;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      b1[n] = bh[n] ? ld8(bh[n] + k0) : zero;
      b2[n] = bl[n] ? ld8(bl[n] + k0) : zero;
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        ah[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b1[n], ah[m][n], 0, 0, 0);
        al[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b2[n], al[m][n], 0, 0, 0);
      }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + m * 16 + lq * 4 + i;
        const int e = e0 + n * 16 + lr;
        if (t < T && e < E) logits[t * E + e] = __builtin_fmaf(al[m][n][i], 0.00390625f, ah[m][n][i]);
      }
}

}  // namespace

hipError_t launch_router_split(const float* w, uint16_t* hi, uint16_t* lo, int64_t n, hipStream_t s) {
  router_split_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w, hi, lo, n);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* hi, const uint16_t* lo, float* logits,
                              int64_t T, int H, int E, hipStream_t s) {
  const int64_t waves = ((T + 31) / 32) * ((E + 63) / 64);
  router_gemm_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(x, hi, lo, logits, T, H, E);
  return hipGetLastError();
}

}  // namespace moe355
