// FP8 quantisers (OCP E4M3FN, nearest-even, saturating).
//  * rows:   per row, per group of 128 columns (activations before the gathered
//            Gate-Up GEMM);
//  * blocks: per 128x128 block of a weight matrix (the FP8 blockwise 128x128
//            checkpoint format of the PR #54160 report, implementation item 4).
// Scale = amax / 448 with a correctly rounded fp32 division (1 when amax is 0);
// code = e4m3(fp32(v / scale)).
//  * rows_mx: MXFP8 (OCP Microscaling, the format the PR #54160 report lists
//            beside the 128x128 scales): per row, per 32 columns, an E8M0
//            byte X + 127 with X = floor(log2(amax)) - 8 and codes
//            e4m3(v * 2^-X) (exact power-of-two scaling, then RNE/saturation).
//  * tensor: one scale per tensor (the per-tensor FP8 mode of the HPC-Ops
//            page's GroupGEMM, main functions), bf16 or fp32 values; the
//            amax is a separate pass (max over every workgroup, combined
//            with an integer atomicMax on the bit patterns of non-negative
//            floats, which orders like the values and does not depend on the
//            order of the updates).
#include "common.hpp"

namespace moe355 {

namespace {

// 16 lanes per 128-column group, 8 columns (16 bytes of bf16) per lane.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                         int cols, uint8_t* __restrict__ q,
                                                         float* __restrict__ sc) {
  const int groups = cols / 128;
  const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int64_t ngroups = rows * groups;
  const bool live = g < ngroups;
  const int64_t r = live ? g / groups : 0;
  const int c0 = live ? (int)(g % groups) * 128 + sub * 8 : 0;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(x + r * cols + c0);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max16(amax);
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint32_t lo = f32x2_to_e4m3(__fdiv_rn(v[0], s), __fdiv_rn(v[1], s)) |
                (f32x2_to_e4m3(__fdiv_rn(v[2], s), __fdiv_rn(v[3], s)) << 16);
  uint32_t hi = f32x2_to_e4m3(__fdiv_rn(v[4], s), __fdiv_rn(v[5], s)) |
                (f32x2_to_e4m3(__fdiv_rn(v[6], s), __fdiv_rn(v[7], s)) << 16);
  if (live) {
    *reinterpret_cast<uint2*>(q + r * cols + c0) = make_uint2(lo, hi);
    if (sub == 0) sc[g] = s;
  }
}

// One workgroup (256 threads) per 128x128 block: 64 elements per thread.
__global__ __launch_bounds__(256) void quant_blocks_kernel(const uint16_t* __restrict__ w, int rows,
                                                           int cols, uint8_t* __restrict__ q,
                                                           float* __restrict__ sc) {
  __shared__ float red[4];
  const int rb = rows / 128, cb = cols / 128;
  const int64_t blk = blockIdx.x;
  const int64_t m = blk / ((int64_t)rb * cb);
  const int bi = (int)((blk / cb) % rb), bj = (int)(blk % cb);
  // pass p covers rows p*16 .. p*16+15; thread (tr, tc) takes 8 columns of row p*16+tr
  const int tr = threadIdx.x >> 4;        // 0..15
  const int tc = (threadIdx.x & 15) * 8;  // 0..120
  const uint16_t* base = w + (m * rows + (int64_t)bi * 128) * cols + (int64_t)bj * 128;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint4 raw = *reinterpret_cast<const uint4*>(base + (int64_t)(p * 16 + tr) * cols + tc);
    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[p][2 * i] = bf16_to_f32(u[i] & 0xFFFFu);
      v[p][2 * i + 1] = bf16_to_f32(u[i] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[p][2 * i]), fabsf(v[p][2 * i + 1])));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint8_t* qb = q + (m * rows + (int64_t)bi * 128) * cols + (int64_t)bj * 128;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    uint32_t lo = f32x2_to_e4m3(__fdiv_rn(v[p][0], s), __fdiv_rn(v[p][1], s)) |
                  (f32x2_to_e4m3(__fdiv_rn(v[p][2], s), __fdiv_rn(v[p][3], s)) << 16);
    uint32_t hi = f32x2_to_e4m3(__fdiv_rn(v[p][4], s), __fdiv_rn(v[p][5], s)) |
                  (f32x2_to_e4m3(__fdiv_rn(v[p][6], s), __fdiv_rn(v[p][7], s)) << 16);
    *reinterpret_cast<uint2*>(qb + (int64_t)(p * 16 + tr) * cols + tc) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) sc[blk] = s;
}

// 4 lanes per 32-column MX block, 8 columns (16 bytes of bf16) per lane.
__global__ __launch_bounds__(256) void quant_rows_mx_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int cols, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sc) {
  const int nb = cols / 32;
  const int64_t blk = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const bool live = blk < rows * nb;
  const int64_t r = live ? blk / nb : 0;
  const int c0 = live ? (int)(blk % nb) * 32 + sub * 8 : 0;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(x + r * cols + c0);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int X = mx_exponent(amax);
  uint32_t lo = f32x2_to_e4m3(ldexp_f32(v[0], -X), ldexp_f32(v[1], -X)) |
                (f32x2_to_e4m3(ldexp_f32(v[2], -X), ldexp_f32(v[3], -X)) << 16);
  uint32_t hi = f32x2_to_e4m3(ldexp_f32(v[4], -X), ldexp_f32(v[5], -X)) |
                (f32x2_to_e4m3(ldexp_f32(v[6], -X), ldexp_f32(v[7], -X)) << 16);
  if (live) {
    *reinterpret_cast<uint2*>(q + r * cols + c0) = make_uint2(lo, hi);
    if (sub == 0) sc[blk] = (uint8_t)(X + 127);
  }
}

// 8 consecutive values of a bf16 (F32 = 0) or fp32 (F32 = 1) array at i
template <int F32>
__device__ __forceinline__ void load8(const void* x, int64_t i, float v[8]) {
  if (F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + i);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + i);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
  }
}

template <int F32>
__device__ __forceinline__ const void* tensor_base(const void* x, int64_t m, int64_t n) {
  return F32 ? static_cast<const void*>(static_cast<const float*>(x) + m * n)
             : static_cast<const void*>(static_cast<const uint16_t*>(x) + m * n);
}

__global__ void zero_words(unsigned* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// amax[m] |= max |x| over tensor m (blockIdx.y); amax starts at 0.  Four
// 8-value loads per thread are in flight per iteration, so a grid of a few
// hundred workgroups (one same-address atomic each) streams at full rate.
template <int F32>
__global__ __launch_bounds__(256) void tensor_amax_kernel(const void* __restrict__ x, int64_t n,
                                                          unsigned* __restrict__ amax) {
  __shared__ float red[4];
  const int64_t m = blockIdx.y;
  const void* base = tensor_base<F32>(x, m, n);
  float mx = 0.0f;
  const int64_t step = (int64_t)gridDim.x * 256 * 8;
  int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  for (; i + 3 * step < n; i += 4 * step) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<F32>(base, i + u * step, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[u][j]));
  }
  for (; i < n; i += step) {
    float v[8];
    load8<F32>(base, i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (mx > 0.0f) atomicMax(amax + m, __float_as_uint(mx));
  }
}

// s[m] = amax[m] / 448 (1 if 0), q = e4m3(fp32(x / s[m])) over tensor m (blockIdx.y)
template <int F32>
__global__ __launch_bounds__(256) void quant_tensor_kernel(const void* __restrict__ x, int64_t n,
                                                           const float* __restrict__ amax,
                                                           uint8_t* __restrict__ q, float* __restrict__ sc) {
  const int64_t m = blockIdx.y;
  const float a = amax[m];
  const float s = a > 0.0f ? __fdiv_rn(a, 448.0f) : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) sc[m] = s;
  const void* base = tensor_base<F32>(x, m, n);
  uint8_t* qm = q + m * n;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (int64_t)gridDim.x * 256 * 8) {
    float v[8];
    load8<F32>(base, i, v);
    const uint32_t lo = f32x2_to_e4m3(__fdiv_rn(v[0], s), __fdiv_rn(v[1], s)) |
                        (f32x2_to_e4m3(__fdiv_rn(v[2], s), __fdiv_rn(v[3], s)) << 16);
    const uint32_t hi = f32x2_to_e4m3(__fdiv_rn(v[4], s), __fdiv_rn(v[5], s)) |
                        (f32x2_to_e4m3(__fdiv_rn(v[6], s), __fdiv_rn(v[7], s)) << 16);
    *reinterpret_cast<uint2*>(qm + i) = make_uint2(lo, hi);
  }
}

// workgroups per tensor: at most `total` over all tensors, none idle
dim3 tensor_grid(int64_t mats, int64_t n, int64_t total) {
  const int64_t per = std::min<int64_t>((n + 2047) / 2048, std::max<int64_t>(1, total / std::max<int64_t>(1, mats)));
  return dim3((unsigned)std::max<int64_t>(1, per), (unsigned)mats);
}

}  // namespace

hipError_t launch_tensor_amax(const void* x, int f32, int64_t mats, int64_t n, float* amax, hipStream_t s) {
  unsigned* a = reinterpret_cast<unsigned*>(amax);
  zero_words<<<(unsigned)std::min<int64_t>((mats + 255) / 256, 64), 256, 0, s>>>(a, mats);
  const dim3 grid = tensor_grid(mats, n, 512);
  if (f32)
    tensor_amax_kernel<1><<<grid, 256, 0, s>>>(x, n, a);
  else
    tensor_amax_kernel<0><<<grid, 256, 0, s>>>(x, n, a);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const void* x, int f32, int64_t mats, int64_t n, const float* amax, uint8_t* q,
                               float* sc, hipStream_t s) {
  const dim3 grid = tensor_grid(mats, n, 2048);
  if (f32)
    quant_tensor_kernel<1><<<grid, 256, 0, s>>>(x, n, amax, q, sc);
  else
    quant_tensor_kernel<0><<<grid, 256, 0, s>>>(x, n, amax, q, sc);
  return hipGetLastError();
}

hipError_t launch_quant_rows_mx(const uint16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* sc,
                                hipStream_t s) {
  const int64_t blocks = rows * (cols / 32);
  quant_rows_mx_kernel<<<(unsigned)((blocks + 63) / 64), 256, 0, s>>>(x, rows, cols, q, sc);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* sc,
                             hipStream_t s) {
  const int64_t groups = rows * (cols / 128);
  quant_rows_kernel<<<(unsigned)((groups + 15) / 16), 256, 0, s>>>(x, rows, cols, q, sc);
  return hipGetLastError();
}

hipError_t launch_quant_blocks(const uint16_t* w, int64_t mats, int rows, int cols, uint8_t* q, float* sc,
                               hipStream_t s) {
  const int64_t nblk = mats * (rows / 128) * (cols / 128);
  quant_blocks_kernel<<<(unsigned)nblk, 256, 0, s>>>(w, rows, cols, q, sc);
  return hipGetLastError();
}

}  // namespace moe355
