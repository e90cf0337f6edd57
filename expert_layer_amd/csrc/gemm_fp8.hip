// Grouped expert GEMMs with FP8 (OCP E4M3FN) operands and 128x128 fp32 block
// scales (GroupGEMM FP8 block-wise, HPC-Ops page "main functions"; the
// 128x128 checkpoint scale format of the PR #54160 report, implementation
// item 4).  Activations carry one fp32 scale per row per 128 columns.
//
// One v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales) covers exactly one
// 128-wide K block, so each block's partial sum comes out of the matrix core
// unscaled and is promoted into the fp32 accumulator with the product of the
// row scale and the weight block scale:
//     acc[m][n] += (xs[m,kb] * ws[n/128,kb]) * partial_kb[m][n].
// The Gate-Up kernel fuses SwiGLU and the activation requantisation stage
// (FusedMoE stage 3): its workgroup owns whole 128-column groups of h, so the
// per-row amax of a group is a workgroup reduction.
//
// MFMA lane layout: lane l supplies A row l%16 and B column l%16, each with the
// 32 bytes k = 32*(l/16) .. +31 of the block (any bijection works as long as A
// and B agree: the whole instruction lies inside one scale block); the
// result sits in lane l as column l%16, rows 4*(l/16) .. +3.
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kD = 4;  // 128-wide K blocks in flight per wave

__device__ __forceinline__ i32x8_t ld32(const uint8_t* p) {
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(p);
  const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(p + 16);
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b) {
  // A and B formats 0 = E4M3; e8m0 scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0,
                                                         127);
}

// ---------------------------------------------------------------- Gate-Up
// Workgroup = 8 waves = one (16-row chunk, 128-column group) item; wave w owns
// columns n0 + 16w .. +15.
__global__ __launch_bounds__(512) void gemm13_fp8_stream(GemmArgs a, const uint8_t* __restrict__ xq,
                                                         const float* __restrict__ xs,
                                                         uint8_t* __restrict__ hq,
                                                         float* __restrict__ hs) {
  __shared__ ChunkTable tab;
  __shared__ float red[8][16];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16);
  const int H = a.H, I = a.I;
  const int KB = H / 128, NB = I / 128;
  const int64_t items = (int64_t)nchunks * NB;
  const int64_t P = a.T * a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const i32x8_t zero = {};

  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int c = (int)(it / NB);
    const int nb = (int)(it % NB);
    const int n0 = nb * 128 + wave * 16;
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16;
    const int rend = min(r0 + 16, a.offsets[g + 1]);
    const bool shared = g == a.E;
    const int64_t mat = (int64_t)I * H, blk = (int64_t)NB * KB;
    const uint8_t* w1 = shared ? static_cast<const uint8_t*>(a.sw1) : static_cast<const uint8_t*>(a.w1) + g * mat;
    const uint8_t* w3 = shared ? static_cast<const uint8_t*>(a.sw3) : static_cast<const uint8_t*>(a.w3) + g * mat;
    const float* s1 = (shared ? a.ss1 : a.s1 + g * blk) + (int64_t)nb * KB;
    const float* s3 = (shared ? a.ss3 : a.s3 + g * blk) + (int64_t)nb * KB;
    const uint8_t* b1 = w1 + (int64_t)(n0 + lr) * H + lq * 32;
    const uint8_t* b3 = w3 + (int64_t)(n0 + lr) * H + lq * 32;
    // A: row r0 + lr (token gathered through the routing index)
    const int ra = r0 + lr;
    const uint8_t* ap = nullptr;
    if (ra < rend) {
      const int64_t t = ra < P ? (int64_t)(a.slot_pair[ra] / a.k) : (int64_t)ra - P;
      ap = xq + t * H + lq * 32;
    }
    // output rows of this lane: r0 + 4*lq + i; their activation scale rows
    const float* xsr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + lq * 4 + i;
      xsr[i] = nullptr;
      if (r < rend) {
        const int64_t t = r < P ? (int64_t)(a.slot_pair[r] / a.k) : (int64_t)r - P;
        xsr[i] = xs + t * KB;
      }
    }
    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    i32x8_t av[kD], bg[kD], bu[kD];
#pragma unroll
    for (int s = 0; s < kD; ++s) {
      if (s < KB) {
        av[s] = ap ? ld32(ap + 128 * s) : zero;
        bg[s] = ld32(b1 + 128 * s);
        bu[s] = ld32(b3 + 128 * s);
      }
    }
    for (int kb0 = 0; kb0 < KB; kb0 += kD) {
#pragma unroll
      for (int s = 0; s < kD; ++s) {
        const int kb = kb0 + s;
        if (kb < KB) {
          const f32x4_t pg = mfma_fp8(av[s], bg[s]);
          const f32x4_t pu = mfma_fp8(av[s], bu[s]);
          const float sg = s1[kb], su = s3[kb];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float xsv = xsr[i] ? xsr[i][kb] : 0.0f;
            accg[i] = __builtin_fmaf(xsv * sg, pg[i], accg[i]);
            accu[i] = __builtin_fmaf(xsv * su, pu[i], accu[i]);
          }
          const int kn = kb + kD;
          if (kn < KB) {
            av[s] = ap ? ld32(ap + 128 * kn) : zero;
            bg[s] = ld32(b1 + 128 * kn);
            bu[s] = ld32(b3 + 128 * kn);
          }
        }
      }
    }
    // SwiGLU, then requantise each row's 128-column group
    float hv[4], am[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hv[i] = silu_mul(accg[i], accu[i]);
      am[i] = wave_max16(fabsf(hv[i]));
    }
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][lq * 4 + i] = am[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = lq * 4 + i;
      float m = red[0][rl];
#pragma unroll
      for (int w = 1; w < 8; ++w) m = fmaxf(m, red[w][rl]);
      const float sc = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
      const int r = r0 + rl;
      if (r < rend) {
        hq[(int64_t)r * I + n0 + lr] = (uint8_t)(f32x2_to_e4m3(__fdiv_rn(hv[i], sc), 0.0f) & 0xFF);
        if (wave == 0 && lr == 0) hs[(int64_t)r * NB + nb] = sc;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- Down
// A wave owns one 16-row chunk x 16 output columns.  Each K block's scales
// travel with its codes, kD blocks in flight: loads retire in issue order, so
// a scale loaded at its point of use would make the block wait for all the
// blocks prefetched after it (Down 0.39 -> 0.30 ms at decode size; the
// Gate-Up measured 1 % slower this way and keeps its scale loads at the point
// of use).  Rows past the chunk's end read the chunk's last row (their
// results are never stored), so no load sits behind a per-lane condition.
template <int YBF16>
__global__ __launch_bounds__(256) void gemm2_fp8_stream(GemmArgs a, const uint8_t* __restrict__ hq,
                                                        const float* __restrict__ hs,
                                                        void* __restrict__ y) {
  __shared__ ChunkTable tab;
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16);
  const int H = a.H, I = a.I;
  const int KB = I / 128, HB = H / 128;
  const int NT = H / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int64_t nwaves = (int64_t)gridDim.x * 4;

  for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += nwaves) {
    const int c = (int)(it / NT);
    const int n0 = (int)(it % NT) * 16;
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16;
    const int rend = min(r0 + 16, a.offsets[g + 1]);
    const bool shared = g == a.E;
    const int64_t mat = (int64_t)I * H, blk = (int64_t)HB * KB;
    const uint8_t* w2 = shared ? static_cast<const uint8_t*>(a.sw2) : static_cast<const uint8_t*>(a.w2) + g * mat;
    const float* s2 = (shared ? a.ss2 : a.s2 + g * blk) + (int64_t)(n0 / 128) * KB;
    const uint8_t* bp = w2 + (int64_t)(n0 + lr) * I + lq * 32;
    const uint8_t* ap = hq + (int64_t)min(r0 + lr, rend - 1) * I + lq * 32;
    const float* hsr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hsr[i] = hs + (int64_t)min(r0 + lq * 4 + i, rend - 1) * KB;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    i32x8_t av[kD], bw[kD];
    float hv[kD][4], sw[kD];
    auto load = [&](int s, int kb) {
      av[s] = ld32(ap + 128 * kb);
      bw[s] = ld32(bp + 128 * kb);
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[s][i] = hsr[i][kb];
      sw[s] = s2[kb];
    };
#pragma unroll
    for (int s = 0; s < kD; ++s)
      if (s < KB) load(s, s);
    for (int kb0 = 0; kb0 < KB; kb0 += kD) {
#pragma unroll
      for (int s = 0; s < kD; ++s) {
        const int kb = kb0 + s;
        if (kb < KB) {
          const f32x4_t p = mfma_fp8(av[s], bw[s]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(hv[s][i] * sw[s], p[i], acc[i]);
          if (kb + kD < KB) load(s, kb + kD);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + lq * 4 + i;
      if (r < rend) {
        if (YBF16)
          static_cast<uint16_t*>(y)[(int64_t)r * H + n0 + lr] = (uint16_t)f32_to_bf16(acc[i]);
        else
          static_cast<float*>(y)[(int64_t)r * H + n0 + lr] = acc[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm13_fp8(const GemmArgs& a, const uint8_t* xq, const float* xs, uint8_t* hq, float* hs,
                             hipStream_t s) {
  if (large_groups(a) && tiled_fp8_gemm13_ok(a)) return launch_gemm13_fp8_tiled(a, xq, xs, hq, hs, s);
  gemm13_fp8_stream<<<device_cus() * 4, 512, 0, s>>>(a, xq, xs, hq, hs);
  return hipGetLastError();
}

hipError_t launch_gemm2_fp8(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, int y_dtype,
                            hipStream_t s) {
  if (large_groups(a) && tiled_fp8_gemm2_ok(a)) return launch_gemm2_fp8_tiled(a, hq, hs, y, y_dtype, s);
  if (y_dtype == 1)
    gemm2_fp8_stream<1><<<device_cus() * 8, 256, 0, s>>>(a, hq, hs, y);
  else
    gemm2_fp8_stream<0><<<device_cus() * 8, 256, 0, s>>>(a, hq, hs, y);
  return hipGetLastError();
}

}  // namespace moe355
