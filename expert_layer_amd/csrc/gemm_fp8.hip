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
// MFMA lane layout: lane l supplies A row l%16 and B column l%16, each with
// bytes 16j .. 16j+15 and 64+16j .. 64+16j+15 of the block, j = l/16 (any
// bijection works as long as A and B agree: the whole instruction lies inside
// one scale block); the result sits in lane l as column l%16, rows
// 4*(l/16) .. +3.
#include "tiles.hpp"

namespace moe355 {

namespace {

// Weight-streaming kernels for decode-sized groups (a 16-row chunk against a
// slab of weight rows, every weight row read once per chunk).  Weight rows
// come in whole 128-byte lines with non-temporal loads (one instruction: 8
// rows x 128 B) and pass through a 2 KB per-wave LDS tile into the fragment
// layout: lane (prow, pch) writes chunk pch of rows prow and prow + 8 at
// XOR-swizzled slots, lane (lr, j) reads chunks j and j + 4 of row lr; the
// activation rows (read by many waves) are loaded in the same layout, so A
// and B agree on the K order inside each block.  LDS operations of one wave
// run in order, so the tile needs no barrier.  D K blocks are in flight per
// wave with their scales (loads retire in issue order: a scale loaded where
// its block is computed would wait for every block prefetched after it), and
// the steady loop has no branches (KB % D == 0).  Rows past the chunk's end
// read its last row; their results are never stored.

__device__ __forceinline__ i32x8_t ld_frag(const uint8_t* p) {
  // a lane's two 16-byte pieces: bytes 0..15 and 64..79 from p
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(p);
  const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(p + 64);
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ i32x4_t ld_line(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(p));
}

__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b) {
  // A and B formats 0 = E4M3; e8m0 scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0,
                                                         127);
}

// one weight fragment (16 rows x 128 B) from its two line loads, through the tile
__device__ __forceinline__ i32x8_t tile_frag(i32x4_t* tile, i32x4_t l0, i32x4_t l1, int ws0, int ws1, int rs0,
                                             int rs1) {
  tile[ws0] = l0;
  tile[ws1] = l1;
  const i32x4_t lo = tile[rs0], hi = tile[rs1];
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------- Gate-Up
// Workgroup = 8 waves = one (16-row chunk, 128-column group) item; wave w owns
// columns n0 + 16w .. +15 (16 gate and 16 up rows).
template <int D>
__global__ __launch_bounds__(512) void gemm13_fp8_stream(GemmArgs a, const uint8_t* __restrict__ xq,
                                                         const float* __restrict__ xs,
                                                         uint8_t* __restrict__ hq,
                                                         float* __restrict__ hs) {
  __shared__ ChunkTable tab;
  __shared__ float red[8][16];
  __shared__ i32x4_t wtile[8][16 * 8];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16);
  const int H = a.H, I = a.I;
  const int KB = H / 128, NB = I / 128;
  const int64_t items = (int64_t)nchunks * NB;
  const int64_t P = a.T * a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;
  const int ws0 = prow * 8 + (pch ^ prow), ws1 = (prow + 8) * 8 + (pch ^ prow);
  const int rs0 = lr * 8 + (lq ^ (lr & 7)), rs1 = lr * 8 + ((lq + 4) ^ (lr & 7));
  i32x4_t* tile = wtile[wave];

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
    const uint8_t* g0 = w1 + (int64_t)(n0 + prow) * H + 16 * pch;
    const uint8_t* u0 = w3 + (int64_t)(n0 + prow) * H + 16 * pch;
    const int64_t r8 = (int64_t)8 * H;
    auto token = [&](int r) -> int64_t { return r < P ? (int64_t)(a.slot_pair[r] / a.k) : (int64_t)r - P; };
    // A: row r0 + lr (token gathered through the routing index)
    const uint8_t* ap = xq + token(min(r0 + lr, rend - 1)) * H + 16 * lq;
    // output rows of this lane: r0 + 4*lq + i; their activation scale rows
    const float* xsr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xsr[i] = xs + token(min(r0 + lq * 4 + i, rend - 1)) * KB;
    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    i32x8_t av[D];
    i32x4_t lg0[D], lg1[D], lu0[D], lu1[D];
    float xv[D][4], sg[D], su[D];
    auto load = [&](int s, int kb) {
      const int k = 128 * kb;
      lg0[s] = ld_line(g0 + k);
      lg1[s] = ld_line(g0 + r8 + k);
      lu0[s] = ld_line(u0 + k);
      lu1[s] = ld_line(u0 + r8 + k);
      av[s] = ld_frag(ap + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[s][i] = xsr[i][kb];
      sg[s] = s1[kb];
      su[s] = s3[kb];
    };
    auto consume = [&](int s) {
      const f32x4_t pg = mfma_fp8(av[s], tile_frag(tile, lg0[s], lg1[s], ws0, ws1, rs0, rs1));
      const f32x4_t pu = mfma_fp8(av[s], tile_frag(tile, lu0[s], lu1[s], ws0, ws1, rs0, rs1));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accg[i] = __builtin_fmaf(xv[s][i] * sg[s], pg[i], accg[i]);
        accu[i] = __builtin_fmaf(xv[s][i] * su[s], pu[i], accu[i]);
      }
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, s);
    int kb0 = 0;
    for (; kb0 < KB - D; kb0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        consume(s);
        load(s, kb0 + s + D);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) consume(s);
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
// A wave owns one 16-row chunk x 16 output columns.
template <int YBF16, int D>
__global__ __launch_bounds__(256) void gemm2_fp8_stream(GemmArgs a, const uint8_t* __restrict__ hq,
                                                        const float* __restrict__ hs,
                                                        void* __restrict__ y) {
  __shared__ ChunkTable tab;
  __shared__ i32x4_t wtile[4][16 * 8];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16);
  const int H = a.H, I = a.I;
  const int KB = I / 128, HB = H / 128;
  const int NT = H / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;
  const int ws0 = prow * 8 + (pch ^ prow), ws1 = (prow + 8) * 8 + (pch ^ prow);
  const int rs0 = lr * 8 + (lq ^ (lr & 7)), rs1 = lr * 8 + ((lq + 4) ^ (lr & 7));
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  i32x4_t* tile = wtile[threadIdx.x >> 6];

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
    const uint8_t* b0 = w2 + (int64_t)(n0 + prow) * I + 16 * pch;
    const int64_t r8 = (int64_t)8 * I;
    const uint8_t* ap = hq + (int64_t)min(r0 + lr, rend - 1) * I + 16 * lq;
    const float* hsr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hsr[i] = hs + (int64_t)min(r0 + lq * 4 + i, rend - 1) * KB;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    i32x8_t av[D];
    i32x4_t l0[D], l1[D];
    float hv[D][4], sw[D];
    auto load = [&](int s, int kb) {
      const int k = 128 * kb;
      l0[s] = ld_line(b0 + k);
      l1[s] = ld_line(b0 + r8 + k);
      av[s] = ld_frag(ap + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[s][i] = hsr[i][kb];
      sw[s] = s2[kb];
    };
    auto consume = [&](int s) {
      const f32x4_t p = mfma_fp8(av[s], tile_frag(tile, l0[s], l1[s], ws0, ws1, rs0, rs1));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(hv[s][i] * sw[s], p[i], acc[i]);
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, s);
    int kb0 = 0;
    for (; kb0 < KB - D; kb0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        consume(s);
        load(s, kb0 + s + D);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) consume(s);
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
  // one workgroup per CU, the number resident (decode shape: 0.433 ms against
  // 0.444 ms with a grid of four per CU)
  const int KB = a.H / 128, grid = device_cus();
  if (KB % 4 == 0)
    gemm13_fp8_stream<4><<<grid, 512, 0, s>>>(a, xq, xs, hq, hs);
  else if (KB % 2 == 0)
    gemm13_fp8_stream<2><<<grid, 512, 0, s>>>(a, xq, xs, hq, hs);
  else
    gemm13_fp8_stream<1><<<grid, 512, 0, s>>>(a, xq, xs, hq, hs);
  return hipGetLastError();
}

template <int YBF16>
static void launch_down_fp8(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, hipStream_t s) {
  const int KB = a.I / 128, grid = device_cus() * 8;
  if (KB % 4 == 0)
    gemm2_fp8_stream<YBF16, 4><<<grid, 256, 0, s>>>(a, hq, hs, y);
  else if (KB % 2 == 0)
    gemm2_fp8_stream<YBF16, 2><<<grid, 256, 0, s>>>(a, hq, hs, y);
  else
    gemm2_fp8_stream<YBF16, 1><<<grid, 256, 0, s>>>(a, hq, hs, y);
}

hipError_t launch_gemm2_fp8(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, int y_dtype,
                            hipStream_t s) {
  if (large_groups(a) && tiled_fp8_gemm2_ok(a)) return launch_gemm2_fp8_tiled(a, hq, hs, y, y_dtype, s);
  if (y_dtype == 1)
    launch_down_fp8<1>(a, hq, hs, y, s);
  else
    launch_down_fp8<0>(a, hq, hs, y, s);
  return hipGetLastError();
}

}  // namespace moe355
