// Grouped expert GEMMs, bf16 operands, fp32 accumulation on the CDNA4 matrix
// cores (v_mfma_f32_16x16x32_bf16).
//
// Stages 2-3 (Gate-Up + SwiGLU) and 4 (Down) of FusedMoE (HPC-Ops page,
// main functions / technical principles).  The Gate-Up GEMM reads its A rows
// straight from x through the routing index (slot -> pair -> token), so no
// gathered copy of x is ever written.
//
// Streaming design (weight-bound shapes): a wave owns a 16-column slab of one
// expert's weight matrix for one chunk of up to 16*MT rows and runs the whole
// K loop.  Weights are read exactly once per chunk, so they are fetched with
// non-temporal loads in whole 128-byte lines (a load instruction covers 8
// weight rows x 128 B), D stages of 64 k in flight per wave.  The MFMA B
// operand wants a different lane layout (16 rows x 4 chunks of 16 B), so each
// stage goes through a 4 KB per-wave LDS tile: lanes write their 16-byte
// pieces at XOR-swizzled slots and read back MFMA fragments.  LDS operations
// of one wave execute in order, so the single tile needs no barrier.  The
// gathered activation rows (reused by many waves through L2) are loaded in
// MFMA layout directly.
// MFMA lane layout (16x16x32 bf16): lane l supplies A row l%16 and B column
// l%16, each with k = 8*(l/16) .. +7; the 16x16 fp32 result sits in lane l as
// column l%16, rows 4*(l/16) .. +3.
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kThreads = 256;
constexpr int kStageK = 64;  // k elements per pipeline stage (128 B per weight row)

__device__ __forceinline__ bf16x8_t ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

__device__ __forceinline__ i32x4_t ldw(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(p));
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Per-wave LDS tile of 16 weight rows x 128 B; 16-byte slot of (row, chunk).
__device__ __forceinline__ int tile_slot(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// ---------------------------------------------------------------- Gate-Up
// K loop shape shared by both kernels: stages 0..D-1 are loaded up front; the
// steady-state loop consumes stage s and immediately refills it D stages
// ahead with no data-dependent control flow (so D stages stay in flight and
// the compiler waits with vmcnt(N > 0)); the last D stages drain.  Rows past
// the end of a chunk read a valid clamped row; their results are never stored.
template <int MT, int D>
__global__ __launch_bounds__(kThreads) void gemm13_stream(GemmArgs a, const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ h) {
  __shared__ ChunkTable tab;
  __shared__ i32x4_t tile[kThreads / 64][2][16 * 8];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16 * MT);
  const int H = a.H, I = a.I;
  const int NT = I / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int64_t P = a.T * a.k;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;  // line-load role: rows prow, prow+8; chunk pch
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  i32x4_t* tg = tile[wave][0];
  i32x4_t* tu = tile[wave][1];
  const int w0 = tile_slot(prow, pch), w1s = tile_slot(prow + 8, pch);
  const int r0s = tile_slot(lr, lq), r1s = tile_slot(lr, lq + 4);

  for (int64_t it = (int64_t)blockIdx.x * (kThreads / 64) + wave; it < items; it += nwaves) {
    const int c = (int)(it / NT);
    const int n0 = (int)(it % NT) * 16;
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16 * MT;
    const int rend = min(r0 + 16 * MT, a.offsets[g + 1]);
    const bool shared = g == a.E;
    const uint16_t* w1 = shared ? static_cast<const uint16_t*>(a.sw1)
                                : static_cast<const uint16_t*>(a.w1) + (int64_t)g * I * H;
    const uint16_t* w3 = shared ? static_cast<const uint16_t*>(a.sw3)
                                : static_cast<const uint16_t*>(a.w3) + (int64_t)g * I * H;
    const uint16_t* g0 = w1 + (int64_t)(n0 + prow) * H + pch * 8;
    const uint16_t* g1 = g0 + (int64_t)8 * H;
    const uint16_t* u0 = w3 + (int64_t)(n0 + prow) * H + pch * 8;
    const uint16_t* u1 = u0 + (int64_t)8 * H;
    const uint16_t* ap[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = min(r0 + mt * 16 + lr, rend - 1);
      const int64_t t = r < P ? (int64_t)(a.slot_pair[r] / a.k) : (int64_t)r - P;
      ap[mt] = x + t * H + lq * 8;
    }
    f32x4_t accg[MT], accu[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accg[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accu[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    i32x4_t sg0[D], sg1[D], su0[D], su1[D];
    bf16x8_t av[D][2][MT];
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int k = kStageK * s;
      sg0[s] = ldw(g0 + k);
      sg1[s] = ldw(g1 + k);
      su0[s] = ldw(u0 + k);
      su1[s] = ldw(u1 + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        av[s][0][mt] = ld8(ap[mt] + k);
        av[s][1][mt] = ld8(ap[mt] + k + 32);
      }
    }
    auto consume = [&](int s) {
      tg[w0] = sg0[s];
      tg[w1s] = sg1[s];
      tu[w0] = su0[s];
      tu[w1s] = su1[s];
      const bf16x8_t bg0 = __builtin_bit_cast(bf16x8_t, tg[r0s]);
      const bf16x8_t bg1 = __builtin_bit_cast(bf16x8_t, tg[r1s]);
      const bf16x8_t bu0 = __builtin_bit_cast(bf16x8_t, tu[r0s]);
      const bf16x8_t bu1 = __builtin_bit_cast(bf16x8_t, tu[r1s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        accg[mt] = mfma16(av[s][0][mt], bg0, accg[mt]);
        accu[mt] = mfma16(av[s][0][mt], bu0, accu[mt]);
        accg[mt] = mfma16(av[s][1][mt], bg1, accg[mt]);
        accu[mt] = mfma16(av[s][1][mt], bu1, accu[mt]);
      }
    };
    int k0 = 0;
    for (; k0 < H - kStageK * D; k0 += kStageK * D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        consume(s);
        const int kn = k0 + kStageK * (s + D);
        sg0[s] = ldw(g0 + kn);
        sg1[s] = ldw(g1 + kn);
        su0[s] = ldw(u0 + kn);
        su1[s] = ldw(u1 + kn);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          av[s][0][mt] = ld8(ap[mt] + kn);
          av[s][1][mt] = ld8(ap[mt] + kn + 32);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) consume(s);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + mt * 16 + lq * 4 + i;
        if (r < rend)
          h[(int64_t)r * I + n0 + lr] = (uint16_t)f32_to_bf16(silu_mul(accg[mt][i], accu[mt][i]));
      }
    }
  }
}

// ---------------------------------------------------------------- Down
template <int MT, int D, int YBF16>
__global__ __launch_bounds__(kThreads) void gemm2_stream(GemmArgs a, const uint16_t* __restrict__ h,
                                                         void* __restrict__ y) {
  __shared__ ChunkTable tab;
  __shared__ i32x4_t tile[kThreads / 64][16 * 8];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16 * MT);
  const int H = a.H, I = a.I;
  const int NT = H / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  i32x4_t* tw = tile[wave];
  const int w0 = tile_slot(prow, pch), w1s = tile_slot(prow + 8, pch);
  const int r0s = tile_slot(lr, lq), r1s = tile_slot(lr, lq + 4);

  for (int64_t it = (int64_t)blockIdx.x * (kThreads / 64) + wave; it < items; it += nwaves) {
    const int c = (int)(it / NT);
    const int n0 = (int)(it % NT) * 16;
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16 * MT;
    const int rend = min(r0 + 16 * MT, a.offsets[g + 1]);
    const uint16_t* w2 = g == a.E ? static_cast<const uint16_t*>(a.sw2)
                                  : static_cast<const uint16_t*>(a.w2) + (int64_t)g * H * I;
    const uint16_t* b0 = w2 + (int64_t)(n0 + prow) * I + pch * 8;
    const uint16_t* b1 = b0 + (int64_t)8 * I;
    const uint16_t* ap[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = min(r0 + mt * 16 + lr, rend - 1);
      ap[mt] = h + (int64_t)r * I + lq * 8;
    }
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    i32x4_t sb0[D], sb1[D];
    bf16x8_t av[D][2][MT];
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int k = kStageK * s;
      sb0[s] = ldw(b0 + k);
      sb1[s] = ldw(b1 + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        av[s][0][mt] = ld8(ap[mt] + k);
        av[s][1][mt] = ld8(ap[mt] + k + 32);
      }
    }
    auto consume = [&](int s) {
      tw[w0] = sb0[s];
      tw[w1s] = sb1[s];
      const bf16x8_t bw0 = __builtin_bit_cast(bf16x8_t, tw[r0s]);
      const bf16x8_t bw1 = __builtin_bit_cast(bf16x8_t, tw[r1s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = mfma16(av[s][0][mt], bw0, acc[mt]);
        acc[mt] = mfma16(av[s][1][mt], bw1, acc[mt]);
      }
    };
    int k0 = 0;
    for (; k0 < I - kStageK * D; k0 += kStageK * D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        consume(s);
        const int kn = k0 + kStageK * (s + D);
        sb0[s] = ldw(b0 + kn);
        sb1[s] = ldw(b1 + kn);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          av[s][0][mt] = ld8(ap[mt] + kn);
          av[s][1][mt] = ld8(ap[mt] + kn + 32);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) consume(s);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + mt * 16 + lq * 4 + i;
        if (r < rend) {
          if (YBF16)
            static_cast<uint16_t*>(y)[(int64_t)r * H + n0 + lr] = (uint16_t)f32_to_bf16(acc[mt][i]);
          else
            static_cast<float*>(y)[(int64_t)r * H + n0 + lr] = acc[mt][i];
        }
      }
    }
  }
}

int stream_grid() { return device_cus() * 8; }



}  // namespace

// The K loops need K % (64 * D) == 0: D = 4 when K is a multiple of 256,
// otherwise D = 2 (K is always a multiple of 128).
hipError_t launch_gemm13_bf16(const GemmArgs& a, const uint16_t* x, uint16_t* h, int* sync, hipStream_t s) {
  if (large_groups(a) && tiled_gemm13_ok(a)) return launch_gemm13_tiled(a, x, h, sync, s);
  const bool deep = a.H % 256 == 0;
  if (!small_groups(a))
    gemm13_stream<4, 2><<<stream_grid(), kThreads, 0, s>>>(a, x, h);
  else if (deep)
    gemm13_stream<1, 4><<<stream_grid(), kThreads, 0, s>>>(a, x, h);
  else
    gemm13_stream<1, 2><<<stream_grid(), kThreads, 0, s>>>(a, x, h);
  return hipGetLastError();
}

template <int YBF16>
void gemm2_dispatch(const GemmArgs& a, const uint16_t* h, void* y, hipStream_t s) {
  const bool deep = a.I % 256 == 0;
  if (!small_groups(a))
    gemm2_stream<4, 2, YBF16><<<stream_grid(), kThreads, 0, s>>>(a, h, y);
  else if (deep)
    gemm2_stream<1, 4, YBF16><<<stream_grid(), kThreads, 0, s>>>(a, h, y);
  else
    gemm2_stream<1, 2, YBF16><<<stream_grid(), kThreads, 0, s>>>(a, h, y);
}

hipError_t launch_gemm2_bf16(const GemmArgs& a, const uint16_t* h, void* y, int y_dtype, hipStream_t s) {
  if (large_groups(a) && tiled_gemm2_ok(a)) return launch_gemm2_tiled(a, h, y, y_dtype, s);
  if (y_dtype == 1)
    gemm2_dispatch<1>(a, h, y, s);
  else
    gemm2_dispatch<0>(a, h, y, s);
  return hipGetLastError();
}

}  // namespace moe355
