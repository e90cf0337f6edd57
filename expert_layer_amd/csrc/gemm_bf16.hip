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
// K loop with the weight fragments going HBM -> VGPR directly, D k-steps in
// flight.  Every weight byte of a touched expert is read once per row chunk.
// MFMA lane layout (16x16x32 bf16): lane l supplies A row l%16 and B column
// l%16, each with k = 8*(l/16) .. +7; the 16x16 fp32 result sits in lane l as
// column l%16, rows 4*(l/16) .. +3.
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8_t ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- Gate-Up
// K loop shape shared by both kernels: stages 0..D-1 are loaded up front; the
// steady-state loop consumes stage s and immediately refills it D steps ahead
// with no data-dependent control flow (so the compiler can keep D k-steps of
// loads in flight and wait with vmcnt(N > 0)); the last D steps drain.
// Rows past the end of a chunk read a valid clamped row; their results are
// never stored.
template <int MT, int D>
__global__ __launch_bounds__(kThreads) void gemm13_stream(GemmArgs a, const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ h) {
  __shared__ ChunkTable tab;
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16 * MT);
  const int H = a.H, I = a.I;
  const int NT = I / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int64_t P = a.T * a.k;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);

  for (int64_t it = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); it < items; it += nwaves) {
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
    const uint16_t* b1 = w1 + (int64_t)(n0 + lr) * H + lq * 8;
    const uint16_t* b3 = w3 + (int64_t)(n0 + lr) * H + lq * 8;
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
    bf16x8_t bg[D], bu[D], av[D][MT];
#pragma unroll
    for (int s = 0; s < D; ++s) {
      bg[s] = ld8(b1 + 32 * s);
      bu[s] = ld8(b3 + 32 * s);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[s][mt] = ld8(ap[mt] + 32 * s);
    }
    int k0 = 0;
    for (; k0 < H - 32 * D; k0 += 32 * D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          accg[mt] = mfma16(av[s][mt], bg[s], accg[mt]);
          accu[mt] = mfma16(av[s][mt], bu[s], accu[mt]);
        }
        const int kn = k0 + 32 * (s + D);
        bg[s] = ld8(b1 + kn);
        bu[s] = ld8(b3 + kn);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) av[s][mt] = ld8(ap[mt] + kn);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        accg[mt] = mfma16(av[s][mt], bg[s], accg[mt]);
        accu[mt] = mfma16(av[s][mt], bu[s], accu[mt]);
      }
    }
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
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16 * MT);
  const int H = a.H, I = a.I;
  const int NT = H / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);

  for (int64_t it = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); it < items; it += nwaves) {
    const int c = (int)(it / NT);
    const int n0 = (int)(it % NT) * 16;
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16 * MT;
    const int rend = min(r0 + 16 * MT, a.offsets[g + 1]);
    const uint16_t* w2 = g == a.E ? static_cast<const uint16_t*>(a.sw2)
                                  : static_cast<const uint16_t*>(a.w2) + (int64_t)g * H * I;
    const uint16_t* b2 = w2 + (int64_t)(n0 + lr) * I + lq * 8;
    const uint16_t* ap[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = min(r0 + mt * 16 + lr, rend - 1);
      ap[mt] = h + (int64_t)r * I + lq * 8;
    }
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t bw[D], av[D][MT];
#pragma unroll
    for (int s = 0; s < D; ++s) {
      bw[s] = ld8(b2 + 32 * s);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[s][mt] = ld8(ap[mt] + 32 * s);
    }
    int k0 = 0;
    for (; k0 < I - 32 * D; k0 += 32 * D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(av[s][mt], bw[s], acc[mt]);
        const int kn = k0 + 32 * (s + D);
        bw[s] = ld8(b2 + kn);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) av[s][mt] = ld8(ap[mt] + kn);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(av[s][mt], bw[s], acc[mt]);
    }
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

// Rows per chunk: 16 when groups are small (decode-shaped), 64 otherwise.
bool small_groups(const GemmArgs& a) { return a.T * a.k <= (int64_t)a.E * 16; }

}  // namespace

// The K loops need K % (32 * D) == 0: D = 8 when K is a multiple of 256,
// otherwise D = 4 (K is always a multiple of 128).
hipError_t launch_gemm13_bf16(const GemmArgs& a, const uint16_t* x, uint16_t* h, hipStream_t s) {
  const bool deep = a.H % 256 == 0;
  if (!small_groups(a))
    gemm13_stream<4, 4><<<stream_grid(), kThreads, 0, s>>>(a, x, h);
  else if (deep)
    gemm13_stream<1, 8><<<stream_grid(), kThreads, 0, s>>>(a, x, h);
  else
    gemm13_stream<1, 4><<<stream_grid(), kThreads, 0, s>>>(a, x, h);
  return hipGetLastError();
}

template <int YBF16>
void gemm2_dispatch(const GemmArgs& a, const uint16_t* h, void* y, hipStream_t s) {
  const bool deep = a.I % 256 == 0;
  if (!small_groups(a))
    gemm2_stream<4, 4, YBF16><<<stream_grid(), kThreads, 0, s>>>(a, h, y);
  else if (deep)
    gemm2_stream<1, 8, YBF16><<<stream_grid(), kThreads, 0, s>>>(a, h, y);
  else
    gemm2_stream<1, 4, YBF16><<<stream_grid(), kThreads, 0, s>>>(a, h, y);
}

hipError_t launch_gemm2_bf16(const GemmArgs& a, const uint16_t* h, void* y, int y_dtype, hipStream_t s) {
  if (y_dtype == 1)
    gemm2_dispatch<1>(a, h, y, s);
  else
    gemm2_dispatch<0>(a, h, y, s);
  return hipGetLastError();
}

}  // namespace moe355
