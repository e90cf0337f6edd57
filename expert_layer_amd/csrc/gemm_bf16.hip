// Grouped expert GEMMs, bf16 operands, weight-streaming kernels (stages 2-3
// and 4 of FusedMoE, HPC-Ops page, main functions / technical principles).
//
// A wave strides over the (chunk, 16-column tile) item list and runs each
// item with the streaming item bodies (one expert weight slab per item, whole
// K loop).  Groups of 64+ rows on average go to the LDS-tiled kernels.
#include "stream_gemm.hpp"
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kThreads = 256;

template <int MT, int D>
__global__ __launch_bounds__(kThreads) void gemm13_stream(GemmArgs a, const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ h) {
  __shared__ ChunkTable tab;
  __shared__ i32x4_t tile[kThreads / 64][2][kStreamTileSlots];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16 * MT);
  const int NT = a.I / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int wave = threadIdx.x >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t it = (int64_t)blockIdx.x * (kThreads / 64) + wave; it < items; it += nwaves) {
    const int c = (int)(it / NT);
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16 * MT;
    const int rend = min(r0 + 16 * MT, a.offsets[g + 1]);
    int64_t trow[MT];
    gemm13_rows<MT>(a, r0, rend, trow);
    gemm13_stream_item<MT, D>(a, x, h, g, r0, rend, (int)(it % NT) * 16, trow, tile[wave][0], tile[wave][1]);
  }
}

template <int MT, int D, int YBF16>
__global__ __launch_bounds__(kThreads) void gemm2_stream(GemmArgs a, const uint16_t* __restrict__ h,
                                                         void* __restrict__ y) {
  __shared__ ChunkTable tab;
  __shared__ i32x4_t tile[kThreads / 64][kStreamTileSlots];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16 * MT);
  const int NT = a.H / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int wave = threadIdx.x >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t it = (int64_t)blockIdx.x * (kThreads / 64) + wave; it < items; it += nwaves) {
    const int c = (int)(it / NT);
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16 * MT;
    const int rend = min(r0 + 16 * MT, a.offsets[g + 1]);
    gemm2_stream_item<MT, D, YBF16>(a, h, y, g, r0, rend, (int)(it % NT) * 16, tile[wave], NoWait{});
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
