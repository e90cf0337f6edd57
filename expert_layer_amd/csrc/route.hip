// Stage 1, routing index: per-token top-k with softmax over the selected
// logits (HPC-Ops page, FusedMoE stage 1; the gate function is the softmax
// over the k selected values, ties to the lower expert id).
//
// One wave64 per token.  Lane l holds experts l, l+64, l+128, ... in
// registers.  Each of the k rounds finds the lane-local best not yet taken
// entry and reduces (value desc, id asc) across the wave with xor shuffles;
// the owning lane marks the winner as taken.  Lane j keeps the j-th winner,
// so ids and weights are written by lanes 0..k-1 with one coalesced store.
#include "common.hpp"

namespace moe355 {

namespace {

__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias,
                                                    const uint8_t* __restrict__ bias_rows, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const bool biased = bias != nullptr && (bias_rows == nullptr || bias_rows[t] != 0);
  float v[VPL];
  bool live[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    live[i] = e < E;
    float l = 0.0f;
    if (live[i]) {
      l = logits[t * E + e];
      if (biased) l = l + bias[e];
    }
    v[i] = l;
  }
  float mine_v = 0.0f;
  int mine_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (live[i] && (bi == 0x7FFFFFFF || beats(v[i], e, bv, bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || beats(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (bi == lane + 64 * i) live[i] = false;
    }
    if (lane == j) {
      mine_v = bv;
      mine_id = bi;
    }
  }
  const float top = __shfl(mine_v, 0);
  float ex = lane < k ? expf(mine_v - top) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[t * k + lane] = mine_id;
    w[t * k + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, const uint8_t* bias_rows, int64_t T,
                        int E, int k, int32_t* ids, float* w, hipStream_t s) {
  const int waves = 4;
  dim3 grid((unsigned)((T + waves - 1) / waves)), block(64 * waves);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)
    route_kernel<1><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else if (vpl <= 2)
    route_kernel<2><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else if (vpl <= 4)
    route_kernel<4><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else if (vpl <= 8)
    route_kernel<8><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, bias, bias_rows, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe355
