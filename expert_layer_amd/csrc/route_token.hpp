// Stage 1 routing of one token by one wave64 (HPC-Ops page, FusedMoE stage 1;
// the gate function is the softmax over the k selected logits, ties to the
// lower expert id).  Shared by the routing kernel and the persistent chain.
//
// Lane l holds experts l, l+64, l+128, ... in registers.  Each of the k
// rounds finds the lane-local best not yet taken entry and reduces (value
// desc, id asc) across the wave with xor shuffles; the owning lane marks the
// winner as taken.  Lane j keeps the j-th winner, so ids and weights are
// written by lanes 0..k-1 with one coalesced store.  VPL >= ceil(E / 64);
// a larger VPL gives the same result.
#pragma once

#include "common.hpp"

namespace moe355 {

__device__ __forceinline__ bool route_beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// COHERENT = 1 writes ids and w with agent-scope atomic stores (read by
// other waves of the same launch).
template <int VPL, int COHERENT = 0>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, const float* __restrict__ bias,
                                            const uint8_t* __restrict__ bias_rows, int64_t t, int E, int k,
                                            int32_t* ids, float* w) {
  const int lane = threadIdx.x & 63;
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
      if (live[i] && (bi == 0x7FFFFFFF || route_beats(v[i], e, bv, bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || route_beats(ov, oi, bv, bi))) {
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
    if (COHERENT) {
      __hip_atomic_store(ids + t * k + lane, mine_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(w + t * k + lane, ex / sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      ids[t * k + lane] = mine_id;
      w[t * k + lane] = ex / sum;
    }
  }
}

}  // namespace moe355
