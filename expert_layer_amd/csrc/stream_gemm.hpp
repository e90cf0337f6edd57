// Work items of the weight-streaming grouped GEMMs (bf16 operands, fp32
// accumulation on v_mfma_f32_16x16x32_bf16), shared by the stand-alone
// Gate-Up / Down kernels and the persistent chain kernel.
//
// Stages 2-3 (Gate-Up + SwiGLU) and 4 (Down) of FusedMoE (HPC-Ops page,
// main functions / technical principles).  The Gate-Up GEMM reads its A rows
// straight from x through the routing index (slot -> pair -> token), so no
// gathered copy of x is ever written.
//
// An item is one wave's share: a 16-column slab of one expert's weight
// matrix for one chunk of up to 16*MT rows, over the whole K loop.  Weights
// are read exactly once per chunk, so they are fetched with non-temporal
// loads in whole 128-byte lines (a load instruction covers 8 weight rows x
// 128 B), D stages of 64 k in flight per wave.  The MFMA B operand wants a
// different lane layout (16 rows x 4 chunks of 16 B), so each stage goes
// through a 4 KB per-wave LDS tile: lanes write their 16-byte pieces at
// XOR-swizzled slots and read back MFMA fragments.  LDS operations of one
// wave execute in order, so the single tile needs no barrier.  The gathered
// activation rows (reused by many waves through L2) are loaded in MFMA
// layout directly.
// MFMA lane layout (16x16x32 bf16): lane l supplies A row l%16 and B column
// l%16, each with k = 8*(l/16) .. +7; the 16x16 fp32 result sits in lane l as
// column l%16, rows 4*(l/16) .. +3.
//
// K loop shape: stages 0..D-1 are loaded up front; the steady-state loop
// consumes stage s and immediately refills it D stages ahead with no
// data-dependent control flow (so D stages stay in flight and the compiler
// waits with vmcnt(N > 0)); the last D stages drain.  Rows past the end of a
// chunk read a valid clamped row; their results are never stored.  The loops
// need K % (64 * D) == 0.
#pragma once

#include "common.hpp"

namespace moe355 {

constexpr int kStreamStageK = 64;  // k elements per pipeline stage (128 B per weight row)
constexpr int kStreamTileSlots = 16 * 8;  // 16-byte slots of one 16 x 128 B weight tile

__device__ __forceinline__ bf16x8_t stream_ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

__device__ __forceinline__ i32x4_t stream_ldw(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(p));
}

__device__ __forceinline__ f32x4_t stream_mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte slot of (row, chunk) in a per-wave tile of 16 weight rows x 128 B
__device__ __forceinline__ int stream_slot(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

struct NoWait {
  __device__ void operator()() const {}
};

// Stores of results that other waves of the same launch read, and loads of
// indices those waves produced.  COHERENT = 1 makes them agent-scope atomic
// accesses (sc1: written through to, and read from, the device coherence
// point) so that a wave on another XCD sees them without a cache flush;
// COHERENT = 0 is an ordinary access (the consumer is a later kernel).
template <int COHERENT, class V>
__device__ __forceinline__ void put(V* p, V v) {
  if (COHERENT)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

template <int COHERENT, class V>
__device__ __forceinline__ V get(const V* p) {
  if (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

// Token of each of this lane's A rows r0 + 16*mt + lane%16 (rows past rend
// clamp to rend-1): routed slots map through slot_pair, shared-expert slots
// P+t are token t.
template <int MT, int COHERENT = 0>
__device__ __forceinline__ void gemm13_rows(const GemmArgs& a, int r0, int rend, int64_t trow[MT]) {
  const int64_t P = a.T * a.k;
  const int lr = threadIdx.x & 15;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(r0 + mt * 16 + lr, rend - 1);
    int64_t t = r < P ? (int64_t)(get<COHERENT>(a.slot_pair + r) / a.k) : (int64_t)r - P;
    if (COHERENT) t = min(max(t, (int64_t)0), a.T - 1);  // an index produced in this launch: keep it in bounds
    trow[mt] = t;
  }
}

// Gate-Up item: rows [r0, rend) of group g (slot space), columns n0..n0+15 of
// h; trow from gemm13_rows.  tg, tu: this wave's two LDS tiles.
template <int MT, int D, int COHERENT = 0>
__device__ __forceinline__ void gemm13_stream_item(const GemmArgs& a, const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ h, int g, int r0, int rend, int n0,
                                                   const int64_t trow[MT], i32x4_t* tg, i32x4_t* tu) {
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;  // line-load role: rows prow, prow+8; chunk pch
  const int w0 = stream_slot(prow, pch), w1s = stream_slot(prow + 8, pch);
  const int r0s = stream_slot(lr, lq), r1s = stream_slot(lr, lq + 4);
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
  for (int mt = 0; mt < MT; ++mt) ap[mt] = x + trow[mt] * H + lq * 8;
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
    const int k = kStreamStageK * s;
    sg0[s] = stream_ldw(g0 + k);
    sg1[s] = stream_ldw(g1 + k);
    su0[s] = stream_ldw(u0 + k);
    su1[s] = stream_ldw(u1 + k);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      av[s][0][mt] = stream_ld8(ap[mt] + k);
      av[s][1][mt] = stream_ld8(ap[mt] + k + 32);
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
      accg[mt] = stream_mfma(av[s][0][mt], bg0, accg[mt]);
      accu[mt] = stream_mfma(av[s][0][mt], bu0, accu[mt]);
      accg[mt] = stream_mfma(av[s][1][mt], bg1, accg[mt]);
      accu[mt] = stream_mfma(av[s][1][mt], bu1, accu[mt]);
    }
  };
  int k0 = 0;
  for (; k0 < H - kStreamStageK * D; k0 += kStreamStageK * D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      consume(s);
      const int kn = k0 + kStreamStageK * (s + D);
      sg0[s] = stream_ldw(g0 + kn);
      sg1[s] = stream_ldw(g1 + kn);
      su0[s] = stream_ldw(u0 + kn);
      su1[s] = stream_ldw(u1 + kn);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        av[s][0][mt] = stream_ld8(ap[mt] + kn);
        av[s][1][mt] = stream_ld8(ap[mt] + kn + 32);
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
        put<COHERENT>(h + (int64_t)r * I + n0 + lr, (uint16_t)f32_to_bf16(silu_mul(accg[mt][i], accu[mt][i])));
    }
  }
}

// Down item: y rows [r0, rend) of group g, columns n0..n0+15.  tw: this
// wave's LDS tile.  wait_a() runs after the first D stages of weights have
// been requested and before the first read of h, so a caller whose h rows
// are still being produced can overlap that wait with the weight fetch.
template <int MT, int D, int YBF16, int COHERENT = 0, class WaitA = NoWait>
__device__ __forceinline__ void gemm2_stream_item(const GemmArgs& a, const uint16_t* __restrict__ h,
                                                  void* __restrict__ y, int g, int r0, int rend, int n0,
                                                  i32x4_t* tw, WaitA wait_a) {
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;
  const int w0 = stream_slot(prow, pch), w1s = stream_slot(prow + 8, pch);
  const int r0s = stream_slot(lr, lq), r1s = stream_slot(lr, lq + 4);
  const uint16_t* w2 = g == a.E ? static_cast<const uint16_t*>(a.sw2)
                                : static_cast<const uint16_t*>(a.w2) + (int64_t)g * H * I;
  const uint16_t* b0 = w2 + (int64_t)(n0 + prow) * I + pch * 8;
  const uint16_t* b1 = b0 + (int64_t)8 * I;
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  i32x4_t sb0[D], sb1[D];
  bf16x8_t av[D][2][MT];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    sb0[s] = stream_ldw(b0 + kStreamStageK * s);
    sb1[s] = stream_ldw(b1 + kStreamStageK * s);
  }
  wait_a();
  const uint16_t* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(r0 + mt * 16 + lr, rend - 1);
    ap[mt] = h + (int64_t)r * I + lq * 8;
  }
#pragma unroll
  for (int s = 0; s < D; ++s) {
    const int k = kStreamStageK * s;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      av[s][0][mt] = stream_ld8(ap[mt] + k);
      av[s][1][mt] = stream_ld8(ap[mt] + k + 32);
    }
  }
  auto consume = [&](int s) {
    tw[w0] = sb0[s];
    tw[w1s] = sb1[s];
    const bf16x8_t bw0 = __builtin_bit_cast(bf16x8_t, tw[r0s]);
    const bf16x8_t bw1 = __builtin_bit_cast(bf16x8_t, tw[r1s]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = stream_mfma(av[s][0][mt], bw0, acc[mt]);
      acc[mt] = stream_mfma(av[s][1][mt], bw1, acc[mt]);
    }
  };
  int k0 = 0;
  for (; k0 < I - kStreamStageK * D; k0 += kStreamStageK * D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      consume(s);
      const int kn = k0 + kStreamStageK * (s + D);
      sb0[s] = stream_ldw(b0 + kn);
      sb1[s] = stream_ldw(b1 + kn);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        av[s][0][mt] = stream_ld8(ap[mt] + kn);
        av[s][1][mt] = stream_ld8(ap[mt] + kn + 32);
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
          put<COHERENT>(static_cast<uint16_t*>(y) + (int64_t)r * H + n0 + lr, (uint16_t)f32_to_bf16(acc[mt][i]));
        else
          put<COHERENT>(static_cast<float*>(y) + (int64_t)r * H + n0 + lr, acc[mt][i]);
      }
    }
  }
}

}  // namespace moe355
