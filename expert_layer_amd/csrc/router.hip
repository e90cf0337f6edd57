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

// Tiled router GEMM: a workgroup computes 128 tokens x 128 experts.  Per
// stage of 64 k, the 128 token rows and the 256 weight rows (128 hi, then 128
// lo) are one whole 128-byte line each, staged into LDS with the gfx950
// direct-to-LDS loads (8 rows per load instruction) in a ring of 2 stages
// (2 x 48 KB).  Eight waves in a 2 (tokens) x 4 (experts) grid; wave (wm, wn)
// owns tokens 64*wm .. +63 and experts 32*wn .. +31 of the tile, i.e. 4 x 2
// MFMA tiles for each of hi and lo.  Rows past T or E load the last valid row
// and are not stored.
//
// The activations cross HBM once: the expert tiles of one token tile are
// consecutive workgroups on one XCD (workgroups are dealt to the 8 XCDs round
// robin), so they start together and the second reads the token rows from
// that XCD's L2.  Workgroup b runs token tile 8 * (j / ET) + b % 8 and expert
// tile j % ET, with j = b / 8 and ET expert tiles; token tiles past T exit.
constexpr int kRT = 128;           // tokens per tile
constexpr int kRE = 128;           // experts per tile
constexpr int kRK = 64;            // k per stage
constexpr int kRSlots = kRK * 2 / 16;  // 16-byte slots per row (8)
constexpr int kRThreads = 512;
constexpr int kRWaitVm0 = 0xF70;   // s_waitcnt vmcnt(0) only

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void load_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

// slot of chunk c of row r inside a 128-byte row: a permutation of the 8
// slots for rows 0..7 and 8..15, rows of either parity on distinct slots, so
// a 16-row fragment read hits 16 distinct 16-byte bank groups; depends on the
// low 4 row bits only
__device__ __forceinline__ int rswz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__global__ __launch_bounds__(kRThreads, 1) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ whi,
                                                                   const uint16_t* __restrict__ wlo,
                                                                   float* __restrict__ logits, int64_t T, int H,
                                                                   int E) {
  __shared__ __attribute__((aligned(1024))) i32x4_t a0[kRT * kRSlots], a1[kRT * kRSlots];
  __shared__ __attribute__((aligned(1024))) i32x4_t b0[2 * kRE * kRSlots], b1[2 * kRE * kRSlots];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int lrow = lane >> 3, lslot = lane & 7;   // direct-load role: 8 rows x 8 slots per load
  const int ET = (E + kRE - 1) / kRE;
  const int j = blockIdx.x >> 3;
  const int64_t t0 = ((int64_t)8 * (j / ET) + (blockIdx.x & 7)) * kRT;
  const int e0 = (j % ET) * kRE;
  if (t0 >= T) return;   // whole workgroup: no barrier is reached

  // A: load i (0, 1) of this wave fills tile rows 8*(2*wave+i) + lane/8
  int64_t a_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (2 * wave + i) + lrow;
    const int64_t t = min(t0 + row, T - 1);
    a_off[i] = t * H + (lslot ^ rswz(row)) * 8;
  }
  // B: load i (0..3) fills tile rows 8*(4*wave+i) + lane/8; rows [0,128) hi, [128,256) lo
  const uint16_t* bsrc = wave < 4 ? whi : wlo;
  int64_t b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + lrow;
    const int e = min(e0 + (row & (kRE - 1)), E - 1);
    b_off[i] = (int64_t)e * H + (lslot ^ rswz(row)) * 8;
  }
  auto issue = [&](int kk, i32x4_t* la, i32x4_t* lb) {
    const int k0 = kk * kRK;
#pragma unroll
    for (int i = 0; i < 2; ++i) load_lds16(x + a_off[i] + k0, &la[(2 * wave + i) * 64]);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16(bsrc + b_off[i] + k0, &lb[(4 * wave + i) * 64]);
  };

  f32x4_t ah[4][2], al[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      ah[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      al[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  // per-lane fragment bases (row lr, chunk lq or lq + 4 of the stage)
  const int off0 = lr * kRSlots + (lq ^ rswz(lr));
  const int off1 = lr * kRSlots + ((lq ^ rswz(lr)) ^ 4);
  auto compute = [&](const i32x4_t* la, const i32x4_t* lb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const i32x4_t* pa = la + 64 * wm * kRSlots + (j ? off1 : off0);
      const i32x4_t* pb = lb + 32 * wn * kRSlots + (j ? off1 : off0);
      bf16x8_t bh[2], bl[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        bh[f] = __builtin_bit_cast(bf16x8_t, pb[16 * f * kRSlots]);
        bl[f] = __builtin_bit_cast(bf16x8_t, pb[(kRE + 16 * f) * kRSlots]);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, pa[16 * m * kRSlots]);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          ah[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh[f], ah[m][f], 0, 0, 0);
          al[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl[f], al[m][f], 0, 0, 0);
        }
      }
    }
  };
  // one stage: its loads are the only ones in flight; wait, barrier, refill
  // the other slot with the next stage, compute (builtin waits: the compiler's
  // own wait insertion sees them)
  auto stage = [&](bool refill, int kk, const i32x4_t* la, const i32x4_t* lb, i32x4_t* fa, i32x4_t* fb) {
    __builtin_amdgcn_s_waitcnt(kRWaitVm0);
    __builtin_amdgcn_s_barrier();
    if (refill) issue(kk + 1, fa, fb);
    compute(la, lb);
  };

  const int nk = H / kRK;   // even: H % 128 == 0
  issue(0, a0, b0);
  for (int kk = 0; kk < nk - 2; kk += 2) {
    stage(true, kk, a0, b0, a1, b1);
    stage(true, kk + 1, a1, b1, a0, b0);
  }
  stage(true, nk - 2, a0, b0, a1, b1);
  stage(false, nk - 1, a1, b1, a0, b0);

#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 64 * wm + 16 * m + 4 * lq + i;
        const int e = e0 + 32 * wn + 16 * f + lr;
        if (t < T && e < E) logits[t * E + e] = __builtin_fmaf(al[m][f][i], 0.00390625f, ah[m][f][i]);
      }
}

}  // namespace

hipError_t launch_router_split(const float* w, uint16_t* hi, uint16_t* lo, int64_t n, hipStream_t s) {
  router_split_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w, hi, lo, n);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* hi, const uint16_t* lo, float* logits,
                              int64_t T, int H, int E, hipStream_t s) {
  // token tiles rounded up to a multiple of 8, times the expert tiles
  const int64_t tt = (T + kRT - 1) / kRT;
  const int64_t nblk = ((tt + 7) / 8) * 8 * ((E + kRE - 1) / kRE);
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  router_gemm_kernel<<<(unsigned)nblk, kRThreads, 0, s>>>(x, hi, lo, logits, T, H, E);
  return hipGetLastError();
}

}  // namespace moe355
