// Grouped expert GEMMs with FP8 (OCP E4M3FN) operands for large groups:
// LDS-tiled, one v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales) per 128-wide
// K block, whose partial sums are promoted into fp32 accumulators with the
// row scale of the activations times the 128x128 weight-block scale
// (GroupGEMM FP8 block-wise, HPC-Ops page, main functions; 128x128 scales,
// PR #54160 report, implementation item 4):
//     acc[m][n] += (xs[m, kb] * ws[n/128, kb]) * partial_kb[m][n].
// The Gate-Up kernel fuses SwiGLU and the activation requantisation stage of
// FusedMoE (one 128-column group of h per tile, the row amax is reduced over
// the four column waves through LDS) and gathers its A rows through the
// routing index.
//
// Tile: up to 256 rows x 256 weight rows, one 128-k block per stage (128 B
// per row: every direct-to-LDS load instruction fills 8 whole rows), a ring
// of 2 stages (2 x 65 KB incl. the activation scales of the stage).  Eight
// waves in a 2 (rows) x 4 (weight rows) grid, two per SIMD, as in the bf16
// kernels; items, the XCD-aware worker order and fragment skipping likewise.
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kTM = 256;
constexpr int kTN = 256;
constexpr int kTK = 128;                 // k per stage = one scale block
constexpr int kThreads = 512;
constexpr int kSlots = kTK / 16;         // 16-byte slots per row (8)
constexpr int kWaitVm0 = 0xF70;          // s_waitcnt vmcnt(0) only (expcnt, lgkmcnt not waited)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void load_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 4, 0, 0);
}

// slot of chunk c of row r: rows 2j, 2j+1 use different halves of a 256-byte
// bank sweep and 8 consecutive rows hit 8 distinct 16-byte bank groups
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0,
                                                         127);
}

// Fragment of 16 rows x 128 k at tile row `row0` (a multiple of 16): lane
// (lr, lq) takes chunks lq and lq + 4 of row row0 + lr (a bijection of the
// block's k shared by A and B).  swz8 depends on the low 4 row bits only, so
// the per-lane slot offsets are the same for every fragment and row0 becomes
// an immediate offset of the LDS read.
__device__ __forceinline__ i32x8_t read_frag(const i32x4_t* plo, const i32x4_t* phi, int row0) {
  const i32x4_t lo = plo[row0 * kSlots];
  const i32x4_t hi = phi[row0 * kSlots];
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int MODE, int YBF16>  // MODE 0: Gate-Up (+SwiGLU, requantised h); MODE 1: Down (y)
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_fp8(GemmArgs a, const uint8_t* __restrict__ A,
                                                              const float* __restrict__ As,
                                                              void* __restrict__ out,
                                                              float* __restrict__ out_s) {
  __shared__ __attribute__((aligned(1024))) i32x4_t a0[kTM * kSlots], a1[kTM * kSlots];
  __shared__ __attribute__((aligned(1024))) i32x4_t b0[kTN * kSlots], b1[kTN * kSlots];
  __shared__ __attribute__((aligned(16))) float s0[kTM], s1[kTM];
  __shared__ float red[4][kTM];
  __shared__ ChunkTable tab;

  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nmt_total = MODE == 1 ? build_chunks_sf(tab, a.offsets, G, a.E, a.has_shared, kTM)
                                   : build_chunks(tab, a.offsets, G, kTM);
  const int H = a.H, I = a.I;
  const int K = MODE == 0 ? H : I;
  const int KB = K / kTK;                 // k blocks
  const int NT = MODE == 0 ? (2 * I) / kTN : H / kTN;
  const int64_t items = (int64_t)nmt_total * NT;
  const int64_t P = a.T * a.k;
  const int IB = I / 128, HB = H / 128;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int lrow = lane >> 3, lslot = lane & 7;   // direct-load role: 8 rows x 8 slots per load
  const int off_lo = lr * kSlots + (lq ^ swz8(lr)), off_hi = lr * kSlots + ((lq + 4) ^ swz8(lr));

  const int nblk = gridDim.x;
  const int per_xcd = nblk / 8;
  const int b = blockIdx.x;
  const int worker = (nblk % 8 == 0) ? (b % 8) * per_xcd + b / 8 : b;

  for (int64_t it = worker; it < items; it += nblk) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)tab.prefix[mid] * NT <= it) lo = mid; else hi = mid - 1;
    }
    const int mtg = tab.prefix[lo + 1] - tab.prefix[lo];
    const int local = (int)(it - (int64_t)tab.prefix[lo] * NT);
    const int g = MODE == 1 ? sf_group(lo, a.E, a.has_shared) : lo;
    int mt, nt;
    item_tile<kBand>(local, mtg, NT, mt, nt);
    const int cnt = a.offsets[g + 1] - a.offsets[g];
    const int rs = mt * kTM;
    const int nrows = min(kTM, cnt - rs);
    const int r0 = a.offsets[g] + rs;
    const int nmf = (nrows + 15) >> 4;
    const bool shared = g == a.E;

    // A rows: load i (0..3) of this wave fills tile rows 8*(4*wave+i) + lane/8
    int a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * (4 * wave + i) + lrow;
      const int r = r0 + min(row, nrows - 1);
      int64_t base;
      if (MODE == 0) {
        const int64_t t = r < P ? (int64_t)(a.slot_pair[r] / a.k) : (int64_t)r - P;
        base = t * H;
      } else {
        base = (int64_t)r * I;
      }
      a_off[i] = (int)base + ((lslot ^ swz8(row)) * 16);
    }
    // activation scales of the tile rows: waves 0..3 load rows 64*wave + lane
    int as_off = 0;
    if (wave < 4) {
      const int row = 64 * wave + lane;
      const int r = r0 + min(row, nrows - 1);
      int64_t base;
      if (MODE == 0) {
        const int64_t t = r < P ? (int64_t)(a.slot_pair[r] / a.k) : (int64_t)r - P;
        base = t * (H / 128);
      } else {
        base = (int64_t)r * IB;
      }
      as_off = (int)base;
    }
    // B rows: same interleaving as the bf16 Gate-Up tile (rows [0,128) gate,
    // [128,256) up of columns n0..n0+127, n0 = 128*nt)
    const uint8_t* bw;
    const float *wsc0, *wsc1;   // weight scales [.., KB] for the wave's gate/up (or down) columns
    int b_off[4];
    const int64_t mat = (int64_t)I * H;
    if (MODE == 0) {
      const int half = wave >> 2;  // waves 0-3 load gate rows, 4-7 up rows
      const uint8_t* wmat = static_cast<const uint8_t*>(half == 0 ? (shared ? a.sw1 : a.w1) : (shared ? a.sw3 : a.w3));
      bw = wmat + (shared ? 0 : g * mat) + (int64_t)(nt * (kTN / 2)) * H;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * wave + i) + lrow;        // 0..255 in the B tile
        const int wrow = row - half * (kTN / 2);
        b_off[i] = wrow * H + ((lslot ^ swz8(row)) * 16);
      }
      const int64_t blk = (int64_t)IB * HB;
      wsc0 = (shared ? a.ss1 : a.s1 + g * blk) + (int64_t)nt * HB;
      wsc1 = (shared ? a.ss3 : a.s3 + g * blk) + (int64_t)nt * HB;
    } else {
      const uint8_t* wmat = static_cast<const uint8_t*>(shared ? a.sw2 : a.w2);
      bw = wmat + (shared ? 0 : g * mat) + (int64_t)(nt * kTN) * I;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * wave + i) + lrow;
        b_off[i] = row * I + ((lslot ^ swz8(row)) * 16);
      }
      const int64_t blk = (int64_t)HB * IB;
      wsc0 = (shared ? a.ss2 : a.s2 + g * blk) + (int64_t)(2 * nt + (wn >> 1)) * IB;
      wsc1 = wsc0;
    }

    // Down: the column tiles of one row tile start their K loop 0-3 blocks
    // apart, so they do not all ask L2 for the same h lines at once; every
    // k-block index (codes, activation and weight scales) is rotated alike
    const int rot = MODE == 1 ? (nt & 3) % KB : 0;
    auto rk = [&](int kbi) { return kbi + rot >= KB ? kbi + rot - KB : kbi + rot; };
    auto issue = [&](int kbi, i32x4_t* la, i32x4_t* lb, float* ls) {
      const int kb = rk(kbi);
      const int k0 = kb * kTK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        load_lds16(A + a_off[i] + k0, &la[(4 * wave + i) * 64]);
        load_lds16(bw + b_off[i] + k0, &lb[(4 * wave + i) * 64]);
      }
      if (wave < 4) load_lds4(As + as_off + kb, &ls[64 * wave]);
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int mfw = min(8, max(0, nmf - 8 * wm));

    // per-lane LDS bases: fragment f / m then sits at a compile-time offset
    const int brow0 = MODE == 0 ? 32 * wn : 64 * wn;   // first B fragment row of this wave
    auto compute = [&](float wg, float wu, const i32x4_t* la, const i32x4_t* lb, const float* ls) {
      if (mfw == 0) return;
      const i32x4_t* alo = la + 128 * wm * kSlots + off_lo;
      const i32x4_t* ahi = la + 128 * wm * kSlots + off_hi;
      const i32x4_t* blo = lb + brow0 * kSlots + off_lo;
      const i32x4_t* bhi = lb + brow0 * kSlots + off_hi;
      // Gate-Up takes the weight fragment as the MFMA's row operand, so lane
      // (lr, lq) holds columns 4*lq .. +3 of tile row lr and needs one
      // activation scale per fragment (one LDS word, two scale products per
      // fragment row instead of eight; Gate-Up 8 % faster).  In the Down kernel
      // the same change was 5 % slower, so it keeps x rows as the row operand.
      const float* lsw = ls + 128 * wm + (MODE == 0 ? lr : 4 * lq);
      i32x8_t bfr[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int fr = MODE == 0 ? (f < 2 ? 16 * f : kTN / 2 + 16 * (f - 2)) : 16 * f;  // relative to brow0
        bfr[f] = read_frag(blo, bhi, fr);
      }
      // the next fragment row's x fragment (Gate-Up: and its scale) is read
      // while this row's MFMAs run and its partials are promoted (Gate-Up 4-6 %
      // faster, where the extra registers spill 24 bytes of per-item
      // addressing, reloaded once per item, nothing inside the K loop; Down
      // 2-3 %, no spill)
      i32x8_t af_next = read_frag(alo, ahi, 0);
      float xs_next = lsw[0];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mfw) {
          const i32x8_t af = af_next;
          // the four block products first, then their promotion: each fma waits
          // only for an MFMA issued three or more slots earlier
          f32x4_t p[4];
#pragma unroll
          for (int f = 0; f < 4; ++f) p[f] = MODE == 0 ? mfma_fp8(bfr[f], af) : mfma_fp8(af, bfr[f]);
          // the promotion runs at raised wave priority, so the SIMD's issue
          // arbiter serves it ahead of the other wave and the matrix core gets
          // that wave's next MFMAs sooner (about 3 % on both fp8 kernels)
          if (MODE == 0) {
            const float xs1 = xs_next;
            if (m + 1 < 8) {
              af_next = read_frag(alo, ahi, 16 * (m + 1));
              xs_next = lsw[16 * (m + 1)];
            }
            const float fg = xs1 * wg, fu = xs1 * wu;
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[m][f][i] = __builtin_fmaf(f >= 2 ? fu : fg, p[f][i], acc[m][f][i]);
            __builtin_amdgcn_s_setprio(0);
          } else {
            const f32x4_t xs4 = *reinterpret_cast<const f32x4_t*>(&lsw[16 * m]);
            if (m + 1 < 8) af_next = read_frag(alo, ahi, 16 * (m + 1));
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[m][f][i] = __builtin_fmaf(xs4[i] * wg, p[f][i], acc[m][f][i]);
            __builtin_amdgcn_s_setprio(0);
          }
        }
        // keep the partial sums of one fragment row in flight at a time (the
        // second wave on the SIMD fills the matrix core meanwhile)
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // Weight scales of the stage being computed.  The next stage's scales are
    // loaded before its direct loads are issued, so the wait for them never
    // includes a whole stage in flight; they are wave-uniform and move to
    // scalar registers after the MFMAs.  Waits are the compiler's s_waitcnt
    // builtin, so its own wait insertion sees them and adds no drain.
    auto uniform = [](float v) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
    };
    float wg = uniform(wsc0[rk(0)]), wu = uniform(wsc1[rk(0)]);
    issue(0, a0, b0, s0);
    // KB is even when K % 256 == 0; otherwise the loop ends after the first stage of a pair
    for (int kb = 0; kb < KB; kb += 2) {
      // stage kb (slot 0): its loads are the only ones in flight
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
      float gn = 0.f, un = 0.f;
      if (kb + 1 < KB) {
        gn = wsc0[rk(kb + 1)];
        un = wsc1[rk(kb + 1)];
        issue(kb + 1, a1, b1, s1);
      }
      compute(wg, wu, a0, b0, s0);
      wg = uniform(gn);
      wu = uniform(un);
      if (kb + 1 >= KB) break;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
      gn = 0.f;
      un = 0.f;
      if (kb + 2 < KB) {
        gn = wsc0[rk(kb + 2)];
        un = wsc1[rk(kb + 2)];
        issue(kb + 2, a0, b0, s0);
      }
      compute(wg, wu, a1, b1, s1);
      wg = uniform(gn);
      wu = uniform(un);
    }

    // ---- epilogue
    if (MODE == 0) {
      // h = SiLU(g) * u; the tile's 128 columns are one quantisation group per row
      uint8_t* hq = static_cast<uint8_t*>(out);
      // h overwrites the gate accumulators (acc[m][0..1]): lane (lr, lq) holds
      // tile row 16*m + lr, columns 4*lq .. +3 of each 16-column fragment.
      // Per-row max over this wave's 32 columns (in the lane, then over the
      // four lane groups), then over the 4 column waves through LDS
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float h0 = silu_mul(acc[m][0][i], acc[m][2][i]);
          const float h1 = silu_mul(acc[m][1][i], acc[m][3][i]);
          acc[m][0][i] = h0;
          acc[m][1][i] = h1;
          v = fmaxf(v, fmaxf(fabsf(h0), fabsf(h1)));
        }
        v = fmaxf(v, __shfl_xor(v, 16));
        v = fmaxf(v, __shfl_xor(v, 32));
        if (lq == 0) red[wn][128 * wm + 16 * m + lr] = v;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mfw) {
          const int row = 128 * wm + 16 * m + lr;
          const float amax = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
          const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
          if (row < nrows) {
            const int64_t r = r0 + row;
            const int col = nt * (kTN / 2) + 32 * wn + 4 * lq;
            // four codes per fragment in one 4-byte store
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const uint32_t lo = f32x2_to_e4m3(__fdiv_rn(acc[m][f][0], sc), __fdiv_rn(acc[m][f][1], sc));
              const uint32_t hi = f32x2_to_e4m3(__fdiv_rn(acc[m][f][2], sc), __fdiv_rn(acc[m][f][3], sc));
              *reinterpret_cast<uint32_t*>(hq + r * I + col + 16 * f) = lo | (hi << 16);
            }
            if (wn == 0 && lq == 0) out_s[r * IB + nt] = sc;
          }
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mfw) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 128 * wm + 16 * m + 4 * lq + i;
            if (row < nrows) {
              const int64_t r = r0 + row;
              const int col = nt * kTN + 64 * wn + lr;
#pragma unroll
              for (int f = 0; f < 4; ++f) {
                if (YBF16)
                  static_cast<uint16_t*>(out)[r * H + col + 16 * f] = (uint16_t)f32_to_bf16(acc[m][f][i]);
                else
                  static_cast<float*>(out)[r * H + col + 16 * f] = acc[m][f][i];
              }
            }
          }
        }
      }
    }
  }
}

}  // namespace

bool tiled_fp8_gemm13_ok(const GemmArgs& a) { return (2 * a.I) % kTN == 0 && tiled_offsets_ok(a); }
bool tiled_fp8_gemm2_ok(const GemmArgs& a) { return a.H % kTN == 0 && tiled_offsets_ok(a); }

hipError_t launch_gemm13_fp8_tiled(const GemmArgs& a, const uint8_t* xq, const float* xs, uint8_t* hq, float* hs,
                                   hipStream_t s) {
  gemm_tiled_fp8<0, 0><<<device_cus(), kThreads, 0, s>>>(a, xq, xs, hq, hs);
  return hipGetLastError();
}

hipError_t launch_gemm2_fp8_tiled(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, int y_dtype,
                                  hipStream_t s) {
  if (y_dtype == 1)
    gemm_tiled_fp8<1, 1><<<device_cus(), kThreads, 0, s>>>(a, hq, hs, y, nullptr);
  else
    gemm_tiled_fp8<1, 0><<<device_cus(), kThreads, 0, s>>>(a, hq, hs, y, nullptr);
  return hipGetLastError();
}

}  // namespace moe355
