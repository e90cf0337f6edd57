// Grouped expert GEMMs with MXFP8 operands on gfx950's block-scaled matrix
// cores.  MXFP8 is the microscaling FP8 format the PR #54160 report lists
// beside the FP8 blockwise 128x128 scales (implementation item 4): 32
// consecutive values along K share a power-of-two scale stored as an E8M0
// byte, elements are E4M3.
//
// v_mfma_scale_f32_16x16x128_f8f6f4 takes one E8M0 scale per lane for each
// operand, and lane (r, j) -- row r = lane % 16 of the 16-row fragment,
// j = lane / 16 -- supplies the scale of row r's j-th 32-value block of the
// instruction's 128 K (established on the hardware with one-hot operands).
// With the fragment layout of the FP8 kernels (lane group j holds K bytes
// 16j..16j+15 and 64+16j..64+16j+15) the hardware applies every block scale
// itself, so the block products accumulate straight into the fp32
// accumulators: no per-block promotion in VALU as with 128x128 fp32 scales.
//
// Tile, 2-slot ring of 128-K stages, 8 waves in a 2 x 4 grid, items, the
// XCD-aware worker order and fragment skipping are those of the FP8 tiled
// kernels.  Per stage every tile row also brings one 4-byte word (its four
// block scales) into LDS.  The Gate-Up epilogue requantises h per row per 32
// columns with the MX rule: a wave's 32 h columns are exactly one block, so
// the row amax is a 16-lane shuffle.  The Gate-Up workgroups of one XCD meet
// at a counter in the caller's workspace after every round of items (bounded
// wait; it only affects timing).
//
// PT = 1 is the per-tensor FP8 mode (HPC-Ops page, main functions: the
// GroupGEMM supports per-tensor as well as block-wise FP8): the same tiles
// and loads without the scale words, unit E8M0 scales for the matrix cores,
// and the code products accumulated over the whole K are scaled once in the
// epilogue by (activation tensor scale x the expert matrix's scale).  The
// Gate-Up epilogue writes h in fp32 and keeps the running max of |h|; each
// workgroup folds it into one word with an integer atomicMax (bit patterns of
// non-negative floats order like their values, so the result does not depend
// on the order of the updates), from which the per-tensor h scale follows.
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kTM = 256;
constexpr int kTN = 256;
constexpr int kTK = 128;                 // k per stage = 4 MX blocks
constexpr int kThreads = 512;
constexpr int kSlots = kTK / 16;         // 16-byte slots per row (8)
constexpr int kWaitVm0 = 0xF70;          // s_waitcnt vmcnt(0) only (expcnt, lgkmcnt not waited)
constexpr int kSyncSpins = 1 << 14;      // bounded round barrier: ~1 ms at most

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

// block-scaled MFMA, E4M3 operands (format 0), scales in byte 0 of sa / sb
__device__ __forceinline__ f32x4_t mfma_mx(i32x8_t a, i32x8_t b, f32x4_t c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Fragment of 16 rows x 128 k at tile row `row0` (a multiple of 16): lane
// (lr, lq) takes chunks lq and lq + 4 of row row0 + lr, the operand layout of
// the instruction; swz8 depends on the low 4 row bits only, so row0 becomes
// an immediate offset of the LDS read.
__device__ __forceinline__ i32x8_t read_frag(const i32x4_t* plo, const i32x4_t* phi, int row0) {
  const i32x4_t lo = plo[row0 * kSlots];
  const i32x4_t hi = phi[row0 * kSlots];
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// sync: 8 round counters; word (may be NULL): the h amax of the per-tensor mode
__global__ void clear_sync_mx(int* sync, unsigned* word) {
  if (threadIdx.x < 8) sync[threadIdx.x] = 0;
  if (threadIdx.x == 8 && word != nullptr) *word = 0u;
}

// MODE 0: Gate-Up (+SwiGLU; MX: requantised h, PT: fp32 h + amax); MODE 1: Down (y)
template <int MODE, int YBF16, int PT = 0>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_mx(GemmArgs a, const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ As,
                                                             void* __restrict__ out,
                                                             uint8_t* __restrict__ out_s,
                                                             int* __restrict__ sync) {
  constexpr int kScaleRows = PT ? 1 : kTM;
  __shared__ __attribute__((aligned(1024))) i32x4_t a0[kTM * kSlots], a1[kTM * kSlots];
  __shared__ __attribute__((aligned(1024))) i32x4_t b0[kTN * kSlots], b1[kTN * kSlots];
  __shared__ __attribute__((aligned(16))) int sa0[kScaleRows], sa1[kScaleRows], sb0[kScaleRows], sb1[kScaleRows];
  __shared__ ChunkTable tab;

  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nmt_total = MODE == 1 ? build_chunks_sf(tab, a.offsets, G, a.E, a.has_shared, kTM)
                                   : build_chunks(tab, a.offsets, G, kTM);
  const int H = a.H, I = a.I;
  const int K = MODE == 0 ? H : I;
  const int KB = K / kTK;                 // stages
  const int KM = K / 32;                  // scale bytes per row
  const int NT = MODE == 0 ? (2 * I) / kTN : H / kTN;
  const int64_t items = (int64_t)nmt_total * NT;
  const int64_t P = a.T * a.k;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int lrow = lane >> 3, lslot = lane & 7;   // direct-load role: 8 rows x 8 slots per load
  const int off_lo = lr * kSlots + (lq ^ swz8(lr)), off_hi = lr * kSlots + ((lq + 4) ^ swz8(lr));
  const int bsh = 8 * lq;                         // this lane's block byte inside a scale word

  const int nblk = gridDim.x;
  const int per_xcd = nblk / 8;
  const int b = blockIdx.x;
  const int worker = (nblk % 8 == 0) ? (b % 8) * per_xcd + b / 8 : b;

  // round barrier per XCD (sync: 8 zeroed counters, or NULL for none)
  __shared__ int sync_on;
  if (threadIdx.x == 0) sync_on = (sync != nullptr && nblk % 8 == 0) ? 1 : 0;
  const int64_t rounds = (items + nblk - 1) / nblk;
  float hmax = 0.0f;  // PT Gate-Up: running max |h| of this thread's outputs
  for (int64_t rnd = 0; rnd < rounds; ++rnd) {
   const int64_t it = worker + rnd * nblk;
   if (it < items) {
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
    // B rows: rows [0,128) gate, [128,256) up of h columns 128*nt .. +127
    // (Gate-Up), or rows 256*nt .. +255 of w2 (Down)
    const uint8_t* bw;
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
    } else {
      const uint8_t* wmat = static_cast<const uint8_t*>(shared ? a.sw2 : a.w2);
      bw = wmat + (shared ? 0 : g * mat) + (int64_t)(nt * kTN) * I;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * wave + i) + lrow;
        b_off[i] = row * I + ((lslot ^ swz8(row)) * 16);
      }
    }
    // scale words: waves 0-3 load the A rows 64*wave + lane, waves 4-7 the
    // weight rows 64*(wave-4) + lane of the tile (KM bytes per row in memory)
    const uint8_t* ssrc = nullptr;
    if (PT) {
    } else if (wave < 4) {
      const int row = 64 * wave + lane;
      const int r = r0 + min(row, nrows - 1);
      const int64_t srow = MODE == 0 ? (r < P ? (int64_t)(a.slot_pair[r] / a.k) : (int64_t)r - P) : (int64_t)r;
      ssrc = As + srow * KM;
    } else {
      const int row = 64 * (wave - 4) + lane;   // 0..255 in the B tile
      if (MODE == 0) {
        const bool up = row >= kTN / 2;
        const uint8_t* s = reinterpret_cast<const uint8_t*>(up ? (shared ? a.ss3 : a.s3) : (shared ? a.ss1 : a.s1));
        const int64_t wrow = (shared ? 0 : (int64_t)g * I) + nt * (kTN / 2) + (row - (up ? kTN / 2 : 0));
        ssrc = s + wrow * KM;
      } else {
        const uint8_t* s = reinterpret_cast<const uint8_t*>(shared ? a.ss2 : a.s2);
        const int64_t wrow = (shared ? 0 : (int64_t)g * H) + nt * kTN + row;
        ssrc = s + wrow * KM;
      }
    }

    // Down: the column tiles of one row tile start their K loop 0-3 blocks
    // apart, so they do not all ask L2 for the same h lines at once
    const int rot = MODE == 1 ? (nt & 3) % KB : 0;
    auto issue = [&](int kbi, i32x4_t* la, i32x4_t* lb, int* lsa, int* lsb) {
      const int kr = kbi + rot;
      const int kb = kr >= KB ? kr - KB : kr;
      const int k0 = kb * kTK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        load_lds16(A + a_off[i] + k0, &la[(4 * wave + i) * 64]);
        load_lds16(bw + b_off[i] + k0, &lb[(4 * wave + i) * 64]);
      }
      if (PT) {
      } else if (wave < 4) {
        load_lds4(ssrc + 4 * kb, &lsa[64 * wave]);
      } else {
        load_lds4(ssrc + 4 * kb, &lsb[64 * (wave - 4)]);
      }
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int mfw = min(8, max(0, nmf - 8 * wm));

    // per-lane LDS bases: fragment f / m then sits at a compile-time offset
    const int brow0 = MODE == 0 ? 32 * wn : 64 * wn;   // first B fragment row of this wave
    auto compute = [&](const i32x4_t* la, const i32x4_t* lb, const int* lsa, const int* lsb) {
      if (mfw == 0) return;
      const i32x4_t* alo = la + 128 * wm * kSlots + off_lo;
      const i32x4_t* ahi = la + 128 * wm * kSlots + off_hi;
      const i32x4_t* blo = lb + brow0 * kSlots + off_lo;
      const i32x4_t* bhi = lb + brow0 * kSlots + off_hi;
      const int* psa = lsa + (PT ? 0 : 128 * wm + lr);
      const int* psb = lsb + (PT ? 0 : brow0 + lr);
      i32x8_t bfr[4];
      int sb[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int fr = MODE == 0 ? (f < 2 ? 16 * f : kTN / 2 + 16 * (f - 2)) : 16 * f;  // relative to brow0
        bfr[f] = read_frag(blo, bhi, fr);
        sb[f] = PT ? 127 : psb[fr] >> bsh;   // byte 0 = this lane's block scale (upper bytes ignored)
      }
      if (MODE == 0 && !PT) {
        // MX Gate-Up: its requantising epilogue leaves no registers for a
        // second fragment row in flight
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m < mfw) {
            const i32x8_t af = read_frag(alo, ahi, 16 * m);
            const int sa = psa[16 * m] >> bsh;
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[m][f] = mfma_mx(af, bfr[f], acc[m][f], sa, sb[f]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
      // software-pipelined: fragment row m+1 is read from LDS while row m's
      // four MFMAs run (rows past the valid ones are read, harmlessly, but
      // not computed)
      i32x8_t acur = read_frag(alo, ahi, 0);
      int sacur = PT ? 127 : psa[0] >> bsh;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        i32x8_t anxt = acur;
        int sanxt = sacur;
        if (m + 1 < 8) {
          anxt = read_frag(alo, ahi, 16 * (m + 1));
          sanxt = PT ? 127 : psa[16 * (m + 1)] >> bsh;
        }
        if (m < mfw) {
          // raised wave priority while this wave issues its MFMAs, so the
          // issue arbiter keeps them back to back against the other wave's
          // LDS reads (1.5-2 % on the MXFP8 kernels)
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[m][f] = mfma_mx(acur, bfr[f], acc[m][f], sacur, sb[f]);
          __builtin_amdgcn_s_setprio(0);
        }
        // at most two fragment rows' operands live at a time
        __builtin_amdgcn_sched_barrier(0);
        acur = anxt;
        sacur = sanxt;
      }
    };

    // one stage: wait for its loads (the only ones in flight), barrier, refill
    // the other slot with the next stage, compute
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    issue(0, a0, b0, sa0, sb0);
    // KB is even when K % 256 == 0; otherwise the loop ends after the first stage of a pair
    for (int kb = 0; kb < KB; kb += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
      if (kb + 1 < KB) issue(kb + 1, a1, b1, sa1, sb1);
      compute(a0, b0, sa0, sb0);
      if (kb + 1 >= KB) break;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
      if (kb + 2 < KB) issue(kb + 2, a0, b0, sa0, sb0);
      compute(a1, b1, sa1, sb1);
    }

    // ---- epilogue
    if (MODE == 0 && PT) {
      // h = SiLU(g) * u in fp32 with g = acc * (xs * s1[g]), u = acc * (xs * s3[g])
      const float xsc = reinterpret_cast<const float*>(As)[0];
      const float gs = xsc * (shared ? a.ss1[0] : a.s1[g]);
      const float us = xsc * (shared ? a.ss3[0] : a.s3[g]);
      float* hf = static_cast<float*>(out);
      const int col = nt * (kTN / 2) + 32 * wn + lr;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mfw) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 128 * wm + 16 * m + 4 * lq + i;
            if (row < nrows) {
              const float h0 = silu_mul(acc[m][0][i] * gs, acc[m][2][i] * us);
              const float h1 = silu_mul(acc[m][1][i] * gs, acc[m][3][i] * us);
              const int64_t r = r0 + row;
              hf[r * I + col] = h0;
              hf[r * I + col + 16] = h1;
              hmax = fmaxf(hmax, fmaxf(fabsf(h0), fabsf(h1)));
            }
          }
        }
      }
    } else if (MODE == 0) {
      // h = SiLU(g) * u; this wave's 32 columns of a row are one MX block
      uint8_t* hq = static_cast<uint8_t*>(out);
      const int col = nt * (kTN / 2) + 32 * wn + lr;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mfw) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float h0 = silu_mul(acc[m][0][i], acc[m][2][i]);
            const float h1 = silu_mul(acc[m][1][i], acc[m][3][i]);
            const int X = mx_exponent(wave_max16(fmaxf(fabsf(h0), fabsf(h1))));
            const uint32_t codes = f32x2_to_e4m3(ldexp_f32(h0, -X), ldexp_f32(h1, -X));
            const int row = 128 * wm + 16 * m + 4 * lq + i;
            if (row < nrows) {
              const int64_t r = r0 + row;
              hq[r * I + col] = (uint8_t)(codes & 0xFF);
              hq[r * I + col + 16] = (uint8_t)(codes >> 8);
              if (lr == 0) out_s[r * (I / 32) + (col >> 5)] = (uint8_t)(X + 127);
            }
          }
        }
      }
    } else {
      // PT: y = acc * (hs * s2[g]); MX: the scales are already applied
      const float ysc = PT ? reinterpret_cast<const float*>(As)[0] * (shared ? a.ss2[0] : a.s2[g]) : 1.0f;
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
                const float v = PT ? acc[m][f][i] * ysc : acc[m][f][i];
                if (YBF16)
                  static_cast<uint16_t*>(out)[r * H + col + 16 * f] = (uint16_t)f32_to_bf16(v);
                else
                  static_cast<float*>(out)[r * H + col + 16 * f] = v;
              }
            }
          }
        }
      }
    }
   }
    // every workgroup of the XCD (workgroup b runs on XCD b % 8) arrives once
    // per round, with or without an item; after kSyncSpins polls it stops waiting
    if (rnd + 1 < rounds) {
      __syncthreads();
      if (threadIdx.x == 0 && sync_on) {
        int* c = &sync[b % 8];
        atomicAdd(c, 1);
        const int target = per_xcd * (int)(rnd + 1);
        int spins = 0;
        while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target && spins < kSyncSpins) {
          __builtin_amdgcn_s_sleep(2);
          ++spins;
        }
        if (spins >= kSyncSpins) sync_on = 0;
      }
      __syncthreads();
    }
  }
  if (MODE == 0 && PT) {
    __shared__ float red[kThreads / 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off));
    if (lane == 0) red[wave] = hmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float mx = red[0];
      for (int w = 1; w < kThreads / 64; ++w) mx = fmaxf(mx, red[w]);
      if (mx > 0.0f) atomicMax(reinterpret_cast<unsigned*>(out_s), __float_as_uint(mx));
    }
  }
}

}  // namespace

// The Down kernel needs H % 256 == 0 (weight-row tile); Gate-Up always tiles
// (2*I % 256 == 0 since I % 128 == 0).

// Groups of up to 16 rows on average take the weight-streaming kernels
// (gemm_mx_stream.hip); larger ones these tiles.
hipError_t launch_gemm13_mx(const GemmArgs& a, const uint8_t* xq, const uint8_t* xs, uint8_t* hq, uint8_t* hs,
                            int* sync, hipStream_t s) {
  if (small_groups(a)) return launch_gemm13_mx_stream(a, xq, xs, hq, hs, s);
  clear_sync_mx<<<1, 64, 0, s>>>(sync, nullptr);
  gemm_tiled_mx<0, 0><<<device_cus(), kThreads, 0, s>>>(a, xq, xs, hq, hs,
                                                       round_barrier(a, kTM) ? sync : nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm13_pt(const GemmArgs& a, const uint8_t* xq, const float* xs, float* h, float* hamax,
                            int* sync, hipStream_t s) {
  clear_sync_mx<<<1, 64, 0, s>>>(sync, reinterpret_cast<unsigned*>(hamax));
  if (small_groups(a)) return launch_gemm13_pt_stream(a, xq, xs, h, hamax, s);
  gemm_tiled_mx<0, 0, 1><<<device_cus(), kThreads, 0, s>>>(a, xq, reinterpret_cast<const uint8_t*>(xs), h,
                                                          reinterpret_cast<uint8_t*>(hamax),
                                                          round_barrier(a, kTM) ? sync : nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm2_pt(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, int y_dtype,
                           hipStream_t s) {
  const uint8_t* hsb = reinterpret_cast<const uint8_t*>(hs);
  if (small_groups(a)) return launch_gemm2_mx_stream(a, hq, hsb, y, y_dtype, 1, s);
  if (y_dtype == 1)
    gemm_tiled_mx<1, 1, 1><<<device_cus(), kThreads, 0, s>>>(a, hq, hsb, y, nullptr, nullptr);
  else
    gemm_tiled_mx<1, 0, 1><<<device_cus(), kThreads, 0, s>>>(a, hq, hsb, y, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm2_mx(const GemmArgs& a, const uint8_t* hq, const uint8_t* hs, void* y, int y_dtype,
                           hipStream_t s) {
  if (small_groups(a)) return launch_gemm2_mx_stream(a, hq, hs, y, y_dtype, 0, s);
  if (y_dtype == 1)
    gemm_tiled_mx<1, 1><<<device_cus(), kThreads, 0, s>>>(a, hq, hs, y, nullptr, nullptr);
  else
    gemm_tiled_mx<1, 0><<<device_cus(), kThreads, 0, s>>>(a, hq, hs, y, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe355
