// Weight-streaming grouped GEMMs for MXFP8 and per-tensor FP8 experts with
// small groups (decode-shaped batches: up to 16 rows per expert on average),
// where the tiled kernels would run mostly padded 256-row tiles.
//
// MXFP8 is the microscaling FP8 format the PR #54160 report lists beside the
// FP8 blockwise 128x128 scales (implementation item 4); per-tensor FP8 is the
// second mode of the HPC-Ops page's FP8 GroupGEMM (main functions).  Both run
// on v_mfma_scale_f32_16x16x128_f8f6f4: lane (r, j) of a 16-row fragment holds
// K bytes 16 j .. +15 and 64 + 16 j .. +15 of row r's 128-byte K block and
// supplies the E8M0 scale of that row's j-th 32-value block, so the matrix
// core applies every MX block scale itself and the block products accumulate
// in place.  Per-tensor mode passes unit scales and scales the whole-K sums
// once in the epilogue (activation scale x the expert matrix's scale).
//
// An item is a 16-row chunk of one group (the chunk table of tiles.hpp) and a
// slab of weight rows; every weight row of the slab is read once per chunk,
// which for these batches means once.  The weight rows are fetched in whole
// 128-byte lines with non-temporal loads (one load instruction: 8 rows x
// 128 B) and pass through a 2 KB per-wave LDS tile into the MFMA fragment
// layout: lane (prow, pch) writes chunk pch of rows prow and prow + 8 at
// XOR-swizzled slots, lane (lr, j) reads chunks j and j + 4 of row lr.  LDS
// operations of one wave run in order, so the one tile, reused fragment
// after fragment, needs no barrier.  (Loading the fragments directly, each
// load instruction covers half of every line it touches; the line loads made
// the Down 13-14 % faster.)  The activation rows, read by many waves, are
// loaded in fragment layout with ordinary loads.  D K blocks are in flight
// per wave; rows past the chunk's end read its last row, and their results
// are not stored.
//   * Gate-Up: a workgroup of 4 waves owns one chunk x 128 h columns; wave w
//     owns columns 32 w .. +31 (gate and up rows), which for MX are exactly
//     one 32-column block of the requantised h, so the row amax is a 16-lane
//     shuffle (the layout of the tiled MX epilogue).  Per-tensor writes h in
//     fp32 and folds max |h| into one word with an integer atomicMax on the
//     float's bits (non-negative floats order like their bit patterns).
//   * Down: a wave owns one chunk x 16 output columns over the whole K = I.
// The A rows of the Gate-Up are gathered from x through the routing index.
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kWaves13 = 4;    // Gate-Up workgroup: 4 waves x 32 columns
constexpr int kStgKB13 = 64;   // staged MX scales: K blocks per row at most (Gate-Up: H <= 8192)
constexpr int kStgKB2 = 32;    // (Down: I <= 4096)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// gfx950 direct-to-LDS load: lane l's 16 bytes land at lds_base + 16 l
__device__ __forceinline__ void load_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

// MX scale staging.  A scale byte is read once per K block, and with the
// weight codes streaming past, its 128-byte line no longer sits in L2 by the
// next block (the Gate-Up read about 1.2x its algorithmic bytes that way).
// So each wave copies the weight scale rows of its fragments (and in the Down
// the h rows' too) into its own LDS region once per item, with direct-to-LDS
// loads issued before the item's first code loads: per fragment row (16
// rows), K blocks in groups of 16, lane (lr, q) of a copy holding the 4 scale
// bytes of blocks 16 g + 4 q .. +3 of row lr.
// Only the wave itself reads its region, and LDS operations of one wave run
// in order, so no barrier is needed; the next item's copy is issued after the
// last block's scales were consumed.  Needs K % 512 == 0 (whole 16-byte pieces).
template <int G16>
__device__ __forceinline__ void stage_row(i32x4_t* region, int frow, const uint8_t* row, int KB, int lq) {
  for (int g = 0; g < (KB + 15) / 16; ++g) {
    const int kb = min(16 * g + 4 * lq, KB - 4);   // lanes past the row copy a valid piece (never read)
    load_lds16(row + 4 * kb, region + (frow * G16 + g) * 64);
  }
}

template <int G16>
__device__ __forceinline__ int staged_byte(const i32x4_t* region, int frow, int kb, int lr, int lq) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(region + (frow * G16 + (kb >> 4)) * 64 + lr + 16 * ((kb & 15) >> 2));
  return p[4 * (kb & 3) + lq];
}

__device__ __forceinline__ i32x8_t ld_frag(const uint8_t* p) {
  // the two 16-byte pieces of a lane: bytes 0..15 and 64..79 from p
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(p);
  const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(p + 64);
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// block-scaled MFMA, E4M3 operands (format 0), scales in byte 0 of sa / sb
__device__ __forceinline__ f32x4_t mfma_mx(i32x8_t a, i32x8_t b, f32x4_t c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// this lane's E8M0 byte (block lq of K block kb) from a row of scale bytes
// [K / 32]; 127 (2^0) for a row that is not there
__device__ __forceinline__ int scale_byte(const uint8_t* row, int kb, int lq) {
  return row ? (int)row[4 * kb + lq] : 127;
}

// ---------------------------------------------------------------- Gate-Up
template <int PT, int STG, int D>
__global__ __launch_bounds__(64 * kWaves13, 2) void gemm13_mx_stream(GemmArgs a, const uint8_t* __restrict__ xq,
                                                                  const uint8_t* __restrict__ xs,
                                                                  void* __restrict__ hout,
                                                                  uint8_t* __restrict__ hs) {
  __shared__ ChunkTable tab;
  constexpr int G16 = kStgKB13 / 16;
  // staged scales: per wave, the weight rows of fragments 0-3 (the activation
  // rows' scale lines, read by every wave of the chunk, stay in L2)
  __shared__ i32x4_t stg[STG ? kWaves13 * 4 * G16 * 64 : 1];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16);
  const int H = a.H, I = a.I;
  const int KB = H / 128, NB = I / 128, HM = H / 32;
  const int64_t items = (int64_t)nchunks * NB;
  const int64_t P = a.T * a.k;
  __shared__ i32x4_t wtile[kWaves13][16 * 8];   // per-wave weight tile (one 16-row fragment)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;   // line-load role: row prow of 8, chunk pch
  const int ws0 = prow * 8 + (pch ^ prow), ws1 = (prow + 8) * 8 + (pch ^ prow);
  const int rs0 = lr * 8 + (lq ^ (lr & 7)), rs1 = lr * 8 + ((lq + 4) ^ (lr & 7));
  float hmax = 0.0f;   // per-tensor: running max |h| of this thread
  i32x4_t* region = stg + (STG ? wave * 4 * G16 * 64 : 0);
  i32x4_t* tile = wtile[wave];

  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int c = (int)(it / NB);
    const int nb = (int)(it % NB);
    const int n0 = nb * 128 + wave * 32;
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16;
    const int rend = min(r0 + 16, a.offsets[g + 1]);
    const bool shared = g == a.E;
    const int64_t mat = (int64_t)I * H;
    const uint8_t* w1 = shared ? static_cast<const uint8_t*>(a.sw1) : static_cast<const uint8_t*>(a.w1) + g * mat;
    const uint8_t* w3 = shared ? static_cast<const uint8_t*>(a.sw3) : static_cast<const uint8_t*>(a.w3) + g * mat;
    // B rows: fragment f = 0, 1 holds gate rows n0 + 16 f + lr, f = 2, 3 the
    // matching up rows.  Line loads: instruction i (0..3) of gate / up covers
    // rows n0 + 8 i + prow, so fragment f is instructions 2 (f & 1) and +1.
    const uint8_t* gl = w1 + (int64_t)(n0 + prow) * H + 16 * pch;
    const uint8_t* ul = w3 + (int64_t)(n0 + prow) * H + 16 * pch;
    const uint8_t* bs[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int row = n0 + 16 * (f & 1) + lr;
      if (PT) {
        bs[f] = nullptr;
      } else {
        const uint8_t* sm = reinterpret_cast<const uint8_t*>(f < 2 ? (shared ? a.ss1 : a.s1) : (shared ? a.ss3 : a.s3));
        bs[f] = sm + ((shared ? 0 : (int64_t)g * I) + row) * HM;
      }
    }
    // A: row r0 + lr (token gathered through the routing index); rows past
    // the chunk read its last row (their results are never stored)
    const int ra = min(r0 + lr, rend - 1);
    const int64_t ta = ra < P ? (int64_t)(a.slot_pair[ra] / a.k) : (int64_t)ra - P;
    const uint8_t* ap = xq + ta * H + 16 * lq;
    const uint8_t* as = PT ? nullptr : xs + ta * HM;
    if (STG) {
#pragma unroll
      for (int f = 0; f < 4; ++f) stage_row<G16>(region, f, bs[f], KB, lq);
    }
    f32x4_t acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // codes and the activation scale bytes (and unstaged weight scale bytes)
    // of D K blocks in flight; staged scales are read from LDS when their
    // block is computed
    i32x8_t av[D];
    i32x4_t bl[D][8];
    int sav[D], sbv[D][4];
    auto load = [&](int s, int kb) {
      av[s] = ld_frag(ap + 128 * kb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bl[s][i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(gl + (int64_t)8 * i * H + 128 * kb));
        bl[s][4 + i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(ul + (int64_t)8 * i * H + 128 * kb));
      }
      sav[s] = PT ? 127 : scale_byte(as, kb, lq);
      if (!STG) {
#pragma unroll
        for (int f = 0; f < 4; ++f) sbv[s][f] = PT ? 127 : scale_byte(bs[f], kb, lq);
      }
    };
    auto consume = [&](int s, int kb) {
      if (STG) {
#pragma unroll
        for (int f = 0; f < 4; ++f) sbv[s][f] = staged_byte<G16>(region, f, kb, lr, lq);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int i0 = (f < 2 ? 0 : 4) + 2 * (f & 1);
        tile[ws0] = bl[s][i0];
        tile[ws1] = bl[s][i0 + 1];
        const i32x4_t lo = tile[rs0], hi = tile[rs1];
        const i32x8_t bf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[f] = mfma_mx(av[s], bf, acc[f], sav[s], sbv[s][f]);
      }
    };
    // KB % D == 0 (KB is even: H % 256 == 0): the steady loop has no branches
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, s);
    int kb0 = 0;
    for (; kb0 < KB - D; kb0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        consume(s, kb0 + s);
        load(s, kb0 + s + D);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) consume(s, kb0 + s);
    // lane (lr, lq) holds rows 4 lq + i, columns lr (f = 0 / 2) and lr + 16 (f = 1 / 3)
    if (PT) {
      const float xsc = reinterpret_cast<const float*>(xs)[0];
      const float gs = xsc * (shared ? a.ss1[0] : a.s1[g]);
      const float us = xsc * (shared ? a.ss3[0] : a.s3[g]);
      float* hf = static_cast<float*>(hout);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * lq + i;
        if (r < rend) {
          const float h0 = silu_mul(acc[0][i] * gs, acc[2][i] * us);
          const float h1 = silu_mul(acc[1][i] * gs, acc[3][i] * us);
          hf[(int64_t)r * I + n0 + lr] = h0;
          hf[(int64_t)r * I + n0 + 16 + lr] = h1;
          hmax = fmaxf(hmax, fmaxf(fabsf(h0), fabsf(h1)));
        }
      }
    } else {
      uint8_t* hq = static_cast<uint8_t*>(hout);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float h0 = silu_mul(acc[0][i], acc[2][i]);
        const float h1 = silu_mul(acc[1][i], acc[3][i]);
        const int X = mx_exponent(wave_max16(fmaxf(fabsf(h0), fabsf(h1))));
        const uint32_t codes = f32x2_to_e4m3(ldexp_f32(h0, -X), ldexp_f32(h1, -X));
        const int r = r0 + 4 * lq + i;
        if (r < rend) {
          hq[(int64_t)r * I + n0 + lr] = (uint8_t)(codes & 0xFF);
          hq[(int64_t)r * I + n0 + 16 + lr] = (uint8_t)(codes >> 8);
          if (lr == 0) hs[(int64_t)r * (I / 32) + (n0 >> 5)] = (uint8_t)(X + 127);
        }
      }
    }
  }
  if (PT) {
    __shared__ float red[kWaves13];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off));
    if (lane == 0) red[wave] = hmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float mx = red[0];
      for (int w = 1; w < kWaves13; ++w) mx = fmaxf(mx, red[w]);
      if (mx > 0.0f) atomicMax(reinterpret_cast<unsigned*>(hs), __float_as_uint(mx));
    }
  }
}

// ---------------------------------------------------------------- Down
// A wave owns one chunk x 16 output columns (one weight fragment per K
// block, through the wave's tile); D K blocks in flight, and the steady loop
// has no branches (KB % D == 0).
template <int PT, int YBF16, int STG, int D>
__global__ __launch_bounds__(256) void gemm2_mx_stream(GemmArgs a, const uint8_t* __restrict__ hq,
                                                       const uint8_t* __restrict__ hs, void* __restrict__ y) {
  __shared__ ChunkTable tab;
  constexpr int G16 = kStgKB2 / 16;
  // staged scales: per wave, fragment row 0 (weights), 1 (h rows)
  __shared__ i32x4_t stg[STG ? 4 * 2 * G16 * 64 : 1];
  __shared__ i32x4_t wtile[4][16 * 8];
  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nchunks = build_chunks(tab, a.offsets, G, 16);
  const int H = a.H, I = a.I;
  const int KB = I / 128, IM = I / 32;
  const int NT = H / 16;
  const int64_t items = (int64_t)nchunks * NT;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int prow = lane >> 3, pch = lane & 7;   // line-load role: rows prow, prow + 8; chunk pch
  const int ws0 = prow * 8 + (pch ^ prow), ws1 = (prow + 8) * 8 + (pch ^ prow);
  const int rs0 = lr * 8 + (lq ^ (lr & 7)), rs1 = lr * 8 + ((lq + 4) ^ (lr & 7));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  i32x4_t* region = stg + (STG ? wave * 2 * G16 * 64 : 0);
  i32x4_t* tile = wtile[wave];

  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < items; it += nwaves) {
    const int c = (int)(it / NT);
    const int n0 = (int)(it % NT) * 16;
    const int g = chunk_group(tab, G, c);
    const int r0 = a.offsets[g] + (c - tab.prefix[g]) * 16;
    const int rend = min(r0 + 16, a.offsets[g + 1]);
    const bool shared = g == a.E;
    const int64_t mat = (int64_t)I * H;
    const uint8_t* w2 = shared ? static_cast<const uint8_t*>(a.sw2) : static_cast<const uint8_t*>(a.w2) + g * mat;
    const uint8_t* b0 = w2 + (int64_t)(n0 + prow) * I + 16 * pch;
    const uint8_t* b1 = b0 + (int64_t)8 * I;
    const uint8_t* bs = nullptr;
    if (!PT) {
      const uint8_t* sm = reinterpret_cast<const uint8_t*>(shared ? a.ss2 : a.s2);
      bs = sm + ((shared ? 0 : (int64_t)g * H) + n0 + lr) * IM;
    }
    const int ra = min(r0 + lr, rend - 1);
    const uint8_t* ap = hq + (int64_t)ra * I + 16 * lq;
    const uint8_t* as = PT ? nullptr : hs + (int64_t)ra * IM;
    if (STG) {
      stage_row<G16>(region, 0, bs, KB, lq);
      stage_row<G16>(region, 1, as, KB, lq);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    i32x8_t av[D];
    i32x4_t sb0[D], sb1[D];
    int sav[D], sbv[D];
    auto load = [&](int s, int kb) {
      sb0[s] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(b0 + 128 * kb));
      sb1[s] = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(b1 + 128 * kb));
      av[s] = ld_frag(ap + 128 * kb);
      if (!STG) {
        sav[s] = PT ? 127 : scale_byte(as, kb, lq);
        sbv[s] = PT ? 127 : scale_byte(bs, kb, lq);
      }
    };
    auto consume = [&](int s, int kb) {
      tile[ws0] = sb0[s];
      tile[ws1] = sb1[s];
      const i32x4_t lo = tile[rs0], hi = tile[rs1];
      const i32x8_t bf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (STG) {
        sav[s] = staged_byte<G16>(region, 1, kb, lr, lq);
        sbv[s] = staged_byte<G16>(region, 0, kb, lr, lq);
      }
      acc = mfma_mx(av[s], bf, acc, sav[s], sbv[s]);
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, s);
    int kb0 = 0;
    for (; kb0 < KB - D; kb0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        consume(s, kb0 + s);
        load(s, kb0 + s + D);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) consume(s, kb0 + s);
    const float ysc = PT ? reinterpret_cast<const float*>(hs)[0] * (shared ? a.ss2[0] : a.s2[g]) : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + lq * 4 + i;
      if (r < rend) {
        const float v = PT ? acc[i] * ysc : acc[i];
        if (YBF16)
          static_cast<uint16_t*>(y)[(int64_t)r * H + n0 + lr] = (uint16_t)f32_to_bf16(v);
        else
          static_cast<float*>(y)[(int64_t)r * H + n0 + lr] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm13_mx_stream(const GemmArgs& a, const uint8_t* xq, const uint8_t* xs, uint8_t* hq,
                                   uint8_t* hs, hipStream_t s) {
  // staged weight scales when K is whole 512-value groups and fits the LDS copy;
  // otherwise scale bytes from global memory, one K block in flight (registers)
  if (a.H % 512 == 0 && a.H / 128 <= kStgKB13)
    gemm13_mx_stream<0, 1, 2><<<device_cus() * 8, 64 * kWaves13, 0, s>>>(a, xq, xs, hq, hs);
  else
    gemm13_mx_stream<0, 0, 1><<<device_cus() * 8, 64 * kWaves13, 0, s>>>(a, xq, xs, hq, hs);
  return hipGetLastError();
}

hipError_t launch_gemm13_pt_stream(const GemmArgs& a, const uint8_t* xq, const float* xs, float* h, float* hamax,
                                   hipStream_t s) {
  // two workgroups per CU, as many as the MX kernel's LDS copy allows: the
  // per-tensor kernel could hold three, but ran 0.444 ms at the decode shape
  // with two against 0.455 with three and 0.485 with a grid of eight per CU
  gemm13_mx_stream<1, 0, 2><<<device_cus() * 2, 64 * kWaves13, 0, s>>>(a, xq, reinterpret_cast<const uint8_t*>(xs), h,
                                                                  reinterpret_cast<uint8_t*>(hamax));
  return hipGetLastError();
}

template <int PT, int YBF16, int STG>
static void launch_down(const GemmArgs& a, const uint8_t* hq, const uint8_t* hs, void* y, hipStream_t s) {
  const int grid = device_cus() * 8;
  const int KB = a.I / 128;
  if (KB % 4 == 0)
    gemm2_mx_stream<PT, YBF16, STG, 4><<<grid, 256, 0, s>>>(a, hq, hs, y);
  else if (KB % 2 == 0)
    gemm2_mx_stream<PT, YBF16, STG, 2><<<grid, 256, 0, s>>>(a, hq, hs, y);
  else
    gemm2_mx_stream<PT, YBF16, STG, 1><<<grid, 256, 0, s>>>(a, hq, hs, y);
}

hipError_t launch_gemm2_mx_stream(const GemmArgs& a, const uint8_t* hq, const uint8_t* hs, void* y, int y_dtype,
                                  int pt, hipStream_t s) {
  const bool stg = a.I % 512 == 0 && a.I / 128 <= kStgKB2;
  if (pt) {
    if (y_dtype == 1) launch_down<1, 1, 0>(a, hq, hs, y, s);
    else launch_down<1, 0, 0>(a, hq, hs, y, s);
  } else if (stg) {
    if (y_dtype == 1) launch_down<0, 1, 1>(a, hq, hs, y, s);
    else launch_down<0, 0, 1>(a, hq, hs, y, s);
  } else {
    if (y_dtype == 1) launch_down<0, 1, 0>(a, hq, hs, y, s);
    else launch_down<0, 0, 0>(a, hq, hs, y, s);
  }
  return hipGetLastError();
}

}  // namespace moe355
