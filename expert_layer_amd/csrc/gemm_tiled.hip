// Grouped expert GEMMs for large groups (prefill-shaped batches): LDS-tiled
// bf16 MFMA kernels, fp32 accumulation.
//
// FusedMoE stages 2-3 (Gate-Up with SwiGLU) and 4 (Down) of the HPC-Ops page
// (main functions / technical principles): the Gate-Up A rows are gathered
// straight from x through the routing index (no gathered copy), the same
// waves load and compute (no warp specialisation) and latency is hidden by a
// multi-stage LDS ring instead.
//
// Tile: up to 256 or 288 rows of one group x 256 weight rows (Gate-Up: 128 gate +
// 128 up columns of h; Down: 256 columns of y), 64 k per stage, so every row
// of a stage is one whole 128-byte line (one L2 request per line; measured
// faster than a deeper ring of half-line stages), a ring of 2 stages in LDS
// (128 or 136 KB, one workgroup per CU).  Stages are filled with the gfx950
// direct-to-LDS 16-byte loads: each load instruction writes 1 KB of LDS (8
// rows x 128 B) and every lane picks the global address whose 16 bytes belong
// at its LDS slot, which realises the XOR swizzle that keeps MFMA fragment
// reads free of bank conflicts.
//
// Eight waves, two per SIMD, in a 2 (rows) x 4 (weight rows) grid: wave w
// computes rows TM/2*(w/4) .. +TM/2-1 against 64 weight rows (Gate-Up: gate
// columns 32*(w%4) .. +31 and the matching up columns).  Waves are dealt to
// SIMDs round robin, so waves w and w+4 share a SIMD and a weight slice: a
// tile of up to 128 rows still keeps every SIMD's matrix core busy, and
// 16-row fragments past the tile's valid rows are skipped.  A group with r
// rows is cut into full TM-row tiles and a remainder tile.
//
// Items (m-tile, n-tile) are ordered group by group (the Down kernel takes
// the shared expert's group first), inside a group in bands of 4 m-tiles with
// the m-tile fastest; a persistent grid of one workgroup per CU strides over
// them, and the physical workgroup -> worker mapping keeps consecutive
// workers on the same XCD (workgroups are dealt to the 8 XCDs round robin),
// so m-tiles that share a weight tile share that XCD's L2.  Where groups span two or more row tiles, the workgroups of one
// XCD also meet at a counter in the caller's workspace after every round of
// Gate-Up items, so the items that share a weight tile start together and
// stream the same lines through L2 at about the same time (router shape:
// 15 % faster; with one tile per group the waits cost more than they save).
// The wait is bounded, so the barrier only ever affects timing, never results.
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kTN = 256;      // weight rows per tile
constexpr int kTK = 64;       // k per stage (one 128-byte line per row)
constexpr int kStages = 2;    // LDS ring depth
constexpr int kThreads = 512;  // 8 waves, two per SIMD
constexpr int kRowSlots = kTK * 2 / 16;  // 16-byte slots per row per stage (8)
constexpr int kWaitVm0 = 0xF70;          // s_waitcnt vmcnt(0) only (expcnt, lgkmcnt not waited)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void load_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

// XOR swizzle of the 16-byte slot of (row, chunk) inside a 128-byte row: a
// permutation of the 8 slots for rows 0..7 and for rows 8..15, and rows of
// either parity map to distinct slots, so a 16-lane fragment read touches 16
// distinct 16-byte bank groups.  Only bits 0-3 are used, so every 16-row
// fragment shares the per-lane slot offsets.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct TileTable {
  int prefix[kMaxGroups + 1];  // m-tiles in groups < g
  int wsum[16];
};

// Tile t of a group of `cnt` rows: full TM-row tiles, then the remainder
// (fragments past the valid rows are skipped, and so are the A loads of
// 8-row groups past them, so a short remainder costs little matrix-core time
// and load bandwidth; its weight tile is read again, from the L2 of the XCD
// that runs the group's full tiles next to it).
template <int TM>
__device__ __forceinline__ void tile_rows(int cnt, int t, int& start, int& rows) {
  start = t * TM;
  rows = min(TM, cnt - start);
}

constexpr int kSyncSpins = 1 << 14;   // bounded round barrier: ~1 ms at most

__global__ void clear_sync(int* sync) {
  if (threadIdx.x < 8) sync[threadIdx.x] = 0;
}

// MODE 0: Gate-Up (+SwiGLU, h bf16); MODE 1: Down (y).  MF: 16-row fragments
// per wave, so a tile holds TM = 32 * MF rows (8: 256, 9: 288).
template <int MODE, int YBF16, int MF>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled(GemmArgs a, const uint16_t* __restrict__ A,
                                                          void* __restrict__ out, int* __restrict__ sync) {
  constexpr int TM = 32 * MF;
  constexpr int NQ = TM / 8;              // 8-row load groups of the A tile
  constexpr int NA = (NQ + 7) / 8;        // A loads per wave and stage: groups wave, wave + 8, ...
  // one named array per ring stage: the stage being read and the stages being
  // filled are then provably distinct objects, so reads wait only for their own stage
  __shared__ __attribute__((aligned(1024))) i32x4_t a0[TM * kRowSlots], a1[TM * kRowSlots];
  __shared__ __attribute__((aligned(1024))) i32x4_t b0[kTN * kRowSlots], b1[kTN * kRowSlots];
  __shared__ ChunkTable tab;

  const int G = a.E + (a.has_shared ? 1 : 0);
  const int nmt_total = MODE == 1 ? build_chunks_sf(tab, a.offsets, G, a.E, a.has_shared, TM)
                                   : build_chunks(tab, a.offsets, G, TM);
  const int H = a.H, I = a.I;
  const int K = MODE == 0 ? H : I;            // reduction length
  const int NT = MODE == 0 ? (2 * I) / kTN : H / kTN;
  const int64_t items = (int64_t)nmt_total * NT;
  const int64_t P = a.T * a.k;
  const int nk = K / kTK;

  // the wave index feeds the LDS destination of the direct loads (M0), so make it provably uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  // direct-to-LDS role: load i (0..3) of this wave fills rows 8*(4*wave+i) + lane/8,
  // slot lane%8 (which holds chunk slot ^ swz(row))
  const int lrow = lane >> 3, lslot = lane & 7;

  // XCD-aware worker id: workgroup b runs on XCD b % 8
  const int nblk = gridDim.x;
  const int per_xcd = nblk / 8;
  const int b = blockIdx.x;
  const int worker = (nblk % 8 == 0) ? (b % 8) * per_xcd + b / 8 : b;

  // round barrier per XCD (sync: 8 zeroed counters, or NULL for none)
  __shared__ int sync_on;
  if (threadIdx.x == 0) sync_on = (sync != nullptr && nblk % 8 == 0) ? 1 : 0;
  const int64_t rounds = (items + nblk - 1) / nblk;
  for (int64_t rnd = 0; rnd < rounds; ++rnd) {
   const int64_t it = worker + rnd * nblk;
   if (it < items) {
    // ---- item -> (group, n-tile, m-tile); items of group g start at prefix[g] * NT
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
    int rs, nrows;
    tile_rows<TM>(cnt, mt, rs, nrows);
    const int r0 = a.offsets[g] + rs;
    const int nmf = (nrows + 15) >> 4;   // valid 16-row fragments
    const bool shared = g == a.E;

    // ---- per-lane global addresses for the direct-to-LDS loads (element offsets)
    int a_off[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = 8 * min(wave + 8 * i, NQ - 1) + lrow;
      const int r = r0 + min(row, nrows - 1);
      int64_t base;
      if (MODE == 0) {
        const int64_t t = r < P ? (int64_t)(a.slot_pair[r] / a.k) : (int64_t)r - P;
        base = t * H;
      } else {
        base = (int64_t)r * I;
      }
      a_off[i] = (int)base + ((lslot ^ swz(row)) * 8);
    }
    const uint16_t* bw;   // weight rows of this wave's loads
    int b_off[4];
    if (MODE == 0) {
      const int half = wave >> 2;  // waves 0-3 load gate rows, waves 4-7 up rows
      const uint16_t* wm = half == 0 ? static_cast<const uint16_t*>(shared ? a.sw1 : a.w1)
                                     : static_cast<const uint16_t*>(shared ? a.sw3 : a.w3);
      bw = wm + (shared ? 0 : (int64_t)g * I * H) + (int64_t)(nt * (kTN / 2)) * H;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * wave + i) + lrow;      // 0..255 in the B tile
        const int wrow = row - half * (kTN / 2);        // 0..127 inside gate or up
        b_off[i] = wrow * H + ((lslot ^ swz(row)) * 8);
      }
    } else {
      const uint16_t* wm = static_cast<const uint16_t*>(shared ? a.sw2 : a.w2);
      bw = wm + (shared ? 0 : (int64_t)g * H * I) + (int64_t)(nt * kTN) * I;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * wave + i) + lrow;
        b_off[i] = row * I + ((lslot ^ swz(row)) * 8);
      }
    }

    // A loads of 8-row groups wholly past the valid rows are skipped (their
    // LDS rows only feed accumulator rows that are never stored)
    const int nq_live = min(NQ, (nrows + 7) / 8);
    // Down: the column tiles of one row tile (which run side by side on an
    // XCD and share its h rows) start their K loop 0-3 stages apart, so they
    // do not all ask L2 for the same lines at once (3-4 % on the Down time;
    // no gain for Gate-Up).  Only the order of the fp32 k sums changes.
    const int rot = MODE == 1 ? (nt & 3) % nk : 0;
    auto issue = [&](int kk, i32x4_t* la, i32x4_t* lb) {
      const int kr = kk + rot;
      const int k0 = (kr >= nk ? kr - nk : kr) * kTK;
#pragma unroll
      for (int i = 0; i < NA; ++i)
        if (wave + 8 * i < nq_live) load_lds16(A + a_off[i] + k0, &la[(wave + 8 * i) * 64]);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_lds16(bw + b_off[i] + k0, &lb[(4 * wave + i) * 64]);
    };

    f32x4_t acc[MF][4];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int mfw = min(MF, max(0, nmf - MF * wm));  // valid fragments of this wave

    // fragments past the valid rows are skipped in halves of 4 (64 rows)
    // per-lane LDS bases: fragment f / m then sits at a compile-time offset
    const int off0 = lr * kRowSlots + (lq ^ swz(lr));        // k 0..31 of the stage
    const int off1 = lr * kRowSlots + ((lq ^ swz(lr)) ^ 4);  // k 32..63
    const int brow0 = MODE == 0 ? 32 * wn : 64 * wn;   // first B fragment row of this wave
    auto compute = [&](const i32x4_t* la, const i32x4_t* lb) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x4_t* pa = la + 16 * MF * wm * kRowSlots + (j ? off1 : off0);
        const i32x4_t* pb = lb + brow0 * kRowSlots + (j ? off1 : off0);
        bf16x8_t bfr[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int fr = MODE == 0 ? (f < 2 ? 16 * f : kTN / 2 + 16 * (f - 2)) : 16 * f;  // relative to brow0
          bfr[f] = __builtin_bit_cast(bf16x8_t, pb[fr * kRowSlots]);
        }
        // A fragments in pairs, software-pipelined: the next pair's LDS reads
        // are in flight while the current pair's 8 MFMAs run (pairs past the
        // valid fragments are read, harmlessly, but not computed)
        constexpr int NP = (MF + 1) / 2;
        auto read_pair = [&](int g, bf16x8_t* af) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            af[u] = __builtin_bit_cast(bf16x8_t, pa[16 * min(2 * g + u, MF - 1) * kRowSlots]);
        };
        bf16x8_t acur[2], anxt[2];
        read_pair(0, acur);
#pragma unroll
        for (int g = 0; g < NP; ++g) {
          if (g + 1 < NP) read_pair(g + 1, anxt);
          if (2 * g < mfw) {
            // raised wave priority while this wave issues its MFMAs (1-2 %)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int u = 0; u < 2; ++u)
              if (2 * g + u < MF)
#pragma unroll
                for (int f = 0; f < 4; ++f) acc[2 * g + u][f] = mfma16(acur[u], bfr[f], acc[2 * g + u][f]);
            __builtin_amdgcn_s_setprio(0);
          }
          acur[0] = anxt[0];
          acur[1] = anxt[1];
        }
      }
    };

    // one stage: wait for this stage's loads (the only ones in flight), barrier,
    // refill the other slot with the next stage, compute.  The waits are the
    // compiler's s_waitcnt builtin rather than inline asm: its own wait
    // insertion then knows that the loads and the previous item's stores are
    // done, and adds no full drain of its own in front of the fragment reads.
    auto stage = [&](bool refill, int kk, const i32x4_t* la, const i32x4_t* lb, i32x4_t* fa, i32x4_t* fb) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      // execution barrier only: a fence here would also wait for the stage still
      // in flight; the wait above already put this stage's bytes in LDS
      __builtin_amdgcn_s_barrier();
      if (refill) issue(kk + 1, fa, fb);
      compute(la, lb);
    };

    // previous item's stores retired (stores also count in vmcnt) and every wave
    // finished reading the ring before it is refilled
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // nk = K / 64 is even (K % 128 == 0); the steady loop has no branches
    issue(0, a0, b0);
    for (int kk = 0; kk < nk - kStages; kk += kStages) {
      stage(true, kk + 0, a0, b0, a1, b1);
      stage(true, kk + 1, a1, b1, a0, b0);
    }
    stage(true, nk - 2, a0, b0, a1, b1);
    stage(false, nk - 1, a1, b1, a0, b0);

    // ---- epilogue
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      if (m < mfw) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * MF * wm + 16 * m + 4 * lq + i;
          if (row < nrows) {
            const int64_t r = r0 + row;
            if (MODE == 0) {
              uint16_t* h = static_cast<uint16_t*>(out);
              const int col = nt * (kTN / 2) + 32 * wn + lr;
              h[r * I + col] = (uint16_t)f32_to_bf16(silu_mul(acc[m][0][i], acc[m][2][i]));
              h[r * I + col + 16] = (uint16_t)f32_to_bf16(silu_mul(acc[m][1][i], acc[m][3][i]));
            } else {
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
}

}  // namespace

// Tiled kernels need the weight-row tile to divide the output width:
// Gate-Up 2*I % 256 == 0 (I % 128 == 0 always holds), Down H % 256 == 0.
bool tiled_gemm13_ok(const GemmArgs& a) { return (2 * a.I) % kTN == 0 && tiled_offsets_ok(a); }
bool tiled_gemm2_ok(const GemmArgs& a) { return a.H % kTN == 0 && tiled_offsets_ok(a); }

// Tile height: 288 rows when groups average 224 to 288 rows, so that a
// typical group fits one tile and streams each weight tile once instead of
// twice; else 256 (larger groups need two tiles at either height, and the
// taller tile then only costs).
static bool tall_tiles(const GemmArgs& a) {
  const int64_t P = a.T * a.k;
  return P > (int64_t)a.E * 224 && P <= (int64_t)a.E * 288;
}

hipError_t launch_gemm13_tiled(const GemmArgs& a, const uint16_t* x, uint16_t* h, int* sync, hipStream_t s) {
  const bool tall = tall_tiles(a);
  int* rb = round_barrier(a, tall ? 288 : 256) ? sync : nullptr;
  if (rb) clear_sync<<<1, 64, 0, s>>>(rb);
  if (tall)
    gemm_tiled<0, 0, 9><<<device_cus(), kThreads, 0, s>>>(a, x, h, rb);
  else
    gemm_tiled<0, 0, 8><<<device_cus(), kThreads, 0, s>>>(a, x, h, rb);
  return hipGetLastError();
}

hipError_t launch_gemm2_tiled(const GemmArgs& a, const uint16_t* h, void* y, int y_dtype, hipStream_t s) {
  const bool tall = tall_tiles(a);
  if (y_dtype == 1) {
    if (tall)
      gemm_tiled<1, 1, 9><<<device_cus(), kThreads, 0, s>>>(a, h, y, nullptr);
    else
      gemm_tiled<1, 1, 8><<<device_cus(), kThreads, 0, s>>>(a, h, y, nullptr);
  } else {
    if (tall)
      gemm_tiled<1, 0, 9><<<device_cus(), kThreads, 0, s>>>(a, h, y, nullptr);
    else
      gemm_tiled<1, 0, 8><<<device_cus(), kThreads, 0, s>>>(a, h, y, nullptr);
  }
  return hipGetLastError();
}

}  // namespace moe355
