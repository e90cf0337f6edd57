// Stage 1b, align: per-expert histogram in LDS, exclusive prefix sum and a
// contiguous slot interval per expert (HPC-Ops page, technical principles:
// the FusedMoE routing stage counts per expert with shared-memory block
// statistics and reserves a contiguous output range for every expert).
//
// The slot order inside an expert is the pair order p = t*k + j (so tokens
// ascend), which makes the result unique and bit-reproducible.  LDS atomics
// only count; positions come from ordered prefix sums:
//   * the pairs are cut into chunks of kChunk, one workgroup per chunk, and
//     each chunk into kWaves contiguous segments of equal length (whole
//     64-pair steps), one wave per segment;
//   * count:   per (chunk, expert) totals            -> ws[B][E]
//   * scan:    one workgroup turns ws into per-chunk bases (exclusive over
//              chunks) and writes counts / offsets (exclusive over experts)
//   * scatter: per chunk, per wave and expert an exclusive prefix over waves,
//              then each wave walks its segment 64 pairs at a time and ranks
//              a pair among equal experts of lower lanes with wave ballots.
// With a single chunk all three phases run in one workgroup (one launch).
#include "common.hpp"

namespace moe355 {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 8192;
constexpr int kSeg = kChunk / kWaves;  // pairs per wave segment (multiple of 64)
constexpr int kMaxE = 1024;

// Pairs per wave segment of the chunk starting at chunk0: the chunk's pairs
// split evenly over the waves in whole 64-pair steps (at most kSeg, so the
// segments never leave the chunk, and together they cover all of it).
__device__ __forceinline__ int seg_len(int64_t P, int64_t chunk0) {
  const int64_t n = min((int64_t)kChunk, P - chunk0);
  const int per = (int)((n + kWaves - 1) / kWaves);
  return min(kSeg, (per + 63) & ~63);
}

// wcnt[w][e] (LDS) := number of pairs of expert e in wave w's segment.
__device__ void count_segments(const int32_t* __restrict__ ids, int64_t P, int64_t chunk0, int E,
                               int* wcnt) {
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = seg_len(P, chunk0);
  const int64_t seg0 = chunk0 + (int64_t)wave * seg;
  for (int i = lane; i < seg; i += 64) {
    const int64_t p = seg0 + i;
    if (p < P) atomicAdd(&wcnt[wave * E + ids[p]], 1);
  }
  __syncthreads();
}

// Turn wcnt into absolute slot bases: wcnt[w][e] = base[e] + sum_{w'<w} count.
__device__ void prefix_over_waves(int* wcnt, const int* base, int E) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int run = base[e];
    for (int w = 0; w < kWaves; ++w) {
      const int c = wcnt[w * E + e];
      wcnt[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
}

__device__ void scatter_segments(const int32_t* __restrict__ ids, int64_t P, int64_t chunk0, int E,
                                 int* wcnt, int32_t* __restrict__ slot_pair,
                                 int32_t* __restrict__ pair_slot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bits = id_bits(E);
  const int seg = seg_len(P, chunk0);
  const int64_t seg0 = chunk0 + (int64_t)wave * seg;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* mine = wcnt + wave * E;
  for (int i = 0; i < seg; i += 64) {
    const int64_t p = seg0 + i + lane;
    if (seg0 + i >= P) break;  // wave-uniform
    const bool valid = p < P;
    const int e = valid ? ids[p] : E;
    const uint64_t peers = match_lanes(e, bits);
    const int rank = __popcll(peers & lt);
    int base = 0;
    if (valid) base = mine[e];
    if (valid) {
      const int s = base + rank;
      slot_pair[s] = (int32_t)p;
      pair_slot[p] = s;
    }
    // the lowest lane of each group advances that expert's running base
    if (valid && rank == 0) mine[e] = base + __popcll(peers);
  }
}

// Exclusive scan of cnt[0..E) (LDS) into out[0..E]; out[E] receives the total.
// Each thread sums a contiguous run of experts, waves scan with shuffles and
// the eight wave totals are scanned by one thread.
__device__ void block_exclusive_scan(const int* cnt, int* out, int E, int* wsum) {
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = threadIdx.x * per;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int local = 0;
  for (int e = e0; e < e0 + per && e < E; ++e) local += cnt[e];
  int v = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wsum[w];
      wsum[w] = run;
      run += c;
    }
    out[E] = run;
  }
  __syncthreads();
  int run = v - local + wsum[wave];
  for (int e = e0; e < e0 + per && e < E; ++e) {
    out[e] = run;
    run += cnt[e];
  }
  __syncthreads();
}

// Whole align in one workgroup (P <= kChunk).
__global__ __launch_bounds__(kThreads) void align_single(const int32_t* __restrict__ ids, int64_t T,
                                                         int E, int k, int shared,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ slot_pair,
                                                         int32_t* __restrict__ pair_slot) {
  __shared__ int wcnt[kWaves * kMaxE];
  __shared__ int tot[kMaxE + 1];
  __shared__ int base[kMaxE + 1];
  __shared__ int tmp[kWaves];
  const int64_t P = T * k;
  count_segments(ids, P, 0, E, wcnt);
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int c = 0;
    for (int w = 0; w < kWaves; ++w) c += wcnt[w * E + e];
    tot[e] = c;
    counts[e] = c;
  }
  __syncthreads();
  block_exclusive_scan(tot, base, E, tmp);
  for (int e = threadIdx.x; e <= E; e += kThreads) offsets[e] = base[e];
  if (threadIdx.x == 0) offsets[E + 1] = (int32_t)(P + (shared ? T : 0));
  prefix_over_waves(wcnt, base, E);
  scatter_segments(ids, P, 0, E, wcnt, slot_pair, pair_slot);
}

__global__ __launch_bounds__(kThreads) void align_count(const int32_t* __restrict__ ids, int64_t P, int E,
                                                        int32_t* __restrict__ ws) {
  __shared__ int cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += kThreads) {
    const int64_t p = c0 + i;
    if (p < P) atomicAdd(&cnt[ids[p]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) ws[(int64_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(kThreads) void align_scan(int32_t* __restrict__ ws, int nblocks, int64_t T,
                                                       int E, int k, int shared,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int tot[kMaxE + 1];
  __shared__ int base[kMaxE + 1];
  __shared__ int tmp[kWaves];
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int run = 0;
    for (int b = 0; b < nblocks; ++b) {
      const int c = ws[(int64_t)b * E + e];
      ws[(int64_t)b * E + e] = run;
      run += c;
    }
    tot[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  block_exclusive_scan(tot, base, E, tmp);
  const int64_t P = T * k;
  for (int e = threadIdx.x; e <= E; e += kThreads) offsets[e] = base[e];
  if (threadIdx.x == 0) offsets[E + 1] = (int32_t)(P + (shared ? T : 0));
}

__global__ __launch_bounds__(kThreads) void align_scatter(const int32_t* __restrict__ ids, int64_t P, int E,
                                                          const int32_t* __restrict__ ws,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ slot_pair,
                                                          int32_t* __restrict__ pair_slot) {
  __shared__ int wcnt[kWaves * kMaxE];
  __shared__ int base[kMaxE];
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  for (int e = threadIdx.x; e < E; e += kThreads) base[e] = offsets[e] + ws[(int64_t)blockIdx.x * E + e];
  count_segments(ids, P, c0, E, wcnt);  // contains the barrier that publishes base
  prefix_over_waves(wcnt, base, E);
  scatter_segments(ids, P, c0, E, wcnt, slot_pair, pair_slot);
}

}  // namespace

int align_blocks(int64_t P) { return (int)((P + kChunk - 1) / kChunk); }

hipError_t launch_align(const int32_t* ids, int64_t T, int E, int k, int shared, int32_t* counts,
                        int32_t* offsets, int32_t* slot_pair, int32_t* pair_slot, int32_t* ws,
                        hipStream_t s) {
  const int64_t P = T * k;
  const int nb = align_blocks(P);
  if (nb <= 1) {
    align_single<<<1, kThreads, 0, s>>>(ids, T, E, k, shared, counts, offsets, slot_pair, pair_slot);
    return hipGetLastError();
  }
  align_count<<<nb, kThreads, 0, s>>>(ids, P, E, ws);
  align_scan<<<1, kThreads, 0, s>>>(ws, nb, T, E, k, shared, counts, offsets);
  align_scatter<<<nb, kThreads, 0, s>>>(ids, P, E, ws, offsets, slot_pair, pair_slot);
  return hipGetLastError();
}

}  // namespace moe355
