// Persistent chain: one launch runs the whole FusedMoE layer step (route,
// align, Gate-Up + SwiGLU, Down, combine) with device-side ready flags
// between the stages instead of kernel boundaries.
//
// The HPC-Ops page chains its five FusedMoE stages with Programmatic
// Dependent Launch so that a stage starts while the previous one drains
// (main functions: FusedMoE; technical principles: PDL removes the launch
// bubbles).  HIP has no dependent launch, so the stages become phases of one
// persistent kernel and each dependency becomes a counter in device memory.
// Phases, in order (W waves, wave w):
//
//   route     tokens w, w+W, ...                              -> route_done += 1
//   align     wave T % W: wait route_done == T, stable counting sort and the
//             chunk list (16-row chunks of each group)       -> align_done = chunks + 1
//   Gate-Up   every wave: wait align_done; then its contiguous block of the
//             (chunk, 16-column) items                       -> done13[c] += items run
//   Down      its block of (chunk, 16-column) items; the first weight stages
//             are requested before waiting for done13[c] == I/16
//                                                            -> done2[c] += items run
//   combine   its block of (token, 512-column) items, after done2 == H/16 for
//             the token's k (+1 shared) chunks
//
// Every wave runs its items in this global order and every item waits only
// for items earlier in it.  The grid is sized so that all of its workgroups
// are resident at once; then the wave holding the earliest unfinished item is
// running that item and never waits for anything unfinished, so the chain
// completes.  Waits are bounded in wall-clock time: on expiry the wave sets
// the error word, and every wave that waits after that stops.
//
// Visibility without cache flushes: everything a wave produces for another
// wave (routing ids and weights, the align outputs, h, y) is written with
// agent-scope atomic stores (sc1: written through to the device coherence
// point), the producer waits for its stores to complete (s_waitcnt vmcnt(0))
// and then bumps the counter with an agent-scope atomic.  Consumers poll with
// agent-scope atomic loads and read indices (slot_pair, ids, pair_slot,
// chunk entries) with agent-scope atomic loads too.  h and y are read with
// ordinary cached loads: no wave reads a line of h or y before the item that
// writes it has been published, and the caches hold no line of them from
// before the launch (kernel start invalidates them), so no cache can return
// a stale copy.  Agent-scope release/acquire fences would write back and
// invalidate a whole L2 per item (about 9 and 7 ns of device time each,
// serialised), which costs more than the chain saves.
//
// The arithmetic of every phase is the stand-alone kernels' (route_token,
// the streaming GEMM items, combine8), so the output is bitwise the same as
// the five-kernel chain's.  Envelope: bf16 weights and the 16-row chunking
// of the streaming kernels (T*k <= 16*E).
#include "combine8.hpp"
#include "route_token.hpp"
#include "stream_gemm.hpp"
#include "tiles.hpp"

namespace moe355 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunkRows = 16;
constexpr int kCombineCols = 512;  // columns per combine item: 64 lanes x 8
constexpr long long kSpinTicks = 1ll << 26;

// control words at the start of the control area
constexpr int kRouteDone = 1, kAlignDone = 2, kError = 3;

struct ChainParams {
  GemmArgs a;  // offsets / slot_pair point into the workspace
  const float* logits;
  const float* bias;
  const uint8_t* bias_rows;
  const uint16_t* x;
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot_pair;
  int32_t* pair_slot;
  uint16_t* h;
  void* y;
  uint16_t* out;
  int* ctl;         // kChainCtlInts control words
  int* chunk;       // [nchunks_max][4]: group, row0, row end, 0
  int* chunk_base;  // [G + 1]: first chunk of each group
  int* done13;      // [nchunks_max]
  int* done2;       // [nchunks_max]
  int max_chunks;   // nchunks_max
};

__device__ __forceinline__ int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wave-uniform word: loaded by every lane from one address, kept in a
// scalar register so that everything derived from it stays scalar too.
__device__ __forceinline__ int ld_uniform(const int* p) { return __builtin_amdgcn_readfirstlane(ld_relaxed(p)); }

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return min(max(v, lo), hi); }

// Publish this wave's earlier coherent stores: wait until they have reached
// the coherence point, then bump the counter.  The asm statement is also a
// compiler barrier, so no store moves below it.
__device__ __forceinline__ void publish_add(int* p, int lane, int n = 1) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(p, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll *p until it reaches target (wave-uniform).  false: timed out, error
// word set.  The fence after the loop is a compiler barrier only (at
// workgroup scope it emits no instruction): no later load moves above the
// poll.
__device__ bool wait_geq(const int* p, int target, int* ctl) {
  if (ld_relaxed(p) < target) {
    const long long t0 = wall_clock64();
    while (ld_relaxed(p) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > kSpinTicks || ld_relaxed(ctl + kError) != 0) {
        __hip_atomic_store(ctl + kError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return true;
}

// Every lane l < n polls its own counter p[idx] until it reaches target (one
// load per round for all of them).  false: timed out, error word set.
__device__ bool wait_all_geq(const int* p, int idx, int n, int target, int* ctl) {
  const int lane = threadIdx.x & 63;
  auto pending = [&]() { return __ballot(lane < n && ld_relaxed(p + idx) < target) != 0; };
  if (pending()) {
    const long long t0 = wall_clock64();
    while (pending()) {
      __builtin_amdgcn_s_sleep(2);
      if (wall_clock64() - t0 > kSpinTicks || ld_relaxed(ctl + kError) != 0) {
        __hip_atomic_store(ctl + kError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return true;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan(int v, int lane) {
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  return v;
}

// Stage 1b in one wave (stable counting sort, HPC-Ops page, technical
// principles: per-expert statistics in shared memory and one contiguous slot
// interval per expert), plus the chunk list the GEMM phases walk.  cnt: E
// ints of this wave's LDS.  Results are unique, so they equal moe_align's.
// Every output goes out with coherent stores; ids come in with coherent loads.
// Returns the number of chunks.
__device__ int align_wave(const ChainParams& p, int* cnt, int lane) {
  const int E = p.a.E;
  const int64_t T = p.a.T;
  const int k = p.a.k;
  const int64_t P = T * k;
  const int32_t* ids = p.ids;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  for (int64_t i = lane; i < P; i += 64) atomicAdd(&cnt[get<1>(ids + i)], 1);
  // per lane a contiguous run of experts: slot and chunk prefix sums
  const int per = (E + 63) / 64;
  const int e0 = lane * per, e1 = min(E, e0 + per);
  int rows = 0, chunks = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    rows += c;
    chunks += (c + kChunkRows - 1) / kChunkRows;
  }
  int run = wave_scan(rows, lane) - rows;
  int crun = wave_scan(chunks, lane) - chunks;
  const int routed_chunks = __shfl(crun + chunks, 63);
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    put<1>(p.counts + e, c);
    put<1>(p.offsets + e, run);
    put<1>(p.chunk_base + e, crun);
    for (int j = 0; j * kChunkRows < c; ++j) {
      int* ch = p.chunk + 4 * (crun + j);
      put<1>(ch, e);
      put<1>(ch + 1, run + j * kChunkRows);
      put<1>(ch + 2, run + min(c, (j + 1) * kChunkRows));
      put<1>(p.done13 + crun + j, 0);
      put<1>(p.done2 + crun + j, 0);
    }
    cnt[e] = run;  // running slot base for the scatter
    run += c;
    crun += (c + kChunkRows - 1) / kChunkRows;
  }
  const int shared_chunks = p.a.has_shared ? (int)((T + kChunkRows - 1) / kChunkRows) : 0;
  for (int j = lane; j < shared_chunks; j += 64) {
    int* ch = p.chunk + 4 * (routed_chunks + j);
    put<1>(ch, E);
    put<1>(ch + 1, (int)P + j * kChunkRows);
    put<1>(ch + 2, (int)(P + std::min<int64_t>(T, (int64_t)(j + 1) * kChunkRows)));
    put<1>(p.done13 + routed_chunks + j, 0);
    put<1>(p.done2 + routed_chunks + j, 0);
  }
  if (lane == 0) {
    put<1>(p.offsets + E, (int32_t)P);
    put<1>(p.offsets + E + 1, (int32_t)(P + (p.a.has_shared ? T : 0)));
    put<1>(p.chunk_base + E, routed_chunks);
    if (p.a.has_shared) put<1>(p.chunk_base + E + 1, routed_chunks + shared_chunks);
  }
  // stable scatter: a pair's rank among equal experts of lower lanes
  const int bits = id_bits(E);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int64_t i0 = 0; i0 < P; i0 += 64) {
    const int64_t q = i0 + lane;
    const bool valid = q < P;
    const int e = valid ? get<1>(ids + q) : E;
    const uint64_t peers = match_lanes(e, bits);
    const int rank = __popcll(peers & lt);
    const int base = valid ? cnt[e] : 0;
    if (valid) {
      put<1>(p.slot_pair + base + rank, (int32_t)q);
      put<1>(p.pair_slot + q, base + rank);
      if (rank == 0) cnt[e] = base + __popcll(peers);
    }
  }
  return routed_chunks + shared_chunks;
}

template <int VPL, int D13, int D2, int YBF16>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainParams p) {
  __shared__ i32x4_t tile[kWaves][2][kStreamTileSlots];  // 4 KB per wave; align scratch, combine staging
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t T = p.a.T;
  const int E = p.a.E, k = p.a.k, H = p.a.H, I = p.a.I;
  const int NT13 = I / 16, NT2 = H / 16;
  const int ncs = (H + kCombineCols - 1) / kCombineCols;
  const int R = (int)(T * k + (p.a.has_shared ? T : 0));
  const int64_t P = T * k;
  const int64_t W = (int64_t)gridDim.x * kWaves;
  const int64_t w = (int64_t)blockIdx.x * kWaves + wave;
  int* ctl = p.ctl;

  // ---- route: tokens w, w+W, ...; align: wave T % W once they are all
  // published.  align_done carries the chunk count + 1.
  for (int64_t t = w; t < T; t += W) {
    route_token<VPL, 1>(p.logits, p.bias, p.bias_rows, t, E, k, p.ids, p.w);
    publish_add(ctl + kRouteDone, lane);
  }
  if (w == T % W) {
    if (!wait_geq(ctl + kRouteDone, (int)T, ctl)) return;
    const int nch = align_wave(p, reinterpret_cast<int*>(tile[wave]), lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(ctl + kAlignDone, nch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!wait_geq(ctl + kAlignDone, 1, ctl)) return;
  const int nchunks = clampi(ld_uniform(ctl + kAlignDone) - 1, 0, p.max_chunks);

  // The GEMM and combine phases are cut into W contiguous blocks, one per
  // wave, so a wave's items mostly share one chunk: its entry, the token rows
  // and the readiness check are fetched once per chunk, and a chunk's counter
  // is bumped once per wave by the number of its items the wave ran.
  auto block = [&](int64_t n, int64_t& lo, int64_t& hi) {
    lo = n * w / W;
    hi = n * (w + 1) / W;
  };
  auto chunk = [&](int c, int& g, int& r0, int& rend) {
    g = clampi(ld_uniform(p.chunk + 4 * c), 0, E);
    r0 = clampi(ld_uniform(p.chunk + 4 * c + 1), 0, R - 1);
    rend = clampi(ld_uniform(p.chunk + 4 * c + 2), r0 + 1, R);
  };

  // ---- Gate-Up + SwiGLU
  int64_t lo, hi;
  block((int64_t)nchunks * NT13, lo, hi);
  {
    int cur = -1, g = 0, r0 = 0, rend = 1, run = 0;
    int64_t trow[1];
    for (int64_t u = lo; u < hi; ++u) {
      const int c = (int)(u / NT13);
      if (c != cur) {
        if (run) publish_add(p.done13 + cur, lane, run);
        cur = c;
        run = 0;
        chunk(c, g, r0, rend);
        gemm13_rows<1, 1>(p.a, r0, rend, trow);
      }
      gemm13_stream_item<1, D13, 1>(p.a, p.x, p.h, g, r0, rend, (int)(u % NT13) * 16, trow, tile[wave][0],
                                    tile[wave][1]);
      ++run;
    }
    if (run) publish_add(p.done13 + cur, lane, run);
  }
  if (ld_relaxed(ctl + kError) != 0) return;

  // ---- Down: the first weight stages are in flight while the chunk's h is awaited
  block((int64_t)nchunks * NT2, lo, hi);
  {
    int cur = -1, g = 0, r0 = 0, rend = 1, run = 0;
    bool ok = true;
    for (int64_t u = lo; u < hi && ok; ++u) {
      const int c = (int)(u / NT2);
      const bool fresh = c != cur;
      if (fresh) {
        if (run) publish_add(p.done2 + cur, lane, run);
        cur = c;
        run = 0;
        chunk(c, g, r0, rend);
      }
      gemm2_stream_item<1, D2, YBF16, 1>(p.a, p.h, p.y, g, r0, rend, (int)(u % NT2) * 16, tile[wave][0], [&]() {
        if (fresh) ok = wait_geq(p.done13 + c, NT13, ctl);
      });
      ++run;
    }
    if (!ok) return;  // the error word is set; nothing of this chunk is published
    if (run) publish_add(p.done2 + cur, lane, run);
  }

  // ---- combine: (token, 512 columns) items
  block(T * ncs, lo, hi);
  int32_t* slot = reinterpret_cast<int32_t*>(tile[wave][0]);
  float* wt = reinterpret_cast<float*>(tile[wave][1]);
  const int nterm = k + (p.a.has_shared ? 1 : 0);
  for (int64_t v = lo; v < hi; ++v) {
    const int64_t tok = v / ncs;
    const int col = (int)(v % ncs) * kCombineCols + lane * 8;
    // this token's chunks: routed pairs (lanes < k) and the shared row
    int myc = 0;
    if (lane < k) {
      const int s = clampi(ld_relaxed(p.pair_slot + tok * k + lane), 0, (int)P - 1);
      const int g = clampi(ld_relaxed(p.ids + tok * k + lane), 0, E - 1);
      myc = ld_relaxed(p.chunk_base + g) + (s - ld_relaxed(p.offsets + g)) / kChunkRows;
      slot[lane] = s;
      wt[lane] = __hip_atomic_load(p.w + tok * k + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (lane == k && p.a.has_shared) {
      myc = ld_relaxed(p.chunk_base + E) + (int)(tok / kChunkRows);
    }
    myc = clampi(myc, 0, p.max_chunks - 1);
    if (!wait_all_geq(p.done2, myc, nterm, NT2, ctl)) return;
    if (col < H) {
      float acc[8];
      combine8<YBF16>(p.y, slot, wt, nterm, k, P, tok, H, col, acc);
      *reinterpret_cast<uint4*>(p.out + tok * H + col) = pack_bf16x8(acc);
    }
  }
}

__global__ void chain_clear(int* ctl) {
  if (threadIdx.x < kChainCtlInts) ctl[threadIdx.x] = 0;
}

// Workgroups of one chain kernel that fit on the device at once.
template <class K>
int64_t resident_blocks(K kernel) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return (int64_t)per_cu * device_cus();
}

template <int VPL, int D13, int D2, int YBF16>
void launch_one(const ChainParams& p, int64_t items, hipStream_t s) {
  auto kernel = chain_kernel<VPL, D13, D2, YBF16>;
  static const int64_t resident = resident_blocks(kernel);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((items + kWaves - 1) / kWaves, resident));
  kernel<<<blocks, kThreads, 0, s>>>(p);
}

template <int VPL, int YBF16>
void launch_vd(const ChainParams& p, int64_t items, hipStream_t s) {
  const bool d13 = p.a.H % 256 == 0, d2 = p.a.I % 256 == 0;
  if (d13 && d2)
    launch_one<VPL, 4, 4, YBF16>(p, items, s);
  else if (d13)
    launch_one<VPL, 4, 2, YBF16>(p, items, s);
  else if (d2)
    launch_one<VPL, 2, 4, YBF16>(p, items, s);
  else
    launch_one<VPL, 2, 2, YBF16>(p, items, s);
}

}  // namespace

int64_t chain_max_chunks(int E, int has_shared, int64_t T, int k) {
  const int64_t R = T * k + (has_shared ? T : 0);
  return E + (has_shared ? 1 : 0) + (R + kChunkRows - 1) / kChunkRows;
}

bool chain_supported(const GemmArgs& a) { return small_groups(a); }

hipError_t launch_chain(const GemmArgs& a, const ChainBuffers& b, hipStream_t s) {
  ChainParams p;
  p.a = a;
  p.a.offsets = b.offsets;
  p.a.slot_pair = b.slot_pair;
  p.logits = b.logits;
  p.bias = b.bias;
  p.bias_rows = b.bias_rows;
  p.x = b.x;
  p.ids = b.ids;
  p.w = b.w;
  p.counts = b.counts;
  p.offsets = b.offsets;
  p.slot_pair = b.slot_pair;
  p.pair_slot = b.pair_slot;
  p.h = b.h;
  p.y = b.y;
  p.out = b.out;
  const int64_t nmax = chain_max_chunks(a.E, a.has_shared, a.T, a.k);
  p.ctl = b.ctl;
  p.chunk = b.ctl + kChainCtlInts;
  p.chunk_base = p.chunk + 4 * nmax;
  p.done13 = p.chunk_base + (a.E + 2);
  p.done2 = p.done13 + nmax;
  p.max_chunks = (int)nmax;
  // enough waves for every item, at most what the device holds at once
  const int64_t items = a.T + 1 + nmax * (a.I / 16 + a.H / 16) + a.T * ((a.H + kCombineCols - 1) / kCombineCols);
  chain_clear<<<1, 64, 0, s>>>(b.ctl);
  const bool ybf16 = b.y_dtype == 1;
  if (a.E <= 256) {
    if (ybf16)
      launch_vd<4, 1>(p, items, s);
    else
      launch_vd<4, 0>(p, items, s);
  } else {
    if (ybf16)
      launch_vd<16, 1>(p, items, s);
    else
      launch_vd<16, 0>(p, items, s);
  }
  return hipGetLastError();
}

}  // namespace moe355
