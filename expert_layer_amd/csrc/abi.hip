// C ABI of libmoe355: host-side validation and dispatch.  Every entry point
// checks all of its arguments before it enqueues anything, so a refused call
// launches nothing; none of the checks touches the device.
#include <cstring>
#include <mutex>

#include "moe355.h"
#include "common.hpp"

namespace moe355 {

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moe355

using namespace moe355;

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 31;  // slot indices are int32
constexpr size_t kGemmWsBytes = 256;              // Gate-Up round-barrier counters (8 used)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int device_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EDEVICE; }

size_t round_up(size_t n) { return (n + 255) & ~(size_t)255; }

int check_route_shape(int64_t T, int E, int k) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return MOE_EINVAL;
  if (E > 1024 || k > 32) return MOE_EUNSUPPORTED;
  if (T * k >= kMaxRows) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_experts(const moe_experts_t* ex) {
  if (ex == nullptr) return MOE_EINVAL;
  if (ex->wtype != MOE_W_BF16 && ex->wtype != MOE_W_FP8 && ex->wtype != MOE_W_MXFP8 &&
      ex->wtype != MOE_W_FP8_TENSOR)
    return MOE_EUNSUPPORTED;
  if (ex->E <= 0 || ex->H <= 0 || ex->I <= 0) return MOE_EINVAL;
  if (ex->has_shared != 0 && ex->has_shared != 1) return MOE_EINVAL;
  if (ex->E > 1024 || ex->H % 128 != 0 || ex->I % 128 != 0) return MOE_EUNSUPPORTED;
  if (!ex->w1 || !ex->w3 || !ex->w2) return MOE_EINVAL;
  if (!aligned16(ex->w1) || !aligned16(ex->w3) || !aligned16(ex->w2)) return MOE_EINVAL;
  const bool scaled = ex->wtype != MOE_W_BF16;
  if (scaled && (!ex->s1 || !ex->s3 || !ex->s2)) return MOE_EINVAL;
  // the MXFP8 and per-tensor Down kernels tile 256 output columns, and read
  // their scales as 4-byte words
  auto a4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  const bool tiled8 =ex->wtype == MOE_W_MXFP8 || ex->wtype == MOE_W_FP8_TENSOR;
  if (tiled8 && ex->H % 256 != 0) return MOE_EUNSUPPORTED;
  if (tiled8 && (!a4(ex->s1) || !a4(ex->s3) || !a4(ex->s2))) return MOE_EINVAL;
  if (ex->has_shared) {
    if (!ex->sw1 || !ex->sw3 || !ex->sw2) return MOE_EINVAL;
    if (!aligned16(ex->sw1) || !aligned16(ex->sw3) || !aligned16(ex->sw2)) return MOE_EINVAL;
    if (scaled && (!ex->ss1 || !ex->ss3 || !ex->ss2)) return MOE_EINVAL;
    if (tiled8 && (!a4(ex->ss1) || !a4(ex->ss3) || !a4(ex->ss2))) return MOE_EINVAL;
  }
  return MOE_OK;
}

int check_rows(const moe_experts_t* ex, int64_t T, int k) {
  int st = check_route_shape(T, ex->E, k);
  if (st != MOE_OK) return st;
  if (T * k + (int64_t)ex->has_shared * T >= kMaxRows) return MOE_EUNSUPPORTED;
  // the MXFP8 and per-tensor GEMMs exist only as tiled kernels, whose 32-bit
  // row offsets bound x and h (the other weight types fall back to the
  // weight-streaming kernels instead)
  if (ex->wtype == MOE_W_MXFP8 || ex->wtype == MOE_W_FP8_TENSOR) {
    GemmArgs a{};
    a.T = T;
    a.k = k;
    a.H = ex->H;
    a.I = ex->I;
    a.has_shared = ex->has_shared;
    if (!tiled_offsets_ok(a)) return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

GemmArgs gemm_args(const moe_experts_t* ex, int64_t T, int k, const int32_t* offsets, const int32_t* slot_pair) {
  GemmArgs a;
  a.w1 = ex->w1; a.w3 = ex->w3; a.w2 = ex->w2;
  a.sw1 = ex->sw1; a.sw3 = ex->sw3; a.sw2 = ex->sw2;
  // fp32 128x128 block scales (MOE_W_FP8), E8M0 bytes (MOE_W_MXFP8) or one
  // fp32 per matrix (MOE_W_FP8_TENSOR); each kernel family reads them in its
  // own format
  a.s1 = static_cast<const float*>(ex->s1); a.s3 = static_cast<const float*>(ex->s3);
  a.s2 = static_cast<const float*>(ex->s2);
  a.ss1 = static_cast<const float*>(ex->ss1); a.ss3 = static_cast<const float*>(ex->ss3);
  a.ss2 = static_cast<const float*>(ex->ss2);
  a.E = ex->E; a.H = ex->H; a.I = ex->I; a.has_shared = ex->has_shared; a.k = k;
  a.T = T;
  a.offsets = offsets;
  a.slot_pair = slot_pair;
  return a;
}

// A persistent chain only completes when every workgroup of its grid is
// resident at once (its waves wait on items that other waves of the same grid
// hold).  Two chains running side by side on one device could each get only
// part of the device and then wait until their waits expire, so the library
// orders its own chains per device: each call's stream waits for the previous
// call's completion event before the chain is enqueued.  Inside a stream
// capture the graph's own ordering applies instead (events from outside a
// capture cannot be waited on there).
constexpr int kMaxDevices = 64;
struct ChainOrder {
  std::mutex m;
  hipEvent_t last[kMaxDevices] = {};
};
ChainOrder& chain_order() {
  static ChainOrder o;
  return o;
}

}  // namespace

#define MOE_GUARD_BEGIN try {
#define MOE_GUARD_END \
  }                   \
  catch (...) {       \
    return MOE_EDEVICE; \
  }

extern "C" {

int moe_abi_version(void) { return MOE355_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or dtype";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EDEVICE: return "device error";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------ router
int moe_router_split(const float* w, uint16_t* w_hi, uint16_t* w_lo, int E, int H, void* stream) {
  MOE_GUARD_BEGIN
  if (E < 0 || H < 0) return MOE_EINVAL;
  const int64_t n = (int64_t)E * H;
  if (n == 0) return MOE_OK;
  if (!w || !w_hi || !w_lo) return MOE_EINVAL;
  if (overlap(w_hi, n * 2, w_lo, n * 2) || overlap(w, n * 4, w_hi, n * 2) || overlap(w, n * 4, w_lo, n * 2))
    return MOE_EINVAL;
  return device_status(launch_router_split(w, w_hi, w_lo, n, (hipStream_t)stream));
  MOE_GUARD_END
}

int moe_router_gemm(const uint16_t* x, const uint16_t* w_hi, const uint16_t* w_lo, float* logits, int64_t T,
                    int H, int E, void* stream) {
  MOE_GUARD_BEGIN
  if (T < 0 || H <= 0 || E <= 0) return MOE_EINVAL;
  if (H % 128 != 0 || E > 1024) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_hi || !w_lo || !logits) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w_hi) || !aligned16(w_lo)) return MOE_EINVAL;
  if (overlap(logits, (size_t)T * E * 4, x, (size_t)T * H * 2)) return MOE_EINVAL;
  return device_status(launch_router_gemm(x, w_hi, w_lo, logits, T, H, E, (hipStream_t)stream));
  MOE_GUARD_END
}

// ------------------------------------------------------------------ route
int moe_route(const float* logits, const float* bias, const uint8_t* bias_rows, int64_t T, int E, int k,
              int32_t* topk_ids, float* topk_w, void* stream) {
  MOE_GUARD_BEGIN
  int st = check_route_shape(T, E, k);
  if (st != MOE_OK) return st;
  if (bias_rows != nullptr && bias == nullptr) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_EINVAL;
  if (overlap(topk_ids, (size_t)T * k * 4, topk_w, (size_t)T * k * 4)) return MOE_EINVAL;
  return device_status(launch_route(logits, bias, bias_rows, T, E, k, topk_ids, topk_w, (hipStream_t)stream));
  MOE_GUARD_END
}

// ------------------------------------------------------------------ align
size_t moe_align_workspace_bytes(int64_t T, int E, int k) {
  if (T <= 0 || E <= 0 || k <= 0) return 0;
  const int nb = align_blocks(T * k);
  return nb <= 1 ? 0 : (size_t)nb * E * sizeof(int32_t);
}

int moe_align(const int32_t* topk_ids, int64_t T, int E, int k, int shared, int32_t* counts, int32_t* offsets,
              int32_t* slot_pair, int32_t* pair_slot, void* ws, size_t ws_bytes, void* stream) {
  MOE_GUARD_BEGIN
  int st = check_route_shape(T, E, k);
  if (st != MOE_OK) return st;
  if (shared != 0 && shared != 1) return MOE_EINVAL;
  if (T * k + shared * T >= kMaxRows) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !slot_pair || !pair_slot) return MOE_EINVAL;
  const size_t P4 = (size_t)T * k * 4;
  const void* outs[4] = {counts, offsets, slot_pair, pair_slot};
  const size_t sz[4] = {(size_t)E * 4, (size_t)(E + 2) * 4, P4, P4};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], sz[i], topk_ids, P4)) return MOE_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], sz[i], outs[j], sz[j])) return MOE_EINVAL;
  }
  const size_t need = moe_align_workspace_bytes(T, E, k);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return MOE_EWORKSPACE;
  return device_status(launch_align(topk_ids, T, E, k, shared, counts, offsets, slot_pair, pair_slot,
                                    static_cast<int32_t*>(ws), (hipStream_t)stream));
  MOE_GUARD_END
}

// ------------------------------------------------------------------ fp8 helpers
int moe_quant_rows_fp8(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s, void* stream) {
  MOE_GUARD_BEGIN
  if (rows < 0 || cols <= 0) return MOE_EINVAL;
  if (cols % 128 != 0) return MOE_EUNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !s) return MOE_EINVAL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u)) return MOE_EINVAL;
  if (overlap(q, (size_t)rows * cols, s, (size_t)rows * (cols / 128) * 4)) return MOE_EINVAL;
  return device_status(launch_quant_rows(x, rows, cols, q, s, (hipStream_t)stream));
  MOE_GUARD_END
}

int moe_quant_rows_mxfp8(const uint16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* s, void* stream) {
  MOE_GUARD_BEGIN
  if (rows < 0 || cols <= 0) return MOE_EINVAL;
  if (cols % 32 != 0) return MOE_EUNSUPPORTED;
  if (rows * (cols / 32) >= kMaxRows) return MOE_EUNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !s) return MOE_EINVAL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u)) return MOE_EINVAL;
  if (overlap(q, (size_t)rows * cols, s, (size_t)rows * (cols / 32)) ||
      overlap(x, (size_t)rows * cols * 2, q, (size_t)rows * cols) ||
      overlap(x, (size_t)rows * cols * 2, s, (size_t)rows * (cols / 32)))
    return MOE_EINVAL;
  return device_status(launch_quant_rows_mx(x, rows, cols, q, s, (hipStream_t)stream));
  MOE_GUARD_END
}

int moe_quant_blocks_fp8(const uint16_t* w, int64_t mats, int rows, int cols, uint8_t* q, float* s,
                         void* stream) {
  MOE_GUARD_BEGIN
  if (mats < 0 || rows <= 0 || cols <= 0) return MOE_EINVAL;
  if (rows % 128 != 0 || cols % 128 != 0) return MOE_EUNSUPPORTED;
  if (mats == 0) return MOE_OK;
  if (!w || !q || !s) return MOE_EINVAL;
  if (!aligned16(w) || (reinterpret_cast<uintptr_t>(q) & 7u)) return MOE_EINVAL;
  if (mats * (rows / 128) * (cols / 128) >= kMaxRows) return MOE_EUNSUPPORTED;
  return device_status(launch_quant_blocks(w, mats, rows, cols, q, s, (hipStream_t)stream));
  MOE_GUARD_END
}

namespace {
int check_tensors(const void* x, int dtype, int64_t mats, int64_t n) {
  if (mats < 0 || n < 0) return MOE_EINVAL;
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return MOE_EUNSUPPORTED;
  if (n % 128 != 0 || mats > 65535 || mats * n >= (int64_t)1 << 40) return MOE_EUNSUPPORTED;
  if (mats == 0 || n == 0) return MOE_OK;
  if (!x || !aligned16(x)) return MOE_EINVAL;
  return MOE_OK;
}
size_t elem_bytes(int dtype) { return dtype == MOE_DTYPE_F32 ? 4 : 2; }
}  // namespace

int moe_tensor_amax(const void* x, int dtype, int64_t mats, int64_t n, float* amax, void* stream) {
  MOE_GUARD_BEGIN
  const int st = check_tensors(x, dtype, mats, n);
  if (st != MOE_OK || mats == 0 || n == 0) return st;
  if (!amax || (reinterpret_cast<uintptr_t>(amax) & 3u)) return MOE_EINVAL;
  if (overlap(amax, (size_t)mats * 4, x, (size_t)(mats * n) * elem_bytes(dtype))) return MOE_EINVAL;
  return device_status(launch_tensor_amax(x, dtype == MOE_DTYPE_F32, mats, n, amax, (hipStream_t)stream));
  MOE_GUARD_END
}

int moe_quant_tensor_fp8(const void* x, int dtype, int64_t mats, int64_t n, const float* amax, uint8_t* q, float* s,
                         void* stream) {
  MOE_GUARD_BEGIN
  const int st = check_tensors(x, dtype, mats, n);
  if (st != MOE_OK || mats == 0 || n == 0) return st;
  if (!amax || !q || !s) return MOE_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 7u) || (reinterpret_cast<uintptr_t>(s) & 3u) ||
      (reinterpret_cast<uintptr_t>(amax) & 3u))
    return MOE_EINVAL;
  const size_t xb = (size_t)(mats * n) * elem_bytes(dtype), qb = (size_t)(mats * n), sb = (size_t)mats * 4;
  if (overlap(q, qb, x, xb) || overlap(s, sb, x, xb) || overlap(s, sb, q, qb) || overlap(q, qb, amax, sb))
    return MOE_EINVAL;
  return device_status(
      launch_quant_tensor(x, dtype == MOE_DTYPE_F32, mats, n, amax, q, s, (hipStream_t)stream));
  MOE_GUARD_END
}

// ------------------------------------------------------------------ grouped GEMMs
size_t moe_gemm_workspace_bytes(const moe_experts_t* ex, int64_t T, int k) {
  (void)ex;
  (void)T;
  (void)k;
  return kGemmWsBytes;
}

int moe_gemm13(const moe_experts_t* ex, const void* x, const void* xs, const int32_t* offsets,
               const int32_t* slot_pair, int64_t T, int k, void* h, void* hs, void* ws, size_t ws_bytes,
               void* stream) {
  MOE_GUARD_BEGIN
  int st = check_experts(ex);
  if (st != MOE_OK) return st;
  st = check_rows(ex, T, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !offsets || !slot_pair || !h) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(h)) return MOE_EINVAL;
  const bool mx = ex->wtype == MOE_W_MXFP8;
  const bool pt = ex->wtype == MOE_W_FP8_TENSOR;
  const bool fp8 = ex->wtype == MOE_W_FP8 || mx || pt;
  if (fp8 && (!xs || !hs)) return MOE_EINVAL;
  if ((mx || pt) && (reinterpret_cast<uintptr_t>(xs) & 3u)) return MOE_EINVAL;   // 4-byte scale words
  if (pt && (reinterpret_cast<uintptr_t>(hs) & 3u)) return MOE_EINVAL;
  const int64_t R = T * k + ex->has_shared * T;
  // per-tensor: h is the unquantised fp32 h (its scale needs the whole tensor)
  const size_t hbytes = (size_t)R * ex->I * (pt ? 4 : fp8 ? 1 : 2);
  const size_t hsbytes = pt ? 4 : mx ? (size_t)R * (ex->I / 32) : (size_t)R * (ex->I / 128) * 4;
  if (overlap(h, hbytes, x, (size_t)T * ex->H * (fp8 ? 1 : 2))) return MOE_EINVAL;
  if (fp8 && overlap(hs, hsbytes, h, hbytes)) return MOE_EINVAL;
  if (ws == nullptr || ws_bytes < kGemmWsBytes) return MOE_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 3u) return MOE_EINVAL;
  if (overlap(ws, kGemmWsBytes, h, hbytes) || overlap(ws, kGemmWsBytes, x, (size_t)T * ex->H * (fp8 ? 1 : 2)))
    return MOE_EINVAL;
  const GemmArgs a = gemm_args(ex, T, k, offsets, slot_pair);
  hipStream_t s = (hipStream_t)stream;
  if (pt)
    return device_status(launch_gemm13_pt(a, static_cast<const uint8_t*>(x), static_cast<const float*>(xs),
                                          static_cast<float*>(h), static_cast<float*>(hs), static_cast<int*>(ws), s));
  if (mx)
    return device_status(launch_gemm13_mx(a, static_cast<const uint8_t*>(x), static_cast<const uint8_t*>(xs),
                                          static_cast<uint8_t*>(h), static_cast<uint8_t*>(hs), static_cast<int*>(ws), s));
  if (fp8)
    return device_status(launch_gemm13_fp8(a, static_cast<const uint8_t*>(x), static_cast<const float*>(xs),
                                           static_cast<uint8_t*>(h), static_cast<float*>(hs), s));
  return device_status(
      launch_gemm13_bf16(a, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(h), static_cast<int*>(ws), s));
  MOE_GUARD_END
}

int moe_gemm2(const moe_experts_t* ex, const void* h, const void* hs, const int32_t* offsets, int64_t T, int k,
              void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  MOE_GUARD_BEGIN
  (void)ws;
  (void)ws_bytes;
  int st = check_experts(ex);
  if (st != MOE_OK) return st;
  st = check_rows(ex, T, k);
  if (st != MOE_OK) return st;
  if (y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_BF16) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!h || !offsets || !y) return MOE_EINVAL;
  if (!aligned16(h) || !aligned16(y)) return MOE_EINVAL;
  const bool mx = ex->wtype == MOE_W_MXFP8;
  const bool pt = ex->wtype == MOE_W_FP8_TENSOR;
  const bool fp8 = ex->wtype == MOE_W_FP8 || mx || pt;
  if (fp8 && !hs) return MOE_EINVAL;
  if ((mx || pt) && (reinterpret_cast<uintptr_t>(hs) & 3u)) return MOE_EINVAL;   // 4-byte scale words
  const int64_t R = T * k + ex->has_shared * T;
  if (overlap(y, (size_t)R * ex->H * (y_dtype == MOE_DTYPE_F32 ? 4 : 2), h, (size_t)R * ex->I * (fp8 ? 1 : 2)))
    return MOE_EINVAL;
  const GemmArgs a = gemm_args(ex, T, k, offsets, nullptr);
  hipStream_t s = (hipStream_t)stream;
  if (pt)
    return device_status(
        launch_gemm2_pt(a, static_cast<const uint8_t*>(h), static_cast<const float*>(hs), y, y_dtype, s));
  if (mx)
    return device_status(launch_gemm2_mx(a, static_cast<const uint8_t*>(h), static_cast<const uint8_t*>(hs), y,
                                         y_dtype, s));
  if (fp8)
    return device_status(
        launch_gemm2_fp8(a, static_cast<const uint8_t*>(h), static_cast<const float*>(hs), y, y_dtype, s));
  return device_status(launch_gemm2_bf16(a, static_cast<const uint16_t*>(h), y, y_dtype, s));
  MOE_GUARD_END
}

// ------------------------------------------------------------------ combine
int moe_combine(const void* y, int y_dtype, const int32_t* pair_slot, const float* topk_w, int64_t T, int k,
                int H, int has_shared, uint16_t* out, void* stream) {
  MOE_GUARD_BEGIN
  if (T < 0 || k <= 0 || H <= 0) return MOE_EINVAL;
  if (has_shared != 0 && has_shared != 1) return MOE_EINVAL;
  if (k > 32 || H % 128 != 0) return MOE_EUNSUPPORTED;
  if (y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_BF16) return MOE_EUNSUPPORTED;
  if (T * k + has_shared * T >= kMaxRows) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y || !pair_slot || !topk_w || !out) return MOE_EINVAL;
  if (!aligned16(y) || !aligned16(out)) return MOE_EINVAL;
  const int64_t R = T * k + has_shared * T;
  if (overlap(out, (size_t)T * H * 2, y, (size_t)R * H * (y_dtype == MOE_DTYPE_F32 ? 4 : 2))) return MOE_EINVAL;
  return device_status(launch_combine(y, y_dtype, pair_slot, topk_w, T, k, H, has_shared, out, (hipStream_t)stream));
  MOE_GUARD_END
}

int moe_combine_rmsnorm(const void* y, int y_dtype, const int32_t* pair_slot, const float* topk_w, int64_t T,
                        int k, int H, int has_shared, const uint16_t* residual, const uint16_t* weight, float eps,
                        uint16_t* out, uint16_t* res_out, void* stream) {
  MOE_GUARD_BEGIN
  if (T < 0 || k <= 0 || H <= 0) return MOE_EINVAL;
  if (has_shared != 0 && has_shared != 1) return MOE_EINVAL;
  if (!(eps >= 0.0f) || !(eps < 3.0e38f)) return MOE_EINVAL;   // finite, >= 0 (NaN fails)
  if (k > 32 || H % 128 != 0 || H > 32768) return MOE_EUNSUPPORTED;
  if (y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_BF16) return MOE_EUNSUPPORTED;
  if (T * k + has_shared * T >= kMaxRows) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y || !pair_slot || !topk_w || !residual || !weight || !out) return MOE_EINVAL;
  if (!aligned16(y) || !aligned16(out) || !aligned16(residual) || !aligned16(weight)) return MOE_EINVAL;
  if (res_out && !aligned16(res_out)) return MOE_EINVAL;
  const int64_t R = T * k + has_shared * T;
  const size_t rowb = (size_t)T * H * 2;
  const size_t yb = (size_t)R * H * (y_dtype == MOE_DTYPE_F32 ? 4 : 2);
  if (overlap(out, rowb, y, yb) || overlap(out, rowb, residual, rowb) || overlap(out, rowb, weight, (size_t)H * 2))
    return MOE_EINVAL;
  if (res_out) {
    if (overlap(res_out, rowb, out, rowb) || overlap(res_out, rowb, y, yb) || overlap(res_out, rowb, weight, (size_t)H * 2))
      return MOE_EINVAL;
    if (res_out != residual && overlap(res_out, rowb, residual, rowb)) return MOE_EINVAL;   // in place or disjoint
  }
  return device_status(launch_combine_rmsnorm(y, y_dtype, pair_slot, topk_w, T, k, H, has_shared, residual, weight,
                                              eps, out, res_out, (hipStream_t)stream));
  MOE_GUARD_END
}

// ------------------------------------------------------------------ whole chain
namespace {

struct FwdLayout {
  size_t ctl, logits, ids, w, counts, offsets, slot_pair, pair_slot, align_ws, gemm_ws, xq, xs, h, hq, hs, y, total;
};

FwdLayout forward_layout(const moe_experts_t* ex, int64_t T, int k, int y_dtype, bool router) {
  FwdLayout L;
  const int64_t P = T * k, R = P + ex->has_shared * T;
  const bool mx = ex->wtype == MOE_W_MXFP8;
  const bool pt = ex->wtype == MOE_W_FP8_TENSOR;
  const bool fp8 = ex->wtype == MOE_W_FP8 || mx || pt;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t at = off;
    off += round_up(n);
    return at;
  };
  // control words of the persistent chain first, so that
  // moe_forward_persistent_status finds them at offset 0
  L.ctl = take((size_t)chain_ctl_ints(ex->E, ex->has_shared, T, k) * 4);
  L.logits = take(router ? (size_t)T * ex->E * 4 : 0);
  L.ids = take((size_t)P * 4);
  L.w = take((size_t)P * 4);
  L.counts = take((size_t)ex->E * 4);
  L.offsets = take((size_t)(ex->E + 2) * 4);
  L.slot_pair = take((size_t)P * 4);
  L.pair_slot = take((size_t)P * 4);
  L.align_ws = take(moe_align_workspace_bytes(T, ex->E, k));
  L.gemm_ws = take(kGemmWsBytes);
  L.xq = take(fp8 ? (size_t)T * ex->H : 0);
  // per-tensor: xs / hs hold {amax, scale}; h is fp32, the codes go to hq
  L.xs = take(pt ? 8 : mx ? (size_t)T * (ex->H / 32) : fp8 ? (size_t)T * (ex->H / 128) * 4 : 0);
  L.h = take((size_t)R * ex->I * (pt ? 4 : fp8 ? 1 : 2));
  L.hq = take(pt ? (size_t)R * ex->I : 0);
  L.hs = take(pt ? 8 : mx ? (size_t)R * (ex->I / 32) : fp8 ? (size_t)R * (ex->I / 128) * 4 : 0);
  L.y = take((size_t)R * ex->H * (y_dtype == MOE_DTYPE_F32 ? 4 : 2));
  L.total = off;
  return L;
}

}  // namespace

size_t moe_forward_workspace_bytes(const moe_experts_t* ex, int64_t T, int k, int y_dtype) {
  if (check_experts(ex) != MOE_OK || check_rows(ex, T, k) != MOE_OK) return 0;
  return forward_layout(ex, T, k, y_dtype, true).total;
}

}  // extern "C"

namespace {

// Argument checks shared by moe_forward, moe_forward_persistent and
// moe_forward_noalloc.  On MOE_OK with T > 0, *L is the workspace layout.
// With fixed_scratch the workspace is the library's own scratch array (ws is
// ignored): the layout must fit in MOE_NOALLOC_SCRATCH_BYTES, else
// MOE_EUNSUPPORTED.
int check_forward(const moe_experts_t* ex, const moe_forward_args_t* args, void* ws, size_t ws_bytes, FwdLayout* L,
                  bool* empty, bool fixed_scratch = false) {
  *empty = false;
  if (!args) return MOE_EINVAL;
  int st = check_experts(ex);
  if (st != MOE_OK) return st;
  const int64_t T = args->T;
  const int k = args->k;
  st = check_rows(ex, T, k);
  if (st != MOE_OK) return st;
  if (args->y_dtype != MOE_DTYPE_F32 && args->y_dtype != MOE_DTYPE_BF16) return MOE_EUNSUPPORTED;
  const bool router = args->logits == nullptr;
  if (router && (!args->router_hi || !args->router_lo)) return MOE_EINVAL;
  if (args->bias_rows && !args->bias) return MOE_EINVAL;
  if (T == 0) {
    *empty = true;
    return MOE_OK;
  }
  if (!args->x || !args->out) return MOE_EINVAL;
  if (!aligned16(args->x) || !aligned16(args->out)) return MOE_EINVAL;
  if (router && (!aligned16(args->router_hi) || !aligned16(args->router_lo))) return MOE_EINVAL;
  // the workspace always has room for the logits, matching moe_forward_workspace_bytes
  *L = forward_layout(ex, T, k, args->y_dtype, true);
  if (fixed_scratch) return L->total <= MOE_NOALLOC_SCRATCH_BYTES ? MOE_OK : MOE_EUNSUPPORTED;
  if (ws == nullptr || ws_bytes < L->total) return MOE_EWORKSPACE;
  if (overlap(ws, L->total, args->out, (size_t)T * ex->H * 2) || overlap(ws, L->total, args->x, (size_t)T * ex->H * 2))
    return MOE_EINVAL;
  return MOE_OK;
}

// Enqueue the whole chain with its intermediates laid out at `base` (already validated).
int forward_enqueue(const moe_experts_t* ex, const moe_forward_args_t* args, char* base, const FwdLayout& L,
                    hipStream_t s) {
  const int64_t T = args->T;
  const int k = args->k;
  const bool router = args->logits == nullptr;
  const int E = ex->E;
  const bool mx = ex->wtype == MOE_W_MXFP8;
  const bool pt = ex->wtype == MOE_W_FP8_TENSOR;
  const bool fp8 = ex->wtype == MOE_W_FP8;
  float* logits = router ? reinterpret_cast<float*>(base + L.logits) : nullptr;
  int32_t* ids = args->topk_ids ? args->topk_ids : reinterpret_cast<int32_t*>(base + L.ids);
  float* w = args->topk_w ? args->topk_w : reinterpret_cast<float*>(base + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* slot_pair = reinterpret_cast<int32_t*>(base + L.slot_pair);
  int32_t* pair_slot = reinterpret_cast<int32_t*>(base + L.pair_slot);
  int32_t* align_ws = reinterpret_cast<int32_t*>(base + L.align_ws);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + L.xq);
  float* xs = reinterpret_cast<float*>(base + L.xs);
  void* h = base + L.h;
  float* hs = reinterpret_cast<float*>(base + L.hs);
  void* y = base + L.y;

  hipError_t e;
  if (router) {
    e = launch_router_gemm(args->x, args->router_hi, args->router_lo, logits, T, ex->H, E, s);
    if (e != hipSuccess) return MOE_EDEVICE;
  }
  e = launch_route(router ? logits : args->logits, args->bias, args->bias_rows, T, E, k, ids, w, s);
  if (e != hipSuccess) return MOE_EDEVICE;
  e = launch_align(ids, T, E, k, ex->has_shared, counts, offsets, slot_pair, pair_slot, align_ws, s);
  if (e != hipSuccess) return MOE_EDEVICE;
  const GemmArgs a = gemm_args(ex, T, k, offsets, slot_pair);
  if (pt) {
    // x: amax, then codes with one scale; Gate-Up: fp32 h and its amax; h:
    // codes with one scale; Down
    float* xsw = reinterpret_cast<float*>(base + L.xs);   // {amax, scale}
    float* hsw = reinterpret_cast<float*>(base + L.hs);
    uint8_t* hq = reinterpret_cast<uint8_t*>(base + L.hq);
    const int64_t R = T * k + ex->has_shared * T;
    e = launch_tensor_amax(args->x, 0, 1, T * ex->H, xsw, s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_quant_tensor(args->x, 0, 1, T * ex->H, xsw, xq, xsw + 1, s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_gemm13_pt(a, xq, xsw + 1, static_cast<float*>(h), hsw, reinterpret_cast<int*>(base + L.gemm_ws), s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_quant_tensor(h, 1, 1, R * ex->I, hsw, hq, hsw + 1, s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_gemm2_pt(a, hq, hsw + 1, y, args->y_dtype, s);
  } else if (mx) {
    uint8_t* xsm = reinterpret_cast<uint8_t*>(base + L.xs);
    uint8_t* hsm = reinterpret_cast<uint8_t*>(base + L.hs);
    e = launch_quant_rows_mx(args->x, T, ex->H, xq, xsm, s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_gemm13_mx(a, xq, xsm, static_cast<uint8_t*>(h), hsm, reinterpret_cast<int*>(base + L.gemm_ws), s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_gemm2_mx(a, static_cast<const uint8_t*>(h), hsm, y, args->y_dtype, s);
  } else if (fp8) {
    e = launch_quant_rows(args->x, T, ex->H, xq, xs, s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_gemm13_fp8(a, xq, xs, static_cast<uint8_t*>(h), hs, s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_gemm2_fp8(a, static_cast<const uint8_t*>(h), hs, y, args->y_dtype, s);
  } else {
    e = launch_gemm13_bf16(a, args->x, static_cast<uint16_t*>(h), reinterpret_cast<int*>(base + L.gemm_ws), s);
    if (e != hipSuccess) return MOE_EDEVICE;
    e = launch_gemm2_bf16(a, static_cast<const uint16_t*>(h), y, args->y_dtype, s);
  }
  if (e != hipSuccess) return MOE_EDEVICE;
  e = launch_combine(y, args->y_dtype, pair_slot, w, T, k, ex->H, ex->has_shared, args->out, s);
  return device_status(e);
}

// Device scratch of moe_forward_noalloc: the chain's intermediates for callers
// that cannot allocate.  Each device the library runs on holds its own copy
// until the process ends.  In host code this name is only a handle for
// hipGetSymbolAddress; kernels get the device address scratch_address returns.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

struct ScratchAddrs {
  std::mutex m;
  void* ptr[kMaxDevices] = {};
};

// Device address of `scratch` on device dev, looked up once per device with
// that device current; nullptr if the lookup fails.
void* scratch_address(int dev) {
  static ScratchAddrs addrs;
  std::lock_guard<std::mutex> lock(addrs.m);
  if (addrs.ptr[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess) return nullptr;
    addrs.ptr[dev] = p;
  }
  return addrs.ptr[dev];
}

}  // namespace

extern "C" {

int moe_forward(const moe_experts_t* ex, const moe_forward_args_t* args, void* ws, size_t ws_bytes, void* stream) {
  MOE_GUARD_BEGIN
  FwdLayout L;
  bool empty;
  const int st = check_forward(ex, args, ws, ws_bytes, &L, &empty);
  if (st != MOE_OK || empty) return st;
  return forward_enqueue(ex, args, static_cast<char*>(ws), L, (hipStream_t)stream);
  MOE_GUARD_END
}

int moe_forward_noalloc(const moe_experts_t* ex, const moe_forward_args_t* args, void* stream) {
  MOE_GUARD_BEGIN
  FwdLayout L;
  bool empty;
  const int st = check_forward(ex, args, nullptr, 0, &L, &empty, true);
  if (st != MOE_OK || empty) return st;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  void* base = scratch_address(dev);
  if (base == nullptr) return MOE_EDEVICE;
  return forward_enqueue(ex, args, static_cast<char*>(base), L, s);
  MOE_GUARD_END
}

int moe_forward_persistent(const moe_experts_t* ex, const moe_forward_args_t* args, void* ws, size_t ws_bytes,
                           void* stream) {
  MOE_GUARD_BEGIN
  FwdLayout L;
  bool empty;
  int st = check_forward(ex, args, ws, ws_bytes, &L, &empty);
  if (st != MOE_OK || empty) return st;
  const int64_t T = args->T;
  const int k = args->k;
  if (ex->wtype != MOE_W_BF16) return MOE_EUNSUPPORTED;
  char* base = static_cast<char*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* slot_pair = reinterpret_cast<int32_t*>(base + L.slot_pair);
  const GemmArgs a = gemm_args(ex, T, k, offsets, slot_pair);
  if (!chain_supported(a)) return MOE_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const bool router = args->logits == nullptr;
  float* logits = router ? reinterpret_cast<float*>(base + L.logits) : nullptr;
  if (router) {
    const hipError_t e = launch_router_gemm(args->x, args->router_hi, args->router_lo, logits, T, ex->H, ex->E, s);
    if (e != hipSuccess) return MOE_EDEVICE;
  }
  // (the router GEMM above is an ordinary kernel; only the chain needs the device to itself)
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return MOE_EDEVICE;
  int dev = 0;
  if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  ChainOrder& order = chain_order();
  std::lock_guard<std::mutex> lock(order.m);
  const bool ordered = cap == hipStreamCaptureStatusNone;
  if (ordered) {
    if (order.last[dev] == nullptr &&
        hipEventCreateWithFlags(&order.last[dev], hipEventDisableTiming) != hipSuccess) {
      order.last[dev] = nullptr;
      return MOE_EDEVICE;
    }
    if (hipStreamWaitEvent(s, order.last[dev], 0) != hipSuccess) return MOE_EDEVICE;
  }
  ChainBuffers b;
  b.logits = router ? logits : args->logits;
  b.bias = args->bias;
  b.bias_rows = args->bias_rows;
  b.x = args->x;
  b.ids = args->topk_ids ? args->topk_ids : reinterpret_cast<int32_t*>(base + L.ids);
  b.w = args->topk_w ? args->topk_w : reinterpret_cast<float*>(base + L.w);
  b.counts = reinterpret_cast<int32_t*>(base + L.counts);
  b.offsets = offsets;
  b.slot_pair = slot_pair;
  b.pair_slot = reinterpret_cast<int32_t*>(base + L.pair_slot);
  b.h = reinterpret_cast<uint16_t*>(base + L.h);
  b.y = base + L.y;
  b.y_dtype = args->y_dtype;
  b.out = args->out;
  b.ctl = reinterpret_cast<int*>(base + L.ctl);
  const hipError_t e = launch_chain(a, b, s);
  if (e != hipSuccess) return MOE_EDEVICE;
  if (ordered && hipEventRecord(order.last[dev], s) != hipSuccess) return MOE_EDEVICE;
  return MOE_OK;
  MOE_GUARD_END
}

int moe_forward_persistent_status(const void* ws, void* stream) {
  MOE_GUARD_BEGIN
  if (ws == nullptr) return MOE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  int words[kChainCtlInts];
  if (hipMemcpyAsync(words, ws, sizeof(words), hipMemcpyDeviceToHost, s) != hipSuccess) return MOE_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_EDEVICE;
  return words[3] != 0 ? MOE_EDEVICE : MOE_OK;
  MOE_GUARD_END
}

}  // extern "C"
