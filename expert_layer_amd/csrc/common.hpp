// Device helpers and internal launcher declarations for libmoe355 (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe355 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 values -> two OCP E4M3FN codes (RNE, saturated to +-448) packed in
// the low 16 bits.  The hardware conversion rounds to nearest even; the clamp
// makes the saturation explicit.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// MXFP8 (OCP Microscaling): shared exponent of a 32-value block whose largest
// magnitude is amax: floor(log2(amax)) - 8, clamped to [-127, 127]; -127 for
// an all-zero block.  Stored as the E8M0 byte X + 127.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  frexpf(amax, &e);   // amax = m * 2^e, 0.5 <= m < 1
  return min(127, max(-127, e - 9));
}

// v * 2^n, exact unless the result leaves the normal range (v_ldexp_f32)
__device__ __forceinline__ float ldexp_f32(float v, int n) { return __builtin_amdgcn_ldexpf(v, n); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max16(float v) {
  // max over the 16 lanes that share (lane / 16)
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}

// Lanes of this wave whose value equals mine, for values in [0, 2^bits).
__device__ __forceinline__ uint64_t match_lanes(int v, int bits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < bits; ++b) {
    const bool set = (v >> b) & 1;
    const uint64_t bal = __ballot(set);
    m &= set ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ int id_bits(int E) {
  int bits = 1;
  while ((1 << bits) < E + 1) ++bits;  // room for the sentinel value E
  return bits;
}

// ------------------------------------------------------------------ launchers
// All launchers enqueue on `s` and return hipGetLastError().  Shapes have been
// validated by the ABI layer.
hipError_t launch_route(const float* logits, const float* bias, const uint8_t* bias_rows, int64_t T,
                        int E, int k, int32_t* ids, float* w, hipStream_t s);

int align_blocks(int64_t P);
hipError_t launch_align(const int32_t* ids, int64_t T, int E, int k, int shared, int32_t* counts,
                        int32_t* offsets, int32_t* slot_pair, int32_t* pair_slot, int32_t* ws,
                        hipStream_t s);

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* sc,
                             hipStream_t s);
hipError_t launch_quant_blocks(const uint16_t* w, int64_t mats, int rows, int cols, uint8_t* q,
                               float* sc, hipStream_t s);
hipError_t launch_quant_rows_mx(const uint16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* sc,
                                hipStream_t s);
// per-tensor FP8: amax[m] = max |x| of tensor m (mats tensors of n values,
// bf16 or fp32 when f32), then s[m] = amax/448 (1 if 0) and q = e4m3(x / s[m])
hipError_t launch_tensor_amax(const void* x, int f32, int64_t mats, int64_t n, float* amax, hipStream_t s);
hipError_t launch_quant_tensor(const void* x, int f32, int64_t mats, int64_t n, const float* amax, uint8_t* q,
                               float* sc, hipStream_t s);

hipError_t launch_combine_rmsnorm(const void* y, int y_dtype, const int32_t* pair_slot, const float* w, int64_t T,
                                  int k, int H, int has_shared, const uint16_t* residual, const uint16_t* weight,
                                  float eps, uint16_t* out, uint16_t* res_out, hipStream_t s);

hipError_t launch_router_split(const float* w, uint16_t* hi, uint16_t* lo, int64_t n, hipStream_t s);
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* hi, const uint16_t* lo, float* logits,
                              int64_t T, int H, int E, hipStream_t s);

struct GemmArgs {
  // expert weights (routed [E,...] and shared)
  const void *w1, *w3, *w2, *sw1, *sw3, *sw2;
  const float *s1, *s3, *s2, *ss1, *ss3, *ss2;
  int E, H, I, has_shared, k;
  int64_t T;
  const int32_t* offsets;    // [E+2]
  const int32_t* slot_pair;  // [P]
};

// The LDS-tiled kernels address the rows they gather (x for Gate-Up, h for
// Down) and the rows of a 256-row weight tile with 32-bit element offsets.
// Shapes past that range go to the weight-streaming kernels (64-bit
// addressing) or, for the weight types that only have tiled kernels, are
// refused.
inline bool tiled_offsets_ok(const GemmArgs& a) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t R = a.T * a.k + (a.has_shared ? a.T : 0);
  return a.T * a.H < lim && R * a.I < lim && (int64_t)256 * a.H < lim && (int64_t)256 * a.I < lim;
}

// sync: 8 ints of device scratch for the tiled kernel's round barrier
hipError_t launch_gemm13_bf16(const GemmArgs& a, const uint16_t* x, uint16_t* h, int* sync, hipStream_t s);
hipError_t launch_gemm2_bf16(const GemmArgs& a, const uint16_t* h, void* y, int y_dtype, hipStream_t s);
hipError_t launch_gemm13_fp8(const GemmArgs& a, const uint8_t* xq, const float* xs, uint8_t* hq,
                             float* hs, hipStream_t s);
hipError_t launch_gemm2_fp8(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, int y_dtype,
                            hipStream_t s);

bool tiled_gemm13_ok(const GemmArgs& a);
bool tiled_gemm2_ok(const GemmArgs& a);
hipError_t launch_gemm13_tiled(const GemmArgs& a, const uint16_t* x, uint16_t* h, int* sync, hipStream_t s);
hipError_t launch_gemm2_tiled(const GemmArgs& a, const uint16_t* h, void* y, int y_dtype, hipStream_t s);

// MXFP8 (E8M0 bytes per 32 K): xs [T, H/32], hs [R, I/32]; weight scales in
// GemmArgs s1/s3/s2 (and the shared ones) point to bytes [rows, K/32]
hipError_t launch_gemm13_mx(const GemmArgs& a, const uint8_t* xq, const uint8_t* xs, uint8_t* hq, uint8_t* hs,
                            int* sync, hipStream_t s);
hipError_t launch_gemm2_mx(const GemmArgs& a, const uint8_t* hq, const uint8_t* hs, void* y, int y_dtype,
                           hipStream_t s);
// per-tensor FP8 (same tiles): weight scales s1/s3/s2 [E] and ss1/ss3/ss2 [1]
// fp32; xs, hs [1]; the Gate-Up writes fp32 h [R, I] and hamax = max |h|
hipError_t launch_gemm13_pt(const GemmArgs& a, const uint8_t* xq, const float* xs, float* h, float* hamax,
                            int* sync, hipStream_t s);
hipError_t launch_gemm2_pt(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, int y_dtype,
                           hipStream_t s);

// weight-streaming MXFP8 / per-tensor kernels for small groups (pt: per-tensor
// Down, hs then holds the fp32 h scale)
hipError_t launch_gemm13_mx_stream(const GemmArgs& a, const uint8_t* xq, const uint8_t* xs, uint8_t* hq,
                                   uint8_t* hs, hipStream_t s);
hipError_t launch_gemm13_pt_stream(const GemmArgs& a, const uint8_t* xq, const float* xs, float* h, float* hamax,
                                   hipStream_t s);
hipError_t launch_gemm2_mx_stream(const GemmArgs& a, const uint8_t* hq, const uint8_t* hs, void* y, int y_dtype,
                                  int pt, hipStream_t s);

bool tiled_fp8_gemm13_ok(const GemmArgs& a);
bool tiled_fp8_gemm2_ok(const GemmArgs& a);
hipError_t launch_gemm13_fp8_tiled(const GemmArgs& a, const uint8_t* xq, const float* xs, uint8_t* hq, float* hs,
                                   hipStream_t s);
hipError_t launch_gemm2_fp8_tiled(const GemmArgs& a, const uint8_t* hq, const float* hs, void* y, int y_dtype,
                                  hipStream_t s);

// Persistent chain (route .. combine in one launch, device-side ready flags).
// ctl: control area of chain_ctl_ints() ints, owned by the caller.
constexpr int kChainCtlInts = 16;
struct ChainBuffers {
  const float* logits;
  const float* bias;
  const uint8_t* bias_rows;
  const uint16_t* x;
  int32_t *ids, *counts, *offsets, *slot_pair, *pair_slot;
  float* w;
  uint16_t* h;
  void* y;
  int y_dtype;
  uint16_t* out;
  int* ctl;
};
int64_t chain_max_chunks(int E, int has_shared, int64_t T, int k);
inline int64_t chain_ctl_ints(int E, int has_shared, int64_t T, int k) {
  return kChainCtlInts + 6 * chain_max_chunks(E, has_shared, T, k) + E + 2;
}
bool chain_supported(const GemmArgs& a);
hipError_t launch_chain(const GemmArgs& a, const ChainBuffers& b, hipStream_t s);

hipError_t launch_combine(const void* y, int y_dtype, const int32_t* pair_slot, const float* w, int64_t T,
                          int k, int H, int has_shared, uint16_t* out, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cus();

}  // namespace moe355
