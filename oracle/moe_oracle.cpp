// Oracle for the fused Mixture-of-Experts layer forward -- TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, obviously-correct CPU implementation of what the GPU path
// computes.  Only the tests, the smoke check and the benchmark's CPU-baseline
// leg may load it; the product path never does.  It shares no code, header or
// table with the HIP kernels.
//
// Sources (web pages describing HPC-Ops and the Hy4-preview MoE block):
//  * "HPC-Ops - Tencent Hunyuan open-source inference operator library"
//    (bestaitool.cc), sections "Main functions" and "Technical principles":
//    FusedMoE is the five-stage chain routing index -> Gate-Up GEMM ->
//    activation quantisation -> Down GEMM -> top-k weighted combine; the
//    router GEMM emulates FP32 with a high BF16 part plus a residual BF16 part
//    scaled by 1/256, combined with one FMA.
//  * "PR #54160 report: [Hy4] support Hy4-preview model" (prhub.com.cn),
//    section "Features and motivation": 256 routed experts, top-8, plus one
//    shared expert; section "Implementation" item 4: FP8 blockwise 128x128
//    weight scales.
// Fused and unfused MoE compute the same function; the fusion only removes
// memory movement and launches.  So this file is the plain layer definition
// in double precision, with the FP8 quantisation steps emulated exactly.
//
// Readings where the pages are silent (each one listed in the design notes):
//  * gate: softmax over the k selected logits; ties broken by lower expert id;
//    ids stored in rank order (value desc, id asc); no capacity limit.
//  * shared expert: SwiGLU of the same size, added with weight 1.
//  * SwiGLU: h = SiLU(x.w1^T) * (x.w3^T), SiLU(z) = z / (1 + e^-z); w1 = gate.
//  * FP8 = OCP E4M3FN (max 448, no infinities), round to nearest even,
//    saturating.  Scale of a group/block = amax / 448 in fp32 (1 if amax = 0);
//    code = encode(fp32(v / scale)).
//  * router split: hi = bf16_rne(w), lo = bf16_rne((w - hi) * 256),
//    logits = acc_hi + acc_lo / 256.
//  * MXFP8 (the microscaling FP8 format the PR report lists beside the
//    128x128 blockwise scales): blocks of 32 consecutive values along the
//    reduction dimension share a power-of-two scale 2^X stored as an E8M0
//    byte X + 127; X = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest
//    power of two), clamped to [-127, 127]; an all-zero block uses X = -127;
//    elements are E4M3FN codes of v * 2^-X, rounded to nearest even and
//    saturated at 448.
//  * per-tensor FP8 (the second FP8 mode the HPC-Ops page lists for its
//    GroupGEMM, main functions): one fp32 scale per tensor, amax / 448 as for
//    a block (1 if amax = 0).  Each expert weight matrix is a tensor; x is one
//    tensor [T, H]; h is one tensor over all of its [R, I] values, quantised
//    from h rounded to fp32 after the whole Gate-Up is known (a per-tensor
//    scale needs the amax of the whole tensor before any code).  Products of
//    codes are summed over the whole K and scaled once by (activation scale
//    x weight scale).
//
// Parity pins for every function here live in tests/test_oracle_*.py.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

double bf16_value(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Nearest bfloat16 to a finite float, ties to the even pattern.  The two
// candidates are the float with its low 16 bits cleared (same sign, smaller or
// equal magnitude) and the next bfloat16 of larger magnitude.
uint16_t bf16_nearest(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  uint16_t down = static_cast<uint16_t>(u >> 16);
  uint16_t up = static_cast<uint16_t>(down + 1);
  double dv = v;
  double e_down = std::fabs(dv - bf16_value(down));
  double e_up = std::fabs(bf16_value(up) - dv);
  if (e_down < e_up) return down;
  if (e_up < e_down) return up;
  return (down & 1u) ? up : down;
}

// OCP 8-bit floating point, E4M3FN: bias 7, 3 mantissa bits, exponent field 0
// is subnormal (m/8 * 2^-6), pattern S.1111.111 is NaN, no infinities.
double e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

// Round a finite value to E4M3FN: nearest representable magnitude, ties to
// even mantissa, magnitudes at or above 448 saturate to 448 (0x7E).
uint8_t e4m3_code(float v) {
  double a = std::fabs(static_cast<double>(v));
  uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  if (a >= 448.0) return sign | 0x7E;
  double quantum;
  if (a < std::ldexp(1.0, -6)) {
    quantum = std::ldexp(1.0, -9);               // subnormal spacing
  } else {
    int ex;
    std::frexp(a, &ex);                           // a = f * 2^ex, f in [0.5, 1)
    quantum = std::ldexp(1.0, (ex - 1) - 3);      // 3 mantissa bits in binade 2^(ex-1)
  }
  double q = std::nearbyint(a / quantum) * quantum;  // default mode: ties to even
  if (q == 0.0) return sign;
  int ex;
  std::frexp(q, &ex);
  int eb = ex - 1;                                // q in [2^eb, 2^(eb+1))
  if (eb < -6) {                                  // subnormal
    int m = static_cast<int>(q / std::ldexp(1.0, -9));
    return sign | static_cast<uint8_t>(m);
  }
  int m = static_cast<int>(q / std::ldexp(1.0, eb) * 8.0) - 8;
  return sign | static_cast<uint8_t>(((eb + 7) << 3) | m);
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// MX shared exponent of a block with largest magnitude amax (finite, >= 0).
int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = 0;
  std::frexp(amax, &e);   // amax = m * 2^e, 0.5 <= m < 1, so floor(log2(amax)) = e - 1
  return std::min(127, std::max(-127, e - 1 - 8));
}

// One MX block of n values: scale byte and E4M3 codes of v * 2^-X.
void mx_quant_block(const float* v, int n, uint8_t* q, uint8_t* sbyte) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  const int X = mx_exponent(amax);
  *sbyte = static_cast<uint8_t>(X + 127);
  for (int i = 0; i < n; ++i) q[i] = e4m3_code(static_cast<float>(std::ldexp(static_cast<double>(v[i]), -X)));
}

template <class F>
void parallel_for(int64_t n, int nthreads, F f) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> pool;
  int64_t nt = std::min<int64_t>(nthreads, n);
  for (int64_t w = 0; w < nt; ++w)
    pool.emplace_back([=] {
      for (int64_t i = w; i < n; i += nt) f(i);
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------- codecs
double orc_bf16_value(uint16_t b) { return bf16_value(b); }
uint16_t orc_bf16_nearest(float v) { return bf16_nearest(v); }
double orc_e4m3_value(uint8_t c) { return e4m3_value(c); }
uint8_t orc_e4m3_code(float v) { return e4m3_code(v); }

void orc_e4m3_code_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_code(v[i]);
}

int orc_mx_exponent(float amax) { return mx_exponent(amax); }

// MXFP8 quantisation of rows of bf16 values (activations, or weight rows with
// K along the columns): per row, per 32 consecutive columns, one E8M0 scale
// byte s[r, c/32] and the codes q[r, c].
void orc_quant_rows_mx(const uint16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* s, int nthreads) {
  const int nb = cols / 32;
  parallel_for(rows, nthreads, [&](int64_t r) {
    float v[32];
    for (int b = 0; b < nb; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = static_cast<float>(bf16_value(x[r * cols + b * 32 + i]));
      mx_quant_block(v, 32, q + r * cols + b * 32, s + r * nb + b);
    }
  });
}

// The same rule on fp32 rows (the requantisation of h).
void orc_quant_rows_mx_f32(const float* x, int64_t rows, int cols, uint8_t* q, uint8_t* s) {
  const int nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b) mx_quant_block(x + r * cols + b * 32, 32, q + r * cols + b * 32, s + r * nb + b);
}

// ---------------------------------------------------------------- router
// HPC-Ops page, "Router GEMM" (main functions, technical principles): split an
// fp32 weight offline into a high bf16 part and a residual bf16 part scaled by
// 256 so that w ~= hi + lo / 256.
void orc_router_split(const float* w, int64_t n, uint16_t* hi, uint16_t* lo) {
  for (int64_t i = 0; i < n; ++i) {
    hi[i] = bf16_nearest(w[i]);
    float resid = w[i] - static_cast<float>(bf16_value(hi[i]));  // exact in fp32
    lo[i] = bf16_nearest(resid * 256.0f);                       // power of two: exact
  }
}

// Exact router logits in double: logits[t,e] = sum_h x[t,h] * w[e,h], with x
// bf16 and w fp32 taken at their exact values.
void orc_router_logits(const uint16_t* x, const float* w, int64_t T, int H, int E,
                       double* logits, int nthreads) {
  parallel_for(T, nthreads, [&](int64_t t) {
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h) acc += bf16_value(x[t * H + h]) * static_cast<double>(w[(int64_t)e * H + h]);
      logits[t * E + e] = acc;
    }
  });
}

// ---------------------------------------------------------------- route
// Stage 1 of FusedMoE ("routing index").  Per token: optional per-expert bias
// added in fp32 (only on rows whose bias_rows flag is set, or on every row if
// bias_rows is NULL), then the k experts with the largest biased logits,
// ordered by (value desc, id asc), and weights = softmax over those k values.
void orc_route(const float* logits, const float* bias, const uint8_t* bias_rows,
               int64_t T, int E, int k, int32_t* ids, double* weights) {
  std::vector<std::pair<float, int>> row(E);
  for (int64_t t = 0; t < T; ++t) {
    bool biased = bias != nullptr && (bias_rows == nullptr || bias_rows[t] != 0);
    for (int e = 0; e < E; ++e) {
      float l = logits[t * E + e];
      if (biased) l = l + bias[e];
      row[e] = {l, e};
    }
    std::sort(row.begin(), row.end(), [](const std::pair<float, int>& a, const std::pair<float, int>& b) {
      if (a.first != b.first) return a.first > b.first;
      return a.second < b.second;
    });
    double top = row[0].first, denom = 0.0;
    for (int j = 0; j < k; ++j) denom += std::exp(static_cast<double>(row[j].first) - top);
    for (int j = 0; j < k; ++j) {
      ids[t * k + j] = row[j].second;
      weights[t * k + j] = std::exp(static_cast<double>(row[j].first) - top) / denom;
    }
  }
}

// ---------------------------------------------------------------- align
// HPC-Ops page, "FusedMoE pipeline": per-expert counts and a contiguous output
// interval per expert.  Counting sort of the P = T*k (token, rank) pairs by
// expert, stable in pair order (hence ascending token inside each expert).
// offsets[0..E] is the exclusive prefix sum of counts; offsets[E+1] adds the
// shared expert's T rows (group E) when shared != 0.
void orc_align(const int32_t* ids, int64_t T, int E, int k, int shared, int32_t* counts,
               int32_t* offsets, int32_t* slot_pair, int32_t* pair_slot) {
  int64_t P = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) counts[ids[p]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  offsets[E + 1] = offsets[E] + (shared ? static_cast<int32_t>(T) : 0);
  std::vector<int32_t> next(offsets, offsets + E);
  for (int64_t p = 0; p < P; ++p) {
    int32_t s = next[ids[p]]++;
    slot_pair[s] = static_cast<int32_t>(p);
    pair_slot[p] = s;
  }
}

// ---------------------------------------------------------------- fp8 quant
// Activation quantisation: per row, per group of 128 columns,
// scale = amax / 448 (fp32 division), code = e4m3(fp32(x / scale)).
void orc_quant_rows_fp8(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s) {
  int groups = cols / 128;
  for (int64_t r = 0; r < rows; ++r)
    for (int g = 0; g < groups; ++g) {
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i)
        amax = std::max(amax, static_cast<float>(std::fabs(bf16_value(x[r * cols + g * 128 + i]))));
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      s[r * groups + g] = sc;
      for (int i = 0; i < 128; ++i) {
        float v = static_cast<float>(bf16_value(x[r * cols + g * 128 + i])) / sc;
        q[r * cols + g * 128 + i] = e4m3_code(v);
      }
    }
}

// Weight quantisation with 128x128 block scales (PR #54160 report,
// implementation item 4): for each matrix [rows, cols] and each 128x128 block,
// scale = amax / 448 (fp32), code = e4m3(fp32(w / scale)).  s has shape
// [mats, rows/128, cols/128].
void orc_quant_blocks_fp8(const uint16_t* w, int64_t mats, int rows, int cols, uint8_t* q, float* s,
                          int nthreads) {
  const int rb = rows / 128, cb = cols / 128;
  parallel_for(mats * rb * cb, nthreads, [&](int64_t b) {
    const int64_t m = b / ((int64_t)rb * cb);
    const int bi = (int)((b / cb) % rb), bj = (int)(b % cb);
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i)
      for (int j = 0; j < 128; ++j) {
        int64_t idx = (m * rows + bi * 128 + i) * (int64_t)cols + bj * 128 + j;
        amax = std::max(amax, static_cast<float>(std::fabs(bf16_value(w[idx]))));
      }
    float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    s[b] = sc;
    for (int i = 0; i < 128; ++i)
      for (int j = 0; j < 128; ++j) {
        int64_t idx = (m * rows + bi * 128 + i) * (int64_t)cols + bj * 128 + j;
        q[idx] = e4m3_code(static_cast<float>(bf16_value(w[idx])) / sc);
      }
  });
}

// Per-tensor quantisation (HPC-Ops page, main functions: GroupGEMM FP8 with
// per-tensor scales): mats tensors of n values each, bf16 bit patterns
// (f32 = 0) or fp32 values (f32 = 1).  s[m] = amax / 448 (fp32, 1 if amax is
// 0), q = e4m3(fp32(v / s[m])).
// The work is split over nthreads threads in contiguous pieces; a maximum does
// not depend on the order it is taken in, so the result is the same for any
// thread count.
void orc_quant_tensor_fp8(const void* x, int f32, int64_t mats, int64_t n, uint8_t* q, float* s, int nthreads) {
  auto val = [&](int64_t i) -> float {
    if (f32) return static_cast<const float*>(x)[i];
    return static_cast<float>(bf16_value(static_cast<const uint16_t*>(x)[i]));
  };
  const int64_t pieces = std::max<int64_t>(1, std::min<int64_t>(nthreads, (n + 65535) / 65536));
  const int64_t len = (n + pieces - 1) / pieces;
  std::vector<float> part(pieces);
  for (int64_t m = 0; m < mats; ++m) {
    parallel_for(pieces, nthreads, [&](int64_t p) {
      float pmax = 0.0f;
      for (int64_t i = p * len; i < std::min(n, (p + 1) * len); ++i) pmax = std::max(pmax, std::fabs(val(m * n + i)));
      part[p] = pmax;
    });
    float amax = 0.0f;
    for (int64_t p = 0; p < pieces; ++p) amax = std::max(amax, part[p]);
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    s[m] = sc;
    parallel_for(pieces, nthreads, [&](int64_t p) {
      for (int64_t i = p * len; i < std::min(n, (p + 1) * len); ++i) q[m * n + i] = e4m3_code(val(m * n + i) / sc);
    });
  }
}

// ---------------------------------------------------------------- expert FFN
// One SwiGLU expert on one token, bf16 operands, everything else in double:
// g = x.w1^T, u = x.w3^T, h = SiLU(g) * u, y = h.w2^T.
// w1, w3: [I, H]; w2: [H, I].  h_out (may be NULL): [I]; y: [H].
void orc_expert_bf16(const uint16_t* x, const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                     int H, int I, double* h_out, double* y) {
  std::vector<double> xv(H), h(I);
  for (int i = 0; i < H; ++i) xv[i] = bf16_value(x[i]);
  for (int n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int i = 0; i < H; ++i) {
      g += xv[i] * bf16_value(w1[(int64_t)n * H + i]);
      u += xv[i] * bf16_value(w3[(int64_t)n * H + i]);
    }
    h[n] = silu(g) * u;
    if (h_out) h_out[n] = h[n];
  }
  for (int m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int n = 0; n < I; ++n) acc += h[n] * bf16_value(w2[(int64_t)m * I + n]);
    y[m] = acc;
  }
}

// Blockwise-scaled fp8 dot product of one activation row with one weight row:
// sum over 128-wide K blocks of (xs[kb] * ws[kb]) * sum_k dec(xq[k]) * dec(wq[k]).
// Value of every E4M3 code, filled once from e4m3_value (a cache, not a
// different definition).
static const double* e4m3_table() {
  static double table[256];
  static bool ready = [] {
    for (int c = 0; c < 256; ++c) table[c] = e4m3_value(static_cast<uint8_t>(c));
    return true;
  }();
  (void)ready;
  return table;
}

static double fp8_dot(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, int K) {
  const double* dec = e4m3_table();
  double acc = 0.0;
  for (int kb = 0; kb < K / 128; ++kb) {
    double part = 0.0;
    for (int i = 0; i < 128; ++i) part += dec[xq[kb * 128 + i]] * dec[wq[kb * 128 + i]];
    acc += static_cast<double>(xs[kb]) * static_cast<double>(ws[kb]) * part;
  }
  return acc;
}

// MXFP8 dot product of one activation row with one weight row: sum over
// 32-wide K blocks of 2^(Xa + Xb) * sum_k dec(xq[k]) * dec(wq[k]), with the
// scale bytes xs[b] = Xa + 127 and ws[b] = Xb + 127.
static double mx_dot(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws, int K) {
  const double* dec = e4m3_table();
  double acc = 0.0;
  for (int b = 0; b < K / 32; ++b) {
    double part = 0.0;
    for (int i = 0; i < 32; ++i) part += dec[xq[b * 32 + i]] * dec[wq[b * 32 + i]];
    acc += std::ldexp(part, (static_cast<int>(xs[b]) - 127) + (static_cast<int>(ws[b]) - 127));
  }
  return acc;
}

// Per-tensor fp8 dot product of code rows: sum_k dec(xq[k]) * dec(wq[k]) over
// the whole K (the scales multiply the result once).  Every E4M3 value is an
// integer multiple of 2^-9 below 2^9, so each product is a multiple of 2^-18
// below 2^18 and, for K < 2^17, every partial sum is a multiple of 2^-18 below
// 2^35: exact in double whatever the order of the additions.
static double tensor_dot(const uint8_t* xq, const uint8_t* wq, int K) {
  const double* dec = e4m3_table();
  double acc = 0.0;
  for (int i = 0; i < K; ++i) acc += dec[xq[i]] * dec[wq[i]];
  return acc;
}

// Per-tensor fp8 h of one (token, expert) column from the code dot products of
// the gate and up rows: g = gdot * xs * s1, u = udot * xs * s3 (scaled once),
// h = SiLU(g) * u rounded to fp32.
static float pt_h(double gdot, double udot, double xsc, double s1, double s3) {
  const double gv = gdot * xsc * s1;
  const double uv = udot * xsc * s3;
  return static_cast<float>(silu(gv) * uv);
}

// One SwiGLU expert on one token with FP8 operands (the "activation
// quantisation" stage of FusedMoE between Gate-Up and Down):
//  xq [H] e4m3 + xs [H/128]; w1q, w3q [I, H] e4m3 + s1, s3 [I/128, H/128];
//  w2q [H, I] e4m3 + s2 [H/128, I/128].
// g, u are blockwise-scaled sums in double; h = SiLU(g) * u is rounded to
// fp32 and requantised per 128 columns (scale amax/448); y uses those codes.
// h_out (may be NULL) receives the fp32-rounded h; y: [H].
void orc_expert_fp8(const uint8_t* xq, const float* xs, const uint8_t* w1q, const float* s1,
                    const uint8_t* w3q, const float* s3, const uint8_t* w2q, const float* s2,
                    int H, int I, double* h_out, double* y) {
  int hb = H / 128, ib = I / 128;
  std::vector<float> h(I);
  std::vector<float> ws(hb);
  for (int n = 0; n < I; ++n) {
    for (int kb = 0; kb < hb; ++kb) ws[kb] = s1[(n / 128) * hb + kb];
    double g = fp8_dot(xq, xs, w1q + (int64_t)n * H, ws.data(), H);
    for (int kb = 0; kb < hb; ++kb) ws[kb] = s3[(n / 128) * hb + kb];
    double u = fp8_dot(xq, xs, w3q + (int64_t)n * H, ws.data(), H);
    h[n] = static_cast<float>(silu(g) * u);
    if (h_out) h_out[n] = h[n];
  }
  std::vector<uint8_t> hq(I);
  std::vector<float> hs(ib);
  for (int g = 0; g < ib; ++g) {
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i) amax = std::max(amax, std::fabs(h[g * 128 + i]));
    float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    hs[g] = sc;
    for (int i = 0; i < 128; ++i) hq[g * 128 + i] = e4m3_code(h[g * 128 + i] / sc);
  }
  std::vector<float> w2s(ib);
  for (int m = 0; m < H; ++m) {
    for (int kb = 0; kb < ib; ++kb) w2s[kb] = s2[(m / 128) * ib + kb];
    y[m] = fp8_dot(hq.data(), hs.data(), w2q + (int64_t)m * I, w2s.data(), I);
  }
}

// ---------------------------------------------------------------- layer
// Expert weights for the layer.  bf16 weights (wtype 0), e4m3 codes with
// 128x128 fp32 block scales (wtype 1: s1, s3 [E, I/128, H/128], s2
// [E, H/128, I/128]), MXFP8 (wtype 2: E8M0 bytes per weight row per 32 K,
// s1, s3 [E, I, H/32], s2 [E, H, I/32]) or per-tensor FP8 (wtype 3: one fp32
// scale per matrix, s1, s3, s2 [E] and ss1, ss3, ss2 [1]).  Routed experts are
// [E, ...]; the shared expert (has_shared) is a single expert of the same
// shape.  For wtype 3, h_scale gives the scale of the whole h tensor; when it
// is NULL the h of the pairs being computed is taken as the whole tensor
// (exact when every token is computed).
struct orc_layer {
  int wtype, E, H, I, has_shared;
  const void *w1, *w3, *w2;
  const void *s1, *s3, *s2;
  const void *sw1, *sw3, *sw2;
  const void *ss1, *ss3, *ss2;
  const float* h_scale;  // per-tensor FP8 only: scale of the whole h, or NULL
};

// The whole layer on a list of tokens ("top-k weighted combine", stage 5):
//   out[r] = sum_j w[t,j] * FFN_{ids[t,j]}(x_t) + FFN_shared(x_t),  t = rows[r].
// bf16 path: x is bf16 [T,H] and xs is NULL.  fp8 path: x is the e4m3 code
// array [T,H] and xs [T,H/128] its fp32 scales (from orc_quant_rows_fp8).
// MXFP8 path: x codes [T,H] and xs [T,H/32] E8M0 bytes (orc_quant_rows_mx);
// h is requantised per row per 32 columns with the MX rule.  Per-tensor FP8:
// x codes [T,H] and xs [1] (orc_quant_tensor_fp8 of the whole x); h is
// requantised with one scale (L->h_scale, or from these pairs' h).
// ids / weights are the route output [T,k].  out: [nrows, H] double.
//
// The arithmetic per (token, expert) is exactly orc_expert_bf16 /
// orc_expert_fp8; the loops only run expert by expert so that each expert's
// weight rows are read once for all the checked tokens that use it.
//
// orc_layer_rows_trace also hands out the intermediate h of every pair it
// computes (tr, any member may be NULL), pair q = r * (k + S) + j for rank j < k
// of token rows[r] and j == k for its shared expert:
//   h       [npairs, I] fp32: h rounded to fp32 (the value the FP8 paths requantise)
//   hq      [npairs, I] the requantised h codes (FP8 paths)
//   hs      [npairs, I/128] fp32 scales (block FP8) or [npairs, I/32] E8M0 bytes (MXFP8)
//   h_scale [1] the scale of the whole h (per-tensor FP8)
struct orc_trace {
  float* h;
  uint8_t* hq;
  void* hs;
  float* h_scale;
};

void orc_layer_rows_trace(const orc_layer* L, const void* x, const void* xs, const int32_t* ids,
                          const double* weights, int k, const int64_t* rows, int64_t nrows, double* out,
                          int nthreads, const orc_trace* tr) {
  const int H = L->H, I = L->I, E = L->E;
  const int hb = H / 128, ib = I / 128;
  const int64_t mat = (int64_t)I * H;
  const int64_t blk = (int64_t)ib * hb;
  const int per_row = k + (L->has_shared ? 1 : 0);
  const int64_t npairs = nrows * per_row;
  const bool fp8 = L->wtype != 0;
  const bool mx = L->wtype == 2;
  const bool pt = L->wtype == 3;
  const int hm = H / 32, im = I / 32;   // MX blocks per row
  auto fs = [](const void* p) { return static_cast<const float*>(p); };
  auto bs = [](const void* p) { return static_cast<const uint8_t*>(p); };

  // pair q = r * per_row + j: token rows[r], expert ids[t,j] (j < k) or the
  // shared expert (group E, j == k)
  std::vector<std::vector<int64_t>> members(E + 1);
  for (int64_t r = 0; r < nrows; ++r)
    for (int j = 0; j < per_row; ++j) {
      const int g = j == k ? E : ids[rows[r] * k + j];
      members[g].push_back(r * per_row + j);
    }
  auto token_of = [&](int64_t q) { return rows[q / per_row]; };

  std::vector<double> hbuf(npairs * (int64_t)I);   // h per pair (double; fp8: fp32-rounded)
  std::vector<uint8_t> hq(fp8 ? npairs * (int64_t)I : 0);
  std::vector<float> hs(fp8 && !mx && !pt ? npairs * (int64_t)ib : 0);
  float h_tensor_scale = 1.0f;
  std::vector<uint8_t> hsm(mx ? npairs * (int64_t)im : 0);
  std::vector<double> ybuf(npairs * (int64_t)H);

  // phase 1: h = SiLU(x.w1^T) * (x.w3^T) for every pair, task = (group, 128 rows of w1/w3)
  const int nt1 = I / 128;
  parallel_for((int64_t)(E + 1) * nt1, nthreads, [&](int64_t task) {
    const int g = (int)(task / nt1), n0 = (int)(task % nt1) * 128;
    if (members[g].empty()) return;
    const bool sh = g == E;
    std::vector<double> xv(H);
    for (int64_t q : members[g]) {
      const int64_t t = token_of(q);
      for (int n = n0; n < n0 + 128; ++n) {
        double gv = 0.0, uv = 0.0;
        if (!fp8) {
          const uint16_t* xr = static_cast<const uint16_t*>(x) + t * H;
          const uint16_t* w1 = (sh ? static_cast<const uint16_t*>(L->sw1) : static_cast<const uint16_t*>(L->w1) + g * mat) + (int64_t)n * H;
          const uint16_t* w3 = (sh ? static_cast<const uint16_t*>(L->sw3) : static_cast<const uint16_t*>(L->w3) + g * mat) + (int64_t)n * H;
          gv = 0.0;
          uv = 0.0;
          for (int i = 0; i < H; ++i) {
            const double xi = bf16_value(xr[i]);
            gv += xi * bf16_value(w1[i]);
            uv += xi * bf16_value(w3[i]);
          }
          hbuf[q * I + n] = silu(gv) * uv;
        } else {
          const uint8_t* xr = static_cast<const uint8_t*>(x) + t * H;
          const uint8_t* w1 = (sh ? static_cast<const uint8_t*>(L->sw1) : static_cast<const uint8_t*>(L->w1) + g * mat) + (int64_t)n * H;
          const uint8_t* w3 = (sh ? static_cast<const uint8_t*>(L->sw3) : static_cast<const uint8_t*>(L->w3) + g * mat) + (int64_t)n * H;
          if (mx) {
            const uint8_t* xsr = bs(xs) + t * hm;
            const uint8_t* s1 = sh ? bs(L->ss1) + (int64_t)n * hm : bs(L->s1) + ((int64_t)g * I + n) * hm;
            const uint8_t* s3 = sh ? bs(L->ss3) + (int64_t)n * hm : bs(L->s3) + ((int64_t)g * I + n) * hm;
            gv = mx_dot(xr, xsr, w1, s1, H);
            uv = mx_dot(xr, xsr, w3, s3, H);
          } else if (pt) {
            const double xsc = fs(xs)[0];
            const double s1 = sh ? fs(L->ss1)[0] : fs(L->s1)[g];
            const double s3 = sh ? fs(L->ss3)[0] : fs(L->s3)[g];
            hbuf[q * I + n] = pt_h(tensor_dot(xr, w1, H), tensor_dot(xr, w3, H), xsc, s1, s3);
          } else {
            const float* xsr = fs(xs) + t * hb;
            const float* s1 = (sh ? fs(L->ss1) : fs(L->s1) + g * blk) + (n / 128) * hb;
            const float* s3 = (sh ? fs(L->ss3) : fs(L->s3) + g * blk) + (n / 128) * hb;
            gv = fp8_dot(xr, xsr, w1, s1, H);
            uv = fp8_dot(xr, xsr, w3, s3, H);
          }
          if (!pt) hbuf[q * I + n] = static_cast<float>(silu(gv) * uv);
        }
      }
    }
  });

  // MXFP8: requantise each pair's fp32-rounded h per 32 columns (MX rule)
  if (mx) {
    parallel_for(npairs, nthreads, [&](int64_t q) {
      std::vector<float> hv(I);
      for (int i = 0; i < I; ++i) hv[i] = static_cast<float>(hbuf[q * I + i]);
      for (int b = 0; b < im; ++b) mx_quant_block(hv.data() + b * 32, 32, &hq[q * I + b * 32], &hsm[q * im + b]);
    });
  }
  // per-tensor fp8: one scale for the whole fp32-rounded h
  if (pt) {
    if (L->h_scale) {
      h_tensor_scale = *L->h_scale;
    } else {
      float amax = 0.0f;
      for (int64_t i = 0; i < npairs * (int64_t)I; ++i) amax = std::max(amax, std::fabs(static_cast<float>(hbuf[i])));
      h_tensor_scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    }
    const float sc = h_tensor_scale;
    parallel_for(npairs, nthreads, [&](int64_t q) {
      for (int i = 0; i < I; ++i) hq[q * I + i] = e4m3_code(static_cast<float>(hbuf[q * I + i]) / sc);
    });
  }
  // fp8: requantise each pair's h per 128 columns (scale amax/448)
  if (fp8 && !mx && !pt) {
    parallel_for(npairs, nthreads, [&](int64_t q) {
      for (int gi = 0; gi < ib; ++gi) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) amax = std::max(amax, std::fabs(static_cast<float>(hbuf[q * I + gi * 128 + i])));
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        hs[q * ib + gi] = sc;
        for (int i = 0; i < 128; ++i)
          hq[q * I + gi * 128 + i] = e4m3_code(static_cast<float>(hbuf[q * I + gi * 128 + i]) / sc);
      }
    });
  }

  if (tr) {
    if (tr->h)
      for (int64_t i = 0; i < npairs * (int64_t)I; ++i) tr->h[i] = static_cast<float>(hbuf[i]);
    if (tr->hq && fp8) std::memcpy(tr->hq, hq.data(), hq.size());
    if (tr->hs && mx) std::memcpy(tr->hs, hsm.data(), hsm.size());
    if (tr->hs && fp8 && !mx && !pt) std::memcpy(tr->hs, hs.data(), hs.size() * sizeof(float));
    if (tr->h_scale && pt) *tr->h_scale = h_tensor_scale;
  }

  // phase 2: y = h.w2^T for every pair, task = (group, 128 rows of w2)
  const int nt2 = H / 128;
  parallel_for((int64_t)(E + 1) * nt2, nthreads, [&](int64_t task) {
    const int g = (int)(task / nt2), m0 = (int)(task % nt2) * 128;
    if (members[g].empty()) return;
    const bool sh = g == E;
    for (int64_t q : members[g]) {
      for (int m = m0; m < m0 + 128; ++m) {
        double acc;
        if (!fp8) {
          const uint16_t* w2 = (sh ? static_cast<const uint16_t*>(L->sw2) : static_cast<const uint16_t*>(L->w2) + g * mat) + (int64_t)m * I;
          acc = 0.0;
          for (int n = 0; n < I; ++n) acc += hbuf[q * I + n] * bf16_value(w2[n]);
        } else {
          const uint8_t* w2 = (sh ? static_cast<const uint8_t*>(L->sw2) : static_cast<const uint8_t*>(L->w2) + g * mat) + (int64_t)m * I;
          if (mx) {
            const uint8_t* s2 = sh ? bs(L->ss2) + (int64_t)m * im : bs(L->s2) + ((int64_t)g * H + m) * im;
            acc = mx_dot(hq.data() + q * I, hsm.data() + q * im, w2, s2, I);
          } else if (pt) {
            const double s2 = sh ? fs(L->ss2)[0] : fs(L->s2)[g];
            acc = tensor_dot(hq.data() + q * I, w2, I) * static_cast<double>(h_tensor_scale) * s2;
          } else {
            const float* s2 = (sh ? fs(L->ss2) : fs(L->s2) + g * blk) + (m / 128) * ib;
            acc = fp8_dot(hq.data() + q * I, hs.data() + q * ib, w2, s2, I);
          }
        }
        ybuf[q * H + m] = acc;
      }
    }
  });

  // combine in fixed order: routed ranks j = 0..k-1, then the shared expert
  parallel_for(nrows, nthreads, [&](int64_t r) {
    const int64_t t = rows[r];
    double* o = out + r * H;
    for (int m = 0; m < H; ++m) o[m] = 0.0;
    for (int j = 0; j < per_row; ++j) {
      const int64_t q = r * per_row + j;
      const double wt = j == k ? 1.0 : weights[t * k + j];
      for (int m = 0; m < H; ++m) o[m] += wt * ybuf[q * H + m];
    }
  });
}

void orc_layer_rows(const orc_layer* L, const void* x, const void* xs, const int32_t* ids,
                    const double* weights, int k, const int64_t* rows, int64_t nrows, double* out,
                    int nthreads) {
  orc_layer_rows_trace(L, x, xs, ids, weights, k, rows, nrows, out, nthreads, nullptr);
}

// Per-tensor FP8 h of n (token, column) entries of one expert from the exact
// code dot products of its gate rows (gdot) and up rows (udot): the arithmetic
// of the layer's Gate-Up step above, for a whole-tensor pass over h.
void orc_pt_h(const double* gdot, const double* udot, int64_t n, double xsc, double s1, double s3, float* h) {
  for (int64_t i = 0; i < n; ++i) h[i] = pt_h(gdot[i], udot[i], xsc, s1, s3);
}

// ---------------------------------------------------------------- combine / norm
// Stage 5 on given expert outputs y [R,H] (fp32 values): out[t] =
// sum_j w[t,j] * y[pair_slot[t*k+j]] + shared * y[T*k + t], in double.
void orc_combine(const float* y, const int32_t* pair_slot, const float* w, int64_t T, int k, int H,
                 int has_shared, double* out) {
  const int64_t P = T * k;
  for (int64_t t = 0; t < T; ++t)
    for (int m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += static_cast<double>(w[t * k + j]) * y[(int64_t)pair_slot[t * k + j] * H + m];
      if (has_shared) acc += y[(P + t) * H + m];
      out[t * H + m] = acc;
    }
}

// Residual add + RMSNorm, the single-GPU half of the HPC-Ops page's fused
// AllReduce+Norm (technical principles: RMSNorm(AllReduce(x) + residual,
// weight); on one GPU the all-reduce is the identity):
//   s = x + residual,  out = s / sqrt(mean(s^2) + eps) * weight   (per row, in double)
// x [rows,H] double, residual and weight bf16; s and out [rows,H] double.
void orc_add_rmsnorm(const double* x, const uint16_t* residual, const uint16_t* weight, double eps,
                     int64_t rows, int H, double* s, double* out) {
  for (int64_t r = 0; r < rows; ++r) {
    double ssq = 0.0;
    for (int m = 0; m < H; ++m) {
      const double v = x[r * H + m] + bf16_value(residual[r * H + m]);
      s[r * H + m] = v;
      ssq += v * v;
    }
    const double inv = 1.0 / std::sqrt(ssq / H + eps);
    for (int m = 0; m < H; ++m) out[r * H + m] = s[r * H + m] * inv * bf16_value(weight[m]);
  }
}

int orc_version(void) { return 1; }

}  // extern "C"
