// oracle.cpp -- plain, slow CPU reference of one MoE decode layer with MXFP4
// experts.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU
// baseline leg of the benchmark call it; the library never does.  It shares
// no code with the GPU library (no headers, helpers or tables) and reads only
// the bytes the seeded generator writes.
//
// What is computed, and where it is stated
//   * The layer: a router over E experts, top-k selection with renormalised
//     softmax gates, one bf16 shared expert, k routed experts stored in MXFP4,
//     each a SwiGLU gate/up/down chain, summed into the fp32 residual.  The
//     per-layer work list (router, shared expert, 16 of 896 routed experts,
//     MXFP4 experts of 17,547,264 bytes) is in "Kimi K3 on GB300: 13 kernels a
//     layer, and what 842 and 423 tokens a second measure" (ai.thesatyajit.com),
//     section "What one decode step of Kimi K3 does".
//   * MXFP4: OCP Microscaling Formats (MX) v1.0 -- E2M1 elements (sign, 2-bit
//     exponent with bias 1, 1-bit mantissa, no inf/NaN) and one E8M0 scale
//     (2^(e-127), 0xFF = NaN) per block of 32 consecutive elements along K.
//     Byte i of a row holds element 2i in bits 3:0 and element 2i+1 in 7:4.
//
// Precision: every dot product is accumulated in double in ascending index
// order and rounded to fp32 once per stage value; elementwise steps are done
// in double from the fp32 stage values and rounded to fp32.  The router logit
// is the fp32 rounding of the double sum of bf16 x bf16 products (each exact
// in double) plus the bias.  Top-k ranks the fp32 logits by (value
// descending, index ascending); -0 and +0 compare equal.
//
// Parity pins for every function here live in tests/test_oracle_*.py.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// fp32 -> bf16 with round-to-nearest-even, via an explicit significand
// rounding in double (finite inputs).
uint16_t float_to_bf16(float f) {
  if (f == 0.0f || !std::isfinite(f)) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
  }
  int e;
  double m = std::frexp((double)f, &e);  // f = m * 2^e, 0.5 <= |m| < 1
  // bf16 keeps 8 significant bits for normal numbers; below 2^-126 the
  // quantum is fixed at 2^-133.
  int keep = 8;
  if (e - 1 < -126) keep = 8 - (-126 - (e - 1));
  double q = std::nearbyint(std::ldexp(m, keep));  // default mode: ties to even
  double r = std::ldexp(q, e - keep);
  float rf = (float)r;  // exact: r has <= 8 significant bits
  uint32_t u;
  std::memcpy(&u, &rf, 4);
  return (uint16_t)(u >> 16);
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

uint64_t round256(uint64_t n) { return (n + 255) / 256 * 256; }

struct Blob {
  const uint8_t* codes[3];
  const uint8_t* scales[3];
};

}  // namespace

extern "C" {

// ---- MXFP4 element and scale decode (OCP MX v1.0) -------------------------

// E2M1: value = (-1)^s * (e == 0 ? m/2 : 2^(e-1) * (1 + m/2)).
double oracle_e2m1(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

// E8M0: 2^(byte - 127); byte 0xFF encodes NaN.
double oracle_e8m0(int byte) {
  if (byte == 0xFF) return std::nan("");
  return std::ldexp(1.0, byte - 127);
}

// ---- MXFP8 activations (OCP MX v1.0, E4M3 elements) ----------------------
//
// The opt-in variant of the layer quantises the routed experts' activations
// to MXFP8, the precision "Kimi K3 on GB300: 13 kernels a layer, and what 842
// and 423 tokens a second measure" (section "Why batch 1 on a rack is not
// only a bandwidth problem") gives for its expert kernel: FP4 weights times
// MXFP8 activations.  E4M3 (OCP 8-bit floating point, the "FN" variant the
// MX formats use): sign, 4-bit exponent with bias 7, 3-bit mantissa; exponent
// field 0 holds the subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no
// infinity; the largest finite magnitude is 1.75 * 2^8 = 448.
double oracle_e4m3(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return std::nan("");
  double mag = (e == 0) ? std::ldexp((double)m / 8.0, -6) : std::ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

// Nearest E4M3 code to v (ties to the even code), magnitudes past the
// largest finite one clamped to it (saturation).  v finite.
static int e4m3_encode(double v) {
  int s = std::signbit(v) ? 1 : 0;
  double a = std::fabs(v);
  int best = 0;
  double best_d = a;  // code 0 (+0)
  for (int c = 1; c < 0x7F; ++c) {  // the finite non-negative codes, ascending
    double d = std::fabs(oracle_e4m3(c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (s << 7) | best;
}

// MXFP8 quantisation of n values (n a multiple of 32), block by block of 32
// consecutive values: the shared scale is X = 2^(floor(log2(amax)) - 8), 8
// being the exponent of E4M3's largest power of two, clamped to the E8M0
// range [2^-127, 2^127] (amax = 0 gives 2^-127); each element is the E4M3
// code nearest v / X.  scales[i] is the E8M0 byte of block i.
void oracle_quantize_mxfp8(const float* v, int n, uint8_t* codes, uint8_t* scales) {
  for (int b = 0; b < n / 32; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs((double)v[32 * b + i]));
    int e = -127;
    if (amax > 0.0) {
      int ex;
      std::frexp(amax, &ex);  // amax = f * 2^ex, 0.5 <= f < 1: floor(log2 amax) = ex - 1
      e = std::min(127, std::max(-127, ex - 1 - 8));
    }
    scales[b] = (uint8_t)(e + 127);
    for (int i = 0; i < 32; ++i) codes[32 * b + i] = (uint8_t)e4m3_encode(std::ldexp((double)v[32 * b + i], -e));
  }
}

// The values an MXFP8 block encodes: e4m3(code) * 2^(scale - 127).
void oracle_dequantize_mxfp8(const uint8_t* codes, const uint8_t* scales, int n, float* v) {
  for (int i = 0; i < n; ++i) v[i] = (float)(oracle_e4m3(codes[i]) * oracle_e8m0(scales[i / 32]));
}

// Byte size of one expert blob: gate codes [I][H/2], up codes [I][H/2],
// down codes [H][I/2], gate scales [I][H/32], up scales [I][H/32],
// down scales [H][I/32], each sub-array starting on a 256-byte boundary.
uint64_t oracle_expert_bytes(int H, int I) {
  uint64_t h = (uint64_t)H, i = (uint64_t)I;
  return round256(i * h / 2) * 2 + round256(h * i / 2) + round256(i * h / 32) * 2 + round256(h * i / 32);
}

// w[n][k] = e2m1(code(n,k)) * e8m0(scale(n, k/32)) (exact in fp32 for the
// scale bytes in use; NaN where the block scale is 0xFF).
void oracle_decode_mxfp4(const uint8_t* codes, const uint8_t* scales, int N, int K, float* w) {
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) {
      uint8_t byte = codes[(size_t)n * (K / 2) + k / 2];
      int code = (k & 1) ? (byte >> 4) : (byte & 15);
      w[(size_t)n * K + k] = (float)(oracle_e2m1(code) * oracle_e8m0(scales[(size_t)n * (K / 32) + k / 32]));
    }
}

static double mx_weight(const uint8_t* codes, const uint8_t* scales, int K, int n, int k) {
  uint8_t byte = codes[(size_t)n * (K / 2) + k / 2];
  int code = (k & 1) ? (byte >> 4) : (byte & 15);
  return oracle_e2m1(code) * oracle_e8m0(scales[(size_t)n * (K / 32) + k / 32]);
}

// y[b][n] = fp32( sum_k w[n][k] * x[b][k] ), x bf16 (x_f32 == 0) or fp32.
void oracle_gemv_mxfp4(const uint8_t* codes, const uint8_t* scales, int N, int K, const void* x, int x_f32, int B,
                       float* y) {
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        double xv = x_f32 ? (double)((const float*)x)[(size_t)b * K + k]
                          : bf16_to_double(((const uint16_t*)x)[(size_t)b * K + k]);
        acc += mx_weight(codes, scales, K, n, k) * xv;
      }
      y[(size_t)b * N + n] = (float)acc;
    }
}

// ---- router -----------------------------------------------------------------

// logits[b][e] = fp32( sum_h x[b][h] * Wr[e][h] + bias[e] ), summed in double.
// Returns the number of logits whose ascending and descending double sums
// differ (0 means the double sum did not depend on the order).
int oracle_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int B, int H, int E,
                         float* logits) {
  int order_dependent = 0;
  for (int b = 0; b < B; ++b)
    for (int e = 0; e < E; ++e) {
      double fwd = 0.0, rev = 0.0;
      for (int h = 0; h < H; ++h)
        fwd += bf16_to_double(x[(size_t)b * H + h]) * bf16_to_double(wr[(size_t)e * H + h]);
      for (int h = H - 1; h >= 0; --h)
        rev += bf16_to_double(x[(size_t)b * H + h]) * bf16_to_double(wr[(size_t)e * H + h]);
      if (fwd != rev) ++order_dependent;
      double l = fwd + (bias ? (double)bias[e] : 0.0);
      logits[(size_t)b * E + e] = (float)l;
    }
  return order_dependent;
}

// Top-k by (logit descending, index ascending), then renormalised softmax over
// the k selected: g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
void oracle_topk(const float* logits, int B, int E, int k, int32_t* idx, float* gate) {
  std::vector<int> order(E);
  for (int b = 0; b < B; ++b) {
    const float* l = logits + (size_t)b * E;
    for (int e = 0; e < E; ++e) order[e] = e;
    std::sort(order.begin(), order.end(), [l](int a, int c) { return l[a] > l[c] || (l[a] == l[c] && a < c); });
    double den = 0.0;
    std::vector<double> num(k);
    for (int j = 0; j < k; ++j) {
      num[j] = std::exp((double)l[order[j]] - (double)l[order[0]]);
      den += num[j];
    }
    for (int j = 0; j < k; ++j) {
      idx[(size_t)b * k + j] = order[j];
      gate[(size_t)b * k + j] = (float)(num[j] / den);
    }
  }
}

// ---- SwiGLU experts ---------------------------------------------------------

}  // extern "C"

// One SwiGLU expert on one activation row, weights given as callables.
// With mx8, the routed experts' FP4 x MXFP8 variant: the row entering FC1
// and the SwiGLU output entering FC2 are each replaced by their MXFP8
// quantisation (oracle_quantize_mxfp8) before the dot products.
template <class WG, class WU, class WD>
static void swiglu_expert(int H, int I, const uint16_t* xrow, WG wg, WU wu, WD wd, float* o, bool mx8 = false) {
  std::vector<float> xin(H), h(I);
  for (int k = 0; k < H; ++k) xin[k] = (float)bf16_to_double(xrow[k]);
  if (mx8) {
    std::vector<uint8_t> c(H), sc(H / 32);
    oracle_quantize_mxfp8(xin.data(), H, c.data(), sc.data());
    oracle_dequantize_mxfp8(c.data(), sc.data(), H, xin.data());
  }
  for (int n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int k = 0; k < H; ++k) {
      double xv = (double)xin[k];
      g += wg(n, k) * xv;
      u += wu(n, k) * xv;
    }
    float gf = (float)g, uf = (float)u;
    h[n] = (float)(silu((double)gf) * (double)uf);
  }
  if (mx8) {
    std::vector<uint8_t> c(I), sc(I / 32);
    oracle_quantize_mxfp8(h.data(), I, c.data(), sc.data());
    oracle_dequantize_mxfp8(c.data(), sc.data(), I, h.data());
  }
  for (int m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int n = 0; n < I; ++n) acc += wd(m, n) * (double)h[n];
    o[m] = (float)acc;
  }
}

extern "C" {

// Shared expert (bf16 weights gate/up [Is][H], down [H][Is]) on x[b].
void oracle_shared_expert(const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, int H, int Is,
                          const uint16_t* x, int B, float* out) {
  for (int b = 0; b < B; ++b)
    swiglu_expert(
        H, Is, x + (size_t)b * H, [&](int n, int k) { return bf16_to_double(wg[(size_t)n * H + k]); },
        [&](int n, int k) { return bf16_to_double(wu[(size_t)n * H + k]); },
        [&](int m, int n) { return bf16_to_double(wd[(size_t)m * Is + n]); }, out + (size_t)b * H);
}

static Blob blob_view(const uint8_t* base, int H, int I) {
  uint64_t h = (uint64_t)H, i = (uint64_t)I;
  uint64_t o0 = 0, o1 = o0 + round256(i * h / 2), o2 = o1 + round256(i * h / 2), o3 = o2 + round256(h * i / 2),
           o4 = o3 + round256(i * h / 32), o5 = o4 + round256(i * h / 32);
  Blob bl;
  bl.codes[0] = base + o0;
  bl.codes[1] = base + o1;
  bl.codes[2] = base + o2;
  bl.scales[0] = base + o3;
  bl.scales[1] = base + o4;
  bl.scales[2] = base + o5;
  return bl;
}

// One routed MXFP4 expert (blob layout of oracle_expert_bytes) on x[b];
// mx8 != 0: its activations quantised to MXFP8 (see swiglu_expert).
void oracle_routed_expert_ex(const uint8_t* blob, int H, int I, const uint16_t* x, int B, float* out, int mx8) {
  Blob bl = blob_view(blob, H, I);
  for (int b = 0; b < B; ++b)
    swiglu_expert(
        H, I, x + (size_t)b * H, [&](int n, int k) { return mx_weight(bl.codes[0], bl.scales[0], H, n, k); },
        [&](int n, int k) { return mx_weight(bl.codes[1], bl.scales[1], H, n, k); },
        [&](int m, int n) { return mx_weight(bl.codes[2], bl.scales[2], I, m, n); }, out + (size_t)b * H,
        mx8 != 0);
}

void oracle_routed_expert(const uint8_t* blob, int H, int I, const uint16_t* x, int B, float* out) {
  oracle_routed_expert_ex(blob, H, I, x, B, out, 0);
}

// ---- whole layer --------------------------------------------------------------

// out[b] = fp32( residual[b] + shared(x[b]) + sum_j gate[b][j] * expert_{idx[b][j]}(x[b]) ),
// the sum over j taken in ascending j, all in double.
// experts[e] points at expert e's blob; entries for experts no row selects
// may be NULL.  Optional outputs: logits [B][E], shared_out [B][H],
// slot_out [B][k][H].  Returns -1 if a selected expert has no blob, else the
// router's order-dependence count.
// mx8 != 0: the routed experts run the FP4 x MXFP8 variant (their
// activations quantised to MXFP8); the router and the bf16 shared expert are
// unchanged.
int oracle_moe_layer_ex(int H, int I, int E, int k, int Is, const uint16_t* router_w, const float* router_bias,
                        const uint16_t* shared_gate, const uint16_t* shared_up, const uint16_t* shared_down,
                        const uint8_t* const* experts, const uint16_t* x, const float* residual, int B, float* out,
                        int32_t* idx, float* gate, float* logits_out, float* shared_out, float* slot_out, int mx8) {
  std::vector<float> logits((size_t)B * E);
  int od = oracle_router_logits(x, router_w, router_bias, B, H, E, logits.data());
  oracle_topk(logits.data(), B, E, k, idx, gate);
  if (logits_out) std::memcpy(logits_out, logits.data(), sizeof(float) * logits.size());
  for (int s = 0; s < B * k; ++s)
    if (!experts[idx[s]]) return -1;
  // The expert evaluations of the B rows (k routed + 1 shared each) are
  // independent of each other; they may run on several host threads
  // (oracle_set_threads), each evaluation exactly as on one thread.
  std::vector<float> os((size_t)B * H, 0.0f), oj((size_t)B * k * H);
  const int per_row = k + 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < B * per_row; ++t) {
    const int b = t / per_row, j = t % per_row;
    const uint16_t* xb = x + (size_t)b * H;
    if (j == k) {
      if (Is > 0) oracle_shared_expert(shared_gate, shared_up, shared_down, H, Is, xb, 1, os.data() + (size_t)b * H);
    } else {
      oracle_routed_expert_ex(experts[idx[(size_t)b * k + j]], H, I, xb, 1, oj.data() + ((size_t)b * k + j) * H, mx8);
    }
  }
  for (int b = 0; b < B; ++b) {
    const float* ob = oj.data() + (size_t)b * k * H;
    for (int m = 0; m < H; ++m) {
      double acc = (double)residual[(size_t)b * H + m] + (double)os[(size_t)b * H + m];
      for (int j = 0; j < k; ++j) acc += (double)gate[(size_t)b * k + j] * (double)ob[(size_t)j * H + m];
      out[(size_t)b * H + m] = (float)acc;
    }
    if (shared_out) std::memcpy(shared_out + (size_t)b * H, os.data() + (size_t)b * H, sizeof(float) * H);
    if (slot_out) std::memcpy(slot_out + (size_t)b * k * H, ob, sizeof(float) * (size_t)k * H);
  }
  return od;
}

int oracle_moe_layer(int H, int I, int E, int k, int Is, const uint16_t* router_w, const float* router_bias,
                     const uint16_t* shared_gate, const uint16_t* shared_up, const uint16_t* shared_down,
                     const uint8_t* const* experts, const uint16_t* x, const float* residual, int B, float* out,
                     int32_t* idx, float* gate, float* logits_out, float* shared_out, float* slot_out) {
  return oracle_moe_layer_ex(H, I, E, k, Is, router_w, router_bias, shared_gate, shared_up, shared_down, experts, x,
                             residual, B, out, idx, gate, logits_out, shared_out, slot_out, 0);
}

// Host threads the layer's expert evaluations may use (OpenMP); the results
// do not depend on it.  Returns the number now in effect.
int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

// ---- dense block pieces of the layer stack ----------------------------------

// bf16 rounding (round to nearest even) of fp32 values, exposed for the pins.
void oracle_to_bf16(const float* in, uint64_t n, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = float_to_bf16(in[i]);
}

// out[b] = bf16( fp32( h[b] / sqrt(mean(h[b]^2) + eps) ) ), gain 1.
void oracle_rmsnorm_bf16(const float* h, int B, int H, double eps, uint16_t* out) {
  for (int b = 0; b < B; ++b) {
    double ss = 0.0;
    for (int i = 0; i < H; ++i) ss += (double)h[(size_t)b * H + i] * (double)h[(size_t)b * H + i];
    double r = 1.0 / std::sqrt(ss / H + eps);
    for (int i = 0; i < H; ++i) out[(size_t)b * H + i] = float_to_bf16((float)((double)h[(size_t)b * H + i] * r));
  }
}

// y[b][n] = bf16( fp32( sum_k W[n][k] * x[b][k] ) ), W bf16 [N][K], x bf16 [B][K].
void oracle_dense_gemv_bf16(const uint16_t* w, int N, int K, const uint16_t* x, int B, uint16_t* y) {
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += bf16_to_double(w[(size_t)n * K + k]) * bf16_to_double(x[(size_t)b * K + k]);
      y[(size_t)b * N + n] = float_to_bf16((float)acc);
    }
}

}  // extern "C"
