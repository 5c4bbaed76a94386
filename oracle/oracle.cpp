// LatentMoE feed-forward layer: plain CPU oracle.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
// reference that the HIP path is checked against.  Only the tests, the smoke
// check and the bench's CPU-baseline leg may load it; the product path never
// calls it.  It shares no code, header or table with the HIP library.
//
// Sources (the pages this layer is described on):
//  [vLLM-K3]   "Kimi K3 Inference Backend Evolution: System Redesign from Hybrid
//              Architecture to Maximum Throughput", section 1, "LatentMoE:
//              Dimensionality Reduction at the Routing Inlet, Restoration at the
//              Outlet" (down-proj before the router, experts and combine in the
//              latent, up-proj after); section 6, "Latent MoE Tail" (routed
//              latent: reduce + RMSNorm, then the up-projection; shared
//              experts' partial added to the projected output).
//  [TS-AgentX] "331 output tokens/s per GPU on AgentX: Serving Kimi K3 on GB300
//              with TokenSpeed", "Model architecture" (16 of 896 routed experts
//              per token and two shared experts) and "Kernel fusion and overlap
//              complete the decode path" (shared experts beside the routed path,
//              combined after its output projection).
//  [TS-K3]     TokenSpeed's Day-0 Kimi K3 post (lightseek.org), "TensorRT-LLM
//              Stable LatentMoE" (expert MLP = gated FC1 then FC2; MXFP4
//              weights with bf16 or MXFP8 activations, FC1's output requantised
//              to MXFP8 in the w4a8 path), "Gluon kernels on AMD GPUs > Stable
//              LatentMoE" and "Iris and communication" (routed latent RMSNorm;
//              shared partial at hidden width).
//  [OCP-MX]    OCP Microscaling Formats (MX) v1.0: e2m1, e4m3 (fn), e8m0 and the
//              shared-scale rule X = 2^(floor(log2 amax) - emax_elem).
//
// Readings where the pages are silent (each one is listed in the design notes):
//  * router: top-k by (logit desc, expert index asc), NaN below every number;
//    combine weights = softmax over the k selected logits; when the logits
//    are computed here, the gate scores the bf16 latent z in fp32;
//  * permutation: stable counting sort of rows r = t*k + j by expert;
//  * "SiTU" gate read as SwiGLU: silu(W1 a) * (W3 a), silu(g) = g / (1 + e^-g);
//  * shared experts are SwiGLU FFNs on the hidden state x, added inside the
//    up-projection; routed RMSNorm is optional (gain pointer may be NULL);
//  * bf16 storage (round to nearest even) at z, H, Y, rhat, hs and y; fp32
//    everywhere else, every dot product accumulated in ascending K order.
//  * MXFP4 experts run w4a8: activations entering each expert GEMM are
//    quantised to MXFP8 (e4m3fn, one e8m0 scale per 32 along K).
//
// Build: g++ -O2 -ffp-contract=off -fopenmp -shared -fPIC oracle.cpp
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------- bf16 / fp32
float from_bf16(uint16_t h) {
  uint32_t u = uint32_t(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round-to-nearest-even fp32 -> bf16.  NaN stays NaN (quiet bit forced).
uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x0040u);
  uint32_t keep = u >> 16;            // truncated value
  uint32_t rest = u & 0xffffu;        // dropped bits
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1;  // ties to even
  return uint16_t(keep);
}

float bf16_round(float f) { return from_bf16(to_bf16(f)); }

// ------------------------------------------------------------------ OCP MX
// e2m1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; no inf/NaN.
float e2m1_value(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  float mag = (e == 0) ? 0.5f * float(m) : std::ldexp(1.0f + 0.5f * float(m), int(e) - 1);
  return s ? -mag : mag;
}

// e8m0: an unsigned power-of-two exponent with bias 127; 0xFF is NaN.
float e8m0_value(unsigned code) {
  return code == 255u ? NAN : std::ldexp(1.0f, int(code) - 127);
}

// e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no inf;
// S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
float e4m3_value(unsigned code) {
  unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
  if (e == 15 && m == 7) return NAN;
  float mag = (e == 0) ? std::ldexp(float(m) / 8.0f, -6)
                       : std::ldexp(1.0f + float(m) / 8.0f, int(e) - 7);
  return s ? -mag : mag;
}

// Nearest e4m3fn code to v (ties to the even code), saturating to +-448;
// NaN gives the NaN code S.1111.111.  Written as a search over all finite
// codes: slow, but its correctness can be read off directly.
unsigned e4m3_encode(float v) {
  unsigned sign = std::signbit(v) ? 0x80u : 0u;
  if (std::isnan(v)) return sign | 0x7Fu;
  float a = std::fabs(v);
  if (a >= 448.0f) return sign | 0x7Eu;
  unsigned best = 0;
  float best_err = a;  // distance to code 0
  for (unsigned c = 1; c < 0x7F; ++c) {
    float err = std::fabs(e4m3_value(c) - a);
    if (err < best_err || (err == best_err && (c & 1u) == 0u && (best & 1u) == 1u)) {
      best = c;
      best_err = err;
    }
  }
  return sign | best;
}

// MXFP8 (e4m3fn) quantise-dequantise of one 32-element block, per OCP MX:
// shared exponent = floor(log2(amax)) - 8 (8 = exponent of e4m3's largest
// normal), clamped to e8m0's range; elements = nearest e4m3 of v / 2^exp.
// An all-zero block gets scale code 0 and zero elements.  A block holding a
// NaN or an infinity (e4m3fn has no infinity) becomes a NaN block: scale code
// 255 (e8m0's NaN) and every element code the e4m3fn NaN 0x7F, so all 32
// values dequantise to NaN.
void mxfp8_block(const float* v, float* out, uint8_t* codes, uint8_t* scale_code) {
  bool finite = true;
  for (int i = 0; i < 32; ++i) finite = finite && std::isfinite(v[i]);
  if (!finite) {
    if (scale_code) *scale_code = 255;
    for (int i = 0; i < 32; ++i) {
      if (codes) codes[i] = 0x7F;
      out[i] = NAN;
    }
    return;
  }
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(v[i]));
  int sexp;
  if (amax == 0.0f) {
    sexp = -127;
  } else {
    int e;
    std::frexp(amax, &e);  // amax = f * 2^e, f in [0.5, 1)
    sexp = (e - 1) - 8;
    sexp = std::min(127, std::max(-127, sexp));
  }
  if (scale_code) *scale_code = uint8_t(sexp + 127);
  for (int i = 0; i < 32; ++i) {
    unsigned c = e4m3_encode(std::ldexp(v[i], -sexp));
    if (codes) codes[i] = uint8_t(c);
    out[i] = e4m3_value(c) * std::ldexp(1.0f, sexp);
  }
}

float silu(float g) { return g / (1.0f + std::exp(-g)); }

// fp32 dot product in ascending index order, or (rev) in descending order.
// Both are valid fp32 evaluations of the same sum; the reversed order exists
// to measure how far two valid orders land apart.
float dot(const float* a, const float* b, int64_t n, bool rev = false) {
  float acc = 0.0f;
  if (rev) {
    for (int64_t i = n - 1; i >= 0; --i) acc += a[i] * b[i];
  } else {
    for (int64_t i = 0; i < n; ++i) acc += a[i] * b[i];
  }
  return acc;
}

void bf16_row(const uint16_t* src, float* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = from_bf16(src[i]);
}

// Row `row` (length K) of a weight matrix stored either as bf16 [.., K] or as
// MXFP4 packed codes [.., K/2] with e8m0 scales [.., K/32], dequantised to fp32.
void weight_row(const void* w, const uint8_t* s, bool mxfp4, int64_t row, int64_t K, float* out) {
  if (!mxfp4) {
    bf16_row(static_cast<const uint16_t*>(w) + row * K, out, K);
    return;
  }
  // the 16 e2m1 values, each from e2m1_value (the products below are the
  // same ones e2m1_value(c) * e8m0_value(scale) gives element by element)
  static const std::vector<float> table = [] {
    std::vector<float> t(16);
    for (unsigned c = 0; c < 16; ++c) t[c] = e2m1_value(c);
    return t;
  }();
  const uint8_t* codes = static_cast<const uint8_t*>(w) + row * (K / 2);
  const uint8_t* sc = s + row * (K / 32);
  for (int64_t b = 0; b < K; b += 32) {
    const float scale = e8m0_value(sc[b / 32]);
    for (int64_t i = b; i < b + 32; ++i) {
      uint8_t byte = codes[i / 2];
      unsigned c = (i % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
      out[i] = table[c] * scale;
    }
  }
}

// MXFP8 quantise-dequantise of a row in place; codes [K] and scales [K/32]
// receive the encoding when not NULL.
void mxfp8_row(float* v, int64_t K, uint8_t* codes = nullptr, uint8_t* scales = nullptr) {
  float tmp[32];
  for (int64_t b = 0; b < K; b += 32) {
    mxfp8_block(v + b, tmp, codes ? codes + b : nullptr, scales ? scales + b / 32 : nullptr);
    std::memcpy(v + b, tmp, sizeof tmp);
  }
}

}  // namespace

extern "C" {

// ------------------------------------------------------------- codec helpers
// Exposed so that tests can check the codecs against the OCP MX definition.
float lmoe_oracle_e2m1_value(unsigned code) { return e2m1_value(code & 15u); }
float lmoe_oracle_e8m0_value(unsigned code) { return e8m0_value(code & 255u); }
float lmoe_oracle_e4m3_value(unsigned code) { return e4m3_value(code & 255u); }
unsigned lmoe_oracle_e4m3_encode(float v) { return e4m3_encode(v); }
uint16_t lmoe_oracle_to_bf16(float v) { return to_bf16(v); }
int lmoe_oracle_num_threads(void) { return omp_get_max_threads(); }
// Threads of the oracle's later parallel loops (called from the caller's thread).
void lmoe_oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

// MXFP8-quantise n (multiple of 32) floats: dequantised values, codes, scales.
void lmoe_oracle_mxfp8(const float* v, int64_t n, float* deq, uint8_t* codes, uint8_t* scales) {
  for (int64_t b = 0; b < n; b += 32)
    mxfp8_block(v + b, deq + b, codes ? codes + b : nullptr, scales ? scales + b / 32 : nullptr);
}

// ------------------------------------------------------------------- router
// [TS-AgentX] "Model architecture": each token selects k of E routed experts.
// ids[t, 0..k-1] = the first k experts under the order (logit descending,
// index ascending); IEEE comparison, so +0 == -0 and the lower index wins;
// NaN ranks below every number (ties among NaNs to the lower index).
// w[t, j] = exp(l_j - l_0) / sum_i exp(l_i - l_0), i.e. the softmax over the
// k selected logits (equal to a full softmax renormalised over the k).
void lmoe_oracle_route(int64_t T, int32_t E, int32_t k, const float* logits, int32_t* ids, float* w) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* lg = logits + t * E;
    std::vector<int32_t> order(E);
    for (int32_t e = 0; e < E; ++e) order[e] = e;
    auto before = [lg](int32_t a, int32_t b) {
      float va = lg[a], vb = lg[b];
      bool na = std::isnan(va), nb = std::isnan(vb);
      if (na != nb) return nb;          // a number ranks above NaN
      if (!na && va != vb) return va > vb;
      return a < b;                     // equal (or both NaN): lower index first
    };
    std::sort(order.begin(), order.end(), before);
    float m = lg[order[0]];
    std::vector<float> ex(k);
    float sum = 0.0f;
    for (int32_t j = 0; j < k; ++j) {
      ex[j] = std::exp(lg[order[j]] - m);
      sum += ex[j];
    }
    for (int32_t j = 0; j < k; ++j) {
      ids[t * k + j] = order[j];
      w[t * k + j] = ex[j] / sum;
    }
  }
}

// ------------------------------------------------------------ router logits
// [vLLM-K3] section 1: the latent down-projection sits in front of the
// router, so the router scores the latent: z = bf16(x W_in^T) (the same z the
// layer computes), then logits[t,e] = z_t . W_r[e] as one fp32 dot product in
// ascending K order, not rounded (the router's top-k decides on these fp32
// values).  w_in == NULL: x already holds z [T,l].  z_out (optional) receives
// z [T,l] as bf16.
void lmoe_oracle_router_logits(int64_t T, int32_t d, int32_t l, int32_t E, const uint16_t* x,
                               const uint16_t* w_in, const uint16_t* w_r, float* logits, uint16_t* z_out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    std::vector<float> xv(w_in ? d : l), z(l), wrow(std::max(d, l));
    if (w_in) {
      bf16_row(x + t * d, xv.data(), d);
      for (int64_t i = 0; i < l; ++i) {
        bf16_row(w_in + i * d, wrow.data(), d);
        z[i] = bf16_round(dot(xv.data(), wrow.data(), d));
      }
    } else {
      bf16_row(x + t * l, z.data(), l);
    }
    if (z_out) for (int64_t i = 0; i < l; ++i) z_out[t * l + i] = to_bf16(z[i]);
    for (int64_t e = 0; e < E; ++e) {
      bf16_row(w_r + e * l, wrow.data(), l);
      logits[t * E + e] = dot(z.data(), wrow.data(), l);
    }
  }
}

// ------------------------------------------------------------------ permute
// The per-expert grouping that a grouped-GEMM MoE builds ([TS-K3] "Gluon
// kernels on AMD GPUs > Stable LatentMoE" names it: route sorting and gather
// buffers).  Stable counting sort of rows r = 0..R-1 by ids[r]:
// offsets[e] = number of rows with expert < e (E+1 entries);
// sorted_row[p] = r (p-th row in expert-major, row-ascending order);
// row_pos[r] = p (the inverse).
// Returns 0, or 1 (nothing written) if an id lies outside [0, E).
int lmoe_oracle_permute(int64_t R, int32_t E, const int32_t* ids, int32_t* offsets,
                        int32_t* sorted_row, int32_t* row_pos) {
  for (int64_t r = 0; r < R; ++r)
    if (ids[r] < 0 || ids[r] >= E) return 1;
  std::vector<int64_t> count(E, 0);
  for (int64_t r = 0; r < R; ++r) count[ids[r]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = int32_t(offsets[e] + count[e]);
  std::vector<int64_t> cursor(offsets, offsets + E);
  for (int64_t r = 0; r < R; ++r) {
    int64_t p = cursor[ids[r]]++;
    sorted_row[p] = int32_t(r);
    row_pos[r] = int32_t(p);
  }
  return 0;
}

// -------------------------------------------------------------------- layer
struct lmoe_oracle_args {
  int64_t T;
  int32_t E, k, d, l, I, S, Is;
  int32_t mxfp4;       // routed expert weights in MXFP4 (codes + e8m0 scales)
  int32_t act_quant;   // with mxfp4: quantise expert-GEMM activations to MXFP8 (w4a8)
  float eps;
  const uint16_t* x;       // [T,d] bf16; rows mode: [T,l]
  const uint16_t* w_in;    // [l,d]; NULL = rows mode
  const uint16_t* w_out;   // [d,l]; NULL = rows mode
  const uint16_t* norm_w;  // [l] RMSNorm gain; NULL = no norm
  const uint16_t* ws1;     // [S,Is,d]
  const uint16_t* ws3;     // [S,Is,d]
  const uint16_t* ws2;     // [S,d,Is]
  const void* w1;          // [E,I,l] bf16 | [E,I,l/2] packed e2m1
  const void* w3;          // [E,I,l]      | [E,I,l/2]
  const void* w2;          // [E,l,I]      | [E,l,I/2]
  const uint8_t* s1;       // [E,I,l/32] e8m0 (mxfp4 only)
  const uint8_t* s3;
  const uint8_t* s2;       // [E,l,I/32]
  const int32_t* ids;      // [T,k] routed expert ids
  const float* wts;        // [T,k] combine weights
  const int32_t* row_pos;  // [T*k] row -> sorted position; only used to lay out H/Y
  int64_t n_eval;          // number of tokens to evaluate
  const int64_t* eval_tokens;  // which tokens; NULL = all T (then n_eval is ignored)
  uint16_t* y;             // [n_eval or T, d] bf16; rows mode: [.., l]
  // Optional intermediates.  All tokens (eval_tokens == NULL): z, hs, rhat
  // and zq/zqs by token, H, Y and hq/hqs by sorted position (needs row_pos).
  // Sampled tokens: row i of z, hs, rhat, zq, zqs belongs to eval_tokens[i],
  // and row i*k + j of H, Y, hq, hqs to its slot j.
  uint16_t* z;             // [.., l]     latent (rows mode: the given rows)
  uint16_t* hs;            // [.., S*Is]  shared experts' SwiGLU output
  uint16_t* rhat;          // [.., l]     combined routed latent after the norm
  uint16_t* H;             // [.., I]     routed SwiGLU output (bf16, before any requantisation)
  uint16_t* Y;             // [.., l]     routed expert output
  int32_t korder;          // 0: every K reduction in ascending order; 1: descending
  uint8_t* zq;             // w4a8: MXFP8 codes [.., l] and e8m0 scales [.., l/32] of FC1's input
  uint8_t* zqs;
  uint8_t* hq;             // w4a8: MXFP8 codes [.., I] and scales [.., I/32] of FC2's input
  uint8_t* hqs;
};

// One token of the LatentMoE layer ([vLLM-K3] section 1 dataflow):
//  z    = bf16(x W_in^T)                       latent down-projection
//  H_j  = bf16(silu(z W1_e^T) * (z W3_e^T))    routed expert e = ids[t,j] (SwiGLU)
//  Y_j  = bf16(H_j W2_e^T)                     still in the latent
//  c    = sum_j w[t,j] * Y_j                   combine (fp32, j ascending)
//  rhat = bf16(c / sqrt(mean(c^2) + eps) * g)  routed-latent RMSNorm ([vLLM-K3]
//                                              section 6; skipped if no gain)
//  hs   = bf16(silu(x Ws1^T) * (x Ws3^T))      shared experts on the hidden state
//  y    = bf16(rhat W_out^T + hs Ws2^T)        up-projection plus shared output
// Rows mode (expert-parallel share, no projections, k = 1):
//  y[r] = bf16(w[r] * Y_r) with z = x.
// oi: the row of the token-indexed intermediates (t, or the index into
// eval_tokens); sampled: H/Y rows go to oi*k + j instead of row_pos[r].
static void one_token(const lmoe_oracle_args& a, int64_t t, int64_t oi, bool sampled, uint16_t* y_row) {
  const bool rows = (a.w_in == nullptr);
  const int64_t d = a.d, l = a.l, I = a.I, Is = a.Is;
  const bool aq = a.mxfp4 && a.act_quant;
  const bool rev = a.korder != 0;
  std::vector<float> xv(rows ? l : d), z(l), wrow(std::max<int64_t>(std::max(d, l), std::max(I, Is)));

  // latent down-projection
  if (rows) {
    bf16_row(a.x + t * l, z.data(), l);
  } else {
    bf16_row(a.x + t * d, xv.data(), d);
    for (int64_t i = 0; i < l; ++i) {
      bf16_row(a.w_in + i * d, wrow.data(), d);
      z[i] = bf16_round(dot(xv.data(), wrow.data(), d, rev));
    }
  }
  if (a.z) for (int64_t i = 0; i < l; ++i) a.z[oi * l + i] = to_bf16(z[i]);

  // routed experts in the latent, then the weighted combine
  std::vector<float> zin(z), h(I), hin(I), yv(l), c(l, 0.0f);
  if (aq) mxfp8_row(zin.data(), l, a.zq ? a.zq + oi * l : nullptr, a.zqs ? a.zqs + oi * (l / 32) : nullptr);
  for (int32_t j = 0; j < a.k; ++j) {
    const int64_t r = t * a.k + j;
    const int64_t e = a.ids[r];
    for (int64_t n = 0; n < I; ++n) {
      weight_row(a.w1, a.s1, a.mxfp4, e * I + n, l, wrow.data());
      float g = dot(zin.data(), wrow.data(), l, rev);
      weight_row(a.w3, a.s3, a.mxfp4, e * I + n, l, wrow.data());
      float u = dot(zin.data(), wrow.data(), l, rev);
      h[n] = bf16_round(silu(g) * u);
    }
    // where this slot's H and Y rows are stored
    const int64_t p = sampled ? oi * a.k + j : (a.row_pos ? int64_t(a.row_pos[r]) : -1);
    hin = h;
    if (aq)
      mxfp8_row(hin.data(), I, (a.hq && p >= 0) ? a.hq + p * I : nullptr,
                (a.hqs && p >= 0) ? a.hqs + p * (I / 32) : nullptr);
    for (int64_t n = 0; n < l; ++n) {
      weight_row(a.w2, a.s2, a.mxfp4, e * l + n, I, wrow.data());
      yv[n] = bf16_round(dot(hin.data(), wrow.data(), I, rev));
    }
    if (p >= 0) {
      if (a.H) for (int64_t n = 0; n < I; ++n) a.H[p * I + n] = to_bf16(h[n]);
      if (a.Y) for (int64_t n = 0; n < l; ++n) a.Y[p * l + n] = to_bf16(yv[n]);
    }
    const float wj = a.wts[r];
    if (rows) {
      for (int64_t n = 0; n < l; ++n) y_row[n] = to_bf16(wj * yv[n]);
      return;
    }
    for (int64_t n = 0; n < l; ++n) c[n] += wj * yv[n];
  }

  // routed-latent RMSNorm
  std::vector<float> rh(l);
  if (a.norm_w) {
    float ss = 0.0f;
    if (rev) {
      for (int64_t n = l - 1; n >= 0; --n) ss += c[n] * c[n];
    } else {
      for (int64_t n = 0; n < l; ++n) ss += c[n] * c[n];
    }
    const float inv = 1.0f / std::sqrt(ss / float(l) + a.eps);
    for (int64_t n = 0; n < l; ++n) rh[n] = bf16_round(c[n] * inv * from_bf16(a.norm_w[n]));
  } else {
    for (int64_t n = 0; n < l; ++n) rh[n] = bf16_round(c[n]);
  }
  if (a.rhat) for (int64_t n = 0; n < l; ++n) a.rhat[oi * l + n] = to_bf16(rh[n]);

  // shared experts on the hidden state (intermediates of all S concatenated)
  std::vector<float> hsv(int64_t(a.S) * Is);
  for (int32_t s = 0; s < a.S; ++s) {
    for (int64_t n = 0; n < Is; ++n) {
      bf16_row(a.ws1 + (int64_t(s) * Is + n) * d, wrow.data(), d);
      float g = dot(xv.data(), wrow.data(), d, rev);
      bf16_row(a.ws3 + (int64_t(s) * Is + n) * d, wrow.data(), d);
      float u = dot(xv.data(), wrow.data(), d, rev);
      hsv[int64_t(s) * Is + n] = bf16_round(silu(g) * u);
    }
  }
  if (a.hs) for (int64_t i = 0; i < int64_t(a.S) * Is; ++i) a.hs[oi * a.S * Is + i] = to_bf16(hsv[i]);

  // latent up-projection plus the shared experts' down-projection, one fp32
  // accumulator per output over the concatenated K = l + S*Is: latent terms
  // first, then the shared experts in order (rev: the exact reverse)
  std::vector<float> wo(l), w2s(int64_t(a.S) * Is);
  for (int64_t o = 0; o < d; ++o) {
    bf16_row(a.w_out + o * l, wo.data(), l);
    for (int32_t s = 0; s < a.S; ++s) bf16_row(a.ws2 + (int64_t(s) * d + o) * Is, w2s.data() + int64_t(s) * Is, Is);
    float acc = 0.0f;
    if (rev) {
      for (int64_t i = int64_t(a.S) * Is - 1; i >= 0; --i) acc += hsv[i] * w2s[i];
      for (int64_t i = l - 1; i >= 0; --i) acc += rh[i] * wo[i];
    } else {
      for (int64_t i = 0; i < l; ++i) acc += rh[i] * wo[i];
      for (int64_t i = 0; i < int64_t(a.S) * Is; ++i) acc += hsv[i] * w2s[i];
    }
    y_row[o] = to_bf16(acc);
  }
}

// Returns 0 on success, 1 on invalid arguments.
int lmoe_oracle_layer(const lmoe_oracle_args* a) {
  if (!a || !a->x || !a->ids || !a->wts || !a->y || !a->w1 || !a->w3 || !a->w2) return 1;
  const bool rows = (a->w_in == nullptr);
  if (rows != (a->w_out == nullptr)) return 1;
  if (rows && (a->k != 1 || a->S != 0)) return 1;
  if (a->mxfp4 && (!a->s1 || !a->s3 || !a->s2 || a->l % 32 || a->I % 32)) return 1;
  if (a->S > 0 && (!a->ws1 || !a->ws3 || !a->ws2)) return 1;
  for (int64_t r = 0; r < a->T * a->k; ++r)
    if (a->ids[r] < 0 || a->ids[r] >= a->E) return 1;
  const bool sampled = a->eval_tokens != nullptr;
  const int64_t n = sampled ? a->n_eval : a->T;
  const int64_t ow = rows ? a->l : a->d;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = sampled ? a->eval_tokens[i] : i;
    one_token(*a, t, i, sampled, a->y + i * ow);
  }
  return 0;
}

}  // extern "C"
