// oracle.cpp -- plain, slow, obviously-correct CPU oracle of the decode hot path.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
// CPU-baseline leg may load this library.  It shares no code, header or table
// with the GPU library; the only thing both sides consume is the canonical block
// bytes written by the seeded input generator.
//
// Conventions
//   * Weights are decoded from the canonical GGUF-style block bytes.  The formats
//     (Q4_0, Q8_0, Q4_K, Q5_K, Q6_K with their block sizes and bits/weight) are the
//     ones in the quantization-format table of the page "Show HN: NVMe経由でCPUを
//     バイパスして単一のRTX 3090上で動作するLlama 3.1 70B"; the byte layouts inside a
//     block are GGUF's published ones, which those pages name but do not print.
//   * A dequantized weight is the fp32 value nearest (ties to even) to its exact
//     value.  Every format's exact value is an integer multiple of 2^-24 (an fp16
//     number is an integer times 2^-24, subnormals included), so the oracle forms
//     that integer in int64 and rounds once.
//   * Everything else is evaluated in fp64 with plain sequential sums.  OpenMP is
//     used only across independent output rows, so results never depend on the
//     number of threads.
//   * The model is the Llama decoder the NTransformer page lists under its key
//     features ("Llama architecture: RoPE, GQA, SwiGLU, RMSNorm, KV cache"); the
//     pages give no formulas, so each function states the standard definition it
//     writes out.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum { QT_F32 = 0, QT_F16 = 1, QT_Q4_0 = 2, QT_Q8_0 = 8, QT_Q4_K = 12, QT_Q5_K = 13, QT_Q6_K = 14 };

// IEEE binary16 -> double, exactly (subnormals honoured).
double half_value(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

bool half_finite(uint16_t h) { return ((h >> 10) & 31) != 31; }

// A finite fp16 value times 2^24, as an exact integer.
int64_t half_times_2p24(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  int64_t v = (e == 0) ? (int64_t)m : ((int64_t)(1024 + m) << (e - 1));
  return sign ? -v : v;
}

uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int block_weights(int qt) {
  switch (qt) {
    case QT_Q8_0: case QT_Q4_0: return 32;
    case QT_Q4_K: case QT_Q5_K: case QT_Q6_K: return 256;
    default: return 0;
  }
}

int block_bytes(int qt) {
  switch (qt) {
    case QT_Q8_0: return 34;
    case QT_Q4_0: return 18;
    case QT_Q4_K: return 144;
    case QT_Q5_K: return 176;
    case QT_Q6_K: return 210;
    default: return 0;
  }
}

// fp32 nearest to N * 2^-24 (N is exact in a double because |N| < 2^53).
float from_units(int64_t n) { return (float)std::ldexp((double)n, -24); }

// The 6-bit scale and min of sub-block s (0..7) of a K-quant superblock, from the
// 12-byte packed field S: s < 4 keeps the low six bits of S[s] and S[s+4]; s >= 4
// joins the nibbles of S[s+4] with the top two bits of S[s-4] (scale) and S[s] (min).
void kquant_scale_min(const uint8_t* S, int s, int* sc, int* m) {
  if (s < 4) {
    *sc = S[s] & 63;
    *m = S[s + 4] & 63;
  } else {
    *sc = (S[s + 4] & 15) | ((S[s - 4] >> 6) << 4);
    *m = (S[s + 4] >> 4) | ((S[s] >> 6) << 4);
  }
}

// Quant of weight i (0..255) in a Q4_K superblock: within each group of 64 weights,
// byte t of the group's 32 bytes holds weight t in its low nibble and t+32 in its high one.
int q4k_quant(const uint8_t* qs, int i) {
  const int c = i / 64, t = i % 64;
  return t < 32 ? (qs[32 * c + t] & 15) : (qs[32 * c + t - 32] >> 4);
}

// Quant of weight i in a Q5_K superblock: the Q4_K nibble plus a fifth bit from qh.
int q5k_quant(const uint8_t* qh, const uint8_t* qs, int i) {
  const int c = i / 64, t = i % 64;
  if (t < 32) return (qs[32 * c + t] & 15) + 16 * ((qh[t] >> (2 * c)) & 1);
  return (qs[32 * c + t - 32] >> 4) + 16 * ((qh[t - 32] >> (2 * c + 1)) & 1);
}

// Unsigned 6-bit quant of weight i in a Q6_K superblock (before the -32 offset).
int q6k_quant(const uint8_t* ql, const uint8_t* qh, int i) {
  const int n = i / 128, r = i % 128, u = r / 32, l = r % 32;
  const uint8_t byte = ql[64 * n + l + 32 * (u & 1)];
  const int nib = (u < 2) ? (byte & 15) : (byte >> 4);
  const int hi2 = (qh[32 * n + l] >> (2 * u)) & 3;
  return nib | (hi2 << 4);
}

// Dequantize one block into w[0 .. block_weights).
void dequant_block(int qt, const uint8_t* b, float* w) {
  switch (qt) {
    case QT_Q8_0: {  // w_i = d * q_i
      const uint16_t d = rd16(b);
      for (int i = 0; i < 32; ++i) {
        const int q = (int8_t)b[2 + i];
        w[i] = half_finite(d) ? from_units(half_times_2p24(d) * q) : (float)(half_value(d) * q);
      }
      break;
    }
    case QT_Q4_0: {  // w_i = d * (q_i - 8), q_i the nibble (low: i < 16, high: i >= 16)
      const uint16_t d = rd16(b);
      for (int i = 0; i < 32; ++i) {
        const int q = (i < 16) ? (b[2 + i] & 15) : (b[2 + i - 16] >> 4);
        w[i] = half_finite(d) ? from_units(half_times_2p24(d) * (q - 8)) : (float)(half_value(d) * (q - 8));
      }
      break;
    }
    case QT_Q4_K:
    case QT_Q5_K: {  // w_i = d * sc_s * q_i - dmin * m_s, s = i / 32
      const uint16_t d = rd16(b), dmin = rd16(b + 2);
      const uint8_t* S = b + 4;
      for (int i = 0; i < 256; ++i) {
        int sc, m;
        kquant_scale_min(S, i / 32, &sc, &m);
        const int q = (qt == QT_Q4_K) ? q4k_quant(b + 16, i) : q5k_quant(b + 16, b + 48, i);
        if (half_finite(d) && half_finite(dmin))
          w[i] = from_units(half_times_2p24(d) * sc * q - half_times_2p24(dmin) * m);
        else
          w[i] = (float)(half_value(d) * sc * q - half_value(dmin) * m);
      }
      break;
    }
    case QT_Q6_K: {  // w_i = d * sc[i / 16] * (q_i - 32)
      const uint8_t *ql = b, *qh = b + 128;
      const int8_t* sc = (const int8_t*)(b + 192);
      const uint16_t d = rd16(b + 208);
      for (int i = 0; i < 256; ++i) {
        const int q = q6k_quant(ql, qh, i) - 32;
        const int s = sc[i / 16];
        w[i] = half_finite(d) ? from_units(half_times_2p24(d) * s * q) : (float)(half_value(d) * s * q);
      }
      break;
    }
    default: break;
  }
}

void dequant_row(int qt, const uint8_t* row, int64_t k, float* w) {
  const int B = block_weights(qt), BB = block_bytes(qt);
  for (int64_t b = 0; b < k / B; ++b) dequant_block(qt, row + b * BB, w + b * B);
}

bool valid_matrix(int qt, int64_t k) {
  const int B = block_weights(qt);
  return B > 0 && k > 0 && k % B == 0;
}

// y[j*rows + r] = sum_c w[r][c] * x[j*k + c] (fp64, sequential in c); a = sum |w x|.
void gemv_cols(int qt, const uint8_t* W, int64_t rows, int64_t k, const double* x, int ncols, double* y, double* a) {
  const size_t rb = (size_t)(k / block_weights(qt)) * block_bytes(qt);
#pragma omp parallel
  {
    std::vector<float> w(k);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      dequant_row(qt, W + (size_t)r * rb, k, w.data());
      for (int j = 0; j < ncols; ++j) {
        const double* xj = x + (size_t)j * k;
        double s = 0.0, sa = 0.0;
        for (int64_t c = 0; c < k; ++c) {
          const double p = (double)w[c] * xj[c];
          s += p;
          sa += std::fabs(p);
        }
        y[(size_t)j * rows + r] = s;
        if (a) a[(size_t)j * rows + r] = sa;
      }
    }
  }
}

// RMSNorm: out_i = g_i * x_i / sqrt(mean(x^2) + eps).
void rmsnorm(const double* x, const float* g, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  const double inv = 1.0 / std::sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = (double)g[i] * (x[i] * inv);
}

// RoPE on adjacent pairs (2i, 2i+1) of every head at position pos:
// theta_i = base^(-2i/hd), phi = pos * theta_i, (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi).
void rope(double* v, int n_heads, int hd, int64_t pos, double base) {
  for (int h = 0; h < n_heads; ++h) {
    double* p = v + (size_t)h * hd;
    for (int i = 0; i < hd / 2; ++i) {
      const double th = std::pow(base, -2.0 * i / (double)hd);
      const double phi = (double)pos * th;
      const double c = std::cos(phi), s = std::sin(phi);
      const double a = p[2 * i], b = p[2 * i + 1];
      p[2 * i] = a * c - b * s;
      p[2 * i + 1] = a * s + b * c;
    }
  }
}

// double -> fp16 bits, rounding through fp32 first (the precision the GPU path holds the
// value in before it stores the cache entry), then to nearest-even fp16, overflow -> inf.
uint16_t half_from_double_via_f32(double v) {
  const float f = (float)v;
  const double a = std::fabs((double)f);
  const uint16_t sign = std::signbit(f) ? 0x8000 : 0;
  if (std::isnan(f)) return 0x7E00;
  if (std::isinf(a)) return sign | 0x7C00;
  if (a < std::ldexp(1.0, -14)) return sign | (uint16_t)std::nearbyint(std::ldexp(a, 24));
  int e;
  std::frexp(a, &e);
  e -= 1;
  double m = std::nearbyint(std::ldexp(a, 10 - e));
  if (m >= 2048.0) { m = 1024.0; e += 1; }
  if (e > 15) return sign | 0x7C00;
  return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

// Grouped-query decode attention for one token.  q: [nq][hd]; K,V caches [ctx][nkv][hd]
// fp16; positions 0 .. n_pos-1 are visible.  Query head h reads kv head h / (nq / nkv).
void attention(const double* q, const uint16_t* kc, const uint16_t* vc, int64_t n_pos, int nq, int nkv, int hd,
               double* out) {
  const int group = nq / nkv;
  std::vector<double> s(n_pos);
  const double scale = 1.0 / std::sqrt((double)hd);
  for (int h = 0; h < nq; ++h) {
    const int g = h / group;
    const double* qh = q + (size_t)h * hd;
    double mx = -INFINITY;
    for (int64_t t = 0; t < n_pos; ++t) {
      const uint16_t* kt = kc + ((size_t)t * nkv + g) * hd;
      double dot = 0.0;
      for (int d = 0; d < hd; ++d) dot += qh[d] * half_value(kt[d]);
      s[t] = dot * scale;
      mx = std::max(mx, s[t]);
    }
    double den = 0.0;
    for (int64_t t = 0; t < n_pos; ++t) {
      s[t] = std::exp(s[t] - mx);
      den += s[t];
    }
    double* oh = out + (size_t)h * hd;
    for (int d = 0; d < hd; ++d) oh[d] = 0.0;
    for (int64_t t = 0; t < n_pos; ++t) {
      const double p = s[t] / den;
      const uint16_t* vt = vc + ((size_t)t * nkv + g) * hd;
      for (int d = 0; d < hd; ++d) oh[d] += p * half_value(vt[d]);
    }
  }
}

// silu(z) = z / (1 + e^-z); for very negative z, e^-z = inf and the quotient is -0, never NaN.
double silu(double z) { return z / (1.0 + std::exp(-z)); }

double cosine(const double* a, const double* b, int64_t n) {
  double ab = 0.0, aa = 0.0, bb = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    ab += a[i] * b[i];
    aa += a[i] * a[i];
    bb += b[i] * b[i];
  }
  if (aa == 0.0 || bb == 0.0) return 0.0;
  return ab / (std::sqrt(aa) * std::sqrt(bb));
}

// Greedy choice on the logits as the GPU holds them (fp32); ties go to the lowest index.
int64_t argmax_f32(const double* x, int64_t n) {
  int64_t best = 0;
  float bv = (float)x[0];
  for (int64_t i = 1; i < n; ++i) {
    const float v = (float)x[i];
    if (v > bv || (std::isnan(v) && !std::isnan(bv))) { bv = v; best = i; }
  }
  return best;
}

}  // namespace

extern "C" {

struct orc_dims {
  int32_t n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab, max_ctx;
  double rope_theta, rms_eps;
};

// tensor order inside a layer: WQ, WK, WV, WO, WGATE, WUP, WDOWN
struct orc_layer {
  const uint8_t* w[7];
  int32_t qt[7];
  const float* g_attn;
  const float* g_ffn;
  uint16_t* kc;  // [max_ctx][n_kv][head_dim] fp16 bits
  uint16_t* vc;
};

struct orc_model {
  orc_dims dims;
  const orc_layer* layers;
  const uint8_t* embed;
  int32_t qt_embed;
  const uint8_t* head;
  int32_t qt_head;
  const float* g_final;
};

int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// Threads of the row loops from here on (for timing the oracle at 1 thread and at all threads; the
// results do not depend on it).  Returns the previous count.
int orc_set_threads(int n) {
#ifdef _OPENMP
  const int prev = omp_get_max_threads();
  if (n > 0) omp_set_num_threads(n);
  return prev;
#else
  (void)n;
  return 1;
#endif
}

int orc_block_weights(int qt) { return block_weights(qt); }
int orc_block_bytes(int qt) { return block_bytes(qt); }
double orc_half_value(uint16_t h) { return half_value(h); }
uint16_t orc_half_from_double(double v) { return half_from_double_via_f32(v); }

// Dequantize rows x k canonical bytes into fp32 (row-major).
int orc_dequant(int qt, const uint8_t* W, int64_t rows, int64_t k, float* out) {
  if (!valid_matrix(qt, k) || rows < 0) return -1;
  const size_t rb = (size_t)(k / block_weights(qt)) * block_bytes(qt);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) dequant_row(qt, W + (size_t)r * rb, k, out + (size_t)r * k);
  return 0;
}

// Y[j][r] = sum_c W[r][c] X[j][c], A[j][r] = sum_c |W[r][c] X[j][c]|, j < ncols.
int orc_gemv(int qt, const uint8_t* W, int64_t rows, int64_t k, const double* X, int ncols, double* Y, double* A) {
  if (!valid_matrix(qt, k) || rows < 0 || ncols < 1) return -1;
  gemv_cols(qt, W, rows, k, X, ncols, Y, A);
  return 0;
}

void orc_rmsnorm(const double* x, const float* g, int64_t n, double eps, double* out) { rmsnorm(x, g, n, eps, out); }
void orc_rope(double* v, int n_heads, int hd, int64_t pos, double base) { rope(v, n_heads, hd, pos, base); }
void orc_attention(const double* q, const uint16_t* kc, const uint16_t* vc, int64_t n_pos, int nq, int nkv, int hd,
                   double* out) {
  attention(q, kc, vc, n_pos, nq, nkv, hd, out);
}
double orc_silu(double z) { return silu(z); }
void orc_swiglu(const double* g, const double* u, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu(g[i]) * u[i];
}
double orc_cosine(const double* a, const double* b, int64_t n) { return cosine(a, b, n); }
int64_t orc_argmax_f32(const double* x, int64_t n) { return argmax_f32(x, n); }

// One pre-norm Llama decoder layer for the token at position pos; h is updated in place
// and the token's K and V rows are written (as fp16) at cache row pos.
//   n1 = RMSNorm(h; g_attn); q, k, v = Wq n1, Wk n1, Wv n1; RoPE(q), RoPE(k) at pos
//   h += Wo . attention(q, K[0..pos], V[0..pos])
//   n2 = RMSNorm(h; g_ffn); h += Wdown . (silu(Wgate n2) * (Wup n2))
int orc_layer_forward(const orc_dims* D, const orc_layer* L, double* h, int64_t pos) {
  const int H = D->hidden, hd = D->head_dim, nq = D->n_q, nkv = D->n_kv, F = D->ffn;
  if (pos < 0 || pos >= D->max_ctx || nq % nkv != 0) return -1;
  std::vector<double> n1(H), q((size_t)nq * hd), kk((size_t)nkv * hd), vv((size_t)nkv * hd), o((size_t)nq * hd);
  std::vector<double> y(H), n2(H), g(F), u(F), act(F);
  rmsnorm(h, L->g_attn, H, D->rms_eps, n1.data());
  gemv_cols(L->qt[0], L->w[0], (int64_t)nq * hd, H, n1.data(), 1, q.data(), nullptr);
  gemv_cols(L->qt[1], L->w[1], (int64_t)nkv * hd, H, n1.data(), 1, kk.data(), nullptr);
  gemv_cols(L->qt[2], L->w[2], (int64_t)nkv * hd, H, n1.data(), 1, vv.data(), nullptr);
  rope(q.data(), nq, hd, pos, D->rope_theta);
  rope(kk.data(), nkv, hd, pos, D->rope_theta);
  for (int i = 0; i < nkv * hd; ++i) {
    L->kc[(size_t)pos * nkv * hd + i] = half_from_double_via_f32(kk[i]);
    L->vc[(size_t)pos * nkv * hd + i] = half_from_double_via_f32(vv[i]);
  }
  attention(q.data(), L->kc, L->vc, pos + 1, nq, nkv, hd, o.data());
  gemv_cols(L->qt[3], L->w[3], H, (int64_t)nq * hd, o.data(), 1, y.data(), nullptr);
  for (int i = 0; i < H; ++i) h[i] += y[i];
  rmsnorm(h, L->g_ffn, H, D->rms_eps, n2.data());
  gemv_cols(L->qt[4], L->w[4], F, H, n2.data(), 1, g.data(), nullptr);
  gemv_cols(L->qt[5], L->w[5], F, H, n2.data(), 1, u.data(), nullptr);
  for (int i = 0; i < F; ++i) act[i] = silu(g[i]) * u[i];
  gemv_cols(L->qt[6], L->w[6], H, F, act.data(), 1, y.data(), nullptr);
  for (int i = 0; i < H; ++i) h[i] += y[i];
  return 0;
}

// Final RMSNorm and output head: logits = Whead . RMSNorm(h; g_final).
int orc_head(const orc_model* M, const double* h, double* logits) {
  const orc_dims* D = &M->dims;
  std::vector<double> n(D->hidden);
  rmsnorm(h, M->g_final, D->hidden, D->rms_eps, n.data());
  gemv_cols(M->qt_head, M->head, D->vocab, D->hidden, n.data(), 1, logits, nullptr);
  return 0;
}

// One greedy decode step for `token` at position pos through layers 0 .. n_run-1:
//   h = dequant(embed[token]); per layer l: if skip[l], h is left unchanged and no K/V is
//   written; else the layer runs and cos[l] = cos(h_in, h_out).  Then logits = head(h) and
//   next = argmax(logits).  hidden (optional) receives h after the embedding and after each
//   layer: (n_layers + 1) x hidden.
int orc_step(const orc_model* M, int32_t token, int64_t pos, int32_t n_run, const uint8_t* skip, double* hidden,
             double* cos_out, double* logits, int32_t* next) {
  const orc_dims* D = &M->dims;
  const int H = D->hidden;
  if (token < 0 || token >= D->vocab || n_run < 0 || n_run > D->n_layers) return -1;
  std::vector<double> h(H), hin(H), lg(D->vocab);
  {
    std::vector<float> e(H);
    const size_t rb = (size_t)(H / block_weights(M->qt_embed)) * block_bytes(M->qt_embed);
    dequant_row(M->qt_embed, M->embed + (size_t)token * rb, H, e.data());
    for (int i = 0; i < H; ++i) h[i] = e[i];
  }
  if (hidden) std::copy(h.begin(), h.end(), hidden);
  for (int l = 0; l < D->n_layers; ++l) {
    const bool run = l < n_run && !(skip && skip[l]);
    if (run) {
      hin = h;
      if (orc_layer_forward(D, &M->layers[l], h.data(), pos) != 0) return -1;
      if (cos_out) cos_out[l] = cosine(hin.data(), h.data(), H);
    } else if (cos_out) {
      cos_out[l] = NAN;
    }
    if (hidden) std::copy(h.begin(), h.end(), hidden + (size_t)(l + 1) * H);
  }
  orc_head(M, h.data(), lg.data());
  if (logits) std::copy(lg.begin(), lg.end(), logits);
  if (next) *next = (int32_t)argmax_f32(lg.data(), D->vocab);
  return 0;
}

}  // extern "C"
