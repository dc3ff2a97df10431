/*
 * synth.c - seeded, counter-based generator of synthetic inputs.
 *
 * This module is shared input preparation: it draws random numbers and
 * writes them out in the canonical GGUF-style block byte layouts (the
 * interchange format both the CPU oracle and the GPU library read).  It
 * performs none of the method's arithmetic: no dequantization, no products,
 * no normalisation.  Both consumers decode the bytes with their own code.
 *
 * Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw(key, i) = mix64(key + (i + 1) * GOLDEN_GAMMA), so any
 * element of any tensor can be regenerated on its own (random access by
 * index), independent of thread count or of which rows are requested.
 *   - uniform integer in [lo, hi]: lo + ((u >> 32) * (hi - lo + 1)) >> 32
 *   - uniform real in (0, 1]: ((u >> 11) + 1) * 2^-53
 *   - standard normal: Box-Muller on draws 2i and 2i+1, in fp64
 *   - fp16: round-to-nearest-even from fp64, subnormals kept, overflow -> inf
 *
 * Block layouts written (little-endian; fp16 = IEEE binary16):
 *   Q8_0 (32 weights, 34 B): d, qs[32] int8
 *   Q4_0 (32 weights, 18 B): d, qs[16]; low nibble = weight j, high = j+16
 *   Q4_K (256 weights, 144 B): d, dmin, S[12] packed 6-bit scales/mins,
 *        qs[128]; in each 64-weight group low nibbles hold the first 32
 *   Q5_K (256 weights, 176 B): d, dmin, S[12], qh[32], qs[128]
 *   Q6_K (256 weights, 210 B): ql[128], qh[64], sc[16] int8, d
 * (Format list and bits/weight: Show HN NTransformer page, quantization
 * format table; byte layouts are GGUF's published block layouts.)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

enum { SYN_F32 = 0, SYN_F16 = 1, SYN_Q4_0 = 2, SYN_Q8_0 = 8, SYN_Q4_K = 12, SYN_Q5_K = 13, SYN_Q6_K = 14 };

/* field identifiers inside one tensor's key space */
enum { FLD_Q = 0, FLD_SC = 1, FLD_M = 2, FLD_D = 3, FLD_DMIN = 4 };

typedef struct {
  int32_t qtype;
  int32_t q_lo, q_hi;   /* quant value range (as stored, before any offset) */
  int32_t sc_lo, sc_hi; /* sub-block scale range */
  int32_t m_lo, m_hi;   /* sub-block min range (Q4_K / Q5_K) */
  double d_sigma;       /* d = fp16(|N(0,1)| * d_sigma * d_mult) */
  double dmin_sigma;    /* dmin = fp16(|N(0,1)| * dmin_sigma * d_mult) */
  double d_mult;        /* extra factor applied before fp16 rounding */
} syn_qparams;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN_GAMMA); }

static inline int64_t uni_int(uint64_t u, int64_t lo, int64_t hi) {
  return lo + (int64_t)(((u >> 32) * (uint64_t)(hi - lo + 1)) >> 32);
}

static inline double uni_open0(uint64_t u) { return (double)((u >> 11) + 1) * 0x1p-53; }

static inline double normal_at(uint64_t key, uint64_t i) {
  double u1 = uni_open0(draw(key, 2 * i));
  double u2 = uni_open0(draw(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
}

static inline uint64_t field_key(uint64_t base, int field) {
  return mix64(base + (uint64_t)(field + 1) * 0xD1B54A32D192ED03ULL);
}

/* Key of one tensor stream, from the seed and a 64-bit stream identifier. */
uint64_t syn_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN_GAMMA) ^ mix64(stream * GOLDEN_GAMMA + 0x2545F4914F6CDD1DULL));
}

uint64_t syn_draw(uint64_t key, uint64_t i) { return draw(key, i); }

/* fp64 -> IEEE binary16 bits, round to nearest even, subnormals kept. */
uint16_t syn_f16_bits(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00;
  if (isinf(a)) return sign | 0x7C00;
  if (a < 0x1p-14) {
    /* subnormal range: value = m * 2^-24, m in [0, 1024] (1024 becomes the smallest normal) */
    double m = rint(a * 0x1p24);
    return sign | (uint16_t)m;
  }
  int e;
  (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) -> a = 1.x * 2^(e-1) */
  e -= 1;
  double m = rint(ldexp(a, 10 - e)); /* in [1024, 2048] */
  if (m >= 2048.0) { m = 1024.0; e += 1; }
  if (e > 15) return sign | 0x7C00;
  return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

static inline void put_f16(uint8_t* p, uint16_t b) { p[0] = (uint8_t)(b & 0xFF); p[1] = (uint8_t)(b >> 8); }

int syn_block_weights(int qtype) {
  switch (qtype) {
    case SYN_Q8_0: case SYN_Q4_0: return 32;
    case SYN_Q4_K: case SYN_Q5_K: case SYN_Q6_K: return 256;
    case SYN_F32: case SYN_F16: return 1;
    default: return 0;
  }
}

int syn_block_bytes(int qtype) {
  switch (qtype) {
    case SYN_Q8_0: return 34;
    case SYN_Q4_0: return 18;
    case SYN_Q4_K: return 144;
    case SYN_Q5_K: return 176;
    case SYN_Q6_K: return 210;
    case SYN_F32: return 4;
    case SYN_F16: return 2;
    default: return 0;
  }
}

static uint16_t draw_scale(uint64_t key, uint64_t idx, double sigma, double mult) {
  return syn_f16_bits(fabs(normal_at(key, idx)) * sigma * mult);
}

/* Pack 8 six-bit scales and 8 six-bit mins into the 12-byte K-quant field. */
static void pack_scales12(const int sc[8], const int m[8], uint8_t S[12]) {
  for (int s = 0; s < 4; ++s) {
    S[s] = (uint8_t)((sc[s] & 63) | ((sc[s + 4] >> 4) << 6));
    S[s + 4] = (uint8_t)((m[s] & 63) | ((m[s + 4] >> 4) << 6));
    S[8 + s] = (uint8_t)((sc[4 + s] & 15) | ((m[4 + s] & 15) << 4));
  }
}

/* One block (index b within row r of a rows x k matrix) written at out. */
static void gen_block(const syn_qparams* p, uint64_t kq, uint64_t ksc, uint64_t km, uint64_t kd, uint64_t kdm,
                      int64_t k, int64_t r, int64_t b, uint8_t* out) {
  const int qt = p->qtype;
  const int B = syn_block_weights(qt);
  const uint64_t w0 = (uint64_t)r * (uint64_t)k + (uint64_t)b * (uint64_t)B; /* global weight index */
  const uint64_t blk = (uint64_t)r * (uint64_t)(k / B) + (uint64_t)b;        /* global block index */
  int q[256];
  for (int i = 0; i < B; ++i) q[i] = (int)uni_int(draw(kq, w0 + i), p->q_lo, p->q_hi);
  switch (qt) {
    case SYN_Q8_0: {
      put_f16(out, draw_scale(kd, blk, p->d_sigma, p->d_mult));
      for (int i = 0; i < 32; ++i) out[2 + i] = (uint8_t)(int8_t)q[i];
      break;
    }
    case SYN_Q4_0: {
      put_f16(out, draw_scale(kd, blk, p->d_sigma, p->d_mult));
      for (int j = 0; j < 16; ++j) out[2 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
      break;
    }
    case SYN_Q4_K:
    case SYN_Q5_K: {
      int sc[8], m[8];
      for (int s = 0; s < 8; ++s) {
        sc[s] = (int)uni_int(draw(ksc, blk * 8 + s), p->sc_lo, p->sc_hi);
        m[s] = (int)uni_int(draw(km, blk * 8 + s), p->m_lo, p->m_hi);
      }
      put_f16(out, draw_scale(kd, blk, p->d_sigma, p->d_mult));
      put_f16(out + 2, draw_scale(kdm, blk, p->dmin_sigma, p->d_mult));
      pack_scales12(sc, m, out + 4);
      uint8_t* qs = out + (qt == SYN_Q4_K ? 16 : 48);
      for (int c = 0; c < 4; ++c)
        for (int t = 0; t < 32; ++t)
          qs[32 * c + t] = (uint8_t)((q[64 * c + t] & 15) | ((q[64 * c + 32 + t] & 15) << 4));
      if (qt == SYN_Q5_K) {
        uint8_t* qh = out + 16;
        for (int t = 0; t < 32; ++t) {
          int v = 0;
          for (int c = 0; c < 4; ++c) {
            v |= ((q[64 * c + t] >> 4) & 1) << (2 * c);
            v |= ((q[64 * c + 32 + t] >> 4) & 1) << (2 * c + 1);
          }
          qh[t] = (uint8_t)v;
        }
      }
      break;
    }
    case SYN_Q6_K: {
      uint8_t* ql = out;
      uint8_t* qh = out + 128;
      int8_t* sc = (int8_t*)(out + 192);
      for (int n = 0; n < 2; ++n)
        for (int l = 0; l < 32; ++l) {
          int i0 = 128 * n + l, i1 = i0 + 32, i2 = i0 + 64, i3 = i0 + 96;
          ql[64 * n + l] = (uint8_t)((q[i0] & 15) | ((q[i2] & 15) << 4));
          ql[64 * n + l + 32] = (uint8_t)((q[i1] & 15) | ((q[i3] & 15) << 4));
          qh[32 * n + l] = (uint8_t)(((q[i0] >> 4) & 3) | (((q[i1] >> 4) & 3) << 2) | (((q[i2] >> 4) & 3) << 4) |
                                     (((q[i3] >> 4) & 3) << 6));
        }
      for (int j = 0; j < 16; ++j) sc[j] = (int8_t)uni_int(draw(ksc, blk * 16 + j), p->sc_lo, p->sc_hi);
      put_f16(out + 208, draw_scale(kd, blk, p->d_sigma, p->d_mult));
      break;
    }
    default: break;
  }
}

/*
 * Canonical bytes of rows [r0, r0+nr) of a rows x k matrix (row-major, each
 * row k/B consecutive blocks).  Returns 0, or -1 on a bad qtype / k.
 */
int syn_matrix(const syn_qparams* p, uint64_t key, int64_t k, int64_t r0, int64_t nr, uint8_t* out) {
  const int B = syn_block_weights(p->qtype);
  const int BB = syn_block_bytes(p->qtype);
  if (B <= 1 || k <= 0 || k % B != 0 || nr < 0 || r0 < 0) return -1;
  const int64_t nb = k / B;
  const uint64_t kq = field_key(key, FLD_Q), ksc = field_key(key, FLD_SC), km = field_key(key, FLD_M);
  const uint64_t kd = field_key(key, FLD_D), kdm = field_key(key, FLD_DMIN);
  const int64_t total = nr * nb;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < total; ++t) {
    int64_t rr = t / nb, b = t % nb;
    gen_block(p, kq, ksc, km, kd, kdm, k, r0 + rr, b, out + (size_t)t * BB);
  }
  return 0;
}

/* out[i] = (float)(mean + sigma * N_{i0+i}) */
void syn_normal_f32(uint64_t key, int64_t i0, int64_t n, double mean, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + sigma * normal_at(key, (uint64_t)(i0 + i)));
}

/* out[i] = fp16(mean + sigma * N_{i0+i}) as raw bits */
void syn_normal_f16(uint64_t key, int64_t i0, int64_t n, double mean, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = syn_f16_bits(mean + sigma * normal_at(key, (uint64_t)(i0 + i)));
}

/* uniform integer in [lo, hi] at counter i */
int64_t syn_uniform_int(uint64_t key, int64_t i, int64_t lo, int64_t hi) { return uni_int(draw(key, (uint64_t)i), lo, hi); }

/*
 * The raw drawn fields of block b of row r (before packing): q[B] as stored (unsigned
 * 4/5/6-bit, or signed int8 for Q8_0), sc[] and m[] per sub-block (8 for Q4_K/Q5_K,
 * 16 for Q6_K), and the fp16 bits of d and dmin.  Used by tests to check that a
 * decoder recovers exactly the values that were packed.
 */
int syn_block_fields(const syn_qparams* p, uint64_t key, int64_t k, int64_t r, int64_t b, int32_t* q, int32_t* sc,
                     int32_t* m, uint16_t* d, uint16_t* dmin) {
  const int qt = p->qtype;
  const int B = syn_block_weights(qt);
  if (B <= 1 || k % B != 0) return -1;
  const uint64_t kq = field_key(key, FLD_Q), ksc = field_key(key, FLD_SC), km = field_key(key, FLD_M);
  const uint64_t kd = field_key(key, FLD_D), kdm = field_key(key, FLD_DMIN);
  const uint64_t w0 = (uint64_t)r * (uint64_t)k + (uint64_t)b * (uint64_t)B;
  const uint64_t blk = (uint64_t)r * (uint64_t)(k / B) + (uint64_t)b;
  for (int i = 0; i < B; ++i) q[i] = (int32_t)uni_int(draw(kq, w0 + i), p->q_lo, p->q_hi);
  *d = draw_scale(kd, blk, p->d_sigma, p->d_mult);
  *dmin = 0;
  if (qt == SYN_Q4_K || qt == SYN_Q5_K) {
    for (int s = 0; s < 8; ++s) {
      sc[s] = (int32_t)uni_int(draw(ksc, blk * 8 + s), p->sc_lo, p->sc_hi);
      m[s] = (int32_t)uni_int(draw(km, blk * 8 + s), p->m_lo, p->m_hi);
    }
    *dmin = draw_scale(kdm, blk, p->dmin_sigma, p->d_mult);
  } else if (qt == SYN_Q6_K) {
    for (int j = 0; j < 16; ++j) sc[j] = (int32_t)uni_int(draw(ksc, blk * 16 + j), p->sc_lo, p->sc_hi);
  }
  return 0;
}
