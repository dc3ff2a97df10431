// qwg_formats.h -- packed device layouts of the block formats and their per-chunk decoders.
//
// The five formats are the GGUF block formats in the quantization-format table of the
// "Show HN ... Llama 3.1 70B" NTransformer page (Q4_0, Q8_0 with 32-weight blocks;
// Q4_K, Q5_K, Q6_K with 256-weight superblocks).  Canonical blocks (34/18/144/176/210 B)
// break 16-byte alignment and mix scales with quants, so at load time every matrix is
// rearranged ("packed") into separate row-major regions with the same payload bytes:
//
//   region Q : the quant bytes, 16 B per "chunk" (Q8_0: 16 weights; others: 32 weights), chunk c
//              of row r at Q + r*q_row + 16c, or row-interleaved by groups of 4 rows when the
//              shape allows (slot_row below) -> a wave reads 1 KiB contiguous per row and load
//   region A : Q8_0 / Q4_0 fp16 d per block; Q4_K / Q5_K 16-B superblock header (d, dmin and the
//              sixteen 6-bit scales/mins, re-laid out below); Q6_K 8 B of 2-bit highs per chunk
//   region B : Q5_K 4 B of fifth bits per chunk; Q6_K the chunk's two int8 sub-block scales
//   region C : Q6_K fp16 d per superblock
//
// Inside a 32-weight chunk (chunk-local weights e = 0..31) the 16 quant bytes hold
// e = j in the low nibble and e = j + 16 in the high nibble of byte j, so 32-bit word m
// carries weights 4m..4m+3 (low nibbles) and 16+4m..16+4m+3 (high nibbles) -- the
// activation for word m is float4 m and float4 4+m of the chunk.
//   Q4_0, Q4_K: each nibble holds q XOR 8, i.e. q - 8 as a 4-bit two's-complement number, so the
//        integer dot takes the quant words as they are.
//   Q4_K / Q5_K header (4 words): the scale of sub-block j (6 bits) at bit 6j of the 64-bit
//        (word 0 | word 1 << 32), its min at bit 6j of (word 2 | word 3 << 32), d in the high half
//        of word 1 and dmin in the high half of word 3 -- the same 16 six-bit values as the
//        canonical 12 bytes, placed so that a lane extracts its sub-block's pair with two 64-bit
//        shifts of even-aligned register pairs whatever j is.
//   Q5_K fifth bits (32 bits): bit 8b + 2m   = bit 4 of weight 4m+b,
//                              bit 8b + 2m+1 = bit 4 of weight 16+4m+b.
//   Q6_K high bits (2 words): word i, byte b, bit pair p: p=0 -> weight 4(2i)+b,
//        p=1 -> 16+4(2i)+b, p=2 -> 4(2i+1)+b, p=3 -> 16+4(2i+1)+b; each pair holds the quant's
//        two high bits XOR 2, so that (pair << 6 | nibble << 2) read as int8 is 4 (q - 32).
//   Q6_K scales: weights 0..15 of a chunk form one 16-weight sub-block, 16..31 the next.
//
// Every change from the canonical blocks is a bit permutation or a fixed bit flip: the packed
// matrix has exactly the canonical payload bytes and decodes to the same values.
//
// Everything here is __host__ __device__ so the same decoders can be exercised on the CPU.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace qwg {

enum QType : int { Q4_0 = 2, Q8_0 = 8, Q4_K = 12, Q5_K = 13, Q6_K = 14 };

__host__ __device__ inline bool qtype_known(int qt) {
  return qt == Q4_0 || qt == Q8_0 || qt == Q4_K || qt == Q5_K || qt == Q6_K;
}
__host__ __device__ inline int block_weights(int qt) { return (qt == Q4_0 || qt == Q8_0) ? 32 : 256; }
__host__ __device__ inline int block_bytes(int qt) {
  switch (qt) {
    case Q8_0: return 34;
    case Q4_0: return 18;
    case Q4_K: return 144;
    case Q5_K: return 176;
    case Q6_K: return 210;
    default: return 0;
  }
}
__host__ __device__ inline int chunk_weights(int qt) { return qt == Q8_0 ? 16 : 32; }

// Geometry of one packed matrix (all offsets in bytes from the matrix base).
struct Layout {
  int32_t qtype;
  int64_t rows, k;
  int64_t nch;    // chunks per row
  int64_t q_row;  // = 16 * nch
  int64_t a_off, a_row;
  int64_t b_off, b_row;
  int64_t c_off, c_row;
  int64_t total;
  int32_t ilv;  // per-chunk regions row-interleaved in groups of 4 rows (see slot_row)
};

__host__ __device__ inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

__host__ __device__ inline Layout make_layout(int qt, int64_t rows, int64_t k) {
  Layout L{};
  L.qtype = qt;
  L.rows = rows;
  L.k = k;
  L.nch = k / chunk_weights(qt);
  L.q_row = 16 * L.nch;
  const int64_t nb = k / block_weights(qt);
  switch (qt) {
    case Q8_0: L.a_row = 2 * nb; break;
    case Q4_0: L.a_row = 2 * nb; break;
    case Q4_K: L.a_row = 16 * nb; break;
    case Q5_K: L.a_row = 16 * nb; L.b_row = 4 * L.nch; break;
    case Q6_K: L.a_row = 8 * L.nch; L.b_row = 2 * L.nch; L.c_row = 2 * nb; break;
    default: break;
  }
  L.a_off = align256(rows * L.q_row);
  L.b_off = align256(L.a_off + rows * L.a_row);
  L.c_off = align256(L.b_off + rows * L.b_row);
  L.total = align256(L.c_off + rows * L.c_row);
  L.ilv = (rows % 4 == 0 && L.nch % 64 == 0) ? 1 : 0;
  return L;
}

// Pointers into one packed matrix, as the kernels take them.
struct MatView {
  const uint8_t* q;
  const uint8_t* a;
  const uint8_t* b;
  const uint8_t* c;
  int64_t q_row, a_row, b_row, c_row;
  int32_t nch;
  int32_t rows;
  int32_t ilv;
};

__host__ __device__ inline MatView make_view(const void* base, const Layout& L) {
  const uint8_t* p = (const uint8_t*)base;
  MatView v;
  v.q = p;
  v.a = p + L.a_off;
  v.b = p + L.b_off;
  v.c = p + L.c_off;
  v.q_row = L.q_row;
  v.a_row = L.a_row;
  v.b_row = L.b_row;
  v.c_row = L.c_row;
  v.nch = (int32_t)L.nch;
  v.rows = (int32_t)L.rows;
  v.ilv = L.ilv;
  return v;
}

// ---------------------------------------------------------------------------- fp16

// IEEE binary16 bits -> fp32, exact for every finite value including subnormals.
__host__ __device__ inline float half_bits_to_float(uint32_t h) {
#if defined(__HIP_DEVICE_COMPILE__)
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
#else
  const uint32_t sign = (h & 0x8000u) << 16, e = (h >> 10) & 31u, m = h & 1023u;
  uint32_t bits;
  if (e == 0) {
    const float v = (float)m * 5.9604644775390625e-8f;  // m * 2^-24, exact
    return (h & 0x8000u) ? -v : v;
  } else if (e == 31) {
    bits = sign | 0x7F800000u | (m << 13);
  } else {
    bits = sign | ((e + 112u) << 23) | (m << 13);
  }
  float f;
  __builtin_memcpy(&f, &bits, 4);
  return f;
#endif
}

// fp32 -> IEEE binary16 bits, round to nearest even, overflow -> inf.
__host__ __device__ inline uint16_t float_to_half_bits(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint16_t, (_Float16)f);
#else
  uint32_t x;
  __builtin_memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                    // below 2^-14: subnormal half
    float a;
    __builtin_memcpy(&a, &ax, 4);
    const float m = __builtin_rintf(a * 16777216.0f);
    return (uint16_t)(sign | (uint32_t)m);
  }
  const uint32_t mant = ax & 0x7FFFFFu;
  uint32_t e = (ax >> 23) - 112u;
  uint32_t hm = mant >> 13;
  const uint32_t rest = mant & 0x1FFFu;
  if (rest > 0x1000u || (rest == 0x1000u && (hm & 1u))) {
    hm += 1;
    if (hm == 1024) { hm = 0; e += 1; }
  }
  return (uint16_t)(sign | (e << 10) | hm);
#endif
}

// ---------------------------------------------------------------------------- byte helpers

__host__ __device__ inline float ubyte(uint32_t v, int i) { return (float)((v >> (8 * i)) & 0xFFu); }

__host__ __device__ inline float sbyte(uint32_t v, int i) { return (float)(int32_t)(int8_t)(uint8_t)(v >> (8 * i)); }

// 6-bit scale and min of sub-block s (0..7) from the 12 packed bytes held in words S0 (bytes
// 0..3), S1 (4..7), S2 (8..11): s < 4 -> low six bits of byte s / byte s+4; s >= 4 -> low/high
// nibble of byte s+4 joined with the top two bits of byte s-4 (scale) / byte s (min).
__host__ __device__ inline void kq_scale_min(uint32_t S0, uint32_t S1, uint32_t S2, int s, int& sc, int& m) {
  const int t = s & 3;
  const uint32_t b0 = (S0 >> (8 * t)) & 0xFFu, b1 = (S1 >> (8 * t)) & 0xFFu, b2 = (S2 >> (8 * t)) & 0xFFu;
  const int lo_sc = (int)(b0 & 63u), lo_m = (int)(b1 & 63u);
  const int hi_sc = (int)((b2 & 15u) | ((b0 >> 6) << 4));
  const int hi_m = (int)((b2 >> 4) | ((b1 >> 6) << 4));
  sc = s < 4 ? lo_sc : hi_sc;
  m = s < 4 ? lo_m : hi_m;
}

// Packed Q4_K / Q5_K superblock header, words h0..h3 (16 bytes, as many as the canonical d, dmin and
// twelve scale bytes): the 6-bit scale of sub-block j at bit 6j of the 64-bit pair h0|h1, its 6-bit
// min at bit 6j of h2|h3, d in the high half of h1 and dmin in the high half of h3.  Each pair is an
// even-aligned register pair of the 16-byte load, so one 64-bit shift extracts a field.
__host__ __device__ inline void kq_packed_scale_min(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3, int j,
                                                    uint32_t& sc, uint32_t& m) {
  const uint64_t ps = (uint64_t)h0 | ((uint64_t)h1 << 32);
  const uint64_t pm = (uint64_t)h2 | ((uint64_t)h3 << 32);
  sc = (uint32_t)(ps >> (6 * j)) & 63u;
  m = (uint32_t)(pm >> (6 * j)) & 63u;
}

// Weight bytes are read exactly once per pass: streaming (non-temporal) loads.
typedef uint32_t qwg_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t qwg_u32x2 __attribute__((ext_vector_type(2)));

__host__ __device__ inline uint4 ld_stream_u4(const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const qwg_u32x4 v = __builtin_nontemporal_load((const qwg_u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *(const uint4*)p;
#endif
}
__host__ __device__ inline uint2 ld_stream_u2(const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const qwg_u32x2 v = __builtin_nontemporal_load((const qwg_u32x2*)p);
  return make_uint2(v.x, v.y);
#else
  return *(const uint2*)p;
#endif
}
__host__ __device__ inline uint32_t ld_stream_u1(const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_nontemporal_load((const uint32_t*)p);
#else
  return *(const uint32_t*)p;
#endif
}

template <class T>
__host__ __device__ inline T ld(const uint8_t* p) {
  return *(const T*)p;
}

// ---------------------------------------------------------------------------- activation digits
//
// The GEMV never multiplies fp32 activations by converted weights.  Instead every 32-element chunk
// of the activation becomes a block fixed-point integer vector: one shared power-of-two scale per
// chunk, x_fix = rint(x * 2^s) with the chunk's largest magnitude at [2^29, 2^30) (32-bit two's-
// complement range, so the largest element keeps 30 significant bits and every element is within
// 2^-30 of the chunk maximum of its exact value), split into balanced digits:
//   nibble digits (Q4_0, Q4_K): x_fix = sum_l d_l 16^l, d_l in [-8, 7], l = 0..7
//   byte digits (Q5_K, Q6_K, Q8_0): x_fix = sum_l d_l 256^l, d_l in [-128, 127], l = 0..3
// Adding 0x88888888 (or 0x80808080) maps the balanced digits to the plain base-16 (base-256) digits
// of the sum, so each digit is a field extract followed by flipping its top bit.  The weight quants
// are then integers too, and each dot product is a sum of exact integer products (v_dot8_i32_i4 /
// v_dot4_i32_i8), recombined per chunk in fp32 and scaled by 2^-s.
//
// A chunk holding a NaN or an infinity gets a NaN scale (and zero digits), so every row it touches
// comes out NaN, as the exact sum would be non-finite; the digits never turn a non-finite input into
// a finite output.
//
// Digit words of a chunk (32 x 32 bits) are laid out to match the packed quant words:
//   nibble: word m*8 + l, nibble 2b+h = digit l of element 16h + 4m + b   (h = 0 low, 1 high nibble)
//   byte:   word (h*4 + m)*4 + l, byte b = digit l of element 16h + 4m + b
// followed by a ChunkDesc (2^-s and the sum of x_fix over the chunk, rounded and exact).

enum DigitKind : int { DIG_NIB = 0, DIG_BYTE = 1, DIG_F16 = 2 };
// DIG_F16 (the operands of the fp16 prompt GEMM, Q4_K / Q5_K with 9..64 columns) is not a fixed-point
// form: per column and 256-element superblock, x' = x 2^sh with the superblock maximum in [2^14, 2^15)
// (2^-sh kept a normal or subnormal fp32 power of two), each element as two fp16 pieces
// hi = fp16(x') and lo = fp16(x' - hi) (lo may be subnormal), and each chunk's sum of x' (times 2^-6)
// as the same two pieces.  In the superblock's 8 x 36 words:
//   words 0..255: [chunk c][piece p][group m] 4 words = eight fp16 of elements 4m, 4m+2, 4m+1, 4m+3,
//                 16+4m, 16+4m+2, 16+4m+1, 16+4m+3 (the order in which one packed quant word's
//                 nibbles unpack into half pairs)
//   words 256..259 / 260..263: hi / lo pieces of the 8 chunk sums (fp16, chunk c in half c)
//   word 264: 2^-sh as fp32 (NaN if the superblock holds a NaN or an infinity)
constexpr int XCHUNK = 32;           // activation elements per digit chunk
constexpr int NIB_LEVELS = 8;        // nibble digit levels
constexpr int BYTE_LEVELS = 4;       // byte digit levels
constexpr int DIG_WORDS = 32;        // digit words per chunk (either kind)
constexpr int DIG_CHUNK_WORDS = 36;  // digit words + ChunkDesc
constexpr int FIX_TOP = 29;          // the chunk maximum times 2^s lies in [2^FIX_TOP, 2^(FIX_TOP+1))
constexpr int F16_SB_WORDS = 8 * DIG_CHUNK_WORDS;  // DIG_F16: a superblock's eight chunk slots
constexpr int F16_SUM_WORD = 256;
constexpr int F16_SCALE_WORD = 264;

__host__ __device__ inline int digit_kind(int qt) { return (qt == Q4_K || qt == Q4_0) ? DIG_NIB : DIG_BYTE; }

struct ChunkDesc {
  float inv_scale;  // 2^-s (NaN if the chunk holds a NaN or an infinity)
  float sum;        // sum of x_fix over the chunk, rounded once to fp32
  int32_t shi, slo; // the same sum exactly: 32768 shi + slo (|shi| <= 2^20, 0 <= slo < 2^15)
};

// Four consecutive lanes (lane & 3 = m) digitize one 32-element chunk together.  Lane m passes the
// chunk elements 4m..4m+3 and 16+4m..16+4m+3 in v[0..7]; the chunk scale and integer sums travel by
// lane shuffles; lane m writes its eight digit words and lane 0 the ChunkDesc at oc (a chunk base of
// DIG_CHUNK_WORDS words).  All four lanes must call it (write = false lets a lane take part without
// storing).
// (byte j of a) << 8 | (byte j of b), j < 4: one v_perm_b32 (bytes 0..3 of the selector pick from
// the second operand, 4..7 from the first, 12 gives zero)
__device__ inline uint32_t byte_gather(uint32_t a, uint32_t b, uint32_t j) {
  return __builtin_amdgcn_perm(a, b, 0x0C0C0000u | ((4u + j) << 8) | j);
}

// put(i, word) stores digit word i (0..31) or descriptor word i (32..35) of the chunk.
// The value of lane (lane ^ 1) or (lane ^ 2) of the same quad: one DPP quad permute, no LDS trip.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __uint_as_float(quad_swap<0xB1>(__float_as_uint(v))));  // quad_perm [1,0,3,2]
  return fmaxf(v, __uint_as_float(quad_swap<0x4E>(__float_as_uint(v))));  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __uint_as_float(quad_swap<0xB1>(__float_as_uint(v)));
  return v + __uint_as_float(quad_swap<0x4E>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ double quad_swap(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = quad_swap<CTRL>((uint32_t)b), hi = quad_swap<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ double quad_sum(double v) {
  v += quad_swap<0xB1>(v);
  return v + quad_swap<0x4E>(v);
}

template <class Put>
__device__ inline void digitize_group_to(const float* v, int m, int kind, Put&& put, bool write) {
  // the chunk maximum, and nf = NaN exactly when an element is a NaN or an infinity (0 * inf is NaN;
  // fmaxf alone would skip a NaN)
  float mx = 0.f, nf = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mx = fmaxf(mx, fabsf(v[i]));
    nf = __builtin_fmaf(v[i], 0.0f, nf);
  }
  mx = quad_max(mx);
  const bool bad = __builtin_isnan(quad_sum(nf));
  // mx * 2^sh in [2^29, 2^30); 2^-sh stays a normal number (ilogb(mx) = frexp exponent - 1)
  int sh = 0;
  if (mx > 0.f && !bad) sh = min(126, max(-126, FIX_TOP + 1 - __builtin_amdgcn_frexp_expf(mx)));
  int32_t xf[8];
  // the sum of x_fix over the chunk, exactly (|sum| < 2^35: an fp64 sum of integers is exact)
  double sx = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xf[i] = bad ? 0 : (int32_t)rintf(ldexpf(v[i], sh));
    sx += (double)xf[i];
  }
  sx = quad_sum(sx);
  if (!write) return;
  // Adding 0x88888888 (0x80808080) and flipping the top bit of every nibble (byte) leaves balanced
  // digit l of x_fix, as a 4-bit (8-bit) two's-complement number, in nibble (byte) l of u.  The digit
  // words are then byte gathers: v_perm_b32 picks byte j of two words into two byte lanes.
  if (kind == DIG_NIB) {
    // word m*8 + l, nibble 2b + h = digit l of element 16h + 4m + b  (v[4h + b]).  Byte b of a
    // word pairs element b (low nibble) with element 4+b (high nibble): e[b] holds those pairs for
    // the even levels (byte j = level 2j), o[b] for the odd ones.
    uint32_t e[4], o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t lo = (uint32_t)(xf[b] + (int32_t)0x88888888u) ^ 0x88888888u;
      const uint32_t hi = (uint32_t)(xf[4 + b] + (int32_t)0x88888888u) ^ 0x88888888u;
      e[b] = (lo & 0x0F0F0F0Fu) | ((hi & 0x0F0F0F0Fu) << 4);
      o[b] = ((lo >> 4) & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u);
    }
#pragma unroll
    for (int l = 0; l < NIB_LEVELS; ++l) {
      const uint32_t* E = (l & 1) ? o : e;
      const uint32_t j = (uint32_t)(l >> 1);
      put(m * NIB_LEVELS + l, byte_gather(E[1], E[0], j) | (byte_gather(E[3], E[2], j) << 16));
    }
  } else {
    // word (h*4 + m)*4 + l, byte b = digit l of element 16h + 4m + b
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t u[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) u[b] = (uint32_t)(xf[4 * h + b] + (int32_t)0x80808080u) ^ 0x80808080u;
#pragma unroll
      for (int l = 0; l < BYTE_LEVELS; ++l)
        put((h * 4 + m) * BYTE_LEVELS + l,
            byte_gather(u[1], u[0], (uint32_t)l) | (byte_gather(u[3], u[2], (uint32_t)l) << 16));
    }
  }
  if (m == 0) {
    // sum = 32768 shi + slo with 0 <= slo < 32768
    const double fh = floor(sx * (1.0 / 32768.0));
    put(DIG_WORDS, __float_as_uint(bad ? __builtin_nanf("") : ldexpf(1.0f, -sh)));
    put(DIG_WORDS + 1, __float_as_uint((float)sx));
    put(DIG_WORDS + 2, (uint32_t)(int32_t)fh);
    put(DIG_WORDS + 3, (uint32_t)(int32_t)__builtin_fma(-32768.0, fh, sx));
  }
}
__device__ inline void digitize_group(const float* v, int m, int kind, uint32_t* oc, bool write) {
  digitize_group_to(v, m, kind, [&](int i, uint32_t w) { oc[i] = w; }, write);
}


// exact integer dot products (device: one v_dot8_i32_i4 / v_dot4_i32_i8 each)
__host__ __device__ inline int32_t sdot8(uint32_t a, uint32_t b, int32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
#else
  for (int i = 0; i < 8; ++i) {
    int x = (int)((a >> (4 * i)) & 15u), y = (int)((b >> (4 * i)) & 15u);
    x = x >= 8 ? x - 16 : x;
    y = y >= 8 ? y - 16 : y;
    c += x * y;
  }
  return c;
#endif
}
__host__ __device__ inline int32_t sdot4(uint32_t a, uint32_t b, int32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
#else
  for (int i = 0; i < 4; ++i) c += (int)(int8_t)(uint8_t)(a >> (8 * i)) * (int)(int8_t)(uint8_t)(b >> (8 * i));
  return c;
#endif
}

// The value of a chunk against its digit levels, sum_l base^l D_l with D_l the integer dot of the
// quants with digit level l, assembled in Horner form: each level's dot chain starts from base x
// the partial of the levels above it, so no level needs its own accumulator or conversion.
//   nibble (base 16, eight levels): hi = ((D7*16 + D6)*16 + D5)*16 + D4, lo likewise from D3..D0,
//     |D_l| <= 32*8*8 = 2048, so |hi|, |lo| < 2^24 (exact in int32 and fp32); value = 65536 hi + lo
//     with one rounding
//   byte (base 256, four levels): hi = D3*256 + D2, lo = D1*256 + D0 with |D_l| <= 32*128*128 = 2^19,
//     so |hi|, |lo| < 2^28 fit int32; value = 65536 hi + lo (each converts to fp32 with relative
//     error 2^-24, then one fma)
// The quant words w[0..NW) pair with digit words dig[m*8 + l] (nibble) / dig[m*4 + l] (byte).
template <int NW>
__host__ __device__ inline int32_t nib_chain(const uint32_t* w, const uint32_t* dig, int l, int32_t c) {
#pragma unroll
  for (int m = 0; m < NW; ++m) c = sdot8(w[m], dig[m * NIB_LEVELS + l], c);
  return c;
}
__host__ __device__ inline void nib_levels(const uint32_t* w, const uint32_t* dig, int32_t& hi, int32_t& lo) {
  hi = nib_chain<4>(w, dig, 7, 0);
  hi = nib_chain<4>(w, dig, 6, hi * 16);
  hi = nib_chain<4>(w, dig, 5, hi * 16);
  hi = nib_chain<4>(w, dig, 4, hi * 16);
  lo = nib_chain<4>(w, dig, 3, 0);
  lo = nib_chain<4>(w, dig, 2, lo * 16);
  lo = nib_chain<4>(w, dig, 1, lo * 16);
  lo = nib_chain<4>(w, dig, 0, lo * 16);
}
__host__ __device__ inline float nib_value(const uint32_t* w, const uint32_t* dig) {
  int32_t hi, lo;
  nib_levels(w, dig, hi, lo);
  return __builtin_fmaf(65536.0f, (float)hi, (float)lo);
}
template <int NW>
__host__ __device__ inline int32_t byte_chain(const uint32_t* w, const uint32_t* dig, int l, int32_t c) {
#pragma unroll
  for (int m = 0; m < NW; ++m) c = sdot4(w[m], dig[m * BYTE_LEVELS + l], c);
  return c;
}
// four quant words against the 16 digit words of one 16-element half
__host__ __device__ inline float byte_value(const uint32_t* w, const uint32_t* dig) {
  int32_t hi = byte_chain<4>(w, dig, 3, 0);
  hi = byte_chain<4>(w, dig, 2, hi * 256);
  int32_t lo = byte_chain<4>(w, dig, 1, 0);
  lo = byte_chain<4>(w, dig, 0, lo * 256);
  return __builtin_fmaf(65536.0f, (float)hi, (float)lo);
}
// both halves of a 32-element chunk (quant words wa against dig[0..16), wb against dig[16..32))
__host__ __device__ inline float byte_value2(const uint32_t* wa, const uint32_t* wb, const uint32_t* dig) {
  int32_t hi = byte_chain<4>(wb, dig + 16, 3, byte_chain<4>(wa, dig, 3, 0));
  hi = byte_chain<4>(wb, dig + 16, 2, byte_chain<4>(wa, dig, 2, hi * 256));
  int32_t lo = byte_chain<4>(wb, dig + 16, 1, byte_chain<4>(wa, dig, 1, 0));
  lo = byte_chain<4>(wb, dig + 16, 0, byte_chain<4>(wa, dig, 0, lo * 256));
  return __builtin_fmaf(65536.0f, (float)hi, (float)lo);
}

// ---------------------------------------------------------------------------- per-format chunk codecs
//
// Each Fmt<QT> provides
//   CW (weights per chunk)
//   Raw load(view, ro, chunk, slot)     -- the chunk's quant bytes and scale data (ro: row_off of
//                                          its row; slot: the chunk's place in the per-chunk
//                                          regions, slot_row + slot_chunk)
//   decode(raw, chunk, w[CW])           -- exact fp32 weights in chunk order (for dequantize);
//                                          a zero weight is +0 ("+ 0.0f" turns -0 into +0)
//   U unpack(raw, chunk, sub)           -- integer quant words for the dot plus the chunk's fp32
//                                          scale coefficients (sub = chunk & 7, its place in the
//                                          256-weight superblock)
//   float dotu(u, digits, desc)         -- sum_e w_e x_e of the chunk from exact integer dot
//                                          products with the activation digits
// Byte offsets inside one packed region are 32-bit (the library refuses matrices of 4 GiB or more),
// so loads take a uniform 64-bit base plus a 32-bit lane offset.

// Byte offset of a row in the per-block region a format reads per row (region A, or C for Q6_K's d),
// computed once per row rather than once per load.
__host__ __device__ inline uint32_t row_off(int qt, const MatView& v, int64_t row) {
  return (uint32_t)row * (uint32_t)(qt == Q6_K ? v.c_row : v.a_row);
}

// Per-chunk regions (one e-byte piece per chunk: quants 16 B, Q5_K fifth bits 4 B, Q6_K high bits
// 8 B and scales 2 B) store the piece of (row, chunk c) at e * slot(row, c).  Row-major: slot =
// row * nch + c.  Row-interleaved (ilv): rows come in groups of 4, and within a group the pieces of
// 64 consecutive chunks of row 0, row 1, row 2, row 3 follow each other -- so the R <= 4 rows a
// wave reads for 64 chunks are one contiguous span (fewer concurrent DRAM streams than 4 rows).
// slot = slot_row(row) + slot_chunk(c), so a kernel adds one per-row and one per-chunk term.
__host__ __device__ inline uint32_t slot_row(int32_t ilv, int64_t nch, int64_t row) {
  return ilv ? ((uint32_t)row >> 2) * 4u * (uint32_t)nch + ((uint32_t)row & 3u) * 64u : (uint32_t)row * (uint32_t)nch;
}
__host__ __device__ inline uint32_t slot_chunk(int32_t ilv, uint32_t c) { return ilv ? (c >> 6) * 256u + (c & 63u) : c; }

template <int QT>
struct Fmt;

template <>
struct Fmt<Q8_0> {
  static constexpr int CW = 16;
  struct Raw {
    uint4 q;
    uint32_t d;
  };
  __host__ __device__ static Raw load(const MatView& v, uint32_t ro, int c, uint32_t slot) {
    Raw r;
    r.q = ld_stream_u4(v.q + slot * 16u);
    r.d = ld<uint16_t>(v.a + ro + (uint32_t)(c >> 1) * 2u);
    return r;
  }
  __host__ __device__ static void decode(const Raw& r, int, float* w) {
    const float d = half_bits_to_float(r.d);
    const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    for (int m = 0; m < 4; ++m)
      for (int b = 0; b < 4; ++b) w[4 * m + b] = d * sbyte(q[m], b) + 0.0f;
  }
  struct U {
    uint32_t w[4];
    float d;
  };
  __host__ __device__ static U unpack(const Raw& r, int, int) {
    U u;
    u.w[0] = r.q.x;
    u.w[1] = r.q.y;
    u.w[2] = r.q.z;
    u.w[3] = r.q.w;
    u.d = half_bits_to_float(r.d);
    return u;
  }
  // dig: the 16 digit words of this chunk's half of the 32-element activation chunk
  __host__ __device__ static float dotu(const U& u, const uint32_t* dig, const ChunkDesc& ds) {
    return ds.inv_scale * (u.d * byte_value(u.w, dig));
  }
};

template <>
struct Fmt<Q4_0> {
  static constexpr int CW = 32;
  struct Raw {
    uint4 q;
    uint32_t d;
  };
  __host__ __device__ static Raw load(const MatView& v, uint32_t ro, int c, uint32_t slot) {
    Raw r;
    r.q = ld_stream_u4(v.q + slot * 16u);
    r.d = ld<uint16_t>(v.a + ro + (uint32_t)c * 2u);
    return r;
  }
  __host__ __device__ static void decode(const Raw& r, int, float* w) {
    const float d = half_bits_to_float(r.d);
    const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    for (int m = 0; m < 4; ++m)
      for (int b = 0; b < 4; ++b) {
        const int byte = (int)((q[m] >> (8 * b)) & 0xFFu) ^ 0x88;  // back to the canonical q
        w[4 * m + b] = d * (float)((byte & 15) - 8) + 0.0f;
        w[16 + 4 * m + b] = d * (float)((byte >> 4) - 8) + 0.0f;
      }
  }
  struct U {
    uint32_t w[4];  // q - 8 as signed nibbles
    float d;
  };
  __host__ __device__ static U unpack(const Raw& r, int, int) {
    U u;
    u.w[0] = r.q.x;
    u.w[1] = r.q.y;
    u.w[2] = r.q.z;
    u.w[3] = r.q.w;
    u.d = half_bits_to_float(r.d);
    return u;
  }
  __host__ __device__ static float dotu(const U& u, const uint32_t* dig, const ChunkDesc& ds) {
    return ds.inv_scale * (u.d * nib_value(u.w, dig));
  }
};

template <>
struct Fmt<Q4_K> {
  static constexpr int CW = 32;
  struct Raw {
    uint4 q;
    uint4 h;  // the re-laid-out scales and mins, d and dmin (kq_packed_scale_min)
  };
  __host__ __device__ static Raw load(const MatView& v, uint32_t ro, int c, uint32_t slot) {
    Raw r;
    r.q = ld_stream_u4(v.q + slot * 16u);
    r.h = ld<uint4>(v.a + ro + (uint32_t)(c >> 3) * 16u);
    return r;
  }
  // d * scale and dmin * min of sub-block j (both exact in fp32)
  __host__ __device__ static void coef(const uint4& h, int j, float& dsc, float& dmm) {
    uint32_t sc, m;
    kq_packed_scale_min(h.x, h.y, h.z, h.w, j, sc, m);
    dsc = half_bits_to_float(h.y >> 16) * (float)sc;
    dmm = half_bits_to_float(h.w >> 16) * (float)m;
  }
  __host__ __device__ static void decode(const Raw& r, int c, float* w) {
    float dsc, dmm;
    coef(r.h, c & 7, dsc, dmm);
    const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    for (int m = 0; m < 4; ++m)
      for (int b = 0; b < 4; ++b) {
        const int byte = (int)((q[m] >> (8 * b)) & 0xFFu) ^ 0x88;  // back to the canonical q
        w[4 * m + b] = __builtin_fmaf(dsc, (float)(byte & 15), -dmm) + 0.0f;
        w[16 + 4 * m + b] = __builtin_fmaf(dsc, (float)(byte >> 4), -dmm) + 0.0f;
      }
  }
  struct U {
    uint32_t w[4];  // q - 8 as signed nibbles
    float c0, c1;   // sum w x = c0 * sum q x + c1 * sum x
  };
  __host__ __device__ static U unpack(const Raw& r, int, int sub) {
    float dsc, dmm;
    coef(r.h, sub, dsc, dmm);
    U u;
    u.w[0] = r.q.x;
    u.w[1] = r.q.y;
    u.w[2] = r.q.z;
    u.w[3] = r.q.w;
    u.c0 = dsc;
    u.c1 = -dmm;
    return u;
  }
  // sum_e q_e x_fix_e stays an exact integer until one conversion: the nibble dots give
  // sum (q - 8) x_fix = 65536 hi + lo, and adding back 8 sum x_fix = 8 (32768 shi + slo) gives
  // 65536 (hi + 4 shi) + (lo + 8 slo).  Folding the 8 into an fp32 coefficient instead would
  // cancel two large rounded terms whenever a chunk's largest element meets a zero quant.
  __host__ __device__ static float dotu(const U& u, const uint32_t* dig, const ChunkDesc& ds) {
    int32_t hi, lo;
    nib_levels(u.w, dig, hi, lo);
    const float qx = __builtin_fmaf(65536.0f, (float)(hi + 4 * ds.shi), (float)(lo + 8 * ds.slo));
    return ds.inv_scale * __builtin_fmaf(u.c0, qx, u.c1 * ds.sum);
  }
};

template <>
struct Fmt<Q5_K> {
  static constexpr int CW = 32;
  struct Raw {
    uint4 q;
    uint4 h;
    uint32_t qh;
  };
  __host__ __device__ static Raw load(const MatView& v, uint32_t ro, int c, uint32_t slot) {
    Raw r;
    r.q = ld_stream_u4(v.q + slot * 16u);
    r.h = ld<uint4>(v.a + ro + (uint32_t)(c >> 3) * 16u);
    r.qh = ld_stream_u1(v.b + slot * 4u);
    return r;
  }
  // the 5-bit quants of word m as bytes: low-nibble weights and high-nibble weights
  __host__ __device__ static void words(const Raw& r, int m, uint32_t& lo, uint32_t& hi) {
    const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    const uint32_t w = q[m];
    // bit 8b + 2m (low) / 8b + 2m + 1 (high) moved to bit 4 of byte b
    const uint32_t l5 = (m <= 2) ? (r.qh << (4 - 2 * m)) : (r.qh >> 2);
    const uint32_t h5 = (m <= 1) ? (r.qh << (3 - 2 * m)) : (r.qh >> (2 * m - 3));
    lo = (w & 0x0F0F0F0Fu) | (l5 & 0x10101010u);
    hi = ((w >> 4) & 0x0F0F0F0Fu) | (h5 & 0x10101010u);
  }
  __host__ __device__ static void decode(const Raw& r, int c, float* w) {
    float dsc, dmm;
    Fmt<Q4_K>::coef(r.h, c & 7, dsc, dmm);
    for (int m = 0; m < 4; ++m) {
      uint32_t lo, hi;
      words(r, m, lo, hi);
      for (int b = 0; b < 4; ++b) {
        w[4 * m + b] = __builtin_fmaf(dsc, ubyte(lo, b), -dmm) + 0.0f;
        w[16 + 4 * m + b] = __builtin_fmaf(dsc, ubyte(hi, b), -dmm) + 0.0f;
      }
    }
  }
  struct U {
    uint32_t lo[4], hi[4];  // 5-bit quants as bytes
    float c0, c1;           // sum w x = c0 * sum q x + c1 * sum x
  };
  __host__ __device__ static U unpack(const Raw& r, int, int sub) {
    float dsc, dmm;
    Fmt<Q4_K>::coef(r.h, sub, dsc, dmm);
    U u;
#pragma unroll
    for (int m = 0; m < 4; ++m) words(r, m, u.lo[m], u.hi[m]);
    u.c0 = dsc;
    u.c1 = -dmm;
    return u;
  }
  __host__ __device__ static float dotu(const U& u, const uint32_t* dig, const ChunkDesc& ds) {
    return ds.inv_scale * __builtin_fmaf(u.c0, byte_value2(u.lo, u.hi, dig), u.c1 * ds.sum);
  }
};

template <>
struct Fmt<Q6_K> {
  static constexpr int CW = 32;
  struct Raw {
    uint4 q;
    uint2 qh;
    uint32_t scw;  // the aligned word holding the chunk's two int8 scales (byte 0 -> weights 0..15,
                   // byte 1 -> 16..31) at bit (sh & 31)
    uint32_t dw;   // the aligned word holding the superblock's fp16 d at bit (sh >> 8)
    uint32_t sh;
  };
  // The 2-byte fields are read as the aligned 32-bit words that hold them (every region is 256-B
  // aligned and padded, so the word is inside the matrix): 16-bit loads made the compiler place the
  // zero-extension of the next iteration's fields in the loop latch, where it waited for the loads.
  __host__ __device__ static Raw load(const MatView& v, uint32_t ro, int c, uint32_t slot) {
    Raw r;
    r.q = ld_stream_u4(v.q + slot * 16u);
    r.qh = ld_stream_u2(v.a + slot * 8u);
    const uint32_t so = slot * 2u, dof = ro + (uint32_t)(c >> 3) * 2u;
    r.scw = ld<uint32_t>(v.b + (so & ~3u));
    r.dw = ld<uint32_t>(v.c + (dof & ~3u));
    r.sh = (so & 2u) * 8u | ((dof & 2u) * 8u) << 8;
    return r;
  }
  __host__ __device__ static uint32_t sc_of(const Raw& r) { return r.scw >> (r.sh & 31u); }
  __host__ __device__ static uint32_t d_of(const Raw& r) { return (r.dw >> (r.sh >> 8)) & 0xFFFFu; }
  // word m as int8 bytes 4 (q - 32): low-nibble weights (4m+b) and high-nibble weights (16+4m+b);
  // the stored high pair (XOR 2) lands in bits 6..7, the nibble in bits 2..5
  __host__ __device__ static void words(const Raw& r, int m, uint32_t& lo, uint32_t& hi) {
    const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    const uint32_t w = q[m];
    const uint32_t h = (m < 2) ? r.qh.x : r.qh.y;
    const uint32_t hl = (m & 1) ? (h << 2) : (h << 6);  // pair 2(m&1) -> bits 6..7
    const uint32_t hh = (m & 1) ? h : (h << 4);         // pair 2(m&1)+1 -> bits 6..7
    lo = ((w << 2) & 0x3C3C3C3Cu) | (hl & 0xC0C0C0C0u);
    hi = ((w >> 2) & 0x3C3C3C3Cu) | (hh & 0xC0C0C0C0u);
  }
  __host__ __device__ static void decode(const Raw& r, int, float* w) {
    const float d = half_bits_to_float(d_of(r));
    const uint32_t sc = sc_of(r);
    const float dA = d * (float)(int8_t)(uint8_t)(sc & 0xFFu);
    const float dB = d * (float)(int8_t)(uint8_t)((sc >> 8) & 0xFFu);
    for (int m = 0; m < 4; ++m) {
      uint32_t lo, hi;
      words(r, m, lo, hi);
      for (int b = 0; b < 4; ++b) {
        w[4 * m + b] = dA * (0.25f * sbyte(lo, b)) + 0.0f;
        w[16 + 4 * m + b] = dB * (0.25f * sbyte(hi, b)) + 0.0f;
      }
    }
  }
  struct U {
    uint32_t lo[4], hi[4];  // 4 (q - 32) as int8 (weights 0..15 and 16..31)
    float dA, dB;           // d * sc / 4 of the two 16-weight sub-blocks
  };
  __host__ __device__ static U unpack(const Raw& r, int, int) {
    const float d = half_bits_to_float(d_of(r));
    const uint32_t sc = sc_of(r);
    U u;
#pragma unroll
    for (int m = 0; m < 4; ++m) words(r, m, u.lo[m], u.hi[m]);
    u.dA = 0.25f * (d * (float)(int8_t)(uint8_t)(sc & 0xFFu));
    u.dB = 0.25f * (d * (float)(int8_t)(uint8_t)((sc >> 8) & 0xFFu));
    return u;
  }
  __host__ __device__ static float dotu(const U& u, const uint32_t* dig, const ChunkDesc& ds) {
    return ds.inv_scale * __builtin_fmaf(u.dA, byte_value(u.lo, dig), u.dB * byte_value(u.hi, dig + 16));
  }
};

// ---------------------------------------------------------------------------- repack (canonical -> packed)
//
// One canonical block of row r, block index b, is scattered to the packed regions.  Pure byte
// movement (nibble re-pairing and bit re-ordering); no arithmetic on values.

__host__ __device__ inline void put16(uint8_t* p, const uint8_t* s) {
  for (int i = 0; i < 16; ++i) p[i] = s[i];
}

// quant (0..63) of weight i of a canonical superblock / block
__host__ __device__ inline int canon_q4k(const uint8_t* qs, int i) {
  const int g = i >> 6, t = i & 63;
  return t < 32 ? (qs[32 * g + t] & 15) : (qs[32 * g + t - 32] >> 4);
}
__host__ __device__ inline int canon_q5k(const uint8_t* qh, const uint8_t* qs, int i) {
  const int g = i >> 6, t = i & 63;
  const int nib = t < 32 ? (qs[32 * g + t] & 15) : (qs[32 * g + t - 32] >> 4);
  const int bit = t < 32 ? ((qh[t] >> (2 * g)) & 1) : ((qh[t - 32] >> (2 * g + 1)) & 1);
  return nib | (bit << 4);
}
__host__ __device__ inline int canon_q6k(const uint8_t* ql, const uint8_t* qh, int i) {
  const int n = i >> 7, r = i & 127, u = r >> 5, l = r & 31;
  const uint8_t byte = ql[64 * n + l + 32 * (u & 1)];
  const int nib = u < 2 ? (byte & 15) : (byte >> 4);
  return nib | (((qh[32 * n + l] >> (2 * u)) & 3) << 4);
}

// write packed chunk pieces for chunk-local quants q[0..31]
__host__ __device__ inline void pack_nibbles(const int* q, uint8_t* dst) {
  for (int j = 0; j < 16; ++j) dst[j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
}

__host__ __device__ inline void repack_block(int qt, const uint8_t* blk, uint8_t* base, const Layout& L, int64_t row,
                                             int64_t b) {
  // per-block pieces (row-major) and per-chunk pieces (coff: possibly row-interleaved)
  uint8_t* A = base + L.a_off + row * L.a_row;
  uint8_t* C = base + L.c_off + row * L.c_row;
  const uint32_t srow = slot_row(L.ilv, L.nch, row);
  auto slot = [&](int64_t c) { return (int64_t)(srow + slot_chunk(L.ilv, (uint32_t)c)); };
  auto Qc = [&](int64_t c) { return base + 16 * slot(c); };
  auto Ac = [&](int64_t c, uint32_t e) { return base + L.a_off + e * slot(c); };
  auto Bc = [&](int64_t c, uint32_t e) { return base + L.b_off + e * slot(c); };
  switch (qt) {
    case Q8_0: {
      A[2 * b] = blk[0];
      A[2 * b + 1] = blk[1];
      put16(Qc(2 * b), blk + 2);
      put16(Qc(2 * b + 1), blk + 18);
      break;
    }
    case Q4_0: {
      A[2 * b] = blk[0];
      A[2 * b + 1] = blk[1];
      // canonical Q4_0 already pairs weight j with j + 16; nibbles become q XOR 8
      uint8_t* q = Qc(b);
      for (int j = 0; j < 16; ++j) q[j] = (uint8_t)(blk[2 + j] ^ 0x88);
      break;
    }
    case Q4_K:
    case Q5_K: {
      // header: the sixteen 6-bit scales/mins re-laid out around d and dmin (kq_packed_scale_min)
      uint32_t S[3];
      for (int i = 0; i < 3; ++i)
        S[i] = (uint32_t)blk[4 + 4 * i] | ((uint32_t)blk[5 + 4 * i] << 8) | ((uint32_t)blk[6 + 4 * i] << 16) |
               ((uint32_t)blk[7 + 4 * i] << 24);
      uint64_t ps = 0, pm = 0;
      for (int j = 0; j < 8; ++j) {
        int sc, mn;
        kq_scale_min(S[0], S[1], S[2], j, sc, mn);
        ps |= (uint64_t)sc << (6 * j);
        pm |= (uint64_t)mn << (6 * j);
      }
      const uint32_t d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8), dmin = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8);
      const uint32_t hw[4] = {(uint32_t)ps, (uint32_t)(ps >> 32) | (d << 16), (uint32_t)pm,
                              (uint32_t)(pm >> 32) | (dmin << 16)};
      for (int i = 0; i < 16; ++i) A[b * 16 + i] = (uint8_t)(hw[i >> 2] >> (8 * (i & 3)));
      const uint8_t* qs = blk + (qt == Q4_K ? 16 : 48);
      const uint8_t* qh = blk + 16;
      for (int s = 0; s < 8; ++s) {
        int q[32];
        for (int e = 0; e < 32; ++e)
          q[e] = qt == Q4_K ? (canon_q4k(qs, 32 * s + e) ^ 8) : canon_q5k(qh, qs, 32 * s + e);
        const int64_t c = 8 * b + s;
        pack_nibbles(q, Qc(c));
        if (qt == Q5_K) {
          uint32_t bits = 0;
          for (int m = 0; m < 4; ++m)
            for (int bb = 0; bb < 4; ++bb) {
              bits |= (uint32_t)((q[4 * m + bb] >> 4) & 1) << (8 * bb + 2 * m);
              bits |= (uint32_t)((q[16 + 4 * m + bb] >> 4) & 1) << (8 * bb + 2 * m + 1);
            }
          uint8_t* bp = Bc(c, 4);
          for (int i = 0; i < 4; ++i) bp[i] = (uint8_t)(bits >> (8 * i));
        }
      }
      break;
    }
    case Q6_K: {
      const uint8_t *ql = blk, *qh = blk + 128, *sc = blk + 192;
      C[2 * b] = blk[208];
      C[2 * b + 1] = blk[209];
      for (int s = 0; s < 8; ++s) {
        int q[32];
        for (int e = 0; e < 32; ++e) q[e] = canon_q6k(ql, qh, 32 * s + e);
        const int64_t c = 8 * b + s;
        pack_nibbles(q, Qc(c));
        uint32_t w[2] = {0, 0};
        for (int i = 0; i < 2; ++i)
          for (int bb = 0; bb < 4; ++bb) {
            const int e0 = 4 * (2 * i) + bb, e1 = 16 + 4 * (2 * i) + bb;
            const int e2 = 4 * (2 * i + 1) + bb, e3 = 16 + 4 * (2 * i + 1) + bb;
            // high pairs XOR 2 (the sign flip of q - 32 in 6-bit two's complement)
            const uint32_t v = (uint32_t)((((q[e0] >> 4) & 3) ^ 2) | ((((q[e1] >> 4) & 3) ^ 2) << 2) |
                                          ((((q[e2] >> 4) & 3) ^ 2) << 4) | ((((q[e3] >> 4) & 3) ^ 2) << 6));
            w[i] |= v << (8 * bb);
          }
        uint8_t* ap = Ac(c, 8);
        for (int i = 0; i < 8; ++i) ap[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        uint8_t* bp = Bc(c, 2);
        bp[0] = sc[2 * s];
        bp[1] = sc[2 * s + 1];
      }
      break;
    }
    default: break;
  }
}

}  // namespace qwg
