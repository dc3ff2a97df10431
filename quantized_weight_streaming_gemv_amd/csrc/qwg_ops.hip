// qwg_ops.hip -- the other kernels of the decode step for gfx950: repack, dequantize, embedding
// row, RMSNorm, RoPE, grouped-query decode attention over the fp16 KV cache, SwiGLU, cosine and
// argmax (the Llama pieces listed under "Key features" on the NTransformer page, [NT] below, and
// the cuda/ kernel list of its "Architecture overview": GEMV, RMSNorm, RoPE, SwiGLU, softmax).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qwg_kernels.h"

namespace qwg {

// ------------------------------------------------------------------------------------------ repack

__global__ void k_repack(int qt, const uint8_t* canon, uint8_t* packed, Layout L, int64_t nrows, int64_t nb,
                         int64_t row_bytes, int64_t dst_row0, int64_t dst_row_step) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nrows * nb) return;
  const int64_t r = i / nb, b = i % nb;
  repack_block(qt, canon + r * row_bytes + b * block_bytes(qt), packed, L, dst_row0 + r * dst_row_step, b);
}

hipError_t launch_repack(int qt, const uint8_t* canon, int64_t rows, int64_t k, uint8_t* packed, const Layout& L,
                         int64_t dst_row0, int64_t dst_row_step, hipStream_t st) {
  const int64_t nb = k / block_weights(qt);
  const int64_t n = rows * nb;
  if (n == 0) return hipSuccess;
  const int64_t row_bytes = nb * block_bytes(qt);
  hipLaunchKernelGGL(k_repack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, qt, canon, packed, L, rows, nb,
                     row_bytes, dst_row0, dst_row_step);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ dequantize

template <int QT>
__global__ void k_dequant(MatView w, int64_t rows, int64_t k, float* out) {
  using F = Fmt<QT>;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * w.nch) return;
  const int64_t row = i / w.nch;
  const int c = (int)(i % w.nch);
  const typename F::Raw r = F::load(w, row_off(QT, w, row), c, slot_row(w.ilv, w.nch, row) + slot_chunk(w.ilv, (uint32_t)c));
  float v[F::CW];
  F::decode(r, c, v);
  float4* o = (float4*)(out + row * k + (int64_t)c * F::CW);
#pragma unroll
  for (int j = 0; j < F::CW / 4; ++j) o[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
}

hipError_t launch_dequant(int qt, const MatView& w, int64_t rows, int64_t k, float* out, hipStream_t st) {
  const int64_t n = rows * w.nch;
  if (n == 0) return hipSuccess;
  dim3 g((unsigned)((n + 255) / 256)), b(256);
  switch (qt) {
    case Q8_0: hipLaunchKernelGGL(k_dequant<Q8_0>, g, b, 0, st, w, rows, k, out); break;
    case Q4_0: hipLaunchKernelGGL(k_dequant<Q4_0>, g, b, 0, st, w, rows, k, out); break;
    case Q4_K: hipLaunchKernelGGL(k_dequant<Q4_K>, g, b, 0, st, w, rows, k, out); break;
    case Q5_K: hipLaunchKernelGGL(k_dequant<Q5_K>, g, b, 0, st, w, rows, k, out); break;
    case Q6_K: hipLaunchKernelGGL(k_dequant<Q6_K>, g, b, 0, st, w, rows, k, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ embedding row

struct Tokens {
  int32_t t[MAX_PREFILL_COLS];
};

template <int QT>
__global__ void k_embed(MatView w, Tokens tok, int nc, float* h, int64_t h_stride) {
  using F = Fmt<QT>;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = blockIdx.y;
  if (c >= w.nch || n >= nc) return;
  const typename F::Raw r =
      F::load(w, row_off(QT, w, tok.t[n]), c, slot_row(w.ilv, w.nch, tok.t[n]) + slot_chunk(w.ilv, (uint32_t)c));
  float v[F::CW];
  F::decode(r, c, v);
  float* o = h + (int64_t)n * h_stride + (int64_t)c * F::CW;
#pragma unroll
  for (int j = 0; j < F::CW; ++j) o[j] = v[j];
}

hipError_t launch_embed(int qt, const MatView& w, int64_t k, const int32_t* tokens, int nc, float* h, int64_t h_stride,
                        hipStream_t st) {
  (void)k;  // the row length is the matrix view's
  if (nc < 1 || nc > MAX_PREFILL_COLS) return hipErrorInvalidValue;  // one token slot per column
  Tokens tk{};
  for (int i = 0; i < nc; ++i) tk.t[i] = tokens[i];
  dim3 g((w.nch + 127) / 128, nc), b(128);
  switch (qt) {
    case Q8_0: hipLaunchKernelGGL(k_embed<Q8_0>, g, b, 0, st, w, tk, nc, h, h_stride); break;
    case Q4_0: hipLaunchKernelGGL(k_embed<Q4_0>, g, b, 0, st, w, tk, nc, h, h_stride); break;
    case Q4_K: hipLaunchKernelGGL(k_embed<Q4_K>, g, b, 0, st, w, tk, nc, h, h_stride); break;
    case Q5_K: hipLaunchKernelGGL(k_embed<Q5_K>, g, b, 0, st, w, tk, nc, h, h_stride); break;
    case Q6_K: hipLaunchKernelGGL(k_embed<Q6_K>, g, b, 0, st, w, tk, nc, h, h_stride); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ block reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// sum over a block of up to 1024 threads; every thread gets the total
__device__ float block_sum(float v, float* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += sh[i];
  return t;
}

// ------------------------------------------------------------------------------------------ RMSNorm

__global__ void k_rmsnorm(const float* x, const float* g, int64_t n, float eps, float* out) {
  __shared__ float sh[16];
  const float* xr = x + (int64_t)blockIdx.x * n;
  float* o = out + (int64_t)blockIdx.x * n;
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += xr[i] * xr[i];
  s = block_sum(s, sh);
  const float rs = 1.0f / sqrtf(s / (float)n + eps);
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) o[i] = g[i] * (xr[i] * rs);
}

hipError_t launch_rmsnorm(const float* x, const float* g, int64_t n, float eps, int nc, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(nc), dim3(1024), 0, st, x, g, n, eps, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ RoPE

__global__ void k_rope(float* v, int n_heads, const float* table, int pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // pair index over all heads
  if (i >= n_heads * (HEAD_DIM / 2)) return;
  const int j = i % (HEAD_DIM / 2);
  const float2 cs = ((const float2*)table)[(int64_t)pos * (HEAD_DIM / 2) + j];
  float2* p = (float2*)v + i;
  const float2 ab = *p;
  *p = make_float2(ab.x * cs.x - ab.y * cs.y, ab.x * cs.y + ab.y * cs.x);
}

hipError_t launch_rope(float* v, int n_heads, const float* table, int pos, hipStream_t st) {
  const int n = n_heads * (HEAD_DIM / 2);
  hipLaunchKernelGGL(k_rope, dim3((n + 255) / 256), dim3(256), 0, st, v, n_heads, table, pos);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ SwiGLU, cosine, argmax

__global__ void k_swiglu(const float* g, const float* u, int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float z = g[i];
    out[i] = z / (1.0f + __expf(-z)) * u[i];
  }
}

hipError_t launch_swiglu(const float* g, const float* u, int64_t n, float* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g, u, n, out);
  return hipGetLastError();
}

__global__ void k_cosine(const float* a, const float* b, int64_t n, float* out) {
  __shared__ float sh[16];
  float ab = 0.f, aa = 0.f, bb = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    ab += a[i] * b[i];
    aa += a[i] * a[i];
    bb += b[i] * b[i];
  }
  ab = block_sum(ab, sh);
  aa = block_sum(aa, sh);
  bb = block_sum(bb, sh);
  if (threadIdx.x == 0) *out = (aa == 0.f || bb == 0.f) ? 0.f : ab / (sqrtf(aa) * sqrtf(bb));
}

hipError_t launch_cosine(const float* a, const float* b, int64_t n, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_cosine, dim3(1), dim3(1024), 0, st, a, b, n, out);
  return hipGetLastError();
}

// Greedy choice over many workgroups: each reduces its slice to (value, index) and folds it into a
// 64-bit key with one atomic max; key = (order-preserving bits of the value) << 32 | ~index, so the
// largest value wins and, among equal values, the lowest index.  A NaN ranks above every number (its
// value bits become all ones), so a non-finite logit vector is visible in the chosen token: the first
// NaN wins, as numpy's argmax does.
__device__ __forceinline__ unsigned long long am_key(float v, int i) {
  uint32_t b = __float_as_uint(v);
  if (v != v) return (0xFFFFFFFFull << 32) | (uint32_t)(~(uint32_t)i);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)b << 32) | (uint32_t)(~(uint32_t)i);
}

__global__ void k_argmax_clear(unsigned long long* keys, int nc) {
  if ((int)threadIdx.x < nc) keys[threadIdx.x] = 0ull;
}

__global__ __launch_bounds__(256) void k_argmax_blocks(const float* x, int64_t n, int64_t stride,
                                                       unsigned long long* keys) {
  const float* xr = x + (int64_t)blockIdx.y * stride;
  unsigned long long best = 0ull;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const unsigned long long k = am_key(xr[i], (int)i);
    best = k > best ? k : best;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if ((threadIdx.x & 63) == 0 && best) atomicMax(keys + blockIdx.y, best);
}

__global__ void k_argmax_final(const unsigned long long* keys, int nc, int32_t* out) {
  const int j = threadIdx.x;
  if (j < nc) out[j] = keys[j] ? (int32_t)(~(uint32_t)(keys[j] & 0xFFFFFFFFull)) : 0;
}

// keys: nc 64-bit words of scratch
hipError_t launch_argmax(const float* x, int64_t n, int nc, int64_t x_stride, int32_t* out, hipStream_t st,
                         unsigned long long* keys) {
  hipLaunchKernelGGL(k_argmax_clear, dim3(1), dim3(64), 0, st, keys, nc);
  const int blocks = (int)std::min<int64_t>(256, (n + 1023) / 1024);
  hipLaunchKernelGGL(k_argmax_blocks, dim3(blocks, nc), dim3(256), 0, st, x, n, x_stride, keys);
  hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(64), 0, st, keys, nc, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ attention
//
// Split over positions (flash-decoding style) so that 8 KV heads still fill 256 CUs: workgroup
// (g, s) takes KV head g and positions [s*T, s*T + T) for every query head of the group and every
// column, and writes (max, sum, unnormalised output) per query; a second kernel merges the splits
// with the usual log-sum-exp rescaling.
//   scores: lane = position (T = 64), the K row (256 B) is read straight into registers with
//           16-B loads; queries come from LDS as broadcasts; wave w takes queries w, w+4, ...
//   output: thread = (2 dimensions, one query slot); V rows are read as coalesced 256-B rows.

struct AttnArgs {
  const float* q;
  int64_t q_stride;
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t kv_stride;
  int n_pos;
  int n_q, n_kv, nc;
  int nsplit;
  int tiles;      // ATT_T-position tiles per split (the matrix-core form; k_attn takes one)
  float* part;    // [n_kv][nsplit][NQ][HEAD_DIM + 2]: split max, sum and unnormalised output
  float* out;
  int64_t out_stride;
  uint32_t* dig;  // digits of the output for the next GEMV (column stride dig_stride words), or null
  int64_t dig_stride;
  int dig_kind;
};

constexpr int ATT_T = 64;                // positions per split (one per lane)
constexpr int KROW = HEAD_DIM + 8;       // halves per K row in LDS: the 16-B pad keeps row reads conflict-free
// waves per workgroup of k_attn: one query row each at G = 8 (four waves of two rows each kept a
// 128-register converted K row per wave and measured 8.0 against 7.3 us per decode layer)
constexpr int ATT_WAVES = 8;
constexpr int ATT_THREADS = 64 * ATT_WAVES;

AttnPlan plan_attn(int n_pos, int n_q, int n_kv, int nc) {
  AttnPlan p{};
  const int nqg = nc * (n_q / n_kv);
  const int span = n_pos + nc - 1;
  p.T = ATT_T;
  if (nqg >= 32) {
    // the matrix-core form: splits of up to four tiles while the grid keeps about two workgroups
    // per CU (fewer, longer splits leave the merge less to combine)
    const int64_t wg1 = (int64_t)n_kv * ((span + ATT_T - 1) / ATT_T) * ((nc + std::max(1, 64 / (n_q / n_kv)) - 1) /
                                                                     std::max(1, 64 / (n_q / n_kv)));
    while (p.T < 4 * ATT_T && wg1 * ATT_T / (2 * p.T) >= 512) p.T *= 2;
  }
  p.nsplit = (span + p.T - 1) / p.T;
  p.work_bytes = (size_t)n_kv * p.nsplit * nqg * (HEAD_DIM + 2) * sizeof(float);
  return p;
}

size_t attn_work_bound(int n_pos, int n_q, int n_kv, int nc) {
  // single-tile splits have the most records; longer splits only ever need fewer
  const int64_t span = (int64_t)n_pos + nc - 1;
  return (size_t)n_kv * (size_t)((span + ATT_T - 1) / ATT_T) * (size_t)nc * (size_t)(n_q / n_kv) * (HEAD_DIM + 2) *
         sizeof(float);
}

// LDS of a k_attn workgroup for G query rows: q, scores, the K and V tiles
static size_t attn_lds_bytes(int rows) {
  return (size_t)rows * HEAD_DIM * 4 + (size_t)rows * ATT_T * 4 + (size_t)ATT_T * KROW * 2 + (size_t)ATT_T * HEAD_DIM * 2;
}
// Grouped-query attention over the fp16 KV cache ([NT] "Key features": GQA, KV cache).
// Decode steps and narrow verify passes (fewer than 32 query rows per KV head): one workgroup per
// (kv head g, split s of ATT_T positions, column n0) for the G = n_q / n_kv query rows of the group
// (GQA: query heads g*G .. g*G+G-1 share K/V head g), so a verify's rows spread over more CUs.  Wave
// w owns query rows w, w + ATT_WAVES, ...:
//   1. the K and V tiles and the queries are staged in LDS (every global load issued up front);
//   2. lane t scores position t0 + t against each of the wave's rows (scale 1/sqrt(128)), reading its
//      K row from LDS in 8-dimension pieces converted inside the FMAs, with causal masking, and keeps
//      the split's max m, sum l and exp(score - m);
//   3. the unnormalised output sum_t exp(.) v_t goes to the workspace with m and l;
// k_attn_merge then combines the splits.
__global__ __launch_bounds__(ATT_THREADS) void k_attn(AttnArgs a) {
  extern __shared__ float sm[];
  const int g = blockIdx.x, s = blockIdx.y, n0 = blockIdx.z;
  const int G = a.n_q / a.n_kv, NQ = a.nc * G;
  const int R = G;  // query rows: head g*G + j of column n0
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* qs = sm;                                // [G][HEAD_DIM]
  float* ps = qs + G * HEAD_DIM;                 // [G][ATT_T]
  uint16_t* ks = (uint16_t*)(ps + G * ATT_T);    // [ATT_T][KROW]
  uint16_t* vs = ks + ATT_T * KROW;              // [ATT_T][HEAD_DIM]
  const int t0 = s * ATT_T;
  const int span = a.n_pos + a.nc - 1;
  const int tn = min(ATT_T, span - t0);

  // 1. tiles: thread i takes 16-B piece i & 15 of rows i >> 4, + ATT_THREADS / 16, ... (rows past
  //    the span re-read the last valid one and are masked below)
  constexpr int TP = ATT_T * 16 / ATT_THREADS;  // tile pieces per thread
  {
    uint4 kv[TP], vv[TP];
#pragma unroll
    for (int j = 0; j < TP; ++j) {
      const int i = tid + ATT_THREADS * j, t = i >> 4, c = i & 15;
      const int64_t off = (int64_t)(t0 + min(t, tn - 1)) * a.kv_stride + (int64_t)g * HEAD_DIM + c * 8;
      kv[j] = *(const uint4*)(a.kc + off);
      vv[j] = *(const uint4*)(a.vc + off);
    }
    for (int i = tid; i < R * (HEAD_DIM / 4); i += ATT_THREADS) {
      const int j = i / (HEAD_DIM / 4), d4 = i % (HEAD_DIM / 4);
      ((float4*)qs)[i] = ((const float4*)(a.q + (int64_t)n0 * a.q_stride + (int64_t)(g * G + j) * HEAD_DIM))[d4];
    }
#pragma unroll
    for (int j = 0; j < TP; ++j) {
      const int i = tid + ATT_THREADS * j, t = i >> 4, c = i & 15;
      *(uint4*)(ks + t * KROW + c * 8) = kv[j];
      *(uint4*)(vs + t * HEAD_DIM + c * 8) = vv[j];
    }
  }
  __syncthreads();

  // 2. scores and split-local softmax statistics (four accumulators per row: dimensions 4i + c)
  const float scale = 0.08838834764831845f;  // 1/sqrt(128)
  for (int j = wave; j < R; j += ATT_WAVES) {
    const float4* qv = (const float4*)(qs + j * HEAD_DIM);
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int i = 0; i < HEAD_DIM / 8; ++i) {
      const uint4 kp = *(const uint4*)(ks + lane * KROW + i * 8);
      const uint32_t kw[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 qq = qv[2 * i + h];
        a0 += qq.x * half_bits_to_float(kw[2 * h] & 0xFFFFu);
        a1 += qq.y * half_bits_to_float(kw[2 * h] >> 16);
        a2 += qq.z * half_bits_to_float(kw[2 * h + 1] & 0xFFFFu);
        a3 += qq.w * half_bits_to_float(kw[2 * h + 1] >> 16);
      }
    }
    const int qi = n0 * G + j;
    const bool ok = lane < tn && t0 + lane < a.n_pos + n0;
    const float sc = ok ? ((a0 + a1) + (a2 + a3)) * scale : -INFINITY;
    const float m = wave_max(sc);
    const float e = ok ? __expf(sc - m) : 0.f;
    const float l = wave_sum(e);
    ps[j * ATT_T + lane] = e;
    if (lane == 0) {
      float* pr = a.part + (((int64_t)g * a.nsplit + s) * NQ + qi) * (HEAD_DIM + 2);
      pr[0] = m;
      pr[1] = l;
    }
  }
  __syncthreads();

  // 3. unnormalised output: wave w takes query rows w, w + ATT_WAVES, ...; lane = dimensions 2 lane,
  //    2 lane + 1.  The weights of four positions come in one broadcast read.
  for (int j = wave; j < R; j += ATT_WAVES) {
    const int qb = n0 * G + j;
    const float* pr = ps + j * ATT_T;
    const uint32_t* vw = (const uint32_t*)vs + lane;  // dimension pair of the lane, row stride HEAD_DIM / 2
    float o0 = 0.f, o1 = 0.f;
    int t = 0;
#pragma unroll 2
    for (; t + 4 <= tn; t += 4) {
      const float4 p4 = *(const float4*)(pr + t);
      const float pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t vv = vw[(t + u) * (HEAD_DIM / 2)];
        o0 += pp[u] * half_bits_to_float(vv & 0xFFFFu);
        o1 += pp[u] * half_bits_to_float(vv >> 16);
      }
    }
    for (; t < tn; ++t) {
      const uint32_t vv = vw[t * (HEAD_DIM / 2)];
      const float p = pr[t];
      o0 += p * half_bits_to_float(vv & 0xFFFFu);
      o1 += p * half_bits_to_float(vv >> 16);
    }
    float* dst = a.part + (((int64_t)g * a.nsplit + s) * NQ + qb) * (HEAD_DIM + 2) + 2;
    *(float2*)(dst + 2 * lane) = make_float2(o0, o1);
  }
}

// Passes of 32 or more query rows per KV head (the prompt pass, [NT] "Quick start": -p; the
// self-speculative verify pass, [NT] "Key features") on the matrix cores: one workgroup per (kv
// head g, split s of ATT_T positions, block of cpw columns) holds up to 64 query rows (cpw = 64 / G
// columns), 16 per wave, and computes them with v_mfma_f32_16x16x32_f16 (fp32 accumulation).  K and
// V enter as the fp16 values the cache holds; a query row is scaled by a power of two (its maximum
// into [2^14, 2^15)) and split into fp16 pieces hi + lo (22 significant bits), and so are the softmax
// weights (in [0, 1]), so every product keeps about fp32 precision.  With lane l = 16 kk + i:
//   1. the K tile (row-major) and the V tile (transposed: dimension-major, the positions of each
//      32-position block ordered 4 kk .. 4 kk + 3, 16 + 4 kk .. 16 + 4 kk + 3 per lane group kk) are
//      staged in LDS; the lane loads dimensions 32 st + 8 kk .. 32 st + 7 + 8 kk of its query row i;
//   2. S^T = K Q^T per 16-position tile: A = K rows (positions), B = the query pieces, contracting
//      over 32 dimensions per MFMA, so the lane receives S[position 4 kk + v][row i], v = 0..3;
//   3. per row: split max m, exp(s - m) and sum l (across the four lanes 16 kk + i) with causal masking;
//   4. O = P V per 32-position block: the eight weights the lane holds (positions 4 kk + v and
//      16 + 4 kk + v of the block) are exactly its A operand, and one 16-byte read of the transposed V
//      tile is the B operand of a 16-dimension tile;
//   5. the unnormalised output, m and l go to the workspace for k_attn_merge, as in k_attn.
constexpr int AM_WAVES = 4;
constexpr int VROW = ATT_T + 8;  // halves per dimension row of the transposed V tile (16-B pad)
typedef float qwg_f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 qwg_h8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ qwg_f32x4 mfma_h16(const uint4& a, const uint4& b, qwg_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(qwg_h8, a), __builtin_bit_cast(qwg_h8, b), c, 0, 0,
                                                0);
}
// fp16 pieces of (a, b): hi = fp16(x) and lo = fp16(x - hi), as half pairs
__device__ __forceinline__ void split_h2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const _Float16 ah = (_Float16)a, bh = (_Float16)b;
  const _Float16 al = (_Float16)(a - (float)ah), bl = (_Float16)(b - (float)bh);
  hi = (uint32_t)__builtin_bit_cast(uint16_t, ah) | ((uint32_t)__builtin_bit_cast(uint16_t, bh) << 16);
  lo = (uint32_t)__builtin_bit_cast(uint16_t, al) | ((uint32_t)__builtin_bit_cast(uint16_t, bl) << 16);
}
static size_t attn_mfma_lds_bytes() { return (size_t)ATT_T * KROW * 2 + (size_t)HEAD_DIM * VROW * 2; }

__global__ __launch_bounds__(64 * AM_WAVES) void k_attn_mfma(AttnArgs a, int cpw) {
  extern __shared__ float sm[];
  uint16_t* ks = (uint16_t*)sm;      // [ATT_T][KROW]
  uint16_t* vt = ks + ATT_T * KROW;  // [HEAD_DIM][VROW]
  const int g = blockIdx.x, s = blockIdx.y, n0 = blockIdx.z * cpw;
  const int G = a.n_q / a.n_kv, NQ = a.nc * G;
  const int R = min(cpw, a.nc - n0) * G;  // rows of this workgroup: column n0 + j / G, head g*G + j % G
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, kk = lane >> 4;
  const int span = a.n_pos + a.nc - 1;
  const bool rows = wave * 16 < R;  // this wave has query rows (wave-uniform)
  const int jr = wave * 16 + i;     // the query row of this lane
  const bool rvalid = jr < R;
  const int jq = min(jr, R - 1);
  const int ncol = n0 + jq / G;

  // the query row's dimensions 32 st + 8 kk .. 32 st + 7 + 8 kk, its scale (its four lanes share the
  // maximum) and pieces
  uint4 qh[4], ql[4];
  int qsh = 0;
  {
    float qf[32];  // dimension 32 st + 8 kk + e at qf[8 st + e]
    const float4* qp =
        (const float4*)(a.q + (int64_t)ncol * a.q_stride + (int64_t)(g * G + jq % G) * HEAD_DIM + 8 * kk);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 v = qp[8 * st + h];
        qf[8 * st + 4 * h] = v.x;
        qf[8 * st + 4 * h + 1] = v.y;
        qf[8 * st + 4 * h + 2] = v.z;
        qf[8 * st + 4 * h + 3] = v.w;
      }
    float qmx = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) qmx = fmaxf(qmx, fabsf(qf[e]));
    qmx = fmaxf(qmx, __shfl_xor(qmx, 16));
    qmx = fmaxf(qmx, __shfl_xor(qmx, 32));
    if (qmx > 0.f && qmx <= 3.4e38f) qsh = min(149, 15 - __builtin_amdgcn_frexp_expf(qmx));
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        split_h2(ldexpf(qf[8 * st + 2 * e], qsh), ldexpf(qf[8 * st + 2 * e + 1], qsh), h[e], l[e]);
      qh[st] = make_uint4(h[0], h[1], h[2], h[3]);
      ql[st] = make_uint4(l[0], l[1], l[2], l[3]);
    }
  }
  const float scale = ldexpf(0.08838834764831845f, -qsh);  // 1/sqrt(128), undoing the query's scale

  // the split's running max and sum of row i, and the unnormalised output (rows 4 kk + v)
  float m = -INFINITY, l = 0.f;
  qwg_f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = {0.f, 0.f, 0.f, 0.f};
  for (int u = 0; u < a.tiles; ++u) {
    const int t0 = (s * a.tiles + u) * ATT_T;
    const int tn = min(ATT_T, span - t0);
    if (tn <= 0) break;  // past the last position (the same for every wave)
    if (u > 0) __syncthreads();  // every wave is done with the previous tile

    // 1. the tile (every global load issued before the first LDS store: K rows with 16 threads per
    //    position, V with one thread per position and 8 dimensions)
    constexpr int TP = ATT_T * 16 / (64 * AM_WAVES);
    uint4 kv[TP], vv[TP];
#pragma unroll
    for (int j = 0; j < TP; ++j) {
      const int idx = tid + 64 * AM_WAVES * j;
      const int t = idx >> 4, c = idx & 15, tv = idx & 63, cv = idx >> 6;
      kv[j] = *(const uint4*)(a.kc + (int64_t)(t0 + min(t, tn - 1)) * a.kv_stride + (int64_t)g * HEAD_DIM + c * 8);
      vv[j] = *(const uint4*)(a.vc + (int64_t)(t0 + min(tv, tn - 1)) * a.kv_stride + (int64_t)g * HEAD_DIM + cv * 8);
    }
#pragma unroll
    for (int j = 0; j < TP; ++j) {
      const int idx = tid + 64 * AM_WAVES * j;
      const int t = idx >> 4, c = idx & 15, tv = idx & 63, cv = idx >> 6;
      *(uint4*)(ks + t * KROW + c * 8) = kv[j];
      const int slot = (tv & 32) + 8 * ((tv & 15) >> 2) + 4 * ((tv >> 4) & 1) + (tv & 3);
      const uint32_t w[4] = {vv[j].x, vv[j].y, vv[j].z, vv[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(8 * cv + e) * VROW + slot] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    if (!rows) continue;

    // 2. scores: per 16-position tile, 4 steps of 32 dimensions x two query pieces
    qwg_f32x4 sc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      qwg_f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint4 kr = *(const uint4*)(ks + (16 * pt + i) * KROW + 32 * st + 8 * kk);
        c = mfma_h16(kr, qh[st], c);
        c = mfma_h16(kr, ql[st], c);
      }
      sc[pt] = c;
    }

    // 3. softmax of row i over the positions 16 pt + 4 kk + v, folded into the split's running max
    //    and sum; alpha rescales what the earlier tiles left (0 before the first visible position)
    const int lim = a.n_pos + ncol - t0;  // positions below lim (and tn) are visible to the row
    float p[4][4], mt = -INFINITY;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int pos = 16 * pt + 4 * kk + v;
        const bool ok = rvalid && pos < tn && pos < lim;
        p[pt][v] = ok ? sc[pt][v] * scale : -INFINITY;
        mt = fmaxf(mt, p[pt][v]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    const float alpha = m == -INFINITY ? 0.f : __expf(m - mn);
    float lt = 0.f;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[pt][v] = p[pt][v] == -INFINITY ? 0.f : __expf(p[pt][v] - mn);
        lt += p[pt][v];
      }
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    l = l * alpha + lt;
    m = mn;
    if (u > 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, 4 * kk + v);  // row 4 kk + v's factor (lane 4 kk + v holds that row)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt][v] *= av;
      }
    }

    // 4. O += P V: per 32-position block, the weights' two pieces against 8 dimension tiles
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      uint32_t h[4], lo[4];
      split_h2(p[2 * b][0], p[2 * b][1], h[0], lo[0]);
      split_h2(p[2 * b][2], p[2 * b][3], h[1], lo[1]);
      split_h2(p[2 * b + 1][0], p[2 * b + 1][1], h[2], lo[2]);
      split_h2(p[2 * b + 1][2], p[2 * b + 1][3], h[3], lo[3]);
      const uint4 ph = make_uint4(h[0], h[1], h[2], h[3]), pl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint4 vb = *(const uint4*)(vt + (16 * dt + i) * VROW + 32 * b + 8 * kk);
        o[dt] = mfma_h16(ph, vb, o[dt]);
        o[dt] = mfma_h16(pl, vb, o[dt]);
      }
    }
  }
  if (!rows) return;

  // 5. records: lane 16 kk + i holds O[row 4 kk + v][dimension 16 dt + i]
  float* base = a.part + ((int64_t)g * a.nsplit + s) * NQ * (HEAD_DIM + 2);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int j = wave * 16 + 4 * kk + v;
    if (j < R) {
      float* dst = base + (int64_t)((n0 + j / G) * G + j % G) * (HEAD_DIM + 2) + 2;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) dst[16 * dt + i] = o[dt][v];
    }
  }
  if (kk == 0 && rvalid) {
    float* pr = base + (int64_t)((n0 + jr / G) * G + jr % G) * (HEAD_DIM + 2);
    pr[0] = m;
    pr[1] = l;
  }
}

// One workgroup of MW waves per (kv head g, query row qi) merges the splits in a fixed order,
//   M = max_s m_s,  o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
// Wave w takes the blocks of MB splits w, w + MW, w + 2 MW, ... (every load of a block goes out
// together: lane j < MB holds split j's (m, l), every lane the (2 lane, 2 lane + 1) outputs of the
// block), rescaling its running max, sum and output from block to block; the waves' partial
// (m, l, o) are then combined in wave order through LDS.  Wave 0 writes the output row (and its
// activation digits).  Spreading a row over four waves shortens the chain of dependent loads that
// bounds this small kernel.
constexpr int MW = 4;   // waves per merged row
constexpr int MB = 16;  // splits per block
__global__ __launch_bounds__(64 * MW) void k_attn_merge(AttnArgs a) {
  __shared__ float wsh[MW][MB];
  __shared__ float part_ml[MW][2];
  __shared__ float2 part_o[MW][64];
  __shared__ float ob[HEAD_DIM];
  const int g = blockIdx.x, qi = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.n_q / a.n_kv, NQ = a.nc * G;
  const int64_t sstride = (int64_t)NQ * (HEAD_DIM + 2);
  const float* base = a.part + ((int64_t)g * a.nsplit * NQ + qi) * (HEAD_DIM + 2);
  float M = -INFINITY, L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int b0 = wave * MB; b0 < a.nsplit; b0 += MW * MB) {
    const int nb = min(MB, a.nsplit - b0);
    const float2 st = *(const float2*)(base + (b0 + min(lane, nb - 1)) * sstride);
    float2 ov[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) ov[j] = *(const float2*)(base + (b0 + min(j, nb - 1)) * sstride + 2 + 2 * lane);
    const bool ok = lane < nb;
    const float mj = ok ? st.x : -INFINITY;
    const float Mn = fmaxf(M, wave_max(mj));
    const float wj = (ok && mj != -INFINITY) ? __expf(mj - Mn) : 0.f;
    const float keep = M == -INFINITY ? 0.f : __expf(M - Mn);
    L = L * keep + wave_sum(ok ? wj * st.y : 0.f);
    if (lane < MB) wsh[wave][lane] = wj;
    __builtin_amdgcn_wave_barrier();  // the weights are read back by every lane of this wave
    o0 *= keep;
    o1 *= keep;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const float w = wsh[wave][j];  // written by lanes of this wave (wave-synchronous)
      o0 += w * ov[j].x;
      o1 += w * ov[j].y;
    }
    __builtin_amdgcn_wave_barrier();
    M = Mn;
  }
  if (lane == 0) {
    part_ml[wave][0] = M;
    part_ml[wave][1] = L;
  }
  part_o[wave][lane] = make_float2(o0, o1);
  __syncthreads();
  if (wave != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < MW; ++w) Mt = fmaxf(Mt, part_ml[w][0]);
  float Lt = 0.f, t0 = 0.f, t1 = 0.f;
#pragma unroll
  for (int w = 0; w < MW; ++w) {
    const float mw = part_ml[w][0];
    const float f = mw == -INFINITY ? 0.f : __expf(mw - Mt);
    Lt += f * part_ml[w][1];
    t0 += f * part_o[w][lane].x;
    t1 += f * part_o[w][lane].y;
  }
  const float inv = 1.0f / Lt;
  const int n = qi / G, j = qi % G;
  const float2 o = make_float2(t0 * inv, t1 * inv);
  *(float2*)(a.out + (int64_t)n * a.out_stride + (int64_t)(g * G + j) * HEAD_DIM + 2 * lane) = o;
  if (a.dig) {
    // the head's 128 outputs are four whole 32-element chunks: four lanes per chunk (wave 0 only:
    // its lanes exchange through LDS without a workgroup barrier)
    ob[2 * lane] = o.x;
    ob[2 * lane + 1] = o.y;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const int m = lane & 3, c = (lane >> 2) & 3;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ob[c * 32 + (i < 4 ? 4 * m + i : 16 + 4 * m + i - 4)];
    const int64_t chunk = (int64_t)(g * G + j) * (HEAD_DIM / 32) + c;
    digitize_group(v, m, a.dig_kind, a.dig + (int64_t)n * a.dig_stride + chunk * DIG_CHUNK_WORDS, lane < 16);
  }
}

hipError_t launch_attn(const float* q, int64_t q_stride, const uint16_t* kc, const uint16_t* vc, int64_t kv_stride,
                       int n_pos, int n_q, int n_kv, int nc, float* out, int64_t out_stride, void* work,
                       const AttnPlan& p, hipStream_t st, uint32_t* dig_out, int64_t dig_stride, int dig_kind) {
  const int NQ = nc * (n_q / n_kv);
  if (n_q / n_kv > 64 || NQ > 4096 || p.nsplit < 1) return hipErrorInvalidValue;
  if (dig_out && dig_kind != DIG_NIB && dig_kind != DIG_BYTE) return hipErrorInvalidValue;  // per-chunk kinds only
  AttnArgs a;
  a.q = q;
  a.q_stride = q_stride;
  a.kc = kc;
  a.vc = vc;
  a.kv_stride = kv_stride;
  a.n_pos = n_pos;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.nc = nc;
  a.nsplit = p.nsplit;
  a.tiles = p.T / ATT_T;
  a.part = (float*)work;
  a.out = out;
  a.out_stride = out_stride;
  a.dig = dig_out;
  a.dig_stride = dig_stride;
  a.dig_kind = dig_kind;
  const int G = n_q / n_kv;
  if (nc * G >= 32) {
    // passes with at least two 16-row blocks of query rows (prompt prefill; a verify pass of 4 or
    // more columns at G = 8): 64 / G columns per workgroup on the matrix cores.  (A decode step's 8
    // rows fill half of one block, and one wave's 256 products measured 4% slower per decode step.)
    const int cpw = std::max(1, 64 / G);
    hipLaunchKernelGGL(k_attn_mfma, dim3(n_kv, p.nsplit, (nc + cpw - 1) / cpw), dim3(64 * AM_WAVES),
                       attn_mfma_lds_bytes(), st, a, cpw);
  } else {
    const size_t lds = attn_lds_bytes(G);
    if (lds > 150 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn, dim3(n_kv, p.nsplit, nc), dim3(ATT_THREADS), lds, st, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(n_kv, NQ), dim3(64 * MW), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ plain read

// Waits `ticks` of the constant-rate wall clock, then exits (a bounded delay for ordering tests).
__global__ void k_spin(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

hipError_t launch_spin(uint64_t ticks, hipStream_t st) {
  hipLaunchKernelGGL(k_spin, dim3(1), dim3(64), 0, st, ticks);
  return hipGetLastError();
}

// Streaming read of n16 16-byte words: wave w of the grid reads one contiguous segment, lane l the
// words l, l+64, ... of it, U 16-B non-temporal loads in flight per lane (the GEMV's own load
// pattern without its arithmetic).  One XOR checksum per wave keeps the loads alive.
template <int U>
__global__ __launch_bounds__(512) void k_read(const uint4* __restrict__ p, int64_t n16, int64_t per_wave,
                                              uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 6);
  const int64_t beg = wave * per_wave, end = min(beg + per_wave, n16);
  uint32_t acc = 0;
  for (int64_t i = beg + lane; i < end; i += 64 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + 64 * u;
      v[u] = j < end ? ld_stream_u4((const uint8_t*)(p + j)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if (lane == 0) sink[wave] = acc;
}

hipError_t launch_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st, int grid, int unroll,
                       hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int64_t n16 = bytes / 16;
  if (grid <= 0) grid = READ_GRID;
  if (unroll <= 0) unroll = 4;
  const int64_t waves = (int64_t)grid * 8;
  const int64_t per_wave = ((n16 + waves - 1) / waves + 63) / 64 * 64;
  const uint4* p = (const uint4*)src;
  switch (unroll) {
    case 4: hipExtLaunchKernelGGL(k_read<4>, dim3(grid), dim3(512), 0, st, ev_start, ev_stop, 0u, p, n16, per_wave, sink); break;
    case 8: hipExtLaunchKernelGGL(k_read<8>, dim3(grid), dim3(512), 0, st, ev_start, ev_stop, 0u, p, n16, per_wave, sink); break;
    case 16: hipExtLaunchKernelGGL(k_read<16>, dim3(grid), dim3(512), 0, st, ev_start, ev_stop, 0u, p, n16, per_wave, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qwg
