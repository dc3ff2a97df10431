// qwg_ops.hip -- the other kernels of the decode step for gfx950: repack, dequantize, embedding
// row, RMSNorm, RoPE, grouped-query decode attention over the fp16 KV cache, SwiGLU, cosine and
// argmax (the Llama pieces listed under "Key features" on the NTransformer page, and the cuda/
// kernel list of its "Architecture overview": GEMV, RMSNorm, RoPE, SwiGLU, softmax).
#include <hip/hip_runtime.h>

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
  const typename F::Raw r = F::load(w, row, c);
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
  int32_t t[MAX_COLS];
};

template <int QT>
__global__ void k_embed(MatView w, int64_t k, Tokens tok, int nc, float* h, int64_t h_stride) {
  using F = Fmt<QT>;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = blockIdx.y;
  if (c >= w.nch || n >= nc) return;
  const typename F::Raw r = F::load(w, tok.t[n], c);
  float v[F::CW];
  F::decode(r, c, v);
  float* o = h + (int64_t)n * h_stride + (int64_t)c * F::CW;
#pragma unroll
  for (int j = 0; j < F::CW; ++j) o[j] = v[j];
}

hipError_t launch_embed(int qt, const MatView& w, int64_t k, const int32_t* tokens, int nc, float* h, int64_t h_stride,
                        hipStream_t st) {
  Tokens tk{};
  for (int i = 0; i < nc && i < MAX_COLS; ++i) tk.t[i] = tokens[i];
  dim3 g((w.nch + 127) / 128, nc), b(128);
  switch (qt) {
    case Q8_0: hipLaunchKernelGGL(k_embed<Q8_0>, g, b, 0, st, w, k, tk, nc, h, h_stride); break;
    case Q4_0: hipLaunchKernelGGL(k_embed<Q4_0>, g, b, 0, st, w, k, tk, nc, h, h_stride); break;
    case Q4_K: hipLaunchKernelGGL(k_embed<Q4_K>, g, b, 0, st, w, k, tk, nc, h, h_stride); break;
    case Q5_K: hipLaunchKernelGGL(k_embed<Q5_K>, g, b, 0, st, w, k, tk, nc, h, h_stride); break;
    case Q6_K: hipLaunchKernelGGL(k_embed<Q6_K>, g, b, 0, st, w, k, tk, nc, h, h_stride); break;
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

// greater-than for (value, index) with NaNs ignored and ties to the lower index
__device__ __forceinline__ bool am_better(float v, int i, float bv, int bi) {
  if (v != v) return false;
  if (bv != bv) return true;
  return v > bv || (v == bv && i < bi);
}

__global__ void k_argmax(const float* x, int64_t n, int64_t stride, int32_t* out) {
  __shared__ float shv[16];
  __shared__ int shi[16];
  const float* xr = x + (int64_t)blockIdx.x * stride;
  float bv = __builtin_nanf("");
  int bi = 0x7FFFFFFF;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const float v = xr[i];
    if (am_better(v, (int)i, bv, bi)) { bv = v; bi = (int)i; }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (am_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) { shv[wave] = bv; shi[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < nw; ++w)
      if (am_better(shv[w], shi[w], bv, bi)) { bv = shv[w]; bi = shi[w]; }
    out[blockIdx.x] = bi == 0x7FFFFFFF ? 0 : bi;
  }
}

hipError_t launch_argmax(const float* x, int64_t n, int nc, int64_t x_stride, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax, dim3(nc), dim3(1024), 0, st, x, n, x_stride, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ attention
//
// Split over positions (flash-decoding style) so that 8 KV heads still fill 256 CUs: workgroup
// (g, s) takes KV head g and positions [s*T, (s+1)*T) for all query heads of the group and all
// columns, writes (max, sum, unnormalised output) per query, and a second kernel merges the
// splits with the usual log-sum-exp rescaling.  K and V tiles are staged in LDS (K rows padded to
// 65 words so that lanes reading different positions hit different banks).

struct AttnArgs {
  const float* q;
  int64_t q_stride;
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t kv_stride;
  int n_pos;
  int n_q, n_kv, nc;
  int T, nsplit;
  float* part;  // [n_kv][nsplit][NQ][HEAD_DIM + 2]
  float* out;
  int64_t out_stride;
};

constexpr int KROW = HEAD_DIM / 2 + 1;  // padded K row in 32-bit words

AttnPlan plan_attn(int n_pos, int n_q, int n_kv, int nc) {
  AttnPlan p{};
  const int nqg = nc * (n_q / n_kv);
  p.T = nqg > 32 ? 32 : 64;
  const int span = n_pos + nc - 1;
  p.nsplit = (span + p.T - 1) / p.T;
  p.work_bytes = (size_t)n_kv * p.nsplit * nqg * (HEAD_DIM + 2) * sizeof(float);
  return p;
}

__global__ __launch_bounds__(256) void k_attn_part(AttnArgs a) {
  extern __shared__ float sm[];
  const int g = blockIdx.x, s = blockIdx.y;
  const int G = a.n_q / a.n_kv, NQ = a.nc * G, T = a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* qs = sm;                                   // [NQ][HEAD_DIM]
  uint32_t* ks = (uint32_t*)(qs + NQ * HEAD_DIM);   // [T][KROW]
  uint16_t* vs = (uint16_t*)(ks + T * KROW);        // [T][HEAD_DIM]
  float* ps = (float*)(vs + T * HEAD_DIM);          // [NQ][T]
  const int t0 = s * T;
  const int span = a.n_pos + a.nc - 1;
  const int tn = min(T, span - t0);                 // positions present in this split

  for (int i = tid; i < NQ * HEAD_DIM; i += blockDim.x) {
    const int qi = i / HEAD_DIM, d = i % HEAD_DIM;
    const int n = qi / G, j = qi % G;
    qs[i] = a.q[(int64_t)n * a.q_stride + (int64_t)(g * G + j) * HEAD_DIM + d];
  }
  for (int i = tid; i < T * (HEAD_DIM / 2); i += blockDim.x) {
    const int t = i / (HEAD_DIM / 2), w = i % (HEAD_DIM / 2);
    uint32_t kv = 0, vv = 0;
    if (t < tn) {
      const int64_t off = (int64_t)(t0 + t) * a.kv_stride + (int64_t)g * HEAD_DIM;
      kv = ((const uint32_t*)(a.kc + off))[w];
      vv = ((const uint32_t*)(a.vc + off))[w];
    }
    ks[t * KROW + w] = kv;
    ((uint32_t*)vs)[t * (HEAD_DIM / 2) + w] = vv;
  }
  __syncthreads();

  // scores: wave w takes queries w, w+4, ...; lane t takes position t0 + t (two passes if T = 64 > lanes? no: T <= 64)
  const float scale = 0.08838834764831845f;  // 1/sqrt(128)
  for (int qi = wave; qi < NQ; qi += 4) {
    const int n = qi / G;
    float sc = -INFINITY;
    if (lane < tn) {
      const float* qv = qs + qi * HEAD_DIM;
      const uint32_t* kr = ks + lane * KROW;
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
      for (int w = 0; w < HEAD_DIM / 2; ++w) {
        const uint32_t kk = kr[w];
        acc0 += qv[2 * w] * half_bits_to_float(kk & 0xFFFFu);
        acc1 += qv[2 * w + 1] * half_bits_to_float(kk >> 16);
      }
      if (t0 + lane < a.n_pos + n) sc = (acc0 + acc1) * scale;
    }
    const float m = wave_max(sc);
    const float e = (sc == -INFINITY) ? 0.f : __expf(sc - m);
    const float l = wave_sum(e);
    if (lane < T) ps[qi * T + lane] = e;
    if (lane == 0) {
      float* pr = a.part + (((int64_t)g * a.nsplit + s) * NQ + qi) * (HEAD_DIM + 2);
      pr[0] = m;
      pr[1] = l;
    }
  }
  __syncthreads();

  // unnormalised output: thread takes dimension d = tid % 128 for queries tid/128, +2, ...
  const int d = tid % HEAD_DIM;
  for (int qi = tid / HEAD_DIM; qi < NQ; qi += blockDim.x / HEAD_DIM) {
    const float* pr = ps + qi * T;
    float o = 0.f;
    for (int t = 0; t < tn; ++t) o += pr[t] * half_bits_to_float(vs[t * HEAD_DIM + d]);
    a.part[(((int64_t)g * a.nsplit + s) * NQ + qi) * (HEAD_DIM + 2) + 2 + d] = o;
  }
}

__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
  const int g = blockIdx.x, qi = blockIdx.y, d = threadIdx.x;
  const int G = a.n_q / a.n_kv, NQ = a.nc * G;
  const float* base = a.part + ((int64_t)g * a.nsplit * NQ + qi) * (HEAD_DIM + 2);
  const int64_t sstride = (int64_t)NQ * (HEAD_DIM + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, base[s * sstride]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float* pr = base + s * sstride;
    const float f = pr[0] == -INFINITY ? 0.f : __expf(pr[0] - M);
    L += f * pr[1];
    O += f * pr[2 + d];
  }
  const int n = qi / G, j = qi % G;
  a.out[(int64_t)n * a.out_stride + (int64_t)(g * G + j) * HEAD_DIM + d] = O / L;
}

hipError_t launch_attn(const float* q, int64_t q_stride, const uint16_t* kc, const uint16_t* vc, int64_t kv_stride,
                       int n_pos, int n_q, int n_kv, int nc, float* out, int64_t out_stride, void* work,
                       const AttnPlan& p, hipStream_t st) {
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
  a.T = p.T;
  a.nsplit = p.nsplit;
  a.part = (float*)work;
  a.out = out;
  a.out_stride = out_stride;
  const int NQ = nc * (n_q / n_kv);
  const size_t lds = (size_t)NQ * HEAD_DIM * 4 + (size_t)p.T * KROW * 4 + (size_t)p.T * HEAD_DIM * 2 +
                     (size_t)NQ * p.T * 4;
  hipLaunchKernelGGL(k_attn_part, dim3(n_kv, p.nsplit), dim3(256), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(n_kv, NQ), dim3(HEAD_DIM), 0, st, a);
  return hipGetLastError();
}

}  // namespace qwg
