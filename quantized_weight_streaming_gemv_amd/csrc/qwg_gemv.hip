// qwg_gemv.hip -- fused dequantize-and-GEMV for gfx950 (the engine's hand-written GEMV kernels,
// NTransformer page "Architecture overview", cuda/; formats from the Show HN page's
// quantization-format table).
//
// Work decomposition (batch-1 decode is HBM-bound: every weight byte is read exactly once):
//   * a workgroup of W wave64s owns W*R consecutive output rows and one K split;
//   * each wave owns R rows; lane l walks chunks l, l+64, ... of those rows, so every wave-wide
//     load instruction reads 1 KiB of contiguous quant bytes (16 B per lane);
//   * the activation arrives as block fixed-point digits (one k_digitize launch per GEMV input,
//     see qwg_formats.h): 28 words per 32 elements, staged once per workgroup into LDS in a
//     chunk-transposed layout -- 16-B slot q of chunk c of column n at (n*7 + q)*nxp + c -- so
//     the 64 lanes of a wave read 64 consecutive slots, free of bank conflicts;
//   * quants stay integers: nibble formats feed v_dot8_i32_i4 directly (q - 8 by one XOR), the
//     others feed v_dot4_i32_i8 with one byte per quant; each chunk's integer sums are recombined
//     in fp32 and scaled once by the block scales and the activation chunk scale;
//   * an RMSNorm in front of the GEMV is folded in: the digits are of g*h and the per-column
//     scale 1/rms multiplies the finished row in the epilogue;
//   * the first chunk's weights are requested before the activation is staged, and each loop
//     iteration requests the next chunk before computing the current one;
//   * a 64-lane butterfly (shuffles) reduces each row; lanes 0..R-1 run the epilogue
//     (store, residual add, SwiGLU on interleaved gate|up rows, or RoPE + fp16 KV append).
//   * K splits (when the activation for all columns does not fit the LDS budget) write partial
//     sums that a second kernel adds in a fixed order, so results never depend on timing.
#include <hip/hip_runtime.h>

#include <cmath>

#include "qwg_kernels.h"

namespace qwg {

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ void run_epilogue(int epi, const EpiArgs& e, int n, int row, float v, float vp) {
  if (e.rs) {
    const float r = e.rs[n];
    v *= r;
    vp *= r;
  }
  switch (epi) {
    case EPI_STORE:
      e.y[(int64_t)n * e.y_stride + row] = v;
      break;
    case EPI_RESID:
      e.y[(int64_t)n * e.y_stride + row] += v;
      break;
    case EPI_SWIGLU:
      if ((row & 1) == 0) e.y[(int64_t)n * e.y_stride + (row >> 1)] = silu_f(v) * vp;
      break;
    case EPI_QKV: {
      const int pos = e.pos + n;
      if (row < e.nq_rows + e.nkv_rows) {
        const int i = (row % HEAD_DIM) >> 1;
        const float2 cs = ((const float2*)e.rope)[(int64_t)pos * (HEAD_DIM / 2) + i];
        // pair (a, b) = rows (2i, 2i+1): a' = a cos - b sin, b' = a sin + b cos
        const float out = (row & 1) == 0 ? (v * cs.x - vp * cs.y) : (vp * cs.y + v * cs.x);
        if (row < e.nq_rows)
          e.y[(int64_t)n * e.y_stride + row] = out;
        else
          e.kc[(int64_t)pos * e.kv_stride + (row - e.nq_rows)] = float_to_half_bits(out);
      } else {
        e.vc[(int64_t)pos * e.kv_stride + (row - e.nq_rows - e.nkv_rows)] = float_to_half_bits(v);
      }
      break;
    }
    default:
      break;
  }
}

struct GemvArgs {
  MatView w;
  const uint4* xd;      // activation digits: column n at xd + n * xd_stride, 7 slots per 32 elements
  int64_t xd_stride;    // in 16-B slots
  int nc;
  int k;
  int ks;
  float* part;
  EpiArgs e;
};

constexpr int XSLOTS = DIG_CHUNK_WORDS / 4;  // 16-B slots per activation chunk (6 digit slots + desc)

template <int QT, int NCM, int R, int EPI>
__global__ __launch_bounds__(512) void k_gemv(GemvArgs a) {
  using F = Fmt<QT>;
  constexpr int CW = F::CW;
  constexpr int WPX = XCHUNK / CW;               // weight chunks per activation chunk (2 for Q8_0)
  constexpr int NDS = (CW == 16) ? 3 : 6;        // digit slots one weight chunk reads
  extern __shared__ uint4 lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int nc = a.nc;
  const int split = blockIdx.y;
  const int kbeg = split * a.ks;
  const int klen = min(a.ks, a.k - kbeg);
  const int nxs = klen / XCHUNK;   // activation chunks of this split
  const int nxp = a.ks / XCHUNK;   // LDS stride
  const int xbase = kbeg / XCHUNK;
  const int nchs = klen / CW;      // weight chunks of this split
  const int cbase = kbeg / CW;
  const int rows = a.w.rows;
  const int row0 = (blockIdx.x * nw + wave) * R;
  const bool active = row0 < rows;

  // 1. request the first chunk of every row of this wave before staging the activation
  //    (rows past the end are clamped to the last row: loads stay in bounds, results are dropped)
  int rr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rr[r] = min(row0 + r, rows - 1);
  typename F::Raw cur[R];
  if (active && lane < nchs) {
#pragma unroll
    for (int r = 0; r < R; ++r) cur[r] = F::load(a.w, rr[r], cbase + lane);
  }

  // 2. stage this split's activation digits (coalesced 16-B reads, chunk-transposed LDS)
  for (int n = 0; n < nc; ++n) {
    const uint4* src = a.xd + (int64_t)n * a.xd_stride + (int64_t)xbase * XSLOTS;
    for (int i = tid; i < nxs * XSLOTS; i += blockDim.x) {
      const int c = i / XSLOTS, q = i % XSLOTS;
      lds[(n * XSLOTS + q) * nxp + c] = src[i];
    }
  }
  __syncthreads();
  if (!active) return;

  // 3. main loop over this lane's chunks
  const int sub = lane & 7;  // chunk index within its 256-weight superblock (splits start on superblocks)
  float acc[R][NCM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int n = 0; n < NCM; ++n) acc[r][n] = 0.f;

  for (int cl = lane; cl < nchs; cl += 64) {
    typename F::Raw nxt[R];
    const int cn = min(cl + 64, nchs - 1);  // the last iteration re-requests a chunk it already has
#pragma unroll
    for (int r = 0; r < R; ++r) nxt[r] = F::load(a.w, rr[r], cbase + cn);
    typename F::U u[R];
#pragma unroll
    for (int r = 0; r < R; ++r) u[r] = F::unpack(cur[r], cbase + cl, sub);
    const int xc = cl / WPX;
    const int s0 = (WPX == 2) ? (cl & 1) * 3 : 0;  // first digit slot of this half (Q8_0)
#pragma unroll
    for (int n = 0; n < NCM; ++n) {
      if (n >= nc) break;
      uint32_t dg[NDS * 4];
#pragma unroll
      for (int q = 0; q < NDS; ++q) {
        const uint4 v = lds[(n * XSLOTS + s0 + q) * nxp + xc];
        dg[4 * q] = v.x;
        dg[4 * q + 1] = v.y;
        dg[4 * q + 2] = v.z;
        dg[4 * q + 3] = v.w;
      }
      const uint4 dv = lds[(n * XSLOTS + 6) * nxp + xc];
      ChunkDesc ds;
      ds.inv_scale = __uint_as_float(dv.x);
      ds.sum = (int32_t)dv.y;
      ds.sumA = (int32_t)dv.z;
      ds.sumB = (int32_t)dv.w;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][n] += F::dotu(u[r], dg, ds);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) cur[r] = nxt[r];
  }

  // 4. reduce over the 64 lanes (every lane ends with every total)
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int n = 0; n < NCM; ++n) {
      float v = acc[r][n];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      acc[r][n] = v;
    }

  // 5. epilogue: lane r finishes row row0 + r (its pair partner is row0 + (r ^ 1))
  if (lane < R) {
    const int row = row0 + lane;
    if (row < rows) {
#pragma unroll
      for (int n = 0; n < NCM; ++n) {
        if (n >= nc) break;
        float v = 0.f, vp = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r == lane) v = acc[r][n];
          if (r == (lane ^ 1)) vp = acc[r][n];
        }
        if (EPI == EPI_PART)
          a.part[((int64_t)split * nc + n) * rows + row] = v;
        else
          run_epilogue(EPI, a.e, n, row, v, vp);
      }
    }
  }
}

// Activation digits of nc columns of length k.  Four threads share a 32-element chunk: thread m
// takes elements 4m..4m+3 and 16+4m..16+4m+3 (two float4 loads), the chunk's scale and integer sums
// come from lane shuffles, and thread m writes the six digit words of its element group.  With a
// gain vector the digits are of g * x and rs[n] = 1 / sqrt(mean(x^2) + eps) (the RMSNorm scale the
// GEMV epilogue applies; that needs the whole column in one workgroup: gridDim.x == 1).
__global__ __launch_bounds__(1024) void k_digitize(const float* x, int64_t x_stride, const float* gain, float eps,
                                                   int k, int kind, uint4* out, int64_t out_stride, float* rs) {
  __shared__ float red[16];
  const int n = blockIdx.y;
  const int nx = k / XCHUNK;
  const float* xr = x + (int64_t)n * x_stride;
  uint32_t* o = (uint32_t*)(out + (int64_t)n * out_stride);
  const int m = threadIdx.x & 3;
  float ss = 0.f;
  for (int base = blockIdx.x * (blockDim.x >> 2); base < nx; base += gridDim.x * (blockDim.x >> 2)) {
    const int c = base + (threadIdx.x >> 2);
    const bool ok = c < nx;
    float v[8];
    if (ok) {
      const float4 lo = *(const float4*)(xr + (int64_t)c * XCHUNK + 4 * m);
      const float4 hi = *(const float4*)(xr + (int64_t)c * XCHUNK + 16 + 4 * m);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      if (gain) {
        const float4 gl = *(const float4*)(gain + (int64_t)c * XCHUNK + 4 * m);
        const float4 gh = *(const float4*)(gain + (int64_t)c * XCHUNK + 16 + 4 * m);
        const float g[8] = {gl.x, gl.y, gl.z, gl.w, gh.x, gh.y, gh.z, gh.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ss += v[i] * v[i];
          v[i] *= g[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    int sh = 0;
    if (mx > 0.f && mx == mx) sh = min(100, max(-100, 21 - ilogbf(mx)));  // mx * 2^sh in [2^21, 2^22)
    int32_t xf[8];
    int32_t sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = ldexpf(v[i], sh);
      xf[i] = (t == t) ? (int32_t)rintf(t) : 0;
      if (i < 4) sa += xf[i];
      else sb += xf[i];
    }
    sa += __shfl_xor(sa, 1);
    sa += __shfl_xor(sa, 2);
    sb += __shfl_xor(sb, 1);
    sb += __shfl_xor(sb, 2);
    if (ok) {
      uint32_t* oc = o + (int64_t)c * DIG_CHUNK_WORDS;
      if (kind == DIG_NIB) {
        // word m*6 + l, nibble 2b + h = digit l of element 16h + 4m + b  (v[4h + b])
        uint32_t u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = (uint32_t)(xf[i] + 0x888888);
#pragma unroll
        for (int l = 0; l < 6; ++l) {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) w |= ((u[4 * h + b] >> (4 * l)) & 15u) << (4 * (2 * b + h));
          oc[m * 6 + l] = w ^ 0x88888888u;
        }
      } else {
        // word (h*4 + m)*3 + l, byte b = digit l of element 16h + 4m + b
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t u[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) u[b] = (uint32_t)(xf[4 * h + b] + 0x808080);
#pragma unroll
          for (int l = 0; l < 3; ++l) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) w |= ((u[b] >> (8 * l)) & 255u) << (8 * b);
            oc[(h * 4 + m) * 3 + l] = w ^ 0x80808080u;
          }
        }
      }
      if (m == 0)
        *(uint4*)(oc + DIG_WORDS) =
            make_uint4(__float_as_uint(ldexpf(1.0f, -sh)), (uint32_t)(sa + sb), (uint32_t)sa, (uint32_t)sb);
    }
  }
  if (gain) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
      rs[n] = 1.0f / sqrtf(t / (float)k + eps);
    }
  }
}

hipError_t launch_digitize(const float* x, int64_t x_stride, const float* gain, float eps, int64_t k, int nc, int qt,
                           void* out, int64_t out_stride_bytes, float* rs, hipStream_t st) {
  const int64_t nx = k / XCHUNK;
  // with an RMSNorm the whole column stays in one workgroup (its sum of squares is needed);
  // otherwise one workgroup per 256 chunks
  const int gx = gain ? 1 : (int)((nx + 255) / 256);
  hipLaunchKernelGGL(k_digitize, dim3(gx, nc), dim3(1024), 0, st, x, x_stride, gain, eps, (int)k, digit_kind(qt),
                     (uint4*)out, out_stride_bytes / 16, rs);
  return hipGetLastError();
}

// Fixed-order sum of the K-split partials, then the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* part, int ksplit, int nc, int rows, EpiArgs e) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  for (int n = 0; n < nc; ++n) {
    float v = 0.f;
    if (row < rows)
      for (int s = 0; s < ksplit; ++s) v += part[((int64_t)s * nc + n) * rows + row];
    const float vp = __shfl_xor(v, 1);
    if (row < rows) run_epilogue(EPI, e, n, row, v, vp);
  }
}

// ------------------------------------------------------------------------------------------ host side


static int g_waves = 0, g_rows = 0;  // launch-geometry overrides (0 = default)

void set_gemv_geometry(int waves, int rows_per_wave) {
  g_waves = waves;
  g_rows = rows_per_wave;
}

// Workgroups of 8 waves; for one column, rows per wave (4, 2 or 1) picked so that the workgroup
// count splits evenly over the 256 CUs (one resident workgroup per CU at this register use),
// weighted by the measured per-wave efficiency of larger row groups (activation reuse).
static int pick_rows_per_wave(int64_t rows, int waves, int ksplit, bool pairs) {
  const int cand[3] = {4, 2, 1};
  const double gain[3] = {1.0, 0.97, 0.83};
  int best = 4;
  double best_score = -1.0;
  for (int i = 0; i < (pairs ? 2 : 3); ++i) {
    const double wgs = (double)((rows + (int64_t)waves * cand[i] - 1) / ((int64_t)waves * cand[i])) * ksplit;
    const double rounds = wgs / 256.0;
    const double balance = rounds / std::ceil(rounds);
    const double score = balance * gain[i];
    if (score > best_score + 1e-9) {
      best_score = score;
      best = cand[i];
    }
  }
  return best;
}

GemvPlan plan_gemv(int qt, int64_t rows, int64_t k, int nc, int epi) {
  // the RoPE and SwiGLU epilogues combine rows (2i, 2i+1), which must sit in one wave
  const bool pairs = epi == EPI_QKV || epi == EPI_SWIGLU;
  GemvPlan p{};
  p.ncm = nc <= 1 ? 1 : (nc <= 4 ? 4 : 8);
  p.rows_per_wave = 2;
  p.waves = 8;
  if (g_waves == 2 || g_waves == 4 || g_waves == 8) p.waves = g_waves;
  const int64_t nx = k / XCHUNK;                        // activation chunks
  const size_t per_chunk = (size_t)p.ncm * DIG_CHUNK_WORDS * 4;  // LDS bytes per chunk (all columns)
  int64_t max_x = (int64_t)(LDS_BUDGET / per_chunk);
  max_x = max_x / 8 * 8;  // splits start on 256-weight superblock boundaries
  if (max_x < 8) max_x = 8;
  int ksplit = (int)((nx + max_x - 1) / max_x);
  if (ksplit < 1) ksplit = 1;
  const int64_t xs = ((nx + ksplit - 1) / ksplit + 7) / 8 * 8;  // activation chunks per split
  p.ks = (int)(xs * XCHUNK);
  p.ksplit = (int)((k + p.ks - 1) / p.ks);
  p.lds = (size_t)xs * per_chunk;
  p.part_bytes = p.ksplit > 1 ? (size_t)p.ksplit * nc * rows * sizeof(float) : 0;
  if (p.ncm == 1) p.rows_per_wave = pick_rows_per_wave(rows, p.waves, p.ksplit, pairs);
  if (p.ncm == 1 && (g_rows == 1 || g_rows == 2 || g_rows == 4)) p.rows_per_wave = g_rows;
  if (pairs && p.rows_per_wave < 2) p.rows_per_wave = 2;
  return p;
}

template <int QT, int NCM, int R>
static hipError_t launch_t(const GemvArgs& a, int epi, int ksplit, dim3 grid, dim3 block, size_t lds,
                           hipStream_t st) {
  switch (ksplit > 1 ? EPI_PART : epi) {
    case EPI_PART: hipLaunchKernelGGL((k_gemv<QT, NCM, R, EPI_PART>), grid, block, lds, st, a); break;
    case EPI_STORE: hipLaunchKernelGGL((k_gemv<QT, NCM, R, EPI_STORE>), grid, block, lds, st, a); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemv<QT, NCM, R, EPI_RESID>), grid, block, lds, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_gemv<QT, NCM, R, EPI_SWIGLU>), grid, block, lds, st, a); break;
    case EPI_QKV: hipLaunchKernelGGL((k_gemv<QT, NCM, R, EPI_QKV>), grid, block, lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QT>
static hipError_t launch_fmt(const GemvArgs& a, const GemvPlan& p, int epi, dim3 grid, dim3 block, hipStream_t st) {
  if (p.ncm == 1 && p.rows_per_wave == 1) return launch_t<QT, 1, 1>(a, epi, p.ksplit, grid, block, p.lds, st);
  if (p.ncm == 1 && p.rows_per_wave == 2) return launch_t<QT, 1, 2>(a, epi, p.ksplit, grid, block, p.lds, st);
  if (p.ncm == 1) return launch_t<QT, 1, 4>(a, epi, p.ksplit, grid, block, p.lds, st);
  if (p.ncm == 4) return launch_t<QT, 4, 2>(a, epi, p.ksplit, grid, block, p.lds, st);
  return launch_t<QT, 8, 2>(a, epi, p.ksplit, grid, block, p.lds, st);
}

hipError_t launch_gemv(int qt, const MatView& w, int64_t k, const void* xd, int64_t xd_stride_bytes, int nc, int epi,
                       const EpiArgs& e, float* part, hipStream_t st, const GemvPlan& p) {
  GemvArgs a;
  a.w = w;
  a.xd = (const uint4*)xd;
  a.xd_stride = xd_stride_bytes / 16;
  a.nc = nc;
  a.k = (int)k;
  a.ks = p.ks;
  a.part = part;
  a.e = e;
  const int rows = w.rows;
  const int rows_per_wg = p.waves * p.rows_per_wave;
  dim3 grid((rows + rows_per_wg - 1) / rows_per_wg, p.ksplit);
  dim3 block(64 * p.waves);
  hipError_t err;
  switch (qt) {
    case Q8_0: err = launch_fmt<Q8_0>(a, p, epi, grid, block, st); break;
    case Q4_0: err = launch_fmt<Q4_0>(a, p, epi, grid, block, st); break;
    case Q4_K: err = launch_fmt<Q4_K>(a, p, epi, grid, block, st); break;
    case Q5_K: err = launch_fmt<Q5_K>(a, p, epi, grid, block, st); break;
    case Q6_K: err = launch_fmt<Q6_K>(a, p, epi, grid, block, st); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess || p.ksplit == 1) return err;
  dim3 rg((rows + 255) / 256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(k_gemv_reduce<EPI_STORE>, rg, dim3(256), 0, st, part, p.ksplit, nc, rows, e); break;
    case EPI_RESID: hipLaunchKernelGGL(k_gemv_reduce<EPI_RESID>, rg, dim3(256), 0, st, part, p.ksplit, nc, rows, e); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemv_reduce<EPI_SWIGLU>, rg, dim3(256), 0, st, part, p.ksplit, nc, rows, e); break;
    case EPI_QKV: hipLaunchKernelGGL(k_gemv_reduce<EPI_QKV>, rg, dim3(256), 0, st, part, p.ksplit, nc, rows, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qwg
