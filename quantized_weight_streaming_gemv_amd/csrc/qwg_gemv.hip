// qwg_gemv.hip -- fused dequantize-and-GEMV for gfx950 (the engine's hand-written GEMV kernels,
// NTransformer page "Architecture overview", cuda/; formats from the Show HN page's
// quantization-format table).
//
// Work decomposition (batch-1 decode is HBM-bound: every weight byte is read exactly once):
//   * a workgroup of W wave64s owns W*R consecutive output rows and one K split;
//   * each wave owns R rows; lane l walks chunks l, l+64, ... of those rows, so every wave-wide
//     load instruction reads 1 KiB of contiguous quant bytes (16 B per lane);
//   * the activation (optionally RMS-normalised in the prologue) is staged once per workgroup
//     into LDS in a chunk-transposed layout: float4 q of chunk c of column n lives at slot
//     (n*XQ + q)*nch + c, so the 64 lanes of a wave read 64 consecutive float4s -- no bank
//     conflicts; the per-chunk activation sums used to fold min/offset terms are staged too;
//   * quants are converted to fp32 in registers (byte extracts + v_cvt_f32_ubyte) and multiplied
//     with the activation; the block scale is applied once per chunk;
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
  const float* x;
  int64_t x_stride;
  const float* gain;
  float eps;
  int nc;
  int k;
  int ks;
  float* part;
  EpiArgs e;
};

template <int QT, int NCM, int R, int RMS, int EPI>
__global__ __launch_bounds__(512) void k_gemv(GemvArgs a) {
  using F = Fmt<QT>;
  constexpr int CW = F::CW, XQ = F::XQ, NS = F::NSUM;
  extern __shared__ float4 lds4[];
  __shared__ float red[8][16];
  __shared__ float rs_sh[NCM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int nc = a.nc;
  const int split = blockIdx.y;
  const int kbeg = split * a.ks;
  const int klen = min(a.ks, a.k - kbeg);
  const int nchs = klen / CW;   // chunks of this split
  const int nchp = a.ks / CW;   // LDS stride (chunks of a full split)
  const int cbase = kbeg / CW;
  const int rows = a.w.rows;
  const int row0 = (blockIdx.x * nw + wave) * R;
  const bool active = row0 < rows;

  // 1. request the first chunk of every row of this wave before staging the activation
  // rows past the end are clamped to the last row (loads stay in bounds, results are dropped)
  int rr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rr[r] = min(row0 + r, rows - 1);
  typename F::Raw cur[R];
  if (active && lane < nchs) {
#pragma unroll
    for (int r = 0; r < R; ++r) cur[r] = F::load(a.w, rr[r], cbase + lane);
  }

  // 2. RMSNorm scale of every column over the full K (prologue of QKV, gate|up and head GEMVs)
  if (RMS) {
    for (int n = 0; n < nc; ++n) {
      const float4* xr = (const float4*)(a.x + (int64_t)n * a.x_stride);
      float s = 0.f;
      for (int f = tid; f < a.k / 4; f += blockDim.x) {
        const float4 v = xr[f];
        s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) red[n & 7][wave] = s;
    }
    __syncthreads();
    if (tid < nc) {
      float s = 0.f;
      for (int wv = 0; wv < nw; ++wv) s += red[tid][wv];
      rs_sh[tid] = 1.0f / sqrtf(s / (float)a.k + a.eps);
    }
    __syncthreads();
  }

  // 3. stage this split's activation, chunk-transposed
  float4* xs = lds4;
  float* sums = (float*)(lds4 + (int64_t)NCM * XQ * nchp);
  for (int n = 0; n < nc; ++n) {
    const float4* xr = (const float4*)(a.x + (int64_t)n * a.x_stride + kbeg);
    const float4* gr = (const float4*)(a.gain + kbeg);
    const float rs = RMS ? rs_sh[n] : 1.0f;
    for (int f = tid; f < nchs * XQ; f += blockDim.x) {
      float4 v = xr[f];
      if (RMS) {
        const float4 g = gr[f];
        v.x = g.x * (v.x * rs);
        v.y = g.y * (v.y * rs);
        v.z = g.z * (v.z * rs);
        v.w = g.w * (v.w * rs);
      }
      const int c = f / XQ, q = f % XQ;
      xs[(n * XQ + q) * nchp + c] = v;
    }
  }
  __syncthreads();
  if (NS > 0) {
    for (int i = tid; i < nc * nchs; i += blockDim.x) {
      const int n = i / nchs, c = i % nchs;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int q = 0; q < XQ; ++q) {
        const float4 v = xs[(n * XQ + q) * nchp + c];
        const float t = (v.x + v.y) + (v.z + v.w);
        if (NS == 2 && q >= XQ / 2)
          s1 += t;
        else
          s0 += t;
      }
      sums[(n * nchp + c) * NS] = s0;
      if (NS == 2) sums[(n * nchp + c) * NS + 1] = s1;
    }
    __syncthreads();
  }
  if (!active) return;

  // 4. main loop over this lane's chunks
  float acc[R][NCM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int n = 0; n < NCM; ++n) acc[r][n] = 0.f;

  const int sub = lane & 7;  // chunk index within its 256-weight superblock (splits start on superblocks)
  for (int cl = lane; cl < nchs; cl += 64) {
    typename F::Raw nxt[R];
    const int cn = min(cl + 64, nchs - 1);  // the last iteration re-requests a chunk it already has
#pragma unroll
    for (int r = 0; r < R; ++r) nxt[r] = F::load(a.w, rr[r], cbase + cn);
    // one column: the chunk's activation lives in registers and serves all R rows
    float4 xr[NCM == 1 ? XQ : 1];
    float sr[NCM == 1 && NS > 0 ? NS : 1];
    if (NCM == 1) {
#pragma unroll
      for (int q = 0; q < XQ; ++q) xr[q] = xs[q * nchp + cl];
#pragma unroll
      for (int j = 0; j < NS; ++j) sr[j] = sums[cl * NS + j];
    }
    auto X = [&](int n, int q) -> float4 { return NCM == 1 ? xr[q] : xs[(n * XQ + q) * nchp + cl]; };
    auto S = [&](int n, int j) -> float { return NCM == 1 ? sr[j] : sums[(n * nchp + cl) * NS + j]; };
#pragma unroll
    for (int r = 0; r < R; ++r) F::template dot<NCM>(cur[r], cbase + cl, sub, nc, X, S, acc[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) cur[r] = nxt[r];
  }

  // 5. reduce over the 64 lanes (every lane ends with every total)
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int n = 0; n < NCM; ++n) {
      float v = acc[r][n];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      acc[r][n] = v;
    }

  // 6. epilogue: lane r finishes row row0 + r (its pair partner is row0 + (r ^ 1))
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

static void fmt_geom(int qt, int& cw, int& xq, int& ns) {
  switch (qt) {
    case Q8_0: cw = 16; xq = 4; ns = 0; break;
    case Q6_K: cw = 32; xq = 8; ns = 2; break;
    default: cw = 32; xq = 8; ns = 1; break;
  }
}

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
  int cw, xq, ns;
  fmt_geom(qt, cw, xq, ns);
  const int64_t nch = k / cw;
  const size_t per_chunk = (size_t)p.ncm * (xq * 16 + ns * 4);
  int64_t max_ch = (int64_t)(LDS_BUDGET / per_chunk);
  if (max_ch < 1) max_ch = 1;
  const int64_t sb = 256 / cw;  // chunks per 256 weights: splits start on superblock boundaries
  max_ch = max_ch / sb * sb;
  if (max_ch < sb) max_ch = sb;
  int ksplit = (int)((nch + max_ch - 1) / max_ch);
  if (ksplit < 1) ksplit = 1;
  int64_t chs = ((nch + ksplit - 1) / ksplit + sb - 1) / sb * sb;  // chunks per split
  p.ks = (int)(chs * cw);
  p.ksplit = (int)((k + p.ks - 1) / p.ks);
  p.lds = (size_t)chs * per_chunk;
  p.part_bytes = p.ksplit > 1 ? (size_t)p.ksplit * nc * rows * sizeof(float) : 0;
  if (p.ncm == 1) p.rows_per_wave = pick_rows_per_wave(rows, p.waves, p.ksplit, pairs);
  if (p.ncm == 1 && (g_rows == 1 || g_rows == 2 || g_rows == 4)) p.rows_per_wave = g_rows;
  if (pairs && p.rows_per_wave < 2) p.rows_per_wave = 2;
  return p;
}

template <int QT, int NCM, int R>
static hipError_t launch_t(const GemvArgs& a, bool rms, int epi, int ksplit, dim3 grid, dim3 block, size_t lds,
                           hipStream_t st) {
  const int main_epi = ksplit > 1 ? EPI_PART : epi;
#define QWG_GEMV_CASE(RMSV, EPIV)                                                                      \
  if ((int)rms == RMSV && main_epi == EPIV) {                                                           \
    hipLaunchKernelGGL((k_gemv<QT, NCM, R, RMSV, EPIV>), grid, block, lds, st, a);                      \
    return hipGetLastError();                                                                          \
  }
  QWG_GEMV_CASE(0, EPI_PART)
  QWG_GEMV_CASE(0, EPI_STORE)
  QWG_GEMV_CASE(0, EPI_RESID)
  QWG_GEMV_CASE(1, EPI_PART)
  QWG_GEMV_CASE(1, EPI_STORE)
  QWG_GEMV_CASE(1, EPI_SWIGLU)
  QWG_GEMV_CASE(1, EPI_QKV)
#undef QWG_GEMV_CASE
  return hipErrorInvalidValue;
}

template <int QT>
static hipError_t launch_fmt(const GemvArgs& a, const GemvPlan& p, bool rms, int epi, dim3 grid, dim3 block,
                             hipStream_t st) {
  if (p.ncm == 1 && p.rows_per_wave == 1) return launch_t<QT, 1, 1>(a, rms, epi, p.ksplit, grid, block, p.lds, st);
  if (p.ncm == 1 && p.rows_per_wave == 2) return launch_t<QT, 1, 2>(a, rms, epi, p.ksplit, grid, block, p.lds, st);
  if (p.ncm == 1) return launch_t<QT, 1, 4>(a, rms, epi, p.ksplit, grid, block, p.lds, st);
  if (p.ncm == 4) return launch_t<QT, 4, 2>(a, rms, epi, p.ksplit, grid, block, p.lds, st);
  return launch_t<QT, 8, 2>(a, rms, epi, p.ksplit, grid, block, p.lds, st);
}

hipError_t launch_gemv(int qt, const MatView& w, int64_t k, const float* x, int64_t x_stride, const float* gain,
                       float eps, bool rms, int nc, int epi, const EpiArgs& e, float* part, hipStream_t st,
                       const GemvPlan& p) {
  GemvArgs a;
  a.w = w;
  a.x = x;
  a.x_stride = x_stride;
  a.gain = gain;
  a.eps = eps;
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
    case Q8_0: err = launch_fmt<Q8_0>(a, p, rms, epi, grid, block, st); break;
    case Q4_0: err = launch_fmt<Q4_0>(a, p, rms, epi, grid, block, st); break;
    case Q4_K: err = launch_fmt<Q4_K>(a, p, rms, epi, grid, block, st); break;
    case Q5_K: err = launch_fmt<Q5_K>(a, p, rms, epi, grid, block, st); break;
    case Q6_K: err = launch_fmt<Q6_K>(a, p, rms, epi, grid, block, st); break;
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
