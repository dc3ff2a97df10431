// qwg_gemv.hip -- fused dequantize-and-GEMV for gfx950 (the engine's hand-written GEMV kernels,
// NTransformer page, [NT] below, "Architecture overview", cuda/; formats from the Show HN page's
// quantization-format table).
//
// Work decomposition (batch-1 decode is HBM-bound: every weight byte is read exactly once):
//   * a workgroup of W wave64s owns P row blocks of W*R consecutive output rows (or, persistent,
//     every gridDim-th row block) and one K split;
//   * each wave owns R rows of each block; lane l walks chunks l, l+64, ... of those rows, so every
//     wave-wide load instruction reads 1 KiB of contiguous quant bytes (16 B per lane);
//   * the activation arrives as block fixed-point digits (see qwg_formats.h): 36 words per 32
//     elements, staged once per workgroup into LDS in a chunk-transposed layout -- 16-B slot q of
//     chunk c of column n at (n*9 + q)*S + c, with the row stride S padded against bank conflicts
//     of the staging writes -- so the 64 lanes of a wave read 64 consecutive slots (or it arrives
//     as fp32 and the workgroup digitizes it into the same layout);
//   * quants stay integers: nibble formats feed v_dot8_i32_i4 directly (stored as q XOR 8), the
//     others feed v_dot4_i32_i8 with one byte per quant; each chunk's integer sums are recombined
//     in fp32 and scaled once by the block scales and the activation chunk scale;
//   * an RMSNorm in front of the GEMV is folded in: the digits are of g*h, and the finished rows are
//     multiplied by 1/rms, reduced in a fixed order from per-chunk sums of h^2 in the prologue;
//   * the first chunks' weights are requested before the activation is staged; a wave's row blocks
//     then run as one software pipeline that keeps PD iterations of loads in flight;
//   * DPP reductions sum each finished row over the 64 lanes and park it in one lane; after the
//     loop those lanes run the epilogue (store, residual add, SwiGLU on interleaved gate|up rows,
//     or RoPE + fp16 KV append), and for the residual and SwiGLU epilogues the workgroup can also
//     digitize its slice of the output vector for the next GEMV (whole 32-element chunks);
//   * K splits (when the activation for all columns does not fit the LDS budget) write partial
//     sums that a second kernel adds in a fixed order, so results never depend on timing;
//   * 2..8 columns of Q4_K, Q5_K and Q6_K (self-speculative verify, chunked prefill) take the
//     matrix-core kernel k_gemv_mfma instead: one v_mfma_i32_16x16x32_i8 per 16-row tile and
//     chunk over byte digits of every column (its own section below).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "qwg_kernels.h"

namespace qwg {

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// v of the lane that DPP control CTRL selects, for the rows in ROW_MASK (0 elsewhere)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes, as a wave-uniform value: quad permutes (lane ^ 1, lane ^ 2) and row mirrors
// give every lane its 16-lane row's sum, two row broadcasts carry it into lane 63, which is read as
// a scalar.  Six DPP adds replace the LDS-routed butterfly of six shuffles; the order is fixed.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141, 0xF>(v);  // row_half_mirror: the other quad of each eight lanes
  v += dpp_f<0x140, 0xF>(v);  // row_mirror: the other eight of each row
  v += dpp_f<0x142, 0xA>(v);  // row_bcast15: rows 1 and 3 add lane 15 of rows 0 and 2
  v += dpp_f<0x143, 0xC>(v);  // row_bcast31: rows 2 and 3 add lane 31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// (cos, sin) of the RoPE pair that q/k row `row` of column n belongs to
__device__ __forceinline__ float2 rope_pair(const EpiArgs& e, int n, int row) {
  return ((const float2*)e.rope)[(int64_t)(e.pos + n) * (HEAD_DIM / 2) + ((row % HEAD_DIM) >> 1)];
}

// The QKV epilogue of row `row`, column n: RoPE with the pair's (cos, sin) cs on q and k, q to y,
// k and v appended to the fp16 caches at position pos + n.
__device__ __forceinline__ void qkv_store(const EpiArgs& e, int n, int row, float v, float vp, float2 cs) {
  const int pos = e.pos + n;
  if (row < e.nq_rows + e.nkv_rows) {
    // pair (a, b) = rows (2i, 2i+1): a' = a cos - b sin, b' = a sin + b cos
    const float out = (row & 1) == 0 ? (v * cs.x - vp * cs.y) : (vp * cs.y + v * cs.x);
    if (row < e.nq_rows)
      e.y[(int64_t)n * e.y_stride + row] = out;
    else
      e.kc[(int64_t)pos * e.kv_stride + (row - e.nq_rows)] = float_to_half_bits(out);
  } else {
    e.vc[(int64_t)pos * e.kv_stride + (row - e.nq_rows - e.nkv_rows)] = float_to_half_bits(v);
  }
}

// Final value of output row `row`, column n (v: its sum; vp: the sum of its pair partner row^1),
// stored by the epilogue; returns the value the output vector holds at that position (the new h
// for RESID, silu(gate)*up for SWIGLU on even rows).
__device__ __forceinline__ float run_epilogue(int epi, const EpiArgs& e, int n, int row, float v, float vp) {
  switch (epi) {
    case EPI_STORE:
      e.y[(int64_t)n * e.y_stride + row] = v;
      return v;
    case EPI_RESID: {
      float* p = e.y + (int64_t)n * e.y_stride + row;
      const float h = *p + v;
      *p = h;
      return h;
    }
    case EPI_SWIGLU:
      if ((row & 1) == 0) {
        const float a = silu_f(v) * vp;
        e.y[(int64_t)n * e.y_stride + (row >> 1)] = a;
        return a;
      }
      return 0.f;
    case EPI_QKV:
      qkv_store(e, n, row, v, vp, row < e.nq_rows + e.nkv_rows ? rope_pair(e, n, row) : make_float2(0.f, 0.f));
      return 0.f;
    default:
      return 0.f;
  }
}

// Per-wave partial sums of the RMSNorm input's chunk sums of squares (column n) into red[n][wave].
__device__ __forceinline__ void rms_partials(const EpiArgs& e, int nc, float (*red)[16]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int n = 0; n < nc; ++n) {
    float s = 0.f;
    for (int i = tid; i < e.sq_in_n; i += blockDim.x) s += e.sq_in[(int64_t)n * e.sq_in_stride + i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) red[n][wave] = s;
  }
}

__device__ __forceinline__ float rms_scale(const EpiArgs& e, float (*red)[16], int n) {
  const int nw = blockDim.x >> 6;
  float s = 0.f;
  for (int w = 0; w < nw; ++w) s += red[n][w];
  return 1.0f / sqrtf(s / e.rms_k + e.eps);
}

// Digitize output values held in LDS (osh[n][0 .. nout), nout a multiple of 32, output elements
// out0 ..) for the next GEMV, with their per-chunk sums of squares.  Every group of four lanes
// takes one (column, chunk); all threads of the block call it.
// With gpre, (g0, g1) are this thread's gain values (elements 4m..4m+3 and 16+4m..16+4m+3 of chunk
// tid / 4; one column, at most blockDim / 4 chunks), requested earlier.
template <int OSTRIDE>
__device__ __forceinline__ void digitize_outputs(const EpiArgs& e, int nc, const float (*osh)[OSTRIDE], int nout,
                                                 int out0, bool gpre = false, float4 g0 = {}, float4 g1 = {}) {
  const float gp[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  const int tid = threadIdx.x, m = tid & 3, g = tid >> 2;
  const int nchunk = nout / XCHUNK;
  for (int base = 0; base < nc * nchunk; base += blockDim.x >> 2) {
    const int job = base + g;
    const bool ok = job < nc * nchunk;
    const int n = ok ? job / nchunk : 0, j = ok ? job % nchunk : 0;
    float v[8], ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int el = j * XCHUNK + (i < 4 ? 4 * m + i : 16 + 4 * m + i - 4);
      float x = ok ? osh[n][el] : 0.f;
      ss += x * x;
      if (e.dig_gain && ok) x *= gpre ? gp[i] : e.dig_gain[out0 + el];
      v[i] = x;
    }
    const int chunk = (out0 / XCHUNK) + j;
    digitize_group(v, m, e.dig_kind, e.dig_out + (int64_t)n * e.dig_stride + (int64_t)chunk * DIG_CHUNK_WORDS, ok);
    if (e.sq_out) {
      ss = quad_sum(ss);
      if (ok && m == 0) e.sq_out[(int64_t)n * e.sq_out_stride + chunk] = ss;
    }
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

constexpr int XSLOTS = DIG_CHUNK_WORDS / 4;  // 16-B slots per activation chunk (8 digit slots + desc)
constexpr int DSLOT = DIG_WORDS / 4;         // the descriptor's slot

// LDS row stride (16-B slots) for n chunks: n rounded up to 9 mod 16.  The staging writes put the 9
// slots of consecutive chunks into 9 rows; with this stride the 16 lanes an LDS write serves at a
// time land on 16 distinct 16-byte bank groups (row q, chunk c -> group (9q + c) mod 16), where a
// stride that is a multiple of 16 put all 9 rows of a chunk on the same banks.
__host__ __device__ constexpr int lds_row_slots(int n) { return n + ((XSLOTS - n) % 16 + 16) % 16; }

// Pipeline: each wave computes ng groups of R rows (group g: R rows at row0_of(g)), every group in
// iterations of 64 chunks (lane l takes chunk l + 64 i).  The loop over all ng * nit iterations is
// wave-uniform and runs as one software pipeline: the fetch cursor stays PD iterations ahead of the
// compute cursor and crosses from one group into the next without draining, so the loads of the
// next rows are in flight while a group is reduced.  Lanes past the end of a ragged row (chunk
// index >= the split's chunks) load the clamped last chunk and add nothing.  A group's 64-lane
// totals are parked in lane g*R + r, and the epilogue runs once after the loop (no stores in it).
// P: groups per wave -- P row blocks of nw*R rows per workgroup (P == 0, persistent: the grid
// strides over the row blocks, at most 64/R of them per workgroup).  Four-row two-group kernels are
// held to 128 registers (four waves per SIMD, two workgroups per CU).  LB: the launch bound.  XIN:
// the input arrives as fp32 (EpiArgs::xf) and every workgroup digitizes the part it needs into LDS:
// XIN == 1 all of it before the loop; XIN == 2 (one column, 512 threads) in segments of 128 chunks:
// the first before the loop, each later one right before the first iteration that reads it, from
// fp32 values requested one segment earlier, so the digitization overlaps the weight stream
// instead of delaying its start.
template <int QT, int NCM, int R, int EPI, int PD, int P = 1, int LB = 512, int XIN = 0>
__global__ __launch_bounds__(LB, (R == 4 && P == 2 ? 4 : 1)) void k_gemv(GemvArgs a) {
  static_assert(PD == 1 || PD == 2, "one or two iterations of loads in flight");
  static_assert(R == 1 || R == 2 || R == 4, "rows per wave");
  using F = Fmt<QT>;
  constexpr int CW = F::CW;
  constexpr int WPX = XCHUNK / CW;               // weight chunks per activation chunk (2 for Q8_0)
  constexpr int NDS = DIG_WORDS / 4 / WPX;       // digit slots one weight chunk reads
  extern __shared__ uint4 lds[];
  __shared__ float red[MAX_COLS][16];
  __shared__ float osh[MAX_COLS][64];

  const int tid = threadIdx.x, lane = tid & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nc = a.nc;
  const int split = blockIdx.y;
  const int kbeg = split * a.ks;
  const int klen = min(a.ks, a.k - kbeg);
  const int nxs = klen / XCHUNK;   // activation chunks of this split
  const int nxp = lds_row_slots(a.ks / XCHUNK);  // LDS row stride in 16-B slots
  const int xbase = kbeg / XCHUNK;
  const int nchs = klen / CW;      // weight chunks of this split
  const int cbase = kbeg / CW;
  const int nit = (nchs + 63) >> 6;  // iterations per group
  const int rows = a.w.rows;
  const int blk_rows = nw * R;
  const int nblk = (rows + blk_rows - 1) / blk_rows;
  const int npass = P > 0 ? P : (nblk - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  auto block_of = [&](int g) { return P > 0 ? (int)blockIdx.x * P + g : (int)blockIdx.x + g * (int)gridDim.x; };
  auto row0_of = [&](int g) { return block_of(g) * blk_rows + wave * R; };
  const int wg_rows = blk_rows * (P > 0 ? P : 1);
  const int wg_row0 = block_of(0) * blk_rows;
  const bool digitize = P > 0 && (EPI == EPI_RESID || EPI == EPI_SWIGLU) && a.e.dig_out != nullptr;
  constexpr bool SEG = XIN == 2;
  static_assert(!SEG || (NCM == 1 && PD == 1 && P > 0 && LB == 512), "segmented staging: one column, 512 threads");
  int ng = 0;  // groups of this wave (its rows of the workgroup's row blocks)
  while (ng < npass && ng < 64 / R && row0_of(ng) < rows) ++ng;
  // segmented staging: every wave runs the same iterations (rows past the end are clamped and their
  // results dropped), so all of them reach the same barriers
  if (SEG) ng = P;

  // rows past the end are clamped to the last row (loads stay in bounds, results are dropped)
  // (per-chunk regions are addressed by slot = per-row part + per-chunk part, see slot_row)
  uint32_t rofs[R], srow[R];
  constexpr int NB = PD + 1;  // buffers in rotation: PD in flight while one is computed
  typename F::Raw buf[NB][R];
  auto set_rows = [&](int r0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(r0 + r, rows - 1);
      rofs[r] = row_off(QT, a.w, row);
      srow[r] = slot_row(a.w.ilv, a.w.nch, row);
    }
  };
  int fg = 0, fi = 0;  // fetch cursor: group, iteration
  auto fetch_next = [&](typename F::Raw* raw) {
    const int c = cbase + min(lane + 64 * fi, nchs - 1);
    const uint32_t sc = slot_chunk(a.w.ilv, (uint32_t)c);
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = F::load(a.w, rofs[r], c, srow[r] + sc);
    if (++fi == nit) {
      if (fg + 1 < ng) {
        fi = 0;
        set_rows(row0_of(++fg));
      } else {
        fi = nit - 1;  // past the last iteration: re-read the last chunks (never used)
      }
    }
  };

  // segmented staging (XIN == 2): thread quad tid / 4 digitizes chunk SEGX s + tid / 4 of segment s
  constexpr int SEGX = 128;                 // activation chunks per segment
  constexpr int IPS = SEGX * WPX / 64;      // loop iterations per segment
  const int nseg = (nxs + SEGX - 1) / SEGX;
  float4 sx_lo, sx_hi;                      // the fp32 values of the next segment, in flight
  auto seg_load = [&](int s) {
    const int c = min(SEGX * s + (tid >> 2), nxs - 1);
    const float* xr = a.e.xf + (int64_t)(xbase + c) * XCHUNK + 4 * (tid & 3);
    sx_lo = *(const float4*)xr;
    sx_hi = *(const float4*)(xr + 16);
  };
  auto seg_put = [&](int s) {
    uint32_t* ldw = (uint32_t*)lds;
    const int c = SEGX * s + (tid >> 2);
    const float v[8] = {sx_lo.x, sx_lo.y, sx_lo.z, sx_lo.w, sx_hi.x, sx_hi.y, sx_hi.z, sx_hi.w};
    digitize_group_to(
        v, tid & 3, digit_kind(QT), [&](int i, uint32_t w) { ldw[(((i >> 2)) * nxp + c) * 4 + (i & 3)] = w; },
        c < nxs);
  };
  if (SEG) seg_load(0);  // requested ahead of the first weights: its wait does not include them

  // 1. request the first chunks of this wave's rows before staging the activation
  if (ng > 0) {
    set_rows(row0_of(0));
#pragma unroll
    for (int k = 0; k < PD; ++k) fetch_next(buf[k]);
  }

  // 2. stage this split's activation digits (coalesced 16-B reads, chunk-transposed LDS) and the
  //    RMSNorm partial sums.  Each thread issues a batch of loads before its first LDS write (a
  //    load-then-write loop serialized one L2 round trip per 8 KiB of the workgroup's slice).
  if (SEG) {
    seg_put(0);
    if (nseg > 1) seg_load(1);
  } else if (XIN) {
    // four threads per 32-element chunk digitize it into the same LDS layout
    constexpr int XU = 4;  // chunks in flight per thread
    uint32_t* ldw = (uint32_t*)lds;
    const int m = tid & 3, cstep = blockDim.x >> 2;
    for (int n = 0; n < nc; ++n) {
      const float* xr = a.e.xf + (int64_t)n * a.e.xf_stride + (int64_t)xbase * XCHUNK;
      for (int c0 = tid >> 2; c0 < nxs; c0 += XU * cstep) {
        float4 lo[XU], hi[XU];
#pragma unroll
        for (int u = 0; u < XU; ++u) {
          const int c = min(c0 + u * cstep, nxs - 1);
          lo[u] = *(const float4*)(xr + (int64_t)c * XCHUNK + 4 * m);
          hi[u] = *(const float4*)(xr + (int64_t)c * XCHUNK + 16 + 4 * m);
        }
#pragma unroll
        for (int u = 0; u < XU; ++u) {
          const int c = c0 + u * cstep;  // the four threads of a chunk agree on c < nxs
          const float v[8] = {lo[u].x, lo[u].y, lo[u].z, lo[u].w, hi[u].x, hi[u].y, hi[u].z, hi[u].w};
          digitize_group_to(
              v, m, digit_kind(QT),
              [&](int i, uint32_t w) { ldw[((n * XSLOTS + (i >> 2)) * nxp + c) * 4 + (i & 3)] = w; }, c < nxs);
        }
      }
    }
  } else {
    constexpr int SU = 8;  // 16-B slots in flight per thread
    const int tot = nxs * XSLOTS, step = blockDim.x;
    for (int n = 0; n < nc; ++n) {
      const uint4* src = a.xd + (int64_t)n * a.xd_stride + (int64_t)xbase * XSLOTS;
      for (int b = tid; b < tot; b += SU * step) {
        uint4 v[SU];
#pragma unroll
        for (int u = 0; u < SU; ++u) v[u] = src[min(b + u * step, tot - 1)];
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          const int i = b + u * step;
          if (i < tot) lds[(n * XSLOTS + i % XSLOTS) * nxp + i / XSLOTS] = v[u];
        }
      }
    }
  }
  if (EPI != EPI_PART && a.e.sq_in) rms_partials(a.e, nc, red);
  __syncthreads();

  // 3. the pipelined loop
  const int sub = lane & 7;  // chunk index within its 256-weight superblock (splits start on superblocks)
  float acc[R][NCM], res[NCM];
#pragma unroll
  for (int n = 0; n < NCM; ++n) {
    res[n] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][n] = 0.f;
  }
  int cg = 0, ci = 0;  // compute cursor: group, iteration
  auto compute_next = [&](const typename F::Raw* raw) {
    const int cl = lane + 64 * ci;
    const bool valid = cl < nchs;
    typename F::U u[R];
#pragma unroll
    for (int r = 0; r < R; ++r) u[r] = F::unpack(raw[r], cbase + cl, sub);
    const int xc = min(cl, nchs - 1) / WPX;
    const int s0 = (WPX == 2) ? (cl & 1) * NDS : 0;  // first digit slot of this half (Q8_0)
#pragma unroll
    for (int n = 0; n < NCM; ++n) {
      if (NCM > 1 && n >= nc) break;  // one-column kernels always have nc == 1
      uint32_t dg[NDS * 4];
#pragma unroll
      for (int q = 0; q < NDS; ++q) {
        const uint4 v = lds[(n * XSLOTS + s0 + q) * nxp + xc];
        dg[4 * q] = v.x;
        dg[4 * q + 1] = v.y;
        dg[4 * q + 2] = v.z;
        dg[4 * q + 3] = v.w;
      }
      const uint4 dv = lds[(n * XSLOTS + DSLOT) * nxp + xc];
      ChunkDesc ds;
      ds.inv_scale = __uint_as_float(dv.x);
      ds.sum = __uint_as_float(dv.y);
      ds.shi = (int32_t)dv.z;
      ds.slo = (int32_t)dv.w;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float d = F::dotu(u[r], dg, ds);
        acc[r][n] += valid ? d : 0.f;
      }
    }
    if (++ci == nit) {
      // the group is done: its 64-lane sums, parked in lane cg*R + r
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int n = 0; n < NCM; ++n) {
          const float v = wave_sum(acc[r][n]);
          if (lane == cg * R + r) res[n] = v;
          acc[r][n] = 0.f;
        }
      ci = 0;
      ++cg;
    }
  };
  const int total = ng * nit;
  // One column, residual epilogue: its operands (the residual and the next RMSNorm gain of the
  // workgroup's output chunks) are requested at the start of the last loop trip, behind the last
  // weights in the in-order return queue, instead of after the loop.  (Requesting the QKV epilogue's
  // RoPE pairs the same way measured 0.2 us slower.)
  constexpr bool PRE = NCM == 1 && P > 0 && EPI == EPI_RESID;
  const int ep_row = row0_of(lane / R) + lane % R;  // the row this lane finishes (lane < ng * R)
  const bool ep_live = lane < ng * R && ep_row < rows;
  const int nout_d = EPI == EPI_RESID ? min(wg_rows, rows - wg_row0) : 0;  // digitized outputs
  float pre_h = 0.f;
  float4 pre_g0 = make_float4(1.f, 1.f, 1.f, 1.f), pre_g1 = pre_g0;
  const bool pre_gain = PRE && digitize && a.e.dig_gain != nullptr && nout_d <= 8 * (int)blockDim.x;
  auto prefetch_epi = [&]() {
    if (ep_live) pre_h = a.e.y[ep_row];
    if (pre_gain && tid < nout_d / 8) {  // thread 4 j + m: chunk j, elements 4m.. and 16 + 4m..
      const float* gp = a.e.dig_gain + wg_row0 + (tid >> 2) * XCHUNK + 4 * (tid & 3);
      pre_g0 = *(const float4*)gp;
      pre_g1 = *(const float4*)(gp + 16);
    }
  };
  // Single-exit loops with scheduling barriers between the fetch and compute phases: a break in the
  // middle of the body let the compiler build an exec-masked exit whose fall-through edge carried
  // unconsumed loads into the loop header (which then waited for every load), and without the
  // barriers the scheduler sank the next fetch into the current compute.
  int t = 0;
  for (; t + NB <= total; t += NB) {
    if (PRE && t + 2 * NB > total) prefetch_epi();  // the last trip (workgroup-uniform)
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      fetch_next(buf[(k + PD) % NB]);
      __builtin_amdgcn_sched_barrier(0);
      compute_next(buf[k]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (SEG) {
      // iteration t + NB (even: IPS is 2 or 4) is the first of segment (t + NB) / IPS: digitize it
      // from the values requested one segment ago and request the next (workgroup-uniform branch)
      const int it = t + NB;
      if (it % IPS == 0 && it / IPS < nseg) {
        seg_put(it / IPS);
        if (it / IPS + 1 < nseg) seg_load(it / IPS + 1);
        __syncthreads();
      }
    }
  }
  if (PRE && total < NB) prefetch_epi();
  // the last total - t < NB iterations are already in flight, in buf[0 ..)
#pragma unroll
  for (int k = 0; k < PD; ++k)
    if (t + k < total) compute_next(buf[k]);

  // 4. epilogue: lane j < ng*R finishes row r = j % R of group g = j / R (its pair partner, row^1,
  //    is lane j^1 of the same group)
  float resp[NCM];
#pragma unroll
  for (int n = 0; n < NCM; ++n) resp[n] = __uint_as_float(quad_swap<0xB1>(__float_as_uint(res[n])));
  if (lane < ng * R) {
    const int row = ep_row;
    if (row < rows) {
#pragma unroll
      for (int n = 0; n < NCM; ++n) {
        if (NCM > 1 && n >= nc) break;
        float v = res[n], vp = resp[n];
        if (EPI == EPI_PART) {
          a.part[((int64_t)split * nc + n) * rows + row] = v;
        } else {
          if (a.e.sq_in) {
            const float rs = rms_scale(a.e, red, n);
            v *= rs;
            vp *= rs;
          }
          float out;
          if (PRE) {
            out = pre_h + v;
            a.e.y[row] = out;
          } else {
            out = run_epilogue(EPI, a.e, n, row, v, vp);
          }
          if (digitize) {
            if (EPI == EPI_RESID) osh[n][row - wg_row0] = out;
            else if ((row & 1) == 0) osh[n][(row - wg_row0) >> 1] = out;
          }
        }
      }
    }
  }

  // 5. digitize this workgroup's slice of the output vector for the next GEMV
  if (digitize) {
    __syncthreads();
    const int nrow = min(wg_rows, rows - wg_row0);  // whole chunks: the host checks rows
    const int nout = EPI == EPI_RESID ? nrow : nrow / 2;
    const int out0 = EPI == EPI_RESID ? wg_row0 : wg_row0 / 2;
    digitize_outputs<64>(a.e, nc, osh, nout, out0, pre_gain, pre_g0, pre_g1);
  }
}

// Fixed-order sum of the K-split partials, then the epilogue (a block of 256 threads = 256 rows;
// with digitization, the block's 256 rows / 128 SwiGLU outputs are whole chunks).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* part, int ksplit, int nc, int rows, EpiArgs e) {
  __shared__ float red[MAX_COLS][16];
  __shared__ float osh[MAX_COLS][256];
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  const bool digitize = (EPI == EPI_RESID || EPI == EPI_SWIGLU) && e.dig_out != nullptr;
  if (e.sq_in) {
    rms_partials(e, nc, red);
    __syncthreads();
  }
  // every column's partials are requested before any is added (a column-by-column loop waited for
  // each column's loads in turn), and for the residual epilogue the residual values too
  float vs[MAX_COLS], hs[MAX_COLS];
#pragma unroll
  for (int n = 0; n < MAX_COLS; ++n) {
    vs[n] = 0.f;
    hs[n] = 0.f;
  }
  if (row < rows) {
    for (int s = 0; s < ksplit; ++s) {
      float t[MAX_COLS];
#pragma unroll
      for (int n = 0; n < MAX_COLS; ++n) t[n] = n < nc ? part[((int64_t)s * nc + n) * rows + row] : 0.f;
#pragma unroll
      for (int n = 0; n < MAX_COLS; ++n) vs[n] += t[n];
    }
    if (EPI == EPI_RESID) {
#pragma unroll
      for (int n = 0; n < MAX_COLS; ++n)
        if (n < nc) hs[n] = e.y[(int64_t)n * e.y_stride + row];
    }
  }
  for (int n = 0; n < nc; ++n) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < MAX_COLS; ++i)
      if (i == n) v = vs[i];
    if (e.sq_in) v *= rms_scale(e, red, n);
    const float vp = __shfl_xor(v, 1);
    if (row < rows) {
      float out;
      if (EPI == EPI_RESID) {
        float h = 0.f;
#pragma unroll
        for (int i = 0; i < MAX_COLS; ++i)
          if (i == n) h = hs[i];
        out = h + v;
        e.y[(int64_t)n * e.y_stride + row] = out;
      } else {
        out = run_epilogue(EPI, e, n, row, v, vp);
      }
      if (digitize) {
        if (EPI == EPI_RESID) osh[n][threadIdx.x] = out;
        else if ((row & 1) == 0) osh[n][threadIdx.x >> 1] = out;
      }
    }
  }
  if (digitize) {
    __syncthreads();
    const int nrow = min((int)blockDim.x, rows - (int)(blockIdx.x * blockDim.x));
    const int nout = EPI == EPI_RESID ? nrow : nrow / 2;
    const int out0 = EPI == EPI_RESID ? (int)(blockIdx.x * blockDim.x) : (int)(blockIdx.x * blockDim.x / 2);
    digitize_outputs<256>(e, nc, osh, nout, out0);
  }
}

// ------------------------------------------------------------------ several columns on the matrix cores
//
// The verify pass of self-speculative decoding multiplies one weight matrix by k+1 activation columns
// ([NT] "Key features": self-speculative decoding), and chunked prefill up to 8 prompt tokens at once.
// This form takes 2..8 columns (one or two groups of four) when K is a multiple of 512.
// For Q4_K, Q5_K and Q6_K (with byte activation digits: the producers of this kernel's input pick
// the kind with gemv_digit_kind) each 16-row tile and 32-weight chunk is one v_mfma_i32_16x16x32_i8 with
//   A (16 x 32): activation digits, slot m = 4 * column + level,
//   B (32 x 16): the chunk's quants as int8 bytes, one column per output row,
// so the 4 x 4 digit levels of all columns meet every weight in one exact integer product.  With
// lane l = 16 g + n:
//   B: row n, weights 4g..4g+3 and 16+4g..16+4g+3 of the chunk (its quant word g);
//   A: slot n (column n / 4, level n % 4), the digits of those same eight elements;
//   D: levels 0..3 of column g, row n -- so every lane finishes one (row, column) pair per chunk:
//      value = 65536 (256 D3 + D2) + (256 D1 + D0), scaled by the chunk's weight scales and
//      activation scale.
// Each lane loads one whole 16-B chunk (chunk c0 + g of row n, 64 contiguous bytes per row and lane
// group) and four permlane swaps turn the four chunks' words into word g of each chunk (a 4 x 4
// transpose across the lane groups).  Q6_K's two 16-weight sub-blocks per chunk take one MFMA each
// (B masked to the low or high four bytes).
// A workgroup of nw waves takes blocks of T = nw / S tiles; the S waves of a tile split its chunks
// (K parts) and add their partial sums in wave order through LDS, so the result does not depend on
// timing.  The grid is persistent over the blocks; the activation of one K split (552 B per chunk:
// 520 B of digits, 4 x 8 B of (2^-s, 2^-s sum x_fix)) is staged once per workgroup.
constexpr int MF_DIG = 64;  // 8-B digit entries per chunk and group of four columns: [word g][column][level]
// LDS stride of a chunk's entries: one entry of padding (130 or 258 words), so the staging writes of
// consecutive chunks spread over the banks
__host__ __device__ constexpr int mf_dig_stride(int ng) { return ng * MF_DIG + 1; }
// LDS bytes per chunk (digit entries and one (2^-s, 2^-s sum) pair per column) and per workgroup
// beyond the chunks (the descriptor rows' padding)
__host__ __device__ constexpr int mf_chunk_lds(int ng) { return mf_dig_stride(ng) * 8 + 4 * ng * 8; }
__host__ __device__ constexpr int mf_fixed_lds(int ng) { return 4 * ng * 2 * 8; }

__device__ __forceinline__ void lane_swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);  // lanes 32..63 of a <-> 0..31 of b
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void lane_swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);  // odd 16-lane rows of a <-> even of b
  a = r[0];
  b = r[1];
}

typedef int qwg_i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ qwg_i32x4 mfma_i8(uint64_t a, uint64_t b) {
  const qwg_i32x4 z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8((long)a, (long)b, z, 0, 0, 0);
}

// 2^24 D3 + 2^16 D2 + 256 D1 + D0 as 65536 (256 D3 + D2) + (256 D1 + D0): each bracket is below 2^28
// in magnitude (|D_l| <= 32 * 128 * 128), exact in int32, and rounds once to fp32 before the fma
__device__ __forceinline__ float mf_value(const qwg_i32x4& d) {
  return __builtin_fmaf(65536.0f, (float)(d[2] + d[3] * 256), (float)(d[0] + d[1] * 256));
}

// Steps are two superblocks (16 chunks) of the lane's row: chunk c0 + 4 qq + g in quarter qq.
template <int QT>
constexpr int mf_step_chunks() { return 16; }

__device__ __forceinline__ uint32_t lane_fetch(int src_lane, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane * 4, (int)v);
}
template <int QT>
struct MfRaw;
// Q4_K: the quants (stored q XOR 8) and the header, as Q5_K without fifth bits.
template <>
struct MfRaw<Q4_K> {
  uint4 q[4];
  uint4 h;
};

// Q5_K steps are two superblocks (16 chunks); each lane group loads a different part of the rows'
// fifth bits and headers, and the quarter steps fetch what they need from the group that holds it
// (ds_bpermute): one 16-B read per lane covers a row's 64 contiguous bytes of fifth bits.
template <>
struct MfRaw<Q5_K> {
  uint4 q[4];  // chunks c0 + 4 qq + g, qq = 0..3
  uint4 qh;    // fifth bits of chunks c0 + 4g .. c0 + 4g + 3
  uint4 h;     // header of superblock (c0 / 8) + (g & 1)
};
// Q6_K: each lane group loads a different part of the rows' high-bit pairs and sub-block scales
// (lane_fetch hands them to the quarter steps); the two superblocks' d share one aligned word.
template <>
struct MfRaw<Q6_K> {
  uint4 q[4];
  uint4 qhA, qhB;  // high-bit pairs of chunks c0 + 2g, c0 + 2g + 1 and c0 + 8 + 2g, c0 + 9 + 2g (8 B each)
  uint2 sc;        // int8 sub-block scales of chunks c0 + 4g .. c0 + 4g + 3 (2 B each)
  uint32_t dw;     // fp16 d of superblocks c0 / 8 (low half) and c0 / 8 + 1 (high half)
};

template <int QT>
__device__ __forceinline__ MfRaw<QT> mf_load(const MatView& w, uint32_t ro, uint32_t srow, int cg, int g) {
  MfRaw<QT> r;
  const uint32_t s0 = srow + slot_chunk(w.ilv, (uint32_t)cg);  // the superblock's 8 chunks are consecutive slots
  if constexpr (QT == Q4_K || QT == Q5_K) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) r.q[qq] = ld_stream_u4(w.q + (s0 + 4u * qq + (uint32_t)g) * 16u);
    if constexpr (QT == Q5_K) r.qh = ld<uint4>(w.b + (s0 + 4u * g) * 4u);
    r.h = ld<uint4>(w.a + ro + (uint32_t)((cg >> 3) + (g & 1)) * 16u);
  } else {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) r.q[qq] = ld_stream_u4(w.q + (s0 + 4u * qq + (uint32_t)g) * 16u);
    r.qhA = ld<uint4>(w.a + (s0 + 2u * g) * 8u);
    r.qhB = ld<uint4>(w.a + (s0 + 8u + 2u * g) * 8u);
    r.sc = ld<uint2>(w.b + (s0 + 4u * g) * 2u);
    r.dw = ld<uint32_t>(w.c + ro + (uint32_t)(cg >> 3) * 2u);  // 4-B aligned: K is a multiple of 512
  }
  return r;
}

// NG column groups of four (NG = 2: 5..8 columns): each group is one more A operand and one more
// MFMA per chunk (Q6_K: two) against the same B operand, processed one group after the other.
template <int QT, int EPI, int NG>
__global__ __launch_bounds__(NG == 1 ? 1024 : 512) void k_gemv_mfma(GemvArgs a, int kparts) {
  static_assert(QT == Q4_K || QT == Q5_K || QT == Q6_K, "K-quant formats with 32-weight chunks");
  static_assert(NG == 1 || NG == 2, "four or eight columns");
  constexpr int DSTR = mf_dig_stride(NG);  // 8-B digit entries per chunk in LDS: [group][word g][column][level]
  extern __shared__ uint4 lds[];
  __shared__ float red[MAX_COLS][16];
  const int tid = threadIdx.x, lane = tid & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nc = a.nc;
  const int split = blockIdx.y;
  const int kbeg = split * a.ks;
  const int klen = min(a.ks, a.k - kbeg);
  const int nxs = klen / XCHUNK;  // chunks of this split (a multiple of 16)
  const int nxp = a.ks / XCHUNK;  // LDS capacity in chunks
  const int xbase = kbeg / XCHUNK;
  // LDS: digit entries [nxp][DSTR]; per column a row of (2^-s, 2^-s sum x_fix) per chunk, rows
  // nxp + 2 apart (the columns' rows then start on different banks); K-part partial sums
  const int dstr = nxp + 2;
  uint2* ldig = (uint2*)lds;
  float2* ldesc = (float2*)(ldig + (size_t)nxp * DSTR);
  float* lpart = (float*)(ldesc + 4 * NG * dstr);           // [NG][nw][64]

  // 1. stage the split's digits: one (column, chunk) per thread; columns >= nc are zeros
  for (int job = tid; job < 4 * NG * nxs; job += blockDim.x) {
    const int col = job / nxs, c = job - col * nxs;
    uint32_t wd[DIG_CHUNK_WORDS];
    if (col < nc) {
      const uint4* src = a.xd + (int64_t)col * a.xd_stride + (int64_t)(xbase + c) * XSLOTS;
#pragma unroll
      for (int q = 0; q < XSLOTS; ++q) {
        const uint4 v = src[q];
        wd[4 * q] = v.x;
        wd[4 * q + 1] = v.y;
        wd[4 * q + 2] = v.z;
        wd[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < DIG_CHUNK_WORDS; ++i) wd[i] = 0;
    }
    const int ent = c * DSTR + (col >> 2) * MF_DIG + (col & 3) * BYTE_LEVELS;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
#pragma unroll
      for (int lv = 0; lv < BYTE_LEVELS; ++lv)
        ldig[ent + gg * 4 * BYTE_LEVELS + lv] =
            make_uint2(wd[gg * BYTE_LEVELS + lv], wd[16 + gg * BYTE_LEVELS + lv]);
    const float inv = __uint_as_float(wd[DIG_WORDS]);
    ldesc[col * dstr + c] = make_float2(inv, inv * __uint_as_float(wd[DIG_WORDS + 1]));
  }
  if (EPI != EPI_PART && a.e.sq_in) rms_partials(a.e, nc, red);
  __syncthreads();

  // 2. blocks of T tiles x S K parts
  const int S = kparts, T = nw / kparts;
  const int t = wave / S, s = wave - t * S;
  const int rows = a.w.rows;
  const int blk_rows = 16 * T;
  const int nblk = (rows + blk_rows - 1) / blk_rows;
  const int nst = nxs / mf_step_chunks<QT>();  // steps of two superblocks
  const int st0 = s * nst / S, st1 = (s + 1) * nst / S;
  const int cbase = kbeg / XCHUNK;
  const int aoff = g * 4 * BYTE_LEVELS + n;  // this lane's A entry within a group: column n / 4, level n % 4
  // per-lane bit-move amounts: Q5_K fifth bits (rotations), Q6_K high pairs (shifts)
  const uint32_t rot_lo = (uint32_t)(28 + 2 * g) & 31u, rot_hi = (uint32_t)(29 + 2 * g) & 31u;
  const uint32_t shl_lo = (g & 1) ? 2u : 6u, shl_hi = (g & 1) ? 0u : 4u;

  // quarter qq (chunks c0 + 4 qq .. + 3) of a step: quant words transposed across the lane groups,
  // the B operands and weight scales of the four chunks, then per column group the A operands,
  // four (Q6_K: eight) MFMAs and the (row n, column 4 cg + g) updates.  hv: the K-quant superblock
  // header of this quarter (fetched by the caller from the lane group that loaded it).
  auto quarter = [&](const MfRaw<QT>& r, int c0, int qq, const uint4& hv, float* acc) {
    const uint4 qv = r.q[qq];
    // the swaps overwrite both operands: copy the loaded words here, where they are used (left to
    // register allocation, the copies sat right after the next step's loads and waited for them)
    uint32_t R[4];
    asm volatile("v_mov_b32 %0, %1" : "=v"(R[0]) : "v"(qv.x));
    asm volatile("v_mov_b32 %0, %1" : "=v"(R[1]) : "v"(qv.y));
    asm volatile("v_mov_b32 %0, %1" : "=v"(R[2]) : "v"(qv.z));
    asm volatile("v_mov_b32 %0, %1" : "=v"(R[3]) : "v"(qv.w));
    lane_swap32(R[0], R[2]);
    lane_swap32(R[1], R[3]);
    lane_swap16(R[0], R[1]);
    lane_swap16(R[2], R[3]);  // R[j] = quant word g of chunk c0 + 4 qq + j
    const int cc = c0 + 4 * qq;
    // A operands and activation scales of column group cg (columns 4 cg .. 4 cg + 3)
    uint64_t A[4];
    float4 d01, d23;
    auto load_group = [&](int cg) {
      d01 = *(const float4*)&ldesc[(4 * cg + g) * dstr + cc];
      d23 = *(const float4*)&ldesc[(4 * cg + g) * dstr + cc + 2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 av = ldig[(cc + j) * DSTR + cg * MF_DIG + aoff];
        A[j] = (uint64_t)av.x | ((uint64_t)av.y << 32);
      }
    };
    load_group(0);
    // B operands (the quants of word g as bytes; Q6_K: the two 16-weight halves separately), each
    // multiplied as soon as it is formed, then the chunk's weight scales (Q4_K / Q5_K: d sc and
    // -dmin m; Q6_K: d sc / 4 of both halves)
    uint64_t B0[4], B1[4];
    float w0[4], w1[4];
    qwg_i32x4 D[4], E[4];
    if constexpr (QT == Q4_K || QT == Q5_K) {
      if constexpr (QT == Q5_K) {
        // fifth bits of this quarter's chunks, from lane group qq of the same row
        const int src = n + 16 * qq;
        const uint32_t qh[4] = {lane_fetch(src, r.qh.x), lane_fetch(src, r.qh.y), lane_fetch(src, r.qh.z),
                                lane_fetch(src, r.qh.w)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t l5 = __builtin_rotateright32(qh[j], rot_lo), h5 = __builtin_rotateright32(qh[j], rot_hi);
          const uint32_t lo = (R[j] & 0x0F0F0F0Fu) | (l5 & 0x10101010u);
          const uint32_t hi = ((R[j] >> 4) & 0x0F0F0F0Fu) | (h5 & 0x10101010u);
          B0[j] = (uint64_t)lo | ((uint64_t)hi << 32);
          D[j] = mfma_i8(A[j], B0[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // the stored nibbles are q XOR 8: flip back to q in 0..15
          const uint32_t lo = (R[j] & 0x0F0F0F0Fu) ^ 0x08080808u;
          const uint32_t hi = ((R[j] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
          B0[j] = (uint64_t)lo | ((uint64_t)hi << 32);
          D[j] = mfma_i8(A[j], B0[j]);
        }
      }
      const uint64_t ps = (uint64_t)hv.x | ((uint64_t)hv.y << 32);
      const uint64_t pm = (uint64_t)hv.z | ((uint64_t)hv.w << 32);
      const float dd = half_bits_to_float(hv.y >> 16), dm = half_bits_to_float(hv.w >> 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sb = 4 * (qq & 1) + j;  // sub-block of the superblock
        w0[j] = dd * (float)((uint32_t)(ps >> (6 * sb)) & 63u);
        w1[j] = -(dm * (float)((uint32_t)(pm >> (6 * sb)) & 63u));
      }
    } else {
      // high-bit pairs of chunk 4 qq + j: words (x, y) of qhA (qq < 2) or qhB held by lane group
      // (2 qq + j / 2) & 3; rows take x for word groups 0, 1 and y for 2, 3
      const int src0 = n + 16 * ((2 * qq) & 3), src1 = n + 16 * ((2 * qq + 1) & 3);
      const uint4 qp = qq < 2 ? r.qhA : r.qhB;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = (j >> 1) ? src1 : src0;
        const uint32_t hx = lane_fetch(src, (j & 1) ? qp.z : qp.x), hy = lane_fetch(src, (j & 1) ? qp.w : qp.y);
        const uint32_t h = g < 2 ? hx : hy;
        const uint32_t lo = ((R[j] << 2) & 0x3C3C3C3Cu) | ((h << shl_lo) & 0xC0C0C0C0u);
        const uint32_t hi = ((R[j] >> 2) & 0x3C3C3C3Cu) | ((h << shl_hi) & 0xC0C0C0C0u);
        B0[j] = (uint64_t)lo;
        B1[j] = (uint64_t)hi << 32;
        D[j] = mfma_i8(A[j], B0[j]);
        E[j] = mfma_i8(A[j], B1[j]);
      }
      const float dq = 0.25f * half_bits_to_float((r.dw >> (16 * (qq >> 1))) & 0xFFFFu);
      // sub-block scales of this quarter's chunks, from lane group qq
      const uint32_t scw[2] = {lane_fetch(n + 16 * qq, r.sc.x), lane_fetch(n + 16 * qq, r.sc.y)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = scw[j >> 1] >> (16 * (j & 1));
        w0[j] = dq * (float)(int32_t)(int8_t)(uint8_t)(w & 0xFFu);
        w1[j] = dq * (float)(int32_t)(int8_t)(uint8_t)((w >> 8) & 0xFFu);
      }
    }
    // (row n, column 4 cg + g) updates from this group's products
    auto consume = [&](float& a_) {
      const float inv[4] = {d01.x, d01.z, d23.x, d23.z};
      if constexpr (QT == Q4_K || QT == Q5_K) {
        const float xs[4] = {d01.y, d01.w, d23.y, d23.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a_ = __builtin_fmaf(inv[j] * w0[j], mf_value(D[j]), a_);
          a_ = __builtin_fmaf(w1[j], xs[j], a_);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a_ = __builtin_fmaf(inv[j] * w0[j], mf_value(D[j]), a_);
          a_ = __builtin_fmaf(inv[j] * w1[j], mf_value(E[j]), a_);
        }
      }
    };
    consume(acc[0]);
    if constexpr (NG == 2) {
      load_group(1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        D[j] = mfma_i8(A[j], B0[j]);
        if constexpr (QT == Q6_K) E[j] = mfma_i8(A[j], B1[j]);
      }
      consume(acc[1]);
    }
  };
  constexpr int SC = mf_step_chunks<QT>();
  auto step = [&](const MfRaw<QT>& r, int st, float* acc) {
    if constexpr (QT == Q4_K || QT == Q5_K) {
#pragma unroll
      for (int sbk = 0; sbk < 2; ++sbk) {  // the step's two superblocks: header from lane group sbk
        const int src = n + 16 * sbk;
        const uint4 hv = make_uint4(lane_fetch(src, r.h.x), lane_fetch(src, r.h.y), lane_fetch(src, r.h.z),
                                    lane_fetch(src, r.h.w));
        quarter(r, SC * st, 2 * sbk, hv, acc);
        quarter(r, SC * st, 2 * sbk + 1, hv, acc);
      }
    } else {
      const uint4 none = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) quarter(r, SC * st, qq, none, acc);
    }
  };

  for (int b = blockIdx.x; b < nblk; b += gridDim.x) {
    const int r0 = b * blk_rows + t * 16;
    const int row = min(r0 + n, rows - 1);  // rows past the end read the last row; results dropped
    const uint32_t ro = row_off(QT, a.w, row), srow = slot_row(a.w.ilv, a.w.nch, row);
    auto load = [&](int st) { return mf_load<QT>(a.w, ro, srow, cbase + SC * min(st, nst - 1), g); };
    float acc[NG];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) acc[cg] = 0.f;
    // two buffers in rotation: the next step's loads are in flight while one is computed (loads past
    // the part's end re-read its last step, in bounds and unused)
    MfRaw<QT> b0 = load(st0), b1;
    int st = st0;
    for (; st + 2 <= st1; st += 2) {
      b1 = load(min(st + 1, st1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      step(b0, st, acc);
      __builtin_amdgcn_sched_barrier(0);
      b0 = load(min(st + 2, st1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      step(b1, st + 1, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (st < st1) step(b0, st, acc);

    // 3. the tile's K parts in wave order, then the epilogue for (row r0 + n, column 4 cg + g)
    if (S > 1) {
#pragma unroll
      for (int cg = 0; cg < NG; ++cg) lpart[(cg * nw + wave) * 64 + lane] = acc[cg];
      __syncthreads();
      if (s == 0) {
#pragma unroll
        for (int cg = 0; cg < NG; ++cg) {
          float v = 0.f;
          for (int i = 0; i < S; ++i) v += lpart[(cg * nw + wave + i) * 64 + lane];
          acc[cg] = v;
        }
      }
    }
    if (s == 0) {
      const int orow = r0 + n;
#pragma unroll
      for (int cg = 0; cg < NG; ++cg) {
        const int col = 4 * cg + g;
        const bool ok = orow < rows && col < nc;
        float v = acc[cg];
        if (EPI == EPI_PART) {
          if (ok) a.part[((int64_t)split * nc + col) * rows + orow] = v;
        } else {
          if (a.e.sq_in) v *= rms_scale(a.e, red, min(col, nc - 1));
          const float vp = __shfl_xor(v, 1);  // row n ^ 1, same column
          if (ok) run_epilogue(EPI, a.e, col, orow, v, vp);
        }
      }
    }
    if (S > 1) __syncthreads();  // lpart is reused by the next block
  }
}

// ------------------------------------------------------------------ prompt prefill: up to 64 columns
//
// Chunked prefill ([NT] "Quick start": the -p prompt) multiplies every weight matrix by up to 64
// prompt-token columns, so each weight is read once per 64 tokens.  This form takes Q6_K (Q4_K and
// Q5_K run on the fp16 matrix cores below).  The activation of one step (16
// chunks: two 256-weight superblocks) for all 64 columns, 128 KB of byte digits, does not leave room
// for the whole K range on chip, so the K loop is outermost: per step the workgroup stages that step's
// digits of every column in LDS, and each wave multiplies its 16-row tile's weights for the step by all
// 16 column groups -- two v_mfma_i32_16x16x32_i8 per (chunk, column group), one per 16-weight
// sub-block, all sharing
// the chunk's B operand, so the weights are unpacked once per 64 columns.  Lane 16 g + n accumulates
// (row n, column 4 cg + g) of group cg in fp32.  A workgroup takes 16 tiles (256 rows) of one K split
// and writes partial sums; k_gemm_reduce adds the splits in a fixed order and runs the epilogue.
constexpr int GM_NG = 16;                    // column groups of four: 64 columns
constexpr int GM_SC = 16;                    // chunks per step
constexpr int GM_DSTR = GM_NG * 64 + 1;      // 8-B digit entries per chunk ([group][lane]) + 1 of padding
constexpr int GM_ESTR = GM_SC + 2;           // descriptor entries per column (+2: rows start on other banks)
constexpr int GM_WAVES = 16;                 // waves (tiles) per workgroup
constexpr size_t GM_LDS = (size_t)GM_SC * GM_DSTR * 8 + (size_t)GM_NG * 4 * GM_ESTR * 8;

template <int QT>
__global__ __launch_bounds__(64 * GM_WAVES) void k_gemm_mfma(GemvArgs a) {
  static_assert(QT == Q6_K, "Q6_K (the other K-quants take the fp16 form)");
  extern __shared__ uint4 lds[];
  uint2* ldig = (uint2*)lds;                            // [GM_SC][GM_DSTR]
  float2* ldesc = (float2*)(ldig + GM_SC * GM_DSTR);   // [64 columns][GM_ESTR]: (2^-s, 2^-s sum x_fix)
  const int tid = threadIdx.x, lane = tid & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nc = a.nc, rows = a.w.rows;
  const int split = blockIdx.y;
  const int kbeg = split * a.ks, klen = min(a.ks, a.k - kbeg);
  const int nst = klen / (XCHUNK * GM_SC);  // steps of this split
  const int cbase = kbeg / XCHUNK;
  const int r0 = (blockIdx.x * nw + wave) * 16;
  const bool live = r0 < rows;  // waves past the last tile stage the activation and compute nothing
  const int row = min(r0 + n, rows - 1);
  const uint32_t ro = row_off(QT, a.w, row), srow = slot_row(a.w.ilv, a.w.nch, row);
  // per-lane shifts of the high-bit pairs
  const uint32_t shl_lo = (g & 1) ? 2u : 6u, shl_hi = (g & 1) ? 0u : 4u;
  float acc[GM_NG];
#pragma unroll
  for (int cg = 0; cg < GM_NG; ++cg) acc[cg] = 0.f;

  // quarter qq (chunks 4 qq .. 4 qq + 3 of the step): the quant words transposed across the lane
  // groups, the B operands and the sub-blocks' weight scales, then for every column group the A
  // operands from LDS, the products and the (row n, column 4 cg + g) updates.
  auto quarter = [&](const MfRaw<QT>& r, int qq) {
    const uint4 qv = r.q[qq];
    uint32_t R[4] = {qv.x, qv.y, qv.z, qv.w};
    lane_swap32(R[0], R[2]);
    lane_swap32(R[1], R[3]);
    lane_swap16(R[0], R[1]);
    lane_swap16(R[2], R[3]);  // R[j] = quant word g of chunk 4 qq + j
    uint64_t B0[4], B1[4];
    float w0[4], w1[4];
    {
      const int src0 = n + 16 * ((2 * qq) & 3), src1 = n + 16 * ((2 * qq + 1) & 3);
      const uint4 qp = qq < 2 ? r.qhA : r.qhB;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = (j >> 1) ? src1 : src0;
        const uint32_t hx = lane_fetch(src, (j & 1) ? qp.z : qp.x), hy = lane_fetch(src, (j & 1) ? qp.w : qp.y);
        const uint32_t h = g < 2 ? hx : hy;
        const uint32_t lo = ((R[j] << 2) & 0x3C3C3C3Cu) | ((h << shl_lo) & 0xC0C0C0C0u);
        const uint32_t hi = ((R[j] >> 2) & 0x3C3C3C3Cu) | ((h << shl_hi) & 0xC0C0C0C0u);
        B0[j] = (uint64_t)lo;
        B1[j] = (uint64_t)hi << 32;
      }
      const float dq = 0.25f * half_bits_to_float((r.dw >> (16 * (qq >> 1))) & 0xFFFFu);
      const uint32_t scw[2] = {lane_fetch(n + 16 * qq, r.sc.x), lane_fetch(n + 16 * qq, r.sc.y)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = scw[j >> 1] >> (16 * (j & 1));
        w0[j] = dq * (float)(int32_t)(int8_t)(uint8_t)(w & 0xFFu);
        w1[j] = dq * (float)(int32_t)(int8_t)(uint8_t)((w >> 8) & 0xFFu);
      }
    }
    // one column group's products at a time (two groups' operands overflow the 128 registers a
    // 16-wave workgroup leaves each wave)
    auto products = [&](int cg, qwg_i32x4* P) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 av = ldig[(4 * qq + j) * GM_DSTR + cg * 64 + lane];
        const uint64_t A = (uint64_t)av.x | ((uint64_t)av.y << 32);
        P[j] = mfma_i8(A, B0[j]);
        P[4 + j] = mfma_i8(A, B1[j]);
      }
    };
    qwg_i32x4 Pc[8];
#pragma unroll
    for (int cg = 0; cg < GM_NG; ++cg) {
      products(cg, Pc);
      __builtin_amdgcn_sched_barrier(0);  // keep the products ahead of this group's scaling
      const float4 d01 = *(const float4*)&ldesc[(4 * cg + g) * GM_ESTR + 4 * qq];
      const float4 d23 = *(const float4*)&ldesc[(4 * cg + g) * GM_ESTR + 4 * qq + 2];
      const float inv[4] = {d01.x, d01.z, d23.x, d23.z};
      float v = acc[cg];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v = __builtin_fmaf(inv[j] * w0[j], mf_value(Pc[j]), v);
        v = __builtin_fmaf(inv[j] * w1[j], mf_value(Pc[4 + j]), v);
      }
      acc[cg] = v;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  MfRaw<QT> cur;
  auto load = [&](int st) { return mf_load<QT>(a.w, ro, srow, cbase + GM_SC * min(st, nst - 1), g); };
  if (live && nst > 0) cur = load(0);
  for (int st = 0; st < nst; ++st) {
    // 1. stage this step's digits of every column (columns >= nc are zeros): one (column, chunk) per job
    if (st > 0) __syncthreads();  // every wave is done with the previous step's digits
    for (int job = tid; job < 4 * GM_NG * GM_SC; job += blockDim.x) {
      const int col = job / GM_SC, c = job - col * GM_SC;
      uint32_t wd[DIG_CHUNK_WORDS];
      if (col < nc) {
        const uint4* src = a.xd + (int64_t)col * a.xd_stride + (int64_t)(cbase + st * GM_SC + c) * XSLOTS;
#pragma unroll
        for (int q = 0; q < XSLOTS; ++q) {
          const uint4 v = src[q];
          wd[4 * q] = v.x;
          wd[4 * q + 1] = v.y;
          wd[4 * q + 2] = v.z;
          wd[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < DIG_CHUNK_WORDS; ++i) wd[i] = 0;
      }
      const int ent = c * GM_DSTR + (col >> 2) * 64 + (col & 3) * BYTE_LEVELS;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int lv = 0; lv < BYTE_LEVELS; ++lv)
          ldig[ent + gg * 16 + lv] = make_uint2(wd[gg * BYTE_LEVELS + lv], wd[16 + gg * BYTE_LEVELS + lv]);
      const float inv = __uint_as_float(wd[DIG_WORDS]);
      ldesc[col * GM_ESTR + c] = make_float2(inv, inv * __uint_as_float(wd[DIG_WORDS + 1]));
    }
    __syncthreads();
    // 2. the next step's weights are requested before this step's products
    if (live) {
      const MfRaw<QT> r = cur;
      if (st + 1 < nst) cur = load(st + 1);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) quarter(r, qq);
    }
  }
  // 3. partial sums of this split: (row r0 + n, column 4 cg + g)
  if (live && r0 + n < rows) {
#pragma unroll
    for (int cg = 0; cg < GM_NG; ++cg) {
      const int col = 4 * cg + g;
      if (col < nc) a.part[((int64_t)split * nc + col) * rows + r0 + n] = acc[cg];
    }
  }
}

// ------------------------------------------------------------------ prompt prefill on fp16 matrix cores
//
// Q4_K and Q5_K prompt passes (9..64 columns) run on v_mfma_f32_16x16x32_f16 instead.  A weight of
// these formats is dd sc q - dm m with integers sc, m < 64 and q < 32 per 32-weight chunk, so sc q
// (< 2048) is an exact fp16 and one chunk of 16 rows is an exact B operand; the activation arrives as
// DIG_F16 pieces (x' = hi + lo, one power-of-two scale 2^-sh per column and superblock).  Per
// superblock and 16 x 16 (rows, columns) tile:
//   P = sum over the 8 chunks of (sc q) . hi + (sc q) . lo         16 MFMAs, fp32 accumulation
//   M = sum over the chunks of m . 2^-6 (sum of x' over the chunk)  one MFMA (chunk sums as pieces)
//   y += 2^-sh (dd P - 64 dm M)
// so the vector unit finishes a product once per superblock (the i8 form merges four digit levels
// and scales once per chunk).  The matrix cores take fp16 subnormal inputs as they are (checked on
// gfx950), so a lo piece below 2^-14 keeps its value to 2^-25.  With lane l = 16 g + n:
//   B: row n's eight weights of the chunk's quant word g (after the transpose of the i8 form);
//   A: column 16 cg + n's pieces of the same eight elements (the DIG_F16 element order);
//   D: (column 16 cg + 4 g + r, row n), r = 0..3.
// A workgroup of 8 waves takes 256 rows (two 16-row tiles per wave, so every A operand read from LDS
// meets two B operands) of one K split.  The K loop is outermost, one superblock of all columns per
// step, in two LDS buffers: while the waves multiply one superblock, the next one's operands are on
// their way from global memory straight into the other buffer (global_load_lds_dwordx4, no
// registers), so the staging no longer stalls every wave between steps.  The kernel is built for
// CG = 1, 2 or 4 column groups of 16 (passes of up to 16, 32 or 64 columns), so that a narrow pass
// multiplies no empty groups and its smaller buffers leave room for a second workgroup per CU.
constexpr int GF_WAVES = 8;
constexpr int GF_BLK = 64;  // 16-B entries of one operand block (64 lanes)
// operand blocks per superblock ([chunk][piece][group]) and 16-B entries per buffer (those, a
// minimum-term block per group and the 64 column scales)
constexpr int gf_frags(int cg) { return 8 * 2 * cg; }
constexpr int gf_buf(int cg) { return (gf_frags(cg) + cg) * GF_BLK + 64 / 4; }

typedef _Float16 qwg_h8 __attribute__((ext_vector_type(8)));
typedef _Float16 qwg_h2 __attribute__((ext_vector_type(2)));
typedef float qwg_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t h2_fma(uint32_t a, uint32_t b, uint32_t c) {
  const qwg_h2 r = __builtin_elementwise_fma(__builtin_bit_cast(qwg_h2, a), __builtin_bit_cast(qwg_h2, b),
                                             __builtin_bit_cast(qwg_h2, c));
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ qwg_f32x4 mfma_f16(const uint4& a, const uint4& b, qwg_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(qwg_h8, a), __builtin_bit_cast(qwg_h8, b), c, 0,
                                                0, 0);
}

// fp16 pairs (a, b) with a, b < 64 small integers t: fma(1024 + t, u, -1024 u) = t u exactly whenever
// t u is an fp16 (the bit pattern 0x6400 | t is 1024 + t)
constexpr uint32_t H2_ONE = 0x3C003C00u, H2_M1024 = 0xE400E400u;

// Eight weights sc q of one quant word in the DIG_F16 element order: byte j of lo holds q of element
// 4g+j, byte j of hi that of 16+4g+j (q < 32).  One byte permute per pair puts 0x64 above bytes (0, 2)
// or (1, 3), the bit patterns of 1024 + q.
__device__ __forceinline__ uint4 f16_weights(uint32_t lo, uint32_t hi, uint32_t s2, uint32_t ns2) {
  const uint32_t e = 0x64646464u;
  uint4 r;
  r.x = h2_fma(__builtin_amdgcn_perm(e, lo, 0x04020400u), s2, ns2);
  r.y = h2_fma(__builtin_amdgcn_perm(e, lo, 0x04030401u), s2, ns2);
  r.z = h2_fma(__builtin_amdgcn_perm(e, hi, 0x04020400u), s2, ns2);
  r.w = h2_fma(__builtin_amdgcn_perm(e, hi, 0x04030401u), s2, ns2);
  return r;
}

// One superblock of one 16-row tile as lane (n, g) loads it: chunks g and 4 + g of row n (q), the
// row's superblock header (h), and (Q5_K) the fifth bits of chunks 4 (g & 1) .. 4 (g & 1) + 3.
template <int QT>
struct SbRaw {
  uint4 q[2];
  uint4 h;
};
template <>
struct SbRaw<Q5_K> {
  uint4 q[2];
  uint4 h;
  uint4 qh;
};
template <int QT>
__device__ __forceinline__ SbRaw<QT> sb_load(const MatView& w, uint32_t ro, uint32_t srow, int sb, int g) {
  SbRaw<QT> r;
  const uint32_t s0 = srow + slot_chunk(w.ilv, 8u * (uint32_t)sb);  // the superblock's chunks are consecutive slots
  r.q[0] = ld_stream_u4(w.q + (s0 + (uint32_t)g) * 16u);
  r.q[1] = ld_stream_u4(w.q + (s0 + 4u + (uint32_t)g) * 16u);
  r.h = ld<uint4>(w.a + ro + (uint32_t)sb * 16u);
  if constexpr (QT == Q5_K) r.qh = ld<uint4>(w.b + (s0 + 4u * (uint32_t)(g & 1)) * 4u);
  return r;
}

typedef const __attribute__((address_space(1))) void* qwg_gptr;
typedef __attribute__((address_space(3))) void* qwg_lptr;

// Requests superblock sb of every column (DIG_F16 pieces) into LDS buffer buf: wave w copies the
// operand blocks (chunk, piece) = w / CG + (8 / CG) j, j = 0..2 CG - 1, of column group w % CG (lane
// 16 g + i: word g of column 16 (w % CG) + i), waves 0..CG - 1 also their group's minimum-term block
// (lanes 0..15 hi sums, 16..31 lo sums), wave 4 the scales.  Lanes of columns >= nc load nothing: their
// entries keep the zeros the kernel wrote at its start.
template <int CG>
__device__ __forceinline__ void f16_stage(uint4* buf, const GemvArgs& a, int sb, int wave, int lane) {
  static_assert(CG == 1 || CG == 2 || CG == 4, "a whole number of groups per wave");
  const int cg = (int)((unsigned)wave % CG), gq = lane >> 4, col = 16 * cg + (lane & 15);
  const uint4* xc = a.xd + (int64_t)col * a.xd_stride + (int64_t)sb * (F16_SB_WORDS / 4);
  if (col < a.nc) {
#pragma unroll
    for (int j = 0; j < 2 * CG; ++j) {
      const int cp = (int)((unsigned)wave / CG) + (8 / CG) * j;  // chunk * 2 + piece
      __builtin_amdgcn_global_load_lds((qwg_gptr)(xc + cp * 4 + gq), (qwg_lptr)(buf + (cp * CG + cg) * GF_BLK), 16, 0,
                                       0);
    }
  }
  if (wave < CG && lane < 32 && col < a.nc)
    __builtin_amdgcn_global_load_lds((qwg_gptr)(xc + F16_SUM_WORD / 4 + gq),
                                     (qwg_lptr)(buf + (gf_frags(CG) + cg) * GF_BLK), 16, 0, 0);
  if (wave == 4 && lane < a.nc)
    __builtin_amdgcn_global_load_lds(
        (qwg_gptr)((const uint32_t*)(a.xd + (int64_t)lane * a.xd_stride + (int64_t)sb * (F16_SB_WORDS / 4)) +
                   F16_SCALE_WORD),
        (qwg_lptr)(buf + (gf_frags(CG) + CG) * GF_BLK), 4, 0, 0);
}

template <int QT, int CG>
__global__ __launch_bounds__(64 * GF_WAVES) void k_gemm_f16(GemvArgs a) {
  static_assert(QT == Q4_K || QT == Q5_K, "formats with integer sub-block scales and minima");
  constexpr int T = 2;  // tiles per wave
  constexpr int FR = gf_frags(CG), BUF = gf_buf(CG);
  // two buffers, each [chunk][piece][group][64] operand blocks, [group][64] minimum-term blocks and
  // the 64 column scales; separate arrays, so the compiler sees that the requests into one buffer
  // never touch the one being read
  __shared__ uint4 buf0[BUF], buf1[BUF];
  __shared__ float lrs[64];  // fused SwiGLU epilogue (no K split, a.part null): each column's RMSNorm scale
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nc = a.nc, rows = a.w.rows;
  const int split = blockIdx.y;
  const int kbeg = split * a.ks, klen = min(a.ks, a.k - kbeg);
  const int nsb = klen / (XCHUNK * 8);  // superblocks of this split (an even number)
  const int sb0 = kbeg / (XCHUNK * 8);
  const int r0 = (blockIdx.x * GF_WAVES + wave) * 16 * T;
  const bool live = r0 < rows;
  uint32_t ro[T], srow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int row = min(r0 + 16 * t + n, rows - 1);
    ro[t] = row_off(QT, a.w, row);
    srow[t] = slot_row(a.w.ilv, a.w.nch, row);
  }
  const uint32_t rot_lo = (uint32_t)(28 + 2 * g) & 31u, rot_hi = (uint32_t)(29 + 2 * g) & 31u;  // Q5_K fifth bits
  qwg_f32x4 y[T][CG];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) y[t][cg] = qwg_f32x4{0.f, 0.f, 0.f, 0.f};

  // the superblock in buffer b, with r[t] its raw weights.  Chunk c's A operands are read from LDS and
  // its B operands built while chunk c - 1's products run (two sets of each, chosen at compile time).
  auto superblock = [&](const uint4* b, const SbRaw<QT>* r) {
    const uint4* lmin = b + FR * GF_BLK;
    const float* lscale = (const float*)(b + (FR + CG) * GF_BLK);
    qwg_f32x4 P[T][CG];
    uint64_t ps[T];
#pragma unroll
    for (int t = 0; t < T; ++t) ps[t] = (uint64_t)r[t].h.x | ((uint64_t)r[t].h.y << 32);
    // Q5_K fifth bits: the narrow builds fetch every chunk's from lane n + 16 q2 at once; the
    // four-group build, short of registers (spills otherwise), fetches each chunk's when it builds
    // the chunk's operand
    constexpr bool late5 = CG == 4;
    uint32_t R[2][T][4], qh[2][T][4];  // transposed quant words (and fifth bits) of quarters 0, 1
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint4 qv = r[t].q[q2];
        R[q2][t][0] = qv.x;
        R[q2][t][1] = qv.y;
        R[q2][t][2] = qv.z;
        R[q2][t][3] = qv.w;
        lane_swap32(R[q2][t][0], R[q2][t][2]);
        lane_swap32(R[q2][t][1], R[q2][t][3]);
        lane_swap16(R[q2][t][0], R[q2][t][1]);
        lane_swap16(R[q2][t][2], R[q2][t][3]);  // R[q2][t][j] = quant word g of chunk 4 q2 + j
        if constexpr (QT == Q5_K && !late5) {
          const int src = n + 16 * q2;
          qh[q2][t][0] = lane_fetch(src, r[t].qh.x);
          qh[q2][t][1] = lane_fetch(src, r[t].qh.y);
          qh[q2][t][2] = lane_fetch(src, r[t].qh.z);
          qh[q2][t][3] = lane_fetch(src, r[t].qh.w);
        }
      }
    uint4 ah[2][CG], al[2][CG], bw[2][T];
    auto fetch_a = [&](int c, uint4* h, uint4* l) {
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        h[cg] = b[((c * 2 + 0) * CG + cg) * GF_BLK + lane];
        l[cg] = b[((c * 2 + 1) * CG + cg) * GF_BLK + lane];
      }
    };
    auto build_b = [&](int c, uint4* bo) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t word = R[c >> 2][t][c & 3];
        const uint32_t sc = (uint32_t)(ps[t] >> (6 * c)) & 63u;
        const uint32_t s2 = h2_fma(sc | (sc << 16) | 0x64006400u, H2_ONE, H2_M1024);  // (sc, sc)
        const uint32_t ns2 = h2_fma(s2, H2_M1024, 0u);
        uint32_t lo, hi;  // q of elements 4g+j and 16+4g+j in byte j
        if constexpr (QT == Q4_K) {
          lo = (word ^ 0x88888888u) & 0x0F0F0F0Fu;  // the stored nibbles are q XOR 8
          hi = ((word >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu;
        } else {
          const uint4& qv = r[t].qh;
          const uint32_t f =
              late5 ? lane_fetch(n + 16 * (c >> 2), (c & 3) == 0 ? qv.x : (c & 3) == 1 ? qv.y : (c & 3) == 2 ? qv.z : qv.w)
                    : qh[c >> 2][t][c & 3];
          const uint32_t l5 = __builtin_rotateright32(f, rot_lo), h5 = __builtin_rotateright32(f, rot_hi);
          lo = (word & 0x0F0F0F0Fu) | (l5 & 0x10101010u);
          hi = ((word >> 4) & 0x0F0F0F0Fu) | (h5 & 0x10101010u);
        }
        bo[t] = f16_weights(lo, hi, s2, ns2);
      }
    };
    fetch_a(0, ah[0], al[0]);
    build_b(0, bw[0]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int cur = c & 1, nxt = cur ^ 1;
      if (c + 1 < 8) fetch_a(c + 1, ah[nxt], al[nxt]);
      __builtin_amdgcn_sched_barrier(0);  // the next chunk's LDS reads go out first
      if (c + 1 < 8) build_b(c + 1, bw[nxt]);
      const qwg_f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int t = 0; t < T; ++t) P[t][cg] = mfma_f16(ah[cur][cg], bw[cur][t], c == 0 ? z : P[t][cg]);
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int t = 0; t < T; ++t) P[t][cg] = mfma_f16(al[cur][cg], bw[cur][t], P[t][cg]);
    }
    // the minimum term (B: the 8 minima of row n) and the superblock's fold
    uint4 mb[T];
    float dd[T], dm64[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint64_t pm = (uint64_t)r[t].h.z | ((uint64_t)r[t].h.w << 32);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t m0 = (uint32_t)(pm >> (12 * i)) & 63u, m1 = (uint32_t)(pm >> (12 * i + 6)) & 63u;
        w[i] = h2_fma(m0 | (m1 << 16) | 0x64006400u, H2_ONE, H2_M1024);
      }
      mb[t] = make_uint4(w[0], w[1], w[2], w[3]);
      dd[t] = half_bits_to_float(r[t].h.y >> 16);
      dm64[t] = 64.0f * half_bits_to_float(r[t].h.w >> 16);
    }
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      const uint4 am = lmin[cg * GF_BLK + lane];
      const float4 s4 = *(const float4*)&lscale[16 * cg + 4 * g];
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const qwg_f32x4 M = mfma_f16(am, mb[t], qwg_f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y[t][cg][i] = __builtin_fmaf(sv[i], __builtin_fmaf(dd[t], P[t][cg][i], -(dm64[t] * M[i])), y[t][cg][i]);
      }
    }
  };

  // zeros in both buffers: the entries of columns >= nc and the minimum-term lanes 32..63 stay zero
  for (int i = tid; i < BUF; i += 64 * GF_WAVES) {
    buf0[i] = make_uint4(0, 0, 0, 0);
    buf1[i] = make_uint4(0, 0, 0, 0);
  }
  const bool fused = a.part == nullptr;
  if (fused) {  // eight threads per column sum its chunks' squares
    const int col = tid >> 3;
    float sq = 0.f;
    if (a.e.sq_in && col < nc)
      for (int i = tid & 7; i < a.e.sq_in_n; i += 8) sq += a.e.sq_in[(int64_t)col * a.e.sq_in_stride + i];
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    sq += __shfl_xor(sq, 4);
    if ((tid & 7) == 0) lrs[col] = a.e.sq_in ? 1.0f / sqrtf(sq / a.e.rms_k + a.e.eps) : 1.0f;
  }
  __syncthreads();
  // raw weights in two named sets (even and odd superblocks), so that a request lands where the
  // multiply after next reads it, without copies on the loop's back-edge
  SbRaw<QT> wa[T], wb[T];
  auto load = [&](SbRaw<QT>* dst, int sbi) {
    if (live && sbi < nsb) {
#pragma unroll
      for (int t = 0; t < T; ++t) dst[t] = sb_load<QT>(a.w, ro[t], srow[t], sb0 + sbi, g);
    }
  };
  // one step: request superblock sbi + 1 (operands into `nxt`, weights into wn), multiply superblock
  // sbi from `now` with weights wc, then wait for this wave's requests and meet the other waves (after
  // which `now` may be overwritten and `nxt` is complete)
  auto step = [&](int sbi, const uint4* now, uint4* nxt, const SbRaw<QT>* wc, SbRaw<QT>* wn) {
    if (sbi + 1 < nsb) f16_stage<CG>(nxt, a, sb0 + sbi + 1, wave, lane);
    load(wn, sbi + 1);
    if (live) superblock(now, wc);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  };
  if (nsb > 0) {
    f16_stage<CG>(buf0, a, sb0, wave, lane);
    load(wa, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's requests are in LDS
    __syncthreads();
  }
  for (int sbi = 0; sbi < nsb; sbi += 2) {
    step(sbi, buf0, buf1, wa, wb);
    if (sbi + 1 < nsb) step(sbi + 1, buf1, buf0, wb, wa);
  }
  // (row r0 + 16 t + n, column 16 cg + 4 g + i): the SwiGLU epilogue (rows n and n ^ 1, the gate and
  // up pair, are lanes l and l ^ 1), or this split's partial sums
  if (live) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int row = r0 + 16 * t + n;
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 16 * cg + 4 * g + i;
          if (fused) {
            const float v = y[t][cg][i] * lrs[col];
            const float vp = __shfl_xor(v, 1);
            if (row < rows && col < nc) run_epilogue(EPI_SWIGLU, a.e, col, row, v, vp);
          } else if (row < rows && col < nc) {
            a.part[((int64_t)split * nc + col) * rows + row] = y[t][cg][i];
          }
        }
    }
  }
}

// Fixed-order sum of the K splits of k_gemm_mfma, the RMSNorm scale and the epilogue: one thread per
// (row, column), 256 rows per workgroup (pairs of rows share a wave for RoPE and SwiGLU), column =
// blockIdx.y.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_reduce(const float* part, int ksplit, int nc, int rows, EpiArgs e) {
  __shared__ float red[16];
  const int n = blockIdx.y, tid = threadIdx.x;
  const int row = blockIdx.x * blockDim.x + tid;
  float rs = 1.0f;
  if (e.sq_in) {
    float sq = 0.f;
    for (int i = tid; i < e.sq_in_n; i += blockDim.x) sq += e.sq_in[(int64_t)n * e.sq_in_stride + i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if ((tid & 63) == 0) red[tid >> 6] = sq;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
    rs = 1.0f / sqrtf(t / e.rms_k + e.eps);
  }
  float v = 0.f;
  if (row < rows)
    for (int s = 0; s < ksplit; ++s) v += part[((int64_t)s * nc + n) * rows + row];
  v *= rs;
  const float vp = __shfl_xor(v, 1);
  const float o = row < rows ? run_epilogue(EPI, e, n, row, v, vp) : 0.f;
  if constexpr (EPI == EPI_RESID) {
    if (e.dig_out) {
      // the block's 256 outputs are superblock blockIdx.x of column n: its DIG_F16 pieces (of gain *
      // h) and per-chunk sums of h^2, as k_digitize writes them (the host checks rows % 256 == 0)
      __shared__ float bmax[4], bnan[4];
      const float x = e.dig_gain ? o * e.dig_gain[row] : o;
      float mx = fabsf(x), nf = __builtin_fmaf(x, 0.0f, 0.f), ss = o * o;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off));
        nf += __shfl_xor(nf, off);
      }
      if ((tid & 63) == 0) {
        bmax[tid >> 6] = mx;
        bnan[tid >> 6] = nf;
      }
      __syncthreads();
      mx = fmaxf(fmaxf(bmax[0], bmax[1]), fmaxf(bmax[2], bmax[3]));
      const bool bad = __builtin_isnan(bnan[0] + bnan[1] + bnan[2] + bnan[3]);
      int sh = 0;
      if (mx > 0.f && !bad) sh = min(149, 15 - __builtin_amdgcn_frexp_expf(mx));
      const float xp = bad ? 0.f : ldexpf(x, sh);
      float cs = xp;  // the chunk's sum of x' (and of h^2): the 32 rows of a chunk are a half-wave
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) {
        cs += __shfl_xor(cs, off);
        ss += __shfl_xor(ss, off);
      }
      uint32_t* sb = e.dig_out + (int64_t)n * e.dig_stride + (int64_t)blockIdx.x * F16_SB_WORDS;
      const int c = tid >> 5, p = tid & 31, m = (p & 15) >> 2, j = p & 3;
      const int el = 4 * (p >> 4) + ((j == 1) ? 2 : (j == 2) ? 1 : j);  // the element order of the pieces
      const _Float16 hi = (_Float16)xp, lo = (_Float16)(xp - (float)hi);
      uint16_t* h16 = (uint16_t*)sb;
      h16[(((c * 2 + 0) * 4 + m) * 4) * 2 + el] = __builtin_bit_cast(uint16_t, hi);
      h16[(((c * 2 + 1) * 4 + m) * 4) * 2 + el] = __builtin_bit_cast(uint16_t, lo);
      if (p == 0) {
        const float s6 = cs * 0.015625f;
        const _Float16 shh = (_Float16)s6, shl = (_Float16)(s6 - (float)shh);
        uint16_t* s16 = (uint16_t*)(sb + F16_SUM_WORD);
        s16[c] = __builtin_bit_cast(uint16_t, shh);
        s16[8 + c] = __builtin_bit_cast(uint16_t, shl);
        if (e.sq_out) e.sq_out[(int64_t)n * e.sq_out_stride + (int64_t)blockIdx.x * 8 + c] = ss;
        if (c == 0) sb[F16_SCALE_WORD] = __float_as_uint(bad ? __builtin_nanf("") : ldexpf(1.0f, -sh));
      }
    }
  }
}

// DIG_F16 pieces of one superblock: the 32 lanes of a half-wave hold its 8 chunks (lane m of each
// quad takes elements 4m..4m+3 and 16+4m..16+4m+3 of its chunk in v), o is the column's base and c
// the lane's chunk.  All 32 lanes must call it.
__device__ inline void digitize_f16(const float* v, int m, uint32_t* o, int c, bool write) {
  float mx = 0.f, nf = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mx = fmaxf(mx, fabsf(v[i]));
    nf = __builtin_fmaf(v[i], 0.0f, nf);  // NaN exactly when an element is a NaN or an infinity
  }
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, d));
    nf += __shfl_xor(nf, d);
  }
  const bool bad = __builtin_isnan(nf);
  // x' = x 2^sh with the maximum in [2^14, 2^15); 2^-sh >= 2^-149 stays representable
  int sh = 0;
  if (mx > 0.f && !bad) sh = min(149, 15 - __builtin_amdgcn_frexp_expf(mx));
  float xp[8], sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xp[i] = bad ? 0.f : ldexpf(v[i], sh);
    sum += xp[i];
  }
  sum = quad_sum(sum) * 0.015625f;  // 2^-6 x the chunk's sum of x' (below 2^14)
  if (!write) return;
  auto pieces = [](float a, float b, uint32_t& hi, uint32_t& lo) {  // (a, b) as hi and lo half pairs
    const _Float16 ah = (_Float16)a, bh = (_Float16)b;
    const _Float16 al = (_Float16)(a - (float)ah), bl = (_Float16)(b - (float)bh);
    hi = (uint32_t)__builtin_bit_cast(uint16_t, ah) | ((uint32_t)__builtin_bit_cast(uint16_t, bh) << 16);
    lo = (uint32_t)__builtin_bit_cast(uint16_t, al) | ((uint32_t)__builtin_bit_cast(uint16_t, bl) << 16);
  };
  uint4 h, l;
  pieces(xp[0], xp[2], h.x, l.x);  // elements 4m, 4m+2
  pieces(xp[1], xp[3], h.y, l.y);  // 4m+1, 4m+3
  pieces(xp[4], xp[6], h.z, l.z);  // 16+4m, 16+4m+2
  pieces(xp[5], xp[7], h.w, l.w);  // 16+4m+1, 16+4m+3
  uint32_t* sb = o + (int64_t)(c >> 3) * F16_SB_WORDS;
  const int cl = c & 7;
  *(uint4*)(sb + ((cl * 2 + 0) * 4 + m) * 4) = h;
  *(uint4*)(sb + ((cl * 2 + 1) * 4 + m) * 4) = l;
  if (m == 0) {
    const _Float16 shh = (_Float16)sum, shl = (_Float16)(sum - (float)shh);
    uint16_t* s16 = (uint16_t*)(sb + F16_SUM_WORD);
    s16[cl] = __builtin_bit_cast(uint16_t, shh);
    s16[8 + cl] = __builtin_bit_cast(uint16_t, shl);
    if (cl == 0) sb[F16_SCALE_WORD] = __float_as_uint(bad ? __builtin_nanf("") : ldexpf(1.0f, -sh));
  }
}

// Activation digits of nc columns of length k, four threads per 32-element chunk (thread m takes
// elements 4m..4m+3 and 16+4m..16+4m+3 with two float4 loads).  With a gain vector the digits are
// of g * x and sq receives each chunk's sum of x^2 (for the consumer's RMSNorm).
__global__ __launch_bounds__(256) void k_digitize(const float* x, int64_t x_stride, const float* gain, int k, int kind,
                                                  uint32_t* out, int64_t out_stride, float* sq, int64_t sq_stride) {
  const int n = blockIdx.y;
  const int nx = k / XCHUNK;
  const float* xr = x + (int64_t)n * x_stride;
  const int m = threadIdx.x & 3;
  const int c = blockIdx.x * (blockDim.x >> 2) + (threadIdx.x >> 2);
  const bool ok = c < nx;
  const int cc = ok ? c : 0;
  const float4 lo = *(const float4*)(xr + (int64_t)cc * XCHUNK + 4 * m);
  const float4 hi = *(const float4*)(xr + (int64_t)cc * XCHUNK + 16 + 4 * m);
  float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  if (gain) {
    const float4 gl = *(const float4*)(gain + (int64_t)cc * XCHUNK + 4 * m);
    const float4 gh = *(const float4*)(gain + (int64_t)cc * XCHUNK + 16 + 4 * m);
    const float g[8] = {gl.x, gl.y, gl.z, gl.w, gh.x, gh.y, gh.z, gh.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= g[i];
  }
  if (kind == DIG_F16)  // whole superblocks: k is a multiple of 256, so a half-wave's chunks are all valid or not
    digitize_f16(v, m, out + (int64_t)n * out_stride, cc, ok);
  else
    digitize_group(v, m, kind, out + (int64_t)n * out_stride + (int64_t)cc * DIG_CHUNK_WORDS, ok);
  if (sq) {
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (ok && m == 0) sq[(int64_t)n * sq_stride + c] = ss;
  }
}

hipError_t launch_digitize(const float* x, int64_t x_stride, const float* gain, int64_t k, int nc, int qt, void* out,
                           int64_t out_stride_bytes, float* sq, int64_t sq_stride, hipStream_t st) {
  const int64_t nx = k / XCHUNK;
  hipLaunchKernelGGL(k_digitize, dim3((unsigned)((nx + 63) / 64), nc), dim3(256), 0, st, x, x_stride, gain, (int)k,
                     gemv_digit_kind(qt, k, nc), (uint32_t*)out, out_stride_bytes / 4, sq, sq_stride);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ host side

static int g_waves = 0, g_rows = 0, g_depth = 0, g_passes = 0;  // launch-geometry overrides (0 = default)
constexpr int PERSISTENT_WGS = 256;   // workgroups of a persistent several-column GEMV: one per CU
constexpr int PERSISTENT_WGS1 = 768;  // of a persistent one-column GEMV: three per CU

void set_gemv_geometry(int waves, int rows_per_wave, int depth, int passes) {
  g_waves = waves;
  g_rows = rows_per_wave;
  g_depth = depth;
  g_passes = passes;
}

static int g_mfma = 1;  // several-column Q5_K / Q6_K GEMVs on the matrix cores
void set_gemv_mfma(int on) { g_mfma = on ? 1 : 0; }

// waves per workgroup of the matrix-core form: four per SIMD with one column group (128 VGPRs), two
// with two (their operands need up to 256)
constexpr int mf_waves(int ng) { return ng == 1 ? 16 : 8; }

// Matrix-core plan: K splits as LDS requires (a power of two, so the splits' grids tile the 256 CUs),
// then the K parts per tile S in {1, 2, 4, 8, 16} that minimise rounds x steps per wave, where a
// round is one block per workgroup and a workgroup runs on each CU.
int gemv_digit_kind(int qt, int64_t k, int nc) {
  const int mf = plan_gemv(qt, 1, k, nc, EPI_STORE).mfma;
  return mf == 3 ? DIG_F16 : mf ? DIG_BYTE : digit_kind(qt);
}

static GemvPlan plan_mfma(int64_t rows, int64_t k, int nc) {
  const int64_t unit = 16;  // chunks per step (two superblocks): splits hold whole steps
  const int ng = nc > 4 ? 2 : 1;
  GemvPlan p{};
  p.mfma = 1;
  p.ncm = 4 * ng;
  p.waves = mf_waves(ng);
  if (g_waves >= 2 && g_waves <= p.waves && g_waves % 2 == 0) p.waves = g_waves;  // tuning override
  p.rows_per_wave = 16;
  p.depth = 1;
  p.passes = 0;
  const int64_t nx = k / XCHUNK;
  const size_t fixed = (size_t)ng * mf_waves(ng) * 64 * 4 + mf_fixed_lds(ng);  // K parts' partial sums, padding
  int64_t max_x = (int64_t)((LDS_BUDGET - fixed) / mf_chunk_lds(ng)) / unit * unit;
  int ksplit = 1;
  while (ksplit < 64 && ((nx + ksplit - 1) / ksplit + unit - 1) / unit * unit > max_x) ksplit *= 2;
  const int64_t xs = ((nx + ksplit - 1) / ksplit + unit - 1) / unit * unit;
  p.ks = (int)(xs * XCHUNK);
  p.ksplit = (int)((k + p.ks - 1) / p.ks);
  p.lds = (size_t)xs * mf_chunk_lds(ng) + fixed;
  p.part_bytes = p.ksplit > 1 ? (size_t)p.ksplit * nc * rows * sizeof(float) : 0;
  const int64_t tiles = (rows + 15) / 16, nst = xs / unit;
  const int64_t G = std::max(1, PERSISTENT_WGS / p.ksplit);
  // A CU runs one workgroup per round: W waves = T tiles x S K parts.  Measured at the 70B shapes,
  // a round costs about T x nst tile-steps of the CU (more waves per tile only hide latency) plus
  // a fixed ~8, so the plan minimises rounds x (T x nst + 8) over W (8..16, or 4..8 with two column
  // groups) and S, then prefers more waves and fewer K parts.
  const int wmax = p.waves, wmin = wmax / 2;
  int64_t best = -1;
  int best_w = wmax;
  for (int W = wmax; W >= wmin; W -= 2) {
    if (g_waves > 0 && W != p.waves) continue;  // tuning override: waves per workgroup
    for (int S = 1; S <= W; S *= 2) {
      if (W % S) continue;
      if (g_passes > 0 && S != g_passes) continue;  // tuning override: K parts per tile
      const int64_t T = W / S, nblk = (tiles + T - 1) / T, rounds = (nblk + G - 1) / G;
      const int64_t cost = rounds * (T * nst + 8);
      if (best < 0 || cost < best) {
        best = cost;
        best_w = W;
        p.kparts = S;
        p.grid_x = (int)std::min(nblk, G);
      }
    }
  }
  p.waves = best_w;
  return p;
}

// formats whose 4-row two-pass kernel fits 128 registers without spilling
static bool two_pass_ok(int qt) { return qt == Q4_0 || qt == Q4_K || qt == Q8_0; }

// The prefill form (9..64 columns): 256 rows per workgroup (Q4_K / Q5_K: 8 waves of two 16-row tiles
// on the fp16 matrix cores; Q6_K: 16 waves of one tile on the i8 ones), and K splits (whole steps of 16
// chunks) until the workgroups cover about one per CU; the splits always go through k_gemm_reduce.
static GemvPlan plan_gemm64(int qt, int64_t rows, int64_t k, int nc) {
  GemvPlan p{};
  const bool f16 = qt == Q4_K || qt == Q5_K;
  p.mfma = f16 ? 3 : 2;
  p.ncm = 4 * GM_NG;
  p.waves = f16 ? GF_WAVES : GM_WAVES;
  p.rows_per_wave = f16 ? 32 : 16;
  p.depth = 1;
  p.passes = 1;
  const int64_t nblk = (rows + 255) / 256;
  const int64_t nsteps = k / (XCHUNK * GM_SC);
  int64_t ksplit = std::max<int64_t>(1, std::min<int64_t>(nsteps, (PERSISTENT_WGS + nblk / 2) / std::max<int64_t>(1, nblk)));
  const int64_t sps = (nsteps + ksplit - 1) / ksplit;
  ksplit = (nsteps + sps - 1) / sps;
  p.ks = (int)(sps * XCHUNK * GM_SC);
  p.ksplit = (int)ksplit;
  p.grid_x = (int)nblk;
  p.lds = f16 ? 0 : GM_LDS;  // the fp16 form's buffers are static
  p.part_bytes = (size_t)ksplit * nc * rows * sizeof(float);
  return p;
}

GemvPlan plan_gemv(int qt, int64_t rows, int64_t k, int nc, int epi, int mfma) {
  if (nc > MAX_COLS && (qt == Q4_K || qt == Q5_K || qt == Q6_K) && k % 512 == 0) return plan_gemm64(qt, rows, k, nc);
  if ((mfma < 0 ? g_mfma : mfma) && nc >= 2 && nc <= 8 && (qt == Q4_K || qt == Q5_K || qt == Q6_K) &&
      k % 512 == 0)  // steps are two superblocks
    return plan_mfma(rows, k, nc);
  // the RoPE and SwiGLU epilogues combine rows (2i, 2i+1), which must sit in one wave
  const bool pairs = epi == EPI_QKV || epi == EPI_SWIGLU;
  GemvPlan p{};
  p.ncm = nc <= 1 ? 1 : (nc <= 4 ? 4 : 8);
  p.rows_per_wave = 2;
  p.waves = 8;
  p.passes = 1;
  p.depth = 1;
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
  p.lds = (size_t)lds_row_slots((int)xs) * per_chunk;
  p.part_bytes = p.ksplit > 1 ? (size_t)p.ksplit * nc * rows * sizeof(float) : 0;
  // one column, two rows per wave (measured on the 70B shapes: a four-row kernel needs about 110
  // registers against about 70, and the occupancy two rows leave wins).  The residual epilogue also
  // writes the next GEMV's input digits, which takes whole 32-element chunks of output per
  // workgroup: 8 waves x two row passes = 32 rows.  SwiGLU runs the same 8 waves x two passes = 32
  // rows (16 outputs, so the down GEMV digitizes its fp32 input itself).  Every workgroup stages the
  // whole activation (36 KB at K = 8192), so four fit a CU: measured at the 70B shapes, 8-wave
  // workgroups beat the 4-wave ones for gate|up (46.3 against 48.8 us) and 10-wave workgroups of 20
  // rows (two per CU, staging the activation 512 times) beat 8-row ones for QKV (14.0 against 17.7).
  if (p.ncm == 1 && p.ksplit == 1) {
    if (epi == EPI_RESID || epi == EPI_SWIGLU) p.passes = 2;
    if (epi == EPI_QKV) p.waves = 10;
  }
  // Very tall one-column GEMVs (the 128256-row head: 8016 blocks of 16 rows) run persistent: a grid
  // of PERSISTENT_WGS1 workgroups strides over the row blocks, so the activation is staged once per
  // workgroup instead of once per 16 rows (224 MB of staging reads at 128256 x 8192).
  const int64_t blk1 = (int64_t)p.waves * p.rows_per_wave;
  const bool tall = p.ncm == 1 && p.ksplit == 1 && epi == EPI_STORE &&
                    (rows + blk1 - 1) / blk1 > 4 * PERSISTENT_WGS1;
  // explicit overrides (tuning and tests)
  if (g_waves >= 1 && (g_waves <= 8 || (g_waves <= 16 && p.ncm == 1))) p.waves = g_waves;
  if (p.ncm == 1 && (g_rows == 1 || g_rows == 2 || g_rows == 4)) p.rows_per_wave = g_rows;
  if (g_depth == 1 || g_depth == 2) p.depth = g_depth;
  if (g_passes == 1 || g_passes == 2 || g_passes == 4 || g_passes == 8) p.passes = g_passes;
  if (pairs && p.rows_per_wave < 2) p.rows_per_wave = 2;
  if (p.waves > 8) {  // the 1024-thread kernels are compiled for two rows and one-ahead loads only
    p.rows_per_wave = 2;
    p.depth = 1;
  }
  if ((p.rows_per_wave == 4 || p.waves > 8) && p.passes >= 4) p.passes = 2;
  // compiled row-pass variants: one column, one-ahead loads, digitizing epilogues; two rows with two
  // or four passes (sixteen waves: two), four rows with two passes for the formats whose four-row
  // kernel fits 128 registers
  const bool pass_ok = p.ncm == 1 && p.depth == 1 && p.ksplit == 1 && (epi == EPI_RESID || epi == EPI_SWIGLU) &&
                       ((p.rows_per_wave == 2 && (p.passes == 2 || p.passes == 4 || p.passes == 8)) ||
                        (p.rows_per_wave == 4 && p.passes == 2 && two_pass_ok(qt)));
  if (!pass_ok) p.passes = 1;
  // several columns: the staged activation (112 B per 32 elements and column) is as large as the
  // weights a workgroup of one pass reads, so one workgroup per CU stages it once and strides over
  // the row blocks (persistent)
  if (tall && p.waves == 8 && p.rows_per_wave == 2 && p.depth == 1 && g_passes == 0) {
    const int64_t blk = (int64_t)p.waves * p.rows_per_wave;
    const int64_t nblk = (rows + blk - 1) / blk;
    p.passes = 0;
    p.grid_x = (int)std::max<int64_t>(PERSISTENT_WGS1, (nblk + 64 / p.rows_per_wave - 1) / (64 / p.rows_per_wave));
  }
  if (p.ncm > 1) {
    p.passes = 0;
    p.depth = 1;
    // four columns: the staged activation leaves one workgroup per CU whatever the registers, so
    // waves take four rows (about 240 registers) for twice the loads in flight -- where that still
    // leaves every workgroup two or more row blocks (gate|up, down; not QKV or Wo)
    const int64_t nblk4 = (rows + (int64_t)p.waves * 4 - 1) / ((int64_t)p.waves * 4);
    const int64_t grid4 = std::max<int64_t>(std::max(1, PERSISTENT_WGS / p.ksplit), (nblk4 + 15) / 16);
    p.rows_per_wave = (p.ncm == 4 && g_rows != 2 && nblk4 >= 2 * grid4) ? 4 : 2;
    // a wave parks each finished row group's totals in R lanes: at most 64 / R groups per workgroup
    const int64_t blk = (int64_t)p.waves * p.rows_per_wave;
    const int64_t nblk = (rows + blk - 1) / blk;
    const int64_t min_grid = (nblk + 64 / p.rows_per_wave - 1) / (64 / p.rows_per_wave);
    p.grid_x = (int)std::max<int64_t>(std::max(1, PERSISTENT_WGS / p.ksplit), min_grid);
  }
  return p;
}

// compiled input-digitizing kernels: 32 rows per workgroup as 8 waves x 4 rows, 8 waves x 2 rows x 2
// passes, or 16 waves x 2 rows; four-column K-split residual GEMVs (the verify pass's down GEMV)
bool gemv_can_digitize_input(const GemvPlan& p, int epi) {
  if (p.mfma) return false;
  if (p.ncm == 4) return epi == EPI_RESID && p.ksplit > 1 && p.passes == 0 && p.depth == 1 && p.waves == 8;
  if (!(p.ncm == 1 && p.ksplit == 1 && epi == EPI_RESID && p.depth == 1)) return false;
  if (p.waves > 8) return p.rows_per_wave == 2 && p.passes == 1;
  return (p.rows_per_wave == 4 && p.passes == 1) || (p.rows_per_wave == 2 && p.passes == 2);
}

bool gemv_can_digitize_output(const GemvPlan& p, int epi, int64_t rows, int kind) {
  if (p.mfma >= 2) return epi == EPI_RESID && kind == DIG_F16 && rows % 256 == 0;
  if (kind != DIG_NIB && kind != DIG_BYTE) return false;
  if (epi != EPI_RESID && epi != EPI_SWIGLU) return false;
  if (rows % (epi == EPI_SWIGLU ? 2 * XCHUNK : XCHUNK) != 0) return false;
  if (p.ksplit > 1) return true;  // the reduce kernel covers 256 rows per block
  if (p.passes == 0) return false;  // persistent workgroups own scattered row blocks
  const int outs = p.waves * p.rows_per_wave * p.passes / (epi == EPI_SWIGLU ? 2 : 1);
  return outs % XCHUNK == 0 && outs <= 64;
}

// A launch on stream st; with events, hipExtLaunchKernelGGL records them at the kernel's own start
// and end (no dispatch latency inside the interval).
struct Dispatch {
  hipStream_t st;
  hipEvent_t start, stop;
};
template <class Kern, class... Args>
static void go(const Dispatch& d, Kern kern, dim3 grid, dim3 block, size_t lds, Args... args) {
  if (d.start || d.stop)
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, d.st, d.start, d.stop, 0u, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, d.st, args...);
}

template <int QT, int NCM, int R, int PD, int P = 1, int LB = 512>
static hipError_t launch_t(const GemvArgs& a, int epi, int ksplit, dim3 grid, dim3 block, size_t lds,
                           const Dispatch& d) {
  switch (ksplit > 1 ? EPI_PART : epi) {
    case EPI_PART: go(d, k_gemv<QT, NCM, R, EPI_PART, PD, P, LB>, grid, block, lds, a); break;
    case EPI_STORE: go(d, k_gemv<QT, NCM, R, EPI_STORE, PD, P, LB>, grid, block, lds, a); break;
    case EPI_RESID: go(d, k_gemv<QT, NCM, R, EPI_RESID, PD, P, LB>, grid, block, lds, a); break;
    case EPI_SWIGLU: go(d, k_gemv<QT, NCM, R, EPI_SWIGLU, PD, P, LB>, grid, block, lds, a); break;
    case EPI_QKV: go(d, k_gemv<QT, NCM, R, EPI_QKV, PD, P, LB>, grid, block, lds, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// P row passes (one column, one-ahead loads, residual or SwiGLU epilogue with output digits)
template <int QT, int R, int P, int LB = 512>
static hipError_t launch_pn(const GemvArgs& a, int epi, dim3 grid, dim3 block, size_t lds, const Dispatch& d) {
  switch (epi) {
    case EPI_RESID: go(d, k_gemv<QT, 1, R, EPI_RESID, 1, P, LB>, grid, block, lds, a); break;
    case EPI_SWIGLU: go(d, k_gemv<QT, 1, R, EPI_SWIGLU, 1, P, LB>, grid, block, lds, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QT>
static hipError_t launch_fmt(const GemvArgs& a, const GemvPlan& p, int epi, dim3 grid, dim3 block,
                             const Dispatch& dd) {
  const int r = p.rows_per_wave, d = p.depth;
  const size_t lds = p.lds;
  if (a.e.xf) {
    if (!gemv_can_digitize_input(p, epi)) return hipErrorInvalidValue;
    if (p.ncm == 4) {  // K-split verify GEMV: partial sums out
      if (r == 4)
        go(dd, k_gemv<QT, 4, 4, EPI_PART, 1, 0, 512, 1>, grid, block, lds, a);
      else
        go(dd, k_gemv<QT, 4, 2, EPI_PART, 1, 0, 512, 1>, grid, block, lds, a);
    } else if (p.waves > 8)
      go(dd, k_gemv<QT, 1, 2, EPI_RESID, 1, 1, 1024, 1>, grid, block, lds, a);
    else if (r == 2 && p.waves == 8)  // segmented staging: 512 threads digitize 128 chunks at a time
      go(dd, k_gemv<QT, 1, 2, EPI_RESID, 1, 2, 512, 2>, grid, block, lds, a);
    else if (r == 2)
      go(dd, k_gemv<QT, 1, 2, EPI_RESID, 1, 2, 512, 1>, grid, block, lds, a);
    else
      go(dd, k_gemv<QT, 1, 4, EPI_RESID, 1, 1, 512, 1>, grid, block, lds, a);
    return hipGetLastError();
  }
  if (p.waves > 8) {  // more than eight waves: two rows, one-ahead loads, one or two passes
    if (p.ncm != 1 || r != 2 || d != 1) return hipErrorInvalidValue;
    if (p.passes == 2) return launch_pn<QT, 2, 2, 1024>(a, epi, grid, block, lds, dd);
    return launch_t<QT, 1, 2, 1, 1, 1024>(a, epi, p.ksplit, grid, block, lds, dd);
  }
  if (p.passes == 2 || p.passes == 4 || p.passes == 8) {
    if (p.ncm != 1 || d != 1 || p.ksplit > 1) return hipErrorInvalidValue;
    if (r == 2 && p.passes == 8) return launch_pn<QT, 2, 8>(a, epi, grid, block, lds, dd);
    if (r == 2) return p.passes == 2 ? launch_pn<QT, 2, 2>(a, epi, grid, block, lds, dd)
                                     : launch_pn<QT, 2, 4>(a, epi, grid, block, lds, dd);
    if (r == 4 && p.passes == 2) return launch_pn<QT, 4, 2>(a, epi, grid, block, lds, dd);
    return hipErrorInvalidValue;
  }
  if (p.ncm == 1 && r == 1) return d == 2 ? launch_t<QT, 1, 1, 2>(a, epi, p.ksplit, grid, block, lds, dd)
                                          : launch_t<QT, 1, 1, 1>(a, epi, p.ksplit, grid, block, lds, dd);
  if (p.ncm == 1 && r == 2 && p.passes == 0) {  // persistent (tall store GEMVs)
    if (epi != EPI_STORE || d != 1 || p.waves != 8) return hipErrorInvalidValue;
    return launch_t<QT, 1, 2, 1, 0>(a, epi, p.ksplit, grid, block, lds, dd);
  }
  if (p.ncm == 1 && r == 2) return d == 2 ? launch_t<QT, 1, 2, 2>(a, epi, p.ksplit, grid, block, lds, dd)
                                          : launch_t<QT, 1, 2, 1>(a, epi, p.ksplit, grid, block, lds, dd);
  if (p.ncm == 1) return d == 2 ? launch_t<QT, 1, 4, 2>(a, epi, p.ksplit, grid, block, lds, dd)
                                : launch_t<QT, 1, 4, 1>(a, epi, p.ksplit, grid, block, lds, dd);
  if (p.passes != 0) return hipErrorInvalidValue;  // several columns run persistent
  if (p.ncm == 4 && r == 4) return launch_t<QT, 4, 4, 1, 0>(a, epi, p.ksplit, grid, block, lds, dd);
  if (p.ncm == 4) return launch_t<QT, 4, 2, 1, 0>(a, epi, p.ksplit, grid, block, lds, dd);
  return launch_t<QT, 8, 2, 1, 0>(a, epi, p.ksplit, grid, block, lds, dd);
}

template <int QT, int NG>
static hipError_t launch_mfma_ng(const GemvArgs& a, int epi, const GemvPlan& p, dim3 grid, dim3 block,
                                 const Dispatch& d) {
  const int S = p.kparts;
  switch (p.ksplit > 1 ? EPI_PART : epi) {
    case EPI_PART: go(d, k_gemv_mfma<QT, EPI_PART, NG>, grid, block, p.lds, a, S); break;
    case EPI_STORE: go(d, k_gemv_mfma<QT, EPI_STORE, NG>, grid, block, p.lds, a, S); break;
    case EPI_RESID: go(d, k_gemv_mfma<QT, EPI_RESID, NG>, grid, block, p.lds, a, S); break;
    case EPI_SWIGLU: go(d, k_gemv_mfma<QT, EPI_SWIGLU, NG>, grid, block, p.lds, a, S); break;
    case EPI_QKV: go(d, k_gemv_mfma<QT, EPI_QKV, NG>, grid, block, p.lds, a, S); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int QT>
static hipError_t launch_mfma(const GemvArgs& a, int epi, const GemvPlan& p, dim3 grid, dim3 block, const Dispatch& d) {
  return p.ncm == 8 ? launch_mfma_ng<QT, 2>(a, epi, p, grid, block, d) : launch_mfma_ng<QT, 1>(a, epi, p, grid, block, d);
}

hipError_t launch_gemv(int qt, const MatView& w, int64_t k, const void* xd, int64_t xd_stride_bytes, int nc, int epi,
                       const EpiArgs& e, float* part, hipStream_t st, const GemvPlan& p, hipEvent_t ev_start,
                       hipEvent_t ev_stop) {
  // the kernels keep per-column sums in arrays of MAX_COLS (the prefill form: 64 columns)
  if (nc < 1 || nc > p.ncm || (p.mfma < 2 && nc > MAX_COLS)) return hipErrorInvalidValue;
  if (e.dig_out && !gemv_can_digitize_output(p, epi, w.rows, e.dig_kind)) return hipErrorInvalidValue;
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
  const int blk_rows = p.waves * p.rows_per_wave;
  const int nblk = (rows + blk_rows - 1) / blk_rows;
  const int gx = p.passes > 0 ? (nblk + p.passes - 1) / p.passes : std::min(nblk, std::max(1, p.grid_x));
  dim3 grid(gx, p.ksplit);
  dim3 block(64 * p.waves);
  // the stop event goes on the last kernel: the GEMV itself, or the split reduction after it
  const Dispatch d1{st, ev_start, p.ksplit == 1 ? ev_stop : nullptr};
  hipError_t err;
  if (p.mfma >= 2) {
    // the fp16 form runs the SwiGLU epilogue itself when K is not split
    const bool fused = p.mfma == 3 && p.ksplit == 1 && epi == EPI_SWIGLU;
    if (e.xf || (!part && !fused)) return hipErrorInvalidValue;
    grid.x = p.grid_x;
    const Dispatch d0{st, ev_start, fused ? ev_stop : nullptr};
    if (p.mfma == 3) {
      GemvArgs af = a;
      if (fused) af.part = nullptr;
      // the narrowest build whose groups hold nc columns
      const int ncg = nc <= 16 ? 1 : nc <= 32 ? 2 : nc <= 64 ? 4 : 0;
      switch (qt * 8 + ncg) {
        case Q4_K * 8 + 1: go(d0, k_gemm_f16<Q4_K, 1>, grid, block, p.lds, af); break;
        case Q4_K * 8 + 2: go(d0, k_gemm_f16<Q4_K, 2>, grid, block, p.lds, af); break;
        case Q4_K * 8 + 4: go(d0, k_gemm_f16<Q4_K, 4>, grid, block, p.lds, af); break;
        case Q5_K * 8 + 1: go(d0, k_gemm_f16<Q5_K, 1>, grid, block, p.lds, af); break;
        case Q5_K * 8 + 2: go(d0, k_gemm_f16<Q5_K, 2>, grid, block, p.lds, af); break;
        case Q5_K * 8 + 4: go(d0, k_gemm_f16<Q5_K, 4>, grid, block, p.lds, af); break;
        default: return hipErrorInvalidValue;
      }
      if (fused) return hipGetLastError();
    } else {
      switch (qt) {
        case Q6_K: go(d0, k_gemm_mfma<Q6_K>, grid, block, p.lds, a); break;
        default: return hipErrorInvalidValue;
      }
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const Dispatch dr{st, nullptr, ev_stop};
    dim3 rg((rows + 255) / 256, nc);
    switch (epi) {
      case EPI_STORE: go(dr, k_gemm_reduce<EPI_STORE>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
      case EPI_RESID: go(dr, k_gemm_reduce<EPI_RESID>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
      case EPI_SWIGLU: go(dr, k_gemm_reduce<EPI_SWIGLU>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
      case EPI_QKV: go(dr, k_gemm_reduce<EPI_QKV>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (p.mfma) {
    if (e.xf || nc < 1 || nc > p.ncm) return hipErrorInvalidValue;
    grid.x = p.grid_x;
    switch (qt) {
      case Q4_K: err = launch_mfma<Q4_K>(a, epi, p, grid, block, d1); break;
      case Q5_K: err = launch_mfma<Q5_K>(a, epi, p, grid, block, d1); break;
      case Q6_K: err = launch_mfma<Q6_K>(a, epi, p, grid, block, d1); break;
      default: return hipErrorInvalidValue;
    }
  } else switch (qt) {
    case Q8_0: err = launch_fmt<Q8_0>(a, p, epi, grid, block, d1); break;
    case Q4_0: err = launch_fmt<Q4_0>(a, p, epi, grid, block, d1); break;
    case Q4_K: err = launch_fmt<Q4_K>(a, p, epi, grid, block, d1); break;
    case Q5_K: err = launch_fmt<Q5_K>(a, p, epi, grid, block, d1); break;
    case Q6_K: err = launch_fmt<Q6_K>(a, p, epi, grid, block, d1); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess || p.ksplit == 1) return err;
  const Dispatch d2{st, nullptr, ev_stop};
  dim3 rg((rows + 255) / 256);
  switch (epi) {
    case EPI_STORE: go(d2, k_gemv_reduce<EPI_STORE>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
    case EPI_RESID: go(d2, k_gemv_reduce<EPI_RESID>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
    case EPI_SWIGLU: go(d2, k_gemv_reduce<EPI_SWIGLU>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
    case EPI_QKV: go(d2, k_gemv_reduce<EPI_QKV>, rg, dim3(256), 0, part, p.ksplit, nc, rows, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qwg
