// qwg_kernels.h -- host-side launchers of the gfx950 kernels (internal to libqwg.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qwg_formats.h"

namespace qwg {

constexpr int HEAD_DIM = 128;   // every supported model uses 128-wide heads
constexpr int MAX_COLS = 8;     // widest multi-column pass of the decode kernels (verify, short prefill)
constexpr int MAX_PREFILL_COLS = 64;  // widest prefill pass (K-quant layers: the 64-column GEMM)
constexpr size_t LDS_BUDGET = 150 * 1024;  // dynamic LDS per workgroup (gfx950: 160 KiB per CU)

// What the GEMV does with each finished output row (columns n < nc).
enum Epi : int {
  EPI_PART = 0,    // partial sum of one K split (written to the split workspace)
  EPI_STORE = 1,   // y[n][r] = v
  EPI_RESID = 2,   // y[n][r] += v                      (Wo, W_down: residual add into h)
  EPI_SWIGLU = 3,  // rows (2i, 2i+1) = (gate_i, up_i): y[n][i] = silu(gate) * up
  EPI_QKV = 4,     // rows = [q heads | k heads | v heads]: RoPE on q,k; k,v -> fp16 KV cache rows
};

struct EpiArgs {
  // fp32 input that the GEMV digitizes itself in its prologue (instead of reading digits), or null
  const float* xf;
  int64_t xf_stride;     // floats between columns
  // RMSNorm in front of this GEMV: its input digits are of g * x, and the row sums are multiplied by
  // 1/sqrt(sum(x^2)/rms_k + eps), with sum(x^2) from per-chunk partials (fixed-order reduction)
  const float* sq_in;    // [nc][sq_in_stride] per-32-element-chunk sums of x^2, or null (no RMSNorm)
  int sq_in_n;           // chunks per column
  int64_t sq_in_stride;
  float rms_k;
  float eps;
  // digitization of this GEMV's output vector for the next GEMV (RESID: the new h; SWIGLU: silu*up)
  uint32_t* dig_out;     // digit words, column stride dig_stride words, or null
  int64_t dig_stride;
  const float* dig_gain; // the next GEMV's RMSNorm gain (digits of gain * out), or null
  int dig_kind;
  float* sq_out;         // per-chunk sums of out^2 for the next RMSNorm, column stride sq_out_stride, or null
  int64_t sq_out_stride;
  float* y;
  int64_t y_stride;      // floats between columns of y
  const float* rope;     // [max_ctx][HEAD_DIM/2] (cos, sin) pairs
  int pos;               // position of column 0
  int nq_rows, nkv_rows; // rows of the q part and of the k part (= v part)
  uint16_t* kc;          // K cache of the layer, [ctx][kv_stride]
  uint16_t* vc;
  int64_t kv_stride;     // n_kv * HEAD_DIM
};

struct GemvPlan {
  int ncm;     // compiled column bound (1, 4 or 8)
  int rows_per_wave;
  int waves;   // per workgroup
  int depth;   // weight-load pipeline depth (iterations in flight)
  int passes;  // row passes per wave (a workgroup covers waves * rows_per_wave * passes rows);
               // 0 = persistent: grid_x workgroups stride over the row blocks
  int grid_x;
  int ks;      // K per split
  int ksplit;
  size_t lds;  // dynamic LDS bytes
  size_t part_bytes;  // split workspace bytes (0 if ksplit == 1)
  int mfma;    // several columns on the matrix cores (k_gemv_mfma): waves = T tiles x kparts
  int kparts;  // waves that split one 16-row tile's chunks (MFMA form)
};

// epi: the epilogue the GEMV will run (pairs of rows must share a wave for RoPE and SwiGLU);
// mfma: 1 = the matrix-core form where one exists (2..8 columns of Q4_K / Q5_K / Q6_K with K a
// multiple of 512), 0 = integer dot
// products only, -1 = the process-wide choice (set_gemv_mfma, on by default)
GemvPlan plan_gemv(int qt, int64_t rows, int64_t k, int nc, int epi, int mfma = -1);
void set_gemv_geometry(int waves, int rows_per_wave, int depth, int passes);
void set_gemv_mfma(int on);

// Bytes of the activation digits of one column of length k (36 words per 32 elements).
inline int64_t digit_bytes(int64_t k) { return k / XCHUNK * DIG_CHUNK_WORDS * 4; }

// Digit kind (DIG_NIB / DIG_BYTE) that a GEMV over weights of type qt with K = k and nc columns
// consumes: byte digits on the matrix cores, else the format's own kind.  Every producer of a GEMV's
// input digits picks its kind with this.
int gemv_digit_kind(int qt, int64_t k, int nc);

// Digits of nc activation columns (x: [nc][x_stride] fp32) for a GEMV over weights of type qt;
// with a gain vector, digits of gain * x and per-chunk sums of x^2 into sq (column stride sq_stride).
hipError_t launch_digitize(const float* x, int64_t x_stride, const float* gain, int64_t k, int nc, int qt, void* out,
                           int64_t out_stride_bytes, float* sq, int64_t sq_stride, hipStream_t st);

// y = W x from activation digits xd (column stride in bytes) with an epilogue; `part` must hold
// plan.part_bytes when plan.ksplit > 1.  With events, ev_start / ev_stop are recorded at the start of
// the first kernel and the end of the last one.  Returns hipSuccess or the launch error.
hipError_t launch_gemv(int qt, const MatView& w, int64_t k, const void* xd, int64_t xd_stride_bytes, int nc, int epi,
                       const EpiArgs& e, float* part, hipStream_t st, const GemvPlan& plan,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

hipError_t launch_repack(int qt, const uint8_t* canon, int64_t rows, int64_t k, uint8_t* packed, const Layout& L,
                         int64_t dst_row0, int64_t dst_row_step, hipStream_t st);
hipError_t launch_dequant(int qt, const MatView& w, int64_t rows, int64_t k, float* out, hipStream_t st);
// h[n][:] = dequantized row tokens[n] of the embedding matrix
hipError_t launch_embed(int qt, const MatView& w, int64_t k, const int32_t* tokens, int nc, float* h, int64_t h_stride,
                        hipStream_t st);

hipError_t launch_rmsnorm(const float* x, const float* g, int64_t n, float eps, int nc, float* out, hipStream_t st);
hipError_t launch_rope(float* v, int n_heads, const float* table, int pos, hipStream_t st);
hipError_t launch_swiglu(const float* g, const float* u, int64_t n, float* out, hipStream_t st);
hipError_t launch_cosine(const float* a, const float* b, int64_t n, float* out, hipStream_t st);
// keys: scratch of nc 64-bit words (cleared by the launch itself, with a kernel: no memset node)
constexpr size_t ARGMAX_WORK_BYTES = MAX_COLS * 8;
hipError_t launch_argmax(const float* x, int64_t n, int nc, int64_t x_stride, int32_t* out, hipStream_t st,
                         unsigned long long* keys);

struct AttnPlan {
  int T;        // positions per split
  int nsplit;
  size_t work_bytes;
};
AttnPlan plan_attn(int n_pos, int n_q, int n_kv, int nc);
// Workspace bytes that cover plan_attn(p, n_q, n_kv, c) for every p <= n_pos and c <= nc (the tile
// count per split depends on the shape, so the plan's own size is not monotonic in either)
size_t attn_work_bound(int n_pos, int n_q, int n_kv, int nc);
// column j attends to positions [0, n_pos + j); with dig_out, the output is also written as
// activation digits (kind dig_kind, column stride dig_stride words) for the next GEMV
hipError_t launch_attn(const float* q, int64_t q_stride, const uint16_t* kc, const uint16_t* vc, int64_t kv_stride,
                       int n_pos, int n_q, int n_kv, int nc, float* out, int64_t out_stride, void* work,
                       const AttnPlan& p, hipStream_t st, uint32_t* dig_out = nullptr, int64_t dig_stride = 0,
                       int dig_kind = 0);

// plain streaming read of `bytes` (a multiple of 16) from src by `grid` workgroups of 8 waves (0:
// READ_GRID), each lane keeping `unroll` (4, 8 or 16; 0: 4) 16-byte loads in flight; one checksum
// word per wave into sink (grid * 8 words); optional events at the kernel's own start and end
constexpr int READ_GRID = 1024;
constexpr int READ_GRID_MAX = 8192;
hipError_t launch_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st, int grid = 0, int unroll = 0,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// a one-wave kernel that waits `ticks` of the wall clock (wall_clock64) and exits
hipError_t launch_spin(uint64_t ticks, hipStream_t st);

// True if the plan's kernels can write the output as activation digits of the given kind
// (gemv_digit_kind of the consumer) themselves: the one- and several-column forms when every
// workgroup writes whole 32-element chunks of a per-chunk kind; the prompt GEMMs' residual reduce
// when the consumer takes fp16 pieces and each of its 256-row blocks is one whole superblock.
bool gemv_can_digitize_output(const GemvPlan& p, int epi, int64_t rows, int kind);
// true if the plan has a variant that digitizes an fp32 input itself (EpiArgs::xf)
bool gemv_can_digitize_input(const GemvPlan& p, int epi);

}  // namespace qwg
