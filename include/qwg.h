/*
 * qwg.h -- C ABI of libqwg.so, the MI355X (gfx950) decode hot path of a
 * layer-streaming Llama inference engine with block-quantized weights.
 *
 * Sources of the operations (the NTransformer pages):
 *   [NT]   "NTransformer" (socker-news.uzaya.net/news/2026-02-22/article-3):
 *          "Key results", "Key features", "Quick start", "Architecture overview".
 *   [HN]   "Show HN: NVMe経由でCPUをバイパスして単一のRTX 3090上で動作するLlama 3.1 70B"
 *          (hakusoku.com/story/5379): quantization-format table, speed-up techniques,
 *          3-tier adaptive cache detail.
 *   [UR]   "RTX 3090 1枚でLlama 70B — NVMe-to-GPU直結でCPUバイパスする革新技術"
 *          (uravation.com): SLEP streaming pipeline, layer-skip mechanism.
 *
 * Conventions (every entry point):
 *   - Returns int status: QWG_OK (0) or a negative QWG_E_* code; the message of
 *     the last failure on the calling thread is qwg_last_error().  No C++
 *     exception crosses this boundary.
 *   - "d_" pointers are device (HBM) pointers owned by the caller; "h_" pointers
 *     are host pointers owned by the caller.  Nothing is retained after return
 *     unless stated.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  Kernel-level calls are asynchronous on that stream; device-side
 *     faults surface at the next call that synchronizes.
 *   - Shapes are validated before any launch: a matrix of qtype T has k a
 *     multiple of qwg_block_weights(T) (32 or 256), else QWG_E_SHAPE.
 *   - The packed device layout of a weight matrix is private to the library: it
 *     is produced by qwg_repack from canonical GGUF block bytes and has the same
 *     payload bytes (plus < 1 KiB of alignment padding per matrix).
 *   - A model handle is not thread-safe: one caller at a time.
 */
#ifndef QWG_H
#define QWG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------- */
#define QWG_OK 0
#define QWG_E_INVAL (-1)       /* bad pointer, enum value or argument */
#define QWG_E_SHAPE (-2)       /* dimension not supported or not a multiple of the block */
#define QWG_E_NOMEM (-3)       /* arena too small, or host allocation failed */
#define QWG_E_HIP (-4)         /* a HIP runtime call failed (message carries hipGetErrorString) */
#define QWG_E_STATE (-5)       /* call not valid in the model's current state (unbound, ctx full) */
#define QWG_E_UNSUPPORTED (-6) /* qtype or mode not implemented */

/* ---- block formats: GGUF type numbers of the formats in the quantization-format table [HN] -- */
#define QWG_Q4_0 2  /* 32 weights, 18 B: fp16 d, 16 B nibbles; w = d (q - 8) */
#define QWG_Q8_0 8  /* 32 weights, 34 B: fp16 d, 32 int8; w = d q */
#define QWG_Q4_K 12 /* 256 weights, 144 B: fp16 d, dmin, 12 B 6-bit scales/mins, 128 B nibbles; w = d sc q - dmin m */
#define QWG_Q5_K 13 /* 256 weights, 176 B: as Q4_K plus 32 B of fifth bits */
#define QWG_Q6_K 14 /* 256 weights, 210 B: 128 B low nibbles, 64 B 2-bit highs, 16 int8 scales, fp16 d; w = d sc (q - 32) */

/* ---- tensor ids of a Llama decoder ([NT] "Key features": RoPE, GQA, SwiGLU, RMSNorm, KV cache) */
#define QWG_T_EMBED 0
#define QWG_T_HEAD 1
#define QWG_T_WQ 2
#define QWG_T_WK 3
#define QWG_T_WV 4
#define QWG_T_WO 5
#define QWG_T_WGATE 6
#define QWG_T_WUP 7
#define QWG_T_WDOWN 8
#define QWG_NORM_ATTN 9
#define QWG_NORM_FFN 10
#define QWG_NORM_FINAL 11

/* Message of the last failed call on this thread ("" if none). Valid until the next failing call. */
const char* qwg_last_error(void);
/* ABI version of this header (major * 100 + minor). */
int qwg_version(void);

/* ---- sizes of the canonical formats -------------------------------------------------------- */
/* Bytes of one canonical block, weights per block ([HN] quantization-format table); 0 if unknown. */
size_t qwg_block_bytes(int qtype);
int qwg_block_weights(int qtype);
/* Canonical bytes of one row of k weights; 0 if k is not a multiple of the block. */
size_t qwg_row_bytes(int qtype, int64_t k);
/* Device bytes of the packed layout of a rows x k matrix (*out); QWG_E_SHAPE on a bad shape. */
int qwg_packed_bytes(int qtype, int64_t rows, int64_t k, size_t* out);

/* ---- kernel-level entry points (caller-owned device memory, caller's stream) ------------ */

/* Rearrange canonical row-major blocks (d_canon: rows x qwg_row_bytes) into the packed layout
 * (d_packed: qwg_packed_bytes).  Pure byte movement; the buffers must not overlap. */
int qwg_repack(int qtype, const void* d_canon, int64_t rows, int64_t k, void* d_packed, void* stream);

/* Dequantize a packed matrix into fp32 d_out[rows][k].  Each weight is the fp32 nearest to its
 * exact value (fp16 subnormal scales honoured), i.e. bit-identical to a correctly rounded decode. */
int qwg_dequantize(int qtype, const void* d_packed, int64_t rows, int64_t k, float* d_out, void* stream);

/* Fused dequantize-and-GEMV, the engine's hand-written GEMV kernels ([NT] "Architecture overview",
 * cuda/: GEMV; [NT] "Key features": no cuBLAS): d_y[j][r] = sum_c W[r][c] d_x[j][c] for
 * j < n_cols, with W decoded from the packed blocks in registers and never written out.
 * d_x is fp32 [n_cols][k], d_y fp32 [n_cols][rows]; 1 <= n_cols <= 8, or up to 64 for Q4_K, Q5_K
 * and Q6_K with k a multiple of 512; k <= 65536.
 * n_cols > 1 is the multi-column form used to verify self-speculative drafts ([NT] "Key features");
 * 9..64 columns run the prompt-prefill GEMM ([NT] "Quick start": -p), which reads each weight once
 * per call on the matrix cores.  Every form is within |y - y_exact| <= 1e-4 sum|W x| + 1e-6 per
 * output; the products are exact integers (32-bit fixed-point activation digits) except for
 * 9..64 columns of Q4_K / Q5_K, which multiply exact fp16 weights by two-piece fp16 activations
 * with fp32 accumulation.
 * d_work: caller-owned device scratch of at least qwg_gemv_work_bytes(qtype, rows, k, n_cols) bytes
 * (16-byte aligned), which the call overwrites with the activation's digits (or fp16 pieces) and,
 * for shapes whose activation does not fit on chip at once, the K-split partial sums.  Calls in flight
 * at the same time (on one stream or several) need their own d_work; the library allocates nothing
 * and never synchronizes here.  d_packed and d_x 16-byte aligned.  rows == 0 leaves d_y untouched.
 * qwg_gemv_work_bytes returns 0 for shapes the call rejects. */
size_t qwg_gemv_work_bytes(int qtype, int64_t rows, int64_t k, int n_cols);
int qwg_gemv(int qtype, const void* d_packed, int64_t rows, int64_t k, const float* d_x, int n_cols, float* d_y,
             void* d_work, size_t work_bytes, void* stream);

/* qwg_gemv that waits for the GEMV and stores the duration (ms) of its kernel(s) in *h_kernel_ms, from
 * events recorded by the dispatch itself at the kernel's start and end (the activation's digitization
 * before it is not included): the measurement behind the single-GEMV bandwidth figures. */
int qwg_gemv_timed(int qtype, const void* d_packed, int64_t rows, int64_t k, const float* d_x, int n_cols,
                   float* d_y, void* d_work, size_t work_bytes, float* h_kernel_ms, void* stream);

/* qwg_gemv for callers that cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid allocation): the same kernels and results, with the scratch in a static
 * device array of the library instead of a work buffer.  Each GPU the library runs on holds its own
 * QWG_NOALLOC_SCRATCH_BYTES (16 MiB) copy from first use until the process ends; the call allocates
 * and frees nothing.  A shape whose qwg_gemv_work_bytes exceeds that size is refused with QWG_E_NOMEM
 * before anything is launched.  Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap on one GPU (several
 * streams, or several threads) race and may return wrong results; serialize them, or use qwg_gemv
 * with separate work buffers.  Arguments and errors otherwise as qwg_gemv; asynchronous on `stream`
 * (the first call on a device also looks up the array's device address, a host-side call). */
#define QWG_NOALLOC_SCRATCH_BYTES (16u << 20)
int qwg_gemv_noalloc(int qtype, const void* d_packed, int64_t rows, int64_t k, const float* d_x, int n_cols,
                     float* d_y, void* stream);

/* Launch geometry of subsequent GEMV launches in this process, for tuning; 0 keeps the default:
 *   waves_per_group  1..8; up to 16 for single-column GEMVs (above 8: 2 rows per wave, depth 1,
 *                    <= 2 passes);
 *                    for the matrix-core form of 2..8 columns any even number up to 16 (2..4
 *                    columns) or 8 (5..8 columns), the waves of one workgroup
 *   rows_per_wave    output rows per wave of single-column GEMVs: 1, 2 or 4
 *   pipeline_depth   iterations of weight loads in flight: 1 or 2
 *   row_passes       (matrix-core form: waves that split one 16-row tile's K, 1, 2, 4 or 8)
 *                    row blocks per workgroup of single-column residual and SwiGLU GEMVs at depth
 *                    1: 1, 2, 4 or 8 with 2 rows per wave; 2 with 4 rows per wave for Q4_0, Q4_K
 *                    and Q8_0
 * Combinations without a compiled kernel fall back to the nearest one.  Results do not depend on
 * the geometry beyond floating-point summation order.  Not thread-safe: call it while no other
 * thread launches GEMVs. */
int qwg_set_gemv_geometry(int waves_per_group, int rows_per_wave, int pipeline_depth, int row_passes);

/* Form of subsequent 2..8-column GEMVs over Q4_K, Q5_K and Q6_K weights with K a multiple of 512
 * (the multi-column verify step of self-speculative decoding, [NT] "Key features", and chunked
 * prefill): on = 1 (the default) runs them on the matrix
 * cores (v_mfma_i32_16x16x32_i8 over the activation's byte digits), on = 0 on the integer dot
 * products of the one-column kernel.  Both are exact integer products recombined in fp32, within
 * the same row tolerance.  Other formats and column counts always take the integer dot products.
 * Returns QWG_E_INVAL for any other value.  Not thread-safe: call it while no other thread
 * launches GEMVs. */
int qwg_set_gemv_mfma(int on);

/* RMSNorm ([NT] "Key features"; cuda/ RMSNorm kernel): d_out[j][i] = g[i] x[j][i] / sqrt(mean_i x[j]^2 + eps),
 * for j < n_cols; x, out fp32 [n_cols][n]; n <= 65536. */
int qwg_rmsnorm(const float* d_x, const float* d_g, int64_t n, float eps, int n_cols, float* d_out, void* stream);

/* Host: rotary table h_table[p][i] = (cos(p theta_i), sin(p theta_i)) as fp32 pairs, computed in fp64,
 * theta_i = base^(-2i/head_dim), p < max_pos, i < head_dim/2.  h_table holds max_pos*head_dim floats. */
int qwg_rope_table(int max_pos, int head_dim, double base, float* h_table);

/* RoPE ([NT] "Key features"; cuda/ RoPE kernel) in place on d_v [n_heads][head_dim] at position pos:
 * adjacent pairs (2i, 2i+1) rotate by angle pos*theta_i, read from a device copy of the table above
 * (pos must be below that table's max_pos, which the call cannot check).  d_v and d_table 8-byte
 * aligned. */
int qwg_rope(float* d_v, int n_heads, int head_dim, const float* d_table, int pos, void* stream);

/* Grouped-query decode attention over an fp16 KV cache ([NT] "Key features": GQA, KV cache; cuda/ softmax).
 * d_q fp32 [n_cols][n_q][head_dim]; d_kc, d_vc fp16 bits [>= n_pos + n_cols - 1][n_kv][head_dim];
 * column j attends to positions 0 .. n_pos - 1 + j (causal), query head h uses kv head h / (n_q / n_kv);
 * scores q.k / sqrt(head_dim), softmax, weighted sum of V.  d_out fp32 [n_cols][n_q][head_dim].
 * d_work: device scratch of qwg_attn_work_bytes(...) bytes, which the call overwrites (calls that share
 * it must not overlap).  d_q, d_kc and d_vc 16-byte aligned, d_out and d_work 8-byte aligned.
 * head_dim must be 128; n_cols <= 64; n_kv <= 64; n_q / n_kv <= 64; n_pos <= 262144.  With fewer than 32
 * query rows per KV head (n_cols * n_q / n_kv < 32: decode steps, short verify passes) each workgroup
 * takes one (kv head, split, column); from 32 rows (a prompt pass, a verify pass of 4+ columns at
 * n_q / n_kv = 8) the call runs on the matrix cores, 64 / (n_q / n_kv) columns (at most 64 query
 * rows) per workgroup and up to four 64-position tiles per split: K and V as the fp16 values given,
 * queries and softmax weights as two fp16 pieces each (22 significant bits), fp32 sums, within the
 * error of fp32 arithmetic.
 * qwg_attn_work_bytes returns 0 for shapes outside these limits. */
size_t qwg_attn_work_bytes(int n_pos, int n_q, int n_kv, int head_dim, int n_cols);
int qwg_attn_decode(const float* d_q, const uint16_t* d_kc, const uint16_t* d_vc, int n_pos, int n_q, int n_kv,
                    int head_dim, int n_cols, float* d_out, void* d_work, size_t work_bytes, void* stream);

/* SwiGLU ([NT] "Key features"; cuda/ SwiGLU kernel): d_out[i] = silu(g[i]) u[i], silu(z) = z / (1 + e^-z). */
int qwg_swiglu(const float* d_g, const float* d_u, int64_t n, float* d_out, void* stream);

/* Cosine similarity of the layer-skip test ([NT] "Key results"; [UR] layer-skip mechanism):
 * *d_out = <a,b> / (|a| |b|) in fp32 (0 if either vector is zero). */
int qwg_cosine(const float* d_a, const float* d_b, int64_t n, float* d_out, void* stream);

/* Greedy sampler ([NT] "Architecture overview", inference/ sampler): *d_out = index of the largest
 * element of d_x[n] (fp32), lowest index on ties; a NaN ranks above every number (the first NaN wins),
 * so non-finite logits show in the chosen token.  d_work: caller-owned device scratch of
 * qwg_argmax_work_bytes() bytes (8-byte aligned), overwritten; calls in flight at the same time need
 * their own.  Asynchronous on `stream`. */
size_t qwg_argmax_work_bytes(void);
int qwg_argmax(const float* d_x, int64_t n, int32_t* d_out, void* d_work, size_t work_bytes, void* stream);

/* ---- model: a Llama decoder held in HBM, optionally with layers streamed from pinned RAM ---- */

typedef struct qwg_model qwg_model;

typedef struct {
  int32_t n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab;
  int32_t max_ctx;    /* KV cache rows per layer (positions 0 .. max_ctx-1) */
  float rope_theta;   /* RoPE base */
  float rms_eps;      /* RMSNorm epsilon */
  int32_t n_resident; /* layers [0, n_resident) live in HBM; the rest stream from pinned host RAM
                         through two HBM slots ([HN] 3-tier cache: tier A resident, tier B pinned RAM;
                         [UR] SLEP double buffering).  -1 = all resident. */
  int32_t qtype_attn; /* WQ, WK, WV, WO */
  int32_t qtype_ffn;  /* WGATE, WUP, WDOWN */
  int32_t qtype_embed;
  int32_t qtype_head;
  int32_t max_cols;   /* widest multi-column pass, 1..64: self-speculative verify (1 + draft k) takes
                         up to 8; qwg_prefill passes of up to 64 prompt tokens when every layer matrix
                         is Q4_K, Q5_K or Q6_K with K a multiple of 512, else of up to 8 */
  const int32_t* layer_qtypes; /* NULL, or a host array [n_layers][4] of per-layer types of (QKV, WO,
                         GATE|UP, DOWN) overriding qtype_attn / qtype_ffn: mixed-type files such as
                         Q4_K_M ([HN] quantization-format table: a mixed 256-weight type).  Read by
                         qwg_model_create / qwg_plan_residency only (the model keeps a copy).  WQ, WK,
                         WV of a layer share one type (one fused GEMV). */
} qwg_model_desc;

/* Validate the description and create an unbound model (no device memory yet). */
int qwg_model_create(const qwg_model_desc* desc, qwg_model** out);
/* Device bytes the caller must provide to qwg_model_bind (weights of resident layers, two
 * streaming slots if any layer streams, KV caches, activations and scratch). */
size_t qwg_model_arena_bytes(const qwg_model* m);
/* Automatic tier placement ([NT] "3-tier adaptive cache": tier sizes computed from the device's free
 * memory and the host's MemAvailable; [HN] 3-tier cache detail; [UR] 3-tier section): the largest
 * n_resident for which the arena of `desc` (with that n_resident; desc->n_resident is ignored) fits
 * device_budget bytes, with the other layers streamed from pinned host images that must fit
 * host_budget bytes.  device_budget 0 = the current device's free memory (hipMemGetInfo) less a
 * reserve of max(1 GiB, 2% of the device); host_budget 0 = 90% of MemAvailable (/proc/meminfo).
 * Layers 0 .. n_resident-1 are the resident ones, so self-speculative drafts run on them.  Outputs:
 * *n_resident; if not NULL, *arena_bytes (the arena at that placement) and *pinned_bytes (the
 * streamed images).  QWG_E_NOMEM if no placement fits (layers are not placed in the file-backed
 * third tier automatically: see qwg_model_spill_layer).
 * With both budgets given it makes no GPU call. */
int qwg_plan_residency(const qwg_model_desc* desc, size_t device_budget, size_t host_budget, int* n_resident,
                       size_t* arena_bytes, size_t* pinned_bytes);
/* Bind caller-owned device memory (>= qwg_model_arena_bytes, 256-B aligned) and the streams:
 * `compute` runs every kernel, `copy` carries host-to-device layer copies (may equal compute).
 * Streamed layers get library-owned pinned host images here. */
int qwg_model_bind(qwg_model* m, void* d_arena, size_t bytes, void* compute, void* copy);
/* Synchronize and free everything the library owns (never the caller's arena). NULL is a no-op. */
void qwg_model_destroy(qwg_model* m);

/* Load one weight matrix from canonical host bytes (h_canon: rows x qwg_row_bytes).  layer = -1 for
 * EMBED and HEAD.  WQ/WK/WV are stored as one fused matrix and WGATE/WUP with interleaved rows; the
 * caller may free h_canon on return.  qtype must equal the description's type for that tensor. */
int qwg_model_set_tensor(qwg_model* m, int layer, int tensor_id, int qtype, const void* h_canon, size_t nbytes);
/* RMSNorm gains (fp32 [hidden]); which = QWG_NORM_ATTN / QWG_NORM_FFN (layer >= 0) or QWG_NORM_FINAL. */
int qwg_model_set_norm(qwg_model* m, int layer, int which, const float* h_g, int n);
/* Write KV rows 0..n_pos-1 of a layer (fp16 bits [n_pos][n_kv][head_dim], already rotated) and set
 * the number of cached positions of the model to n_pos. */
int qwg_model_set_kv(qwg_model* m, int layer, const uint16_t* h_k, const uint16_t* h_v, int n_pos);
/* Read back KV rows 0..n_pos-1 of a layer (synchronizes). */
int qwg_model_get_kv(qwg_model* m, int layer, uint16_t* h_k, uint16_t* h_v, int n_pos);

/* One greedy decode step ([NT] "Quick start": resident and streaming modes): the token goes at
 * position n_past; every non-skipped layer runs (RMSNorm, fused QKV GEMV with RoPE and KV append,
 * attention, Wo GEMV + residual, RMSNorm, gate|up GEMV with SwiGLU, down GEMV + residual), then the
 * final RMSNorm, head GEMV and argmax.  Streamed layers are double-buffered through two HBM slots,
 * copying layer l+1 while layer l computes ([UR] SLEP streaming pipeline).  n_past advances by one.
 * h_logits (optional) receives the fp32 logits [vocab]. Synchronizes. */
int qwg_decode_step(qwg_model* m, int32_t token, int32_t* next_token, float* h_logits);

/* Prompt prefill ([NT] "Quick start": the -p prompt): tokens[0..n-1] go at positions n_past ..
 * n_past+n-1, each attending causally to the positions before it, as n decode steps would, in passes
 * of up to max_cols columns that read each weight once per pass: passes of 9..64 columns run the
 * prompt-prefill GEMM on the matrix cores (every layer matrix Q4_K, Q5_K or Q6_K with K a multiple of
 * 512; otherwise passes are of at most 8 columns).  Only the last pass runs the final norm, head and
 * argmax, for its last column.  *next_token (optional) is the greedy token after the prompt, h_logits
 * (optional) its fp32 logits [vocab].  n_past advances by n.  Synchronizes. */
int qwg_prefill(qwg_model* m, const int32_t* tokens, int n, int32_t* next_token, float* h_logits);

/* Layer-skip calibration ([NT] "Key results"/"Key features"; [UR] layer-skip mechanism): one decode
 * step with every layer computed that records c_l = cos(h_in, h_out) per layer (h_cos, fp32
 * [n_layers], optional) and sets skip[l] = (c_l >= tau) (h_mask, optional).  Skipped layers then do no
 * work and no copy in later steps and write no KV.  Returns the step's token in *next_token. */
int qwg_calibrate_skip(qwg_model* m, float tau, int32_t token, int32_t* next_token, float* h_cos, uint8_t* h_mask);
int qwg_set_layer_skip(qwg_model* m, int layer, int skip);
int qwg_get_layer_skip(qwg_model* m, uint8_t* h_mask);

/* Self-speculative round ([NT] "Key features"; [HN] speed-up techniques; [NT] "Quick start"
 * --self-spec --draft-k): draft k tokens greedily with layers [0, draft_layers) + final norm + head,
 * verify the k+1 tokens [token, d1..dk] in one k+1-column pass through all layers, accept the longest
 * prefix of drafts that matches the verifier's argmax, emit accepted drafts plus one verifier token
 * (out_tokens[0 .. *n_out-1], *n_out = *n_accepted + 1) and roll the KV length back to
 * n_past + *n_out.  1 <= k, k + 1 <= min(max_cols, 8). */
int qwg_spec_step(qwg_model* m, int32_t token, int draft_layers, int k, int32_t* out_tokens, int* n_out,
                  int* n_accepted);
/* The verify pass alone (1 <= n <= min(max_cols, 8)): tokens[0..n-1] at positions n_past ..
 * n_past+n-1 through all layers;
 * h_logits fp32 [n][vocab] (optional), h_argmax [n] (optional).  n_past is left unchanged (the
 * KV rows written stay beyond it). */
int qwg_verify(qwg_model* m, const int32_t* tokens, int n, float* h_logits, int32_t* h_argmax);

int qwg_model_n_past(const qwg_model* m);
/* Set the number of cached positions (only shrink, or grow up to the rows written). */
int qwg_model_truncate(qwg_model* m, int n_past);
/* Keep the residual stream after every layer of the next steps (for parity checks). */
int qwg_model_set_capture(qwg_model* m, int on);
/* Residual stream captured in the last step: layer = -1 after the embedding, l after layer l;
 * h_out fp32 [hidden] (column 0). Synchronizes. */
int qwg_model_get_hidden(qwg_model* m, int layer, float* h_out);
/* Time the GEMV kernels of one weight class over the next steps with HIP events on the compute
 * stream, recorded by the kernel dispatch itself at the kernel's start and end (tensor_id
 * QWG_T_WQ = fused QKV, WO, WGATE = fused gate|up, WDOWN, HEAD; QWG_TIME_ALL_GEMV = every GEMV of
 * the step, each under its own class; -1 = off).  Clears the accumulated times. */
#define QWG_TIME_ALL_GEMV (-2)
int qwg_model_set_timing(qwg_model* m, int tensor_id);
/* Accumulated time of one class (or of all with QWG_TIME_ALL_GEMV) since qwg_model_set_timing: the
 * sum of the timed kernels' durations (ms), their count and their summed algorithmic bytes (canonical
 * weight bytes plus fp32 activations in and out, per launch). */
int qwg_model_get_timing_class(qwg_model* m, int tensor_id, double* total_ms, int64_t* n_launches,
                               int64_t* total_bytes);
/* The same for the class being timed (all classes if timing is off or QWG_TIME_ALL_GEMV), with the
 * mean algorithmic bytes per launch. */
int qwg_model_get_timing(qwg_model* m, double* total_ms, int64_t* n_launches, int64_t* bytes_per_launch);
/* Bytes copied host-to-device for streamed layers in the last step, and the copy-stream time (ms). */
int qwg_model_stream_stats(qwg_model* m, int64_t* h2d_bytes, double* h2d_ms);

/* Test hooks for failure handling and ordering checks (all off by default):
 *   QWG_DEBUG_SPIN_US       every streamed layer first waits `value` microseconds (0..100000) on the
 *                           compute stream (a bounded one-wave wait kernel), so compute lags the
 *                           copies: a copy that did not wait for "compute on this slot done" would
 *                           overwrite weights still to be read (the double buffer's write-after-read).
 *   QWG_DEBUG_FAIL_AT_LAYER a pass that reaches layer `value` (-1 = off) returns QWG_E_STATE there,
 *                           after the copies of the layers before it and of the next two streamed
 *                           layers were issued, without waiting for them: the state an error leaves.
 *                           n_past does not advance; a later call (or qwg_model_destroy, which
 *                           synchronizes first) is safe. */
#define QWG_DEBUG_SPIN_US 1
#define QWG_DEBUG_FAIL_AT_LAYER 2
int qwg_model_set_debug(qwg_model* m, int knob, int64_t value);
/* The failure check of the captured residual streams (qwg_model_set_capture on, after a step): *layer
 * = the first l in -1 (after the embedding) .. n_layers-1 whose hidden state holds a NaN or an
 * infinity, n_layers if only the logits do, -2 if everything is finite ([NT] "Key features": a
 * non-finite fp16 scale or overflowed cache entry surfaces here with the layer that produced it).
 * Synchronizes. */
int qwg_model_first_nonfinite(qwg_model* m, int* layer);

/* File-backed third tier ([NT] "3-tier adaptive cache": tier C, storage / mmap, used only when the
 * other tiers are full; [HN] 3-tier detail; data path storage -> pinned staging -> H2D -> GPU): move a
 * streamed layer's packed image from its pinned host image to the file `path` (created or
 * truncated, mode 0600), free the pinned image and map the file read-only.  From then on each pass
 * that runs the layer has the host copy the mapped image (page cache or storage) into one of two
 * library-owned pinned staging images, with several threads, before the copy stream moves it into
 * an HBM slot; a staging image is refilled only after the copy out of it is done.  Results are
 * identical to the pinned tier.  The layer must be streamed (not resident) and loaded; its tensors
 * cannot be set again afterwards.  The library unmaps at qwg_model_destroy; the caller removes the
 * file.  Synchronizes. */
int qwg_model_spill_layer(qwg_model* m, int layer, const char* path);
/* Bytes the host read from file-backed images and the milliseconds it spent, since the last call. */
int qwg_model_file_stats(qwg_model* m, int64_t* bytes, double* ms);
int qwg_sync(qwg_model* m);

/* Plain streaming read of `bytes` (a positive multiple of 16; d_src 16-byte aligned) with the
 * GEMV's own 16-byte non-temporal load pattern and no arithmetic: the measured achievable HBM
 * bandwidth, against which the pages' rule that decode speed is bounded by memory bandwidth over
 * the bytes read per token ([UR] benchmark discussion) is checked.  `grid` workgroups of 8 waves
 * (1..8192; 0 = 1024) each read a contiguous share, every lane keeping `unroll` loads in flight (4, 8
 * or 16; 0 = 4).  Writes grid * 8 checksum words to d_sink (device, caller-owned, at least
 * qwg_read_sink_words() words).  Asynchronous on `stream`, unless h_kernel_ms is given: then the
 * call waits for the kernel and stores its duration (ms, from events at the kernel's own start and
 * end) there. */
size_t qwg_read_sink_words(void);
int qwg_read_bytes(const void* d_src, size_t bytes, uint32_t* d_sink, int grid, int unroll, float* h_kernel_ms,
                   void* stream);

/* Pinned host memory (hipHostMalloc) for callers that stage weights. */
int qwg_host_alloc(size_t bytes, void** out);
int qwg_host_free(void* p);

#ifdef __cplusplus
}
#endif

#endif /* QWG_H */
