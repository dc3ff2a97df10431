// qwg_api.hip -- host runtime behind the C ABI of include/qwg.h.
//
// Model placement follows the pages' tiers, re-sized for one MI355X: the NTransformer pages keep
// as many layers as fit in VRAM resident (tier A) and move the rest from pinned host RAM with
// double-buffered copies (tier B; "3-tier adaptive cache" and the SLEP streaming pipeline on the
// Show HN page and the RTX 3090 article).  With 288 GB of HBM a 70B model at these bit widths is
// fully resident, so residency is the primary mode; streaming is kept for layers >= n_resident.
#include <hip/hip_runtime.h>

#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <chrono>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <thread>
#include <cstring>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "../../include/qwg.h"
#include "qwg_kernels.h"

using namespace qwg;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define QWG_HIP(expr)                                                                                \
  do {                                                                                               \
    hipError_t e_ = (expr);                                                                          \
    if (e_ != hipSuccess) return fail(QWG_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// No C++ exception crosses the ABI: every entry point that allocates runs inside guarded().
template <class Fn>
int guarded(Fn&& fn) {
  try {
    return fn();
  } catch (const std::bad_alloc&) {
    return fail(QWG_E_NOMEM, "host allocation failed");
  } catch (const std::exception& ex) {
    return fail(QWG_E_INVAL, std::string("exception: ") + ex.what());
  } catch (...) {
    return fail(QWG_E_INVAL, "unknown exception");
  }
}

int64_t canon_row_bytes(int qt, int64_t k) {
  if (!qtype_known(qt) || k <= 0 || k % block_weights(qt)) return 0;
  return k / block_weights(qt) * block_bytes(qt);
}

size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// ===================================================================================== model

struct MatPlan {
  Layout L;
  size_t off;  // from the layer image base (layer matrices) or the arena base (embed, head)
  int64_t canon_bytes;
};

struct LayerPlan {
  MatPlan qkv, o, gu, down;
  size_t image;       // bytes of the packed layer image (qkv | o | gu | down)
  bool resident;
  size_t arena_off;   // resident image in the arena
  uint8_t* host;      // streamed image in pinned host memory
  const uint8_t* map; // or: file-backed image (read-only mapping of map_len bytes)
  size_t map_len;
  size_t g_attn, g_ffn, kc, vc;
};

struct qwg_model {
  qwg_model_desc d{};
  std::vector<int32_t> lq;  // per-layer types [n_layers][4] of (QKV, WO, GATE|UP, DOWN); empty = class types
  std::vector<LayerPlan> L;
  MatPlan embed{}, head{};
  size_t g_final = 0, rope = 0, h = 0, hin = 0, qb = 0, ob = 0, act = 0, logits = 0, amax = 0, keys = 0, cosv = 0;
  size_t capture = 0, part = 0, attn = 0, slot[2] = {0, 0}, staging = 0, xd[2] = {0, 0}, sq = 0;
  int64_t xd_col = 0;  // bytes of one column of activation digits
  int64_t sq_col = 0;  // floats of one column of per-chunk sums of squares
  size_t part_bytes = 0, attn_bytes = 0, staging_bytes = 0, image_max = 0, total = 0;
  int n_streamed = 0;
  uint8_t* arena = nullptr;
  hipStream_t cs = nullptr, xs = nullptr;
  hipEvent_t ev_full[2] = {}, ev_free[2] = {};
  bool bound = false;
  int n_past = 0;
  std::vector<uint8_t> skip;
  bool capture_on = false;
  // kernel timing of one weight class
  int timing_tensor = -1;  // one class, QWG_TIME_ALL_GEMV, or -1 (off)
  std::vector<hipEvent_t> tev;
  std::vector<int> tev_cls;        // class slot of each event pair
  std::vector<int64_t> tev_bytes;  // algorithmic bytes of each event pair's launch
  int tev_used = 0;
  double t_ms[5] = {};             // per class slot (QKV, WO, GATE|UP, DOWN, HEAD)
  int64_t t_n[5] = {}, t_bytes[5] = {};
  // host-to-device copy timing
  std::vector<hipEvent_t> cev;
  int cev_used = 0;
  int64_t h2d_bytes = 0;
  double h2d_ms = 0.0;
  // file-backed tier: two pinned staging images the host fills from the mappings
  uint8_t* stage[2] = {nullptr, nullptr};
  hipEvent_t ev_staged[2] = {};  // the H2D copy out of stage[i] is done
  int64_t file_bytes = 0;
  double file_ms = 0.0;
  // test hooks (qwg_model_set_debug)
  uint64_t spin_ticks = 0;  // wall-clock ticks each streamed layer waits before its kernels
  int fail_layer = -1;      // a pass reaching this layer fails (after its copies were issued)

  int H() const { return d.hidden; }
  int QR() const { return d.n_q * d.head_dim; }
  int KR() const { return d.n_kv * d.head_dim; }
  float* f(size_t off) const { return (float*)(arena + off); }
};

enum LayerMat : int { LM_QKV = 0, LM_O = 1, LM_GU = 2, LM_DOWN = 3 };

// type of layer l's matrix group `which` (LayerMat) under description d and per-layer table lq
static int layer_qt(const qwg_model_desc& d, const std::vector<int32_t>& lq, int l, int which) {
  if (!lq.empty()) return lq[(size_t)l * 4 + which];
  return which <= LM_O ? d.qtype_attn : d.qtype_ffn;
}

// copy the description (and its per-layer type table) into a model
static void init_desc(qwg_model* m, const qwg_model_desc* desc) {
  m->d = *desc;
  m->d.layer_qtypes = nullptr;
  m->lq.clear();
  if (desc->layer_qtypes) m->lq.assign(desc->layer_qtypes, desc->layer_qtypes + (size_t)desc->n_layers * 4);
}

static MatPlan mat_plan(int qt, int64_t rows, int64_t k, size_t& cursor) {
  MatPlan p;
  p.L = make_layout(qt, rows, k);
  p.off = cursor;
  p.canon_bytes = rows * canon_row_bytes(qt, k);
  cursor = align_up(cursor + (size_t)p.L.total);
  return p;
}

static int plan_model(qwg_model* m) {
  const qwg_model_desc& d = m->d;
  const int H = d.hidden, F = d.ffn, V = d.vocab, C = d.max_cols;
  const int n_res = d.n_resident < 0 ? d.n_layers : d.n_resident;
  size_t cur = 0;
  m->L.assign(d.n_layers, LayerPlan{});
  // each layer's image layout (the same for every layer unless the types mix); streaming slots hold
  // the largest
  m->image_max = 0;
  m->n_streamed = 0;
  for (int l = 0; l < d.n_layers; ++l) {
    LayerPlan& P = m->L[l];
    size_t ic = 0;
    P.qkv = mat_plan(layer_qt(d, m->lq, l, LM_QKV), (int64_t)(d.n_q + 2 * d.n_kv) * d.head_dim, H, ic);
    P.o = mat_plan(layer_qt(d, m->lq, l, LM_O), H, (int64_t)d.n_q * d.head_dim, ic);
    P.gu = mat_plan(layer_qt(d, m->lq, l, LM_GU), 2 * (int64_t)F, H, ic);
    P.down = mat_plan(layer_qt(d, m->lq, l, LM_DOWN), H, F, ic);
    P.image = ic;
    m->image_max = std::max(m->image_max, ic);
    P.resident = l < n_res;
    P.host = nullptr;
    P.map = nullptr;
    P.map_len = 0;
    if (P.resident) {
      P.arena_off = cur;
      cur = align_up(cur + P.image);
    } else {
      ++m->n_streamed;
    }
  }
  m->embed = mat_plan(d.qtype_embed, V, H, cur);
  m->head = mat_plan(d.qtype_head, V, H, cur);
  auto take = [&](size_t bytes) {
    size_t o = cur;
    cur = align_up(cur + bytes);
    return o;
  };
  const size_t kv_bytes = (size_t)d.max_ctx * d.n_kv * d.head_dim * 2;
  for (int l = 0; l < d.n_layers; ++l) {
    m->L[l].g_attn = take((size_t)H * 4);
    m->L[l].g_ffn = take((size_t)H * 4);
    m->L[l].kc = take(kv_bytes);
    m->L[l].vc = take(kv_bytes);
  }
  m->g_final = take((size_t)H * 4);
  m->rope = take((size_t)d.max_ctx * d.head_dim * 4);
  m->h = take((size_t)C * H * 4);
  m->hin = take((size_t)H * 4);
  m->qb = take((size_t)C * m->QR() * 4);
  m->ob = take((size_t)C * m->QR() * 4);
  m->act = take((size_t)C * F * 4);
  m->logits = take((size_t)C * V * 4);
  m->amax = take((size_t)C * 4);
  m->keys = take((size_t)MAX_COLS * 8);
  m->cosv = take((size_t)d.n_layers * 4);
  m->capture = take((size_t)(d.n_layers + 1) * H * 4);
  const int64_t kmax = std::max<int64_t>(std::max<int64_t>(H, F), (int64_t)d.n_q * d.head_dim);
  m->xd_col = digit_bytes(kmax);
  m->xd[0] = take((size_t)C * m->xd_col);
  m->xd[1] = take((size_t)C * m->xd_col);
  m->sq_col = kmax / XCHUNK;
  m->sq = take((size_t)C * m->sq_col * 4);
  size_t pb = 0;
  for (int nc : {1, C}) {
    const int64_t shapes[5][2] = {{(int64_t)(d.n_q + 2 * d.n_kv) * d.head_dim, H},
                                  {H, (int64_t)d.n_q * d.head_dim},
                                  {2 * (int64_t)F, H},
                                  {H, F},
                                  {V, H}};
    for (int i = 0; i < 5; ++i)
      for (int l = 0; l < (i < 4 ? d.n_layers : 1); ++l) {
      const int qt = i < 4 ? layer_qt(d, m->lq, l, i) : d.qtype_head;
      if (i < 4 && l > 0 && qt == layer_qt(d, m->lq, l - 1, i)) continue;
      for (int mf : {0, 1}) {  // either form of a several-column GEMV may run (qwg_set_gemv_mfma)
        const GemvPlan gp = plan_gemv(qt, shapes[i][0], shapes[i][1], nc, EPI_STORE, mf);
        pb = std::max(pb, gp.part_bytes);
      }
    }
  }
  m->part_bytes = pb;
  m->part = take(pb > 0 ? pb : 256);
  m->attn_bytes = attn_work_bound(d.max_ctx, d.n_q, d.n_kv, C);
  m->attn = take(m->attn_bytes);
  if (m->n_streamed > 0) {
    m->slot[0] = take(m->image_max);
    m->slot[1] = take(m->image_max);
  }
  m->staging_bytes = 64u << 20;
  m->staging = take(m->staging_bytes);
  m->total = cur;
  return QWG_OK;
}

static int check_desc(const qwg_model_desc* d) {
  if (!d) return fail(QWG_E_INVAL, "desc is NULL");
  if (d->n_layers < 1 || d->hidden < 1 || d->n_q < 1 || d->n_kv < 1 || d->ffn < 1 || d->vocab < 1 || d->max_ctx < 1)
    return fail(QWG_E_SHAPE, "model dimensions must be positive");
  if (d->head_dim != HEAD_DIM) return fail(QWG_E_SHAPE, "head_dim must be 128");
  if (d->n_q % d->n_kv) return fail(QWG_E_SHAPE, "n_q must be a multiple of n_kv");
  if (d->max_cols < 1 || d->max_cols > MAX_PREFILL_COLS) return fail(QWG_E_SHAPE, "max_cols must be in 1..64");
  if (d->n_q / d->n_kv * std::min(d->max_cols, MAX_COLS) > 64)
    return fail(QWG_E_SHAPE, "(n_q / n_kv) * min(max_cols, 8) must be <= 64");
  const int qts[4] = {d->qtype_attn, d->qtype_ffn, d->qtype_embed, d->qtype_head};
  for (int q : qts)
    if (!qtype_known(q)) return fail(QWG_E_UNSUPPORTED, "unknown qtype " + std::to_string(q));
  const int64_t H = d->hidden, F = d->ffn, QR = (int64_t)d->n_q * d->head_dim;
  if (canon_row_bytes(d->qtype_attn, H) == 0 || canon_row_bytes(d->qtype_attn, QR) == 0 ||
      canon_row_bytes(d->qtype_ffn, H) == 0 || canon_row_bytes(d->qtype_ffn, F) == 0 ||
      canon_row_bytes(d->qtype_embed, H) == 0 || canon_row_bytes(d->qtype_head, H) == 0)
    return fail(QWG_E_SHAPE, "hidden, ffn and n_q*head_dim must be multiples of the block size");
  if (H > 65536 || F > 65536 || QR > 65536) return fail(QWG_E_SHAPE, "K dimensions above 65536 are not supported");
  if (d->n_resident < -1 || d->n_resident > d->n_layers) return fail(QWG_E_SHAPE, "bad n_resident");
  if (d->n_kv > 64) return fail(QWG_E_SHAPE, "n_kv above 64 is not supported");
  if (d->max_ctx > 131072) return fail(QWG_E_SHAPE, "max_ctx above 131072 is not supported");
  const int64_t shapes[6][3] = {{d->qtype_attn, (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim, H},
                                {d->qtype_attn, H, QR},
                                {d->qtype_ffn, 2 * F, H},
                                {d->qtype_ffn, H, F},
                                {d->qtype_embed, d->vocab, H},
                                {d->qtype_head, d->vocab, H}};
  for (const auto& sh : shapes)
    if (make_layout((int)sh[0], sh[1], sh[2]).total >= ((int64_t)1 << 32))
      return fail(QWG_E_SHAPE, "a packed matrix of 4 GiB or more is not supported");
  if (d->layer_qtypes) {
    const int64_t ks[4] = {H, QR, H, F};
    const int64_t rs[4] = {(int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim, H, 2 * F, H};
    for (int l = 0; l < d->n_layers; ++l)
      for (int i = 0; i < 4; ++i) {
        const int q = d->layer_qtypes[(size_t)l * 4 + i];
        if (!qtype_known(q)) return fail(QWG_E_UNSUPPORTED, "unknown layer qtype " + std::to_string(q));
        if (canon_row_bytes(q, ks[i]) == 0) return fail(QWG_E_SHAPE, "layer matrix K is not a multiple of its block");
        if (make_layout(q, rs[i], ks[i]).total >= ((int64_t)1 << 32))
          return fail(QWG_E_SHAPE, "a packed matrix of 4 GiB or more is not supported");
      }
  }
  return QWG_OK;
}

static MatView view_at(const uint8_t* base, const MatPlan& p) { return make_view(base + p.off, p.L); }

// ---------------------------------------------------------------------------- timing helpers

// flags 0: default events; the kernel-timing events are created without the system-scope fence
// (their times are read only after the stream has been synchronized), so recording them does not
// write back and invalidate the caches around the kernels they time
static hipEvent_t pool_event(std::vector<hipEvent_t>& pool, int& used, unsigned flags = 0) {
  if (used == (int)pool.size()) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, flags) != hipSuccess) return nullptr;
    pool.push_back(e);
  }
  return pool[used++];
}

// slot of a timing class (the tensor ids of the five GEMV launches of a step), or -1
static int timing_slot(int tensor_id) {
  switch (tensor_id) {
    case QWG_T_WQ: return 0;
    case QWG_T_WO: return 1;
    case QWG_T_WGATE: return 2;
    case QWG_T_WDOWN: return 3;
    case QWG_T_HEAD: return 4;
    default: return -1;
  }
}

static int collect_timing(qwg_model* m) {
  for (int i = 0; i + 1 < m->tev_used; i += 2) {
    float ms = 0.f;
    QWG_HIP(hipEventElapsedTime(&ms, m->tev[i], m->tev[i + 1]));
    const int c = m->tev_cls[i / 2];
    m->t_ms[c] += ms;
    m->t_n[c] += 1;
    m->t_bytes[c] += m->tev_bytes[i / 2];
  }
  m->tev_used = 0;
  for (int i = 0; i + 1 < m->cev_used; i += 2) {
    float ms = 0.f;
    QWG_HIP(hipEventElapsedTime(&ms, m->cev[i], m->cev[i + 1]));
    m->h2d_ms += ms;
  }
  m->cev_used = 0;
  return QWG_OK;
}

// ---------------------------------------------------------------------------- one pass

static int64_t gemv_alg_bytes(const MatPlan& p, int nc, int out_rw) {
  return p.canon_bytes + (int64_t)nc * p.L.k * 4 + (int64_t)nc * p.L.rows * 4 * out_rw;
}

// Where a GEMV's output vector goes next: digits for the next GEMV (of gain * out when a gain is
// given, with per-chunk sums of out^2 when sq is given).
struct OutDigits {
  int buf = -1;  // digit buffer index, or -1 (no digits)
  const float* gain = nullptr;
  int qt = 0;    // the consuming GEMV's qtype (picks nibble or byte digits)
  bool sq = false;
};

// The input of a GEMV: the digits in buffer `buf` (with the RMSNorm folded in when rms is set), or
// an fp32 vector xf that the GEMV digitizes itself (through buffer `buf` and a separate
// digitization kernel when the launch geometry has no such variant).
struct InDigits {
  int buf = 0;
  bool rms = false;
  const float* xf = nullptr;
  int64_t xf_stride = 0;
};

// Run one GEMV; its epilogue also digitizes the output per `od` when the launch geometry allows
// it, else a separate digitization kernel follows.  With timing on for this weight class, HIP
// events on the compute stream bracket the GEMV kernel(s).
static int gemv(qwg_model* m, int tensor_class, int qt, const MatView& w, const MatPlan& mp, const InDigits& in, int nc,
                int epi, EpiArgs e, const OutDigits& od) {
  const GemvPlan gp = plan_gemv(qt, w.rows, mp.L.k, nc, epi);
  if (gp.part_bytes > m->part_bytes) return fail(QWG_E_NOMEM, "split workspace too small");
  const bool rms = in.rms;
  if (in.xf) {
    if (gemv_can_digitize_input(gp, epi)) {
      e.xf = in.xf;
      e.xf_stride = in.xf_stride;
    } else {
      QWG_HIP(launch_digitize(in.xf, in.xf_stride, nullptr, mp.L.k, nc, qt, m->arena + m->xd[in.buf], m->xd_col,
                              nullptr, 0, m->cs));
    }
  }
  if (rms) {
    e.sq_in = m->f(m->sq);
    e.sq_in_n = (int)(mp.L.k / XCHUNK);
    e.sq_in_stride = m->sq_col;
    e.rms_k = (float)mp.L.k;
    e.eps = m->d.rms_eps;
  }
  const bool want = od.buf >= 0;
  const int okind = want ? gemv_digit_kind(od.qt, epi == EPI_SWIGLU ? w.rows / 2 : w.rows, nc) : -1;
  const bool fused = want && gemv_can_digitize_output(gp, epi, w.rows, okind);
  if (fused) {
    e.dig_out = (uint32_t*)(m->arena + m->xd[od.buf]);
    e.dig_stride = m->xd_col / 4;
    e.dig_gain = od.gain;
    e.dig_kind = okind;
    e.sq_out = od.sq ? m->f(m->sq) : nullptr;
    e.sq_out_stride = m->sq_col;
  }
  const bool timed = m->timing_tensor == tensor_class || m->timing_tensor == QWG_TIME_ALL_GEMV;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timed) {
    e0 = pool_event(m->tev, m->tev_used, hipEventDisableSystemFence);
    e1 = pool_event(m->tev, m->tev_used, hipEventDisableSystemFence);
    if (!e0 || !e1) return fail(QWG_E_HIP, "hipEventCreate failed");
    const size_t pair = (size_t)(m->tev_used / 2 - 1);
    if (m->tev_cls.size() <= pair) {
      m->tev_cls.resize(pair + 1);
      m->tev_bytes.resize(pair + 1);
    }
    const int rw = epi == EPI_RESID ? 2 : 1;
    m->tev_cls[pair] = timing_slot(tensor_class);
    m->tev_bytes[pair] = gemv_alg_bytes(mp, nc, epi == EPI_SWIGLU ? 0 : rw) +
                         (epi == EPI_SWIGLU ? (int64_t)nc * mp.L.rows / 2 * 4 : 0);
  }
  QWG_HIP(launch_gemv(qt, w, mp.L.k, m->arena + m->xd[in.buf], m->xd_col, nc, epi, e, m->f(m->part), m->cs, gp, e0,
                      e1));
  if (want && !fused) {
    const int64_t nout = epi == EPI_SWIGLU ? w.rows / 2 : w.rows;
    QWG_HIP(launch_digitize(e.y, e.y_stride, od.gain, nout, nc, od.qt, m->arena + m->xd[od.buf], m->xd_col,
                            od.sq ? m->f(m->sq) : nullptr, m->sq_col, m->cs));
  }
  return QWG_OK;
}

// One decoder layer.  Digit buffer 0 holds g_attn * h on entry (with the sums of squares of h);
// on exit it holds the digits that `next` describes (the next layer's g_attn * h, or g_final * h).
static int layer_kernels(qwg_model* m, int l, const uint8_t* base, int nc, int pos, const OutDigits& next) {
  const qwg_model_desc& d = m->d;
  const LayerPlan& P = m->L[l];
  const int H = d.hidden, F = d.ffn, QR = m->QR(), KR = m->KR();
  int rc;
  EpiArgs e{};
  e.y = m->f(m->qb);
  e.y_stride = QR;
  e.rope = m->f(m->rope);
  e.pos = pos;
  e.nq_rows = QR;
  e.nkv_rows = KR;
  e.kc = (uint16_t*)(m->arena + P.kc);
  e.vc = (uint16_t*)(m->arena + P.vc);
  e.kv_stride = KR;
  InDigits in_qkv;
  in_qkv.buf = 0;
  in_qkv.rms = true;
  const int qt_qkv = P.qkv.L.qtype, qt_o = P.o.L.qtype, qt_gu = P.gu.L.qtype, qt_down = P.down.L.qtype;
  if ((rc = gemv(m, QWG_T_WQ, qt_qkv, view_at(base, P.qkv), P.qkv, in_qkv, nc, EPI_QKV, e, OutDigits{})))
    return rc;
  const AttnPlan ap = plan_attn(pos + 1, d.n_q, d.n_kv, nc);
  if (ap.work_bytes > m->attn_bytes) return fail(QWG_E_NOMEM, "attention workspace too small");
  // the merge writes Wo's input digits itself, except fp16 pieces (their scale spans a superblock,
  // two heads), which are digitized from its fp32 output
  const int dk_o = gemv_digit_kind(qt_o, QR, nc);
  QWG_HIP(launch_attn(m->f(m->qb), QR, e.kc, e.vc, KR, pos + 1, d.n_q, d.n_kv, nc, m->f(m->ob), QR,
                      m->arena + m->attn, ap, m->cs,
                      dk_o == DIG_F16 ? nullptr : (uint32_t*)(m->arena + m->xd[1]), m->xd_col / 4, dk_o));
  if (dk_o == DIG_F16)
    QWG_HIP(launch_digitize(m->f(m->ob), QR, nullptr, QR, nc, qt_o, m->arena + m->xd[1], m->xd_col, nullptr, 0,
                            m->cs));
  EpiArgs r{};
  r.y = m->f(m->h);
  r.y_stride = H;
  OutDigits to_ffn;
  to_ffn.buf = 0;
  to_ffn.gain = m->f(P.g_ffn);
  to_ffn.qt = qt_gu;
  to_ffn.sq = true;
  InDigits in_o;
  in_o.buf = 1;
  if ((rc = gemv(m, QWG_T_WO, qt_o, view_at(base, P.o), P.o, in_o, nc, EPI_RESID, r, to_ffn))) return rc;
  EpiArgs s{};
  s.y = m->f(m->act);
  s.y_stride = F;
  InDigits in_ffn;
  in_ffn.buf = 0;
  in_ffn.rms = true;
  // silu(gate) * up reaches the down GEMV as digits written by the gate|up epilogue when its launch
  // geometry covers whole 32-output chunks, else the down GEMV digitizes the fp32 vector itself
  const int64_t gu_rows = P.gu.L.rows;
  const bool act_digits = gemv_can_digitize_output(plan_gemv(qt_gu, gu_rows, H, nc, EPI_SWIGLU), EPI_SWIGLU, gu_rows,
                                                   gemv_digit_kind(qt_down, gu_rows / 2, nc));
  OutDigits to_down;
  if (act_digits) {
    to_down.buf = 1;
    to_down.qt = qt_down;
  }
  if ((rc = gemv(m, QWG_T_WGATE, qt_gu, view_at(base, P.gu), P.gu, in_ffn, nc, EPI_SWIGLU, s, to_down)))
    return rc;
  InDigits in_act;
  in_act.buf = 1;
  if (!act_digits) {
    in_act.xf = m->f(m->act);
    in_act.xf_stride = F;
  }
  if ((rc = gemv(m, QWG_T_WDOWN, qt_down, view_at(base, P.down), P.down, in_act, nc, EPI_RESID, r, next)))
    return rc;
  return QWG_OK;
}

// Host copy of n bytes by several threads (the file-backed tier's read into pinned staging).
static void parallel_copy(uint8_t* dst, const uint8_t* src, size_t n) {
  const int T = (int)std::max(1u, std::min(8u, std::thread::hardware_concurrency()));
  const size_t part = (n / T + 4095) & ~(size_t)4095;
  std::vector<std::thread> th;
  for (int t = 1; t < T; ++t) {
    const size_t b = (size_t)t * part;
    if (b >= n) break;
    th.emplace_back([=] { std::memcpy(dst + b, src + b, std::min(part, n - b)); });
  }
  std::memcpy(dst, src, std::min(part, n));
  for (auto& x : th) x.join();
}

static int issue_copy(qwg_model* m, const std::vector<int>& sl, int j) {
  const int slot = j & 1;
  const LayerPlan& P = m->L[sl[j]];
  const uint8_t* src = P.host;
  if (P.map) {
    // file-backed: the host reads the image into staging image `slot` once the copy that last read
    // it (two streamed layers ago) is done, then the copy stream moves it to the HBM slot
    QWG_HIP(hipEventSynchronize(m->ev_staged[slot]));
    const auto t0 = std::chrono::steady_clock::now();
    parallel_copy(m->stage[slot], P.map, P.image);
    m->file_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    m->file_bytes += (int64_t)P.image;
    src = m->stage[slot];
  }
  QWG_HIP(hipStreamWaitEvent(m->xs, m->ev_free[slot], 0));
  hipEvent_t c0 = pool_event(m->cev, m->cev_used);
  hipEvent_t c1 = pool_event(m->cev, m->cev_used);
  if (!c0 || !c1) return fail(QWG_E_HIP, "hipEventCreate failed");
  QWG_HIP(hipEventRecord(c0, m->xs));
  QWG_HIP(hipMemcpyAsync(m->arena + m->slot[slot], src, P.image, hipMemcpyHostToDevice, m->xs));
  if (P.map) QWG_HIP(hipEventRecord(m->ev_staged[slot], m->xs));
  QWG_HIP(hipEventRecord(c1, m->xs));
  QWG_HIP(hipEventRecord(m->ev_full[slot], m->xs));
  m->h2d_bytes += (int64_t)P.image;
  return QWG_OK;
}

// Embedding, layers [0, n_run) (skipped layers bypassed unless calibrating), then (with head) final
// norm, head, argmax.
static int run_pass(qwg_model* m, const int32_t* toks, int nc, int pos, int n_run, bool calib, bool head = true) {
  const qwg_model_desc& d = m->d;
  const int H = d.hidden;
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  if (nc < 1 || nc > d.max_cols) return fail(QWG_E_SHAPE, "column count outside 1..max_cols");
  if (pos < 0 || pos + nc > d.max_ctx) return fail(QWG_E_STATE, "context full (n_past + columns > max_ctx)");
  for (int i = 0; i < nc; ++i)
    if (toks[i] < 0 || toks[i] >= d.vocab) return fail(QWG_E_INVAL, "token id out of range");
  QWG_HIP(launch_embed(d.qtype_embed, view_at(m->arena, m->embed), H, toks, nc, m->f(m->h), H, m->cs));
  // the digits every layer leaves behind are for the next layer that runs (its g_attn), or for the
  // head (g_final) after the last one
  std::vector<int> runs;
  for (int l = 0; l < n_run; ++l)
    if (calib || !m->skip[l]) runs.push_back(l);
  auto digits_for = [&](int ri) {
    OutDigits od;
    od.buf = 0;
    od.sq = true;
    if (ri < (int)runs.size()) {
      od.gain = m->f(m->L[runs[ri]].g_attn);
      od.qt = m->L[runs[ri]].qkv.L.qtype;
    } else {
      od.gain = m->f(m->g_final);
      od.qt = d.qtype_head;
    }
    return od;
  };
  {
    const OutDigits od = digits_for(0);
    QWG_HIP(launch_digitize(m->f(m->h), H, od.gain, H, nc, od.qt, m->arena + m->xd[0], m->xd_col, m->f(m->sq),
                            m->sq_col, m->cs));
  }
  int ri = 0;
  if (m->capture_on) QWG_HIP(hipMemcpyAsync(m->f(m->capture), m->f(m->h), (size_t)H * 4, hipMemcpyDeviceToDevice, m->cs));
  std::vector<int> sl;
  for (int l = 0; l < n_run; ++l)
    if (!m->L[l].resident && (calib || !m->skip[l])) sl.push_back(l);
  for (int j = 0; j < (int)sl.size() && j < 2; ++j)
    if (int rc = issue_copy(m, sl, j)) return rc;
  int sj = 0;
  for (int l = 0; l < n_run; ++l) {
    const bool run = calib || !m->skip[l];
    if (run) {
      const LayerPlan& P = m->L[l];
      const uint8_t* base;
      int slot = 0;
      if (P.resident) {
        base = m->arena + P.arena_off;
      } else {
        slot = sj & 1;
        QWG_HIP(hipStreamWaitEvent(m->cs, m->ev_full[slot], 0));
        base = m->arena + m->slot[slot];
      }
      if (l == m->fail_layer) return fail(QWG_E_STATE, "forced failure at layer " + std::to_string(l));
      if (!P.resident && m->spin_ticks) QWG_HIP(launch_spin(m->spin_ticks, m->cs));
      if (calib) QWG_HIP(hipMemcpyAsync(m->f(m->hin), m->f(m->h), (size_t)H * 4, hipMemcpyDeviceToDevice, m->cs));
      if (int rc = layer_kernels(m, l, base, nc, pos, digits_for(++ri))) return rc;
      if (!P.resident) {
        QWG_HIP(hipEventRecord(m->ev_free[slot], m->cs));
        if (sj + 2 < (int)sl.size())
          if (int rc = issue_copy(m, sl, sj + 2)) return rc;
        ++sj;
      }
      if (calib) QWG_HIP(launch_cosine(m->f(m->hin), m->f(m->h), H, m->f(m->cosv) + l, m->cs));
    }
    if (m->capture_on)
      QWG_HIP(hipMemcpyAsync(m->f(m->capture) + (size_t)(l + 1) * H, m->f(m->h), (size_t)H * 4,
                             hipMemcpyDeviceToDevice, m->cs));
  }
  for (int l = n_run; l < d.n_layers && m->capture_on; ++l)
    QWG_HIP(hipMemcpyAsync(m->f(m->capture) + (size_t)(l + 1) * H, m->f(m->h), (size_t)H * 4,
                           hipMemcpyDeviceToDevice, m->cs));
  if (!head) return QWG_OK;
  // a wide prefill pass needs only its last column's logits: that column is digitized again for the
  // one-column head GEMV (whose digit kind may differ from the wide GEMMs' byte digits)
  int hc = nc;
  if (nc > MAX_COLS) {
    hc = 1;
    QWG_HIP(launch_digitize(m->f(m->h) + (size_t)(nc - 1) * H, H, m->f(m->g_final), H, 1, d.qtype_head,
                            m->arena + m->xd[0], m->xd_col, m->f(m->sq), m->sq_col, m->cs));
  }
  EpiArgs e{};
  e.y = m->f(m->logits);
  e.y_stride = d.vocab;
  InDigits in_head;
  in_head.buf = 0;
  in_head.rms = true;
  if (int rc = gemv(m, QWG_T_HEAD, d.qtype_head, view_at(m->arena, m->head), m->head, in_head, hc, EPI_STORE, e,
                    OutDigits{}))
    return rc;
  QWG_HIP(launch_argmax(m->f(m->logits), d.vocab, hc, d.vocab, (int32_t*)(m->arena + m->amax), m->cs,
                        (unsigned long long*)(m->arena + m->keys)));
  return QWG_OK;
}

// Widest pass the 64-column GEMM can take for this model: every layer matrix a K-quant with K a
// multiple of 512 (else the multi-column kernels, up to MAX_COLS).
static int prefill_width(const qwg_model* m) {
  const int C = m->d.max_cols;
  if (C <= MAX_COLS) return C;
  for (const LayerPlan& P : m->L)
    for (const MatPlan* mp : {&P.qkv, &P.o, &P.gu, &P.down}) {
      const int qt = mp->L.qtype;
      if (!(qt == Q4_K || qt == Q5_K || qt == Q6_K) || mp->L.k % 512) return MAX_COLS;
    }
  return C;
}

static int finish_pass(qwg_model* m, int nc, int32_t* h_amax, float* h_logits) {
  QWG_HIP(hipStreamSynchronize(m->cs));
  QWG_HIP(hipStreamSynchronize(m->xs));
  if (h_amax) QWG_HIP(hipMemcpy(h_amax, m->arena + m->amax, (size_t)nc * 4, hipMemcpyDeviceToHost));
  if (h_logits)
    QWG_HIP(hipMemcpy(h_logits, m->f(m->logits), (size_t)nc * m->d.vocab * 4, hipMemcpyDeviceToHost));
  return collect_timing(m);
}

// ===================================================================================== C ABI

extern "C" {

const char* qwg_last_error(void) { return g_err.c_str(); }
int qwg_version(void) { return 100; }

size_t qwg_block_bytes(int qtype) { return qtype_known(qtype) ? (size_t)block_bytes(qtype) : 0; }
int qwg_block_weights(int qtype) { return qtype_known(qtype) ? block_weights(qtype) : 0; }
size_t qwg_row_bytes(int qtype, int64_t k) { return (size_t)canon_row_bytes(qtype, k); }

int qwg_packed_bytes(int qtype, int64_t rows, int64_t k, size_t* out) {
  if (!out) return fail(QWG_E_INVAL, "out is NULL");
  if (!qtype_known(qtype)) return fail(QWG_E_UNSUPPORTED, "unknown qtype");
  if (rows < 0 || canon_row_bytes(qtype, k) == 0) return fail(QWG_E_SHAPE, "k must be a positive multiple of the block");
  *out = (size_t)make_layout(qtype, rows, k).total;
  return QWG_OK;
}

static int check_matrix(int qtype, int64_t rows, int64_t k) {
  if (!qtype_known(qtype)) return fail(QWG_E_UNSUPPORTED, "unknown qtype " + std::to_string(qtype));
  if (rows < 0 || rows > (int64_t)1 << 30) return fail(QWG_E_SHAPE, "rows out of range");
  if (canon_row_bytes(qtype, k) == 0) return fail(QWG_E_SHAPE, "k must be a positive multiple of the block");
  if (k > 65536) return fail(QWG_E_SHAPE, "k above 65536");
  if (make_layout(qtype, rows, k).total >= ((int64_t)1 << 32)) return fail(QWG_E_SHAPE, "packed matrix of 4 GiB or more");
  return QWG_OK;
}

int qwg_repack(int qtype, const void* d_canon, int64_t rows, int64_t k, void* d_packed, void* stream) {
  if (int rc = check_matrix(qtype, rows, k)) return rc;
  if ((!d_canon || !d_packed) && rows > 0) return fail(QWG_E_INVAL, "NULL pointer");
  const Layout L = make_layout(qtype, rows, k);
  QWG_HIP(launch_repack(qtype, (const uint8_t*)d_canon, rows, k, (uint8_t*)d_packed, L, 0, 1, (hipStream_t)stream));
  return QWG_OK;
}

int qwg_dequantize(int qtype, const void* d_packed, int64_t rows, int64_t k, float* d_out, void* stream) {
  if (int rc = check_matrix(qtype, rows, k)) return rc;
  if ((!d_packed || !d_out) && rows > 0) return fail(QWG_E_INVAL, "NULL pointer");
  if (!aligned16(d_packed) || !aligned16(d_out)) return fail(QWG_E_INVAL, "pointers must be 16-byte aligned");
  const Layout L = make_layout(qtype, rows, k);
  QWG_HIP(launch_dequant(qtype, make_view(d_packed, L), rows, k, d_out, (hipStream_t)stream));
  return QWG_OK;
}

// Scratch of one qwg_gemv call: the activation digits of every column, then (256-B aligned) the
// K-split partial sums of whichever form a several-column GEMV may take.
// Widest column count qwg_gemv takes: 64 for K-quants with K a multiple of 512 (the prefill GEMM),
// else 8.
static int gemv_max_cols(int qtype, int64_t k) {
  return ((qtype == Q4_K || qtype == Q5_K || qtype == Q6_K) && k % 512 == 0) ? MAX_PREFILL_COLS : MAX_COLS;
}

static bool gemv_work_layout(int qtype, int64_t rows, int64_t k, int n_cols, size_t* dig_bytes, size_t* total) {
  if (!qtype_known(qtype) || rows < 0 || rows > (int64_t)1 << 30 || canon_row_bytes(qtype, k) == 0 || k > 65536 ||
      n_cols < 1 || n_cols > gemv_max_cols(qtype, k))
    return false;
  const size_t dig = align_up((size_t)n_cols * (size_t)digit_bytes(k));
  size_t part = 0;
  for (int mf : {0, 1}) part = std::max(part, plan_gemv(qtype, rows, k, n_cols, EPI_STORE, mf).part_bytes);
  *dig_bytes = dig;
  *total = dig + align_up(part);
  return true;
}

size_t qwg_gemv_work_bytes(int qtype, int64_t rows, int64_t k, int n_cols) {
  size_t dig = 0, total = 0;
  return gemv_work_layout(qtype, rows, k, n_cols, &dig, &total) ? total : 0;
}

// One GEMV through caller-provided (or static) scratch `work` of `work_bytes`; with events, they are
// recorded at the start and end of the GEMV kernel(s) (not the digitization before them).
static int gemv_run(int qtype, const void* d_packed, int64_t rows, int64_t k, const float* d_x, int n_cols,
                    float* d_y, void* work, size_t work_bytes, hipStream_t stream, hipEvent_t ev0 = nullptr,
                    hipEvent_t ev1 = nullptr) {
  size_t dig = 0, need = 0;
  gemv_work_layout(qtype, rows, k, n_cols, &dig, &need);
  if (work_bytes < need) return fail(QWG_E_NOMEM, "work buffer smaller than qwg_gemv_work_bytes");
  const Layout L = make_layout(qtype, rows, k);
  const GemvPlan p = plan_gemv(qtype, rows, k, n_cols, EPI_STORE);
  uint8_t* xd = (uint8_t*)work;
  float* part = p.part_bytes ? (float*)(xd + dig) : nullptr;
  QWG_HIP(launch_digitize(d_x, k, nullptr, k, n_cols, qtype, xd, digit_bytes(k), nullptr, 0, stream));
  EpiArgs e{};
  e.y = d_y;
  e.y_stride = rows;
  QWG_HIP(launch_gemv(qtype, make_view(d_packed, L), k, xd, digit_bytes(k), n_cols, EPI_STORE, e, part, stream, p,
                      ev0, ev1));
  return QWG_OK;
}

int qwg_gemv_timed(int qtype, const void* d_packed, int64_t rows, int64_t k, const float* d_x, int n_cols,
                   float* d_y, void* d_work, size_t work_bytes, float* h_kernel_ms, void* stream) {
  if (!h_kernel_ms) return fail(QWG_E_INVAL, "NULL pointer");
  if (int rc = check_matrix(qtype, rows, k)) return rc;
  if (n_cols < 1 || n_cols > gemv_max_cols(qtype, k))
    return fail(QWG_E_SHAPE, "n_cols must be in 1..8 (1..64 for Q4_K, Q5_K, Q6_K with k a multiple of 512)");
  if (rows == 0) return fail(QWG_E_SHAPE, "rows must be positive to time a GEMV");
  if (!d_packed || !d_x || !d_y || !d_work) return fail(QWG_E_INVAL, "NULL pointer");
  if (!aligned16(d_packed) || !aligned16(d_x) || !aligned16(d_work))
    return fail(QWG_E_INVAL, "d_packed, d_x and d_work must be 16-byte aligned");
  hipEvent_t e[2] = {nullptr, nullptr};
  for (auto& x : e) QWG_HIP(hipEventCreateWithFlags(&x, hipEventDisableSystemFence));
  int rc = gemv_run(qtype, d_packed, rows, k, d_x, n_cols, d_y, d_work, work_bytes, (hipStream_t)stream, e[0], e[1]);
  hipError_t err = hipSuccess;
  if (rc == QWG_OK) err = hipEventSynchronize(e[1]);
  if (rc == QWG_OK && err == hipSuccess) err = hipEventElapsedTime(h_kernel_ms, e[0], e[1]);
  for (auto x : e) (void)hipEventDestroy(x);
  if (rc != QWG_OK) return rc;
  if (err != hipSuccess) return fail(QWG_E_HIP, std::string("timed GEMV: ") + hipGetErrorString(err));
  return QWG_OK;
}

int qwg_gemv(int qtype, const void* d_packed, int64_t rows, int64_t k, const float* d_x, int n_cols, float* d_y,
             void* d_work, size_t work_bytes, void* stream) {
  if (int rc = check_matrix(qtype, rows, k)) return rc;
  if (n_cols < 1 || n_cols > gemv_max_cols(qtype, k))
    return fail(QWG_E_SHAPE, "n_cols must be in 1..8 (1..64 for Q4_K, Q5_K, Q6_K with k a multiple of 512)");
  if (rows == 0) return QWG_OK;
  if (!d_packed || !d_x || !d_y || !d_work) return fail(QWG_E_INVAL, "NULL pointer");
  if (!aligned16(d_packed) || !aligned16(d_x) || !aligned16(d_work))
    return fail(QWG_E_INVAL, "d_packed, d_x and d_work must be 16-byte aligned");
  return gemv_run(qtype, d_packed, rows, k, d_x, n_cols, d_y, d_work, work_bytes, (hipStream_t)stream);
}

// ---- the allocation-free GEMV: scratch in a static device array, one copy per GPU.  Host code never
// uses the array's name as an address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[QWG_NOALLOC_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64] = {};

static int scratch_of_current_device(void** out) {
  int dev = 0;
  QWG_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(QWG_E_HIP, "device index outside 0..63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    QWG_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(QWG_E_HIP, "hipGetSymbolAddress gave a null address for the static scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QWG_OK;
}

int qwg_gemv_noalloc(int qtype, const void* d_packed, int64_t rows, int64_t k, const float* d_x, int n_cols,
                     float* d_y, void* stream) {
  if (int rc = check_matrix(qtype, rows, k)) return rc;
  if (n_cols < 1 || n_cols > gemv_max_cols(qtype, k))
    return fail(QWG_E_SHAPE, "n_cols must be in 1..8 (1..64 for Q4_K, Q5_K, Q6_K with k a multiple of 512)");
  if (rows == 0) return QWG_OK;
  if (!d_packed || !d_x || !d_y) return fail(QWG_E_INVAL, "NULL pointer");
  if (!aligned16(d_packed) || !aligned16(d_x)) return fail(QWG_E_INVAL, "d_packed and d_x must be 16-byte aligned");
  size_t dig = 0, need = 0;
  gemv_work_layout(qtype, rows, k, n_cols, &dig, &need);
  if (need > (size_t)QWG_NOALLOC_SCRATCH_BYTES)
    return fail(QWG_E_NOMEM, "this GEMV needs " + std::to_string(need) + " bytes of scratch, more than the " +
                                 std::to_string((size_t)QWG_NOALLOC_SCRATCH_BYTES) +
                                 " of the static scratch (use qwg_gemv with a work buffer)");
  void* work = nullptr;
  if (int rc = scratch_of_current_device(&work)) return rc;
  return gemv_run(qtype, d_packed, rows, k, d_x, n_cols, d_y, work, (size_t)QWG_NOALLOC_SCRATCH_BYTES,
                  (hipStream_t)stream);
}

int qwg_set_gemv_geometry(int waves_per_group, int rows_per_wave, int pipeline_depth, int row_passes) {
  if (waves_per_group < 0 || waves_per_group > 16)
    return fail(QWG_E_INVAL, "waves_per_group must be 0..16");
  if (!(rows_per_wave == 0 || rows_per_wave == 1 || rows_per_wave == 2 || rows_per_wave == 4))
    return fail(QWG_E_INVAL, "rows_per_wave must be 0, 1, 2 or 4");
  if (!(pipeline_depth == 0 || pipeline_depth == 1 || pipeline_depth == 2))
    return fail(QWG_E_INVAL, "pipeline_depth must be 0, 1 or 2");
  if (!(row_passes == 0 || row_passes == 1 || row_passes == 2 || row_passes == 4 || row_passes == 8))
    return fail(QWG_E_INVAL, "row_passes must be 0, 1, 2, 4 or 8");
  set_gemv_geometry(waves_per_group, rows_per_wave, pipeline_depth, row_passes);
  return QWG_OK;
}

int qwg_set_gemv_mfma(int on) {
  if (on != 0 && on != 1) return fail(QWG_E_INVAL, "on must be 0 or 1");
  set_gemv_mfma(on);
  return QWG_OK;
}

size_t qwg_read_sink_words(void) { return (size_t)READ_GRID_MAX * 8; }

int qwg_read_bytes(const void* d_src, size_t bytes, uint32_t* d_sink, int grid, int unroll, float* h_kernel_ms,
                   void* stream) {
  if (!d_src || !d_sink) return fail(QWG_E_INVAL, "NULL pointer");
  if (bytes == 0 || bytes % 16) return fail(QWG_E_SHAPE, "bytes must be a positive multiple of 16");
  if (!aligned16(d_src)) return fail(QWG_E_INVAL, "d_src must be 16-byte aligned");
  if (grid < 0 || grid > READ_GRID_MAX) return fail(QWG_E_INVAL, "grid must be 0..8192");
  if (!(unroll == 0 || unroll == 4 || unroll == 8 || unroll == 16)) return fail(QWG_E_INVAL, "unroll must be 0, 4, 8 or 16");
  hipStream_t st = (hipStream_t)stream;
  if (!h_kernel_ms) {
    QWG_HIP(launch_read(d_src, (int64_t)bytes, d_sink, st, grid, unroll));
    return QWG_OK;
  }
  // timed: events recorded by the dispatch itself at the kernel's start and end, then a wait
  hipEvent_t e[2] = {nullptr, nullptr};
  for (auto& x : e) QWG_HIP(hipEventCreateWithFlags(&x, hipEventDisableSystemFence));
  hipError_t err = launch_read(d_src, (int64_t)bytes, d_sink, st, grid, unroll, e[0], e[1]);
  if (err == hipSuccess) err = hipEventSynchronize(e[1]);
  if (err == hipSuccess) err = hipEventElapsedTime(h_kernel_ms, e[0], e[1]);
  for (auto x : e) (void)hipEventDestroy(x);
  if (err != hipSuccess) return fail(QWG_E_HIP, std::string("timed read: ") + hipGetErrorString(err));
  return QWG_OK;
}

int qwg_rmsnorm(const float* d_x, const float* d_g, int64_t n, float eps, int n_cols, float* d_out, void* stream) {
  if (!d_x || !d_g || !d_out) return fail(QWG_E_INVAL, "NULL pointer");
  if (n < 1 || n > 65536 || n_cols < 1 || n_cols > 65535) return fail(QWG_E_SHAPE, "bad n or n_cols");
  QWG_HIP(launch_rmsnorm(d_x, d_g, n, eps, n_cols, d_out, (hipStream_t)stream));
  return QWG_OK;
}

int qwg_rope_table(int max_pos, int head_dim, double base, float* h_table) {
  if (!h_table) return fail(QWG_E_INVAL, "NULL pointer");
  if (max_pos < 1 || head_dim < 2 || head_dim % 2) return fail(QWG_E_SHAPE, "bad max_pos or head_dim");
  const int half = head_dim / 2;
  for (int i = 0; i < half; ++i) {
    const double th = std::pow(base, -2.0 * i / (double)head_dim);
    for (int p = 0; p < max_pos; ++p) {
      const double phi = (double)p * th;
      h_table[((size_t)p * half + i) * 2] = (float)std::cos(phi);
      h_table[((size_t)p * half + i) * 2 + 1] = (float)std::sin(phi);
    }
  }
  return QWG_OK;
}

int qwg_rope(float* d_v, int n_heads, int head_dim, const float* d_table, int pos, void* stream) {
  if (!d_v || !d_table) return fail(QWG_E_INVAL, "NULL pointer");
  if (head_dim != HEAD_DIM) return fail(QWG_E_SHAPE, "head_dim must be 128");
  if (n_heads < 1 || pos < 0) return fail(QWG_E_SHAPE, "n_heads must be positive and pos non-negative");
  if (((uintptr_t)d_v & 7) || ((uintptr_t)d_table & 7)) return fail(QWG_E_INVAL, "pointers must be 8-byte aligned");
  QWG_HIP(launch_rope(d_v, n_heads, d_table, pos, (hipStream_t)stream));
  return QWG_OK;
}

size_t qwg_attn_work_bytes(int n_pos, int n_q, int n_kv, int head_dim, int n_cols) {
  if (n_pos < 1 || n_pos > 262144 || n_q < 1 || n_kv < 1 || n_kv > 64 || n_q % n_kv || head_dim != HEAD_DIM ||
      n_cols < 1 || n_cols > MAX_PREFILL_COLS || n_q / n_kv > 64)
    return 0;
  return plan_attn(n_pos, n_q, n_kv, n_cols).work_bytes;
}

int qwg_attn_decode(const float* d_q, const uint16_t* d_kc, const uint16_t* d_vc, int n_pos, int n_q, int n_kv,
                    int head_dim, int n_cols, float* d_out, void* d_work, size_t work_bytes, void* stream) {
  if (!d_q || !d_kc || !d_vc || !d_out || !d_work) return fail(QWG_E_INVAL, "NULL pointer");
  if (head_dim != HEAD_DIM) return fail(QWG_E_SHAPE, "head_dim must be 128");
  if (n_pos < 1 || n_pos > 262144 || n_q < 1 || n_kv < 1 || n_kv > 64 || n_q % n_kv || n_cols < 1 ||
      n_cols > MAX_PREFILL_COLS)
    return fail(QWG_E_SHAPE, "bad attention shape");
  if (n_q / n_kv > 64) return fail(QWG_E_SHAPE, "n_q / n_kv must be <= 64");
  const AttnPlan p = plan_attn(n_pos, n_q, n_kv, n_cols);
  if (work_bytes < p.work_bytes) return fail(QWG_E_NOMEM, "work buffer smaller than qwg_attn_work_bytes");
  if (!aligned16(d_q) || !aligned16(d_kc) || !aligned16(d_vc) || ((uintptr_t)d_out & 7) || ((uintptr_t)d_work & 7))
    return fail(QWG_E_INVAL, "d_q, d_kc, d_vc must be 16-byte aligned, d_out and d_work 8-byte aligned");
  QWG_HIP(launch_attn(d_q, (int64_t)n_q * HEAD_DIM, d_kc, d_vc, (int64_t)n_kv * HEAD_DIM, n_pos, n_q, n_kv, n_cols,
                      d_out, (int64_t)n_q * HEAD_DIM, d_work, p, (hipStream_t)stream));
  return QWG_OK;
}

int qwg_swiglu(const float* d_g, const float* d_u, int64_t n, float* d_out, void* stream) {
  if (!d_g || !d_u || !d_out) return fail(QWG_E_INVAL, "NULL pointer");
  if (n < 0) return fail(QWG_E_SHAPE, "n < 0");
  QWG_HIP(launch_swiglu(d_g, d_u, n, d_out, (hipStream_t)stream));
  return QWG_OK;
}

int qwg_cosine(const float* d_a, const float* d_b, int64_t n, float* d_out, void* stream) {
  if (!d_a || !d_b || !d_out) return fail(QWG_E_INVAL, "NULL pointer");
  if (n < 1) return fail(QWG_E_SHAPE, "n < 1");
  QWG_HIP(launch_cosine(d_a, d_b, n, d_out, (hipStream_t)stream));
  return QWG_OK;
}

size_t qwg_argmax_work_bytes(void) { return ARGMAX_WORK_BYTES; }

int qwg_argmax(const float* d_x, int64_t n, int32_t* d_out, void* d_work, size_t work_bytes, void* stream) {
  if (!d_x || !d_out || !d_work) return fail(QWG_E_INVAL, "NULL pointer");
  if (n < 1 || n > 0x7FFFFFFE) return fail(QWG_E_SHAPE, "n out of range");
  if (work_bytes < ARGMAX_WORK_BYTES) return fail(QWG_E_NOMEM, "work buffer smaller than qwg_argmax_work_bytes");
  if ((uintptr_t)d_work & 7) return fail(QWG_E_INVAL, "d_work must be 8-byte aligned");
  QWG_HIP(launch_argmax(d_x, n, 1, n, d_out, (hipStream_t)stream, (unsigned long long*)d_work));
  return QWG_OK;
}

// ------------------------------------------------------------------------------------- model ABI

int qwg_model_create(const qwg_model_desc* desc, qwg_model** out) {
  if (!out) return fail(QWG_E_INVAL, "out is NULL");
  *out = nullptr;
  if (int rc = check_desc(desc)) return rc;
  return guarded([&]() -> int {
    qwg_model* m = new qwg_model();
    init_desc(m, desc);
    m->skip.assign(desc->n_layers, 0);
    plan_model(m);
    *out = m;
    return QWG_OK;
  });
}

size_t qwg_model_arena_bytes(const qwg_model* m) { return m ? m->total : 0; }

// MemAvailable of /proc/meminfo in bytes, or 0 if it cannot be read
static size_t host_mem_available() {
  FILE* f = std::fopen("/proc/meminfo", "r");
  if (!f) return 0;
  char line[256];
  size_t kib = 0;
  while (std::fgets(line, sizeof line, f)) {
    unsigned long long v = 0;
    if (std::sscanf(line, "MemAvailable: %llu kB", &v) == 1) {
      kib = (size_t)v;
      break;
    }
  }
  std::fclose(f);
  return kib * 1024;
}

int qwg_plan_residency(const qwg_model_desc* desc, size_t device_budget, size_t host_budget, int* n_resident,
                       size_t* arena_bytes, size_t* pinned_bytes) {
  if (!n_resident) return fail(QWG_E_INVAL, "n_resident is NULL");
  if (int rc = check_desc(desc)) return rc;
  return guarded([&]() -> int {
    size_t dev = device_budget, host = host_budget;
    if (dev == 0) {
      size_t fr = 0, tot = 0;
      QWG_HIP(hipMemGetInfo(&fr, &tot));
      const size_t reserve = std::max<size_t>((size_t)1 << 30, tot / 50);  // runtime and other allocations
      dev = fr > reserve ? fr - reserve : 0;
    }
    if (host == 0) host = host_mem_available() / 10 * 9;  // leave a tenth to the rest of the system
    // the most layers whose arena fits the device budget (the arena grows with every resident layer)
    qwg_model m;
    init_desc(&m, desc);
    int best = -1;
    size_t best_total = 0, image = 0;
    for (int n = desc->n_layers; n >= 0; --n) {
      m.d.n_resident = n;
      plan_model(&m);
      image = m.image_max;
      if (m.total <= dev) {
        best = n;
        best_total = m.total;
        break;
      }
    }
    if (best < 0) return fail(QWG_E_NOMEM, "the model's non-layer arena does not fit the device budget");
    const size_t pinned = (size_t)(desc->n_layers - best) * image;
    if (pinned > host) return fail(QWG_E_NOMEM, "streamed layers do not fit the pinned host budget (no file-backed tier)");
    *n_resident = best;
    if (arena_bytes) *arena_bytes = best_total;
    if (pinned_bytes) *pinned_bytes = pinned;
    return QWG_OK;
  });
}

int qwg_model_bind(qwg_model* m, void* d_arena, size_t bytes, void* compute, void* copy) {
  if (!m || !d_arena) return fail(QWG_E_INVAL, "NULL pointer");
  if (m->bound) return fail(QWG_E_STATE, "model already bound");
  if (bytes < m->total) return fail(QWG_E_NOMEM, "arena smaller than qwg_model_arena_bytes");
  if ((uintptr_t)d_arena & 255) return fail(QWG_E_INVAL, "arena must be 256-byte aligned");
  m->arena = (uint8_t*)d_arena;
  m->cs = (hipStream_t)compute;
  m->xs = copy ? (hipStream_t)copy : (hipStream_t)compute;
  for (int i = 0; i < 2; ++i) {
    QWG_HIP(hipEventCreateWithFlags(&m->ev_full[i], hipEventDisableTiming));
    QWG_HIP(hipEventCreateWithFlags(&m->ev_free[i], hipEventDisableTiming));
    QWG_HIP(hipEventRecord(m->ev_free[i], m->cs));
  }
  for (auto& P : m->L) {
    if (P.resident) continue;
    void* p = nullptr;
    hipError_t e = hipHostMalloc(&p, P.image, hipHostMallocDefault);
    if (e != hipSuccess) return fail(QWG_E_NOMEM, std::string("pinned host image: ") + hipGetErrorString(e));
    P.host = (uint8_t*)p;
  }
  // rope table (fp64 -> fp32) and zeroed caches / activations
  std::vector<float> tab((size_t)m->d.max_ctx * m->d.head_dim);
  qwg_rope_table(m->d.max_ctx, m->d.head_dim, (double)m->d.rope_theta, tab.data());
  QWG_HIP(hipMemcpyAsync(m->arena + m->rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, m->cs));
  for (auto& P : m->L) {
    QWG_HIP(hipMemsetAsync(m->arena + P.kc, 0, (size_t)m->d.max_ctx * m->KR() * 2, m->cs));
    QWG_HIP(hipMemsetAsync(m->arena + P.vc, 0, (size_t)m->d.max_ctx * m->KR() * 2, m->cs));
  }
  QWG_HIP(hipStreamSynchronize(m->cs));
  m->bound = true;
  return QWG_OK;
}

void qwg_model_destroy(qwg_model* m) {
  if (!m) return;
  if (m->bound) {
    (void)hipStreamSynchronize(m->cs);
    (void)hipStreamSynchronize(m->xs);
  }
  for (auto& P : m->L) {
    if (P.host) (void)hipHostFree(P.host);
    if (P.map) munmap((void*)P.map, P.map_len);
  }
  for (int i = 0; i < 2; ++i) {
    if (m->ev_full[i]) (void)hipEventDestroy(m->ev_full[i]);
    if (m->ev_free[i]) (void)hipEventDestroy(m->ev_free[i]);
    if (m->ev_staged[i]) (void)hipEventDestroy(m->ev_staged[i]);
    if (m->stage[i]) (void)hipHostFree(m->stage[i]);
  }
  for (auto e : m->tev) (void)hipEventDestroy(e);
  for (auto e : m->cev) (void)hipEventDestroy(e);
  delete m;
}

int qwg_model_set_tensor(qwg_model* m, int layer, int tensor_id, int qtype, const void* h_canon, size_t nbytes) {
  if (!m || !h_canon) return fail(QWG_E_INVAL, "NULL pointer");
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  const qwg_model_desc& d = m->d;
  const MatPlan* mp = nullptr;
  int64_t rows = 0, k = 0, row0 = 0, step = 1;
  int want_qt = -1;
  bool global = tensor_id == QWG_T_EMBED || tensor_id == QWG_T_HEAD;
  if (global ? layer != -1 : (layer < 0 || layer >= d.n_layers)) return fail(QWG_E_INVAL, "bad layer index");
  LayerPlan* P = global ? nullptr : &m->L[layer];
  switch (tensor_id) {
    case QWG_T_EMBED: mp = &m->embed; rows = d.vocab; k = d.hidden; want_qt = d.qtype_embed; break;
    case QWG_T_HEAD: mp = &m->head; rows = d.vocab; k = d.hidden; want_qt = d.qtype_head; break;
    case QWG_T_WQ: mp = &P->qkv; rows = m->QR(); k = d.hidden; break;
    case QWG_T_WK: mp = &P->qkv; rows = m->KR(); k = d.hidden; row0 = m->QR(); break;
    case QWG_T_WV: mp = &P->qkv; rows = m->KR(); k = d.hidden; row0 = m->QR() + m->KR(); break;
    case QWG_T_WO: mp = &P->o; rows = d.hidden; k = m->QR(); break;
    case QWG_T_WGATE: mp = &P->gu; rows = d.ffn; k = d.hidden; step = 2; break;
    case QWG_T_WUP: mp = &P->gu; rows = d.ffn; k = d.hidden; row0 = 1; step = 2; break;
    case QWG_T_WDOWN: mp = &P->down; rows = d.hidden; k = d.ffn; break;
    default: return fail(QWG_E_INVAL, "unknown tensor id");
  }
  if (!global) want_qt = mp->L.qtype;  // the layer's type for this matrix
  if (qtype != want_qt) return fail(QWG_E_UNSUPPORTED, "qtype differs from the model description");
  const int64_t rb = canon_row_bytes(qtype, k);
  if ((int64_t)nbytes != rows * rb) return fail(QWG_E_SHAPE, "nbytes != rows * row_bytes");
  const bool streamed = P && !P->resident;
  if (streamed && P->map) return fail(QWG_E_STATE, "the layer's image is file-backed (spilled)");
  uint8_t* dst;
  if (global) dst = m->arena + mp->off;
  else if (!streamed) dst = m->arena + P->arena_off + mp->off;
  else dst = m->arena + m->slot[0] + mp->off;
  if (streamed)  // keep the rows of the fused matrix that other tensors already wrote
    QWG_HIP(hipMemcpyAsync(dst, P->host + mp->off, (size_t)mp->L.total, hipMemcpyHostToDevice, m->cs));
  const int64_t chunk_rows = std::max<int64_t>(1, (int64_t)m->staging_bytes / rb);
  for (int64_t r = 0; r < rows; r += chunk_rows) {
    const int64_t n = std::min(chunk_rows, rows - r);
    QWG_HIP(hipMemcpyAsync(m->arena + m->staging, (const uint8_t*)h_canon + r * rb, (size_t)(n * rb),
                           hipMemcpyHostToDevice, m->cs));
    QWG_HIP(launch_repack(qtype, m->arena + m->staging, n, k, dst, mp->L, row0 + r * step, step, m->cs));
  }
  if (streamed)
    QWG_HIP(hipMemcpyAsync(P->host + mp->off, dst, (size_t)mp->L.total, hipMemcpyDeviceToHost, m->cs));
  QWG_HIP(hipStreamSynchronize(m->cs));
  return QWG_OK;
}

int qwg_model_set_norm(qwg_model* m, int layer, int which, const float* h_g, int n) {
  if (!m || !h_g) return fail(QWG_E_INVAL, "NULL pointer");
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  if (n != m->d.hidden) return fail(QWG_E_SHAPE, "gain length must equal hidden");
  size_t off;
  if (which == QWG_NORM_FINAL && layer == -1) off = m->g_final;
  else if ((which == QWG_NORM_ATTN || which == QWG_NORM_FFN) && layer >= 0 && layer < m->d.n_layers)
    off = which == QWG_NORM_ATTN ? m->L[layer].g_attn : m->L[layer].g_ffn;
  else return fail(QWG_E_INVAL, "bad norm id / layer");
  QWG_HIP(hipMemcpy(m->arena + off, h_g, (size_t)n * 4, hipMemcpyHostToDevice));
  return QWG_OK;
}

int qwg_model_set_kv(qwg_model* m, int layer, const uint16_t* h_k, const uint16_t* h_v, int n_pos) {
  if (!m || (n_pos > 0 && (!h_k || !h_v))) return fail(QWG_E_INVAL, "NULL pointer");
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  if (layer < 0 || layer >= m->d.n_layers) return fail(QWG_E_INVAL, "bad layer");
  if (n_pos < 0 || n_pos > m->d.max_ctx) return fail(QWG_E_SHAPE, "n_pos outside 0..max_ctx");
  const size_t bytes = (size_t)n_pos * m->KR() * 2;
  QWG_HIP(hipStreamSynchronize(m->cs));
  QWG_HIP(hipMemcpy(m->arena + m->L[layer].kc, h_k, bytes, hipMemcpyHostToDevice));
  QWG_HIP(hipMemcpy(m->arena + m->L[layer].vc, h_v, bytes, hipMemcpyHostToDevice));
  m->n_past = n_pos;
  return QWG_OK;
}

int qwg_model_get_kv(qwg_model* m, int layer, uint16_t* h_k, uint16_t* h_v, int n_pos) {
  if (!m || (n_pos > 0 && (!h_k || !h_v))) return fail(QWG_E_INVAL, "NULL pointer");
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  if (layer < 0 || layer >= m->d.n_layers) return fail(QWG_E_INVAL, "bad layer");
  if (n_pos < 0 || n_pos > m->d.max_ctx) return fail(QWG_E_SHAPE, "n_pos outside 0..max_ctx");
  const size_t bytes = (size_t)n_pos * m->KR() * 2;
  QWG_HIP(hipStreamSynchronize(m->cs));
  QWG_HIP(hipMemcpy(h_k, m->arena + m->L[layer].kc, bytes, hipMemcpyDeviceToHost));
  QWG_HIP(hipMemcpy(h_v, m->arena + m->L[layer].vc, bytes, hipMemcpyDeviceToHost));
  return QWG_OK;
}

int qwg_decode_step(qwg_model* m, int32_t token, int32_t* next_token, float* h_logits) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  return guarded([&]() -> int {
    if (int rc = run_pass(m, &token, 1, m->n_past, m->d.n_layers, false)) return rc;
    int32_t nt = 0;
    if (int rc = finish_pass(m, 1, &nt, h_logits)) return rc;
    if (next_token) *next_token = nt;
    m->n_past += 1;
    return QWG_OK;
  });
}

int qwg_prefill(qwg_model* m, const int32_t* tokens, int n, int32_t* next_token, float* h_logits) {
  if (!m || !tokens) return fail(QWG_E_INVAL, "NULL pointer");
  if (n < 1) return fail(QWG_E_SHAPE, "n must be >= 1");
  return guarded([&]() -> int {
    if (m->n_past + n > m->d.max_ctx) return fail(QWG_E_STATE, "context full (n_past + n > max_ctx)");
    const int C = prefill_width(m);
    for (int i = 0; i < n; i += C) {
      const int c = std::min(C, n - i);
      const bool last = i + c == n;
      if (int rc = run_pass(m, tokens + i, c, m->n_past, m->d.n_layers, false, last)) return rc;
      if (last) {
        // a wide pass computes the head for its last column only (column 0 of the logits)
        const int hc = c > MAX_COLS ? 1 : c;
        std::vector<int32_t> am(hc);
        if (int rc = finish_pass(m, hc, am.data(), nullptr)) return rc;
        if (next_token) *next_token = am[hc - 1];
        if (h_logits)
          QWG_HIP(hipMemcpy(h_logits, m->f(m->logits) + (size_t)(hc - 1) * m->d.vocab, (size_t)m->d.vocab * 4,
                            hipMemcpyDeviceToHost));
      }
      m->n_past += c;
    }
    return QWG_OK;
  });
}

int qwg_calibrate_skip(qwg_model* m, float tau, int32_t token, int32_t* next_token, float* h_cos, uint8_t* h_mask) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  return guarded([&]() -> int {
    if (int rc = run_pass(m, &token, 1, m->n_past, m->d.n_layers, true)) return rc;
    int32_t nt = 0;
    if (int rc = finish_pass(m, 1, &nt, nullptr)) return rc;
    std::vector<float> cs(m->d.n_layers);
    QWG_HIP(hipMemcpy(cs.data(), m->f(m->cosv), cs.size() * 4, hipMemcpyDeviceToHost));
    for (int l = 0; l < m->d.n_layers; ++l) m->skip[l] = cs[l] >= tau ? 1 : 0;
    if (h_cos) std::memcpy(h_cos, cs.data(), cs.size() * 4);
    if (h_mask) std::memcpy(h_mask, m->skip.data(), m->skip.size());
    if (next_token) *next_token = nt;
    m->n_past += 1;
    return QWG_OK;
  });
}

int qwg_set_layer_skip(qwg_model* m, int layer, int skip) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  if (layer < 0 || layer >= m->d.n_layers) return fail(QWG_E_INVAL, "bad layer");
  m->skip[layer] = skip ? 1 : 0;
  return QWG_OK;
}

int qwg_get_layer_skip(qwg_model* m, uint8_t* h_mask) {
  if (!m || !h_mask) return fail(QWG_E_INVAL, "NULL pointer");
  std::memcpy(h_mask, m->skip.data(), m->skip.size());
  return QWG_OK;
}

int qwg_spec_step(qwg_model* m, int32_t token, int draft_layers, int k, int32_t* out_tokens, int* n_out,
                  int* n_accepted) {
  if (!m || !out_tokens || !n_out || !n_accepted) return fail(QWG_E_INVAL, "NULL pointer");
  if (k < 1 || k + 1 > std::min(m->d.max_cols, MAX_COLS)) return fail(QWG_E_SHAPE, "need 1 <= k and k + 1 <= min(max_cols, 8)");
  if (draft_layers < 0 || draft_layers > m->d.n_layers) return fail(QWG_E_SHAPE, "bad draft_layers");
  return guarded([&]() -> int {
    const int p = m->n_past;
    if (p + k + 1 > m->d.max_ctx) return fail(QWG_E_STATE, "context full");
    std::vector<int32_t> cols(k + 1), verdict(k + 1);
    cols[0] = token;
    int32_t t = token;
    for (int j = 0; j < k; ++j) {
      if (int rc = run_pass(m, &t, 1, p + j, draft_layers, false)) return rc;
      if (int rc = finish_pass(m, 1, &t, nullptr)) return rc;
      cols[j + 1] = t;
    }
    if (int rc = run_pass(m, cols.data(), k + 1, p, m->d.n_layers, false)) return rc;
    if (int rc = finish_pass(m, k + 1, verdict.data(), nullptr)) return rc;
    int a = 0;
    while (a < k && verdict[a] == cols[a + 1]) ++a;
    for (int j = 0; j < a; ++j) out_tokens[j] = cols[j + 1];
    out_tokens[a] = verdict[a];
    *n_out = a + 1;
    *n_accepted = a;
    m->n_past = p + a + 1;
    return QWG_OK;
  });
}

int qwg_verify(qwg_model* m, const int32_t* tokens, int n, float* h_logits, int32_t* h_argmax) {
  if (!m || !tokens) return fail(QWG_E_INVAL, "NULL pointer");
  if (n < 1 || n > MAX_COLS) return fail(QWG_E_SHAPE, "verify takes 1..8 columns");
  return guarded([&]() -> int {
    if (int rc = run_pass(m, tokens, n, m->n_past, m->d.n_layers, false)) return rc;
    std::vector<int32_t> am(n);
    if (int rc = finish_pass(m, n, am.data(), h_logits)) return rc;
    if (h_argmax) std::memcpy(h_argmax, am.data(), (size_t)n * 4);
    return QWG_OK;
  });
}

int qwg_model_n_past(const qwg_model* m) { return m ? m->n_past : -1; }

int qwg_model_truncate(qwg_model* m, int n_past) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  if (n_past < 0 || n_past > m->d.max_ctx) return fail(QWG_E_STATE, "n_past outside 0..max_ctx");
  m->n_past = n_past;
  return QWG_OK;
}

int qwg_model_set_capture(qwg_model* m, int on) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  m->capture_on = on != 0;
  return QWG_OK;
}

int qwg_model_get_hidden(qwg_model* m, int layer, float* h_out) {
  if (!m || !h_out) return fail(QWG_E_INVAL, "NULL pointer");
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  if (layer < -1 || layer >= m->d.n_layers) return fail(QWG_E_INVAL, "bad layer");
  QWG_HIP(hipStreamSynchronize(m->cs));
  QWG_HIP(hipMemcpy(h_out, m->f(m->capture) + (size_t)(layer + 1) * m->d.hidden, (size_t)m->d.hidden * 4,
                    hipMemcpyDeviceToHost));
  return QWG_OK;
}

int qwg_model_set_timing(qwg_model* m, int tensor_id) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  if (tensor_id != -1 && tensor_id != QWG_TIME_ALL_GEMV && timing_slot(tensor_id) < 0)
    return fail(QWG_E_INVAL, "timing class must be WQ, WO, WGATE, WDOWN, HEAD, QWG_TIME_ALL_GEMV or -1");
  m->timing_tensor = tensor_id;
  for (int c = 0; c < 5; ++c) {
    m->t_ms[c] = 0.0;
    m->t_n[c] = 0;
    m->t_bytes[c] = 0;
  }
  return QWG_OK;
}

int qwg_model_get_timing_class(qwg_model* m, int tensor_id, double* total_ms, int64_t* n_launches,
                               int64_t* total_bytes) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  double ms = 0.0;
  int64_t n = 0, b = 0;
  for (int c = 0; c < 5; ++c) {
    static const int ids[5] = {QWG_T_WQ, QWG_T_WO, QWG_T_WGATE, QWG_T_WDOWN, QWG_T_HEAD};
    if (tensor_id != QWG_TIME_ALL_GEMV && ids[c] != tensor_id) continue;
    ms += m->t_ms[c];
    n += m->t_n[c];
    b += m->t_bytes[c];
  }
  if (tensor_id != QWG_TIME_ALL_GEMV && timing_slot(tensor_id) < 0) return fail(QWG_E_INVAL, "bad timing class");
  if (total_ms) *total_ms = ms;
  if (n_launches) *n_launches = n;
  if (total_bytes) *total_bytes = b;
  return QWG_OK;
}

int qwg_model_get_timing(qwg_model* m, double* total_ms, int64_t* n_launches, int64_t* bytes_per_launch) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  const int cls = m->timing_tensor == -1 ? QWG_TIME_ALL_GEMV : m->timing_tensor;
  double ms = 0.0;
  int64_t n = 0, b = 0;
  if (int rc = qwg_model_get_timing_class(m, cls, &ms, &n, &b)) return rc;
  if (total_ms) *total_ms = ms;
  if (n_launches) *n_launches = n;
  if (bytes_per_launch) *bytes_per_launch = n > 0 ? b / n : 0;
  return QWG_OK;
}

int qwg_model_set_debug(qwg_model* m, int knob, int64_t value) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  switch (knob) {
    case QWG_DEBUG_SPIN_US: {
      if (value < 0 || value > 100000) return fail(QWG_E_INVAL, "spin must be 0..100000 us");
      int khz = 0, dev = 0;
      QWG_HIP(hipGetDevice(&dev));
      QWG_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
      m->spin_ticks = (uint64_t)value * (uint64_t)khz / 1000u;
      return QWG_OK;
    }
    case QWG_DEBUG_FAIL_AT_LAYER:
      if (value < -1 || value >= m->d.n_layers) return fail(QWG_E_INVAL, "layer must be -1..n_layers-1");
      m->fail_layer = (int)value;
      return QWG_OK;
    default:
      return fail(QWG_E_INVAL, "unknown debug knob");
  }
}

int qwg_model_first_nonfinite(qwg_model* m, int* layer) {
  if (!m || !layer) return fail(QWG_E_INVAL, "NULL pointer");
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  return guarded([&]() -> int {
    const int H = m->d.hidden, L = m->d.n_layers;
    std::vector<float> cap((size_t)(L + 1) * H), lg((size_t)m->d.vocab);
    QWG_HIP(hipStreamSynchronize(m->cs));
    QWG_HIP(hipMemcpy(cap.data(), m->f(m->capture), cap.size() * 4, hipMemcpyDeviceToHost));
    QWG_HIP(hipMemcpy(lg.data(), m->f(m->logits), lg.size() * 4, hipMemcpyDeviceToHost));
    *layer = -2;
    for (int l = -1; l < L && *layer == -2; ++l)
      for (int i = 0; i < H; ++i)
        if (!std::isfinite(cap[(size_t)(l + 1) * H + i])) {
          *layer = l;
          break;
        }
    if (*layer == -2)
      for (float v : lg)
        if (!std::isfinite(v)) {
          *layer = L;
          break;
        }
    return QWG_OK;
  });
}

int qwg_model_spill_layer(qwg_model* m, int layer, const char* path) {
  if (!m || !path) return fail(QWG_E_INVAL, "NULL pointer");
  if (!m->bound) return fail(QWG_E_STATE, "model is not bound");
  if (layer < 0 || layer >= m->d.n_layers) return fail(QWG_E_INVAL, "bad layer index");
  LayerPlan& P = m->L[layer];
  if (P.resident) return fail(QWG_E_STATE, "only streamed layers can be file-backed");
  if (P.map) return fail(QWG_E_STATE, "layer already file-backed");
  return guarded([&]() -> int {
    QWG_HIP(hipStreamSynchronize(m->cs));
    QWG_HIP(hipStreamSynchronize(m->xs));
    if (!m->stage[0]) {
      for (int i = 0; i < 2; ++i) {
        void* p = nullptr;
        hipError_t e = hipHostMalloc(&p, m->image_max, hipHostMallocDefault);
        if (e != hipSuccess) return fail(QWG_E_NOMEM, std::string("pinned staging: ") + hipGetErrorString(e));
        m->stage[i] = (uint8_t*)p;
        QWG_HIP(hipEventCreateWithFlags(&m->ev_staged[i], hipEventDisableTiming));
        QWG_HIP(hipEventRecord(m->ev_staged[i], m->xs));
      }
    }
    const int fd = open(path, O_RDWR | O_CREAT | O_TRUNC, 0600);
    if (fd < 0) return fail(QWG_E_INVAL, std::string("cannot create ") + path);
    size_t done = 0;
    while (done < P.image) {
      const ssize_t w = write(fd, P.host + done, P.image - done);
      if (w <= 0) {
        close(fd);
        return fail(QWG_E_NOMEM, std::string("write failed: ") + path);
      }
      done += (size_t)w;
    }
    void* map = mmap(nullptr, P.image, PROT_READ, MAP_SHARED, fd, 0);
    close(fd);
    if (map == MAP_FAILED) return fail(QWG_E_NOMEM, std::string("mmap failed: ") + path);
    QWG_HIP(hipHostFree(P.host));
    P.host = nullptr;
    P.map = (const uint8_t*)map;
    P.map_len = P.image;
    return QWG_OK;
  });
}

int qwg_model_file_stats(qwg_model* m, int64_t* bytes, double* ms) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  if (bytes) *bytes = m->file_bytes;
  if (ms) *ms = m->file_ms;
  m->file_bytes = 0;
  m->file_ms = 0.0;
  return QWG_OK;
}

int qwg_model_stream_stats(qwg_model* m, int64_t* h2d_bytes, double* h2d_ms) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  if (h2d_bytes) *h2d_bytes = m->h2d_bytes;
  if (h2d_ms) *h2d_ms = m->h2d_ms;
  m->h2d_ms = 0.0;
  m->h2d_bytes = 0;
  return QWG_OK;
}

int qwg_sync(qwg_model* m) {
  if (!m) return fail(QWG_E_INVAL, "NULL model");
  if (!m->bound) return QWG_OK;
  QWG_HIP(hipStreamSynchronize(m->cs));
  QWG_HIP(hipStreamSynchronize(m->xs));
  return QWG_OK;
}

int qwg_host_alloc(size_t bytes, void** out) {
  if (!out) return fail(QWG_E_INVAL, "out is NULL");
  hipError_t e = hipHostMalloc(out, bytes, hipHostMallocDefault);
  if (e != hipSuccess) return fail(QWG_E_NOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  return QWG_OK;
}

int qwg_host_free(void* p) {
  if (!p) return QWG_OK;
  QWG_HIP(hipHostFree(p));
  return QWG_OK;
}

}  // extern "C"
