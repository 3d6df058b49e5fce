// nt_api.hip -- the extern "C" boundary of libnt: argument validation,
// launch planning and kernel launches.  No allocation, no synchronization.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "nt_internal.h"

using namespace nt;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace of one decode layer for M tokens (offsets from the base).  With
// M >= 2 it also holds the small-M GEMM's staged activation and partial sums.
// qx_o, qx_h, qx_a: the quantized activations (qx_bytes each per token) that
// the attention, O and gate/up launches hand to the next launch.
// stage, part, ss: the small-M GEMM's staged activation, partial sums and the
// staged residual stream's sums of squares per 256-block.
struct LayerWs {
  size_t q, part_o, part_ml, o, a, err, qx_o, qx_h, qx_a, stage, part, ss, total;
  int chunk, nsplit;
};

bool cfg_ok(const nt_layer_cfg& c) {
  if (c.hidden <= 0 || c.n_head <= 0 || c.n_kv_head <= 0 || c.ffn <= 0 || c.max_ctx <= 0) return false;
  if (c.n_head % c.n_kv_head != 0 || c.n_head / c.n_kv_head > 8) return false;
  if (c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256) return false;
  if (c.hidden % 32 || c.ffn % 32 || (c.n_head * c.head_dim) % 32) return false;
  if (c.hidden > kMaxCols || c.ffn > kMaxCols || c.n_head * c.head_dim > kMaxCols) return false;
  if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.f)) return false;
  int chunk = 0, nsplit = 0;
  attn_plan(c.head_dim, c.max_ctx, chunk, nsplit);
  if (nsplit > 1024) return false;  // the combine merges at most 1024 splits
  return true;
}

LayerWs layer_ws(const nt_layer_cfg& c, int M) {
  LayerWs w{};
  attn_plan(c.head_dim, c.max_ctx, w.chunk, w.nsplit);
  const size_t nq = (size_t)c.n_head * c.head_dim;
  size_t off = 0;
  w.q = off; off += up256((size_t)M * nq * 4);
  w.part_o = off; off += up256((size_t)M * w.nsplit * nq * 4);
  w.part_ml = off; off += up256((size_t)M * w.nsplit * c.n_head * 2 * 4);
  w.o = off; off += up256((size_t)M * nq * 4);
  w.a = off; off += up256((size_t)M * c.ffn * 4);
  w.err = off; off += 256;
  w.qx_o = off; off += up256((size_t)M * qx_bytes(nq));
  w.qx_h = off; off += up256((size_t)M * qx_bytes(c.hidden));
  w.qx_a = off; off += up256((size_t)M * qx_bytes(c.ffn));
  if (M >= 2) {
    const int64_t nkv = (int64_t)c.n_kv_head * c.head_dim;
    w.stage = off; off += up256(stage_m_bytes(std::max<int>(std::max<int>(c.hidden, (int)nq), c.ffn)));
    size_t pb = part_m_bytes((int64_t)nq + 2 * nkv, 0, c.hidden, M);
    pb = std::max(pb, part_m_bytes(c.hidden, 0, (int)nq, M));
    pb = std::max(pb, part_m_bytes(c.ffn, 1, c.hidden, M));
    pb = std::max(pb, part_m_bytes(c.hidden, 0, c.ffn, M));
    w.part = off; off += up256(pb);
    w.ss = off; off += up256((size_t)M * ((size_t)c.hidden / 256 + 1) * 4);
  }
  w.total = off;
  return w;
}

// Does a matrix of this format have the expected shape's column count?
bool fmt_cols_ok(int fmt, int64_t cols) { return block_elems(fmt) != 0 && cols % block_elems(fmt) == 0; }

int check_layer(const nt_layer_cfg& c, const nt_layer& L) {
  const int64_t nq = (int64_t)c.n_head * c.head_dim;
  const nt_qmat* mats[7] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
  const int64_t cols[7] = {c.hidden, c.hidden, c.hidden, nq, c.hidden, c.hidden, c.ffn};
  for (int i = 0; i < 7; ++i) {
    if (!fmt_cols_ok(mats[i]->fmt, cols[i])) return NT_EINVAL;
    if (block_elems(mats[i]->fmt) == 1) return NT_EUNSUPPORTED;  // F16/F32: GEMV only
    if (!mats[i]->data) return NT_EINVAL;
    if (!aligned16(mats[i]->data)) return NT_EALIGN;
  }
  if (!L.attn_norm || !L.ffn_norm || !L.k_cache || !L.v_cache) return NT_EINVAL;
  if (!aligned16(L.attn_norm) || !aligned16(L.ffn_norm)) return NT_EALIGN;
  return NT_OK;
}

const uint8_t* u8(const void* p) { return static_cast<const uint8_t*>(p); }

// How a small-M layer takes its input and hands its output on already staged
// (the small-M GEMM's activation layout, written by the reduce launch before;
// see RedArgs): the residual stream times the next launch's RMSNorm gains,
// with its sums of squares per 256-block for the normalization factor.
struct LayerStM {
  bool in_staged = false;            // the layer's input is staged (times attn_norm)
  const float* next_gain = nullptr;  // the gains of the next normalizing launch; null: no staging out
  bool out_staged = false;           // set when the down projection staged the output
};

// The launches of one layer for 2 <= M <= 8 tokens: each projection reads the
// weights once for all M tokens (int8 MFMA).  Its activation is staged by the
// launch before where the rows are whole 256-blocks (the attention combine ->
// O, the reduce launches O -> gate/up -> down -> the next layer's Q/K/V),
// else by a staging launch.
int run_layer_m(const nt_layer_cfg& c, const nt_layer& L, float* x, int M, const int32_t* pos, uint8_t* ws,
                const LayerWs& w, hipStream_t st, LayerStM* ls = nullptr) {
  const int nq = c.n_head * c.head_dim, nkv = c.n_kv_head * c.head_dim;
  float* q = reinterpret_cast<float*>(ws + w.q);
  float* part_o = reinterpret_cast<float*>(ws + w.part_o);
  float* part_ml = reinterpret_cast<float*>(ws + w.part_ml);
  float* o = reinterpret_cast<float*>(ws + w.o);
  float* a = reinterpret_cast<float*>(ws + w.a);
  int* err = reinterpret_cast<int*>(ws + w.err);
  void* stage = ws + w.stage;
  void* part = ws + w.part;
  float* ss = reinterpret_cast<float*>(ws + w.ss);
  const ProArgs none{nullptr, nullptr, 0.f, 0, 0, 0.f, nullptr, 0};
  const bool h256 = c.hidden % 256 == 0, f256 = c.ffn % 256 == 0;
  RedArgs rn_hidden;  // the RMSNorm factor of a staged residual stream
  rn_hidden.rn_ss = ss;
  rn_hidden.rn_nb = c.hidden / 256;
  rn_hidden.rn_cols = c.hidden;
  rn_hidden.rn_eps = c.rms_eps;
  const bool in_staged = ls && ls->in_staged && h256;
  if (ls) ls->out_staged = false;
  int rc;
  // 1. RMSNorm -> Q,K,V projections -> RoPE -> q, K/V append (token t at pos + t)
  {
    JobM job;
    const uint8_t* W[3] = {u8(L.wq.data), u8(L.wk.data), u8(L.wv.data)};
    const int fmt[3] = {L.wq.fmt, L.wk.fmt, L.wv.fmt};
    const int rows[3] = {nq, nkv, nkv};
    if ((rc = plan_job_m(job, 3, W, fmt, rows, c.hidden, 0, 1, M)) != NT_OK) return rc;
    if (!in_staged && (rc = launch_stage_m(x, c.hidden, L.attn_norm, c.rms_eps, M, c.hidden, stage, st)) != NT_OK)
      return rc;
    ProArgs pro = none;
    pro.rope_hd = c.head_dim;
    pro.rope_theta = c.rope_theta;
    pro.pos = pos;
    EpiArgs ea{};
    ea.q_out = q;
    ea.ld = nq;
    ea.k_cache = L.k_cache;
    ea.v_cache = L.v_cache;
    ea.pos = pos;
    ea.err = err;
    ea.head_dim = c.head_dim;
    ea.max_ctx = c.max_ctx;
    ea.rope_theta = c.rope_theta;
    ea.q_rows = nq;
    ea.kv_rows = nkv;
    if ((rc = launch_gemm_m(job, stage, part, pro, EPI_QKV, ea, st, in_staged ? rn_hidden : RedArgs{})) != NT_OK)
      return rc;
  }
  // 2. attention over the cache (token t sees positions 0..pos+t); its
  // combine stages the output for O where it is whole 256-blocks
  const bool o256 = nq % 256 == 0;
  if ((rc = launch_attention(q, L.k_cache, L.v_cache, pos, M, c.n_head, c.n_kv_head, c.head_dim, c.max_ctx, w.chunk,
                             w.nsplit, part_o, part_ml, o, nullptr, st,
                             o256 ? static_cast<uint8_t*>(stage) : nullptr)) != NT_OK)
    return rc;
  // 3. h = x + Wo o
  {
    JobM job;
    const uint8_t* W[1] = {u8(L.wo.data)};
    const int fmt[1] = {L.wo.fmt};
    const int rows[1] = {c.hidden};
    if ((rc = plan_job_m(job, 1, W, fmt, rows, nq, 0, 0, M)) != NT_OK) return rc;
    if (!o256 && (rc = launch_stage_m(o, nq, nullptr, 0.f, M, nq, stage, st)) != NT_OK) return rc;
    EpiArgs ea{};
    ea.y = x;
    ea.ld = c.hidden;
    RedArgs ra;  // h staged for gate/up, times ffn_norm
    if (h256) {
      ra.st_stage = stage;
      ra.st_gain = L.ffn_norm;
      ra.st_ss = ss;
    }
    if ((rc = launch_gemm_m(job, stage, part, none, EPI_RESID, ea, st, ra)) != NT_OK) return rc;
  }
  // 4. a = silu(Wg hn) * (Wu hn), hn = RMSNorm(h)
  {
    JobM job;
    const uint8_t* W[2] = {u8(L.wg.data), u8(L.wu.data)};
    const int fmt[2] = {L.wg.fmt, L.wu.fmt};
    const int rows[2] = {c.ffn, c.ffn};
    if ((rc = plan_job_m(job, 2, W, fmt, rows, c.hidden, 1, 0, M)) != NT_OK) return rc;
    if (!h256 && (rc = launch_stage_m(x, c.hidden, L.ffn_norm, c.rms_eps, M, c.hidden, stage, st)) != NT_OK)
      return rc;
    EpiArgs ea{};
    ea.y = a;
    ea.ld = c.ffn;
    RedArgs ra = h256 ? rn_hidden : RedArgs{};
    if (f256) ra.st_stage = stage;  // a staged for down
    if ((rc = launch_gemm_m(job, stage, part, none, EPI_SWIGLU, ea, st, ra)) != NT_OK) return rc;
  }
  // 5. x = h + Wd a
  {
    JobM job;
    const uint8_t* W[1] = {u8(L.wd.data)};
    const int fmt[1] = {L.wd.fmt};
    const int rows[1] = {c.hidden};
    if ((rc = plan_job_m(job, 1, W, fmt, rows, c.ffn, 0, 0, M)) != NT_OK) return rc;
    if (!f256 && (rc = launch_stage_m(a, c.ffn, nullptr, 0.f, M, c.ffn, stage, st)) != NT_OK) return rc;
    EpiArgs ea{};
    ea.y = x;
    ea.ld = c.hidden;
    ea.err = err;  // NaN out when a position was out of range
    RedArgs ra;  // the output staged for the next normalizing launch
    const bool out = ls && ls->next_gain && h256;
    if (out) {
      ra.st_stage = stage;
      ra.st_gain = ls->next_gain;
      ra.st_ss = ss;
    }
    if ((rc = launch_gemm_m(job, stage, part, none, EPI_RESID, ea, st, ra)) != NT_OK) return rc;
    if (out) ls->out_staged = true;
  }
  return NT_OK;
}

// Up to this many tokens a layer runs the GEMV engine once per token rather
// than the small-M GEMM (the two tokens then come out bitwise as two decode
// steps), unless its matrices are all Q4_K / Q6_K: the small-M GEMM's paired
// and split forms for up to four tokens read the 70B-shaped Q4_K gate in
// ~44 us and the Q6_K down in ~56 us for every token at once, against 2 x
// 28.4 and 2 x 38 us for two engine passes.  For the LM head, whose single
// launch is long, the engine wins up to three tokens.
constexpr int kEngineLayerTokens = 2;
constexpr int kEngineHeadTokens = 3;

bool small_m_layer(const nt_layer& L, int M) {
  if (M > kEngineLayerTokens) return true;
  if (M < 2) return false;
  const nt_qmat* mats[7] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
  for (const nt_qmat* q : mats)
    if (q->fmt != NT_Q4_K && q->fmt != NT_Q6_K) return false;
  return true;
}

// How a layer hands its input and output on as quantized activations
// (qx_bytes(hidden) per token).
struct LayerQx {
  const uint8_t* x_in = nullptr;    // the layer's input times attn_norm, quantized by the launch before; or null
  uint8_t* x_out = nullptr;         // where the down projection quantizes the output for the next launch, or null
  const float* next_gain = nullptr; // the gains the next launch normalizes with (null: none)
  bool x_out_written = false;       // set when the down projection did write x_out
};

// The launches of one layer (arguments already validated).
int run_layer(const nt_layer_cfg& c, const nt_layer& L, float* x, int M, const int32_t* pos, uint8_t* ws,
              const LayerWs& w, hipStream_t st, LayerQx* lq = nullptr, LayerStM* ls = nullptr) {
  if (lq) lq->x_out_written = false;
  if (small_m_layer(L, M)) return run_layer_m(c, L, x, M, pos, ws, w, st, ls);
  if (ls) ls->out_staged = false;
  const int nq = c.n_head * c.head_dim, nkv = c.n_kv_head * c.head_dim;
  float* q = reinterpret_cast<float*>(ws + w.q);
  float* part_o = reinterpret_cast<float*>(ws + w.part_o);
  float* part_ml = reinterpret_cast<float*>(ws + w.part_ml);
  float* o = reinterpret_cast<float*>(ws + w.o);
  float* a = reinterpret_cast<float*>(ws + w.a);
  int* err = reinterpret_cast<int*>(ws + w.err);
  int rc;
  // 1. RMSNorm -> Q,K,V projections -> RoPE -> q, K/V append
  {
    Job job;
    const uint8_t* W[3] = {u8(L.wq.data), u8(L.wk.data), u8(L.wv.data)};
    const int fmt[3] = {L.wq.fmt, L.wk.fmt, L.wv.fmt};
    const int rows[3] = {nq, nkv, nkv};
    if ((rc = plan_job(job, 3, W, fmt, rows, c.hidden, 0, 1)) != NT_OK) return rc;
    for (int i = 0; i < M; ++i) {
      ProArgs pro{x + (int64_t)i * c.hidden, L.attn_norm, c.rms_eps, 0, c.head_dim, c.rope_theta, pos, i};
      if (lq && lq->x_in) {  // already normalized-and-quantized by the launch before
        pro.src = nullptr;
        pro.gain = nullptr;
        pro.qx = lq->x_in + (int64_t)i * qx_bytes(c.hidden);
        pro.qx_norm = 1;
      }
      EpiArgs ea{};
      ea.q_out = q + (int64_t)i * nq;
      ea.k_cache = L.k_cache;
      ea.v_cache = L.v_cache;
      ea.pos = pos;
      ea.err = err;
      ea.head_dim = c.head_dim;
      ea.max_ctx = c.max_ctx;
      ea.rope_theta = c.rope_theta;
      ea.q_rows = nq;
      ea.kv_rows = nkv;
      ea.pos_add = i;
      ea.n_tok = M;
      if ((rc = launch_gemv(job, pro, EPI_QKV, ea, st)) != NT_OK) return rc;
    }
  }
  // 2. attention over the cache (split over positions) and combine; the
  // combine also hands o on quantized (each of its workgroups is one block)
  const size_t qo = qx_bytes(nq), qh = qx_bytes(c.hidden), qa = qx_bytes(c.ffn);
  uint8_t* qx_o = qx_ok(nq) ? ws + w.qx_o : nullptr;
  if ((rc = launch_attention(q, L.k_cache, L.v_cache, pos, M, c.n_head, c.n_kv_head, c.head_dim, c.max_ctx, w.chunk,
                             w.nsplit, part_o, part_ml, o, qx_o, st)) != NT_OK)
    return rc;
  // O, gate/up and down hand their outputs on quantized where their rows
  // split into whole 32-row blocks per workgroup (Job::qblock)
  Job jo, jf, jd;
  {
    const uint8_t* W[1] = {u8(L.wo.data)};
    const int fmt[1] = {L.wo.fmt};
    const int rows[1] = {c.hidden};
    if ((rc = plan_job(jo, 1, W, fmt, rows, nq, 0, 0, 1)) != NT_OK) return rc;
  }
  {
    const uint8_t* W[2] = {u8(L.wg.data), u8(L.wu.data)};
    const int fmt[2] = {L.wg.fmt, L.wu.fmt};
    const int rows[2] = {c.ffn, c.ffn};
    if ((rc = plan_job(jf, 2, W, fmt, rows, c.hidden, 1, 0, 1)) != NT_OK) return rc;
  }
  {
    const uint8_t* W[1] = {u8(L.wd.data)};
    const int fmt[1] = {L.wd.fmt};
    const int rows[1] = {c.hidden};
    if ((rc = plan_job(jd, 1, W, fmt, rows, c.ffn, 0, 0, lq && lq->x_out ? 1 : 0)) != NT_OK) return rc;
  }
  for (int i = 0; i < M; ++i) {
    float* xi = x + (int64_t)i * c.hidden;
    // 3. h = x + Wo o
    {
      ProArgs pro{o + (int64_t)i * nq, nullptr, 0.f, 0, 0, 0.f, nullptr, 0};
      if (qx_o) {
        pro.src = nullptr;
        pro.qx = qx_o + i * qo;
      }
      EpiArgs ea{};
      ea.y = xi;
      if (jo.qblock) {
        ea.qx_out = ws + w.qx_h + i * qh;
        ea.qx_gain = L.ffn_norm;
      }
      if ((rc = launch_gemv(jo, pro, EPI_RESID, ea, st)) != NT_OK) return rc;
    }
    // 4. a = silu(Wg hn) * (Wu hn), hn = RMSNorm(h)
    {
      ProArgs pro{xi, L.ffn_norm, c.rms_eps, 0, 0, 0.f, nullptr, 0};
      if (jo.qblock) {
        pro.src = nullptr;
        pro.gain = nullptr;
        pro.qx = ws + w.qx_h + i * qh;
        pro.qx_norm = 1;
      }
      EpiArgs ea{};
      ea.y = a;
      if (jf.qblock) ea.qx_out = ws + w.qx_a + i * qa;
      if ((rc = launch_gemv(jf, pro, EPI_SWIGLU, ea, st)) != NT_OK) return rc;
    }
    // 5. x = h + Wd a
    {
      ProArgs pro{a, nullptr, 0.f, 0, 0, 0.f, nullptr, 0};
      if (jf.qblock) {
        pro.src = nullptr;
        pro.qx = ws + w.qx_a + i * qa;
      }
      EpiArgs ea{};
      ea.y = xi;
      ea.err = err;  // NaN out when a position was out of range
      if (jd.qblock) {
        ea.qx_out = lq->x_out + i * qh;
        ea.qx_gain = lq->next_gain;
      }
      if ((rc = launch_gemv(jd, pro, EPI_RESID, ea, st)) != NT_OK) return rc;
    }
  }
  if (lq) lq->x_out_written = jd.qblock != 0;
  return NT_OK;
}

// ---- decode step
struct StepWs {
  size_t x, x_in, qx_x, layer, logits, pv, pi, part_lm, total;
  LayerWs lw;
};

int64_t qmat_bytes(int fmt, int64_t rows, int64_t cols) {
  const int qk = block_elems(fmt);
  return qk ? rows * (cols / qk) * block_bytes(fmt) : 0;
}

// Seven matrices of a streamed layer, back to back, each padded to 256 B.
void blob_offsets(const nt_layer_cfg& c, const nt_layer& L, size_t (&off)[8]) {
  const int64_t nq = (int64_t)c.n_head * c.head_dim, nkv = (int64_t)c.n_kv_head * c.head_dim;
  const nt_qmat* m[7] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
  const int64_t rows[7] = {nq, nkv, nkv, c.hidden, c.ffn, c.ffn, c.hidden};
  const int64_t cols[7] = {c.hidden, c.hidden, c.hidden, nq, c.hidden, c.hidden, c.ffn};
  size_t o = 0;
  for (int i = 0; i < 7; ++i) {
    off[i] = o;
    o += up256((size_t)qmat_bytes(m[i]->fmt, rows[i], cols[i]));
  }
  off[7] = o;
}

StepWs step_ws(const nt_model& m, int M) {
  StepWs w{};
  w.lw = layer_ws(m.cfg, M);
  size_t off = 0;
  w.x = off; off += up256((size_t)M * m.cfg.hidden * 4);
  w.x_in = off; off += up256((size_t)m.cfg.hidden * 4);  // a layer's input, for the similarity of calibration
  w.qx_x = off; off += up256((size_t)M * qx_bytes(m.cfg.hidden));  // the next layer's input, quantized
  w.layer = off; off += w.lw.total;
  w.logits = off; off += up256((size_t)M * m.vocab * 4);
  w.pv = off; off += up256((size_t)M * 256 * 4);
  w.pi = off; off += up256((size_t)M * 256 * 4);
  if (M >= 2) {
    w.part_lm = off;
    off += up256(part_m_bytes(m.vocab, 0, m.cfg.hidden, M));
  }
  w.total = off;
  return w;
}

// Events of the streaming pipeline: one set per (device, staging buffer),
// made on first use and kept for the process.  Steps of models with
// different staging buffers can therefore run concurrently on different
// streams; steps that share staging buffers must not overlap (they share
// the buffers themselves).
struct StreamEvents {
  int dev = -1;
  const void* stage = nullptr;
  hipEvent_t ready[2] = {nullptr, nullptr};
  hipEvent_t freed[2] = {nullptr, nullptr};
};

std::mutex g_ev_mu;

StreamEvents* stream_events(const void* stage0) {
  static std::vector<StreamEvents*> sets;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_ev_mu);
  for (StreamEvents* e : sets)
    if (e->dev == dev && e->stage == stage0) return e;
  StreamEvents* e = new StreamEvents;
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(&e->ready[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&e->freed[i], hipEventDisableTiming) != hipSuccess) {
      delete e;
      return nullptr;
    }
  }
  e->dev = dev;
  e->stage = stage0;
  sets.push_back(e);
  return e;
}

// Test hook (nt_test_fail_stream_copy): the next streamed pass fails, with
// NT_EHIP, where it would issue the copy of this streamed layer (-1: off).
std::atomic<int> g_fail_copy{-1};

// Arguments of one pass through the stack beyond the model itself.
struct StepArgs {
  const uint8_t* skip2 = nullptr;  // extra skip flags [n_layer] (the draft of a speculative round) or null
  float* cos_acc = nullptr;        // per-layer similarity sums [n_layer] (M == 1) or null
};

// One pass (decode for M == 1, verify for M > 1).  With check_only, the
// arguments are validated and nothing is enqueued.
int run_step(const nt_model& m, const int32_t* tokens, int M, const int32_t* pos, int32_t* out, float* logits_user,
             void* ws_v, size_t ws_bytes, hipStream_t st, const StepArgs& sa = StepArgs(), bool check_only = false) {
  if (M < 1 || M > 8) return NT_EINVAL;
  if (!cfg_ok(m.cfg) || m.n_layer < 0 || m.vocab <= 0 || !tokens || !pos || !out || !ws_v) return NT_EINVAL;
  if (m.n_layer > 0 && !m.layers) return NT_EINVAL;
  if (sa.cos_acc && M != 1) return NT_EINVAL;
  if (!fmt_cols_ok(m.tok_emb.fmt, m.cfg.hidden) || !fmt_cols_ok(m.lm_head.fmt, m.cfg.hidden)) return NT_EINVAL;
  if (!m.tok_emb.data || !m.lm_head.data || !m.out_norm) return NT_EINVAL;
  if (block_elems(m.lm_head.fmt) == 1) return NT_EUNSUPPORTED;  // the LM head runs on the block-format engine
  if (!aligned16(m.lm_head.data) || !aligned16(m.out_norm) || !aligned16(ws_v)) return NT_EALIGN;
  if (!aligned16(m.tok_emb.data)) return NT_EALIGN;
  const int fs = m.first_streamed;
  if (fs < 0 || fs > m.n_layer) return NT_EINVAL;
  auto skipped = [&](int l) { return (m.skip && m.skip[l]) || (sa.skip2 && sa.skip2[l]); };
  // streamed layers that run, in order: the copy pipeline walks only these
  int ns = 0;
  for (int l = fs; l < m.n_layer; ++l) ns += !skipped(l);
  auto streamed_layer = [&](int j) {
    for (int l = fs; l < m.n_layer; ++l)
      if (!skipped(l) && j-- == 0) return l;
    return -1;
  };
  const bool streaming = ns > 0;
  const StepWs w = step_ws(m, M);
  if (ws_bytes < w.total) return NT_EWORKSPACE;
  size_t boff[8] = {0};
  for (int l = 0; l < m.n_layer; ++l) {
    if (skipped(l)) continue;
    nt_layer L = m.layers[l];
    if (l >= fs) {
      // streamed: matrix pointers come from the staging buffers
      blob_offsets(m.cfg, L, boff);
      if (!m.host_layer || !m.host_layer[l] || !m.stage[0] || !m.stage[1]) return NT_EINVAL;
      if (m.stage_bytes < boff[7]) return NT_EINVAL;
      if (!aligned16(m.stage[0]) || !aligned16(m.stage[1])) return NT_EALIGN;
      const nt_qmat* mats[7] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
      for (int i = 0; i < 7; ++i) const_cast<nt_qmat*>(mats[i])->data = m.stage[0];
    }
    const int rc = check_layer(m.cfg, L);
    if (rc != NT_OK) return rc;
  }
  if (check_only) return NT_OK;
  uint8_t* ws = static_cast<uint8_t*>(ws_v);
  float* x = reinterpret_cast<float*>(ws + w.x);
  float* x_in = reinterpret_cast<float*>(ws + w.x_in);
  float* logits = logits_user ? logits_user : reinterpret_cast<float*>(ws + w.logits);
  // the layers' status word (one for the whole step: every layer writes it
  // from the same position); the embedding clears it, so a step without
  // layers reports no error
  int* err = reinterpret_cast<int*>(ws + w.layer + w.lw.err);
  // Each launch hands the residual stream on to the next normalizing launch
  // as a quantized activation (times that launch's RMSNorm gains) where the
  // layers run the GEMV engine: the embedding to the first layer, each
  // layer's down projection to the next layer that runs, the last one to the
  // LM head (a layer that runs the small-M GEMM breaks the chain: the next
  // launch reads the fp32 stream).
  const bool qx_step = M <= kEngineLayerTokens && qx_ok(m.cfg.hidden);
  uint8_t* qx_x = ws + w.qx_x;
  auto gain_after = [&](int l) {  // the gains of the first launch after layer l that normalizes
    for (int k = l + 1; k < m.n_layer; ++k)
      if (!skipped(k)) return m.layers[k].attn_norm;
    return m.out_norm;
  };
  int rc = launch_embed(m.tok_emb.fmt, m.tok_emb.data, tokens, M, m.vocab, m.cfg.hidden, x, err,
                        qx_step ? qx_x : nullptr, qx_step ? gain_after(-1) : nullptr, st);
  if (rc != NT_OK) return rc;
  bool x_quantized = qx_step;
  bool x_staged = false;  // x staged for a small-M launch by the last layer (times the next gains)
  StreamEvents* ev = nullptr;
  hipStream_t cs = static_cast<hipStream_t>(m.copy_stream);
  auto issue_copy = [&](int j) -> int {
    // streamed layer j (0-based among the streamed layers that run) into stage[j % 2]
    const int l = streamed_layer(j), b = j & 1;
    int armed = j;
    if (g_fail_copy.load() == j && g_fail_copy.compare_exchange_strong(armed, -1)) return NT_EHIP;
    nt_layer L = m.layers[l];
    blob_offsets(m.cfg, L, boff);
    if (j >= 2 && hipStreamWaitEvent(cs, ev->freed[b], 0) != hipSuccess) return NT_EHIP;
    if (hipMemcpyAsync(m.stage[b], m.host_layer[l], boff[7], hipMemcpyHostToDevice, cs) != hipSuccess) return NT_EHIP;
    if (hipEventRecord(ev->ready[b], cs) != hipSuccess) return NT_EHIP;
    return NT_OK;
  };
  if (streaming) {
    if (!(ev = stream_events(m.stage[0]))) return NT_EHIP;
    // the copies may only start once everything queued before this step on
    // the compute stream (e.g. a previous step still reading the staging
    // buffers) is done
    if (hipEventRecord(ev->freed[0], st) != hipSuccess || hipStreamWaitEvent(cs, ev->freed[0], 0) != hipSuccess)
      return NT_EHIP;
    for (int j = 0; j < std::min(2, ns); ++j)
      if ((rc = issue_copy(j)) != NT_OK) return rc;
  }
  int j = 0;  // streamed layers run so far
  for (int l = 0; l < m.n_layer; ++l) {
    if (skipped(l)) continue;
    nt_layer L = m.layers[l];
    const int b = j & 1;
    if (l >= fs) {
      blob_offsets(m.cfg, L, boff);
      uint8_t* base = static_cast<uint8_t*>(m.stage[b]);
      L.wq.data = base + boff[0];
      L.wk.data = base + boff[1];
      L.wv.data = base + boff[2];
      L.wo.data = base + boff[3];
      L.wg.data = base + boff[4];
      L.wu.data = base + boff[5];
      L.wd.data = base + boff[6];
      if (hipStreamWaitEvent(st, ev->ready[b], 0) != hipSuccess) return NT_EHIP;
    }
    if (sa.cos_acc &&
        hipMemcpyAsync(x_in, x, (size_t)m.cfg.hidden * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return NT_EHIP;
    LayerQx lq;
    lq.x_in = x_quantized ? qx_x : nullptr;
    lq.x_out = qx_step ? qx_x : nullptr;
    lq.next_gain = gain_after(l);
    LayerStM lsm;
    lsm.in_staged = x_staged;
    lsm.next_gain = gain_after(l);
    if ((rc = run_layer(m.cfg, L, x, M, pos, ws + w.layer, w.lw, st, &lq, &lsm)) != NT_OK) return rc;
    x_quantized = lq.x_out_written;
    x_staged = lsm.out_staged;
    if (sa.cos_acc && (rc = launch_cos_acc(x_in, x, m.cfg.hidden, sa.cos_acc + l, st)) != NT_OK) return rc;
    if (l >= fs) {
      if (hipEventRecord(ev->freed[b], st) != hipSuccess) return NT_EHIP;
      if (j + 2 < ns && (rc = issue_copy(j + 2)) != NT_OK) return rc;
      ++j;
    }
  }
  // final RMSNorm -> LM head -> argmax
  const uint8_t* Wl[1] = {u8(m.lm_head.data)};
  const int fmtl[1] = {m.lm_head.fmt};
  const int rowsl[1] = {m.vocab};
  if (M > kEngineHeadTokens) {
    JobM jm;
    if ((rc = plan_job_m(jm, 1, Wl, fmtl, rowsl, m.cfg.hidden, 0, 0, M)) != NT_OK) return rc;
    void* stage = ws + w.layer + w.lw.stage;
    RedArgs ra;
    if (x_staged) {  // by the last layer, times out_norm
      ra.rn_ss = reinterpret_cast<const float*>(ws + w.layer + w.lw.ss);
      ra.rn_nb = m.cfg.hidden / 256;
      ra.rn_cols = m.cfg.hidden;
      ra.rn_eps = m.cfg.rms_eps;
    } else if ((rc = launch_stage_m(x, m.cfg.hidden, m.out_norm, m.cfg.rms_eps, M, m.cfg.hidden, stage, st)) !=
               NT_OK) {
      return rc;
    }
    const ProArgs none{nullptr, nullptr, 0.f, 0, 0, 0.f, nullptr, 0};
    EpiArgs ea{};
    ea.y = logits;
    ea.ld = m.vocab;
    if ((rc = launch_gemm_m(jm, stage, ws + w.part_lm, none, EPI_STORE, ea, st, ra)) != NT_OK) return rc;
  } else {
    Job jl;
    if ((rc = plan_job(jl, 1, Wl, fmtl, rowsl, m.cfg.hidden, 0, 0)) != NT_OK) return rc;
    for (int i = 0; i < M; ++i) {
      ProArgs pro{x + (int64_t)i * m.cfg.hidden, m.out_norm, m.cfg.rms_eps, 0, 0, 0.f, nullptr, 0};
      if (x_quantized) {
        pro.src = nullptr;
        pro.gain = nullptr;
        pro.qx = qx_x + (int64_t)i * qx_bytes(m.cfg.hidden);
        pro.qx_norm = 1;
      }
      EpiArgs ea{};
      ea.y = logits + (int64_t)i * m.vocab;
      if ((rc = launch_gemv(jl, pro, EPI_STORE, ea, st)) != NT_OK) return rc;
    }
  }
  return launch_argmax(logits, M, m.vocab, reinterpret_cast<float*>(ws + w.pv), reinterpret_cast<int*>(ws + w.pi), err,
                       out, st);
}

// Workspace of a speculative round: one pass's workspace (the draft steps
// and the verify pass run one after the other in it), then the drafted
// tokens, the verified tokens and the draft positions.
struct SpecWs {
  size_t d, a, posj, total;
};

SpecWs spec_ws(const nt_model& m, int K) {
  SpecWs s{};
  size_t off = std::max(step_ws(m, 1).total, step_ws(m, K + 1).total);
  s.d = off; off += 256;
  s.a = off; off += 256;
  s.posj = off; off += 256;
  s.total = off;
  return s;
}

// Workspace of nt_decode_step_noalloc: a file-scope device array, so that
// callers that cannot allocate (graph capture, tight serving loops) need no
// buffer of their own.  Each device that runs the entry point holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels and copies take the address that
// hipGetSymbolAddress gives, kept per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};

// The device address of `scratch` on the current device (looked up once per
// device, with that device current); null if the lookup fails.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_dev[dev] = p;
  }
  return g_scratch_dev[dev];
}

}  // namespace

extern "C" {

int nt_block_elems(int fmt) { return block_elems(fmt); }
int nt_block_bytes(int fmt) { return block_bytes(fmt); }

int64_t nt_row_bytes(int fmt, int64_t cols) {
  const int qk = block_elems(fmt);
  if (qk == 0 || cols < 0 || cols % qk != 0) return 0;
  return cols / qk * block_bytes(fmt);
}

int64_t nt_max_cols(void) { return kMaxCols; }

const char* nt_status_str(int status) {
  switch (status) {
    case NT_OK: return "ok";
    case NT_EINVAL: return "invalid argument";
    case NT_EALIGN: return "pointer not 16-byte aligned";
    case NT_EWORKSPACE: return "workspace too small";
    case NT_EHIP: return "HIP launch or copy failed";
    case NT_EUNSUPPORTED: return "shape not supported";
  }
  return "unknown status";
}

int nt_gemv_q(int fmt, const void* W, const float* x, float* y, int64_t rows, int64_t cols, void* stream) {
  const int qk = block_elems(fmt);
  if (qk == 0 || rows < 0 || cols <= 0 || cols % qk != 0) return NT_EINVAL;
  if (rows > INT32_MAX) return NT_EUNSUPPORTED;
  if (cols > kMaxCols) return NT_EUNSUPPORTED;
  if (rows == 0) return NT_OK;
  if (!W || !x || !y) return NT_EINVAL;
  if (!aligned16(W) || !aligned16(x)) return NT_EALIGN;
  if (qk == 1) {  // F16 / F32: rows of 16-byte loads
    if ((cols * block_bytes(fmt)) % 16 != 0) return NT_EINVAL;
    return launch_gemv_f(fmt, W, x, y, 1, (int)rows, (int)cols, static_cast<hipStream_t>(stream));
  }
  Job job;
  const uint8_t* Wp = static_cast<const uint8_t*>(W);
  const int r = (int)rows;
  int rc = plan_job(job, 1, &Wp, &fmt, &r, (int)cols, 0, 0);
  if (rc != NT_OK) return rc;
  ProArgs pro{x, nullptr, 0.f, 0, 0, 0.f, nullptr, 0};
  EpiArgs ea{};
  ea.y = y;
  return launch_gemv(job, pro, EPI_STORE, ea, static_cast<hipStream_t>(stream));
}

size_t nt_gemm_q_small_workspace_bytes(int M, int64_t rows, int64_t cols) {
  if (M < 2 || M > 8 || rows <= 0 || cols <= 0 || cols > kMaxCols || rows > INT32_MAX / 16) return 0;
  return up256(stage_m_bytes((int)cols)) + up256(part_m_bytes(rows, 0, (int)cols, M));
}

int nt_gemm_q_small(int fmt, const void* W, const float* X, float* Y, int M, int64_t rows, int64_t cols, void* ws,
                    size_t ws_bytes, void* stream) {
  if (M < 1 || M > 8) return NT_EINVAL;
  const int qk = block_elems(fmt);
  if (qk == 0 || rows < 0 || cols <= 0 || cols % qk != 0) return NT_EINVAL;
  if (rows > INT32_MAX / 16 || cols > kMaxCols) return NT_EUNSUPPORTED;
  if (rows == 0) return NT_OK;
  if (!W || !X || !Y) return NT_EINVAL;
  if (!aligned16(W) || !aligned16(X) || (M > 1 && (cols * 4) % 16 != 0)) return NT_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (qk == 1) {  // F16 / F32: no staging, no workspace
    if ((cols * block_bytes(fmt)) % 16 != 0) return NT_EINVAL;
    return launch_gemv_f(fmt, W, X, Y, M, (int)rows, (int)cols, st);
  }
  const uint8_t* Wp = static_cast<const uint8_t*>(W);
  const int r = (int)rows;
  int rc;
  if (M == 1) {
    Job job;
    if ((rc = plan_job(job, 1, &Wp, &fmt, &r, (int)cols, 0, 0)) != NT_OK) return rc;
    ProArgs pro{X, nullptr, 0.f, 0, 0, 0.f, nullptr, 0};
    EpiArgs ea{};
    ea.y = Y;
    return launch_gemv(job, pro, EPI_STORE, ea, st);
  }
  if (!ws) return NT_EINVAL;
  if (!aligned16(ws)) return NT_EALIGN;
  if (ws_bytes < nt_gemm_q_small_workspace_bytes(M, rows, cols)) return NT_EWORKSPACE;
  JobM job;
  if ((rc = plan_job_m(job, 1, &Wp, &fmt, &r, (int)cols, 0, 0, M)) != NT_OK) return rc;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  void* stage = wsb;
  void* part = wsb + up256(stage_m_bytes((int)cols));
  if ((rc = launch_stage_m(X, cols, nullptr, 0.f, M, (int)cols, stage, st)) != NT_OK) return rc;
  const ProArgs none{nullptr, nullptr, 0.f, 0, 0, 0.f, nullptr, 0};
  EpiArgs ea{};
  ea.y = Y;
  ea.ld = rows;
  return launch_gemm_m(job, stage, part, none, EPI_STORE, ea, st);
}

size_t nt_layer_workspace_bytes(const nt_layer_cfg* cfg, int M) {
  if (!cfg || !cfg_ok(*cfg) || M < 1 || M > 8) return 0;
  return layer_ws(*cfg, M).total;
}

int nt_decode_layer(const nt_layer_cfg* cfg, const nt_layer* layer, float* x, int M, const int32_t* pos_dev,
                    void* ws, size_t ws_bytes, void* stream) {
  if (!cfg || !layer || !x || !pos_dev || !ws) return NT_EINVAL;
  if (M < 1 || M > 8 || !cfg_ok(*cfg)) return NT_EINVAL;
  int rc = check_layer(*cfg, *layer);
  if (rc != NT_OK) return rc;
  if (!aligned16(x) || !aligned16(ws)) return NT_EALIGN;
  const LayerWs w = layer_ws(*cfg, M);
  if (ws_bytes < w.total) return NT_EWORKSPACE;
  return run_layer(*cfg, *layer, x, M, pos_dev, static_cast<uint8_t*>(ws), w, static_cast<hipStream_t>(stream));
}

size_t nt_step_workspace_bytes(const nt_model* model, int M) {
  if (!model || !cfg_ok(model->cfg) || M < 1 || M > 8 || model->vocab <= 0) return 0;
  return step_ws(*model, M).total;
}

size_t nt_layer_blob_bytes(const nt_layer_cfg* cfg, const nt_layer* fmts_only) {
  if (!cfg || !fmts_only || !cfg_ok(*cfg)) return 0;
  size_t off[8];
  blob_offsets(*cfg, *fmts_only, off);
  return off[7];
}

int nt_decode_step(const nt_model* model, const int32_t* token_dev, const int32_t* pos_dev, int32_t* next_token_dev,
                   float* logits_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!model) return NT_EINVAL;
  return run_step(*model, token_dev, 1, pos_dev, next_token_dev, logits_dev, ws, ws_bytes,
                  static_cast<hipStream_t>(stream));
}

size_t nt_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

int nt_decode_step_noalloc(const nt_model* model, const int32_t* token_dev, const int32_t* pos_dev,
                           int32_t* next_token_dev, float* logits_dev, void* stream) {
  if (!model) return NT_EINVAL;
  // streamed layers need the pipeline's events, which are made on first use
  if (model->first_streamed != model->n_layer) return NT_EUNSUPPORTED;
  const size_t need = nt_step_workspace_bytes(model, 1);
  if (need == 0) return NT_EINVAL;
  if (need > kScratchBytes) return NT_EWORKSPACE;
  // validate everything before the first call on a device looks the array up
  int rc = run_step(*model, token_dev, 1, pos_dev, next_token_dev, logits_dev, reinterpret_cast<void*>(256), need,
                    nullptr, StepArgs(), true);
  if (rc != NT_OK) return rc;
  void* ws = scratch_ptr();
  if (!ws) return NT_EHIP;
  return run_step(*model, token_dev, 1, pos_dev, next_token_dev, logits_dev, ws, kScratchBytes,
                  static_cast<hipStream_t>(stream));
}

int nt_verify_step(const nt_model* model, const int32_t* tokens_dev, int M, const int32_t* pos_dev,
                   int32_t* argmax_dev, float* logits_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!model) return NT_EINVAL;
  return run_step(*model, tokens_dev, M, pos_dev, argmax_dev, logits_dev, ws, ws_bytes,
                  static_cast<hipStream_t>(stream));
}

int nt_calibrate_step(const nt_model* model, const int32_t* token_dev, const int32_t* pos_dev,
                      int32_t* next_token_dev, float* cos_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!model || !cos_dev) return NT_EINVAL;
  StepArgs sa;
  sa.cos_acc = cos_dev;
  return run_step(*model, token_dev, 1, pos_dev, next_token_dev, nullptr, ws, ws_bytes,
                  static_cast<hipStream_t>(stream), sa);
}

int nt_test_fail_stream_copy(int j) {
  if (j < -1) return NT_EINVAL;
  g_fail_copy.store(j);
  return NT_OK;
}

int nt_select_skip(const float* score, int n_layer, int n_skip, int first, int last, uint8_t* mask) {
  if (!score || !mask || n_layer < 0 || first < 0 || first > last || last > n_layer || n_skip < 0 ||
      n_skip > last - first)
    return NT_EINVAL;
  for (int l = first; l < last; ++l)
    if (score[l] != score[l]) return NT_EINVAL;  // NaN
  for (int l = 0; l < n_layer; ++l) mask[l] = 0;
  for (int k = 0; k < n_skip; ++k) {
    int best = -1;
    for (int l = first; l < last; ++l)
      if (!mask[l] && (best < 0 || score[l] > score[best])) best = l;
    mask[best] = 1;
  }
  return NT_OK;
}

int nt_plan_tiers(const nt_model* model, int M, size_t device_budget, size_t host_budget, nt_tier_plan* plan) {
  if (!model || !plan || M < 1 || M > 8) return NT_EINVAL;
  const nt_model& m = *model;
  if (!cfg_ok(m.cfg) || m.n_layer < 0 || m.vocab <= 0 || (m.n_layer > 0 && !m.layers)) return NT_EINVAL;
  const nt_layer_cfg& c = m.cfg;
  if (!fmt_cols_ok(m.tok_emb.fmt, c.hidden) || !fmt_cols_ok(m.lm_head.fmt, c.hidden)) return NT_EINVAL;
  const int n = m.n_layer;
  std::vector<size_t> blob(n);
  for (int l = 0; l < n; ++l) {
    const nt_layer& L = m.layers[l];
    const int64_t nq = (int64_t)c.n_head * c.head_dim;
    const nt_qmat* mats[7] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
    const int64_t cols[7] = {c.hidden, c.hidden, c.hidden, nq, c.hidden, c.hidden, c.ffn};
    for (int i = 0; i < 7; ++i)
      if (!fmt_cols_ok(mats[i]->fmt, cols[i]) || block_elems(mats[i]->fmt) == 1) return NT_EINVAL;
    size_t off[8];
    blob_offsets(c, L, off);
    blob[l] = off[7];
  }
  // what every placement keeps on the device
  const size_t gains = up256((size_t)c.hidden * 4);
  const size_t kv = up256((size_t)c.n_kv_head * c.max_ctx * c.head_dim * 2);
  size_t fixed = up256((size_t)qmat_bytes(m.tok_emb.fmt, m.vocab, c.hidden)) +
                 up256((size_t)qmat_bytes(m.lm_head.fmt, m.vocab, c.hidden)) + gains;
  fixed += (size_t)n * (2 * gains + 2 * kv);
  fixed += M == 1 ? step_ws(m, 1).total : spec_ws(m, M - 1).total;
  // streamed suffix sums and their largest blob, for every first_streamed k
  std::vector<size_t> host(n + 1, 0), stage(n + 1, 0);
  for (int k = n - 1; k >= 0; --k) {
    host[k] = host[k + 1] + blob[k];
    stage[k] = std::max(stage[k + 1], blob[k]);
  }
  size_t resident = 0;
  for (int l = 0; l < n; ++l) resident += blob[l];
  int best = -1;
  nt_tier_plan p{};
  for (int k = n; k >= 0; --k) {
    if (k < n) resident -= blob[k];
    p.first_streamed = k;
    p.n_streamed = n - k;
    p.fixed_bytes = fixed;
    p.resident_bytes = resident;
    p.stage_bytes = stage[k];
    p.device_bytes = fixed + resident + 2 * stage[k];
    p.host_bytes = host[k];
    if (p.device_bytes <= device_budget && p.host_bytes <= host_budget) {
      best = k;
      break;
    }
  }
  *plan = p;
  return best >= 0 ? NT_OK : NT_EUNSUPPORTED;
}

size_t nt_spec_workspace_bytes(const nt_model* model, int K) {
  if (!model || K < 1 || K > 7 || !cfg_ok(model->cfg)) return 0;
  return spec_ws(*model, K).total;
}

int nt_spec_step(const nt_model* model, const uint8_t* draft_skip, int K, int32_t* cur_dev, int32_t* pos_dev,
                 int32_t* out_dev, int32_t* n_out_dev, void* ws_v, size_t ws_bytes, void* stream) {
  if (!model || K < 1 || K > 7 || !cur_dev || !pos_dev || !out_dev || !n_out_dev || !ws_v) return NT_EINVAL;
  if (!cfg_ok(model->cfg)) return NT_EINVAL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const SpecWs s = spec_ws(*model, K);
  if (ws_bytes < s.total) return NT_EWORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(ws_v);
  int32_t* d = reinterpret_cast<int32_t*>(ws + s.d);
  int32_t* a = reinterpret_cast<int32_t*>(ws + s.a);
  int32_t* posj = reinterpret_cast<int32_t*>(ws + s.posj);
  StepArgs draft;
  draft.skip2 = draft_skip;
  // validate both kinds of pass before anything is enqueued
  int rc = run_step(*model, d, 1, posj, d + 1, nullptr, ws, ws_bytes, st, draft, true);
  if (rc != NT_OK) return rc;
  if ((rc = run_step(*model, d, K + 1, pos_dev, a, nullptr, ws, ws_bytes, st, StepArgs(), true)) != NT_OK) return rc;
  if ((rc = launch_spec_init(cur_dev, pos_dev, K, d, posj, st)) != NT_OK) return rc;
  for (int j = 0; j < K; ++j)
    if ((rc = run_step(*model, d + j, 1, posj + j, d + j + 1, nullptr, ws, ws_bytes, st, draft)) != NT_OK) return rc;
  if ((rc = run_step(*model, d, K + 1, pos_dev, a, nullptr, ws, ws_bytes, st)) != NT_OK) return rc;
  return launch_spec_accept(d, a, K, cur_dev, pos_dev, out_dev, n_out_dev, st);
}

}  // extern "C"
