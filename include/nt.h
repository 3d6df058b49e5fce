/*
 * nt.h -- C ABI of libnt, a gfx950 (MI355X) library for batch-1 decode of a
 * Llama decoder whose projections are block-quantized GGUF tensors.
 *
 * What the library computes comes from the ntransformer pages:
 *   p1  = "Ntransformer" (unwiki summary page)
 *   p2  = "ntransformer - moteur d'inference NVMe-to-GPU ..." (GeekNews FR)
 * The pages list the weight formats (p1 "About"; p2 "Presentation de
 * NTransformer"), the Llama pieces RoPE, GQA, SwiGLU, RMSNorm and the KV cache
 * (p1 feature list; p2 "Fonctionnalites principales"), the per-token kernels
 * GEMV, RMSNorm, RoPE, SwiGLU and softmax plus a sampler (p2 "Architecture et
 * structure du code"), the F16 KV cache (p1 roadmap phase 3), self-speculative
 * decoding (p1 feature list) and the double-buffered layer streaming (p1
 * "SLEP streaming"; p2 "Streaming direct NVMe").  A public C API is only
 * planned there (p1 roadmap phase 5); the calls below are this library's.
 *
 * Conventions for every call:
 *  - Ownership: the caller allocates and owns every buffer (device memory for
 *    weights, activations, caches and workspace; pinned host memory for
 *    streamed layers).  The library never allocates, frees or synchronizes.
 *  - Streams: `stream` / `copy_stream` are hipStream_t values passed as void*.
 *    NULL means the default stream.  Every call only enqueues work.
 *  - Errors: arguments are validated before anything is enqueued; a negative
 *    nt_status is returned and nothing runs.  A failed launch returns
 *    NT_EHIP.  Faults inside kernels surface at the caller's next sync.
 *    The decode position lives in device memory (so a captured graph can be
 *    replayed), so a position out of range (pos < 0 or pos + M > max_ctx)
 *    can only be seen on the device: the kernels then leave the KV cache
 *    untouched and skip attention, the residual stream x of a layer call
 *    comes out NaN, and a step writes -1 as its token (see each call).
 *  - Alignment: weight matrices, activation vectors and workspaces must be
 *    16-byte aligned (NT_EALIGN otherwise).
 *  - Calls are re-entrant, except the tracing calls (nt_trace_*), which are
 *    per process; concurrent calls on different streams must not share
 *    output, cache, workspace or staging buffers.  The streaming pipeline
 *    keeps one set of HIP events per staging buffer, so steps of models
 *    with different staging buffers may run concurrently.
 */
#ifndef NT_H
#define NT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nt_status {
  NT_OK = 0,
  NT_EINVAL = -1,       /* bad argument: unknown format, bad size, NULL pointer */
  NT_EALIGN = -2,       /* a pointer is not 16-byte aligned                     */
  NT_EWORKSPACE = -3,   /* workspace smaller than the *_workspace_bytes query   */
  NT_EHIP = -4,         /* a HIP launch or copy failed                          */
  NT_EUNSUPPORTED = -5  /* shape outside what the kernels handle (see limits)   */
} nt_status;

/* GGUF weight formats (p1 "About" format list).  Byte layouts:
 *   NT_Q8_0  34 B / 32 weights : f16 d, int8 q[32];          w = d*q
 *   NT_Q4_0  18 B / 32 weights : f16 d, u8 qs[16];           w = d*(q-8),
 *            q of element j<16 = low nibble of qs[j], of j+16 = high nibble.
 *   NT_Q4_K 144 B / 256 weights: f16 d, f16 dmin, u8 scales[12], u8 qs[128];
 *            8 sub-blocks of 32 with 6-bit scale sc and min m (GGUF packing),
 *            w = d*sc*q - dmin*m; chunk c (64 weights) uses qs[32c..32c+31],
 *            low nibbles first 32 weights, high nibbles next 32.
 *   NT_Q6_K 210 B / 256 weights: u8 ql[128], u8 qh[64], int8 sc[16], f16 d;
 *            w_e = d*sc[e/16]*(q_e-32), q_e 6-bit from ql nibble + qh 2 bits
 *            (GGUF order).
 *   NT_Q5_K 176 B / 256 weights: f16 d, f16 dmin, u8 scales[12], u8 qh[32],
 *            u8 qs[128]; scales, mins and nibbles as NT_Q4_K, and the fifth
 *            bit of element l (< 32) of sub-block s is bit s of qh[l];
 *            q in 0..31, w = d*sc*q - dmin*m.
 *   NT_F16    2 B / weight: IEEE binary16.    NT_F32  4 B / weight: binary32.
 * A matrix is `rows` consecutive rows, each cols/QK consecutive blocks.
 * NT_F16 and NT_F32 are GEMV/small-M formats (nt_gemv_q, nt_gemm_q_small)
 * and embedding rows; decoder layers and the LM head take the block formats. */
typedef enum nt_fmt {
  NT_Q8_0 = 0, NT_Q4_0 = 1, NT_Q4_K = 2, NT_Q6_K = 3, NT_Q5_K = 4, NT_F16 = 5, NT_F32 = 6
} nt_fmt;

/* Weights per block (32, 256, or 1 for F16/F32), 0 for an unknown format. */
int nt_block_elems(int fmt);
/* Bytes per block (34, 18, 144, 210, 176, 2, 4), 0 for an unknown format. */
int nt_block_bytes(int fmt);
/* Bytes of one row of `cols` weights; 0 if fmt is unknown or cols % QK != 0. */
int64_t nt_row_bytes(int fmt, int64_t cols);
/* Static text for a status code. */
const char* nt_status_str(int status);
/* Largest `cols` a GEMV accepts (the activation vector is staged on chip). */
int64_t nt_max_cols(void);

/*
 * y = W x (GEMV on quantized weights; p2 "Architecture et structure du code").
 *   W: device, fmt blocks, rows x cols, 16-byte aligned.
 *   x: device fp32 [cols], 16-byte aligned.   y: device fp32 [rows], overwritten.
 *   cols must be a positive multiple of the format's QK and <= nt_max_cols()
 *   (F16: a multiple of 8, F32: of 4, so rows are whole 16-byte loads).
 *   rows == 0 is a no-op.  For the block formats x is held inside the kernel
 *   as 16-bit fixed point per 32-element block (relative error of y about
 *   1e-5); F16/F32 weights multiply x in fp32.
 */
int nt_gemv_q(int fmt, const void* W, const float* x, float* y, int64_t rows, int64_t cols, void* stream);

/*
 * Workspace bytes nt_gemm_q_small needs for 2 <= M <= 8 tokens (0 for other
 * M or an unsupported shape; M == 1 needs none).
 */
size_t nt_gemm_q_small_workspace_bytes(int M, int64_t rows, int64_t cols);

/*
 * Y[m] = W X[m] for M tokens (the verify pass of self-speculative decoding
 * runs M drafted tokens through every projection in one pass; p1 "Features").
 *   X: device fp32 [M][cols], rows 16-byte aligned; Y: device fp32 [M][rows],
 *   overwritten; 1 <= M <= 8.  The weights are read once for all M tokens:
 *   int8 MFMA tiles over the same 16-bit fixed-point activation as nt_gemv_q
 *   (M == 1 is nt_gemv_q).  F16/F32 weights: one fp32 stream over the rows,
 *   no workspace (ws may be NULL).
 *   ws: device workspace of ws_bytes >= nt_gemm_q_small_workspace_bytes(M,
 *   rows, cols), 16-byte aligned (may be NULL when M == 1); its contents need
 *   no initialisation.  Calls that share a workspace must not overlap.
 */
int nt_gemm_q_small(int fmt, const void* W, const float* X, float* Y, int M, int64_t rows, int64_t cols, void* ws,
                    size_t ws_bytes, void* stream);

/* Shape of one Llama decoder layer. */
typedef struct nt_layer_cfg {
  int32_t hidden;     /* model width                                   */
  int32_t n_head;     /* query heads                                   */
  int32_t n_kv_head;  /* key/value heads (GQA: n_head % n_kv_head == 0) */
  int32_t head_dim;   /* even, <= 256                                  */
  int32_t ffn;        /* SwiGLU inner width                            */
  int32_t max_ctx;    /* capacity of the KV cache in positions         */
  float rope_theta;   /* RoPE base                                     */
  float rms_eps;      /* RMSNorm epsilon                               */
} nt_layer_cfg;

/* A quantized matrix: format and device pointer to its blocks. */
typedef struct nt_qmat {
  int32_t fmt;
  const void* data;
} nt_qmat;

/* Device pointers of one layer.  Matrix shapes (rows x cols):
 *   wq [n_head*head_dim x hidden], wk/wv [n_kv_head*head_dim x hidden],
 *   wo [hidden x n_head*head_dim], wg/wu [ffn x hidden], wd [hidden x ffn].
 * k_cache / v_cache: f16 bits [n_kv_head][max_ctx][head_dim]. */
typedef struct nt_layer {
  const float* attn_norm; /* RMSNorm gains before attention [hidden] */
  const float* ffn_norm;  /* RMSNorm gains before the FFN   [hidden] */
  nt_qmat wq, wk, wv, wo, wg, wu, wd;
  uint16_t* k_cache;
  uint16_t* v_cache;
} nt_layer;

/* Workspace bytes nt_decode_layer needs for M tokens (0 on bad cfg). */
size_t nt_layer_workspace_bytes(const nt_layer_cfg* cfg, int M);

/*
 * One pre-norm Llama decoder layer for M tokens at positions pos..pos+M-1
 * (p1 feature list: RoPE, GQA, SwiGLU, RMSNorm, KV cache):
 *   xn = RMSNorm(x, attn_norm); q,k,v = Wq xn, Wk xn, Wv xn; RoPE(q, k);
 *   K,V[pos+i] = f16(k_i), f16(v_i); token i attends to 0..pos+i;
 *   h = x + Wo o;  x <- h + Wd (silu(Wg hn) * Wu hn),  hn = RMSNorm(h, ffn_norm).
 *   cfg/layer: host structs (copied at the call); layer's pointers are device.
 *   x: device fp32 [M][hidden], updated in place.
 *   pos_dev: device int32 holding pos (read by the kernels, so a captured
 *            graph can be replayed with a new position); if pos < 0 or
 *            pos + M > max_ctx no token writes the cache, attention is
 *            skipped and every row of x comes out as NaN.
 *   ws: device workspace of ws_bytes >= nt_layer_workspace_bytes(cfg, M);
 *       its contents need no initialisation.  Calls that share a workspace
 *       must not overlap.
 * The call does not advance pos.
 */
int nt_decode_layer(const nt_layer_cfg* cfg, const nt_layer* layer, float* x, int M, const int32_t* pos_dev,
                    void* ws, size_t ws_bytes, void* stream);

/* A whole decoder stack. */
typedef struct nt_model {
  nt_layer_cfg cfg;
  int32_t n_layer;
  int32_t vocab;
  nt_qmat tok_emb;          /* [vocab x hidden] embedding rows             */
  nt_qmat lm_head;          /* [vocab x hidden]                            */
  const float* out_norm;    /* final RMSNorm gains [hidden]                */
  const nt_layer* layers;   /* host array of n_layer layers                */
  /* Layer streaming (p1 "SLEP streaming"): layers >= first_streamed keep
   * their seven matrices in pinned host memory and are copied, one layer at
   * a time, into two device staging buffers on copy_stream while the
   * previous layer computes.  first_streamed == n_layer disables it. */
  int32_t first_streamed;
  const void* const* host_layer; /* [n_layer] pinned blob of layer i's matrices
                                    (wq,wk,wv,wo,wg,wu,wd back to back, each
                                    padded to 256 B), used for i >= first_streamed */
  void* stage[2];                /* device staging buffers                   */
  size_t stage_bytes;            /* bytes of each staging buffer             */
  void* copy_stream;             /* hipStream_t for the copies               */
  /* Layer skip (p1 feature list; p1 roadmap phase 3): NULL, or a host array
   * of n_layer flags.  A layer with skip[i] != 0 is not run (and, when
   * streamed, not copied): the residual stream passes it unchanged.
   * nt_calibrate_step and nt_select_skip choose the layers. */
  const uint8_t* skip;
} nt_model;

/* Workspace bytes nt_decode_step / nt_verify_step need for M tokens. */
size_t nt_step_workspace_bytes(const nt_model* model, int M);

/* Bytes of a streamed layer blob (the sum of its seven padded matrices). */
size_t nt_layer_blob_bytes(const nt_layer_cfg* cfg, const nt_layer* fmts_only);

/*
 * One greedy decode step of the whole stack (p1 "About": a Llama 70B model
 * run token by token; p1 "Llama architecture support" and p2 "Architecture
 * et structure du code": the model composed of attention, FFN and
 * normalisation, with a sampler and an engine on top):
 *   embedding row of *token_dev -> n_layer layers at *pos_dev (nt_decode_layer
 *   with M = 1; layers >= first_streamed streamed, flagged layers skipped) ->
 *   final RMSNorm (out_norm) -> LM head -> argmax (lowest index on ties)
 *   written to *next_token_dev.
 *   token_dev, pos_dev: device int32, read by the kernels (the token is
 *     clamped to [0, vocab)); they live on the device so the step can be
 *     captured in a graph and replayed.  The call does not advance pos.
 *   next_token_dev: device int32; -1 when the position is out of range
 *     (pos < 0 or pos >= max_ctx; the caches are then left untouched).
 *   logits_dev: device fp32 [vocab] or NULL.
 *   ws: device workspace of ws_bytes >= nt_step_workspace_bytes(model, 1),
 *     16-byte aligned, no initialisation needed; steps sharing it must not
 *     overlap.
 * Errors as for every call (validated before anything is enqueued:
 * NT_EINVAL, NT_EALIGN, NT_EWORKSPACE, NT_EUNSUPPORTED; NT_EHIP on a failed
 * launch or copy).
 */
int nt_decode_step(const nt_model* model, const int32_t* token_dev, const int32_t* pos_dev,
                   int32_t* next_token_dev, float* logits_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * nt_decode_step for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step with no ws argument.  Its workspace is a file-scope device array of
 * nt_decode_step_noalloc_max_bytes() bytes (32 MiB) that each device holds
 * from the first call until the process ends; the call itself allocates
 * nothing.  Arguments, results and errors are nt_decode_step's, plus:
 *   NT_EWORKSPACE when nt_step_workspace_bytes(model, 1) exceeds the array
 *     (e.g. a 70B-shaped model with max_ctx beyond ~60000 positions);
 *   NT_EUNSUPPORTED for a model with streamed layers (first_streamed <
 *     n_layer: the pipeline makes HIP events on first use);
 *   NT_EHIP if the array's device address cannot be looked up.
 * Every call on one device shares that device's array: calls that overlap
 * on one device (different streams or host threads) race and must not be
 * made.  The array's contents are left from the last call; the step needs
 * none of them.
 */
int nt_decode_step_noalloc(const nt_model* model, const int32_t* token_dev, const int32_t* pos_dev,
                           int32_t* next_token_dev, float* logits_dev, void* stream);
size_t nt_decode_step_noalloc_max_bytes(void);

/*
 * Verify pass of self-speculative decoding (p1 "About" and feature list:
 * self-speculative decoding with the resident layers as the draft model;
 * p2 "Fonctionnalites principales"; the drafted tokens are checked by one
 * pass of the whole model): M (1..8) tokens at positions pos..pos+M-1
 * through the whole stack in one pass, token i attending to 0..pos+i;
 * argmax_dev[i] (device int32 [M]) is the greedy token after token i, or -1
 * for every i when pos < 0 or pos + M > max_ctx.  tokens_dev: device int32
 * [M].  logits_dev (fp32 [M][vocab]) may be NULL.  ws: ws_bytes >=
 * nt_step_workspace_bytes(model, M).  Ownership, errors and pos as
 * nt_decode_step.  M == 1 is nt_decode_step.
 */
int nt_verify_step(const nt_model* model, const int32_t* tokens_dev, int M, const int32_t* pos_dev,
                   int32_t* argmax_dev, float* logits_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * Calibration of layer skip (p1 feature list: the skipped layers are chosen by
 * cosine similarity): one nt_decode_step that also adds, for every layer l
 * that runs, the cosine similarity of the residual stream entering layer l
 * and leaving it, x_in . x_out / (|x_in| |x_out|) (fp64 sums, added as fp32),
 * to cos_dev[l].  cos_dev: device fp32 [n_layer]; the caller zeroes it before
 * the first calibration token, so that after T tokens cos_dev[l] / T is the
 * layer's mean similarity.  Entries of skipped layers are not touched.  Other
 * arguments as nt_decode_step (same workspace size); with the position out
 * of range the token is -1 and NaN is added.
 */
int nt_calibrate_step(const nt_model* model, const int32_t* token_dev, const int32_t* pos_dev,
                      int32_t* next_token_dev, float* cos_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * Host helper choosing the layers to skip: mask[l] = 1 for the n_skip layers
 * l in [first, last) with the largest score[l] (a layer whose output is most
 * like its input changes the stream least), picked one at a time with the
 * lower index first among equal scores; mask[l] = 0 elsewhere.  score and
 * mask are host arrays of n_layer entries.  NT_EINVAL unless
 * 0 <= first <= last <= n_layer and 0 <= n_skip <= last - first, or if a score
 * in [first, last) is NaN.  No GPU work.
 */
int nt_select_skip(const float* score, int n_layer, int n_skip, int first, int last, uint8_t* mask);

/*
 * Tier placement (p1 "3-Tier Adaptive Caching": layers resident in GPU memory
 * need no I/O, layers in pinned RAM need a host-to-device copy per pass, and
 * the split is made automatically; p1 notes that Q4_K_M fits 36 layers of a
 * 70B model in 24 GB where the larger format fits 26).  The NVMe/mmap tier is
 * not part of this library.
 *
 * nt_plan_tiers picks the largest prefix of layers whose weights stay in
 * device memory within `device_budget` bytes, next to what every placement
 * keeps on the device; the rest are streamed from pinned host memory through
 * two staging buffers (nt_model.first_streamed, stage, stage_bytes).  Byte
 * counts (each buffer rounded up to 256 B):
 *   fixed    = embedding + LM head + final gains + every layer's two gains and
 *              K/V caches (cfg.max_ctx positions) + workspace (nt_decode_step
 *              for M == 1; nt_spec_step with K = M - 1 for M >= 2, which also
 *              covers nt_verify_step with M tokens);
 *   resident = nt_layer_blob_bytes of the layers below first_streamed;
 *   stage    = the largest nt_layer_blob_bytes among the streamed layers;
 *   device   = fixed + resident + 2 * stage  (<= device_budget);
 *   host     = nt_layer_blob_bytes summed over the streamed layers, the bytes
 *              copied per pass (<= host_budget; pass SIZE_MAX for no limit).
 * The largest first_streamed in 0..n_layer meeting both limits is chosen
 * (n_layer: nothing streamed, stage 0).  Skip flags are not considered.
 *   model: host struct; only cfg, n_layer, vocab, the formats of tok_emb and
 *          lm_head and the formats of layers[] are read (pointers may be NULL).
 *   M: tokens per pass the workspace must hold, 1..8.
 * Returns NT_EINVAL for a bad model or M, NT_EUNSUPPORTED when no placement
 * meets the limits (*plan then describes first_streamed = 0).  No GPU work.
 */
typedef struct nt_tier_plan {
  int32_t first_streamed;   /* layers [0, first_streamed) resident            */
  int32_t n_streamed;       /* n_layer - first_streamed                       */
  uint64_t fixed_bytes;     /* device bytes every placement needs             */
  uint64_t resident_bytes;  /* weights of the resident layers                 */
  uint64_t stage_bytes;     /* bytes of each of the two staging buffers       */
  uint64_t device_bytes;    /* fixed + resident + 2 * stage                   */
  uint64_t host_bytes;      /* pinned bytes of the streamed layers (per pass) */
} nt_tier_plan;
int nt_plan_tiers(const nt_model* model, int M, size_t device_budget, size_t host_budget, nt_tier_plan* plan);

/* Workspace bytes nt_spec_step needs for K draft tokens (0 if K is outside 1..7). */
size_t nt_spec_workspace_bytes(const nt_model* model, int K);

/*
 * One round of self-speculative greedy decoding (p1 feature list: the layers
 * resident in GPU memory serve as the draft model, with no second model):
 *   1. draft: K (1..7) greedy decode steps of the stack without the layers
 *      flagged in draft_skip (host [n_layer] flags, typically the streamed
 *      layers; NULL drafts with the whole stack): d_0 = *cur_dev and d_{j+1}
 *      is the draft's greedy token after d_j at position *pos_dev + j;
 *   2. verify: the whole stack (model->skip still applies) on d_0..d_K at
 *      positions pos..pos+K in one pass (nt_verify_step, M = K + 1), giving
 *      the greedy tokens a_0..a_K;
 *   3. accept: n is the number of leading j < K with d_{j+1} == a_j; the
 *      round emits a_0..a_n: out_dev[0..n] (out_dev[n+1..K] = -1),
 *      *n_out_dev = n + 1, *pos_dev += n + 1, *cur_dev = a_n.
 * The emitted tokens are the ones plain greedy decoding of the stack gives
 * (the draft only sets how many come per round).  Cache entries past the new
 * position are stale and get overwritten before anything reads them.
 * cur_dev, pos_dev, out_dev ([K + 1]) and n_out_dev are device int32; the
 * state stays on the device, so rounds can be queued back to back.
 * ws: nt_spec_workspace_bytes(model, K).  The draft steps and the verify pass
 * must fit the cache: pos + K + 1 <= max_ctx.  Otherwise the round emits
 * nothing: out_dev[0..K] = -1, *n_out_dev = 0, and pos and cur stay.
 */
int nt_spec_step(const nt_model* model, const uint8_t* draft_skip, int K, int32_t* cur_dev, int32_t* pos_dev,
                 int32_t* out_dev, int32_t* n_out_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * Instrumentation.  nt_trace_begin(kind) makes the library time every
 * following launch of one kernel kind (up to 16384 launches) with a pair of
 * HIP events that the runtime stamps with the kernel's own start and end on
 * the launch stream (hipExtLaunchKernel); nt_trace_end waits for those events
 * and returns the number of launches traced and their summed duration in
 * milliseconds (*total_ms).  Kinds: 0 plain GEMV, 1 GEMV + residual add (O
 * and down projections), 2 QKV + RoPE + KV append, 3 gate/up + SwiGLU,
 * 4 attention (the first split launch's start to the combine's end).
 * nt_trace_begin_every(kind, k) records only launches 0, k, 2k, ... of the
 * kind (k >= 1).  Tracing is per process and not thread safe, and is for
 * eager launches: a traced launch made under HIP stream capture is not
 * supported (end tracing before capturing).
 */
typedef enum nt_trace_kind {
  NT_TRACE_GEMV = 0,
  NT_TRACE_GEMV_RESID = 1,
  NT_TRACE_QKV = 2,
  NT_TRACE_FFN_UP = 3,
  NT_TRACE_ATTN = 4
} nt_trace_kind;
int nt_trace_begin(int kind);
int nt_trace_begin_every(int kind, int every);
int nt_trace_end(int* launches, double* total_ms);

/*
 * Test hook for the streaming pipeline's failure path: the next streamed
 * pass (nt_decode_step, nt_verify_step, nt_calibrate_step or a pass of
 * nt_spec_step) returns NT_EHIP where it would issue the copy of its j-th
 * streamed layer (0-based among the streamed layers that run), as if that
 * copy had failed; the hook then disarms itself.  Work already enqueued
 * (the layers before it) still runs, writing only cache entries at the
 * pass's own positions, so the caller repeats the pass at the same position.
 * j == -1 disarms.  NT_EINVAL for j < -1.  Per process; no GPU work.
 */
int nt_test_fail_stream_copy(int j);

/*
 * Measurement aid: a pure streaming read of `bytes` (a multiple of 16) from
 * the 16-byte aligned device buffer `buf`, with non-temporal 16-byte loads,
 * eight in flight per lane and 12 waves per CU; a checksum goes to the device
 * word *out.  Its time gives the achievable HBM read bandwidth.
 */
int nt_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NT_H */
