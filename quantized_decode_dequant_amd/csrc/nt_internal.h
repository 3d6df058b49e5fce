// Internal declarations shared by the HIP translation units of libnt.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nt.h"

namespace nt {

constexpr int kMaxWaves = 16;     // waves per workgroup of the GEMV engine (one workgroup per CU)
constexpr int kMaxThreads = 64 * kMaxWaves;
constexpr int kFmtK46 = -2;  // kernel variant for launches that mix only Q4_K and Q6_K matrices
constexpr int kUnitsPerLane = 1;  // 64-weight column units a lane owns in one column slice
constexpr int kSliceUnits = 64 * kUnitsPerLane;  // column units per slice (4096 weights)
constexpr int kSlabLoads = 5;     // 16-B loads per lane for the largest segment (Q8_0: 4352 B + alignment)
constexpr int kSlab = kSlabLoads * 64 * 16;  // bytes of one wave's LDS staging slab
constexpr int kAccFloats = 4096;  // per-workgroup table of (row, slice) partial sums, in floats
constexpr int kMaxMats = 3;       // matrices one engine launch walks (Q, K, V)
constexpr int64_t kMaxCols = 49152;

__host__ __device__ inline int block_elems(int fmt) {
  switch (fmt) {
    case NT_Q8_0: case NT_Q4_0: return 32;
    case NT_Q4_K: case NT_Q5_K: case NT_Q6_K: return 256;
    case NT_F16: case NT_F32: return 1;
  }
  return 0;
}
__host__ __device__ inline int block_bytes(int fmt) {
  switch (fmt) {
    case NT_Q8_0: return 34;
    case NT_Q4_0: return 18;
    case NT_Q4_K: return 144;
    case NT_Q6_K: return 210;
    case NT_Q5_K: return 176;
    case NT_F16: return 2;
    case NT_F32: return 4;
  }
  return 0;
}

// How a launch of the GEMV engine walks its matrices.
//  - Columns are cut into `nslice` slices of `ups` 64-weight units; a lane
//    owns unit `lane` of the current slice and keeps its staged activation
//    in registers.
//  - Output rows are the matrices' rows one after the other (`nmat` <= 3,
//    e.g. Q, K, V), or, with `paired`, the rows of W[0] each together with
//    the same row of W[1] (SwiGLU needs gate and up).  With `pairs`, rows
//    are handed out in even-aligned pairs (RoPE rotates adjacent rows).
//  - Workgroup b owns output rows (or row pairs) b, b + G, b + 2G, ... of
//    the G workgroups.  Its work is the list of segments (one row of one
//    matrix within one column slice: a contiguous byte range), slice-major;
//    its waves claim segments two at a time from a counter in LDS, so waves
//    that the SIMD arbiter favours take more and all finish together.  Each segment's dot product lands in an
//    LDS table of (row, slice) partial sums; after a workgroup barrier the
//    epilogue adds the slices in order (deterministic) and writes the rows.
struct Job {
  const uint8_t* W[kMaxMats];
  int64_t rb[kMaxMats];       // bytes per row
  int fmt[kMaxMats];
  int rows[kMaxMats];
  int row_base[kMaxMats];     // first output row of each matrix (concatenated outputs)
  int64_t slice_bytes[kMaxMats];  // bytes of one full column slice of a row
  int64_t last_bytes[kMaxMats];   // bytes of the last column slice of a row
  int orows;                  // output rows
  int unit;                   // rows are handed to workgroups in multiples of this (2 with pairs)
  int ups;                    // units per slice
  int nslice;
  int last_units;             // units of the last slice (may be partial)
  int last_ne;                // weights of the last slice
  int nmat;
  int paired;
  int pairs;
  int cols;
  int nwaves;                 // waves per workgroup
  int grid;                   // workgroups
  int wg_base, wg_rem;        // workgroup b owns wg_base (+1 if b < wg_rem) units of `unit` output rows
  uint32_t magic[2];          // floor((2^32-1)/nv) for the two segment-row counts nv of a workgroup
  int lpl;                    // 16-B loads per lane per segment (3, 4 or 5)
  // With qblock, workgroup b's rows are one contiguous range of whole
  // 32-row blocks (unit == 32), so its epilogue can quantize its outputs
  // into the activation layout the next launch copies (EpiArgs::qx_out).
  int qblock;
  // dynamic LDS layout (byte offsets); the staged activation is laid out as
  // a quantized activation in memory (x_hi .. x_ss, see qx_bytes)
  uint32_t x_hi, x_lo, x_sc, x_sum, x_ss, red, slab, acc, ctl, rope, qo;
  uint32_t lds_bytes;
};

// A quantized activation of n values (n a multiple of 32), as launches hand
// it to each other: per 32-block a scale s = max|v| / 32639 and integers
// X = rint(v / s), split X = 256 hi + lo into two int8 planes; v is the
// vector times its RMSNorm gains where the consumer normalizes, and the
// block's sum of squares of the unscaled vector is kept for the
// normalization factor.  Bytes: hi [n], lo [n], s (f32) [n/32], sums of X
// over 16 values (i32) [n/16], sums of squares (f32) [n/32].  Launches copy
// it with 16-byte loads, which needs n to be a multiple of 128.
__host__ __device__ inline size_t qx_bytes(int64_t n) { return (size_t)n * 5 / 2; }
__host__ __device__ inline size_t qx_lo_off(int64_t n) { return (size_t)n; }
__host__ __device__ inline size_t qx_sc_off(int64_t n) { return (size_t)n * 2; }
__host__ __device__ inline size_t qx_sum_off(int64_t n) { return (size_t)n * 2 + (size_t)n / 8; }
__host__ __device__ inline size_t qx_ss_off(int64_t n) { return (size_t)n * 2 + (size_t)n * 3 / 8; }
inline bool qx_ok(int64_t n) { return n > 0 && n % 128 == 0; }

// Activation source of the engine prologue.
struct ProArgs {
  const float* src;    // fp32 [cols] (per token: + m * src_stride)
  const float* gain;   // RMSNorm gains or nullptr
  float eps;
  int64_t src_stride;
  // RoPE table for the QKV epilogue (rope_hd == 0: none): cos/sin of
  // pos * theta^(-2i/rope_hd), i < rope_hd/2, pos = *pos + pos_add
  int rope_hd;
  float rope_theta;
  const int32_t* pos;
  int pos_add;
  // A quantized activation (see qx_bytes) to copy instead of src; with
  // qx_norm the launch applies RMSNorm through the stored sums of squares
  // (the gains are already in it).
  const uint8_t* qx;
  int qx_norm;
};

enum Epi : int {
  EPI_STORE = 0,   // y[r] = acc
  EPI_RESID = 1,   // y[r] += acc              (residual add, in place)
  EPI_QKV = 2,     // RoPE + q store + f16 K/V append
  EPI_SWIGLU = 3,  // y[r] = silu(acc_gate) * acc_up
  // EPI_STORE for a launch whose whole share is in flight at once (at most
  // two segments per wave) and has no RMSNorm: the weight loads are issued
  // right behind the activation's, without waiting for it
  EPI_STORE_BURST = 4,
};

struct EpiArgs {
  float* y;            // EPI_STORE / EPI_RESID / EPI_SWIGLU output
  int64_t ld;          // small-M GEMM: distance between the tokens' rows of y (or q_out)
  // EPI_QKV
  float* q_out;        // fp32 [n_head*head_dim]
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* pos;
  int* err;            // layer status word: EPI_QKV writes 1 when a position is out of range, else 0;
                       // an EPI_RESID launch given it writes NaN when it is set
  int head_dim;
  int max_ctx;
  float rope_theta;
  int q_rows;          // n_head*head_dim
  int kv_rows;         // n_kv_head*head_dim
  int pos_add;         // this token sits at *pos + pos_add
  int n_tok;           // tokens of the layer call (positions *pos .. *pos + n_tok - 1)
  // EPI_RESID / EPI_SWIGLU on a qblock launch: the outputs (times qx_gain,
  // when given) also go out as a quantized activation of orows values
  uint8_t* qx_out;
  const float* qx_gain;
};

// The engine's LDS starts with copies of its three argument structs, made
// by the first threads at the start: the epilogue reads its arguments from
// there (argument loads issued after the stream miss the scalar cache and
// each costs a memory round trip).
constexpr uint32_t lds_align16(size_t n) { return (uint32_t)((n + 15) & ~size_t(15)); }
constexpr uint32_t kLdsJob = 0;
constexpr uint32_t kLdsPro = kLdsJob + lds_align16(sizeof(Job));
constexpr uint32_t kLdsEpi = kLdsPro + lds_align16(sizeof(ProArgs));
constexpr uint32_t kArgsLds = kLdsEpi + lds_align16(sizeof(EpiArgs));
static_assert(kArgsLds <= 1024, "engine argument copies");
static_assert(sizeof(Job) % 4 == 0 && sizeof(ProArgs) % 4 == 0 && sizeof(EpiArgs) % 4 == 0, "copied as words");

// Planner: fills job geometry for `nmat` matrices; returns NT_OK or an error.
// With qblock, the shares are whole 32-row blocks when the rows split into
// enough of them to keep the chip busy (job.qblock says whether they do).
int plan_job(Job& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
             int pairs, int qblock = 0);

// Launch the engine (prologue: optional RMSNorm; epilogue: epi).
int launch_gemv(const Job& job, const ProArgs& pro, int epi, const EpiArgs& ea, hipStream_t stream);

// ---- small-M GEMM on int8 MFMA (nt_gemm.hip)
constexpr int kMaxTokens = 8;     // tokens of one small-M pass
constexpr int kTS = 256;          // columns per tile-slice (one K-quant superblock)
constexpr int kTileRows = 16;     // weight rows per MFMA tile
constexpr int kMaxTsPer = 8;      // tile-slices per column range (its staged activation is 40 KB of LDS)
constexpr int kAccM = 8192;       // per-workgroup (row, sub-range, token) table, in floats

// How one small-M launch walks its matrices.  Rows are cut into 16-row tiles
// (tiles of W[0], W[1], W[2] one after the other; with `paired`, W[0]'s tiles
// each with the same tile of W[1]) and columns into `nsup` ranges of `tsper`
// tile-slices.  Workgroup b works on range b / gps and a share of the tiles;
// it stages that range's activation in LDS and its waves claim units (one
// tile over `tsu` tile-slices) from an LDS counter.  Each workgroup writes
// per-range partial sums; a reduce launch adds the ranges and applies the
// epilogue.
struct JobM {
  const uint8_t* W[kMaxMats];
  int64_t rb[kMaxMats];       // bytes per row
  int fmt[kMaxMats];
  int rows[kMaxMats];
  int row_base[kMaxMats];     // first output row of each matrix (concatenated outputs)
  int tile_base[kMaxMats + 1];  // first tile of each matrix (paired: W[0] only)
  int tsb[kMaxMats];          // bytes of a full tile-slice row piece
  int P[kMaxMats];            // 16-B chunks per row piece (worst alignment)
  uint32_t magicP[kMaxMats];  // ceil(65536 / P): chunk -> row by a multiply
  int nmat, paired, pairs, cols, M;
  int fast;                   // every matrix's rows are whole 16-byte chunks apart (fixed-offset tile loads)
  int bmode;                  // B tiles for M <= 4: 0 plain, 1 paired (Q4_K, Q6_K), 2 split (Q6_K)
  int orows;                  // output rows (paired: of each matrix)
  int nts;                    // tile-slices per row
  int tsper, nsup;            // tile-slices per column range, column ranges
  int tsu, nsub;              // tile-slices per unit, units per tile in a range
  int otiles;                 // output tiles
  int gps;                    // workgroups per column range
  int wg_base, wg_rem;        // tiles per workgroup of a range: wg_base (+1 if g < wg_rem)
  uint32_t magicV[2];         // floor((2^32-1)/nvt) for the two tile counts of a workgroup
  int nwaves, grid, lpl;
  const uint8_t* xb;          // staged activation in MFMA B layout [cols/32][64 lanes][8 B]
  const int4* xs;             // [cols/32][8 tokens]: per B column (hi plane, lo plane) the X sums of the
                              // block's two halves (zero on the hi plane)
  const float* xsc;           // [cols/256][8 tokens]: scale s of each 256-block
  float* part;                // partial sums [nsup][M][ldp]
  int64_t ldp;                // (paired ? 2 : 1) * orows
  uint32_t xbl, xsl, xscl, slab, scl, acc, ctl, lds_bytes;
};

int plan_job_m(JobM& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
               int pairs, int M);
size_t stage_m_bytes(int cols);          // bytes of the staged activation (B layout, X sums, scales)
// Bytes of the partial sums of a launch over `orows` output rows (paired: of
// each matrix) and `cols` columns; independent of the device.
size_t part_m_bytes(int64_t orows, int paired, int cols, int M);
// Stage M activation rows (optionally RMSNorm'ed) into `stage` (stage_m_bytes(cols) bytes).
int launch_stage_m(const float* src, int64_t stride, const float* gain, float eps, int M, int cols, void* stage,
                   hipStream_t stream);
// What the reduce launch of a small-M GEMM does besides its epilogue.
//  - rn_ss: the staged input carries its RMSNorm gains but not the factor:
//    the outputs are multiplied by r_t = 1 / sqrt(sum_b rn_ss[t rn_nb + b] /
//    rn_cols + rn_eps) (rn_ss: the input rows' sums of squares per
//    256-block, written by the launch that staged it).
//  - st_stage: the epilogue's outputs (EPI_STORE, EPI_RESID, EPI_SWIGLU),
//    times st_gain where given, also go out staged for the next small-M GEMM
//    (stage_m layout over orows columns; orows a multiple of 256), and with
//    st_ss their sums of squares per 256-block ([M][orows / 256]).
struct RedArgs {
  const float* rn_ss = nullptr;
  int rn_nb = 0, rn_cols = 0;
  float rn_eps = 0.f;
  void* st_stage = nullptr;
  const float* st_gain = nullptr;
  float* st_ss = nullptr;
};

// The GEMM over a staged activation into `part` (part_m_bytes), then the
// reduce and epilogue; `pro` supplies only the RoPE fields (rope_hd,
// rope_theta, pos) for EPI_QKV.
int launch_gemm_m(JobM& job, const void* stage, void* part, const ProArgs& pro, int epi, const EpiArgs& ea,
                  hipStream_t stream, const RedArgs& ra = RedArgs{});

// Launch tracing (nt_trace.hip): true when this launch of `kind` is
// recorded, with the events to hand to hipExtLaunchKernel (start: the first
// kernel of the launch, stop: its last); both null otherwise.
bool trace_events(int kind, hipEvent_t* start, hipEvent_t* stop);

// Attention and step kernels (nt_attn.hip).
void attn_plan(int head_dim, int max_ctx, int& chunk, int& nsplit);
// o [n_query][n_head * head_dim] fp32; with qx_o (may be null) each query's
// output also goes out as a quantized activation of n_head * head_dim values
// (qx_bytes apart per query); with stage_o (may be null; n_head * head_dim a
// multiple of 256, no qx_o) the outputs also go out staged for a small-M GEMM
// (stage_m_bytes(n_head * head_dim) bytes).
int launch_attention(const float* q, const uint16_t* kc, const uint16_t* vc, const int32_t* pos, int n_query,
                     int n_head, int n_kv, int head_dim, int max_ctx, int chunk, int nsplit, float* part_o,
                     float* part_ml, float* o, uint8_t* qx_o, hipStream_t stream, uint8_t* stage_o = nullptr);
// Embedding rows of tokens[0..M) into x; also clears the status word *err
// (may be null).  With qx (may be null) each row, times qx_gain, also goes
// out as a quantized activation (qx_bytes(cols) apart per token).
int launch_embed(int fmt, const void* E, const int32_t* tokens, int M, int vocab, int cols, float* x, int* err,
                 uint8_t* qx, const float* qx_gain, hipStream_t stream);
int argmax_parts(int n);
// Greedy tokens of M logit rows; -1 for every row when *err (may be null) is set.
int launch_argmax(const float* logits, int M, int n, float* pv, int* pi, const int* err, int32_t* out,
                  hipStream_t stream);

// F16 / F32 weights (nt_gemv_f.hip): Y[t][r] = W X[t] for M <= 8 tokens,
// Y rows `rows` apart; cols a multiple of 16 / element size, W and X 16-byte aligned.
int launch_gemv_f(int fmt, const void* W, const float* X, float* Y, int M, int rows, int cols, hipStream_t stream);

// Layer-skip calibration and speculative-round kernels (nt_spec.hip).
// acc[0] += cosine similarity of a and b (n floats).
int launch_cos_acc(const float* a, const float* b, int n, float* acc, hipStream_t stream);
// d[0] = *cur, posj[j] = *pos + j (j <= K).
int launch_spec_init(const int32_t* cur, const int32_t* pos, int K, int32_t* d, int32_t* posj, hipStream_t stream);
// Accept drafted d[1..K] against verified a[0..K]; emit, advance pos and cur.
int launch_spec_accept(const int32_t* d, const int32_t* a, int K, int32_t* cur, int32_t* pos, int32_t* out,
                       int32_t* n_out, hipStream_t stream);

}  // namespace nt
