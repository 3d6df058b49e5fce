// Internal declarations shared by the HIP translation units of libnt.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nt.h"

namespace nt {

constexpr int kMaxWaves = 12;     // waves per workgroup of the GEMV engine
constexpr int kMaxThreads = 64 * kMaxWaves;
constexpr int kSlab = 8192;       // bytes of one wave's LDS staging slab
constexpr int kSlabLoads = kSlab / (64 * 16);  // 16-B loads per lane to fill a slab
constexpr int kSegMax = kSlab - 32;            // weight bytes of one segment, at most
constexpr int kMaxMats = 3;       // matrices one engine launch walks (Q, K, V)
constexpr int64_t kMaxCols = 49152;

__host__ __device__ inline int block_elems(int fmt) { return fmt == NT_Q4_K || fmt == NT_Q6_K ? 256 : (fmt == NT_Q8_0 || fmt == NT_Q4_0 ? 32 : 0); }
__host__ __device__ inline int block_bytes(int fmt) {
  switch (fmt) {
    case NT_Q8_0: return 34;
    case NT_Q4_0: return 18;
    case NT_Q4_K: return 144;
    case NT_Q6_K: return 210;
  }
  return 0;
}

// How a launch of the GEMV engine walks its matrices.  The work is a list of
// items; an item is one row, an adjacent row pair of one matrix (`pairs`:
// RoPE needs both rows), or row r of W[0] and of W[1] (`paired`: SwiGLU
// needs gate and up).  Each wave takes a contiguous range of items and
// streams their rows, in segments of at most kSegMax bytes, through its own
// LDS slab.  All matrices share `cols`.
struct Job {
  const uint8_t* W[kMaxMats];
  int64_t rb[kMaxMats];       // bytes per row
  int fmt[kMaxMats];
  int rows[kMaxMats];
  int row_base[kMaxMats];     // first output row of each matrix (concatenated outputs)
  int item_start[kMaxMats + 1];
  int seg_blocks[kMaxMats];   // blocks per segment
  int nseg[kMaxMats];         // segments per row
  int nmat;
  int paired;
  int pairs;
  int cols;
  int nwaves;                 // waves per workgroup
  // dynamic LDS layout (byte offsets)
  uint32_t x_hi, x_lo, x_sc, x_sum, red, slab;
  uint32_t lds_bytes;
};

// Activation source of the engine prologue.
struct ProArgs {
  const float* src;    // fp32 [cols] (per token: + m * src_stride)
  const float* gain;   // RMSNorm gains or nullptr
  float eps;
  int64_t src_stride;
};

enum Epi : int {
  EPI_STORE = 0,   // y[r] = acc
  EPI_RESID = 1,   // y[r] += acc              (residual add, in place)
  EPI_QKV = 2,     // RoPE + q store + f16 K/V append
  EPI_SWIGLU = 3,  // y[r] = silu(acc_gate) * acc_up
};

struct EpiArgs {
  float* y;            // EPI_STORE / EPI_RESID / EPI_SWIGLU output
  // EPI_QKV
  float* q_out;        // fp32 [n_head*head_dim]
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* pos;
  int* err;            // set to 1 when pos is out of range
  int head_dim;
  int max_ctx;
  float rope_theta;
  int q_rows;          // n_head*head_dim
  int kv_rows;         // n_kv_head*head_dim
  int pos_add;         // this token sits at *pos + pos_add
};

// Planner: fills job geometry for `nmat` matrices; returns NT_OK or an error.
int plan_job(Job& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
             int pairs);

// Launch the engine (prologue: optional RMSNorm; epilogue: epi).
int launch_gemv(const Job& job, const ProArgs& pro, int epi, const EpiArgs& ea, hipStream_t stream);

// Attention and step kernels (nt_attn.hip).
void attn_plan(int n_kv, int max_ctx, int& chunk, int& nsplit);
int launch_attention(const float* q, const uint16_t* kc, const uint16_t* vc, const int32_t* pos, int n_query,
                     int n_head, int n_kv, int head_dim, int max_ctx, int chunk, int nsplit, float* part_o,
                     float* part_ml, float* o, hipStream_t stream);
int launch_embed(int fmt, const void* E, const int32_t* tokens, int M, int vocab, int cols, float* x,
                 hipStream_t stream);
int argmax_parts(int n);
int launch_argmax(const float* logits, int M, int n, float* pv, int* pi, int32_t* out, hipStream_t stream);

}  // namespace nt
