// Internal declarations shared by the HIP translation units of libnt.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nt.h"

namespace nt {

constexpr int kMaxThreads = 512;  // threads per workgroup of the GEMV engine
constexpr int kLpwMax = 8;        // 16-B loads per lane per tile, at most
constexpr int kMaxMats = 3;       // matrices one engine launch walks (Q, K, V)
constexpr int64_t kMaxCols = 49152;

inline int block_elems(int fmt) { return fmt == NT_Q4_K || fmt == NT_Q6_K ? 256 : (fmt == NT_Q8_0 || fmt == NT_Q4_0 ? 32 : 0); }
inline int block_bytes(int fmt) {
  switch (fmt) {
    case NT_Q8_0: return 34;
    case NT_Q4_0: return 18;
    case NT_Q4_K: return 144;
    case NT_Q6_K: return 210;
  }
  return 0;
}

// How a launch of the GEMV engine walks its matrices.  Tiles are groups of
// consecutive rows of one matrix (or, when `paired`, the same rows of W[0]
// and W[1]).  All matrices share `cols`.
struct TileJob {
  const uint8_t* W[kMaxMats];
  int64_t rb[kMaxMats];       // bytes per row
  int fmt[kMaxMats];
  int rows[kMaxMats];
  int tile_rows[kMaxMats];    // rows per tile (1, 2 or a multiple of the wave count)
  int tile_start[kMaxMats + 1];
  int row_base[kMaxMats];     // first output row of each matrix (concatenated outputs)
  int nmat;
  int paired;
  int cols;
  int lpw;                    // 16-B loads per lane per tile
  int nthreads;               // workgroup size (256 or 512)
  // dynamic LDS layout (byte offsets)
  uint32_t tile_cap;          // tile buffer bytes = lpw * nthreads * 16
  uint32_t x_hi, x_lo, x_sc, x_sum, ypart, red;
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
};

// Planner: fills job geometry for `nmat` matrices; returns NT_OK or an error.
int plan_job(TileJob& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
             int rope_pairs);

// Launch the engine (prologue: optional RMSNorm; epilogue: epi).
int launch_gemv(const TileJob& job, const ProArgs& pro, int epi, const EpiArgs& ea, hipStream_t stream);

}  // namespace nt
