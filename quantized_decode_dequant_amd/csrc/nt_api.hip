// nt_api.hip -- the extern "C" boundary of libnt: argument validation,
// launch planning and kernel launches.  No allocation, no synchronization.
#include <stdint.h>

#include "nt_internal.h"

using namespace nt;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

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
  TileJob job;
  const uint8_t* Wp = static_cast<const uint8_t*>(W);
  const int r = (int)rows;
  int rc = plan_job(job, 1, &Wp, &fmt, &r, (int)cols, 0, 0);
  if (rc != NT_OK) return rc;
  ProArgs pro{x, nullptr, 0.f, 0};
  EpiArgs ea{};
  ea.y = y;
  return launch_gemv(job, pro, EPI_STORE, ea, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- entry points not yet implemented in this file (filled in below as they land)
extern "C" {
int nt_gemm_q_small(int, const void*, const float*, float*, int, int64_t, int64_t, void*) { return NT_EUNSUPPORTED; }
size_t nt_layer_workspace_bytes(const nt_layer_cfg*, int) { return 0; }
int nt_decode_layer(const nt_layer_cfg*, const nt_layer*, float*, int, const int32_t*, void*, size_t, void*) {
  return NT_EUNSUPPORTED;
}
size_t nt_step_workspace_bytes(const nt_model*, int) { return 0; }
size_t nt_layer_blob_bytes(const nt_layer_cfg*, const nt_layer*) { return 0; }
int nt_decode_step(const nt_model*, const int32_t*, const int32_t*, int32_t*, float*, void*, size_t, void*) {
  return NT_EUNSUPPORTED;
}
int nt_verify_step(const nt_model*, const int32_t*, int, const int32_t*, int32_t*, float*, void*, size_t, void*) {
  return NT_EUNSUPPORTED;
}
}
