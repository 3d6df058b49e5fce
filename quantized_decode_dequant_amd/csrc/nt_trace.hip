// nt_trace.hip -- optional event timing of one kernel kind (instrumentation
// for benchmarks: the measured durations come from HIP events on the stream
// the kernels are launched on).
#include <vector>

#include "nt_internal.h"

namespace nt {
namespace {

constexpr int kTraceCap = 4096;

struct Trace {
  int kind = -1;
  int n = 0;
  std::vector<hipEvent_t> start, stop;
};

Trace g_trace;

}  // namespace

void trace_before(int kind, hipStream_t stream) {
  if (kind != g_trace.kind || g_trace.n >= kTraceCap) return;
  (void)hipEventRecord(g_trace.start[g_trace.n], stream);
}

void trace_after(int kind, hipStream_t stream) {
  if (kind != g_trace.kind || g_trace.n >= kTraceCap) return;
  (void)hipEventRecord(g_trace.stop[g_trace.n], stream);
  ++g_trace.n;
}

}  // namespace nt

extern "C" {

int nt_trace_begin(int kind) {
  using nt::g_trace;
  if (kind < 0 || kind > NT_TRACE_ATTN) return NT_EINVAL;
  if (g_trace.start.empty()) {
    g_trace.start.resize(nt::kTraceCap);
    g_trace.stop.resize(nt::kTraceCap);
    for (int i = 0; i < nt::kTraceCap; ++i) {
      if (hipEventCreate(&g_trace.start[i]) != hipSuccess || hipEventCreate(&g_trace.stop[i]) != hipSuccess)
        return NT_EHIP;
    }
  }
  g_trace.kind = kind;
  g_trace.n = 0;
  return NT_OK;
}

int nt_trace_end(int* launches, double* total_ms) {
  using nt::g_trace;
  double tot = 0.0;
  for (int i = 0; i < g_trace.n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_trace.stop[i]) != hipSuccess) return NT_EHIP;
    if (hipEventElapsedTime(&ms, g_trace.start[i], g_trace.stop[i]) != hipSuccess) return NT_EHIP;
    tot += ms;
  }
  if (launches) *launches = g_trace.n;
  if (total_ms) *total_ms = tot;
  g_trace.kind = -1;
  g_trace.n = 0;
  return NT_OK;
}

}  // extern "C"
