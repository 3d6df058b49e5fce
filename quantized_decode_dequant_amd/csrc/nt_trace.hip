// nt_trace.hip -- optional event timing of one kernel kind (instrumentation
// for benchmarks).  A recorded launch goes out through hipExtLaunchKernel
// with a pair of HIP events, which the runtime stamps with that dispatch's
// own start and end on the stream it runs on: the interval is the kernel's
// execution, without the queue's other packets or the gap before it.
#include <vector>

#include "nt_internal.h"

namespace nt {
namespace {

constexpr int kTraceCap = 16384;

struct Trace {
  int kind = -1;
  int n = 0;            // launches recorded
  int every = 1;        // record one launch in `every`
  int seen = 0;         // launches of the kind since trace_begin
  std::vector<hipEvent_t> start, stop;
};

Trace g_trace;

}  // namespace

bool trace_events(int kind, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (kind != g_trace.kind || g_trace.n >= kTraceCap) return false;
  if (g_trace.seen++ % g_trace.every != 0) return false;
  *start = g_trace.start[g_trace.n];
  *stop = g_trace.stop[g_trace.n];
  ++g_trace.n;
  return true;
}

}  // namespace nt

extern "C" {

int nt_trace_begin(int kind) { return nt_trace_begin_every(kind, 1); }

int nt_trace_begin_every(int kind, int every) {
  using nt::g_trace;
  if (kind < 0 || kind > NT_TRACE_ATTN || every < 1) return NT_EINVAL;
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
  g_trace.every = every;
  g_trace.seen = 0;
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

namespace nt {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4_t* gp_u32x4;

// Grid-stride over groups of 8 chunks per lane; all 8 loads issued before use.
__global__ __launch_bounds__(256) void k_read_probe(const uint8_t* buf, size_t n16, uint32_t* out) {
  const size_t tid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t nthr = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (size_t base = tid; base < n16; base += 8 * nthr) {
    u32x4_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const size_t c = base + i * nthr;
      v[i] = __builtin_nontemporal_load((gp_u32x4)(buf + 16 * (c < n16 ? c : base)));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (acc == 0x9E3779B9u) *out = acc;  // keeps the loads; practically never taken
}

}  // namespace
}  // namespace nt

extern "C" int nt_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out || bytes % 16 != 0) return NT_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return NT_EALIGN;
  if (bytes == 0) return NT_OK;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  hipLaunchKernelGGL(nt::k_read_probe, dim3(cus * 3), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}
