// nt_spec.hip -- small step kernels of layer-skip calibration and of
// self-speculative decoding (ntransformer pages, p1 feature list: layer skip
// by cosine similarity; self-speculative decoding with the layers resident in
// GPU memory as the draft model).  The heavy work of both (the decode steps
// and the verify pass) runs in the GEMV, small-M GEMM and attention kernels.
#include "nt_internal.h"

namespace nt {
namespace {

constexpr int kCosThreads = 256;

// acc[0] += a.b / (|a| |b|) over n floats, sums in fp64 (one workgroup).
__global__ __launch_bounds__(kCosThreads) void k_cos_acc(const float* __restrict__ a, const float* __restrict__ b,
                                                         int n, float* __restrict__ acc) {
  __shared__ double s_ab[kCosThreads], s_aa[kCosThreads], s_bb[kCosThreads];
  const int t = threadIdx.x;
  double ab = 0.0, aa = 0.0, bb = 0.0;
  for (int i = t; i < n; i += kCosThreads) {
    const double x = a[i], y = b[i];
    ab += x * y;
    aa += x * x;
    bb += y * y;
  }
  s_ab[t] = ab;
  s_aa[t] = aa;
  s_bb[t] = bb;
  __syncthreads();
  for (int w = kCosThreads / 2; w > 0; w >>= 1) {
    if (t < w) {
      s_ab[t] += s_ab[t + w];
      s_aa[t] += s_aa[t + w];
      s_bb[t] += s_bb[t + w];
    }
    __syncthreads();
  }
  if (t == 0) acc[0] += (float)(s_ab[0] / (sqrt(s_aa[0]) * sqrt(s_bb[0])));
}

// Start of a speculative round: d[0] = *cur and posj[j] = *pos + j for j <= K.
__global__ void k_spec_init(const int32_t* __restrict__ cur, const int32_t* __restrict__ pos, int K,
                            int32_t* __restrict__ d, int32_t* __restrict__ posj) {
  const int t = threadIdx.x;
  if (t <= K) posj[t] = *pos + t;
  if (t == 0) d[0] = *cur;
}

// End of a speculative round: accept the drafted tokens d[1..K] while they
// equal the verify pass's greedy tokens a[0..K-1]; emit a[0..n].
__global__ void k_spec_accept(const int32_t* __restrict__ d, const int32_t* __restrict__ a, int K,
                              int32_t* __restrict__ cur, int32_t* __restrict__ pos, int32_t* __restrict__ out,
                              int32_t* __restrict__ n_out) {
  if (threadIdx.x != 0) return;
  if (a[0] < 0) {
    // the verify pass met a position out of range: nothing is emitted and
    // the position and current token stay
    for (int i = 0; i <= K; ++i) out[i] = -1;
    *n_out = 0;
    return;
  }
  int n = 0;
  while (n < K && d[n + 1] == a[n]) ++n;
  for (int i = 0; i <= K; ++i) out[i] = i <= n ? a[i] : -1;
  *n_out = n + 1;
  *pos += n + 1;
  *cur = a[n];
}

}  // namespace

int launch_cos_acc(const float* a, const float* b, int n, float* acc, hipStream_t st) {
  hipLaunchKernelGGL(k_cos_acc, dim3(1), dim3(kCosThreads), 0, st, a, b, n, acc);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

int launch_spec_init(const int32_t* cur, const int32_t* pos, int K, int32_t* d, int32_t* posj, hipStream_t st) {
  if (K < 1 || K > 63) return NT_EINVAL;
  hipLaunchKernelGGL(k_spec_init, dim3(1), dim3(64), 0, st, cur, pos, K, d, posj);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

int launch_spec_accept(const int32_t* d, const int32_t* a, int K, int32_t* cur, int32_t* pos, int32_t* out,
                       int32_t* n_out, hipStream_t st) {
  if (K < 1 || K > 63) return NT_EINVAL;
  hipLaunchKernelGGL(k_spec_accept, dim3(1), dim3(64), 0, st, d, a, K, cur, pos, out, n_out);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

}  // namespace nt
