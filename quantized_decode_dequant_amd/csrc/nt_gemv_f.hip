// nt_gemv_f.hip -- GEMV and small-M GEMM on unquantized F16 / F32 weights
// (the pages' format list also names F16 and F32; p1 "About"):
// Y[t][r] = sum_k W[r][k] X[t][k] for t < M <= 8 tokens.
//
// The kernel is a plain stream: there is no block decode to amortise and no
// dense contraction worth a matrix core at M <= 8, so each wave owns two
// rows, its lanes read 16 consecutive bytes of each row per step (1 KB per
// row per wave-wide load, coalesced, non-temporal since weights are read
// once), and every lane multiplies them by the matching activation elements
// of every token, read through the caches (the activation is small and
// shared by all rows).  Sums are fp32, in a fixed order: per lane in column
// order, then a butterfly over the wave.
#include "nt_dev.h"

namespace nt {
namespace {

constexpr int kRowsPerWave = 2;
constexpr int kWavesF = 4;

template <typename T>
__device__ __forceinline__ void decode16(const uint4& v, float (&w)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = h2f(u[i] & 0xffffu);
      w[2 * i + 1] = h2f(u[i] >> 16);
    }
  } else {
    w[0] = __builtin_bit_cast(float, v.x);
    w[1] = __builtin_bit_cast(float, v.y);
    w[2] = __builtin_bit_cast(float, v.z);
    w[3] = __builtin_bit_cast(float, v.w);
  }
}

template <typename T, int M>
__global__ __launch_bounds__(64 * kWavesF) void k_gemv_f(const uint8_t* __restrict__ W, const float* __restrict__ X,
                                                        float* __restrict__ Y, int rows, int cols, int64_t ldy) {
  constexpr int R = kRowsPerWave;
  constexpr int EPL = 16 / sizeof(T);  // weights per 16-byte load
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWavesF + (threadIdx.x >> 6);
  const int r0 = wave * R;
  if (r0 >= rows) return;
  const int64_t rb = (int64_t)cols * sizeof(T);
  const uint8_t* wr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) wr[i] = W + (int64_t)min(r0 + i, rows - 1) * rb;
  float acc[R][M];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < M; ++t) acc[i][t] = 0.f;
#pragma unroll 4
  for (int c = EPL * lane; c < cols; c += EPL * 64) {
    float w[R][EPL];
#pragma unroll
    for (int i = 0; i < R; ++i) decode16<T>(load_chunk(wr[i] + (int64_t)c * sizeof(T)), w[i]);
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const float* x = X + (int64_t)t * cols + c;
#pragma unroll
      for (int q = 0; q < EPL / 4; ++q) {
        const float4 xv = *reinterpret_cast<const float4*>(x + 4 * q);
#pragma unroll
        for (int i = 0; i < R; ++i) {
          acc[i][t] += w[i][4 * q] * xv.x;
          acc[i][t] += w[i][4 * q + 1] * xv.y;
          acc[i][t] += w[i][4 * q + 2] * xv.z;
          acc[i][t] += w[i][4 * q + 3] * xv.w;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const float s = wave_sum(acc[i][t]);
      if (lane == 0 && r0 + i < rows) Y[(int64_t)t * ldy + r0 + i] = s;
    }
}

template <typename T>
int launch_t(const void* W, const float* X, float* Y, int M, int rows, int cols, hipStream_t st) {
  const int waves = (rows + kRowsPerWave - 1) / kRowsPerWave;
  const dim3 grid((waves + kWavesF - 1) / kWavesF), block(64 * kWavesF);
  const uint8_t* w = static_cast<const uint8_t*>(W);
  const int64_t ldy = rows;
  switch (M) {
    case 1: hipLaunchKernelGGL((k_gemv_f<T, 1>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    case 2: hipLaunchKernelGGL((k_gemv_f<T, 2>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    case 3: hipLaunchKernelGGL((k_gemv_f<T, 3>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    case 4: hipLaunchKernelGGL((k_gemv_f<T, 4>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    case 5: hipLaunchKernelGGL((k_gemv_f<T, 5>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    case 6: hipLaunchKernelGGL((k_gemv_f<T, 6>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    case 7: hipLaunchKernelGGL((k_gemv_f<T, 7>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    case 8: hipLaunchKernelGGL((k_gemv_f<T, 8>), grid, block, 0, st, w, X, Y, rows, cols, ldy); break;
    default: return NT_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

}  // namespace

int launch_gemv_f(int fmt, const void* W, const float* X, float* Y, int M, int rows, int cols, hipStream_t stream) {
  if (rows <= 0) return NT_OK;
  if (fmt == NT_F16) return launch_t<uint16_t>(W, X, Y, M, rows, cols, stream);
  if (fmt == NT_F32) return launch_t<float>(W, X, Y, M, rows, cols, stream);
  return NT_EINVAL;
}

}  // namespace nt
