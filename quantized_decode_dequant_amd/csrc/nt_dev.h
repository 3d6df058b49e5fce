// Device helpers shared by the GEMV engine, the small-M GEMM and attention: LDS
// accessors on the dynamic LDS block, DPP reductions, non-temporal weight
// loads and the GGUF Q4_K scale unpacking.
#pragma once

#include "nt_internal.h"

extern __shared__ __attribute__((aligned(16))) uint8_t nt_smem[];

namespace nt {
namespace {

constexpr float kXMax = 32639.0f;  // |X| bound of the 16-bit activation; keeps the high plane in [-127, 127]

__device__ __forceinline__ uint32_t ld32(uint32_t off) { return *reinterpret_cast<const uint32_t*>(nt_smem + off); }
__device__ __forceinline__ int ldi32(uint32_t off) { return *reinterpret_cast<const int*>(nt_smem + off); }
__device__ __forceinline__ float ldf(uint32_t off) { return *reinterpret_cast<const float*>(nt_smem + off); }
__device__ __forceinline__ uint32_t ld16(uint32_t off) { return *reinterpret_cast<const uint16_t*>(nt_smem + off); }
__device__ __forceinline__ uint4 ld128(uint32_t off) { return *reinterpret_cast<const uint4*>(nt_smem + off); }
__device__ __forceinline__ void st128(uint32_t off, uint4 v) { *reinterpret_cast<uint4*>(nt_smem + off) = v; }
__device__ __forceinline__ void stf(uint32_t off, float v) { *reinterpret_cast<float*>(nt_smem + off) = v; }
__device__ __forceinline__ void sti32(uint32_t off, int v) { *reinterpret_cast<int*>(nt_smem + off) = v; }

__device__ __forceinline__ float h2f(uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); }
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}
// The first product of a chain: the three-operand form with a zero
// accumulator (the builtin with c = 0 becomes a register clear plus the
// two-operand form).
__device__ __forceinline__ int dot4z(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// N dwords starting at an LDS byte offset that is only 2-byte aligned:
// read N+1 aligned dwords and funnel-shift them.
template <int N>
__device__ __forceinline__ void ld_unaligned(uint32_t off, uint32_t (&out)[N]) {
  const uint32_t base = off & ~3u, sh = off & 3u;
  uint32_t w[N + 1];
#pragma unroll
  for (int i = 0; i <= N; ++i) w[i] = ld32(base + 4 * i);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
}

// Sum over the 64 lanes of a wave: an inclusive scan with DPP row shifts and
// row broadcasts leaves the total in lane 63, which is read into a scalar.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_shift<0x111, 0xf>(v);  // row_shr:1 within rows of 16 lanes
  v += dpp_shift<0x112, 0xf>(v);  // row_shr:2
  v += dpp_shift<0x114, 0xf>(v);  // row_shr:4
  v += dpp_shift<0x118, 0xf>(v);  // row_shr:8
  v += dpp_shift<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_shift<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maximum over the 64 lanes of a wave, the same scan with -inf for lanes
// that receive nothing.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift_max(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -__builtin_huge_valf()),
                                                                __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_shift_max<0x111, 0xf>(v));
  v = fmaxf(v, dpp_shift_max<0x112, 0xf>(v));
  v = fmaxf(v, dpp_shift_max<0x114, 0xf>(v));
  v = fmaxf(v, dpp_shift_max<0x118, 0xf>(v));
  v = fmaxf(v, dpp_shift_max<0x142, 0xa>(v));
  v = fmaxf(v, dpp_shift_max<0x143, 0xc>(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Reductions over the lane groups that hold one 32-block (8 lanes) and one
// 16-sum (4 lanes): DPP quad permutations and the half-row mirror.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, dpp_i<0xB1>(__builtin_bit_cast(int, x))));  // quad_perm 1,0,3,2
  x = fmaxf(x, __builtin_bit_cast(float, dpp_i<0x4E>(__builtin_bit_cast(int, x))));  // quad_perm 2,3,0,1
  return fmaxf(x, __builtin_bit_cast(float, dpp_i<0x141>(__builtin_bit_cast(int, x))));  // row_half_mirror
}
__device__ __forceinline__ int sum4(int x) {
  x += dpp_i<0xB1>(x);
  return x + dpp_i<0x4E>(x);
}

// Q4_K: 6-bit scale and min of sub-block s from the 12 packed bytes
// (bytes 0-3 in s0, 4-7 in s1, 8-11 in s2).  GGUF packing: for s < 4 the low
// six bits of bytes s (scale) and s+4 (min); for s >= 4 the nibbles of byte
// s+4 give the low four bits and the top two bits of bytes s-4 (scale) and
// s (min) give the high two.
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int s, int& sc, int& m) {
  if (s < 4) {
    sc = (s0 >> (8 * s)) & 63;
    m = (s1 >> (8 * s)) & 63;
  } else {
    const int t = 8 * (s - 4);
    const uint32_t b = s2 >> t;
    sc = (b & 15) | (((s0 >> t) >> 6 & 3) << 4);
    m = ((b >> 4) & 15) | (((s1 >> t) >> 6 & 3) << 4);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* gptr_u32x4;

// One 16-byte chunk of weights.  Chunks are 16-byte aligned and contain at
// least one byte of the matrix, so a chunk never crosses a page boundary and
// is always mapped, even where it runs past the matrix's last byte (those
// bytes are never used).  Weights are read once: the load is non-temporal.
__device__ __forceinline__ uint4 load_chunk(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load((gptr_u32x4)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A segment of weights as a raw buffer: 16-byte loads at byte offsets
// below `bytes` read memory, loads at or past it return zeros without a
// memory access (the buffer instructions' range check), non-temporal like
// load_chunk.  The resource's last word is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seg_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kAuxNt = 2;  // cache-policy bits of a non-temporal load
__device__ __forceinline__ uint4 load_seg_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAuxNt);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// The 16-bit fixed point of the activations: a 32-block with largest
// magnitude amax has scale amax / 32639 and X = rint(v * 32639 / amax),
// clamped to [-32639, 32639]; X = 256 hi + lo with hi = (X + 128) >> 8, so
// both planes fit int8.  (A zero block has X = 0 and scale 0.)
__device__ __forceinline__ int fx_quant(float v, float amax) {
  const float inv = amax > 0.f ? kXMax / amax : 0.f;
  const int X = __float2int_rn(v * inv);
  return max(-32639, min(32639, X));
}
__device__ __forceinline__ int fx_hi(int X) { return (X + 128) >> 8; }
__device__ __forceinline__ int fx_lo(int X) { return X - (fx_hi(X) << 8); }

// Quantized-activation output of one 32-block held by 32 consecutive lanes
// (lanes 0-31 or 32-63 of a wave, all active): lane l has value v (already
// times the gains) and y (the value whose square goes into the block's sum
// of squares); b is the block's index in the n-value vector at q.
__device__ __forceinline__ void qx_store_block32(uint8_t* q, int64_t n, int b, int l, float v, float y) {
  float amax = fabsf(v);
#pragma unroll
  for (int m = 16; m > 0; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
  const int X = fx_quant(v, amax);
  int s16 = X;
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) s16 += __shfl_xor(s16, m, 16);
  float ss = y * y;
#pragma unroll
  for (int m = 16; m > 0; m >>= 1) ss += __shfl_xor(ss, m, 32);
  const int64_t e = 32 * (int64_t)b + l;
  q[e] = (uint8_t)(fx_hi(X) & 255);
  q[qx_lo_off(n) + e] = (uint8_t)(fx_lo(X) & 255);
  if ((l & 15) == 0) reinterpret_cast<int*>(q + qx_sum_off(n))[2 * b + (l >> 4)] = s16;
  if (l == 0) {
    reinterpret_cast<float*>(q + qx_sc_off(n))[b] = amax / kXMax;
    reinterpret_cast<float*>(q + qx_ss_off(n))[b] = ss;
  }
}

// The first 256 threads of a block stage one 256-block of an activation row
// for the small-M GEMM (the layout k_stage_m writes over `ncols` columns at
// `stage`): thread i holds element R = 256 b + i of token t with value gv
// (already times any gains); one fixed-point scale for the 256-block, X =
// 256 hi + lo in the MFMA B layout (column 2t + plane), the X sums of each
// 32-block's two 16-element halves; with ss (may be null) also the sum of
// squares of the values y, at ss[t * ncols / 256 + b].  Every thread of the
// block calls it (threads past 256 only for the barriers).
__device__ __forceinline__ void stage_block256(float gv, float y, int t, int R, int ncols, uint8_t* stage, float* ss) {
  __shared__ float red[8];
  __shared__ uint32_t hw[64], lw[64];  // the hi and lo bytes of the 256 values
  __shared__ int xv[256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (wv < 4) {
    const float ws = wave_sum(y * y), wm = wave_max(fabsf(gv));
    if (lane == 0) {
      red[wv] = ws;
      red[4 + wv] = wm;
    }
  }
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
  if (tid < 256) {
    const int X = fx_quant(gv, amax);
    reinterpret_cast<uint8_t*>(hw)[tid] = (uint8_t)(fx_hi(X) & 255);
    reinterpret_cast<uint8_t*>(lw)[tid] = (uint8_t)(fx_lo(X) & 255);
    xv[tid] = X;
  }
  __syncthreads();
  const int b0 = (R - tid) >> 5;  // the 256-block's first 32-block
  const int64_t nb = ncols / 32;
  int4* xs = reinterpret_cast<int4*>(stage + nb * 512);
  float* xsc = reinterpret_cast<float*>(stage + nb * 512 + nb * kMaxTokens * 16);
  if (tid < 128) {
    // four values' bytes of one plane: column 2t + plane of lane (kq, ...)
    const int q = tid & 63, pl = tid >> 6, b = b0 + (q >> 3), gi = q & 7;
    *reinterpret_cast<uint32_t*>(stage + 512 * (int64_t)b + 128 * (gi >> 1) + 4 * (gi & 1) + 8 * (2 * t + pl)) =
        pl ? lw[q] : hw[q];
  } else if (tid < 136) {
    const int j = tid - 128;
    int s0 = 0, s1 = 0;
    for (int k = 0; k < 16; ++k) {
      s0 += xv[32 * j + k];
      s1 += xv[32 * j + 16 + k];
    }
    xs[(int64_t)(b0 + j) * kMaxTokens + t] = make_int4(0, 0, s0, s1);
  } else if (tid == 136) {
    xsc[(int64_t)(b0 >> 3) * kMaxTokens + t] = amax / kXMax;
    if (ss) ss[(int64_t)t * (ncols / 256) + (b0 >> 3)] = red[0] + red[1] + red[2] + red[3];
  }
}

}  // namespace
}  // namespace nt
