// nt_gemv.hip -- the quantized GEMV engine for gfx950.
//
// One engine serves every projection of the decode (GEMV is the per-token
// kernel the ntransformer pages list first; p2 "Architecture et structure du
// code").  Structure of one workgroup:
//
//   prologue  The activation vector (optionally RMSNorm'ed with gains) is
//             staged on chip as 16-bit fixed point per 32-element block: an
//             fp32 scale s_b and integers X in [-32639, 32639], split into a
//             high and a low int8 plane (X = 256*hi + lo) plus per-16 sums of
//             X.  Weight x activation products then run on v_dot4_i32_i8
//             with exact integer sums per quantization sub-block.
//   tiles     A tile is a group of consecutive rows of one matrix -- a
//             contiguous byte range -- streamed HBM -> registers with 16-byte
//             coalesced loads (one tile in flight while the previous one is
//             computed), then written to LDS.  Lanes read their blocks from
//             LDS at any byte alignment (Q8_0, Q4_0 and Q6_K blocks are only
//             2-byte aligned), unpack quants in registers and accumulate.
//   reduce    Lanes of a wave sum with a butterfly; waves sharing a row sum
//             through LDS.
//   epilogue  Plain store, residual add, SwiGLU (gate and up rows in one
//             tile) or RoPE + q store + f16 K/V append.
//
// The block layouts are the GGUF ones the pages' format list refers to
// (p1 "About"); the unpacking below follows them.

#include <algorithm>

#include "nt_internal.h"

extern __shared__ __attribute__((aligned(16))) uint8_t nt_smem[];

namespace nt {
namespace {

constexpr int kMaxYpart = 128;
constexpr float kXMax = 32639.0f;  // |X| bound; keeps the high plane in [-127, 127]

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Offsets of the staged activation in LDS.
struct XL {
  uint32_t hi, lo, sc, sum;
};

// ---------------------------------------------------------------- units
// A unit is the work of one lane on one row: 32 weights (Q8_0, Q4_0, Q4_K)
// or 64 weights (Q6_K).  `row` is the LDS byte offset of the row's first block.

// Q8_0: unit u is block u.  w = d*q.
__device__ __forceinline__ float unit_q8_0(uint32_t row, int u, const XL& x) {
  const uint32_t blk = row + 34u * u;
  const float d = h2f(ld16(blk));
  uint32_t q[8];
  ld_unaligned<8>(blk + 2, q);
  const uint32_t e0 = 32u * u;
  const uint4 h0 = ld128(x.hi + e0), h1 = ld128(x.hi + e0 + 16);
  const uint4 l0 = ld128(x.lo + e0), l1 = ld128(x.lo + e0 + 16);
  int H = 0, L = 0;
  H = dot4(q[0], h0.x, H); L = dot4(q[0], l0.x, L);
  H = dot4(q[1], h0.y, H); L = dot4(q[1], l0.y, L);
  H = dot4(q[2], h0.z, H); L = dot4(q[2], l0.z, L);
  H = dot4(q[3], h0.w, H); L = dot4(q[3], l0.w, L);
  H = dot4(q[4], h1.x, H); L = dot4(q[4], l1.x, L);
  H = dot4(q[5], h1.y, H); L = dot4(q[5], l1.y, L);
  H = dot4(q[6], h1.z, H); L = dot4(q[6], l1.z, L);
  H = dot4(q[7], h1.w, H); L = dot4(q[7], l1.w, L);
  const int S = (H << 8) + L;
  return d * ldf(x.sc + 4u * u) * (float)S;
}

// Q4_0: unit u is block u.  Byte j: low nibble -> element j, high -> j+16.
// w = d*(q-8), so sum w*X = d*(sum q*X - 8*sum X).
__device__ __forceinline__ float unit_q4_0(uint32_t row, int u, const XL& x) {
  const uint32_t blk = row + 18u * u;
  const float d = h2f(ld16(blk));
  uint32_t q[4];
  ld_unaligned<4>(blk + 2, q);
  const uint32_t e0 = 32u * u;
  const uint4 h0 = ld128(x.hi + e0), h1 = ld128(x.hi + e0 + 16);
  const uint4 l0 = ld128(x.lo + e0), l1 = ld128(x.lo + e0 + 16);
  int H = 0, L = 0;
#define NT_Q40_STEP(W, HA, LA, HB, LB)                 \
  {                                                    \
    const uint32_t lo4 = (W) & 0x0F0F0F0Fu;            \
    const uint32_t hi4 = ((W) >> 4) & 0x0F0F0F0Fu;    \
    H = dot4(lo4, HA, H); L = dot4(lo4, LA, L);        \
    H = dot4(hi4, HB, H); L = dot4(hi4, LB, L);        \
  }
  NT_Q40_STEP(q[0], h0.x, l0.x, h1.x, l1.x)
  NT_Q40_STEP(q[1], h0.y, l0.y, h1.y, l1.y)
  NT_Q40_STEP(q[2], h0.z, l0.z, h1.z, l1.z)
  NT_Q40_STEP(q[3], h0.w, l0.w, h1.w, l1.w)
#undef NT_Q40_STEP
  const int xs = ldi32(x.sum + 8u * u) + ldi32(x.sum + 8u * u + 4);
  const int S = (H << 8) + L - 8 * xs;
  return d * ldf(x.sc + 4u * u) * (float)S;
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

// Q4_K: unit u = 16 bytes of quants: superblock u/8, chunk c = (u%8)/2 (64
// weights, bytes 32c..32c+31), half h = u%2.  Low nibbles are elements
// 64c+16h+i (sub-block 2c), high nibbles 64c+32+16h+i (sub-block 2c+1).
// w = d*sc*q - dmin*m.
__device__ __forceinline__ float unit_q4_k(uint32_t row, int u, const XL& x) {
  const int sb = u >> 3, part = u & 7, c = part >> 1, h = part & 1;
  const uint32_t blk = row + 144u * sb;
  const uint4 hd = ld128(blk);
  const uint4 qs = ld128(blk + 16 + 32 * c + 16 * h);
  const float d = h2f(hd.x & 0xffffu), dmin = h2f(hd.x >> 16);
  int scA, mA, scB, mB;
  q4k_scale_min(hd.y, hd.z, hd.w, 2 * c, scA, mA);
  q4k_scale_min(hd.y, hd.z, hd.w, 2 * c + 1, scB, mB);
  const uint32_t eA = 256u * sb + 64 * c + 16 * h, eB = eA + 32;
  const uint4 ah = ld128(x.hi + eA), al = ld128(x.lo + eA);
  const uint4 bh = ld128(x.hi + eB), bl = ld128(x.lo + eB);
  int AH = 0, AL = 0, BH = 0, BL = 0;
#define NT_Q4K_STEP(W, AHX, ALX, BHX, BLX)             \
  {                                                    \
    const uint32_t lo4 = (W) & 0x0F0F0F0Fu;            \
    const uint32_t hi4 = ((W) >> 4) & 0x0F0F0F0Fu;     \
    AH = dot4(lo4, AHX, AH); AL = dot4(lo4, ALX, AL);  \
    BH = dot4(hi4, BHX, BH); BL = dot4(hi4, BLX, BL);  \
  }
  NT_Q4K_STEP(qs.x, ah.x, al.x, bh.x, bl.x)
  NT_Q4K_STEP(qs.y, ah.y, al.y, bh.y, bl.y)
  NT_Q4K_STEP(qs.z, ah.z, al.z, bh.z, bl.z)
  NT_Q4K_STEP(qs.w, ah.w, al.w, bh.w, bl.w)
#undef NT_Q4K_STEP
  const int SA = (AH << 8) + AL, SB = (BH << 8) + BL;
  const int XA = ldi32(x.sum + 4u * (eA >> 4)), XB = ldi32(x.sum + 4u * (eB >> 4));
  const float sA = ldf(x.sc + 4u * (eA >> 5)), sB = ldf(x.sc + 4u * (eB >> 5));
  return sA * (d * (float)scA * (float)SA - dmin * (float)mA * (float)XA) +
         sB * (d * (float)scB * (float)SB - dmin * (float)mB * (float)XB);
}

// Q6_K: unit u = 64 weights: superblock u/4, half n = (u%4)/2, l0 = 16*(u%2).
// For quarter k = 0..3 the elements are 128n + 32k + l0 + i (i < 16), with
// low four bits from nibble k/2 of ql[64n + 32(k%2) + l0 + i], high two bits
// from bits 2k..2k+1 of qh[32n + l0 + i], and scale sc[8n + 2k + l0/16].
// w = d*sc*(q-32).
__device__ __forceinline__ float unit_q6_k(uint32_t row, int u, const XL& x) {
  const int sb = u >> 2, part = u & 3, n = part >> 1, hl = part & 1;
  const uint32_t blk = row + 210u * sb;
  uint32_t qa[4], qb[4], qh[4], scw[3];
  ld_unaligned<4>(blk + 64 * n + 16 * hl, qa);
  ld_unaligned<4>(blk + 64 * n + 32 + 16 * hl, qb);
  ld_unaligned<4>(blk + 128 + 32 * n + 16 * hl, qh);
  ld_unaligned<3>(blk + 192 + 8 * n, scw);  // sc[8n .. 8n+7] (+4 spare bytes)
  const float d = h2f(ld16(blk + 208));
  const uint32_t e0 = 256u * sb + 128 * n + 16 * hl;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t e = e0 + 32 * k;
    const uint4 xh = ld128(x.hi + e), xl = ld128(x.lo + e);
    const uint32_t xhv[4] = {xh.x, xh.y, xh.z, xh.w}, xlv[4] = {xl.x, xl.y, xl.z, xl.w};
    int H = 0, L = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t q;
      if (k == 0) q = (qa[i] & 0x0F0F0F0Fu) | ((qh[i] << 4) & 0x30303030u);
      else if (k == 1) q = (qb[i] & 0x0F0F0F0Fu) | ((qh[i] << 2) & 0x30303030u);
      else if (k == 2) q = ((qa[i] >> 4) & 0x0F0F0F0Fu) | (qh[i] & 0x30303030u);
      else q = ((qb[i] >> 4) & 0x0F0F0F0Fu) | ((qh[i] >> 2) & 0x30303030u);
      H = dot4(q, xhv[i], H);
      L = dot4(q, xlv[i], L);
    }
    const int S = (H << 8) + L - 32 * ldi32(x.sum + 4u * (e >> 4));
    const int sidx = 2 * k + hl;  // scale byte within sc[8n .. 8n+7]
    const int sc = (int)(int8_t)(scw[sidx >> 2] >> (8 * (sidx & 3)));
    acc += (float)S * ((float)sc * ldf(x.sc + 4u * (e >> 5)));
  }
  return d * acc;
}

// ------------------------------------------------------------ tile geometry
struct Geo {
  int m, r0, nr;
  const uint8_t* a0;  // 16-B aligned chunk bases of the tile's byte segments
  const uint8_t* a1;
  int n0, n1;           // 16-B chunks per segment
  uint32_t d0, d1;      // LDS byte offset of each segment's first row
};

__device__ __forceinline__ Geo tile_geo(const TileJob& job, int tile) {
  Geo g;
  int m = 0;
  while (m + 1 < job.nmat && tile >= job.tile_start[m + 1]) ++m;
  g.m = m;
  const int T = job.tile_rows[m];
  g.r0 = (tile - job.tile_start[m]) * T;
  g.nr = min(T, job.rows[m] - g.r0);
  const uint8_t* p0 = job.W[m] + (int64_t)g.r0 * job.rb[m];
  g.a0 = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(p0) & ~uintptr_t(15));
  g.d0 = (uint32_t)(p0 - g.a0);
  g.n0 = (int)((g.d0 + (int64_t)g.nr * job.rb[m] + 15) >> 4);
  if (job.paired) {
    const uint8_t* p1 = job.W[1] + (int64_t)g.r0 * job.rb[1];
    g.a1 = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(p1) & ~uintptr_t(15));
    g.d1 = 16u * g.n0 + (uint32_t)(p1 - g.a1);
    g.n1 = (int)(((uint32_t)(p1 - g.a1) + (int64_t)g.nr * job.rb[1] + 15) >> 4);
  } else {
    g.a1 = g.a0;
    g.n1 = 0;
    g.d1 = 0;
  }
  return g;
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

__device__ __forceinline__ void prefetch(const Geo& g, int lpw, int tid, int NT, uint4 (&pre)[kLpwMax]) {
#pragma unroll
  for (int i = 0; i < kLpwMax; ++i) {
    if (i < lpw) {
      const int c = tid + i * NT;
      if (c < g.n0)
        pre[i] = load_chunk(g.a0 + 16 * (int64_t)c);
      else if (c < g.n0 + g.n1)
        pre[i] = load_chunk(g.a1 + 16 * (int64_t)(c - g.n0));
    }
  }
}

__device__ __forceinline__ void store_tile(const Geo& g, int lpw, int tid, int NT, const uint4 (&pre)[kLpwMax]) {
#pragma unroll
  for (int i = 0; i < kLpwMax; ++i) {
    if (i < lpw) {
      const int c = tid + i * NT;
      if (c < g.n0 + g.n1) st128(16u * c, pre[i]);  // segment 1 follows segment 0's chunks
    }
  }
}

// ----------------------------------------------------------------- prologue
// Stage the activation: v = src (or RMSNorm(src) * gain), then per 32-block
// s = max|v| / 32639, X = rint(v / s), hi = (X + 128) >> 8, lo = X - 256 hi.
__device__ __forceinline__ void stage_x(const TileJob& job, const ProArgs& pro, int tid) {
  const int cols = job.cols, NT = job.nthreads;
  const float* src = pro.src;
  float r = 1.0f;
  if (pro.gain) {
    float ss = 0.f;
    for (int i = 4 * tid; i < cols; i += 4 * NT) {
      const float4 v = *reinterpret_cast<const float4*>(src + i);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) stf(job.red + 4u * (tid >> 6), ss);
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < (NT >> 6); ++w) tot += ldf(job.red + 4u * w);
    r = 1.0f / sqrtf(tot / (float)cols + pro.eps);
  }
  const int nb = cols >> 5;
  for (int b = tid; b < nb; b += NT) {
    float v[32];
    const float4* s4 = reinterpret_cast<const float4*>(src + 32 * b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 t = s4[j];
      v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
    }
    if (pro.gain) {
      const float4* g4 = reinterpret_cast<const float4*>(pro.gain + 32 * b);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 t = g4[j];
        v[4 * j] = v[4 * j] * r * t.x;
        v[4 * j + 1] = v[4 * j + 1] * r * t.y;
        v[4 * j + 2] = v[4 * j + 2] * r * t.z;
        v[4 * j + 3] = v[4 * j + 3] * r * t.w;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const float inv = amax > 0.f ? kXMax / amax : 0.f;
    const float scale = amax / kXMax;
    uint32_t H[8], L[8];
    int s0 = 0, s1 = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) { H[j] = 0; L[j] = 0; }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      int X = __float2int_rn(v[j] * inv);
      X = max(-32639, min(32639, X));
      const int hi = (X + 128) >> 8;
      const int lo = X - (hi << 8);
      H[j >> 2] |= (uint32_t)(hi & 255) << (8 * (j & 3));
      L[j >> 2] |= (uint32_t)(lo & 255) << (8 * (j & 3));
      if (j < 16) s0 += X; else s1 += X;
    }
    st128(job.x_hi + 32u * b, make_uint4(H[0], H[1], H[2], H[3]));
    st128(job.x_hi + 32u * b + 16, make_uint4(H[4], H[5], H[6], H[7]));
    st128(job.x_lo + 32u * b, make_uint4(L[0], L[1], L[2], L[3]));
    st128(job.x_lo + 32u * b + 16, make_uint4(L[4], L[5], L[6], L[7]));
    stf(job.x_sc + 4u * b, scale);
    sti32(job.x_sum + 8u * b, s0);
    sti32(job.x_sum + 8u * b + 4, s1);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ compute
__device__ __forceinline__ int units_per_row(int fmt, int cols) { return fmt == NT_Q6_K ? cols >> 6 : cols >> 5; }

__device__ __forceinline__ void tile_dims(const TileJob& job, const Geo& g, int& T, int& nv, int& WPR) {
  const int NW = job.nthreads >> 6;
  T = job.tile_rows[g.m] * (job.paired ? 2 : 1);
  nv = g.nr * (job.paired ? 2 : 1);
  WPR = T >= NW ? 1 : NW / T;
}

__device__ __forceinline__ void compute_tile(const TileJob& job, const Geo& g, int tid) {
  const int NW = job.nthreads >> 6, wave = tid >> 6, lane = tid & 63;
  int T, nv, WPR;
  tile_dims(job, g, T, nv, WPR);
  const int vstep = NW / WPR;
  const int part = wave % WPR;
  const XL x{job.x_hi, job.x_lo, job.x_sc, job.x_sum};
  for (int v = wave / WPR; v < nv; v += vstep) {
    const int seg = (job.paired && v >= g.nr) ? 1 : 0;
    const int mi = seg ? 1 : g.m;
    const int fmt = job.fmt[mi];
    const uint32_t row = (seg ? g.d1 : g.d0) + (uint32_t)((seg ? v - g.nr : v) * job.rb[mi]);
    const int U = units_per_row(fmt, job.cols);
    float acc = 0.f;
    const int u0 = part * 64 + lane, us = 64 * WPR;
    switch (fmt) {
      case NT_Q4_K:
        for (int u = u0; u < U; u += us) acc += unit_q4_k(row, u, x);
        break;
      case NT_Q6_K:
        for (int u = u0; u < U; u += us) acc += unit_q6_k(row, u, x);
        break;
      case NT_Q8_0:
        for (int u = u0; u < U; u += us) acc += unit_q8_0(row, u, x);
        break;
      default:
        for (int u = u0; u < U; u += us) acc += unit_q4_0(row, u, x);
        break;
    }
    acc = wave_sum(acc);
    if (lane == 0) stf(job.ypart + 4u * (v * WPR + part), acc);
  }
}

__device__ __forceinline__ float row_sum(const TileJob& job, int v, int WPR) {
  float s = 0.f;
  for (int p = 0; p < WPR; ++p) s += ldf(job.ypart + 4u * (v * WPR + p));
  return s;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <int EPI>
__device__ __forceinline__ void epilogue(const TileJob& job, const Geo& g, const EpiArgs& ea, int tid) {
  int T, nv, WPR;
  tile_dims(job, g, T, nv, WPR);
  const int NT = job.nthreads;
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    for (int t = tid; t < g.nr; t += NT) {
      const int R = job.row_base[g.m] + g.r0 + t;
      const float s = row_sum(job, t, WPR);
      if constexpr (EPI == EPI_RESID) ea.y[R] += s;
      else ea.y[R] = s;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int t = tid; t < g.nr; t += NT) {
      const float gate = row_sum(job, t, WPR), up = row_sum(job, g.nr + t, WPR);
      ea.y[g.r0 + t] = silu(gate) * up;
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int pos = *ea.pos;
    const bool pos_ok = pos >= 0 && pos < ea.max_ctx;
    if (!pos_ok && tid == 0 && ea.err) *ea.err = 1;
    for (int t = tid; 2 * t < g.nr; t += NT) {
      const int R = job.row_base[g.m] + g.r0 + 2 * t;  // even row of an adjacent pair
      float a = row_sum(job, 2 * t, WPR), b = row_sum(job, 2 * t + 1, WPR);
      const int dd = R % ea.head_dim;
      if (R < ea.q_rows + ea.kv_rows) {
        // RoPE: pair (2i, 2i+1) of a head turns by pos * theta^(-2i/head_dim);
        // the angle is formed in double so large positions keep fp32 accuracy.
        const double freq = exp2(-(double)dd / (double)ea.head_dim * log2((double)ea.rope_theta));
        const double ang = (double)pos * freq;
        const float c = (float)cos(ang), s = (float)sin(ang);
        const float a2 = a * c - b * s, b2 = a * s + b * c;
        a = a2;
        b = b2;
      }
      if (R < ea.q_rows) {
        ea.q_out[R] = a;
        ea.q_out[R + 1] = b;
      } else if (pos_ok) {
        const bool is_k = R < ea.q_rows + ea.kv_rows;
        const int rr = R - ea.q_rows - (is_k ? 0 : ea.kv_rows);
        const int kh = rr / ea.head_dim;
        uint16_t* cache = is_k ? ea.k_cache : ea.v_cache;
        const int64_t off = ((int64_t)kh * ea.max_ctx + pos) * ea.head_dim + dd;
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        cache[off] = __builtin_bit_cast(uint16_t, ha);
        cache[off + 1] = __builtin_bit_cast(uint16_t, hb);
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kMaxThreads) void k_qgemv(TileJob job, ProArgs pro, EpiArgs ea) {
  const int tid = threadIdx.x, NT = job.nthreads;
  const int ntiles = job.tile_start[job.nmat];
  int tile = blockIdx.x;
  uint4 pre[kLpwMax];
  Geo g = tile_geo(job, tile < ntiles ? tile : 0);
  if (tile < ntiles) prefetch(g, job.lpw, tid, NT, pre);
  stage_x(job, pro, tid);
  for (; tile < ntiles; tile += gridDim.x) {
    store_tile(g, job.lpw, tid, NT, pre);
    __syncthreads();
    const Geo cur = g;
    const int nxt = tile + gridDim.x;
    if (nxt < ntiles) {
      g = tile_geo(job, nxt);
      prefetch(g, job.lpw, tid, NT, pre);
    }
    compute_tile(job, cur, tid);
    __syncthreads();
    epilogue<EPI>(job, cur, ea, tid);
  }
}

struct DevInfo {
  int cus = 0;
};

DevInfo& dev_info() {
  static DevInfo info[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  DevInfo& d = info[dev & 63];
  if (d.cus == 0) {
    int v = 0;
    (void)hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    d.cus = v > 0 ? v : 256;
  }
  return d;
}

template <int EPI>
int launch_epi(const TileJob& job, const ProArgs& pro, const EpiArgs& ea, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_qgemv<EPI>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) !=
        hipSuccess)
      return NT_EHIP;
    attr_set = true;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_qgemv<EPI>, job.nthreads, job.lds_bytes) != hipSuccess)
    return NT_EHIP;
  if (per_cu < 1) return NT_EUNSUPPORTED;
  const int ntiles = job.tile_start[job.nmat];
  const int grid = min(ntiles, per_cu * dev_info().cus);
  if (grid <= 0) return NT_OK;
  hipLaunchKernelGGL(k_qgemv<EPI>, dim3(grid), dim3(job.nthreads), job.lds_bytes, stream, job, pro, ea);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

}  // namespace

// Geometry of a launch: workgroup size from the size of the staged
// activation, rows per tile so a tile carries ~20 KB (256 threads) or ~48 KB
// (512 threads) of weights, and the LDS layout.
int plan_job(TileJob& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
             int rope_pairs) {
  if (nmat < 1 || nmat > kMaxMats || (paired && nmat != 2)) return NT_EINVAL;
  if (cols <= 0 || cols > kMaxCols) return NT_EUNSUPPORTED;
  const int64_t x_bytes = (int64_t)cols * 2 + (cols / 32) * 4 + (cols / 16) * 4;
  job = TileJob{};
  job.nmat = nmat;
  job.paired = paired;
  job.cols = cols;
  job.nthreads = x_bytes <= 24 * 1024 ? 256 : 512;
  const int NW = job.nthreads / 64;
  const int64_t target = job.nthreads == 256 ? 20 * 1024 : 48 * 1024;
  int64_t need = 0;
  int tiles = 0, rbase = 0;
  for (int m = 0; m < nmat; ++m) {
    const int qk = block_elems(fmt[m]);
    if (qk == 0 || cols % qk != 0) return NT_EINVAL;
    job.W[m] = W[m];
    job.fmt[m] = fmt[m];
    job.rows[m] = rows[m];
    job.rb[m] = (int64_t)(cols / qk) * block_bytes(fmt[m]);
  }
  for (int m = 0; m < nmat; ++m) {
    const int64_t rb_eff = paired ? job.rb[0] + job.rb[1] : job.rb[m];
    int T = 1;
    while (T < 64 && 2 * T * rb_eff <= target) T *= 2;
    if (rope_pairs && T < 2) T = 2;
    job.tile_rows[m] = T;
    const int nseg = paired ? 2 : 1;
    need = std::max<int64_t>(need, T * rb_eff + 32 * nseg);
    (void)NW;
    job.tile_start[m] = tiles;
    job.row_base[m] = rbase;
    rbase += rows[m];
    if (!paired || m == 0) tiles += (rows[m] + T - 1) / T;
  }
  if (paired) {
    job.tile_rows[1] = job.tile_rows[0];
    job.tile_start[1] = tiles;
  }
  job.tile_start[nmat] = tiles;
  const int64_t per_load = (int64_t)job.nthreads * 16;
  job.lpw = (int)((need + per_load - 1) / per_load);
  if (job.lpw > kLpwMax) return NT_EUNSUPPORTED;
  job.tile_cap = (uint32_t)(job.lpw * per_load);
  uint32_t off = job.tile_cap;
  job.x_hi = off; off += cols;
  job.x_lo = off; off += cols;
  job.x_sc = off; off += (cols / 32) * 4;
  job.x_sum = off; off += (cols / 16) * 4;
  job.ypart = off; off += kMaxYpart * 4;
  job.red = off; off += 16 * 4;
  job.lds_bytes = (off + 15) & ~15u;
  if (job.lds_bytes > 160 * 1024) return NT_EUNSUPPORTED;
  return NT_OK;
}

int launch_gemv(const TileJob& job, const ProArgs& pro, int epi, const EpiArgs& ea, hipStream_t stream) {
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(job, pro, ea, stream);
    case EPI_RESID: return launch_epi<EPI_RESID>(job, pro, ea, stream);
    case EPI_QKV: return launch_epi<EPI_QKV>(job, pro, ea, stream);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(job, pro, ea, stream);
  }
  return NT_EINVAL;
}

}  // namespace nt
