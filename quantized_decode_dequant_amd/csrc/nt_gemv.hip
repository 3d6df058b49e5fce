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
//   stream    After the prologue every wave works alone (no more workgroup
//             barriers).  It owns a contiguous range of work items (rows, or
//             row pairs) and streams their bytes through a private 8 KB LDS
//             slab: a segment of a row -- a contiguous byte range -- is
//             loaded HBM -> registers with 16-byte coalesced loads, written
//             to the slab, and the next segment's loads are issued before the
//             current one is computed, so every wave keeps ~8 KB in flight.
//             Lanes read their blocks from the slab at any byte alignment
//             (Q8_0, Q4_0 and Q6_K blocks are only 2-byte aligned), unpack
//             quants in registers and accumulate.
//   reduce    Lanes of a wave sum with a butterfly per row.
//   epilogue  Plain store, residual add, SwiGLU (gate and up rows in one
//             item) or RoPE + q store + f16 K/V append (row pairs).
//
// The block layouts are the GGUF ones the pages' format list refers to
// (p1 "About"); the unpacking below follows them.

#include <algorithm>

#include "nt_internal.h"

extern __shared__ __attribute__((aligned(16))) uint8_t nt_smem[];

namespace nt {
namespace {

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
__device__ __forceinline__ float unit_q8_0(uint32_t row, int u, uint32_t xe, const XL& x) {
  const uint32_t blk = row + 34u * u;
  const float d = h2f(ld16(blk));
  uint32_t q[8];
  ld_unaligned<8>(blk + 2, q);
  const uint32_t e0 = xe + 32u * u;
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
  return d * ldf(x.sc + (e0 >> 3)) * (float)S;
}

// Q4_0: unit u is block u.  Byte j: low nibble -> element j, high -> j+16.
// w = d*(q-8), so sum w*X = d*(sum q*X - 8*sum X).
__device__ __forceinline__ float unit_q4_0(uint32_t row, int u, uint32_t xe, const XL& x) {
  const uint32_t blk = row + 18u * u;
  const float d = h2f(ld16(blk));
  uint32_t q[4];
  ld_unaligned<4>(blk + 2, q);
  const uint32_t e0 = xe + 32u * u;
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
  const int xs = ldi32(x.sum + (e0 >> 2)) + ldi32(x.sum + (e0 >> 2) + 4);
  const int S = (H << 8) + L - 8 * xs;
  return d * ldf(x.sc + (e0 >> 3)) * (float)S;
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
__device__ __forceinline__ float unit_q4_k(uint32_t row, int u, uint32_t xe, const XL& x) {
  const int sb = u >> 3, part = u & 7, c = part >> 1, h = part & 1;
  const uint32_t blk = row + 144u * sb;
  const uint4 hd = ld128(blk);
  const uint4 qs = ld128(blk + 16 + 32 * c + 16 * h);
  const float d = h2f(hd.x & 0xffffu), dmin = h2f(hd.x >> 16);
  int scA, mA, scB, mB;
  q4k_scale_min(hd.y, hd.z, hd.w, 2 * c, scA, mA);
  q4k_scale_min(hd.y, hd.z, hd.w, 2 * c + 1, scB, mB);
  const uint32_t eA = xe + 256u * sb + 64 * c + 16 * h, eB = eA + 32;
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
__device__ __forceinline__ float unit_q6_k(uint32_t row, int u, uint32_t xe, const XL& x) {
  const int sb = u >> 2, part = u & 3, n = part >> 1, hl = part & 1;
  const uint32_t blk = row + 210u * sb;
  uint32_t qa[4], qb[4], qh[4], scw[3];
  ld_unaligned<4>(blk + 64 * n + 16 * hl, qa);
  ld_unaligned<4>(blk + 64 * n + 32 + 16 * hl, qb);
  ld_unaligned<4>(blk + 128 + 32 * n + 16 * hl, qh);
  ld_unaligned<3>(blk + 192 + 8 * n, scw);  // sc[8n .. 8n+7] (+4 spare bytes)
  const float d = h2f(ld16(blk + 208));
  const uint32_t e0 = xe + 256u * sb + 128 * n + 16 * hl;
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

// ----------------------------------------------------------------- prologue
// Stage the activation: v = src (or RMSNorm(src) * gain), then per 32-block
// s = max|v| / 32639, X = rint(v / s), hi = (X + 128) >> 8, lo = X - 256 hi.
__device__ __forceinline__ void stage_x(const Job& job, const ProArgs& pro, int tid) {
  const int cols = job.cols, NT = job.nwaves * 64;
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
    for (int w = 0; w < job.nwaves; ++w) tot += ldf(job.red + 4u * w);
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

// ----------------------------------------------------------- segment stream
// Position in a wave's stream: item `it`, row `g` within the item, segment
// `s` within the row.
struct Pos {
  int it, g, s;
};

// Byte range of one segment and where its data sits in the slab.
struct Seg {
  const uint8_t* a;  // 16-B aligned address of the first chunk
  int nchunks;
  uint32_t d;        // byte offset of the segment's first block in the slab
  int m;             // matrix
  int row;           // row within the matrix
  int nblk;          // blocks in the segment
  uint32_t xe;       // element index (column) of the segment's first weight
};

__device__ __forceinline__ int item_matrix(const Job& job, int it) {
  int m = 0;
  while (m + 1 < job.nmat && it >= job.item_start[m + 1]) ++m;
  return m;
}

__device__ __forceinline__ int rows_per_item(const Job& job) { return (job.paired || job.pairs) ? 2 : 1; }

__device__ __forceinline__ Seg seg_of(const Job& job, const Pos& p) {
  Seg sg;
  const int mi = item_matrix(job, p.it);
  const int li = p.it - job.item_start[mi];
  if (job.paired) {
    sg.m = p.g;
    sg.row = li;
  } else {
    sg.m = mi;
    sg.row = job.pairs ? 2 * li + p.g : li;
  }
  const int m = sg.m;
  const int fmt = job.fmt[m];
  const int bb = block_bytes(fmt);
  const int nbr = job.cols / block_elems(fmt);
  const int b0 = p.s * job.seg_blocks[m];
  sg.nblk = min(job.seg_blocks[m], nbr - b0);
  sg.xe = (uint32_t)b0 * block_elems(fmt);
  const uint8_t* start = job.W[m] + (int64_t)sg.row * job.rb[m] + (int64_t)b0 * bb;
  sg.a = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(start) & ~uintptr_t(15));
  sg.d = (uint32_t)(start - sg.a);
  sg.nchunks = (int)((sg.d + (uint32_t)(sg.nblk * bb) + 15) >> 4);
  return sg;
}

// Advance to the next segment; returns false past the wave's last item.
__device__ __forceinline__ bool advance(const Job& job, Pos& p, int it_end) {
  const int m = job.paired ? p.g : item_matrix(job, p.it);
  if (++p.s < job.nseg[m]) return true;
  p.s = 0;
  if (++p.g < rows_per_item(job)) return true;
  p.g = 0;
  return ++p.it < it_end;
}

__device__ __forceinline__ void seg_load(const Seg& sg, int lane, uint4 (&pre)[kSlabLoads]) {
#pragma unroll
  for (int i = 0; i < kSlabLoads; ++i) {
    const int c = lane + 64 * i;
    if (c < sg.nchunks) pre[i] = load_chunk(sg.a + 16 * (int64_t)c);
  }
}

__device__ __forceinline__ void seg_store(const Seg& sg, uint32_t slab, int lane, const uint4 (&pre)[kSlabLoads]) {
#pragma unroll
  for (int i = 0; i < kSlabLoads; ++i) {
    const int c = lane + 64 * i;
    if (c < sg.nchunks) st128(slab + 16u * c, pre[i]);
  }
}

__device__ __forceinline__ float seg_compute(const Job& job, const Seg& sg, uint32_t slab, int lane) {
  const XL x{job.x_hi, job.x_lo, job.x_sc, job.x_sum};
  const uint32_t row = slab + sg.d;
  float acc = 0.f;
  switch (job.fmt[sg.m]) {
    case NT_Q4_K:
      for (int u = lane; u < 8 * sg.nblk; u += 64) acc += unit_q4_k(row, u, sg.xe, x);
      break;
    case NT_Q6_K:
      for (int u = lane; u < 4 * sg.nblk; u += 64) acc += unit_q6_k(row, u, sg.xe, x);
      break;
    case NT_Q8_0:
      for (int u = lane; u < sg.nblk; u += 64) acc += unit_q8_0(row, u, sg.xe, x);
      break;
    default:
      for (int u = lane; u < sg.nblk; u += 64) acc += unit_q4_0(row, u, sg.xe, x);
      break;
  }
  return acc;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Results of one item (row sums s0 and, for two-row items, s1).
template <int EPI>
__device__ __forceinline__ void item_epilogue(const Job& job, int it, float s0, float s1, const EpiArgs& ea) {
  const int mi = item_matrix(job, it);
  const int li = it - job.item_start[mi];
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    const int R = job.row_base[mi] + li;
    if constexpr (EPI == EPI_RESID) ea.y[R] += s0;
    else ea.y[R] = s0;
  } else if constexpr (EPI == EPI_SWIGLU) {
    ea.y[li] = silu(s0) * s1;
  } else if constexpr (EPI == EPI_QKV) {
    const int pos = *ea.pos + ea.pos_add;
    const bool pos_ok = pos >= ea.pos_add && pos < ea.max_ctx;
    if (!pos_ok && ea.err) *ea.err = 1;
    const int R = job.row_base[mi] + 2 * li;  // even row of an adjacent pair
    float a = s0, b = s1;
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

template <int EPI>
__global__ __launch_bounds__(kMaxThreads) void k_qgemv(Job job, ProArgs pro, EpiArgs ea) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nitems = job.item_start[job.nmat];
  const int64_t gw = (int64_t)blockIdx.x * job.nwaves + wave;
  const int64_t GW = (int64_t)gridDim.x * job.nwaves;
  const int it_begin = (int)(gw * nitems / GW), it_end = (int)((gw + 1) * nitems / GW);
  const uint32_t slab = job.slab + (uint32_t)wave * kSlab;
  uint4 pre[kSlabLoads];
  Pos p{it_begin, 0, 0};
  bool live = it_begin < it_end;
  Seg cur = seg_of(job, Pos{live ? it_begin : 0, 0, 0});
  if (live) seg_load(cur, lane, pre);
  stage_x(job, pro, tid);  // the only workgroup barrier
  float acc0 = 0.f, acc1 = 0.f;
  while (live) {
    seg_store(cur, slab, lane, pre);
    const Pos here = p;
    const Seg seg = cur;
    live = advance(job, p, it_end);
    if (live) {
      cur = seg_of(job, p);
      seg_load(cur, lane, pre);
    }
    const float part = seg_compute(job, seg, slab, lane);
    if (here.g == 0) acc0 += part;
    else acc1 += part;
    // last segment of the item: reduce and finish it
    if (!live || p.it != here.it) {
      const float s0 = wave_sum(acc0);
      const float s1 = wave_sum(acc1);
      if (lane == 0) item_epilogue<EPI>(job, here.it, s0, s1, ea);
      acc0 = 0.f;
      acc1 = 0.f;
    }
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
int launch_epi(const Job& job, const ProArgs& pro, const EpiArgs& ea, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_qgemv<EPI>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) !=
        hipSuccess)
      return NT_EHIP;
    attr_set = true;
  }
  const int nitems = job.item_start[job.nmat];
  // one workgroup per CU; fewer when there are not enough items for its waves
  const int grid = std::max(1, std::min(dev_info().cus, (nitems + job.nwaves - 1) / job.nwaves));
  if (nitems <= 0) return NT_OK;
  hipLaunchKernelGGL(k_qgemv<EPI>, dim3(grid), dim3(64 * job.nwaves), job.lds_bytes, stream, job, pro, ea);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

}  // namespace

// Geometry of a launch: segments of at most kSegMax bytes (whole blocks,
// rows split evenly), the LDS layout, and as many waves (<= 12) as LDS
// allows once the staged activation is in.
int plan_job(Job& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
             int pairs) {
  if (nmat < 1 || nmat > kMaxMats || (paired && nmat != 2)) return NT_EINVAL;
  if (cols <= 0 || cols > kMaxCols) return NT_EUNSUPPORTED;
  job = Job{};
  job.nmat = nmat;
  job.paired = paired;
  job.pairs = pairs;
  job.cols = cols;
  int items = 0, rbase = 0;
  for (int m = 0; m < nmat; ++m) {
    const int qk = block_elems(fmt[m]);
    if (qk == 0 || cols % qk != 0) return NT_EINVAL;
    if (pairs && (rows[m] & 1)) return NT_EINVAL;
    if (paired && rows[m] != rows[0]) return NT_EINVAL;
    job.W[m] = W[m];
    job.fmt[m] = fmt[m];
    job.rows[m] = rows[m];
    const int bb = block_bytes(fmt[m]);
    const int nbr = cols / qk;
    job.rb[m] = (int64_t)nbr * bb;
    const int nseg = (int)((job.rb[m] + kSegMax - 1) / kSegMax);
    job.seg_blocks[m] = (nbr + nseg - 1) / nseg;
    job.nseg[m] = (nbr + job.seg_blocks[m] - 1) / job.seg_blocks[m];
    job.item_start[m] = items;
    job.row_base[m] = rbase;
    rbase += rows[m];
    if (!paired || m == 0) items += pairs ? rows[m] / 2 : rows[m];
  }
  if (paired) job.item_start[1] = items;
  job.item_start[nmat] = items;
  uint32_t off = 0;
  job.x_hi = off; off += cols;
  job.x_lo = off; off += cols;
  job.x_sc = off; off += (cols / 32) * 4;
  job.x_sum = off; off += (cols / 16) * 4;
  job.red = off; off += 16 * 4;
  off = (off + 15) & ~15u;
  job.slab = off;
  const int64_t room = 160 * 1024 - (int64_t)off;
  const int nw = (int)std::min<int64_t>(kMaxWaves, room / kSlab);
  if (nw < 4) return NT_EUNSUPPORTED;
  job.nwaves = nw;
  job.lds_bytes = off + (uint32_t)nw * kSlab;
  return NT_OK;
}

int launch_gemv(const Job& job, const ProArgs& pro, int epi, const EpiArgs& ea, hipStream_t stream) {
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(job, pro, ea, stream);
    case EPI_RESID: return launch_epi<EPI_RESID>(job, pro, ea, stream);
    case EPI_QKV: return launch_epi<EPI_QKV>(job, pro, ea, stream);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(job, pro, ea, stream);
  }
  return NT_EINVAL;
}

}  // namespace nt
