// The GEMV engine's device code (kernel and launch in nt_gemv.hip): the
// staged activation, the format units, the segment stream and the
// epilogues.  The design is described at the top of nt_gemv.hip.
//
// The block layouts are the GGUF ones the pages' format list refers to
// (p1 "About"); the unpacking below follows them.
#pragma once

#include "nt_dev.h"

namespace nt {
namespace {

// Activation of the lane's two column units in the current slice: int8 high
// and low planes of 64 elements each, the scale of each 32-block and the sum
// of X over each 16 elements.
struct XR {
  uint32_t hi[kUnitsPerLane][16], lo[kUnitsPerLane][16];
  float sc[kUnitsPerLane][2];
  int sm[kUnitsPerLane][4];
  float sf[kUnitsPerLane][2];  // s * (sum of X) over each 32-block (formats with a per-block offset)
};

__device__ __forceinline__ void load_xr(const Job& job, int slice, int lane, XR& xr) {
#pragma unroll
  for (int j = 0; j < kUnitsPerLane; ++j) {
    const int k = lane + 64 * j;
    const uint32_t e0 = 64u * (uint32_t)(slice * job.ups + k);
    if (k < job.ups && e0 < (uint32_t)job.cols) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 h = ld128(job.x_hi + e0 + 16 * i), l = ld128(job.x_lo + e0 + 16 * i);
        xr.hi[j][4 * i] = h.x; xr.hi[j][4 * i + 1] = h.y; xr.hi[j][4 * i + 2] = h.z; xr.hi[j][4 * i + 3] = h.w;
        xr.lo[j][4 * i] = l.x; xr.lo[j][4 * i + 1] = l.y; xr.lo[j][4 * i + 2] = l.z; xr.lo[j][4 * i + 3] = l.w;
      }
      xr.sc[j][0] = ldf(job.x_sc + (e0 >> 3));
      xr.sc[j][1] = ldf(job.x_sc + (e0 >> 3) + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) xr.sm[j][i] = ldi32(job.x_sum + (e0 >> 2) + 4 * i);
      xr.sf[j][0] = xr.sc[j][0] * (float)(xr.sm[j][0] + xr.sm[j][1]);
      xr.sf[j][1] = xr.sc[j][1] * (float)(xr.sm[j][2] + xr.sm[j][3]);
    }
  }
}

// ---------------------------------------------------------------- units
// A unit is 64 consecutive weights of one row: column unit k of the slice.
// `seg` is the LDS byte offset of the segment's first block; XH/XL/XS/XM the
// lane's activation registers for the unit.

#define NT_XARGS \
  const uint32_t(&xh)[16], const uint32_t(&xl)[16], const float(&xs)[2], const int(&xm)[4], const float(&xf)[2]

// Q8_0: blocks 2k and 2k+1 (the second only if `two`).  w = d*q.
__device__ __forceinline__ float unit_q8_0(uint32_t seg, int k, bool two, NT_XARGS) {
  float acc = 0.f;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b == 1 && !two) break;
    const uint32_t blk = seg + 34u * (2 * k + b);
    const float d = h2f(ld16(blk));
    uint32_t q[8];
    ld_unaligned<8>(blk + 2, q);
    int H = dot4z(q[0], xh[8 * b]), L = dot4z(q[0], xl[8 * b]);
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      H = dot4(q[i], xh[8 * b + i], H);
      L = dot4(q[i], xl[8 * b + i], L);
    }
    acc += d * xs[b] * (float)((H << 8) + L);
  }
  return acc;
}

// Q4_0: blocks 2k and 2k+1.  Byte j of a block: low nibble -> element j,
// high nibble -> element j+16.  w = d*(q-8), so sum w*X = d*(sum q*X - 8 sum X).
__device__ __forceinline__ float unit_q4_0(uint32_t seg, int k, bool two, NT_XARGS) {
  float acc = 0.f;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b == 1 && !two) break;
    const uint32_t blk = seg + 18u * (2 * k + b);
    const float d = h2f(ld16(blk));
    uint32_t q[4];
    ld_unaligned<4>(blk + 2, q);
    int H = 0, L = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo4 = q[i] & 0x0F0F0F0Fu, hi4 = (q[i] >> 4) & 0x0F0F0F0Fu;
      H = i == 0 ? dot4z(lo4, xh[8 * b]) : dot4(lo4, xh[8 * b + i], H);
      L = i == 0 ? dot4z(lo4, xl[8 * b]) : dot4(lo4, xl[8 * b + i], L);
      H = dot4(hi4, xh[8 * b + 4 + i], H);
      L = dot4(hi4, xl[8 * b + 4 + i], L);
    }
    const int S = (H << 8) + L - 8 * (xm[2 * b] + xm[2 * b + 1]);
    acc += d * xs[b] * (float)S;
  }
  return acc;
}

// K-quant superblock header (Q4_K, Q5_K): the 6-bit scales and mins of
// sub-blocks 2c and 2c+1, byte-parallel in bytes 0 and 1 of SC and MN.
// Sub-blocks 0..3 sit in the low six bits of scale bytes 0..7; 4..7 take four
// bits from bytes 8..11 and two from the top of bytes 0..7.  hd: the
// superblock's first 16 bytes (d, dmin, scales).
__device__ __forceinline__ void kq_scale_min(const uint4& hd, int c, uint32_t& SC, uint32_t& MN) {
  const int h = 16 * (c & 1);
  const uint32_t a0 = hd.y >> h, a1 = hd.z >> h, a2 = hd.w >> h;
  const bool lowsb = c < 2;
  SC = lowsb ? (a0 & 0x3F3Fu) : ((a2 & 0x0F0Fu) | ((a0 >> 2) & 0x3030u));
  MN = lowsb ? (a1 & 0x3F3Fu) : (((a2 >> 4) & 0x0F0Fu) | ((a1 >> 2) & 0x3030u));
}

// Q4_K: unit k is chunk c = k%4 (64 weights) of superblock k/4: quant bytes
// 32c..32c+31, whose low nibbles are the chunk's first 32 weights (sub-block
// 2c) and high nibbles the next 32 (sub-block 2c+1).  w = d*sc*q - dmin*m.
// q0, q1: the chunk's 32 quant bytes.
__device__ __forceinline__ float q4k_dot(const uint4& hd, const uint4& q0, const uint4& q1, int c, NT_XARGS) {
  const float d = h2f(hd.x & 0xffffu), dmin = h2f(hd.x >> 16);
  uint32_t SC, MN;
  kq_scale_min(hd, c, SC, MN);
  const uint32_t qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  int AH = 0, AL = 0, BH = 0, BL = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo4 = qv[i] & 0x0F0F0F0Fu, hi4 = (qv[i] >> 4) & 0x0F0F0F0Fu;
    AH = i == 0 ? dot4z(lo4, xh[0]) : dot4(lo4, xh[i], AH);
    AL = i == 0 ? dot4z(lo4, xl[0]) : dot4(lo4, xl[i], AL);
    BH = i == 0 ? dot4z(hi4, xh[8]) : dot4(hi4, xh[8 + i], BH);
    BL = i == 0 ? dot4z(hi4, xl[8]) : dot4(hi4, xl[8 + i], BL);
  }
  const int SA = (AH << 8) + AL, SB = (BH << 8) + BL;
  const float t = xs[0] * (float)(SC & 0xffu) * (float)SA + xs[1] * (float)(SC >> 8) * (float)SB;
  const float u = (float)(MN & 0xffu) * xf[0] + (float)(MN >> 8) * xf[1];
  return d * t - dmin * u;
}

__device__ __forceinline__ float unit_q4_k(uint32_t seg, int k, NT_XARGS) {
  const uint32_t blk = seg + 144u * (k >> 2);
  const int c = k & 3;
  return q4k_dot(ld128(blk), ld128(blk + 16 + 32 * c), ld128(blk + 32 + 32 * c), c, xh, xl, xs, xm, xf);
}

// Q5_K: the layout of Q4_K with 32 bytes qh between the scales and the
// nibbles (176 bytes per superblock).  Element l (< 32) of sub-block s takes
// its fifth bit from bit s of qh[l]; for chunk c the first 32 weights use
// bit 2c and the next 32 bit 2c+1.  q in 0..31, w = d*sc*q - dmin*m.
__device__ __forceinline__ float unit_q5_k(uint32_t seg, int k, NT_XARGS) {
  const uint32_t blk = seg + 176u * (k >> 2);
  const int c = k & 3;
  const uint4 hd = ld128(blk), h0 = ld128(blk + 16), h1 = ld128(blk + 32);
  const uint4 q0 = ld128(blk + 48 + 32 * c), q1 = ld128(blk + 64 + 32 * c);
  const float d = h2f(hd.x & 0xffffu), dmin = h2f(hd.x >> 16);
  uint32_t SC, MN;
  kq_scale_min(hd, c, SC, MN);
  const uint32_t qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  const uint32_t hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  const int sa = 2 * c, sb = 2 * c + 1;
  int AH = 0, AL = 0, BH = 0, BL = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo5 = (qv[i] & 0x0F0F0F0Fu) | (((hv[i] >> sa) & 0x01010101u) << 4);
    const uint32_t hi5 = ((qv[i] >> 4) & 0x0F0F0F0Fu) | (((hv[i] >> sb) & 0x01010101u) << 4);
    AH = i == 0 ? dot4z(lo5, xh[0]) : dot4(lo5, xh[i], AH);
    AL = i == 0 ? dot4z(lo5, xl[0]) : dot4(lo5, xl[i], AL);
    BH = i == 0 ? dot4z(hi5, xh[8]) : dot4(hi5, xh[8 + i], BH);
    BL = i == 0 ? dot4z(hi5, xl[8]) : dot4(hi5, xl[8 + i], BL);
  }
  const int SA = (AH << 8) + AL, SB = (BH << 8) + BL;
  const float t = xs[0] * (float)(SC & 0xffu) * (float)SA + xs[1] * (float)(SC >> 8) * (float)SB;
  const float u = (float)(MN & 0xffu) * xf[0] + (float)(MN >> 8) * xf[1];
  return d * t - dmin * u;
}

// Q6_K: unit k covers elements 64p..64p+63 of superblock k/4, p = k%4, i.e.
// half n = p/2, quarters q = 2h and 2h+1 (h = p%2).  Element 32q'+l of half n
// (q' = 0..3, l < 32) takes its low four bits from nibble q'/2 of
// ql[64n + 32(q'%2) + l], its high two bits from bits 2q'..2q'+1 of
// qh[32n + l], and scale sc[8n + 2q' + l/16].  w = d*sc*(q-32).
__device__ __forceinline__ float unit_q6_k(uint32_t seg, int k, NT_XARGS) {
  const int sb = k >> 2, p = k & 3, n = p >> 1, h = p & 1;
  const uint32_t blk = seg + 210u * sb;
  uint32_t qa[8], qb[8], qh[8], scw[1];
  ld_unaligned<8>(blk + 64 * n, qa);       // ql[64n .. 64n+31]
  ld_unaligned<8>(blk + 64 * n + 32, qb);  // ql[64n+32 .. 64n+63]
  ld_unaligned<8>(blk + 128 + 32 * n, qh); // qh[32n .. 32n+31]
  ld_unaligned<1>(blk + 192 + 8 * n + 4 * h, scw);
  const float d = h2f(ld16(blk + 208));
  const int sh = 4 * h;
  int H[4] = {0, 0, 0, 0}, L[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t hb = qh[i] >> sh;
    const uint32_t a = ((qa[i] >> sh) & 0x0F0F0F0Fu) | ((hb << 4) & 0x30303030u);
    const uint32_t b = ((qb[i] >> sh) & 0x0F0F0F0Fu) | ((hb << 2) & 0x30303030u);
    const bool first = (i & 3) == 0;
    H[i >> 2] = first ? dot4z(a, xh[i]) : dot4(a, xh[i], H[i >> 2]);
    L[i >> 2] = first ? dot4z(a, xl[i]) : dot4(a, xl[i], L[i >> 2]);
    H[2 + (i >> 2)] = first ? dot4z(b, xh[8 + i]) : dot4(b, xh[8 + i], H[2 + (i >> 2)]);
    L[2 + (i >> 2)] = first ? dot4z(b, xl[8 + i]) : dot4(b, xl[8 + i], L[2 + (i >> 2)]);
  }
  float acc = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int S = (H[g] << 8) + L[g] - 32 * xm[g];
    const int sc = (int)(int8_t)(scw[0] >> (8 * g));
    acc += (float)S * ((float)sc * xs[g >> 1]);
  }
  return d * acc;
}

#undef NT_XARGS

// ----------------------------------------------------------------- prologue
// Stage the activation: v = src (times the RMSNorm gains where the launch
// normalizes), then per 32-block s = max|v| / 32639, X = rint(v / s),
// hi = (X + 128) >> 8, lo = X - 256 hi.  Quantizing v rather than the
// normalized vector changes nothing but the block scales (a block's X do not
// depend on a common factor), so the normalization factor r is applied to
// the row sums in the epilogue, and no barrier is needed before the first
// weight loads.  A launch given an already quantized activation (ProArgs::qx,
// written by the epilogue of the launch before it) copies it instead.  For
// the QKV launch the prologue also tabulates the RoPE rotation of this
// position.
//
// Loads are coalesced: in round r thread t holds elements 4(NT r + t) ..
// +3, so the 8 lanes of an aligned lane group hold one 32-block and a
// wave's load covers 1 KB of consecutive bytes.  A wave's activation must
// have arrived (stage_load, stage_norm) before it issues its first weight
// loads: behind the launch's burst of weight requests an activation miss
// would wait several microseconds in the memory queues, and the quantization
// then overlaps the weights' latency instead.

constexpr int kXRounds = 8;  // rounds held in registers: inputs up to 4 * 1024 * 8 = 32768 wide

struct XStage {
  float4 v[kXRounds];  // src (times the gains once stage_norm has run); or the chunks of a quantized activation
  float4 g[kXRounds];  // RMSNorm gains
  int pos;             // RoPE position
};

// A quantized activation is copied with 16-byte loads, kXRounds per thread.
__device__ __forceinline__ int qx_chunks(const Job& job) { return (int)(qx_bytes(job.cols) / 16); }

__device__ __forceinline__ void qstage_load(const Job& job, const ProArgs& pro, int tid, XStage& st) {
  const int NT = job.nwaves * 64, nch = qx_chunks(job);
#pragma unroll
  for (int r = 0; r < kXRounds; ++r) {
    const int c = tid + NT * r;
    if (c < nch) st.v[r] = *reinterpret_cast<const float4*>(pro.qx + 16 * (int64_t)c);
  }
  st.pos = pro.rope_hd > 0 ? __builtin_nontemporal_load(pro.pos) + pro.pos_add : 0;
}

// The quantized activation's layout in memory is the staging area's in LDS
// (x_hi at 0, then x_lo, x_sc, x_sum, x_ss).
__device__ __forceinline__ void qstage_store(const Job& job, int tid, const XStage& st) {
  const int NT = job.nwaves * 64, nch = qx_chunks(job);
#pragma unroll
  for (int r = 0; r < kXRounds; ++r) {
    const int c = tid + NT * r;
    if (c < nch) st128(job.x_hi + 16u * (uint32_t)c, __builtin_bit_cast(uint4, st.v[r]));
  }
}

__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float4 mul4(float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); }
__device__ __forceinline__ float4 scale4(float4 a, float r) { return make_float4(a.x * r, a.y * r, a.z * r, a.w * r); }
__device__ __forceinline__ float sq4(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }

// Issues the loads of the source (and of the gains, with RMSNorm): thread t
// holds elements 4 (NT r + t) .. +3 of round r.
__device__ __forceinline__ void stage_load(const Job& job, const ProArgs& pro, int tid, XStage& st) {
  const int NT = job.nwaves * 64;
#pragma unroll
  for (int r = 0; r < kXRounds; ++r) {
    const int e = 4 * (NT * r + tid);
    if (e < job.cols) {
      st.v[r] = ld_f4(pro.src + e);
      if (pro.gain) st.g[r] = ld_f4(pro.gain + e);
    }
  }
  // after the activation's loads, so their latencies overlap
  st.pos = pro.rope_hd > 0 ? __builtin_nontemporal_load(pro.pos) + pro.pos_add : 0;
}

// Uses the loaded values (so their loads are waited for here, before any
// weight load is issued): the sum of squares of the source, then the gains
// applied in place.
__device__ __forceinline__ float stage_norm(const Job& job, const ProArgs& pro, int tid, XStage& st) {
  const int NT = job.nwaves * 64;
  float ss = 0.f;
  if (pro.gain) {
#pragma unroll
    for (int k = 0; k < kXRounds; ++k) {
      const int e = 4 * (NT * k + tid);
      if (e < job.cols) {
        ss += sq4(st.v[k]);
        st.v[k] = mul4(st.v[k], st.g[k]);
      }
    }
  } else {
    // a use of every loaded value, so the waits happen here
#pragma unroll
    for (int k = 0; k < kXRounds; ++k) {
      const int e = 4 * (NT * k + tid);
      if (e < job.cols) ss += st.v[k].x;
    }
  }
  if (pro.rope_hd > 0) ss += (float)(st.pos & 1) * 0.f;  // the position has arrived too
  return ss;
}

// Quantize elements e..e+3 (held by this lane, already scaled) into the LDS
// planes; the group's first lanes write the block scale and the 16-sums.
__device__ __forceinline__ void quant4(const Job& job, int lane, int e, float4 w) {
  float amax = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
  amax = max8(amax);
  const float f[4] = {w.x, w.y, w.z, w.w};
  uint32_t H = 0, L = 0;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int X = fx_quant(f[k], amax);
    H |= (uint32_t)(fx_hi(X) & 255) << (8 * k);
    L |= (uint32_t)(fx_lo(X) & 255) << (8 * k);
    sum += X;
  }
  *reinterpret_cast<uint32_t*>(nt_smem + job.x_hi + e) = H;
  *reinterpret_cast<uint32_t*>(nt_smem + job.x_lo + e) = L;
  sum = sum4(sum);
  if ((lane & 3) == 0) sti32(job.x_sum + 4u * (uint32_t)(e >> 4), sum);
  if ((lane & 7) == 0) stf(job.x_sc + 4u * (uint32_t)(e >> 5), amax / kXMax);
}


// ss: this thread's sum of squares from stage_norm.  The wave's part of the
// sum of squares of the source goes to the workgroup's table for the
// epilogue's normalization factor (norm_factor); no barrier here.
__device__ __forceinline__ void stage_ss(const Job& job, const ProArgs& pro, int tid, float ss) {
  if (!pro.gain) return;
  const int NT = job.nwaves * 64, lane = tid & 63;
  const int nround = (job.cols + 4 * NT - 1) / (4 * NT);
  // rounds past the registers (inputs wider than 4 * 64 * nwaves * kXRounds)
  for (int k = kXRounds; k < nround; ++k) {
    const int e = 4 * (NT * k + tid);
    if (e < job.cols) ss += sq4(ld_f4(pro.src + e));
  }
  ss = wave_sum(ss);
  if (lane == 0) stf(job.red + 4u * (tid >> 6), ss);
}

// The RMSNorm factor r = 1/sqrt(mean(src^2) + eps) of a normalizing launch
// (1 otherwise), after the prologue's barrier: from the waves' sums of
// squares (staged from fp32) or the blocks' (a quantized activation).
// Every wave adds the same values in the same order.
__device__ __forceinline__ float norm_factor(const Job& job, const ProArgs& pro, int lane) {
  float tot = 0.f;
  if (pro.qx) {
    if (!pro.qx_norm) return 1.0f;
    for (int b = lane; b < job.cols / 32; b += 64) tot += ldf(job.x_ss + 4u * (uint32_t)b);
    tot = wave_sum(tot);
  } else {
    if (!pro.gain) return 1.0f;
    for (int w = 0; w < job.nwaves; ++w) tot += ldf(job.red + 4u * w);
  }
  return 1.0f / sqrtf(tot / (float)job.cols + pro.eps);
}

// Cos and sin of the RoPE rotation of this position for the QKV epilogue.
__device__ __forceinline__ void rope_table(const Job& job, const ProArgs& pro, int tid, int pos) {
  if (pro.rope_hd <= 0) return;
  const int NT = job.nwaves * 64;
  // pair i turns by pos * theta^(-2i/head_dim); the angle is formed in
  // double so large positions keep fp32 accuracy
  for (int i = tid; i < pro.rope_hd / 2; i += NT) {
    const double freq = exp2(-(double)(2 * i) / (double)pro.rope_hd * log2((double)pro.rope_theta));
    const double ang = (double)pos * freq;
    stf(job.rope + 8u * i, (float)cos(ang));
    stf(job.rope + 8u * i + 4, (float)sin(ang));
  }
}

// Quantize the staged source (times the gains) into the LDS planes.  The
// caller ends the staging with a workgroup barrier.
__device__ __forceinline__ void stage_finish(const Job& job, const ProArgs& pro, int tid, XStage& st) {
  const int NT = job.nwaves * 64, lane = tid & 63;
  const int nround = (job.cols + 4 * NT - 1) / (4 * NT);
#pragma unroll
  for (int k = 0; k < kXRounds; ++k) {
    const int e = 4 * (NT * k + tid);
    if (e < job.cols) quant4(job, lane, e, st.v[k]);
  }
  for (int k = kXRounds; k < nround; ++k) {
    const int e = 4 * (NT * k + tid);
    if (e < job.cols) {
      float4 v = ld_f4(pro.src + e);
      if (pro.gain) v = mul4(v, ld_f4(pro.gain + e));
      quant4(job, lane, e, v);
    }
  }
}

// ----------------------------------------------------------- segment stream
// Workgroup b's share: units (rows, or row pairs for RoPE) b, b + G, b + 2G,
// ... of the G workgroups, interleaved so that every share takes the same
// mix of the launch's matrices (Q/K/V rows differ in format and size) and
// the same spread over the weight bytes.  Local row t of the share is global
// row srow(t); `nv` segment rows (twice the output rows with paired
// matrices) times `nslice` slices.  Segment id k = s * nv + v (slice-major),
// so a wave's successive claims mostly stay in one slice and its activation
// registers rarely change.  Everything here is wave-uniform and lives in
// scalar registers.
struct Share {
  int o0, no;      // global row of local row 0, output rows
  int ostep;       // global rows between consecutive units of the share
  int nv;          // segment rows
  int nseg;        // segments
  uint32_t magic;  // floor((2^32 - 1) / nv): slice of a segment id by a multiply
};

__device__ __forceinline__ Share share_of(const Job& job, int b) {
  Share sh;
  const bool big = b < job.wg_rem;
  const int nu = job.wg_base + (big ? 1 : 0);
  if (job.qblock) {
    // whole 32-row blocks, one contiguous range per workgroup
    sh.o0 = (b * job.wg_base + min(b, job.wg_rem)) * job.unit;
    sh.ostep = 1;
  } else {
    sh.o0 = b * job.unit;
    sh.ostep = job.grid * job.unit;
  }
  sh.no = nu * job.unit;
  sh.nv = job.paired ? 2 * sh.no : sh.no;
  sh.nseg = sh.nv * job.nslice;
  sh.magic = big ? job.magic[1] : job.magic[0];
  return sh;
}

// Global row of local row t of a share.
__device__ __forceinline__ int srow(const Job& job, const Share& sh, int t) {
  return job.unit == 2 ? sh.o0 + (t >> 1) * sh.ostep + (t & 1) : sh.o0 + t * sh.ostep;
}

// Byte range of one segment and where its data sits in the slab.
struct Seg {
  const uint8_t* a;  // 16-B aligned address of the first chunk
  int nchunks;
  uint32_t d;        // offset of the segment's first block from the first chunk
  int fmt;
  int nunits;        // column units in the slice
  int half;          // the last unit holds a single 32-weight block
  int s, v;          // slice and segment row
};

__device__ __forceinline__ Seg seg_at(const Job& job, const Share& sh, int k) {
  Seg sg;
  // s = k / nv: the multiply undershoots by at most one
  uint32_t q = __umulhi((uint32_t)k, sh.magic);
  int v = k - (int)q * sh.nv;
  if (v >= sh.nv) {
    ++q;
    v -= sh.nv;
  }
  const int s = (int)q;
  sg.s = s;
  sg.v = v;
  int m, row;
  if (job.paired) {
    const bool up = v >= sh.no;
    m = up ? 1 : 0;
    row = srow(job, sh, up ? v - sh.no : v);
  } else {
    row = srow(job, sh, v);
    m = (job.nmat > 2 && row >= job.row_base[2]) ? 2 : ((job.nmat > 1 && row >= job.row_base[1]) ? 1 : 0);
    row -= m == 2 ? job.row_base[2] : (m == 1 ? job.row_base[1] : 0);
  }
  // per-matrix fields by selects (a dynamic index would leave scalar registers)
  const uint8_t* W = m == 2 ? job.W[2] : (m == 1 ? job.W[1] : job.W[0]);
  const int64_t rb = m == 2 ? job.rb[2] : (m == 1 ? job.rb[1] : job.rb[0]);
  const int64_t sbytes = m == 2 ? job.slice_bytes[2] : (m == 1 ? job.slice_bytes[1] : job.slice_bytes[0]);
  sg.fmt = m == 2 ? job.fmt[2] : (m == 1 ? job.fmt[1] : job.fmt[0]);
  const uint8_t* ptr = W + (int64_t)row * rb + (int64_t)s * sbytes;
  const bool last = s == job.nslice - 1;
  const int ne = last ? job.last_ne : job.ups * 64;
  sg.nunits = last ? job.last_units : job.ups;
  sg.half = (ne & 63) != 0;
  const int64_t lbytes = m == 2 ? job.last_bytes[2] : (m == 1 ? job.last_bytes[1] : job.last_bytes[0]);
  const int64_t bytes = last ? lbytes : sbytes;
  sg.a = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(ptr) & ~uintptr_t(15));
  sg.d = (uint32_t)(ptr - sg.a);
  sg.nchunks = (int)((sg.d + bytes + 15) >> 4);
  return sg;
}

// Stand-in when a wave has no segment to load: an empty range at the start
// of the first matrix.  Loads are still issued for it (they return zeros
// without a memory access), so every path through the stream issues the
// same number of loads and the waits before a slab store count exactly the
// older segment (waits merge across paths pessimistically).
__device__ __forceinline__ Seg seg_null(const Job& job) {
  Seg sg;
  sg.a = job.W[0];
  sg.nchunks = 0;
  sg.d = 0;
  sg.fmt = job.fmt[0];
  sg.nunits = 0;
  sg.half = 0;
  sg.s = 0;
  sg.v = 0;
  return sg;
}

// Every lane issues exactly LPL loads (those past the segment's end return
// zeros without a memory access), so the number of loads in flight is the
// same on every path and the waits before the slab store count exactly the
// older segment.  A stand-in's loads complete at once: the epilogue, whose
// registers overlap the buffers, does not wait for memory behind them.
template <int LPL>
__device__ __forceinline__ void seg_load(const Seg& sg, int lane, uint4 (&pre)[LPL]) {
  const __amdgpu_buffer_rsrc_t r = seg_rsrc(sg.a, 16u * (uint32_t)sg.nchunks);
#pragma unroll
  for (int i = 0; i < LPL; ++i) pre[i] = load_seg_chunk(r, 16u * (uint32_t)(lane + 64 * i));
}

// The slab holds LPL KB, so every chunk slot is written (slots past the
// segment's end get zeros, which nothing reads): no divergent branch.
template <int LPL>
__device__ __forceinline__ void seg_store(uint32_t slab, int lane, const uint4 (&pre)[LPL]) {
#pragma unroll
  for (int i = 0; i < LPL; ++i) st128(slab + 16u * (lane + 64 * i), pre[i]);
}

// This lane's part of one segment's dot product, from the slab.
// FMT >= 0: every segment of the launch has that format (the other paths
// are compiled out); kFmtK46: Q4_K and Q6_K segments only (the K-quant mix
// of a Q/K/V launch); other FMT < 0: any format, read per segment.
template <int FMT>
__device__ __forceinline__ float seg_compute(const Seg& sg, uint32_t slab, int lane, const XR& xr) {
  const uint32_t seg = slab + sg.d;
  float acc = 0.f;
  const bool full = sg.nunits >= 64 * kUnitsPerLane && !sg.half;  // uniform
#pragma unroll
  for (int j = 0; j < kUnitsPerLane; ++j) {
    const int k = lane + 64 * j;
    if (full || k < sg.nunits) {
      switch (FMT >= 0 ? FMT : (FMT == kFmtK46 ? (sg.fmt == NT_Q6_K ? NT_Q6_K : NT_Q4_K) : sg.fmt)) {
        case NT_Q4_K: acc += unit_q4_k(seg, k, xr.hi[j], xr.lo[j], xr.sc[j], xr.sm[j], xr.sf[j]); break;
        case NT_Q6_K: acc += unit_q6_k(seg, k, xr.hi[j], xr.lo[j], xr.sc[j], xr.sm[j], xr.sf[j]); break;
        case NT_Q5_K: acc += unit_q5_k(seg, k, xr.hi[j], xr.lo[j], xr.sc[j], xr.sm[j], xr.sf[j]); break;
        case NT_Q8_0:
          acc += unit_q8_0(seg, k, !(sg.half && k == sg.nunits - 1), xr.hi[j], xr.lo[j], xr.sc[j], xr.sm[j], xr.sf[j]);
          break;
        default:
          acc += unit_q4_0(seg, k, !(sg.half && k == sg.nunits - 1), xr.hi[j], xr.lo[j], xr.sc[j], xr.sm[j], xr.sf[j]);
          break;
      }
    }
  }
  return acc;
}

// Sum of segment row v over the slices, in slice order (deterministic).
__device__ __forceinline__ float row_total(const Job& job, int v) {
  const uint32_t a = job.acc + 4u * (uint32_t)(v * job.nslice);
  float t = ldf(a);
  for (int s = 1; s < job.nslice; ++s) t += ldf(a + 4u * s);
  return t;
}

// A struct in the engine's LDS (the argument copies).
template <class T>
__device__ __forceinline__ const T& lds_ref(uint32_t off) {
  return *reinterpret_cast<const T*>(nt_smem + off);
}

// Copy the launch's argument structs into LDS (threads 0 .. ~110, one word
// each); the prologue's barrier publishes them.
template <class T>
__device__ __forceinline__ void copy_words(const T& v, uint32_t off, int i) {
  constexpr int n = (int)(sizeof(T) / 4);
  if (i >= 0 && i < n) sti32(off + 4u * (uint32_t)i, reinterpret_cast<const int*>(&v)[i]);
}
__device__ __forceinline__ void args_to_lds(const Job& job, const ProArgs& pro, const EpiArgs& ea, int tid) {
  constexpr int nj = (int)(sizeof(Job) / 4), np = (int)(sizeof(ProArgs) / 4);
  copy_words(job, kLdsJob, tid);
  copy_words(pro, kLdsPro, tid - nj);
  copy_words(ea, kLdsEpi, tid - nj - np);
}

// The epilogue's values from memory, loaded at the start so they have
// arrived when the stream ends: the residual and the gain of this thread's
// first output row, the layer's status word, the position.
struct EpiPre {
  float y = 0.f, g = 1.f;
  int err = 0, pos = 0;
};
template <int EPI>
__device__ __forceinline__ EpiPre epi_prefetch(const Job& job, const Share& sh, int tid, const EpiArgs& ea) {
  EpiPre p;
  if constexpr (EPI == EPI_RESID || EPI == EPI_SWIGLU) {
    if (tid < sh.no) {
      const int R = srow(job, sh, tid);
      if constexpr (EPI == EPI_RESID) p.y = ea.y[R];
      if (ea.qx_out && ea.qx_gain) p.g = ea.qx_gain[R];
    }
    if constexpr (EPI == EPI_RESID) {
      if (ea.err) p.err = *ea.err;
    }
  } else if constexpr (EPI == EPI_QKV) {
    p.pos = *ea.pos;
  }
  return p;
}

// Finish the workgroup's rows (after the barrier that follows the stream):
// thread t of `nthreads` handles output rows (or row pairs) t, t + nthreads,
// ...; r is the RMSNorm factor of the launch's input (norm_factor); pre
// holds what epi_prefetch loaded for the first of them.
template <int EPI>
__device__ __forceinline__ void share_epilogue(const Job& job, const Share& sh, int tid, int nthreads,
                                               const EpiArgs& ea, float r, const EpiPre& pre) {
  const bool qout = (EPI == EPI_RESID || EPI == EPI_SWIGLU) && ea.qx_out != nullptr;  // uniform
  float qv = 0.f;  // this thread's first output (row tid), for the quantized output
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    // a residual launch given the layer's status word turns the stream into
    // NaN when the layer's position was out of range
    const bool bad = EPI == EPI_RESID && pre.err != 0;
    for (int t = tid; t < sh.no; t += nthreads) {
      const float s = r * row_total(job, t);
      float* y = ea.y + srow(job, sh, t);
      if constexpr (EPI == EPI_RESID) {
        const float v = bad ? __builtin_nanf("") : (t == tid ? pre.y : *y) + s;
        *y = v;
        if (t == tid) qv = v;
        if (qout && sh.no > nthreads) stf(job.qo + 4u * (uint32_t)t, v);
      } else {
        *y = s;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int t = tid; t < sh.no; t += nthreads) {
      const float v = silu(r * row_total(job, t)) * (r * row_total(job, sh.no + t));
      ea.y[srow(job, sh, t)] = v;
      if (t == tid) qv = v;
      if (qout && sh.no > nthreads) stf(job.qo + 4u * (uint32_t)t, v);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int pos = pre.pos + ea.pos_add;
    // every position of the call (*pos .. *pos + n_tok - 1) must fit the
    // cache, or no token of the call writes its entries
    const bool pos_ok = pre.pos >= 0 && pre.pos + max(ea.n_tok, 1) - 1 < ea.max_ctx;
    // the layer's status word: every workgroup writes the same value
    if (ea.err && tid == 0) *ea.err = pos_ok ? 0 : 1;
    for (int t = tid; 2 * t < sh.no; t += nthreads) {
      const int R = srow(job, sh, 2 * t);  // even row of an adjacent pair (concatenated Q, K, V rows)
      float a = r * row_total(job, 2 * t), b = r * row_total(job, 2 * t + 1);
      const int dd = R % ea.head_dim;
      if (R < ea.q_rows + ea.kv_rows) {
        // RoPE: pair (2i, 2i+1) of a head turns by pos * theta^(-2i/head_dim)
        // (the prologue tabulated cos and sin)
        const float c = ldf(job.rope + 4u * dd), s = ldf(job.rope + 4u * dd + 4);
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
        const int64_t off = ((int64_t)kh * ea.max_ctx + pos) * ea.head_dim + dd;  // even: one aligned 32-bit word
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        *reinterpret_cast<uint32_t*>(cache + off) =
            (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
      }
    }
  }
  if (qout && sh.no <= nthreads) {
    // the share is whole 32-row blocks (qblock), one output per thread: the
    // half-waves of threads 0 .. no-1 quantize their block from registers
    // into the next launch's activation (times ea.qx_gain)
    if (tid < sh.no) {
      const int R = srow(job, sh, tid);
      qx_store_block32(ea.qx_out, job.orows, R >> 5, tid & 31, qv * (ea.qx_gain ? pre.g : 1.0f), qv);
    }
  } else if (qout) {
    // more rows than threads: through LDS, half-waves one block at a time
    __syncthreads();
    const int l = tid & 31;
    for (int blk = tid >> 5; blk < (sh.no >> 5); blk += nthreads >> 5) {
      const int t = 32 * blk + l, R = srow(job, sh, t);
      const float y = ldf(job.qo + 4u * (uint32_t)t);
      const float g = ea.qx_gain ? (t == tid ? pre.g : ea.qx_gain[R]) : 1.0f;
      qx_store_block32(ea.qx_out, job.orows, R >> 5, l, y * g, y);
    }
  }
}

// Next two segments for this wave: one claim of two consecutive ids on the
// workgroup's LDS counter.  Ids below 2 * nwaves were handed out statically
// (wave w: w and w + nwaves).
__device__ __forceinline__ int claim2(const Job& job, int lane) {
  int old = 0;
  int* ctr = static_cast<int*>(__builtin_assume_aligned(nt_smem + job.ctl, 16));
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return 2 * job.nwaves + __builtin_amdgcn_readfirstlane(old);
}

// One step of the stream: the segment in buffer `pre` (described by `sg`,
// id k_cur) is stored to the slab, the next segment's loads are issued into
// `pre`, and the stored segment is computed into its (row, slice) partial
// sum.  The other buffer holds segment k_nxt (already in flight).  Ids are
// claimed two at a time: the first step of a pair claims, the second takes
// the spare.  A step past the wave's last segment only issues its stand-in
// loads: the stream loop then has a single exit, at the bottom, so the wait
// analysis never sees the buffers' load order swapped.
template <int LPL, int FMT, bool FIRST>
__device__ __forceinline__ void stream_step(const Job& job, const Share& sh, int lane, uint32_t slab, int& k_cur,
                                            int& k_nxt, int& k_spare, bool& claiming, int& xslice, XR& xr,
                                            uint4 (&pre)[LPL], Seg& sg) {
  const Seg cur = sg;
  const bool valid = k_cur < sh.nseg;
  seg_store(slab, lane, pre);
  int k2 = sh.nseg;
  if (claiming) {
    if constexpr (FIRST) {
      k2 = claim2(job, lane);
      k_spare = k2 + 1;
    } else {
      k2 = k_spare;
    }
    claiming = k2 < sh.nseg;
  }
  sg = k2 < sh.nseg ? seg_at(job, sh, k2) : seg_null(job);
  seg_load(sg, lane, pre);
  if (valid) {
    if (cur.s != xslice) {
      load_xr(job, cur.s, lane, xr);
      xslice = cur.s;
    }
    const float part = wave_sum(seg_compute<FMT>(cur, slab, lane, xr));
    // every lane writes the same uniform value: no divergent branch
    stf(job.acc + 4u * (uint32_t)(cur.v * job.nslice + cur.s), part);
  }
  k_cur = k_nxt;
  k_nxt = k2;
}

}  // namespace
}  // namespace nt
