// nt_gemm.hip -- quantized small-M GEMM on int8 MFMA: Y[t][r] = sum_k W[r][k]
// X[t][k] for t < M <= 8 tokens, the verify pass of self-speculative decoding
// (p1 "Features": self-speculative decoding; p2 "Architecture et structure du
// code": several draft tokens checked in one pass).  Weights are read once
// for all M tokens.
//
//   staging   k_stage_m puts the M activation rows (optionally RMSNorm'ed)
//             into 16-bit fixed point: per token and 256-block a scale s and
//             integers X = 256 hi + lo.  The int8 planes are laid out as the
//             B operand of v_mfma_i32_16x16x32_i8 (column n = 2t + plane: hi,
//             lo), 512 contiguous bytes per 32-block, followed by the X sums
//             of each block's two 16-element halves per B column (zero in the
//             hi-plane column) and the scales.  Within a layer the reduce
//             launch before (and the attention combine) writes this layout
//             directly where its rows are whole 256-blocks (stage_block256).
//   product   One MFMA multiplies a 16-row x 32-weight tile of raw quants by
//             every token and plane with exact int32 sums.  Adjacent columns
//             are combined, S = 256 C_hi + C_lo (exact), and scaled:
//             y += alpha_r * (s S) - beta_r * (s sum X), where alpha and beta
//             are the row's scale and offset for that block in its format
//             (Q6_K: per 16-weight half, two MFMAs with the other half zeroed).
//             Up to four tokens fill only columns 0..7: over Q4_K one
//             v_mfma_i32_16x16x64_i8 then takes two 32-blocks, the second
//             block's activations in columns 8..15 (the paired form); over
//             Q6_K alone one 16x16x32 MFMA takes both 16-weight groups of a
//             block, one per column half (the split form).
//   stream    A wave streams tile-slices (16 rows x 256 columns: 16 row
//             pieces) HBM -> registers -> its LDS slab with 16-byte loads
//             (cached, range-checked buffer loads where the rows are whole
//             16-byte chunks apart), two in flight, as the GEMV engine
//             streams segments.  A unit (one tile over one column range) accumulates
//             in registers; units are claimed from an LDS counter inside the
//             workgroup's share of tiles and land in a (row, column range,
//             token) table that the epilogue adds in order (deterministic).
//   epilogue  Store, residual add, SwiGLU or RoPE + q store + f16 K/V append,
//             per token (token t sits at position pos + t).
//
// MFMA operand layout (measured on gfx950): A[i][k] in lane i + 16*(k/8),
// byte k%8; B[k][n] in lane n + 16*(k/8), byte k%8; C[i][n] in lane
// n + 16*(i/4), element i%4.  v_mfma_i32_16x16x64_i8: 16 bytes per lane,
// A[i][k] in lane i + 16*(k/16), B[k][n] in lane n + 16*(k/16), byte k%16
// (any order of the k slots that is the same in both operands gives the
// same product); C as above.

#include <algorithm>

#include "nt_dev.h"

namespace nt {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kStageThreads = 1024;

// ------------------------------------------------------------------ staging
// Workgroup (c, t) stages columns 4096 c .. 4096 c + 4095 of token t: thread
// groups of 8 lanes hold one 32-block (4 elements each, coalesced as in the
// GEMV prologue); a wave holds one 256-block, which shares one fixed-point
// scale (every lane takes part in the wave's maximum: lanes past the end hold
// zeros).  With gains, each workgroup first forms the token's sum of squares
// over the whole row, in the same order in every workgroup (the RMSNorm
// factor is the same everywhere); its own elements are among those loads.
__global__ __launch_bounds__(kStageThreads) void k_stage_m(const float* __restrict__ src, int64_t stride,
                                                           const float* __restrict__ gain, float eps, int cols,
                                                           uint8_t* __restrict__ xb, int4* __restrict__ xs,
                                                           float* __restrict__ xsc) {
  __shared__ float red[kStageThreads / 64];
  const int t = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const float* x = src + (int64_t)t * stride;
  const int base = 4 * kStageThreads * (int)blockIdx.x;
  const int e = base + 4 * tid;
  const bool ok = e < cols;
  float4 v = ok ? *reinterpret_cast<const float4*>(x + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 g = make_float4(1.f, 1.f, 1.f, 1.f);
  if (gain && ok) g = *reinterpret_cast<const float4*>(gain + e);
  float r = 1.0f;
  if (gain) {
    float ss = 0.f;
#pragma unroll 4
    for (int e2 = 4 * tid; e2 < cols; e2 += 4 * kStageThreads) {
      const float4 w = e2 == e ? v : *reinterpret_cast<const float4*>(x + e2);
      ss += w.x * w.x + w.y * w.y + w.z * w.z + w.w * w.w;
    }
    ss = wave_sum(ss);
    if (lane == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < kStageThreads / 64; ++w) tot += red[w];
    r = 1.0f / sqrtf(tot / (float)cols + eps);
  }
  if (gain) v = make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w);
  v = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
  const float amax = wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  const float inv = amax > 0.f ? kXMax / amax : 0.f;
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t H = 0, L = 0;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int X = __float2int_rn(f[k] * inv);
    X = max(-32639, min(32639, X));
    const int hi = (X + 128) >> 8;
    const int lo = X - (hi << 8);
    H |= (uint32_t)(hi & 255) << (8 * k);
    L |= (uint32_t)(lo & 255) << (8 * k);
    sum += X;
  }
  // elements k = 4g..4g+3 of block b (g = lane's place in its group):
  // B-layout lane n + 16*(k/8), byte k%8, for n = 2t (hi) and 2t + 1 (lo)
  const int b = e >> 5, gi = (e >> 2) & 7;
  const int s16 = sum4(sum);            // lanes gi<4: first half, gi>=4: second half
  const int other = dpp_i<0x141>(s16);  // row_half_mirror: the other half's sum
  if (ok) {
    uint8_t* blk = xb + 512 * (int64_t)b + 128 * (gi >> 1) + 4 * (gi & 1);
    *reinterpret_cast<uint32_t*>(blk + 8 * (2 * t)) = H;
    *reinterpret_cast<uint32_t*>(blk + 8 * (2 * t + 1)) = L;
    if (gi == 0) {
      // column 2t (hi plane) carries no X sums, column 2t + 1 (lo plane)
      // the block's two halves; the scale once per 256-block
      xs[(int64_t)b * kMaxTokens + t] = make_int4(0, 0, s16, other);
      if ((b & 7) == 0) xsc[(int64_t)(b >> 3) * kMaxTokens + t] = amax / kXMax;
    }
  }
}

// --------------------------------------------------------------------- GEMM
// Workgroup b's share: column range su = b / gps (tile-slices ts0 ..
// ts0 + nts_r - 1, 32-blocks from gb0) and output tiles [t0, t0 + nt) of it;
// nvt tiles to stream (2 nt with paired matrices); units u = sub * nvt + vt.
struct ShareM {
  int su, ts0, nts_r, gb0, nb;  // range, its tile-slices, first block and blocks
  int t0, nt, nvt, nsub, nunits;
  uint32_t magic;               // floor((2^32-1)/nvt)
};

__device__ __forceinline__ ShareM share_m(const JobM& job, int b) {
  ShareM sh;
  sh.su = b / job.gps;
  const int g = b - sh.su * job.gps;
  sh.ts0 = sh.su * job.tsper;
  sh.nts_r = min(job.tsper, job.nts - sh.ts0);
  sh.gb0 = 8 * sh.ts0;
  sh.nb = min(8 * (sh.ts0 + sh.nts_r), job.cols / 32) - sh.gb0;
  const bool big = g < job.wg_rem;
  sh.t0 = g * job.wg_base + (big ? g : job.wg_rem);
  sh.nt = job.wg_base + (big ? 1 : 0);
  sh.nvt = job.paired ? 2 * sh.nt : sh.nt;
  sh.nsub = (sh.nts_r + job.tsu - 1) / job.tsu;
  sh.nunits = sh.nvt * sh.nsub;
  sh.magic = big ? job.magicV[1] : job.magicV[0];
  return sh;
}

// One tile-slice: 16 row pieces of one matrix, the unit it belongs to and
// where it sits in that unit.  Wave-uniform (scalar registers).
struct TSeg {
  const uint8_t* base;  // first byte of row 0's piece
  const uint8_t* ab;    // its 16-byte aligned start (row strides of whole chunks)
  uint32_t nrec;        // bytes from ab to the matrix's end (0: a stand-in)
  uint32_t d;           // offset of the pieces in their first chunk (row strides of whole chunks)
  int64_t rb;
  int fmt, P, piece;    // chunks per piece (worst alignment), bytes per piece
  uint32_t magicP;
  int nrow;             // rows of the tile inside the matrix (<= 16)
  int nblk;             // 32-weight blocks in the tile-slice (<= 8)
  int lb0;              // first 32-block of the tile-slice, counted from the range's first
  int ts, tsb;          // tile-slice of the row, bytes of a full tile-slice row piece
  int vt, sub;          // unit
  int first, last;      // first / last tile-slice of its unit
};

__device__ __forceinline__ int unit_len(const JobM& job, const ShareM& sh, int sub) {
  return min(job.tsu, sh.nts_r - sub * job.tsu);
}

__device__ __forceinline__ void unit_of(const ShareM& sh, int u, int& sub, int& vt) {
  uint32_t q = __umulhi((uint32_t)u, sh.magic);
  vt = u - (int)q * sh.nvt;
  if (vt >= sh.nvt) {
    ++q;
    vt -= sh.nvt;
  }
  sub = (int)q;
}

__device__ __forceinline__ int matrix_of_tile(const JobM& job, int tile) {
  if (job.paired) return 0;
  return (job.nmat > 2 && tile >= job.tile_base[2]) ? 2 : ((job.nmat > 1 && tile >= job.tile_base[1]) ? 1 : 0);
}

__device__ __forceinline__ TSeg tseg_at(const JobM& job, const ShareM& sh, int u, int j) {
  TSeg sg;
  int sub, vt;
  unit_of(sh, u, sub, vt);
  sg.vt = vt;
  sg.sub = sub;
  sg.first = j == 0;
  sg.last = j == unit_len(job, sh, sub) - 1;
  const int lts = sub * job.tsu + j;  // tile-slice within the range
  const int ts = sh.ts0 + lts;
  int m, tile;
  if (job.paired) {
    const bool up = vt >= sh.nt;
    m = up ? 1 : 0;
    tile = sh.t0 + (up ? vt - sh.nt : vt);
  } else {
    tile = sh.t0 + vt;
    m = matrix_of_tile(job, tile);
  }
  const int lt = tile - (job.paired ? 0 : (m == 2 ? job.tile_base[2] : (m == 1 ? job.tile_base[1] : 0)));
  const uint8_t* W = m == 2 ? job.W[2] : (m == 1 ? job.W[1] : job.W[0]);
  sg.rb = m == 2 ? job.rb[2] : (m == 1 ? job.rb[1] : job.rb[0]);
  sg.fmt = m == 2 ? job.fmt[2] : (m == 1 ? job.fmt[1] : job.fmt[0]);
  sg.P = m == 2 ? job.P[2] : (m == 1 ? job.P[1] : job.P[0]);
  sg.magicP = m == 2 ? job.magicP[2] : (m == 1 ? job.magicP[1] : job.magicP[0]);
  const int tsb = m == 2 ? job.tsb[2] : (m == 1 ? job.tsb[1] : job.tsb[0]);
  const int rows = m == 2 ? job.rows[2] : (m == 1 ? job.rows[1] : job.rows[0]);
  sg.nrow = min(kTileRows, rows - kTileRows * lt);
  const bool kq = block_elems(sg.fmt) == 256;
  sg.nblk = kq ? 8 : min(8, (job.cols - kTS * ts) >> 5);
  sg.piece = kq ? tsb : sg.nblk * block_bytes(sg.fmt);
  sg.lb0 = 8 * lts;
  sg.ts = ts;
  sg.tsb = tsb;
  const int64_t r0 = (int64_t)(kTileRows * lt) * sg.rb, o = (int64_t)ts * tsb;
  sg.base = W + r0 + o;
  sg.d = (uint32_t)(o & 15);
  sg.ab = W + r0 + (o & ~(int64_t)15);
  sg.nrec = (uint32_t)((int64_t)rows * sg.rb - r0 - (o & ~(int64_t)15));
  return sg;
}

// The next tile-slice of the same unit (the next 256 columns of the same 16
// rows): only the column position moves, so this replaces tseg_at's matrix
// and unit lookups by a few scalar adds.
__device__ __forceinline__ TSeg tseg_next(const JobM& job, const TSeg& p, bool last) {
  TSeg sg = p;
  sg.first = 0;
  sg.last = last;
  sg.ts = p.ts + 1;
  sg.lb0 = p.lb0 + 8;
  const int nb = min(8, (job.cols - kTS * sg.ts) >> 5);  // 8 for the K-quants (whole superblocks)
  if (nb < 8) {
    sg.nblk = nb;
    sg.piece = nb * block_bytes(sg.fmt);
  }
  sg.base = p.base + p.tsb;
  sg.d = (p.d + (uint32_t)p.tsb) & 15u;
  sg.ab = sg.base - sg.d;
  sg.nrec = p.nrec - (uint32_t)(sg.ab - p.ab);
  return sg;
}

// Stand-in when a wave has nothing left: one chunk at the start of W[0]
// (loads are still issued, so every path issues the same number).
__device__ __forceinline__ TSeg tseg_null(const JobM& job) {
  TSeg sg{};
  sg.base = job.W[0];
  sg.ab = job.W[0];
  sg.nrec = 0;
  sg.d = 0;
  sg.rb = 0;
  sg.fmt = job.fmt[0];
  sg.P = 1;
  sg.piece = 1;
  sg.magicP = 65536;
  sg.nrow = 1;
  return sg;
}

// Chunk c of the tile-slice: row c / P, chunk c % P of that row's aligned
// range.  Chunks a row's piece does not reach (its alignment is better than
// the worst case) and chunks past 16 P re-read the row's or row 0's first
// chunk, so every chunk read holds a byte of the matrix.
template <int LPL>
__device__ __forceinline__ void tseg_load(const TSeg& sg, int lane, uint4 (&pre)[LPL]) {
#pragma unroll
  for (int i = 0; i < LPL; ++i) {
    const int c = lane + 64 * i;
    int r = (int)(((uint32_t)c * sg.magicP) >> 16);
    int k = c - r * sg.P;
    if (r >= kTileRows) {
      r = 0;
      k = 0;
    }
    const uint8_t* p = sg.base + (int64_t)min(r, sg.nrow - 1) * sg.rb;
    const uint32_t d = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 15);
    if (16 * k >= (int)d + sg.piece) k = 0;
    pre[i] = load_chunk(reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(p) & ~uintptr_t(15)) + 16 * k);
  }
}

// Matrices whose rows are whole 16-byte chunks apart (job.fast): every tile-
// slice's row pieces sit at the same offsets from its aligned start, so a
// lane's LPL chunk offsets (chunk c = lane + 64 i is chunk c % P of row
// c / P; past 16 P, chunk 0 of row 0) are kept while the matrix geometry
// (P, row stride) stays, and each tile-slice's loads are raw buffer loads
// from its aligned start whose range ends at the matrix's end: rows past the
// matrix read zeros (their results are never stored), a stand-in reads
// nothing.  The loads are cached (not non-temporal): a row piece (144 bytes
// of Q4_K, 210 of Q6_K) is not a whole number of 128-byte cache lines, so
// neighbouring tile-slices of a row share a line, and the wave that reads
// the next tile-slice a step later finds it in L2 (HBM bytes fetched per
// weight byte: 1.53 -> 1.16 for Q4_K, 1.58 -> 1.26 for Q6_K).
template <int LPL>
struct TLoad {
  int P = -1;
  int64_t rb = -1;
  uint32_t off[LPL] = {};
};

template <int LPL>
__device__ __forceinline__ void tseg_load_fast(const TSeg& sg, TLoad<LPL>& tl, int lane, uint4 (&pre)[LPL]) {
  if (sg.nrec != 0 && (sg.P != tl.P || sg.rb != tl.rb)) {
    tl.P = sg.P;
    tl.rb = sg.rb;
#pragma unroll
    for (int i = 0; i < LPL; ++i) {
      const int c = lane + 64 * i;
      const int r = (int)(((uint32_t)c * sg.magicP) >> 16);
      const int k = c - r * sg.P;
      tl.off[i] = r < kTileRows ? (uint32_t)r * (uint32_t)sg.rb + 16u * (uint32_t)k : 0u;
    }
  }
  const __amdgpu_buffer_rsrc_t rs = seg_rsrc(sg.ab, sg.nrec);
#pragma unroll
  for (int i = 0; i < LPL; ++i) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)tl.off[i], 0, 0);
    pre[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <int LPL>
__device__ __forceinline__ void tseg_store(uint32_t slab, int lane, const uint4 (&pre)[LPL]) {
#pragma unroll
  for (int i = 0; i < LPL; ++i) st128(slab + 16u * (lane + 64 * i), pre[i]);
}

// LDS offset of row r's piece data in the slab (rows past the tile re-read
// the last row, or with fixed-offset loads hold zeros: their results are
// never stored).
template <bool FAST>
__device__ __forceinline__ uint32_t piece_off(const TSeg& sg, uint32_t slab, int r) {
  if constexpr (FAST) return slab + 16u * (uint32_t)(sg.P * r) + sg.d;
  const int rr = min(r, sg.nrow - 1);
  const uint32_t d = (uint32_t)(reinterpret_cast<uintptr_t>(sg.base + (int64_t)rr * sg.rb) & 15);
  return slab + 16u * (uint32_t)(sg.P * r) + d;
}

__device__ __forceinline__ long pack2(uint32_t lo, uint32_t hi) { return (long)(((uint64_t)hi << 32) | lo); }

// Scale table of the tile-slice, per (entry, row), from the lanes that read
// row lane % 16: Q8_0 / Q4_0 the block's d (float, scl + 4 (16 block + row));
// Q4_K / Q5_K the sub-block's six-bit scale and min (int2, scl + 8 (16 j +
// row)); Q6_K the 16-weight group's signed scale (int, scl + 4 (16 g +
// row)).  Returns the row's superblock d (and dmin), K-quants only.
__device__ __forceinline__ float2 scale_table(const TSeg& sg, uint32_t po, uint32_t scl, int lane) {
  const int row = lane & 15, kq = lane >> 4;
  switch (sg.fmt) {
    case NT_Q8_0:
    case NT_Q4_0: {
      const uint32_t bb = sg.fmt == NT_Q8_0 ? 34u : 18u;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = kq + 4 * q;
        const float a = e < sg.nblk ? h2f(ld16(po + bb * e)) : 0.f;
        stf(scl + 4u * (uint32_t)(16 * e + row), a);
      }
      return make_float2(0.f, 0.f);
    }
    case NT_Q4_K:
    case NT_Q5_K: {  // same superblock header
      uint32_t h[3];
      ld_unaligned<3>(po + 4, h);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = kq + 4 * q;
        int sc, m;
        q4k_scale_min(h[0], h[1], h[2], e, sc, m);
        *reinterpret_cast<int2*>(nt_smem + scl + 8u * (uint32_t)(16 * e + row)) = make_int2(sc, m);
      }
      return make_float2(h2f(ld16(po)), h2f(ld16(po + 2)));
    }
    default: {  // Q6_K: 16 scales of 16 weights
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = kq + 4 * q;
        sti32(scl + 4u * (uint32_t)(16 * e + row), (int)(int8_t)nt_smem[po + 192 + e]);
      }
      return make_float2(h2f(ld16(po + 208)), 0.f);
    }
  }
}

// A operand: 8 quants (one byte each) of row lane%16, weights 8*(lane/16)..+7
// of block kb of the tile-slice.
// Two dwords at an 8-byte aligned LDS offset (AL) or at any 2-byte aligned one.
template <bool AL>
__device__ __forceinline__ void ld_pair(uint32_t off, uint32_t (&v)[2]) {
  if constexpr (AL) {
    const uint2 w = *reinterpret_cast<const uint2*>(nt_smem + off);
    v[0] = w.x;
    v[1] = w.y;
  } else {
    ld_unaligned<2>(off, v);
  }
}

// AL: the row pieces start 16-byte aligned (K-quant offsets below are then
// 8-byte aligned).
template <int F, bool AL = false>
__device__ __forceinline__ long a_operand(const TSeg& sg, uint32_t po, int kb, int kq) {
  uint32_t v[2];
  switch (F >= 0 ? F : sg.fmt) {
    case NT_Q8_0:
      ld_unaligned<2>(po + 34u * kb + 2 + 8 * kq, v);
      return pack2(v[0], v[1]);
    case NT_Q4_0: {
      ld_unaligned<2>(po + 18u * kb + 2 + 8 * (kq & 1), v);
      const int sh = 4 * (kq >> 1);
      return pack2((v[0] >> sh) & 0x0F0F0F0Fu, (v[1] >> sh) & 0x0F0F0F0Fu);
    }
    case NT_Q4_K: {
      ld_pair<AL>(po + 16 + 32 * (kb >> 1) + 8 * kq, v);
      const int sh = 4 * (kb & 1);
      return pack2((v[0] >> sh) & 0x0F0F0F0Fu, (v[1] >> sh) & 0x0F0F0F0Fu);
    }
    case NT_Q5_K: {  // Q4_K nibbles (after 32 bytes qh) plus bit kb of qh[l] as the fifth bit
      uint32_t h[2];
      ld_pair<AL>(po + 48 + 32 * (kb >> 1) + 8 * kq, v);
      ld_pair<AL>(po + 16 + 8 * kq, h);
      const int sh = 4 * (kb & 1);
      return pack2(((v[0] >> sh) & 0x0F0F0F0Fu) | (((h[0] >> kb) & 0x01010101u) << 4),
                   ((v[1] >> sh) & 0x0F0F0F0Fu) | (((h[1] >> kb) & 0x01010101u) << 4));
    }
    default: {  // Q6_K: elements 32 kb + 8 kq .. +7: half n, quarter q'
      // as the signed bytes q - 32 = ql + 16 (qh - 2): the high nibble is
      // (qh + 14) mod 16 (no carry leaves a byte: qh + 14 <= 17)
      const int n = kb >> 2, qq = kb & 3;
      uint32_t h[2];
      ld_unaligned<2>(po + 64 * n + 32 * (qq & 1) + 8 * kq, v);
      ld_unaligned<2>(po + 128 + 32 * n + 8 * kq, h);
      const int sl = 4 * (qq >> 1), shh = 2 * qq;
      const uint32_t a0 = ((v[0] >> sl) & 0x0F0F0F0Fu) | ((((h[0] >> shh) & 0x03030303u) + 0x0E0E0E0Eu) & 0x0F0F0F0Fu) << 4;
      const uint32_t a1 = ((v[1] >> sl) & 0x0F0F0F0Fu) | ((((h[1] >> shh) & 0x03030303u) + 0x0E0E0E0Eu) & 0x0F0F0F0Fu) << 4;
      return pack2(a0, a1);
    }
  }
}

__device__ __forceinline__ int mad24(int a, int b, int c) { return __mul24(a, b) + c; }

// One tile-slice (16 rows x 256 columns, one superblock of the K-quants)
// into this lane's accumulators: rows 4 kq .. 4 kq + 3 of the tile, token t,
// plane p (column 2 t + p of the products).  The activation's 256-block
// shares one scale s, so a K-quant superblock is summed exactly in integers
// first: AI = sum_j sc_j C_j over its sub-blocks (C_j the MFMA's sums of
// q X in this lane's plane) and, on the lo-plane lane only, MI = sum_j m_j
// SX_j (SX_j the sub-block's sum of X); with X = 256 hi + lo the
// superblock's contribution is s (256 P_hi + P_lo), P = d AI - dmin MI
// (Q6_K: P = d AI with the signed 16-weight scales, its quants entering the
// MFMA as q - 32).  Q8_0 / Q4_0 blocks carry their own fp16 d: P = sum_b d_b
// (C_b - off SX_b), off 8 for Q4_0.  Every bound: |AI| < 2^27 (Q6_K: 16
// groups of |sc| <= 128 times 16 products |q - 32| |plane| <= 32 x 128),
// |MI| < 2^30 (eight 32-sums of |X| <= 32639 times m <= 63); every factor
// of a 24-bit multiply-add fits 24 bits.
//
// BM 1 (up to four tokens, Q4_K): one v_mfma_i32_16x16x64_i8 covers
// the adjacent 32-blocks 2p and 2p + 1.  Lane group g = lane / 16 carries 16
// weights of block 2p + g / 2 (weights 16 (g % 2) .. + 15) in A and the same
// 16 activations in B, and the B tile (laid out by the prologue) holds block
// 2p's activations in columns 0..7 and block 2p + 1's in columns 8..15, zero
// elsewhere.  Column n of the product then sums block 2p + n / 8 alone, so
// the 16x16x32 form's empty columns (tokens 4..7) carry the second block:
// half the MFMAs and half the per-block scale work.  The two column halves
// of a token are added (integers, exact) before the row scales.  A Q6_K
// matrix of such a launch keeps the 16x16x32 form (its 16-weight scales
// would need two MFMAs per pair, and the pair form measured slower) and
// reads its B operand out of the paired tiles.
//
// BM 2 (up to four tokens, Q6_K alone): split B tiles of one 32-block, its
// activations 0..15 in columns 0..7 and 16..31 in columns 8..15, zero
// elsewhere: one v_mfma_i32_16x16x32_i8 per block gives both 16-weight
// groups' sums (column n: group 2 kb + n / 8), instead of two MFMAs with
// half of A zeroed; the halves are added as above.
template <int F, int LPL, bool AL, bool FAST, int BM = 0>
__device__ __forceinline__ void tseg_compute_f(const JobM& job, const TSeg& sg, uint32_t slab, uint32_t scl, int lane,
                                               float (&acc)[4]) {
  const int kq = lane >> 4, t = (lane & 15) >> 1;
  const uint32_t po = piece_off<FAST>(sg, slab, lane & 15);
  const float2 dd = scale_table(sg, po, scl, lane);
  if (sg.first) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = 0.f;
  }
  const v4i zero = {0, 0, 0, 0};
  constexpr bool kq_fmt = F == NT_Q4_K || F == NT_Q5_K || F == NT_Q6_K;
  int ai[4] = {0, 0, 0, 0}, mi[4] = {0, 0, 0, 0};
  float af[4] = {0.f, 0.f, 0.f, 0.f};
  const int hb = (lane >> 3) & 1;  // paired and split B tiles: this lane's column half
  auto block = [&](int kb) {
    const int lb = sg.lb0 + kb;
    const long a = a_operand<F, AL>(sg, po, kb, kq);
    // with the paired B tiles (BM 1, a Q6_K matrix in a launch with Q4_K
    // ones) this lane's 8 activations of column lane % 8 (columns 8..15
    // repeat 0..7: tokens past four, never stored)
    const uint32_t boa = BM == 1 ? job.xbl + 512u * (uint32_t)lb + 128u * (uint32_t)(lb & 1) + 16u * (uint32_t)(lane & 7) +
                                  256u * (uint32_t)(kq >> 1) + 8u * (uint32_t)(kq & 1)
                            : job.xbl + 512u * (uint32_t)lb + 8u * lane;
    const long bo = *reinterpret_cast<const long*>(nt_smem + boa);
    // the X sums of this lane's column: zero on the hi plane, so they enter once
    const int2 sx = *reinterpret_cast<const int2*>(nt_smem + job.xsl + 8u * (uint32_t)(16 * lb + (lane & 15)));
    const int sxa = sx.x, sxb = sx.y;
    if constexpr (F == NT_Q6_K && BM == 2) {
      // split B tile: column n sees the block's weights 16 (n / 8) .. + 15
      // alone, the 16-weight group 2 kb + n / 8
      const v4i c = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bo, zero, 0, 0, 0);
      const int4 g = *reinterpret_cast<const int4*>(nt_smem + scl + 4u * (uint32_t)(16 * (2 * kb + hb) + 4 * kq));
      const int s0[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) ai[j] = mad24(s0[j], c[j], ai[j]);
    } else if constexpr (F == NT_Q6_K) {
      // the quants enter as q - 32, so the offset is inside the exact sums
      const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(kq < 2 ? a : 0l, bo, zero, 0, 0, 0);
      const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(kq < 2 ? 0l : a, bo, zero, 0, 0, 0);
      const int4 g0 = *reinterpret_cast<const int4*>(nt_smem + scl + 4u * (uint32_t)(16 * (2 * kb) + 4 * kq));
      const int4 g1 = *reinterpret_cast<const int4*>(nt_smem + scl + 4u * (uint32_t)(16 * (2 * kb + 1) + 4 * kq));
      const int s0[4] = {g0.x, g0.y, g0.z, g0.w}, s1[4] = {g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) ai[j] = mad24(s1[j], c1[j], mad24(s0[j], c0[j], ai[j]));
    } else if constexpr (kq_fmt) {
      const v4i c = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bo, zero, 0, 0, 0);
      const uint32_t e = scl + 8u * (uint32_t)(16 * kb + 4 * kq);
      const int4 p0 = *reinterpret_cast<const int4*>(nt_smem + e);
      const int4 p1 = *reinterpret_cast<const int4*>(nt_smem + e + 16);
      const int sc[4] = {p0.x, p0.z, p1.x, p1.z}, m[4] = {p0.y, p0.w, p1.y, p1.w};
      const int sxs = sxa + sxb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ai[j] = mad24(sc[j], c[j], ai[j]);
        mi[j] = mad24(m[j], sxs, mi[j]);
      }
    } else {
      const v4i c = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bo, zero, 0, 0, 0);
      const float4 d4 = *reinterpret_cast<const float4*>(nt_smem + scl + 4u * (uint32_t)(16 * kb + 4 * kq));
      const float d[4] = {d4.x, d4.y, d4.z, d4.w};
      const int off = F == NT_Q4_0 ? 8 * (sxa + sxb) : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) af[j] = fmaf(d[j], (float)(c[j] - off), af[j]);
    }
  };
  if constexpr (BM == 1 && F == NT_Q4_K) {
    const uint32_t xq = job.xbl + 512u * (uint32_t)sg.lb0 + 16u * (uint32_t)lane;
    const uint32_t xsa = job.xsl + 8u * (uint32_t)(16 * (sg.lb0 + hb) + (lane & 7));
    // pairs UP at a time (more spill)
    constexpr int UP = 2;
#pragma unroll 1
    for (int pp = 0; pp < kTS / 64 / UP; ++pp) {
#pragma unroll
      for (int ph = 0; ph < UP; ++ph) {
        const int p = UP * pp + ph;
        const uint4 b4 = *reinterpret_cast<const uint4*>(nt_smem + xq + 1024u * p);
        const v4i b = {(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
        // qs bytes 16 (g % 2) .. + 15 of the pair's 32: block 2p in the low
        // nibbles, 2p + 1 in the high
        uint32_t v[4];
        if constexpr (AL) {
          const uint4 w = *reinterpret_cast<const uint4*>(nt_smem + po + 16u + 32u * p + 16u * (kq & 1));
          v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
        } else {
          ld_unaligned<4>(po + 16u + 32u * p + 16u * (kq & 1), v);
        }
        const int sh = 4 * (kq >> 1);
        const v4i a = {(int)((v[0] >> sh) & 0x0F0F0F0Fu), (int)((v[1] >> sh) & 0x0F0F0F0Fu),
                       (int)((v[2] >> sh) & 0x0F0F0F0Fu), (int)((v[3] >> sh) & 0x0F0F0F0Fu)};
        const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, zero, 0, 0, 0);
        const int2 sx = *reinterpret_cast<const int2*>(nt_smem + xsa + 256u * p);
        const uint32_t e = scl + 8u * (uint32_t)(16 * (2 * p + hb) + 4 * kq);
        const int4 p0 = *reinterpret_cast<const int4*>(nt_smem + e);
        const int4 p1 = *reinterpret_cast<const int4*>(nt_smem + e + 16);
        const int sc[4] = {p0.x, p0.z, p1.x, p1.z}, m[4] = {p0.y, p0.w, p1.y, p1.w};
        const int sxs = sx.x + sx.y;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ai[j] = mad24(sc[j], c[j], ai[j]);
          mi[j] = mad24(m[j], sxs, mi[j]);
        }
      }
    }
  } else if (sg.nblk == kTS / 32) {
    // blocks unrolled U at a time (more spill)
    constexpr int U = LPL >= 5 ? 1 : (F == NT_Q6_K && BM != 2 ? 2 : 4);
#pragma unroll 1
    for (int h = 0; h < kTS / 32; h += U) {
#pragma unroll
      for (int kb = 0; kb < U; ++kb) block(h + kb);
    }
  } else {
    for (int kb = 0; kb < sg.nblk; ++kb) block(kb);
  }
  if constexpr ((F == NT_Q4_K && BM == 1) || (F == NT_Q6_K && BM == 2)) {
    // a token's two column halves (lanes n and n + 8 of a row of 16)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ai[j] += dpp_i<0x128>(ai[j]);  // row_ror:8
      if constexpr (F == NT_Q4_K) mi[j] += dpp_i<0x128>(mi[j]);
    }
  }
  // the activation's scale of this 256-block, and the rows' d (dmin)
  const float s = ldf(job.xscl + 4u * (uint32_t)((sg.lb0 >> 3) * kMaxTokens + t));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float P;
    if constexpr (kq_fmt) {
      const int src = 4 * (4 * kq + j);  // a lane holding row 4 kq + j in scale_table
      const float d = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dd.x)));
      if constexpr (F == NT_Q6_K) {
        P = d * (float)ai[j];
      } else {
        const float dmin = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dd.y)));
        P = d * (float)ai[j] - dmin * (float)mi[j];
      }
    } else {
      P = af[j];
    }
    const float Pl = __int_as_float(dpp_i<0xB1>(__float_as_int(P)));  // quad_perm 1,0,3,2: the lo-plane lane's
    acc[j] = fmaf(s, fmaf(256.f, P, Pl), acc[j]);
  }
  if (sg.last && (lane & 1) == 0 && t < job.M && (BM == 0 || (lane & 8) == 0)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = kTileRows * sg.vt + 4 * kq + j;
      stf(job.acc + 4u * (uint32_t)((v * job.nsub + sg.sub) * job.M + t), acc[j]);
    }
  }
}

template <int LPL, bool FAST, int BM>
__device__ __forceinline__ void tseg_compute(const JobM& job, const TSeg& sg, uint32_t slab, uint32_t scl, int lane,
                                             float (&acc)[4]) {
  // row pieces laid out without alignment slack (the planner's exact P)
  // start 16-byte aligned
  const bool al = sg.P * 16 == sg.piece;
  if constexpr (BM == 1) {  // paired B tiles: Q4_K and Q6_K matrices only
    if (sg.fmt == NT_Q4_K) {
      if (al) tseg_compute_f<NT_Q4_K, LPL, true, FAST, 1>(job, sg, slab, scl, lane, acc);
      else tseg_compute_f<NT_Q4_K, LPL, false, FAST, 1>(job, sg, slab, scl, lane, acc);
    } else {
      tseg_compute_f<NT_Q6_K, LPL, false, FAST, 1>(job, sg, slab, scl, lane, acc);
    }
    return;
  }
  if constexpr (BM == 2) {  // split B tiles: Q6_K matrices only
    tseg_compute_f<NT_Q6_K, LPL, false, FAST, 2>(job, sg, slab, scl, lane, acc);
    return;
  }
  switch (sg.fmt) {
    case NT_Q4_K:
      if (al) tseg_compute_f<NT_Q4_K, LPL, true, FAST>(job, sg, slab, scl, lane, acc);
      else tseg_compute_f<NT_Q4_K, LPL, false, FAST>(job, sg, slab, scl, lane, acc);
      break;
    case NT_Q6_K: tseg_compute_f<NT_Q6_K, LPL, false, FAST>(job, sg, slab, scl, lane, acc); break;
    case NT_Q8_0: tseg_compute_f<NT_Q8_0, LPL, false, FAST>(job, sg, slab, scl, lane, acc); break;
    case NT_Q4_0: tseg_compute_f<NT_Q4_0, LPL, false, FAST>(job, sg, slab, scl, lane, acc); break;
    default:
      if (al) tseg_compute_f<NT_Q5_K, LPL, true, FAST>(job, sg, slab, scl, lane, acc);
      else tseg_compute_f<NT_Q5_K, LPL, false, FAST>(job, sg, slab, scl, lane, acc);
      break;
  }
}

// Cursor over a wave's units: the first two are static (wave w: units w and
// w + nwaves), later ones are claimed from the LDS counter.
struct UCur {
  int u, j, len;
  bool second_used, done;
};

__device__ __forceinline__ int claim_m(const JobM& job, int lane) {
  int old = 0;
  int* ctr = static_cast<int*>(__builtin_assume_aligned(nt_smem + job.ctl, 16));
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return 2 * job.nwaves + __builtin_amdgcn_readfirstlane(old);
}

__device__ __forceinline__ void ucur_set(const JobM& job, const ShareM& sh, UCur& c, int u) {
  c.u = u;
  c.j = 0;
  c.done = u >= sh.nunits;
  if (!c.done) {
    int sub, vt;
    unit_of(sh, u, sub, vt);
    c.len = unit_len(job, sh, sub);
  }
}

// Advance to the next tile-slice; before the LDS counter is initialised
// (may_claim false) only the static second unit can be taken, and a claim
// is left pending (u = -1).
__device__ __forceinline__ void ucur_next(const JobM& job, const ShareM& sh, UCur& c, int wave, int lane,
                                          bool may_claim) {
  if (c.done) return;
  if (++c.j < c.len) return;
  if (!c.second_used) {
    c.second_used = true;
    ucur_set(job, sh, c, wave + job.nwaves);
    return;  // when that unit does not exist, no later unit does
  }
  if (!may_claim) {
    c.u = -1;
    return;
  }
  ucur_set(job, sh, c, claim_m(job, lane));
}

// One step: store the tile-slice in `pre`, issue the next one's loads into
// `pre`, compute the stored one.  A step with nothing to compute only issues
// stand-in loads: the loop has a single exit (see the GEMV engine).
template <int LPL, bool FAST>
__device__ __forceinline__ void tseg_issue(const TSeg& sg, TLoad<LPL>& tl, int lane, uint4 (&pre)[LPL]) {
  if constexpr (FAST) tseg_load_fast(sg, tl, lane, pre);
  else tseg_load(sg, lane, pre);
}

template <int LPL, bool FAST, int BM>
__device__ __forceinline__ void stream_m(const JobM& job, const ShareM& sh, int wave, int lane, uint32_t slab,
                                         uint32_t scl, UCur& ah, float (&acc)[4], uint4 (&pre)[LPL], TSeg& sg,
                                         const TSeg& prev, TLoad<LPL>& tl, bool& cur_valid, bool& nxt_valid) {
  const TSeg cur = sg;
  const bool valid = cur_valid;
  tseg_store(slab, lane, pre);
  if (!ah.done && ah.u < 0) ucur_set(job, sh, ah, claim_m(job, lane));  // claim left pending before the barrier
  const bool issue = !ah.done;
  // past a unit's first tile-slice the one issued last (the other buffer's,
  // prev) is the slice before
  sg = issue ? (ah.j > 0 ? tseg_next(job, prev, ah.j == ah.len - 1) : tseg_at(job, sh, ah.u, ah.j)) : tseg_null(job);
  tseg_issue<LPL, FAST>(sg, tl, lane, pre);
  if (issue) ucur_next(job, sh, ah, wave, lane, true);
  if (valid) tseg_compute<LPL, FAST, BM>(job, cur, slab, scl, lane, acc);
  cur_valid = nxt_valid;
  nxt_valid = issue;
}

// Output row of share row v (tile v/16 of the share, row v%16; up rows of a
// paired launch are offset by orows), or -1 past the matrix.
__device__ __forceinline__ int64_t part_row(const JobM& job, const ShareM& sh, int v) {
  int vt = v / kTileRows, up = 0;
  if (job.paired && vt >= sh.nt) {
    vt -= sh.nt;
    up = 1;
  }
  const int tile = sh.t0 + vt;
  const int m = matrix_of_tile(job, tile);
  const int lr = kTileRows * (tile - (job.paired ? 0 : job.tile_base[m])) + v % kTileRows;
  if (lr >= job.rows[m]) return -1;
  return (int64_t)up * job.orows + job.row_base[m] + lr;
}

template <int LPL, bool FAST, int BM>
__global__ __launch_bounds__(kMaxThreads) void k_qgemm_m(JobM job) {
  const int tid = threadIdx.x, lane = tid & 63, NT = job.nwaves * 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ShareM sh = share_m(job, blockIdx.x);
  const uint32_t slab = job.slab + (uint32_t)wave * (uint32_t)(LPL * 1024);
  const uint32_t scl = job.scl + (uint32_t)wave * 1024u;
  if (tid == 0) sti32(job.ctl, 0);
  // the range's staged activation (B operands, X sums, scales), loaded before
  // any weight so waiting for it does not wait for the weights
  const int cb = 32 * sh.nb, cr = 8 * sh.nb, cs = 2 * ((sh.nb + 7) >> 3);  // 16-byte chunks
  uint4 xa[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = tid + NT * i;
    if (c < cb) {
      if constexpr (BM == 2) {
        // split form: chunk c % 32 of block c / 32 holds lanes l, l + 1 (l =
        // 2 (c % 32) = n + 16 kq): activations 8 kq .. + 7 of columns n % 8
        // and n % 8 + 1 where n / 8 == kq / 2, else zero
        const int l = 2 * (c & 31), n = l & 15, kq = l >> 4;
        if ((n >> 3) == (kq >> 1))
          xa[i] = *reinterpret_cast<const uint4*>(job.xb + 512 * ((int64_t)sh.gb0 + (c >> 5)) + 8 * ((n & 7) + 16 * kq));
        else
          xa[i] = make_uint4(0u, 0u, 0u, 0u);
      } else if constexpr (BM == 1) {
        // paired form: the B tile of blocks (2q, 2q + 1), lane l = n + 16 g:
        // block 2q + g / 2's activations 16 (g % 2) .. + 15 of column n % 8
        // where n / 8 == g / 2, else zero
        const int q = c >> 6, l = c & 63, n = l & 15, g = l >> 4;
        if ((n >> 3) == (g >> 1)) {
          const uint8_t* s = job.xb + 512 * ((int64_t)sh.gb0 + 2 * q + (g >> 1)) + 8 * ((n & 7) + 32 * (g & 1));
          const uint2 u0 = *reinterpret_cast<const uint2*>(s), u1 = *reinterpret_cast<const uint2*>(s + 128);
          xa[i] = make_uint4(u0.x, u0.y, u1.x, u1.y);
        } else {
          xa[i] = make_uint4(0u, 0u, 0u, 0u);
        }
      } else {
        xa[i] = *reinterpret_cast<const uint4*>(job.xb + 512 * (int64_t)sh.gb0 + 16 * c);
      }
    } else if (c < cb + cr)
      xa[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(job.xs) + 128 * (int64_t)sh.gb0 +
                                              16 * (c - cb));
    else if (c < cb + cr + cs)
      xa[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(job.xsc) + 4 * (int64_t)sh.gb0 +
                                              16 * (c - cb - cr));
  }
  // two tile-slices in flight before the barrier (static units only)
  UCur ah{};
  ah.second_used = false;
  ucur_set(job, sh, ah, wave);
  uint4 pa[LPL], pb[LPL];
  TSeg sa, sb;
  TLoad<LPL> tl;
  const bool va = !ah.done;
  sa = va ? tseg_at(job, sh, ah.u, ah.j) : tseg_null(job);
  tseg_issue<LPL, FAST>(sa, tl, lane, pa);
  if (va) ucur_next(job, sh, ah, wave, lane, false);
  const bool vb = !ah.done && ah.u >= 0;
  sb = vb ? tseg_at(job, sh, ah.u, ah.j) : tseg_null(job);
  tseg_issue<LPL, FAST>(sb, tl, lane, pb);
  if (vb) ucur_next(job, sh, ah, wave, lane, false);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = tid + NT * i;
    if (c < cb) st128(job.xbl + 16u * c, xa[i]);
    else if (c < cb + cr) st128(job.xsl + 16u * (c - cb), xa[i]);
    else if (c < cb + cr + cs) st128(job.xscl + 16u * (c - cb - cr), xa[i]);
  }
  __syncthreads();
  if (va) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    bool cur_valid = va, nxt_valid = vb;
    do {
      stream_m<LPL, FAST, BM>(job, sh, wave, lane, slab, scl, ah, acc, pa, sa, sb, tl, cur_valid, nxt_valid);
      stream_m<LPL, FAST, BM>(job, sh, wave, lane, slab, scl, ah, acc, pb, sb, sa, tl, cur_valid, nxt_valid);
    } while (cur_valid);
  }
  __syncthreads();
  // this range's partial sums of the share's rows: part[su][t][row], rows
  // fastest (coalesced), sub-ranges added in order
  const int nv = sh.nvt * kTileRows, M = job.M;
  for (int i = tid; i < nv * M; i += NT) {
    const int t = i / nv, v = i - t * nv;
    const int64_t R = part_row(job, sh, v);
    if (R < 0) continue;
    float s = 0.f;
    for (int sub = 0; sub < sh.nsub; ++sub) s += ldf(job.acc + 4u * (uint32_t)((v * job.nsub + sub) * M + t));
    job.part[((int64_t)sh.su * M + t) * job.ldp + R] = s;
  }
}

// ------------------------------------------------------------ reduce + epilogue
// Adds the column ranges' partial sums in order and applies the epilogue for
// (token, row) = thread (row pairs for EPI_QKV); see RedArgs for the RMSNorm
// factor of a prestaged input and the staging of the outputs.
template <int EPI>
__global__ __launch_bounds__(256) void k_reduce_m(const float* __restrict__ part, int nsup, int M, int64_t ldp,
                                                  int orows, ProArgs pro, EpiArgs ea, RedArgs ra) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // the column ranges' partial sums, added in order; the first 16 are
  // loaded at once (predicated), so their latencies overlap
  auto total = [&](int t, int64_t R) {
    const float* p = part + (int64_t)t * ldp + R;
    const int64_t st = (int64_t)M * ldp;
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = k < nsup ? p[k * st] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < nsup) s += v[k];
    for (int su = 16; su < nsup; ++su) s += p[su * st];
    return s;
  };
  // token t's RMSNorm factor (1 where the staging applied it): four
  // interleaved partial sums, so the loads go out together
  auto rnorm = [&](int t) {
    if (!ra.rn_ss) return 1.0f;
    const float* p = ra.rn_ss + (int64_t)t * ra.rn_nb;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    int b = 0;
#pragma unroll 4
    for (; b + 4 <= ra.rn_nb; b += 4) {
      s0 += p[b];
      s1 += p[b + 1];
      s2 += p[b + 2];
      s3 += p[b + 3];
    }
    for (; b < ra.rn_nb; ++b) s0 += p[b];
    return 1.0f / sqrtf(((s0 + s1) + (s2 + s3)) / (float)ra.rn_cols + ra.rn_eps);
  };
  if constexpr (EPI == EPI_QKV) {
    const int npr = orows / 2;
    if (i >= (int64_t)npr * M) return;
    const int t = (int)(i / npr), R = 2 * (int)(i - (int64_t)t * npr);
    const int pos = *ea.pos + t;
    // all M positions must fit the cache, or no token writes its entries;
    // the layer's status word says which
    const bool pos_ok = *ea.pos >= 0 && *ea.pos + M - 1 < ea.max_ctx;
    if (ea.err && i == 0) *ea.err = pos_ok ? 0 : 1;
    const float rn = rnorm(t);
    float a = rn * total(t, R), b = rn * total(t, R + 1);
    const int dd = R % ea.head_dim;
    if (R < ea.q_rows + ea.kv_rows) {
      // RoPE: the pair turns by pos * theta^(-dd/head_dim), the angle in double
      const double freq = exp2(-(double)dd / (double)pro.rope_hd * log2((double)pro.rope_theta));
      const double ang = (double)pos * freq;
      const float c = (float)cos(ang), s = (float)sin(ang);
      const float a2 = a * c - b * s, b2 = a * s + b * c;
      a = a2;
      b = b2;
    }
    if (R < ea.q_rows) {
      ea.q_out[t * ea.ld + R] = a;
      ea.q_out[t * ea.ld + R + 1] = b;
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
  } else {
    // (with staging, orows * M is a whole number of blocks: no block returns
    // in part)
    if (i >= (int64_t)orows * M) return;
    const int t = (int)(i / orows), R = (int)(i - (int64_t)t * orows);
    const float rn = rnorm(t);
    float v;
    if constexpr (EPI == EPI_SWIGLU) {
      v = silu(rn * total(t, R)) * (rn * total(t, (int64_t)orows + R));
    } else if constexpr (EPI == EPI_RESID) {
      // NaN when the layer's status word says a position was out of range
      const bool bad = ea.err && *ea.err != 0;
      v = bad ? __builtin_nanf("") : ea.y[t * ea.ld + R] + rn * total(t, R);
    } else {
      v = rn * total(t, R);
    }
    ea.y[t * ea.ld + R] = v;
    // the outputs staged for the next small-M GEMM (times the next gains)
    if (ra.st_stage)
      stage_block256(ra.st_gain ? v * ra.st_gain[R] : v, v, t, R, orows, static_cast<uint8_t*>(ra.st_stage), ra.st_ss);
  }
}

int gemm_cus() {
  int dev = 0, v = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  return v > 0 ? v : 256;
}

template <int LPL, bool FAST, int BM>
int launch_m_kernel(const JobM& job, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_qgemm_m<LPL, FAST, BM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024) != hipSuccess)
      return NT_EHIP;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_qgemm_m<LPL, FAST, BM>), dim3(job.grid), dim3(64 * job.nwaves), job.lds_bytes, stream, job);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

template <int LPL>
int launch_m_lpl(const JobM& job, hipStream_t stream) {
  if constexpr (LPL <= 4) {
    if (job.bmode == 1)
      return job.fast ? launch_m_kernel<LPL, true, 1>(job, stream) : launch_m_kernel<LPL, false, 1>(job, stream);
  }
  if constexpr (LPL == 4) {
    if (job.bmode == 2)
      return job.fast ? launch_m_kernel<LPL, true, 2>(job, stream) : launch_m_kernel<LPL, false, 2>(job, stream);
  }
  return job.fast ? launch_m_kernel<LPL, true, 0>(job, stream) : launch_m_kernel<LPL, false, 0>(job, stream);
}

template <int EPI>
int launch_reduce(const JobM& job, const ProArgs& pro, const EpiArgs& ea, const RedArgs& ra, hipStream_t stream) {
  const int64_t n = (int64_t)(EPI == EPI_QKV ? job.orows / 2 : job.orows) * job.M;
  const int64_t blocks = (n + 255) / 256;
  if (blocks <= 0) return NT_OK;
  hipLaunchKernelGGL(k_reduce_m<EPI>, dim3((unsigned)blocks), dim3(256), 0, stream, job.part, job.nsup, job.M, job.ldp,
                     job.orows, pro, ea, ra);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

}  // namespace

size_t stage_m_bytes(int cols) {
  const size_t nb = (size_t)(cols + 31) / 32;
  return nb * 512 + nb * kMaxTokens * 16 + (nb + 7) / 8 * kMaxTokens * 4;
}

// Column ranges of a launch: as few as the per-workgroup LDS allows.
static void ranges_m(int cols, int& nts, int& tsper, int& nsup) {
  nts = (cols + kTS - 1) / kTS;
  nsup = (nts + kMaxTsPer - 1) / kMaxTsPer;
  tsper = (nts + nsup - 1) / nsup;
  nsup = (nts + tsper - 1) / tsper;
}

size_t part_m_bytes(int64_t orows, int paired, int cols, int M) {
  int nts, tsper, nsup;
  ranges_m(cols, nts, tsper, nsup);
  return (size_t)nsup * (size_t)M * (size_t)(paired ? 2 : 1) * (size_t)orows * 4;
}

int launch_stage_m(const float* src, int64_t stride, const float* gain, float eps, int M, int cols, void* stage,
                   hipStream_t stream) {
  if (M < 1 || M > kMaxTokens || cols <= 0 || cols % 32) return NT_EINVAL;
  const size_t nb = (size_t)cols / 32;
  uint8_t* xb = static_cast<uint8_t*>(stage);
  int4* xs = reinterpret_cast<int4*>(xb + nb * 512);
  float* xsc = reinterpret_cast<float*>(xb + nb * 512 + nb * kMaxTokens * 16);
  const dim3 grid((unsigned)((cols + 4 * kStageThreads - 1) / (4 * kStageThreads)), (unsigned)M);
  hipLaunchKernelGGL(k_stage_m, grid, dim3(kStageThreads), 0, stream, src, stride, gain, eps, cols, xb, xs, xsc);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

// Geometry: tiles per matrix, column ranges, workgroups per range (about
// one workgroup per CU overall, enough that a share's table fits kAccM),
// units of about four per wave, chunks per row piece, the LDS layout.
int plan_job_m(JobM& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
               int pairs, int M) {
  if (nmat < 1 || nmat > kMaxMats || (paired && nmat != 2)) return NT_EINVAL;
  if (M < 1 || M > kMaxTokens) return NT_EINVAL;
  if (cols <= 0 || cols > kMaxCols) return NT_EUNSUPPORTED;
  job = JobM{};
  job.nmat = nmat;
  job.paired = paired;
  job.pairs = pairs;
  job.cols = cols;
  job.M = M;
  int64_t otiles = 0, orows = 0;
  int lpl = 3;
  for (int m = 0; m < nmat; ++m) {
    const int qk = block_elems(fmt[m]);
    if (qk == 0 || cols % qk != 0 || rows[m] < 0) return NT_EINVAL;
    if (qk == 1) return NT_EUNSUPPORTED;  // F16/F32 have their own kernel
    if (pairs && (rows[m] & 1)) return NT_EINVAL;
    if (paired && rows[m] != rows[0]) return NT_EINVAL;
    job.W[m] = W[m];
    job.fmt[m] = fmt[m];
    job.rows[m] = rows[m];
    job.rb[m] = (int64_t)(cols / qk) * block_bytes(fmt[m]);
    job.row_base[m] = paired ? 0 : (int)orows;
    job.tile_base[m] = paired ? 0 : (int)otiles;
    job.tsb[m] = (kTS / qk) * block_bytes(fmt[m]);
    // chunks per row piece: exact when every piece starts 16-byte aligned
    // (the rows' stride then keeps the 16 rows' reads on distinct LDS
    // banks), else room for the worst alignment
    const bool al16 = job.tsb[m] % 16 == 0 && job.rb[m] % 16 == 0 && (reinterpret_cast<uintptr_t>(W[m]) & 15) == 0;
    job.P[m] = al16 ? job.tsb[m] / 16 : (job.tsb[m] + 15 + 15) / 16;
    job.magicP[m] = (65536u + (uint32_t)job.P[m] - 1) / (uint32_t)job.P[m];
    lpl = std::max(lpl, (kTileRows * job.P[m] + 63) / 64);
    if (!paired || m == 0) {
      orows += rows[m];
      otiles += (rows[m] + kTileRows - 1) / kTileRows;
    }
  }
  job.tile_base[nmat] = (int)otiles;
  // rows whole 16-byte chunks apart (and each matrix under 4 GB, the reach
  // of a buffer load's offset): the kernel's fixed-offset tile loads
  job.fast = 1;
  for (int m = 0; m < nmat; ++m) {
    if (job.rb[m] % 16 != 0 || (reinterpret_cast<uintptr_t>(W[m]) & 15) != 0 ||
        (int64_t)rows[m] * job.rb[m] >= ((int64_t)1 << 32))
      job.fast = 0;
  }
  // up to four tokens (B columns 0..7): Q4_K (with Q6_K beside it) in the
  // paired 16x16x64 form, Q6_K alone in the split 16x16x32 form
  job.bmode = 0;
  if (M <= 4) {
    bool q4k = false, q6k = false, other = false;
    for (int m = 0; m < nmat; ++m) {
      q4k |= fmt[m] == NT_Q4_K;
      q6k |= fmt[m] == NT_Q6_K;
      other |= fmt[m] != NT_Q4_K && fmt[m] != NT_Q6_K;
    }
    job.bmode = other ? 0 : (q4k ? 1 : (q6k ? 2 : 0));
  }
  if (lpl > 4 || (job.bmode == 2 && lpl != 4)) job.bmode = 0;  // (Q4_K and Q6_K pieces take 3 and 4 loads per lane)
  if (lpl > kSlabLoads) return NT_EUNSUPPORTED;
  if (orows > INT32_MAX / 16) return NT_EUNSUPPORTED;
  job.lpl = lpl;
  job.orows = (int)orows;
  job.otiles = (int)otiles;
  const int vper = paired ? 2 : 1;
  job.ldp = (int64_t)vper * orows;
  ranges_m(cols, job.nts, job.tsper, job.nsup);
  job.nwaves = kMaxWaves;
  const int cus = gemm_cus();
  // workgroups per range, then units per tile so a workgroup has ~4 per wave
  int64_t gps = std::max<int64_t>(1, std::min<int64_t>(otiles, cus / job.nsup));
  const int64_t tiles_cap = kAccM / ((int64_t)kTileRows * vper * M);  // tiles a share's table holds with nsub = 1
  if (tiles_cap < 1) return NT_EUNSUPPORTED;
  gps = std::max<int64_t>(gps, (otiles + tiles_cap - 1) / tiles_cap);
  const int64_t nt_max = (otiles + gps - 1) / gps;
  const int64_t nvt = nt_max * vper;
  int64_t nsub = std::max<int64_t>(1, std::min<int64_t>(job.tsper, (4 * job.nwaves + nvt - 1) / nvt));
  while (nsub > 1 && nvt * kTileRows * nsub * M > kAccM) --nsub;
  job.tsu = (int)((job.tsper + nsub - 1) / nsub);
  job.nsub = (job.tsper + job.tsu - 1) / job.tsu;
  job.gps = (int)gps;
  job.grid = (int)(gps * job.nsup);
  job.wg_base = (int)(otiles / gps);
  job.wg_rem = (int)(otiles % gps);
  for (int i = 0; i < 2; ++i) {
    const int64_t n = (int64_t)(job.wg_base + i) * vper;
    job.magicV[i] = n > 0 ? (uint32_t)(0xffffffffull / (uint64_t)n) : 0u;
  }
  uint32_t off = 0;
  job.ctl = off; off += 16;
  job.xbl = off; off += (uint32_t)(8 * job.tsper * 512);
  job.xsl = off; off += (uint32_t)(8 * job.tsper * kMaxTokens * 16);
  job.xscl = off; off += (uint32_t)(job.tsper * kMaxTokens * 4);
  job.acc = off; off += (uint32_t)(nvt * kTileRows * job.nsub * M * 4);
  off = (off + 15) & ~15u;
  job.scl = off; off += (uint32_t)job.nwaves * 1024u;  // per wave: 16 entries x 16 rows x alpha (Q4_K: 8 x 16 x pairs)
  job.slab = off; off += (uint32_t)(job.nwaves * job.lpl * 1024);
  job.lds_bytes = off;
  if (job.lds_bytes > 160 * 1024) return NT_EUNSUPPORTED;
  return NT_OK;
}

int launch_gemm_m(JobM& job, const void* stage, void* part, const ProArgs& pro, int epi, const EpiArgs& ea,
                  hipStream_t stream, const RedArgs& ra) {
  // staging needs whole 256-blocks of rows per reduce block (not QKV's pairs)
  if (ra.st_stage && (epi == EPI_QKV || job.orows % 256 != 0)) return NT_EINVAL;
  if (ra.rn_ss && (ra.rn_nb <= 0 || ra.rn_cols <= 0)) return NT_EINVAL;
  if (job.otiles <= 0) return NT_OK;
  job.xb = static_cast<const uint8_t*>(stage);
  job.xs = reinterpret_cast<const int4*>(job.xb + (size_t)(job.cols / 32) * 512);
  job.xsc = reinterpret_cast<const float*>(job.xb + (size_t)(job.cols / 32) * (512 + kMaxTokens * 16));
  job.part = static_cast<float*>(part);
  int rc = NT_EUNSUPPORTED;
  switch (job.lpl) {
    case 3: rc = launch_m_lpl<3>(job, stream); break;
    case 4: rc = launch_m_lpl<4>(job, stream); break;
    case 5: rc = launch_m_lpl<5>(job, stream); break;
  }
  if (rc != NT_OK) return rc;
  switch (epi) {
    case EPI_STORE: return launch_reduce<EPI_STORE>(job, pro, ea, ra, stream);
    case EPI_RESID: return launch_reduce<EPI_RESID>(job, pro, ea, ra, stream);
    case EPI_QKV: return launch_reduce<EPI_QKV>(job, pro, ea, ra, stream);
    case EPI_SWIGLU: return launch_reduce<EPI_SWIGLU>(job, pro, ea, ra, stream);
  }
  return NT_EINVAL;
}

}  // namespace nt
