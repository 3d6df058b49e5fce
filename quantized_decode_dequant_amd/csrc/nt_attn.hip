// nt_attn.hip -- grouped-query decode attention over an f16 KV cache, plus
// the small kernels of a decode step (embedding row, argmax).
//
// Attention (p1 feature list: GQA and KV cache; p2 "Architecture et
// structure du code": softmax kernel): for query head h of kv group
// g = h / (n_head / n_kv), scores s_t = q_h . K_g[t] / sqrt(head_dim) over
// t = 0..n_pos-1, p = softmax(s), o_h = sum_t p_t V_g[t].
//
// Split over positions: workgroup (g, s) of a query takes positions
// [s*chunk, (s+1)*chunk) of kv head g for all query heads of the group, so
// every K/V byte is read once per query.  It writes an unnormalised partial
// (running max m, sum l, sum p*v) per head; k_attn_combine merges the
// splits.  The two products of a split run on f16 matrix cores
// (k_attn_split below).

#include <float.h>

#include <algorithm>

#include "nt_dev.h"

namespace nt {
namespace {

constexpr int kMaxGroup = 8;  // query heads per kv head
constexpr int kMaxSplits = 1024;  // position splits of one attention

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Split shape per head size: positions per split (K and V tiles of 16 KB
// each, 64 to 256 positions) over four waves, so a 4096-position cache of
// 8 kv heads makes ~520 workgroups, two per CU.  (Tiles of 256 positions
// over 16 waves at head_dim 128 -- 136 workgroups, a quarter of the
// partials -- took the split from 8.3 to 10.5 us per 70B layer and left
// the combine unchanged.)
template <int HD>
constexpr int attn_chunk() { return 8192 / HD < 64 ? 64 : (8192 / HD > 256 ? 256 : 8192 / HD); }
template <int HD>
constexpr int attn_waves() { return 4; }

// q: fp32 [n_query][n_head][HD] (query i at position pos+i attends to
// 0..pos+i).  Workgroup (g, s, i) takes split s of kv head g for query i:
// one launch covers every query of a verify pass, and the queries' reads of
// one K/V tile run at the same time (the later ones find it in the caches).
// Partials: part_o [n_query][nsplit][n_head][HD], part_ml
// [n_query][nsplit][n_head][2].
//
// Both products run on v_mfma_f32_16x16x32_f16 with the group's query heads
// as the 16 rows (rows past the group are zero).  K and V are f16 in the
// cache, so they enter exactly; q and the softmax numerators p are split as
// x = hi + lo (hi = f16(x), lo = f16(x - hi), about 22 significant bits) and
// each product is two MFMAs accumulating in fp32.
//   scores  S = Q K^T: of the NW waves, wave w takes positions
//           [w C/NW, (w+1) C/NW) in 16-column tiles, K loaded straight from
//           HBM in the B-operand layout;
//   P V     the V tile is staged position-major in LDS; each wave takes
//           output columns (16 dims per tile), over all positions, or over
//           one half of them when there are twice as many waves as tiles (the
//           two halves summed in LDS).
// Operand layout (16x16x32): A[i][k] in lane i + 16 (k / 8), element k % 8;
// B[k][n] in lane n + 16 (k / 8), element k % 8; C[i][n] in lane
// n + 16 (i / 4), element i % 4.
template <int HD>
__global__ __launch_bounds__(64 * attn_waves<HD>()) void k_attn_split(
    const float* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* pos_ptr, int n_head, int n_kv, int max_ctx, int nsplit, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int C = attn_chunk<HD>();
  constexpr int NW = attn_waves<HD>();           // waves per workgroup
  constexpr int NT = 64 * NW;                    // threads
  constexpr int KS = HD / 32;                    // k-steps of a score tile
  constexpr int PW = C / NW;                     // positions per wave (scores)
  constexpr int TW = PW / 16;                    // score tiles per wave
  constexpr int NTT = HD / 16;                   // output tiles
  constexpr int TPW = NTT >= NW ? NTT / NW : 1;  // output tiles per wave
  constexpr int KSPLIT = NW * TPW / NTT;         // waves per output tile (over position parts)
  constexpr int PKS = C / 32 / KSPLIT;           // P.V k-steps per wave
  constexpr int VST = HD + 8;                    // V row stride in LDS (f16), rows 16-byte aligned
  constexpr int NV = C * HD / 8 / NT;            // 16-byte V chunks per thread
  constexpr int CPR = HD / 8;                    // 16-byte chunks per row
  static_assert(TW >= 1 && NV >= 1 && PKS >= 1 && KSPLIT <= 2 && NV * NT * 8 == C * HD && TW * 16 * NW == C,
                "attention tile shape");
  __shared__ __attribute__((aligned(16))) _Float16 s_v[C * VST];
  __shared__ __attribute__((aligned(16))) _Float16 s_ph[kMaxGroup][C];
  __shared__ __attribute__((aligned(16))) _Float16 s_pl[kMaxGroup][C];
  __shared__ float s_s[kMaxGroup][C];
  __shared__ float s_m[kMaxGroup], s_l[kMaxGroup];
  __shared__ v4f s_red[KSPLIT > 1 ? NTT * 64 : 1];

  const int g = blockIdx.x, split = blockIdx.y, query = blockIdx.z;
  const int G = n_head / n_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  // the query rows do not depend on the position: their loads go out first,
  // beside the position's, and are converted once the K/V loads are issued
  const bool hv = r16 < G;
  float4 qa[KS], qb[KS];
  {
    const float* qp = q + ((int64_t)query * n_head + g * G + (hv ? r16 : 0)) * HD + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = *reinterpret_cast<const float4*>(qp + 32 * ks);
      qb[ks] = *reinterpret_cast<const float4*>(qp + 32 * ks + 4);
    }
  }
  // the position's load (and its wait) may not move above the query's loads
  __builtin_amdgcn_sched_barrier(0);
  const int pos = *pos_ptr;
  const int n_pos = pos + query + 1;
  const bool ok = pos >= 0 && pos + query < max_ctx;
  const int t0 = split * C;
  const int nt = ok ? max(0, min(C, n_pos - t0)) : 0;
  // a split past the position (a cache longer than the context so far, or an
  // out-of-range position) has nothing to do: the combine uses no partial of
  // it (nt is uniform, and no barrier has been reached)
  if (nt == 0) return;
  const uint16_t* kg = kc + ((int64_t)g * max_ctx + t0) * HD;
  const uint16_t* vg = vc + ((int64_t)g * max_ctx + t0) * HD;

  // all K and V loads of the tile up front (positions past the end re-read
  // row t0 and are masked).  K: lane (r16, q4) of wave w, tile j, step ks
  // holds dims 32 ks + 8 q4 .. +7 of position w PW + 16 j + r16.
  uint4 kb[TW][KS];
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int t = wave * PW + 16 * j + r16;
    const int64_t row = (int64_t)(t < nt ? t : 0) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[j][ks] = *reinterpret_cast<const uint4*>(kg + row + 32 * ks + 8 * q4);
  }
  {
    uint4 vr[NV];
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int c = tid + NT * r, t = c / CPR, d8 = c % CPR;
      vr[r] = *reinterpret_cast<const uint4*>(vg + (int64_t)(t < nt ? t : 0) * HD + 8 * d8);
    }
    // every K and V load is issued before the first wait for V
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int c = tid + NT * r, t = c / CPR, d8 = c % CPR;
      *reinterpret_cast<uint4*>(s_v + t * VST + 8 * d8) = vr[r];
    }
  }
  // query rows (heads of the group), scaled by 1/sqrt(HD), as hi + lo
  v8h qh[KS], ql[KS];
  {
    const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 a = qa[ks], b = qb[ks];
      const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = hv ? f[i] * scale : 0.f;
        const _Float16 hi = (_Float16)x;
        qh[ks][i] = hi;
        ql[ks][i] = (_Float16)(x - (float)hi);
      }
    }
  }

  // scores -> LDS s_s[h][t] (masked positions -inf)
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const v8h b = __builtin_bit_cast(v8h, kb[j][ks]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[ks], b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[ks], b, acc, 0, 0, 0);
    }
    const int t = wave * PW + 16 * j + r16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = 4 * q4 + e;
      if (h < G) s_s[h][t] = t < nt ? acc[e] : -INFINITY;
    }
  }
  __syncthreads();

  // softmax numerators (as hi + lo f16) and sums over this split, one wave per head
  for (int h = wave; h < G; h += NW) {
    float m = -FLT_MAX;
    for (int t = lane; t < nt; t += 64) m = fmaxf(m, s_s[h][t]);
    m = fmaxf(wave_max(m), -FLT_MAX);
    float l = 0.f;
    for (int t = lane; t < C; t += 64) {
      const float e = t < nt ? expf(s_s[h][t] - m) : 0.f;
      const _Float16 hi = (_Float16)e;
      s_ph[h][t] = hi;
      s_pl[h][t] = (_Float16)(e - (float)hi);
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      s_m[h] = m;
      s_l[h] = l;
    }
  }
  __syncthreads();

  // o = P V over this split
  const int tg = wave % (NW / KSPLIT), kp = wave / (NW / KSPLIT);
  const int hr = hv ? r16 : 0;
  v4f oacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) oacc[i] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < PKS; ++s) {
    const int tb = (kp * PKS + s) * 32 + 8 * q4;  // this lane's 8 positions
    const v8h zero = {};
    const v8h ah = hv ? *reinterpret_cast<const v8h*>(&s_ph[hr][tb]) : zero;
    const v8h al = hv ? *reinterpret_cast<const v8h*>(&s_pl[hr][tb]) : zero;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int d = 16 * (tg * TPW + i) + r16;
      v8h b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = s_v[(tb + e) * VST + d];
      oacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, b, oacc[i], 0, 0, 0);
      oacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, b, oacc[i], 0, 0, 0);
    }
  }
  if constexpr (KSPLIT > 1) {
    // the second position part hands its sums to the first
    if (kp == 1) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) s_red[(tg * TPW + i) * 64 + lane] = oacc[i];
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) oacc[i] += s_red[(tg * TPW + i) * 64 + lane];
    }
  }
  if (kp == 0) {
    float* dst = part_o + (((int64_t)query * nsplit + split) * n_head + g * G) * HD;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int d = 16 * (tg * TPW + i) + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = 4 * q4 + e;
        if (h < G) dst[(int64_t)h * HD + d] = oacc[i][e];
      }
    }
  }
  if (tid < G) {
    const int64_t mi = (((int64_t)query * nsplit + split) * n_head + g * G + tid) * 2;
    part_ml[mi] = s_m[tid];
    part_ml[mi + 1] = s_l[tid];
  }
}

// o[query][h][d] = sum_s e^(m_s - M) o_s[d] / sum_s e^(m_s - M) l_s over the
// splits that hold positions.  One workgroup per (head, 32 dims, query):
// thread (d, j) sums splits j, j + 8, ... of dimension d and the eight
// partial sums are added in order.  Once the position is known every load
// is issued at once (each thread's first eight splits of o with the (m, l)
// pairs), so the kernel waits on memory twice.
// With qx_o the 32 values of the workgroup (one 32-block of the output) also
// go out as a quantized activation of n_head * head_dim values per query.
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                      const int32_t* pos_ptr, int n_head, int head_dim, int chunk,
                                                      int nsplit, int max_ctx, float* __restrict__ o,
                                                      uint8_t* __restrict__ qx_o) {
  constexpr int kPre = 12;  // splits per thread held in registers
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[8];
  __shared__ float s_acc[8][32];
  const int nch = head_dim / 32;
  const int h = blockIdx.x / nch, d0 = 32 * (blockIdx.x % nch), query = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* ml = part_ml + ((int64_t)query * nsplit * n_head + h) * 2;
  const int dl = tid & 31, j = tid >> 5;
  const float* po = part_o + ((int64_t)query * nsplit * n_head + h) * head_dim + d0 + dl;
  const int64_t sst = (int64_t)n_head * head_dim;
  // the partials of every split that holds positions were written by this
  // attention's split kernel, so their loads go out with the position's;
  // splits past the position (their slots hold whatever an earlier call left)
  // are masked by selects below
  // (indices clamped to the last split rather than branched around, so all
  // loads issue back to back)
  float ov[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) ov[k] = po[min(j + 8 * k, nsplit - 1) * sst];
  const int sm = min(tid, nsplit - 1);
  float m0 = ml[(int64_t)sm * n_head * 2];
  float l0 = ml[(int64_t)sm * n_head * 2 + 1];
  __builtin_amdgcn_sched_barrier(0);
  const int pos = *pos_ptr;
  const bool ok = pos >= 0 && pos + query < max_ctx;
  const int n_pos = pos + query + 1;
  const int ns = ok ? min(nsplit, (n_pos + chunk - 1) / chunk) : 0;
  if (tid >= ns) {
    m0 = -FLT_MAX;
    l0 = 0.f;
  }
  // M = max over splits
  float m = m0;
  for (int s = tid + blockDim.x; s < ns; s += blockDim.x) m = fmaxf(m, ml[(int64_t)s * n_head * 2]);
  m = wave_max(m);
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  // weights e^(m_s - M) and L = sum of weighted l_s
  float lsum = 0.f;
  if (tid < ns) {
    const float w = expf(m0 - m);
    s_w[tid] = w;
    lsum = w * l0;
  }
  for (int s = tid + blockDim.x; s < ns; s += blockDim.x) {
    const float w = expf(ml[(int64_t)s * n_head * 2] - m);
    s_w[s] = w;
    lsum += w * ml[(int64_t)s * n_head * 2 + 1];
  }
  lsum = wave_sum(lsum);
  if (lane == 0) s_red[4 + wave] = lsum;
  __syncthreads();
  const float L = s_red[4] + s_red[5] + s_red[6] + s_red[7];
  const float inv = ns > 0 ? 1.0f / L : 0.f;
  float v = 0.f;
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int s = j + 8 * k;
    if (s < ns) v += s_w[s] * ov[k];
  }
  for (int s = j + 8 * kPre; s < ns; s += 8) v += s_w[s] * po[s * sst];
  s_acc[j][dl] = v;
  __syncthreads();
  if (tid < 32) {
    float t = s_acc[0][tid];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += s_acc[k][tid];
    const float v = t * inv;
    o[((int64_t)query * n_head + h) * head_dim + d0 + tid] = v;
    if (qx_o) {
      const int64_t n = (int64_t)n_head * head_dim;
      qx_store_block32(qx_o + query * qx_bytes(n), n, (h * head_dim + d0) >> 5, tid, v, v);
    }
  }
}

// ------------------------------------------------------------ embedding row
// Element e of an embedding row: the block definitions of nt.h.
__device__ __forceinline__ float embed_elem(int fmt, const uint8_t* __restrict__ row, int e) {
  auto h2f = [](const uint8_t* p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p[0] | (p[1] << 8))); };
  const int j = e & 31;
  if (fmt == NT_Q8_0) {
    const uint8_t* b = row + (int64_t)(e >> 5) * 34;
    return h2f(b) * (float)(int8_t)b[2 + j];
  }
  if (fmt == NT_Q4_0) {
    const uint8_t* b = row + (int64_t)(e >> 5) * 18;
    const int q = j < 16 ? (b[2 + j] & 15) : (b[2 + j - 16] >> 4);
    return h2f(b) * (float)(q - 8);
  }
  if (fmt == NT_F16) return h2f(row + 2 * (int64_t)e);
  if (fmt == NT_F32) return reinterpret_cast<const float*>(row)[e];
  if (fmt == NT_Q6_K) {
    const uint8_t* b = row + (int64_t)(e >> 8) * 210;
    const int i = e & 255, n = i >> 7, k = (i & 127) >> 5;
    const uint8_t lo = b[64 * n + 32 * (k & 1) + j];
    const int nib = (k >> 1) ? (lo >> 4) : (lo & 15);
    const int hi = (b[128 + 32 * n + j] >> (2 * k)) & 3;
    return h2f(b + 208) * (float)(int8_t)b[192 + i / 16] * (float)((nib | (hi << 4)) - 32);
  }
  // Q4_K and Q5_K: sub-block s of a 256-element superblock with 6-bit scale and min
  const int bb = fmt == NT_Q4_K ? 144 : 176;
  const uint8_t* b = row + (int64_t)(e >> 8) * bb;
  const int s = (e & 255) >> 5;
  const uint8_t* sc = b + 4;
  int scale, mn;
  if (s < 4) {
    scale = sc[s] & 63;
    mn = sc[s + 4] & 63;
  } else {
    scale = (sc[s + 4] & 15) | ((sc[s - 4] >> 6) << 4);
    mn = (sc[s + 4] >> 4) | ((sc[s] >> 6) << 4);
  }
  int q;
  if (fmt == NT_Q4_K) {
    const uint8_t v = b[16 + 32 * (s / 2) + j];
    q = (s & 1) ? (v >> 4) : (v & 15);
  } else {
    const uint8_t v = b[48 + 32 * (s / 2) + j];
    q = ((s & 1) ? (v >> 4) : (v & 15)) | (((b[16 + j] >> s) & 1) << 4);
  }
  return h2f(b) * (float)scale * (float)q - h2f(b + 2) * (float)mn;
}

// The combine for a small-M consumer: workgroup (b, query) merges the splits
// of output values 256 b .. 256 b + 255 (256 / head_dim heads of the query)
// as k_attn_combine does, writes them to o and stages them as one 256-block
// of the O projection's activation (stage_block256), so O needs no staging
// launch.  Thread (v, j) of the 1024 sums splits j, j + 4, ... of value v,
// the first 16 of them loaded before the position is known (clamped
// indices, masked below), and the four partial sums are added in order.
__global__ __launch_bounds__(1024) void k_attn_combine_st(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, const int32_t* pos_ptr,
                                                          int n_head, int head_dim, int chunk, int nsplit, int max_ctx,
                                                          float* __restrict__ o, uint8_t* __restrict__ stage) {
  constexpr int kPre = 16;  // splits per thread held in registers
  __shared__ float s_w[256 / 32][kMaxSplits];  // e^(m_s - M) per head of the block and split
  __shared__ float s_inv[256 / 32];
  __shared__ float s_acc[4][256];
  const int b = blockIdx.x, query = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vi = tid & 255, j = tid >> 8;
  const int nq = n_head * head_dim, hpb = 256 / head_dim, h0 = 256 * b / head_dim;
  const int d = 256 * b + vi, h = d / head_dim, dd = d - h * head_dim;
  const float* po = part_o + ((int64_t)query * nsplit * n_head + h) * head_dim + dd;
  const float* ml = part_ml + (int64_t)query * nsplit * n_head * 2;
  const int64_t sst = (int64_t)n_head * head_dim;
  float ov[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) ov[k] = po[min(j + 4 * k, nsplit - 1) * sst];
  __builtin_amdgcn_sched_barrier(0);
  const int pos = *pos_ptr;
  const bool ok = pos >= 0 && pos + query < max_ctx;
  const int ns = ok ? min(nsplit, (pos + query + 1 + chunk - 1) / chunk) : 0;
  // per head (one wave each): M = max over splits, the weights and 1 / L
  if (wave < hpb) {
    const float* mh = ml + (int64_t)(h0 + wave) * 2;
    float m = -FLT_MAX;
    for (int s = lane; s < ns; s += 64) m = fmaxf(m, mh[(int64_t)s * n_head * 2]);
    m = wave_max(m);
    float l = 0.f;
    for (int s = lane; s < ns; s += 64) {
      const float w = expf(mh[(int64_t)s * n_head * 2] - m);
      s_w[wave][s] = w;
      l += w * mh[(int64_t)s * n_head * 2 + 1];
    }
    l = wave_sum(l);
    if (lane == 0) s_inv[wave] = ns > 0 ? 1.0f / l : 0.f;
  }
  __syncthreads();
  const float* wv = s_w[h - h0];
  float v = 0.f;
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int s = j + 4 * k;
    if (s < ns) v += wv[s] * ov[k];
  }
  for (int s = j + 4 * kPre; s < ns; s += 4) v += wv[s] * po[s * sst];
  s_acc[j][vi] = v;
  __syncthreads();
  float y = 0.f;
  if (tid < 256) {
    y = ((s_acc[0][tid] + s_acc[1][tid]) + s_acc[2][tid] + s_acc[3][tid]) * s_inv[h - h0];
    o[(int64_t)query * nq + d] = y;
  }
  stage_block256(y, y, query, d, nq, stage, nullptr);
}

// x[m][:] = decoded row tokens[m] of an embedding matrix (fp32), one thread
// per element.  It also clears the step's status word (err), which the layers
// set when a position is out of range.
// With qx the row times qx_gain also goes out as a quantized activation
// (qx_bytes(cols) per token; cols is then a multiple of 128, so the 32 lanes
// of a block are all active).
__global__ __launch_bounds__(256) void k_embed(int fmt, const uint8_t* __restrict__ E, const int32_t* tokens, int vocab,
                                               int cols, float* __restrict__ x, int* __restrict__ err,
                                               uint8_t* __restrict__ qx, const float* __restrict__ qx_gain) {
  const int m = blockIdx.y;
  if (err && m == 0 && blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
  int tok = tokens[m];
  tok = min(max(tok, 0), vocab - 1);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= cols) return;
  const uint8_t* row = E + (int64_t)tok * (cols / block_elems(fmt)) * block_bytes(fmt);
  const float y = embed_elem(fmt, row, e);
  x[(int64_t)m * cols + e] = y;
  if (qx) qx_store_block32(qx + (int64_t)m * qx_bytes(cols), cols, e >> 5, e & 31, qx_gain ? y * qx_gain[e] : y, y);
}

// ------------------------------------------------------------------ argmax
// Greedy sampling (p2 "Architecture et structure du code": sampler): index
// of the largest logit, lowest index among equal maxima.
__device__ __forceinline__ void better(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__global__ __launch_bounds__(256) void k_argmax_part(const float* __restrict__ logits, int n, int per_block,
                                                     float* __restrict__ pv, int* __restrict__ pi) {
  const int m = blockIdx.y;
  const float* lg = logits + (int64_t)m * n;
  const int b0 = blockIdx.x * per_block, b1 = min(n, b0 + per_block);
  float v = -INFINITY;
  int idx = INT32_MAX;
  for (int i = b0 + threadIdx.x; i < b1; i += blockDim.x) better(v, idx, lg[i], i);
  for (int o = 32; o > 0; o >>= 1) better(v, idx, __shfl_xor(v, o, 64), __shfl_xor(idx, o, 64));
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = v;
    si[threadIdx.x >> 6] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) better(v, idx, sv[w], si[w]);
    pv[(int64_t)m * gridDim.x + blockIdx.x] = v;
    pi[(int64_t)m * gridDim.x + blockIdx.x] = idx;
  }
}

// A step whose status word is set (a position out of range) writes -1.
__global__ __launch_bounds__(64) void k_argmax_final(const float* __restrict__ pv, const int* __restrict__ pi, int nparts,
                                                     const int* __restrict__ err, int32_t* __restrict__ out) {
  const int m = blockIdx.x;
  float v = -INFINITY;
  int idx = INT32_MAX;
  for (int i = threadIdx.x; i < nparts; i += 64) better(v, idx, pv[(int64_t)m * nparts + i], pi[(int64_t)m * nparts + i]);
  for (int o = 32; o > 0; o >>= 1) better(v, idx, __shfl_xor(v, o, 64), __shfl_xor(idx, o, 64));
  if (threadIdx.x == 0) out[m] = (err && *err != 0) ? -1 : (idx == INT32_MAX ? 0 : idx);
}

}  // namespace

// Split geometry: attn_chunk positions per split.  Independent of the
// device, so workspace sizes are.
void attn_plan(int head_dim, int max_ctx, int& chunk, int& nsplit) {
  switch (head_dim) {
    case 32: chunk = attn_chunk<32>(); break;
    case 64: chunk = attn_chunk<64>(); break;
    case 128: chunk = attn_chunk<128>(); break;
    default: chunk = attn_chunk<256>(); break;
  }
  nsplit = (max_ctx + chunk - 1) / chunk;
}

int launch_attention(const float* q, const uint16_t* kc, const uint16_t* vc, const int32_t* pos, int n_query,
                     int n_head, int n_kv, int head_dim, int max_ctx, int chunk, int nsplit, float* part_o,
                     float* part_ml, float* o, uint8_t* qx_o, hipStream_t stream, uint8_t* stage_o) {
  // traced: the interval from the split launch's start to the combine's end
  hipEvent_t t0, t1;
  (void)trace_events(NT_TRACE_ATTN, &t0, &t1);
  const dim3 grid(n_kv, nsplit, n_query);
#define NT_ATTN_CASE(HD)                                                                                      \
  case HD:                                                                                                    \
    hipExtLaunchKernelGGL(k_attn_split<HD>, grid, dim3(64 * attn_waves<HD>()), 0, stream, t0, nullptr, 0, q, kc, vc, \
                          pos, n_head, n_kv, max_ctx, nsplit, part_o, part_ml);                              \
    break;
  switch (head_dim) {
    NT_ATTN_CASE(32)
    NT_ATTN_CASE(64)
    NT_ATTN_CASE(128)
    NT_ATTN_CASE(256)
    default: return NT_EUNSUPPORTED;
  }
#undef NT_ATTN_CASE
  if (stage_o) {
    if ((n_head * head_dim) % 256 != 0 || qx_o) return NT_EINVAL;
    hipExtLaunchKernelGGL(k_attn_combine_st, dim3(n_head * head_dim / 256, n_query), dim3(1024), 0, stream, nullptr, t1,
                          0, part_o, part_ml, pos, n_head, head_dim, chunk, nsplit, max_ctx, o, stage_o);
  } else {
    hipExtLaunchKernelGGL(k_attn_combine, dim3(n_head * (head_dim / 32), n_query), dim3(256), 0, stream, nullptr, t1, 0,
                          part_o, part_ml, pos, n_head, head_dim, chunk, nsplit, max_ctx, o, qx_o);
  }
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

int launch_embed(int fmt, const void* E, const int32_t* tokens, int M, int vocab, int cols, float* x, int* err,
                 uint8_t* qx, const float* qx_gain, hipStream_t stream) {
  hipLaunchKernelGGL(k_embed, dim3((cols + 255) / 256, M), dim3(256), 0, stream, fmt,
                     static_cast<const uint8_t*>(E), tokens, vocab, cols, x, err, qx, qx_gain);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

int argmax_parts(int n) { return std::min(256, (n + 1023) / 1024); }

int launch_argmax(const float* logits, int M, int n, float* pv, int* pi, const int* err, int32_t* out,
                  hipStream_t stream) {
  const int parts = argmax_parts(n);
  const int per = (n + parts - 1) / parts;
  hipLaunchKernelGGL(k_argmax_part, dim3(parts, M), dim3(256), 0, stream, logits, n, per, pv, pi);
  hipLaunchKernelGGL(k_argmax_final, dim3(M), dim3(64), 0, stream, pv, pi, parts, err, out);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

}  // namespace nt
