// nt_gemv.hip -- the quantized GEMV engine for gfx950.
//
// One engine serves every projection of the decode (GEMV is the per-token
// kernel the ntransformer pages list first; p2 "Architecture et structure du
// code").  One workgroup runs per CU.
//
//   prologue  The activation vector (optionally RMSNorm'ed with gains) is
//             staged on chip as 16-bit fixed point per 32-element block: an
//             fp32 scale s_b and integers X in [-32639, 32639], split into a
//             high and a low int8 plane (X = 256*hi + lo) plus per-16 sums of
//             X.  Weight x activation products then run on v_dot4_i32_i8
//             with exact integer sums per quantization sub-block.  Its loads
//             are issued before the first weight loads, so it does not wait
//             for them.
//   columns   A lane owns one 64-weight column unit of the current column
//             slice (4096 weights) and keeps its staged activation in
//             registers, reloaded only when the wave moves to another slice.
//   schedule  Workgroup b owns output rows (or RoPE row pairs) b, b + G,
//             b + 2G, ... of the G workgroups, so every share holds the same
//             mix of matrices; its work is a list of segments (one row of
//             one matrix within one column slice: a contiguous byte range),
//             slice-major.  Waves claim segments two at a time from an LDS
//             counter, so the waves that the SIMD arbiter favours simply take
//             more of them and all finish together.
//   stream    Segments move HBM -> registers with 16-byte coalesced
//             non-temporal loads, two in flight per wave while the previous
//             one is written to the wave's LDS slab and computed: lanes read
//             their blocks from the slab at any byte alignment (Q8_0, Q4_0
//             and Q6_K blocks are only 2-byte aligned), unpack quants in
//             registers and accumulate.
//   reduce    Per segment, a butterfly over the wave's lanes into an LDS
//             table of (row, slice) partial sums.
//   epilogue  After a workgroup barrier, each output row adds its slices in
//             order (deterministic) and is stored: plain, residual add,
//             SwiGLU (gate and up rows) or RoPE + q store + f16 K/V append
//             (row pairs).
//
// The block layouts are the GGUF ones the pages' format list refers to
// (p1 "About"); the unpacking below follows them.

#include <algorithm>

#include "nt_engine.h"

namespace nt {
namespace {


template <int EPI, int LPL, int FMT>
__global__ __launch_bounds__(kMaxThreads) void k_qgemv(Job job, ProArgs pro_in, EpiArgs ea) {
  constexpr bool kBurst = EPI == EPI_STORE_BURST;
  // a burst launch has no RMSNorm and no RoPE (the host checks): with the
  // gains known absent, their registers stay free for the weight buffers
  ProArgs pro = pro_in;
  if constexpr (kBurst) {
    pro.gain = nullptr;
    pro.rope_hd = 0;
    pro.qx_norm = 0;
  }
  const bool qin = pro.qx != nullptr;  // a quantized activation to copy (uniform)
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: keep everything derived from it (segment ids
  // and addresses) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Share sh = share_of(job, blockIdx.x);
  const uint32_t slab = job.slab + (uint32_t)wave * (uint32_t)(LPL * 1024);
  if (tid == 0) sti32(job.ctl, 0);  // claim counter; the prologue's barrier publishes it
  args_to_lds(job, pro_in, ea, tid);   // for the epilogue; the prologue's barrier publishes them
  XStage xst;
  if (qin) qstage_load(job, pro, tid, xst);
  else stage_load(job, pro, tid, xst);
  // the epilogue's loads from memory (residual, gains, position), issued now
  const EpiPre pre = epi_prefetch<kBurst ? EPI_STORE : EPI>(job, sh, tid, ea);
  uint4 pa[LPL], pb[LPL];
  Seg sa, sb;
  int k_cur = wave, k_nxt = wave + job.nwaves;
  // two segments in flight before the stream (unconditional loads: see
  // seg_null); a burst launch issues them behind the activation's loads, so
  // the activation's wait below leaves them in flight
  if constexpr (kBurst) {
    sa = k_cur < sh.nseg ? seg_at(job, sh, k_cur) : seg_null(job);
    seg_load(sa, lane, pa);
    sb = k_nxt < sh.nseg ? seg_at(job, sh, k_nxt) : seg_null(job);
    seg_load(sb, lane, pb);
  }
  if (!qin) stage_ss(job, pro, tid, stage_norm(job, pro, tid, xst));  // the activation has arrived
  if constexpr (kBurst) {
    if (qin) qstage_store(job, tid, xst);
    else stage_finish(job, pro, tid, xst);
  } else {
    // The first segment's loads go out before the quantization (or the copy
    // of a quantized activation) and the second's after it.  A wave cannot
    // issue loads faster than the memory system drains them, so with both
    // issued first the quantization waited behind the whole first burst (and
    // the compute behind the quantization): this way it runs while the first
    // segment is in flight.
    sa = k_cur < sh.nseg ? seg_at(job, sh, k_cur) : seg_null(job);
    seg_load(sa, lane, pa);
    if (qin) qstage_store(job, tid, xst);
    else stage_finish(job, pro, tid, xst);
    rope_table(job, pro, tid, xst.pos);
    sb = k_nxt < sh.nseg ? seg_at(job, sh, k_nxt) : seg_null(job);
    seg_load(sb, lane, pb);
  }
  __syncthreads();  // the staged activation is complete
  // the RMSNorm factor, from sums of squares the barrier published; formed
  // here so the epilogue does not wait for its LDS round trips
  const float r = kBurst ? 1.0f : norm_factor(job, pro, lane);
  if (k_cur < sh.nseg) {
    XR xr;
    int xslice = -1;
    bool claiming = k_nxt < sh.nseg;
    int k_spare = sh.nseg;
    do {
      stream_step<LPL, FMT, true>(job, sh, lane, slab, k_cur, k_nxt, k_spare, claiming, xslice, xr, pa, sa);
      stream_step<LPL, FMT, false>(job, sh, lane, slab, k_cur, k_nxt, k_spare, claiming, xslice, xr, pb, sb);
    } while (k_cur < sh.nseg);
  }
  __syncthreads();
  const Job& J = lds_ref<Job>(kLdsJob);
  share_epilogue<kBurst ? EPI_STORE : EPI>(J, share_of(J, blockIdx.x), tid, J.nwaves * 64, lds_ref<EpiArgs>(kLdsEpi),
                                          r, pre);
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

template <int EPI, int LPL, int FMT>
int launch_k(const Job& job, const ProArgs& pro, const EpiArgs& ea, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_qgemv<EPI, LPL, FMT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024) != hipSuccess)
      return NT_EHIP;
    attr_set = true;
  }
  constexpr int kind = EPI == EPI_STORE_BURST ? EPI_STORE : EPI;  // trace kinds are the epilogues
  hipEvent_t t0, t1;
  (void)trace_events(kind, &t0, &t1);
  hipExtLaunchKernelGGL((k_qgemv<EPI, LPL, FMT>), dim3(job.grid), dim3(64 * job.nwaves), job.lds_bytes, stream, t0,
                        t1, 0, job, pro, ea);
  return hipGetLastError() == hipSuccess ? NT_OK : NT_EHIP;
}

// A launch whose matrices share one format runs a kernel compiled for that
// format where one exists for its loads per lane (the segment size a format
// reaches sets them); otherwise the kernel that reads the format per segment.
template <int EPI, int LPL>
int launch_lpl(const Job& job, const ProArgs& pro, const EpiArgs& ea, hipStream_t stream) {
  int f = job.fmt[0];
  bool k46 = true;
  for (int m = 0; m < job.nmat; ++m) {
    if (job.fmt[m] != f) f = -1;
    k46 = k46 && (job.fmt[m] == NT_Q4_K || job.fmt[m] == NT_Q6_K);
  }
  if constexpr (LPL == 3) {
    if (f == NT_Q4_K) return launch_k<EPI, LPL, NT_Q4_K>(job, pro, ea, stream);
    if (f == NT_Q4_0) return launch_k<EPI, LPL, NT_Q4_0>(job, pro, ea, stream);
    if (f == NT_Q5_K) return launch_k<EPI, LPL, NT_Q5_K>(job, pro, ea, stream);
  }
  if constexpr (LPL <= 4) {
    if (f == NT_Q6_K) return launch_k<EPI, LPL, NT_Q6_K>(job, pro, ea, stream);
  }
  if (f == NT_Q8_0) return launch_k<EPI, LPL, NT_Q8_0>(job, pro, ea, stream);
  if constexpr (LPL <= 4) {
    if (k46) return launch_k<EPI, LPL, kFmtK46>(job, pro, ea, stream);
  }
  return launch_k<EPI, LPL, -1>(job, pro, ea, stream);
}

template <int EPI>
int launch_epi(const Job& job, const ProArgs& pro, const EpiArgs& ea, hipStream_t stream) {
  if (job.orows <= 0) return NT_OK;
  switch (job.lpl) {
    case 3: return launch_lpl<EPI, 3>(job, pro, ea, stream);
    case 4: return launch_lpl<EPI, 4>(job, pro, ea, stream);
    case 5: return launch_lpl<EPI, 5>(job, pro, ea, stream);
  }
  return NT_EUNSUPPORTED;
}

}  // namespace

// Geometry of a launch: column slices of at most 4096 weights (whole
// blocks), each workgroup's share of output rows, the LDS layout, and the
// grid (one workgroup per CU, fewer when there is little work, more when a
// share's partial-sum table would not fit).
int plan_job(Job& job, int nmat, const uint8_t* const* W, const int* fmt, const int* rows, int cols, int paired,
             int pairs, int qblock) {
  if (nmat < 1 || nmat > kMaxMats || (paired && nmat != 2)) return NT_EINVAL;
  if (cols <= 0 || cols > kMaxCols) return NT_EUNSUPPORTED;
  job = Job{};
  job.nmat = nmat;
  job.paired = paired;
  job.pairs = pairs;
  job.cols = cols;
  bool kquant = false;
  int64_t orows = 0;
  for (int m = 0; m < nmat; ++m) {
    const int qk = block_elems(fmt[m]);
    if (qk == 0 || cols % qk != 0) return NT_EINVAL;
    if (qk == 1) return NT_EUNSUPPORTED;  // F16/F32 have their own GEMV kernel
    if (pairs && (rows[m] & 1)) return NT_EINVAL;
    if (paired && rows[m] != rows[0]) return NT_EINVAL;
    if (rows[m] < 0) return NT_EINVAL;
    kquant |= qk == 256;
    job.W[m] = W[m];
    job.fmt[m] = fmt[m];
    job.rows[m] = rows[m];
    job.rb[m] = (int64_t)(cols / qk) * block_bytes(fmt[m]);
    job.row_base[m] = paired ? 0 : (int)orows;
    if (!paired || m == 0) orows += rows[m];
  }
  if (orows > INT32_MAX / 2) return NT_EUNSUPPORTED;
  job.orows = (int)orows;
  job.unit = pairs ? 2 : 1;
  // whole 32-row blocks per workgroup, when one launch's rows make enough of
  // them to keep nearly every CU busy (p blocks each on ceil(blocks / p)
  // workgroups, at least 7/8 of the CUs)
  const int cus = dev_info().cus;
  if (qblock && !pairs && (nmat == 1 || paired) && orows % 32 == 0 && qx_ok(orows)) {
    const int64_t nb = orows / 32, per = (nb + cus - 1) / cus, g = (nb + per - 1) / per;
    if (8 * g >= 7 * (int64_t)cus && nb % g == 0) job.qblock = 1;
  }
  if (job.qblock) job.unit = 32;
  const int units = (cols + 63) / 64;
  job.nslice = (units + kSliceUnits - 1) / kSliceUnits;
  int ups = (units + job.nslice - 1) / job.nslice;
  if (kquant) ups = (ups + 3) & ~3;  // slices end on 256-weight superblocks
  job.ups = ups;
  job.nslice = (units + ups - 1) / ups;
  job.last_ne = cols - (job.nslice - 1) * ups * 64;
  job.last_units = (job.last_ne + 63) / 64;
  for (int m = 0; m < nmat; ++m) job.slice_bytes[m] = (int64_t)(ups * 64 / block_elems(fmt[m])) * block_bytes(fmt[m]);
  for (int m = 0; m < nmat; ++m) job.last_bytes[m] = (int64_t)(job.last_ne / block_elems(fmt[m])) * block_bytes(fmt[m]);
  // loads per lane: the largest segment plus its misalignment, in 1 KB rounds
  int64_t seg_max = 0;
  for (int m = 0; m < nmat; ++m)
    seg_max = std::max<int64_t>(seg_max, (int64_t)std::min(cols, ups * 64) / block_elems(fmt[m]) * block_bytes(fmt[m]));
  const int need = (int)((seg_max + 15 + 15) / 16 + 63) / 64;
  job.lpl = need <= 3 ? 3 : need;
  if (need > kSlabLoads) return NT_EUNSUPPORTED;
  job.nwaves = kMaxWaves;
  // workgroups: about one per CU, no more than one per wave's worth of
  // segments, and enough that a share's (row, slice) table fits kAccFloats
  const int vper = paired ? 2 : 1;  // segment rows per output row
  const int64_t nu = orows / job.unit;
  const int64_t segs = orows * vper * job.nslice;
  int64_t grid = std::min<int64_t>(cus, (segs + job.nwaves - 1) / job.nwaves);
  const int64_t units_cap = kAccFloats / ((int64_t)job.nslice * job.unit * vper);
  if (job.qblock) {
    const int64_t per = (nu + cus - 1) / cus;
    grid = nu / per;  // whole blocks, the same number in every share
    if (per > units_cap) job.qblock = 0;
  }
  if (!job.qblock && job.unit == 32) return plan_job(job, nmat, W, fmt, rows, cols, paired, pairs, 0);
  if (units_cap < 1) return NT_EUNSUPPORTED;
  grid = std::max<int64_t>(grid, (nu + units_cap - 1) / units_cap);
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, std::max<int64_t>(nu, 1)));
  if (grid > INT32_MAX) return NT_EUNSUPPORTED;
  job.grid = (int)grid;
  job.wg_base = (int)(nu / grid);
  job.wg_rem = (int)(nu % grid);
  for (int i = 0; i < 2; ++i) {
    const int64_t nv = (int64_t)(job.wg_base + i) * job.unit * vper;
    job.magic[i] = nv > 0 ? (uint32_t)(0xffffffffull / (uint64_t)nv) : 0u;
  }
  const int64_t nv_max = (int64_t)(job.wg_base + (job.wg_rem ? 1 : 0)) * job.unit * vper;
  // the staged activation in the layout of a quantized activation in memory
  // (a copy of one is a straight copy), then 256 bytes of slack for the
  // last unit's reads past the end (a unit of a 32-weight format may hold
  // only one block)
  uint32_t off = kArgsLds;
  job.x_hi = off;
  job.x_lo = off + (uint32_t)qx_lo_off(cols);
  job.x_sc = off + (uint32_t)qx_sc_off(cols);
  job.x_sum = off + (uint32_t)qx_sum_off(cols);
  job.x_ss = off + (uint32_t)qx_ss_off(cols);
  off += (uint32_t)qx_bytes(cols) + 256;
  off = (off + 15) & ~15u;
  job.red = off; off += 16 * 4;
  job.ctl = off; off += 16;
  job.rope = off; off += 128 * 8;  // cos/sin of up to 128 rotation pairs (head_dim <= 256)
  job.acc = off; off += (uint32_t)(nv_max * job.nslice * 4);
  job.qo = off;
  if (job.qblock) off += (uint32_t)(nv_max / vper * 4);  // the share's outputs, for their quantization
  off = (off + 15) & ~15u;
  job.slab = off;
  off += (uint32_t)(job.nwaves * job.lpl * 1024);
  job.lds_bytes = off;
  if (job.lds_bytes > 160 * 1024) return NT_EUNSUPPORTED;
  return NT_OK;
}

int launch_gemv(const Job& job, const ProArgs& pro, int epi, const EpiArgs& ea, hipStream_t stream) {
  switch (epi) {
    case EPI_STORE: {
      // every share's segments fit the two buffers of its waves: one burst
      const int vper = job.paired ? 2 : 1;
      const int64_t nseg_max = (int64_t)(job.wg_base + (job.wg_rem ? 1 : 0)) * job.unit * vper * job.nslice;
      if (!pro.gain && !pro.qx_norm && pro.rope_hd == 0 && nseg_max <= 2 * job.nwaves)
        return launch_epi<EPI_STORE_BURST>(job, pro, ea, stream);
      return launch_epi<EPI_STORE>(job, pro, ea, stream);
    }
    case EPI_RESID: return launch_epi<EPI_RESID>(job, pro, ea, stream);
    case EPI_QKV: return launch_epi<EPI_QKV>(job, pro, ea, stream);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(job, pro, ea, stream);
  }
  return NT_EINVAL;
}

}  // namespace nt
