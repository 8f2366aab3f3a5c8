// Dense MLA decode over a paged bf16 latent cache, and the log-sum-exp combine of rows
// split over several work-groups (split-KV) (gfx950).
//
// What is computed follows generic_flare_mla_decode_kv_cache_ragged (summary; Args q,
// input_row_offsets, scale, output, num_partitions_in; Parameters mask_str,
// local_window_size): for each query row t and head h, softmax over the visible cache
// rows of scale * <q, row>, applied to the rows' 512 latent columns.
//
// Per work-group: all heads of one query row (4 waves x 32 heads at H = 128, one wave per
// SIMD, O in the accumulation registers), so each cache row is read from HBM exactly once.
// Keys stream through LDS in 32-key stages (4 buffers, 3 in flight) by direct global->LDS
// loads; page ids come from an LDS window of the row's page-table entries.  The work split
// is in mla_plan.h, the per-stage MFMA / softmax work in mla_stage.h.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_plan.h"
#include "mla_rows.h"
#include "mla_stage.h"

namespace mla {

// ---------------------------------------------------------------------------------------
// One row segment: tiles [ta, tc) (relative to the row's first visible tile) of row t.
//
// Page ids reach the stage loop through an LDS window of kPidWindow consecutive page-table
// entries (refilled, after draining the loads in flight, when a segment outruns it).  A
// scalar load would be cheaper to issue, but scalar loads complete out of order, so one in
// flight turns every LDS-read wait of the stage compute into a full wait for it.
// KPAGES = 1: PS is a multiple of 32, so a stage lies in one page, read one stage ahead;
// KPAGES = 0: any other page size, each lane looks up the page of its own key.
// ---------------------------------------------------------------------------------------
constexpr int kPidWindow = 1024;
static_assert(sizeof(PlanLds::scan) == kPidWindow * sizeof(int), "the window lives in the planning scratch");

template <int HB, int NW, int KPAGES>
__device__ __forceinline__ void decode_segment(const DecodeArgs& a, MLA_LDS uint8_t* tiles, MLA_LDS int* pids,
                                               int t, const RowGeo& g, int ta, int tc, bool full, int slot) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int gq = lane >> 4, ln = lane & 15;
  const int h0 = wave * 16 * HB;
  // the stage's kDmaPerStage wave-wide loads are dealt round-robin to the waves
  const int dpw = (kDmaPerStage - wave + NW - 1) / NW;

  // all of these are block-uniform; readfirstlane keeps them (and the page-table
  // addresses derived from them) in scalar registers
  const int first_tile = __builtin_amdgcn_readfirstlane(g.lo / kTileKeys);
  const int klo = __builtin_amdgcn_readfirstlane(max(g.lo, (first_tile + ta) * kTileKeys));
  const int khi = __builtin_amdgcn_readfirstlane(min(g.hi, (first_tile + tc) * kTileKeys));
  const int s_first = klo / kStageKeys;
  const int nst = (khi - 1) / kStageKeys - s_first + 1;
  const int32_t* pt = a.page_table + (int64_t)__builtin_amdgcn_readfirstlane(g.b) * a.pt_row;

  const int p_last = (khi - 1) / a.PS;  // last logical page of the segment

  // every wave must be done with the previous segment's buffers and page window
  all_wait0();
  stage_barrier();

  // ---- page-id window [pbase, pbase + kPidWindow): loads issued here, stored to LDS by
  // the caller once they have landed (entries past the segment read as -1)
  int pbase = klo / a.PS;
  int pv[kPidWindow / NT];
  auto window_load = [&]() {
#pragma unroll
    for (int i = 0; i < kPidWindow / NT; ++i) {
      const int p = pbase + tid + i * NT;
      pv[i] = p <= p_last ? pt[p] : -1;
    }
  };
  auto window_store = [&]() {
#pragma unroll
    for (int i = 0; i < kPidWindow / NT; ++i) pids[tid + i * NT] = pv[i];
  };
  // moves the window to start at page `base` (block-uniform call; drains the stage loads)
  auto window_move = [&](int base) {
    all_wait0();
    stage_barrier();
    pbase = base;
    window_load();
    all_wait0();
    window_store();
    lgkm_wait0();
    stage_barrier();
  };
  if (KPAGES == 0) {
    // the per-lane lookups of the prologue's stages need the window already
    window_load();
    all_wait0();
    window_store();
    lgkm_wait0();
    stage_barrier();
  }

  // Byte offset of each of this lane's stage loads within a block of 32 consecutive cache
  // rows: fixed per lane, so a stage that lies wholly inside one valid page costs one
  // scalar base and one load instruction per 1 KB.
  constexpr int kDmaMax = (kDmaPerStage + NW - 1) / NW;
  uint32_t dma_off[kDmaMax];
#pragma unroll
  for (int jj = 0; jj < kDmaMax; ++jj) {
    const int sl = (jj * NW + wave) * 64 + lane;
    const int row = sl / kRowChunks;
    dma_off[jj] = (uint32_t)(row * kRowBytes + swz_chunk(row, sl - row * kRowChunks) * 16);
  }

  bool bad_page = false;
  // page of stage st from the window (KPAGES = 1); consecutive stages of one page reuse
  // the id read last
  int lp_last = -1, pid_last = -1;
  auto stage_page = [&](int st) {
    const int lp = st * kStageKeys / a.PS;
    if (lp == lp_last) return pid_last;
    if (lp >= pbase + kPidWindow) window_move(lp);
    lp_last = lp;
    pid_last = __builtin_amdgcn_readfirstlane(pids[lp - pbase]);
    return pid_last;
  };
  // A stage whose keys are all visible and lie in one valid page is loaded from a scalar
  // base: fast_base() returns it, or null when the stage needs the general path.
  // (stage keys are never negative: the in-page offset is an unsigned remainder; the pool
  // bound is compared in 32 bits, page ids being int32)
  const int npages32 = (int)min(a.num_pages, (int64_t)INT32_MAX);
  auto fast_base = [&](int st, int pa) -> const uint8_t* {
    const int kbase = st * kStageKeys;
    if (KPAGES != 0 && kbase >= klo && kbase + kStageKeys <= khi && pa >= 0 && pa < npages32)
      return a.cache + (int64_t)pa * a.page_bytes + (int64_t)((uint32_t)kbase % (uint32_t)a.PS) * kRowBytes;
    return nullptr;
  };
  // load jj of this wave for a fast stage (no-op past the wave's share)
  auto fast_load = [&](const uint8_t* base, MLA_LDS uint8_t* dst, int jj) {
    const int J = jj * NW + wave;
    if (kDmaPerStage % NW == 0 || J < kDmaPerStage) dma16_base_nt(base, dma_off[jj], dst + J * 1024);
  };
  // general case: per-lane keys, pages and bounds (segment edges, invalid pages, page
  // sizes that are not a multiple of the stage)
  auto issue_general = [&](int st, int bi, int pa) {
    MLA_LDS uint8_t* dst = tiles + bi * kStageBytes;
    const int kbase = st * kStageKeys;
    const int lpa = kbase / a.PS;
    if (KPAGES == 0) {
      const int lp_hi = (min(kbase + kStageKeys, khi) - 1) / a.PS;
      if (lp_hi >= pbase + kPidWindow) window_move(max(kbase, klo) / a.PS);
    }
    // the lane's slot arithmetic is redone per call (opaque copy of the lane id) rather
    // than hoisted out of the stage loop into registers
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
#pragma unroll
    for (int jj = 0; jj < (kDmaPerStage + NW - 1) / NW; ++jj) {
      const int J = jj * NW + wave;
      if (kDmaPerStage % NW != 0 && J >= kDmaPerStage) break;
      const int sl = J * 64 + lane_v;
      const int row = sl / kRowChunks;
      const int cg = swz_chunk(row, sl - row * kRowChunks);
      const int key = kbase + row;
      const uint8_t* src = a.zero_row + cg * 16;
      if (key >= klo && key < khi) {
        int pid, lp;
        if (KPAGES == 0) {
          lp = key / a.PS;
          pid = pids[lp - pbase];
        } else {
          lp = lpa;
          pid = pa;
        }
        if (pid >= 0 && pid < npages32)
          src = a.cache + (int64_t)pid * a.page_bytes + (int64_t)(key - lp * a.PS) * kRowBytes + cg * 16;
        else
          bad_page = true;
      }
      dma16_nt(src, dst + J * 1024);
    }
  };
  auto issue = [&](int st, int bi, int pa) {
    const uint8_t* fb = fast_base(st, pa);
    if (fb == nullptr) {
      issue_general(st, bi, pa);
      return;
    }
    MLA_LDS uint8_t* dst = tiles + bi * kStageBytes;
#pragma unroll
    for (int jj = 0; jj < kDmaMax; ++jj) fast_load(fb, dst, jj);
  };

  // ---- query fragments: B operand of S^T = K Q^T (lane holds q[h][32ks + 8gq .. +8]),
  // issued first so that their latency overlaps the page-id loads of the first stage.
  // They are waited for completely below: the stage loads are invisible to the compiler's
  // wait bookkeeping, so no ordinary vector-memory access may still be in flight, in its
  // view, once the stage loop starts.
  bf16x8 qf[HB][18];
  {
    const uint16_t* qrow = a.q + (int64_t)t * a.q_tok + 8 * gq;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const uint16_t* qh = qrow + (int64_t)(h0 + 16 * hb + ln) * a.q_head;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[hb][ks] = *(const bf16x8*)(qh + 32 * ks);
    }
  }

  // ---- prologue: stage 0 (KPAGES = 1: the page ids of the first stages by scalar loads,
  // which the full wait below covers) and the window for the loop.  Stages 1 and 2 are
  // issued at the top of the first step, after the wait: the wait then covers only what
  // the first step needs, not a full pipeline of stages.
  int pa_n = 0;
  const int npro = nst < kNumBuf - 1 ? nst : kNumBuf - 1;
  auto direct_page = [&](int st) { return ld_const(pt + st * kStageKeys / a.PS); };
  // all the prologue's page ids first (independent scalar loads: one latency, not four)
  int pa_pro[kNumBuf];
#pragma unroll
  for (int k = 0; k < kNumBuf; ++k) pa_pro[k] = (KPAGES != 0 && k < nst) ? direct_page(s_first + k) : 0;
  issue(s_first, 0, pa_pro[0]);
  if (KPAGES != 0 && kNumBuf - 1 < nst) pa_n = pa_pro[kNumBuf - 1];
  if (KPAGES != 0) window_load();

  all_wait0();
  if (KPAGES != 0) {
    window_store();
    lgkm_wait0();  // made visible to the other waves by the barrier at the loop top
  }

  // HB = 2: one 32-head wave per SIMD with O in the accumulation registers
  using Acc = std::conditional_t<HB == 2, WaveAcc2, WaveAcc<HB>>;
  Acc acc;
  if constexpr (HB == 2) wave_acc2_init(acc); else wave_acc_init(acc);
  const LaneGeo lg = make_lane_geo(lane);

#pragma unroll 1
  for (int k = 0; k < nst; ++k) {
    // ---- wait for stage k, then refill the buffer stage k-1 used
    {
      // stages issued after stage k and possibly still in flight: k+1 .. k+kNumBuf-2
      static_assert(kNumBuf == 4, "the wait below assumes two younger stages");
      const int younger = KPAGES == 0 ? 0 : min(kNumBuf - 2, nst - 1 - k);
      constexpr int kDhi = (kDmaPerStage + NW - 1) / NW, kDlo = kDmaPerStage / NW;
      if (younger == 0) vm_wait_imm<0>();
      else if (kDhi == kDlo || dpw == kDhi) {
        if (younger >= 2) vm_wait_imm<2 * kDhi>(); else vm_wait_imm<kDhi>();
      } else {
        if (younger >= 2) vm_wait_imm<2 * kDlo>(); else vm_wait_imm<kDlo>();
      }
      stage_barrier();
    }
    if (k == 0) {
#pragma unroll
      for (int j = 1; j < kNumBuf - 1; ++j)
        if (j < npro) issue(s_first + j, j, pa_pro[j]);
    }
    // Refill the buffer stage k-1 used with stage k + kNumBuf - 1: a fast stage's loads are
    // spread over the score k-steps of this stage's compute, any other is issued here.
    const int kn = k + kNumBuf - 1;
    const uint8_t* fb = nullptr;
    MLA_LDS uint8_t* fdst = tiles + (kn % kNumBuf) * kStageBytes;
    if (kn < nst) {
      fb = fast_base(s_first + kn, pa_n);
      if (fb == nullptr) issue_general(s_first + kn, kn % kNumBuf, pa_n);
      if (KPAGES != 0 && kn + 1 < nst) pa_n = stage_page(s_first + kn + 1);
    }
    auto hook = [&](int ks) {
      if (fb == nullptr) return;
#pragma unroll
      for (int jj = 0; jj < kDmaMax; ++jj)
        if (jj * 18 / kDmaMax == ks) fast_load(fb, fdst, jj);
    };
    const int kbase = (s_first + k) * kStageKeys;
    if constexpr (HB == 2)
      stage_compute2<false>(tiles + (k % kNumBuf) * kStageBytes, qf, acc, range_bits(kbase, klo, khi),
                            a.scale_log2, nullptr, lg, hook);
    else
      stage_compute<HB, false>(tiles + (k % kNumBuf) * kStageBytes, qf, acc, range_bits(kbase, klo, khi),
                               a.scale_log2, nullptr, lg, hook);
  }

  if (bad_page) atomicOr(a.err, kErrPageId);
  if constexpr (HB == 2) {
    // every wave is done with the stage buffers before they take the output rows
    stage_barrier();
    stage_epilogue2(acc, lane, h0, t, full, slot, a.H, a.out, a.o_tok, a.o_head, a.part_o, a.part_lse,
                    tiles + wave * 32 * 1024, nullptr);
  }
  else
    stage_epilogue<HB>(acc, lane, h0, t, full, slot, a.H, a.out, a.o_tok, a.o_head, a.part_o, a.part_lse, nullptr);
}

// SMALL: balanced batch of at most 64 rows and 64 sequences, no more rows than work-groups
// (planned per wave, see plan_run).
template <int HB, int NW, int KPAGES, bool SMALL>
__global__ __launch_bounds__(NW * 64, 1) void mla_decode_kernel(const DecodeArgs a, const SplitPlan plan) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles_raw[kNumBuf * kStageBytes];
  static_assert(kNumBuf * kStageBytes >= 4 * 32 * 1024, "epilogue staging");
  __shared__ PlanLds L;
  MLA_LDS uint8_t* tiles = (MLA_LDS uint8_t*)tiles_raw;
  plan_run<NW * 64, SMALL>(
      plan, L, [&](PlanLds& l) { decode_fill<NW * 64>(a, l); },
      [&](int t) { return decode_row_geo(a, t); },
      [&](RowGeo* geo, int lane) { decode_fill_wave(a, geo, lane); },
      [&](int r, const RowGeo& g, int ta, int tc, bool full, int slot) {
        decode_segment<HB, NW, KPAGES>(a, tiles, (MLA_LDS int*)L.scan, r, g, ta, tc, full, slot);
      });
}

// ---------------------------------------------------------------------------------------
// Combine: out = sum_c 2^(lse_c - M) O_c / sum_c 2^(lse_c - M) over the parts of a split
// row, in a fixed order.  Block = (row, 4 heads); thread = (head, 8 columns).  The parts
// are read kCombineBatch at a time with every load of a batch in flight together (the
// kernel is latency-bound: a serial chain of part loads would dominate it); a later batch
// with a larger maximum rescales what is summed so far.
// ---------------------------------------------------------------------------------------
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(256) void mla_combine_kernel(const SplitPlan p) {
  const int groups = p.H / 4;
  const int t = blockIdx.x / groups, hg = blockIdx.x - t * groups;
  const int h = hg * 4 + (threadIdx.x >> 6), col = (threadIdx.x & 63) * 8;
  int n;
  const RowSplit rs = row_split(p, t, n);
  if (n == 0) return;  // the row was written whole (or cleared)
  float M = -INFINITY, den = 0.f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int c0 = 0; c0 < n; c0 += kCombineBatch) {
    float lv[kCombineBatch];
    uint4 xv[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      lv[j] = -INFINITY;
      xv[j] = make_uint4(0, 0, 0, 0);
      if (c0 + j < n) {
        const int64_t sl = (int64_t)split_slot(rs, c0 + j) * p.H + h;
        lv[j] = p.part_lse[sl];
        xv[j] = *(const uint4*)(p.part_o + sl * kLatentDim + col);
      }
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) mb = fmaxf(mb, lv[j]);
    if (mb == -INFINITY) continue;
    if (mb > M) {
      const float r = fast_exp2(M - mb);  // 0 while M is -inf
      den *= r;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= r;
      M = mb;
    }
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      if (lv[j] == -INFINITY) continue;  // a part that saw no key
      const float w = fast_exp2(lv[j] - M);
      den += w;
      const uint32_t xw[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w * __builtin_bit_cast(float, xw[i] << 16);
        acc[2 * i + 1] += w * __builtin_bit_cast(float, xw[i] & 0xFFFF0000u);
      }
    }
  }
  uint16_t* dst = p.out + (int64_t)t * p.o_tok + (int64_t)h * p.o_head + col;
  if (M == -INFINITY) {  // no part saw a key (an empty row split by a fixed count)
    *(uint4*)dst = make_uint4(0, 0, 0, 0);
    return;
  }
  // a sink logit weighs into the denominator only (it carries no value)
  if (p.sink != nullptr) den += fast_exp2(p.sink[h] * 1.4426950408889634f - M);
  const float inv = 1.f / den;
  uint32_t wd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wd[j] = (uint32_t)bf16_bits_rne(acc[2 * j] * inv) | ((uint32_t)bf16_bits_rne(acc[2 * j + 1] * inv) << 16);
  *(uint4*)dst = make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
size_t decode_slots(int64_t T, int32_t nparts, int32_t grid) {
  return nparts >= 1 ? (size_t)T * (size_t)nparts : 2 * (size_t)grid;
}

hipError_t launch_combine(const SplitPlan& p, hipStream_t stream) {
  if (p.nparts == 1) return hipSuccess;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(p.T * (p.H / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

static SplitPlan plan_of(const DecodeArgs& a) {
  SplitPlan p;
  p.T = a.T;
  p.H = a.H;
  p.nparts = a.nparts;
  p.grid = a.grid;
  p.out = a.out;
  p.o_tok = a.o_tok;
  p.o_head = a.o_head;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  p.row_meta = a.row_meta;
  p.sink = nullptr;
  return p;
}

template <int HB, int NW>
static hipError_t launch_decode_h(const DecodeArgs& a, const SplitPlan& p, hipStream_t stream) {
  const dim3 grid(a.nparts >= 1 ? a.T * a.nparts : a.grid), block(NW * 64);
  const bool small = a.nparts == 0 && a.T <= 64 && a.B <= 64 && a.T <= a.grid;
  if (a.PS % kStageKeys == 0) {
    if (small) hipLaunchKernelGGL((mla_decode_kernel<HB, NW, 1, true>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_decode_kernel<HB, NW, 1, false>), grid, block, 0, stream, a, p);
  } else {
    if (small) hipLaunchKernelGGL((mla_decode_kernel<HB, NW, 0, true>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_decode_kernel<HB, NW, 0, false>), grid, block, 0, stream, a, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, const KernelTimer* timer) {
  const SplitPlan p = plan_of(a);
  hipError_t e;
  if (timer && (e = hipEventRecord(timer->start, stream)) != hipSuccess) return e;
  const bool small = a.nparts == 0 && a.T <= 64 && a.B <= 64 && a.T <= a.grid;
  switch (a.H) {
    case 128: e = small ? launch_decode2(a, p, stream) : launch_decode_h<2, 4>(a, p, stream); break;
    case 64: e = launch_decode_h<2, 2>(a, p, stream); break;
    case 32: e = launch_decode_h<1, 2>(a, p, stream); break;
    case 16: e = launch_decode_h<1, 1>(a, p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (timer && (e = hipEventRecord(timer->stop, stream)) != hipSuccess) return e;
  return launch_combine(p, stream);
}

}  // namespace mla
