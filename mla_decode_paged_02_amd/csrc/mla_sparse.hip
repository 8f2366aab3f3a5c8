// Sparse MLA decode over an fp8 e4m3 latent cache (gfx950).
//
// What is computed follows generic_flare_mla_decode_kv_cache_ragged (Parameters
// sparse_mla; Args q_scale_ptr, d_indices, indices_stride, topk_lengths,
// num_partitions_in): query row t attends to the cache rows its index list names (the
// first topk_lengths[t] entries, negative entries skipped, no positional mask), a row
// being page * PS + slot of the pool; the key of a listed row is its e4m3 codes times
// the row's scale, the query the e4m3 codes times the token's scale.
//
// The work split, the per-stage compute, the epilogue and the combine are those of the
// dense decode (mla_plan.h, mla_stage.h, mla_decode.hip).  What differs is the loader:
// the 32 listed rows of a stage (576 fp8 bytes each, gathered) land in an LDS staging
// buffer by direct global->LDS loads, together with their scales; the block then widens
// them to bf16 (exact: every e4m3 value is a bf16 value) into the swizzled tile layout
// the compute reads.  The row scale enters the logit and the value weight (KSCALE), the
// token scale the logit scale.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_plan.h"
#include "mla_stage.h"

namespace mla {

constexpr int kRawRowBytes = 576;                           // one fp8 cache row
constexpr int kRawStageBytes = kStageKeys * kRawRowBytes;   // 18432
constexpr int kRawPieces = kRawStageBytes / 16;             // 1152 sixteen-byte pieces
constexpr int kRawPiecesPerRow = kRawRowBytes / 16;         // 36
constexpr int kRawDma = kRawPieces / 64;                    // 18 wave-wide loads per stage
constexpr int kSpTiles = 3;                                 // widened bf16 stage buffers
constexpr int kSpRaw = 2;                                   // fp8 landing buffers
constexpr int kSpScale = 4;                                 // per-key scale slots (64 floats)
constexpr int kIdxWindow = 1024;                            // list positions held in LDS
static_assert(sizeof(PlanLds::scan) == kIdxWindow * sizeof(int), "the window lives in the planning scratch");

// Row t's list positions [0, min(topk[t], shape[1] of d_indices)).
__device__ __forceinline__ RowGeo sparse_row_geo(const SparseArgs& a, int t) {
  const int k = ld_const(a.topk + t);
  return RowGeo{t, 0, max(0, min(k, a.idx_cols))};
}

template <int NT>
__device__ __forceinline__ void sparse_fill(const SparseArgs& a, PlanLds& L) {
  for (int t = threadIdx.x; t < a.T; t += NT) L.geo[t] = RowGeo{t, 0, max(0, min(a.topk[t], a.idx_cols))};
}

// One row segment: list positions of tiles [ta, tc) of row t.
template <int HB, int NW>
__device__ __forceinline__ void sparse_segment(const SparseArgs& a, MLA_LDS uint8_t* tiles, MLA_LDS uint8_t* raw,
                                               MLA_LDS float* kscale, MLA_LDS int* win, int t, const RowGeo& g,
                                               int ta, int tc, bool full, int slot) {
  constexpr int NT = NW * 64;
  constexpr int kSlots = kRawDma + 1;                // the rows' pieces, then their scales
  constexpr int kPerWave = (kSlots + NW - 1) / NW;   // loads every wave issues per stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, ln = lane & 15;
  const int h0 = wave * 16 * HB;

  const int first_tile = __builtin_amdgcn_readfirstlane(g.lo / kTileKeys);
  const int klo = __builtin_amdgcn_readfirstlane(max(g.lo, (first_tile + ta) * kTileKeys));
  const int khi = __builtin_amdgcn_readfirstlane(min(g.hi, (first_tile + tc) * kTileKeys));
  const int s_first = klo / kStageKeys;
  const int nst = (khi - 1) / kStageKeys - s_first + 1;
  const int32_t* ilist = a.idx + (int64_t)t * a.idx_row;

  // every wave must be done with the previous segment's buffers and window
  all_wait0();
  stage_barrier();

  // ---- index window: list positions [wbase, wbase + kIdxWindow), -1 outside [klo, khi)
  int wbase = klo;
  auto window_fill = [&]() {  // block-uniform, with no stage load in flight
    int v[kIdxWindow / NT];
#pragma unroll
    for (int i = 0; i < kIdxWindow / NT; ++i) {
      const int p = wbase + tid + i * NT;
      v[i] = p < khi ? ilist[p] : -1;
    }
    all_wait0();
#pragma unroll
    for (int i = 0; i < kIdxWindow / NT; ++i) win[tid + i * NT] = v[i];
    lgkm_wait0();
    stage_barrier();
  };
  window_fill();

  bool bad = false;
  // row of list position p (in the window), or -1 when the key does not count
  auto row_of = [&](int p) -> int {
    if (p < klo || p >= khi) return -1;
    const int r = win[p - wbase];
    if (r < 0) return -1;  // the -1 fill (and any negative entry) is skipped
    if ((int64_t)r >= a.num_rows) {
      bad = true;
      return -1;
    }
    return r;
  };
  auto row_bytes_off = [&](int r) -> int64_t {
    const int pg = r / a.PS;
    return (int64_t)pg * a.page_bytes + (int64_t)(r - pg * a.PS) * kRawRowBytes;
  };
  auto scale_ptr = [&](int r) -> const void* {
    if (r < 0) return a.zero_row;  // a key that does not count: weight 0
    if (a.cache_scale == nullptr) return a.zero_row + kSparseOneOffset;
    const int pg = r / a.PS;
    return a.cache_scale + (int64_t)pg * a.cs_page + (r - pg * a.PS);
  };

  // Loads of stage st into landing buffer rb and scale slot sb; returns the stage's mask of
  // counting keys (block-uniform).  Every wave issues exactly kPerWave loads (the spare
  // slots repeat the scale load), so one wait count serves all waves.
  auto issue = [&](int st, int rb, int sb) -> uint32_t {
    const int kbase = st * kStageKeys;
    if (min(kbase + kStageKeys, khi) - 1 >= wbase + kIdxWindow) {
      all_wait0();
      stage_barrier();
      wbase = max(kbase, klo);
      window_fill();
    }
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
#pragma unroll
    for (int jj = 0; jj < kPerWave; ++jj) {
      int J = jj * NW + wave;
      if (J >= kSlots) J = kSlots - 1;
      if (J < kRawDma) {
        const int c = J * 64 + lane_v;
        const int row = c / kRawPiecesPerRow, piece = c - row * kRawPiecesPerRow;
        const int r = row_of(kbase + row);
        const uint8_t* src = r >= 0 ? a.cache + row_bytes_off(r) + piece * 16 : a.zero_row + piece * 16;
        dma16(src, raw + rb * kRawStageBytes + J * 1024);
      } else {
        // lanes 32..63 repeat lanes 0..31 (the slot holds 64 floats)
        dma4(scale_ptr(row_of(kbase + (lane_v & 31))), kscale + sb * 64);
      }
    }
    return (uint32_t)__builtin_amdgcn_ballot_w64(lane < 32 && row_of(kbase + lane) >= 0);
  };

  // landing buffer rb (fp8 rows) -> bf16 tile dst, swizzled like the dense tiles
  auto widen = [&](int rb, MLA_LDS uint8_t* dst) {
    for (int c = tid; c < kRawPieces; c += NT) {
      const int row = c / kRawPiecesPerRow, piece = c - row * kRawPiecesPerRow;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 w = *(const MLA_LDS u32x4*)(raw + rb * kRawStageBytes + c * 16);
      const uint2 b0 = e4m3x4_to_bf16x4(w[0]), b1 = e4m3x4_to_bf16x4(w[1]);
      const uint2 b2 = e4m3x4_to_bf16x4(w[2]), b3 = e4m3x4_to_bf16x4(w[3]);
      MLA_LDS uint8_t* rowp = dst + row * kRowBytes;
      *(MLA_LDS u32x4*)(rowp + swz_chunk(row, 2 * piece) * 16) = u32x4{b0.x, b0.y, b1.x, b1.y};
      *(MLA_LDS u32x4*)(rowp + swz_chunk(row, 2 * piece + 1) * 16) = u32x4{b2.x, b2.y, b3.x, b3.y};
    }
    lgkm_wait0();  // visible to the other waves after the next barrier
  };

  // ---- prologue: stages 0 and 1 in flight, q, then stage 0 widened and stage 2 issued
  uint32_t m0 = issue(s_first, 0, 0), m1 = 0, m2 = 0, m3 = 0;
  if (nst > 1) m1 = issue(s_first + 1, 1, 1);

  // query fragments (B operand of S^T = K Q^T), widened to bf16; the token scale goes
  // into the logit scale
  bf16x8 qf[HB][18];
  if (a.q_bf16) {
    const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)t * a.q_tok + 8 * gq;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const uint16_t* qh = qrow + (int64_t)(h0 + 16 * hb + ln) * a.q_head;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[hb][ks] = *(const bf16x8*)(qh + 32 * ks);
    }
  } else {
    const uint8_t* qrow = a.q + (int64_t)t * a.q_tok + 8 * gq;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const uint8_t* qh = qrow + (int64_t)(h0 + 16 * hb + ln) * a.q_head;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const uint2 w = *(const uint2*)(qh + 32 * ks);
        const uint2 lo = e4m3x4_to_bf16x4(w.x), hi = e4m3x4_to_bf16x4(w.y);
        qf[hb][ks] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
  }
  const float q_scale = a.q_scale != nullptr ? ld_const(a.q_scale + t) : 1.f;
  const float scale_log2 = a.scale_log2 * q_scale;
  all_wait0();
  stage_barrier();
  widen(0, tiles);
  stage_barrier();
  if (nst > 2) m2 = issue(s_first + 2, 0, 2);

  using Acc = std::conditional_t<HB == 2, WaveAcc2, WaveAcc<HB>>;
  Acc acc;
  if constexpr (HB == 2) wave_acc2_init(acc); else wave_acc_init(acc);
  const LaneGeo lg = make_lane_geo(lane);

#pragma unroll 1
  for (int k = 0; k < nst; ++k) {
    // stage k+1 has landed (k+2 may still be in flight); every wave is past stage k-1
    if (k + 2 < nst) vm_wait_imm<kPerWave>(); else vm_wait_imm<0>();
    stage_barrier();
    if (k + 1 < nst) widen((k + 1) % kSpRaw, tiles + ((k + 1) % kSpTiles) * kStageBytes);
    stage_barrier();
    if (k + 3 < nst) m3 = issue(s_first + k + 3, (k + 3) % kSpRaw, (k + 3) % kSpScale);
    const MLA_LDS float* ks = kscale + (k % kSpScale) * 64;
    if constexpr (HB == 2)
      stage_compute2<true>(tiles + (k % kSpTiles) * kStageBytes, qf, acc, m0, scale_log2, ks, lg);
    else
      stage_compute<HB, true>(tiles + (k % kSpTiles) * kStageBytes, qf, acc, m0, scale_log2, ks, lg);
    m0 = m1;
    m1 = m2;
    m2 = m3;
  }

  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(a.err, kErrSparseIndex);
  if constexpr (HB == 2) {
    // every wave is done with the stage buffers before they take the output rows
    stage_barrier();
    stage_epilogue2(acc, lane, h0, t, full, slot, a.H, a.out, a.o_tok, a.o_head, a.part_o, a.part_lse,
                    tiles + wave * 32 * 1024);
  }
  else
    stage_epilogue<HB>(acc, lane, h0, t, full, slot, a.H, a.out, a.o_tok, a.o_head, a.part_o, a.part_lse);
}

template <int HB, int NW>
__global__ __launch_bounds__(NW * 64, 1) void mla_sparse_kernel(const SparseArgs a, const SplitPlan plan) {
  // the widened tiles, then the fp8 landing buffers, in one block: the epilogue stages up
  // to 4 x 32 KB of output rows across both
  __shared__ __attribute__((aligned(1024))) uint8_t buf_raw[kSpTiles * kStageBytes + kSpRaw * kRawStageBytes];
  static_assert(kSpTiles * kStageBytes + kSpRaw * kRawStageBytes >= 4 * 32 * 1024, "epilogue staging");
  __shared__ __attribute__((aligned(256))) float ksc_raw[kSpScale * 64];
  __shared__ PlanLds L;
  MLA_LDS uint8_t* tiles = (MLA_LDS uint8_t*)buf_raw;
  MLA_LDS uint8_t* land = tiles + kSpTiles * kStageBytes;
  MLA_LDS float* ksc = (MLA_LDS float*)ksc_raw;
  plan_run<NW * 64>(
      plan, L, [&](PlanLds& l) { sparse_fill<NW * 64>(a, l); }, [&](int t) { return sparse_row_geo(a, t); },
      [&](int r, const RowGeo& g, int ta, int tc, bool full, int slot) {
        sparse_segment<HB, NW>(a, tiles, land, ksc, (MLA_LDS int*)L.scan, r, g, ta, tc, full, slot);
      });
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static SplitPlan plan_of(const SparseArgs& a) {
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
  return p;
}

template <int HB, int NW>
static hipError_t launch_sparse_h(const SparseArgs& a, const SplitPlan& p, hipStream_t stream) {
  const dim3 grid(a.nparts >= 1 ? a.T * a.nparts : a.grid), block(NW * 64);
  hipLaunchKernelGGL((mla_sparse_kernel<HB, NW>), grid, block, 0, stream, a, p);
  return hipGetLastError();
}

hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream, const KernelTimer* timer) {
  const SplitPlan p = plan_of(a);
  hipError_t e;
  if (timer && (e = hipEventRecord(timer->start, stream)) != hipSuccess) return e;
  switch (a.H) {
    case 128: e = launch_sparse_h<2, 4>(a, p, stream); break;
    case 64: e = launch_sparse_h<2, 2>(a, p, stream); break;
    case 32: e = launch_sparse_h<1, 2>(a, p, stream); break;
    case 16: e = launch_sparse_h<1, 1>(a, p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (timer && (e = hipEventRecord(timer->stop, stream)) != hipSuccess) return e;
  return launch_combine(p, stream);
}

}  // namespace mla
