// Sparse MLA decode over an fp8 e4m3 latent cache (gfx950).
//
// What is computed follows generic_flare_mla_decode_kv_cache_ragged (Parameters
// sparse_mla; Args q_scale_ptr, d_indices, indices_stride, topk_lengths,
// num_partitions_in): query row t attends to the cache rows its index list names (the
// first topk_lengths[t] entries, negative entries skipped, no positional mask), a row
// being page * PS + slot of the pool; the key of a listed row is its e4m3 codes times
// the row's scale, the query the e4m3 codes times the token's scale.
//
// With dense = 1 the same kernel is the dense decode over a paged fp8 cache ([DEC]
// Args kv_collection, q_scale_ptr; Parameters mask_str, local_window_size): the rows of
// query row t are the positions its mask leaves visible, each mapped through the page
// table of its sequence, so list position p is logical key p.
//
// The work split, the per-stage compute, the epilogue and the combine are those of the
// dense decode (mla_plan.h, mla_stage.h, mla_decode.hip).  What differs is the loader:
// the 32 listed rows of a stage (576 fp8 bytes each, gathered) land in an LDS staging
// buffer by direct global->LDS loads, together with their scales; the block then widens
// them to bf16 (exact: every e4m3 value is a bf16 value) into the swizzled tile layout
// the compute reads.  The row scale enters the logit and the value weight (KSCALE), the
// token scale the logit scale.
//
// With ROPE the rows of q and the cache are in the rope-aware layout ([DEC] Parameters
// per_token_scale_rope_aware): 640 bytes, the 512 latent values as e4m3 codes, then the 64
// rope values as bf16, the token / row scale applying to the codes only.  The widening
// stores a key's rope values divided by its scale (and the query fragments the query's
// rope values divided by the token scale), so the scaled logit of the common path is
// sigma_q sigma_k <q8, k8> + <q_rope, k_rope>, up to the bf16 rounding of those quotients.
// A scale of magnitude below 2^-40 is taken as 2^-40 on both sides of that quotient: the
// latent part of such a row or token then contributes (about 2^-31 of a code) nothing
// while its rope still counts in full, and a product of two such quotients (2^80 times the
// rope values) stays far inside the fp32 range of the accumulators.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_plan.h"
#include "mla_rows.h"
#include "mla_stage.h"

namespace mla {

// Geometry of the raw rows: 576 bytes (all e4m3), or 640 in the rope-aware layout.
template <bool ROPE>
struct RawRows {
  static constexpr int kRowBytes = ROPE ? 640 : 576;            // one cache row
  static constexpr int kStageBytes = kStageKeys * kRowBytes;     // 18432 / 20480
  static constexpr int kPieces = kStageBytes / 16;               // sixteen-byte pieces
  static constexpr int kPiecesPerRow = kRowBytes / 16;           // 36 / 40
  static constexpr int kDma = kPieces / 64;                      // 18 / 20 wave-wide loads
};
constexpr int kRawStageBytesMax = RawRows<true>::kStageBytes;
constexpr float kRopeMinScale = 0x1p-40f;
// the row or token scale as the rope-aware path uses it (see the header)
__device__ __forceinline__ float rope_scale(float s) { return fabsf(s) < kRopeMinScale ? kRopeMinScale : s; }
constexpr int kSpTiles = 2;    // widened bf16 tiles: the one computed, the one being widened
constexpr int kSpRaw = 3;      // fp8 landing buffers: the one being widened, two in flight
constexpr int kSpScale = 4;    // per-key scale slots (64 floats): stages k .. k+3
constexpr int kIdxWindow = 1024;                            // list positions held in LDS
constexpr int kSpStageLds = kSpTiles * kStageBytes + kSpRaw * kRawStageBytesMax;
// the epilogue stages 4 x 32 KB of output rows over the same block
constexpr int kSpLdsBytes = kSpStageLds > 4 * 32 * 1024 ? kSpStageLds : 4 * 32 * 1024;
static_assert(sizeof(PlanLds::scan) == kIdxWindow * sizeof(int), "the window lives in the planning scratch");

template <int NT, bool XTRA>
__device__ __forceinline__ void sparse_fill(const SparseArgs& a, PlanLds& L) {
  if (!a.shared) {
    for (int t = threadIdx.x; t < a.T; t += NT) L.geo[t] = RowGeo{t, 0, sparse_len<XTRA>(a, t)};
    return;
  }
  for (int t = threadIdx.x; t < a.T; t += NT) L.geo[t] = RowGeo{-1, 0, 0};
  __syncthreads();
  for (int b = threadIdx.x; b < a.B; b += NT) sparse_fill_seq(a, L.geo, b);
}

// One row segment: list positions of tiles [ta, tc) of row t.
//
// Pipeline (stage k = 32 list positions): at the top of step k the fp8 rows of stage k+1
// have landed and stage k+2 may still be in flight; the step issues stage k+3 into the
// landing buffer stage k was widened from, then computes stage k from its bf16 tile while
// the hook of the score k-steps widens stage k+1 into the other tile.  One barrier per
// stage orders all of it.
// DENSE: rows from the page table (mla_decode_paged_fp8), else from d_indices.  XTRA (the
// extended sparse decode): the sink logits, and the second list when there is one, whose
// rows are held in the window with kExtraRowBit set.
template <int HB, int NW, bool DENSE, bool XTRA, bool ROPE>
__device__ __forceinline__ void sparse_segment(const SparseArgs& a, MLA_LDS uint8_t* tiles, MLA_LDS uint8_t* raw,
                                               MLA_LDS float* kscale, MLA_LDS int* win, int t, const RowGeo& g,
                                               int ta, int tc, bool full, int slot) {
  constexpr int NT = NW * 64;
  static_assert(!(ROPE && XTRA), "the second stream is read in the all-e4m3 layout only");
  constexpr int kRawRowBytes = RawRows<ROPE>::kRowBytes;
  constexpr int kRawStageBytes = RawRows<ROPE>::kStageBytes;
  constexpr int kRawPieces = RawRows<ROPE>::kPieces;
  constexpr int kRawPiecesPerRow = RawRows<ROPE>::kPiecesPerRow;
  constexpr int kRawDma = RawRows<ROPE>::kDma;
  constexpr int kSlots = kRawDma + 1;                // the rows' pieces, then their scales
  constexpr int kPerWave = (kSlots + NW - 1) / NW;   // loads every wave issues per stage
  constexpr int kWp = (kRawPieces + NT - 1) / NT;    // pieces each thread widens per stage
  constexpr bool kTwoPhase = 2 * kWp <= 18;          // read and convert in separate k-steps
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, ln = lane & 15;
  const int h0 = wave * 16 * HB;

  // list positions [klo, khi) of the tiles
  const int first_tile = __builtin_amdgcn_readfirstlane(g.lo / kTileKeys);
  const int klo = __builtin_amdgcn_readfirstlane(max(g.lo, (first_tile + ta) * kTileKeys));
  const int khi = __builtin_amdgcn_readfirstlane(min(g.hi, (first_tile + tc) * kTileKeys));
  const int s_first = klo / kStageKeys;
  const int nst = (khi - 1) / kStageKeys - s_first + 1;
  const int32_t* ilist = a.idx + (int64_t)g.b * a.idx_row;  // g.b: the list row of t
  // XTRA: positions from nmain on are the second list's (block-uniform)
  const int nmain = XTRA && a.xidx != nullptr ? __builtin_amdgcn_readfirstlane(sparse_main_len(a, t)) : INT32_MAX;
  const int32_t* xlist = XTRA ? a.xidx + (int64_t)t * a.xidx_row : nullptr;
  // dense: the page-table row of the sequence (g.b), list position p = logical key p
  const int32_t* prow = DENSE ? a.page_table + (int64_t)__builtin_amdgcn_readfirstlane(g.b) * a.pt_row : nullptr;
  const int npages32 = (int)min(a.num_rows / a.PS, (int64_t)INT32_MAX);

  // every wave must be done with the previous segment's buffers and window
  all_wait0();
  stage_barrier();

  // ---- index window: list positions [wbase, wbase + kIdxWindow), checked against the pool
  // as they are stored: -1 outside [klo, khi), for negative entries (skipped) and for rows
  // past the end of the pool (skipped and flagged)
  int wbase = klo;
  bool bad = false, bad_page = false;
  auto window_fill = [&]() {  // block-uniform, with no stage load in flight
    int v[kIdxWindow / NT];
#pragma unroll
    for (int i = 0; i < kIdxWindow / NT; ++i) {
      const int p = wbase + tid + i * NT;
      if (XTRA)
        v[i] = p < khi ? (p < nmain ? ilist[p] : xlist[p - nmain]) : -1;
      else
        v[i] = p < khi ? (DENSE ? prow[p / a.PS] : ilist[p]) : -1;
    }
    all_wait0();
#pragma unroll
    for (int i = 0; i < kIdxWindow / NT; ++i) {
      int r = v[i];
      if (XTRA && wbase + tid + i * NT >= nmain) {
        // a second-stream row: checked against its own pool, then marked
        if (r >= 0) {
          if ((int64_t)r >= a.xnum_rows) {
            bad = true;
            r = -1;
          } else {
            r |= kExtraRowBit;
          }
        }
      } else if (DENSE) {
        // page id -> physical row; a page outside the pool is skipped and flagged
        const int p = wbase + tid + i * NT;
        if (p < khi) {
          if (r >= 0 && r < npages32) {
            r = r * a.PS + (p - (p / a.PS) * a.PS);
          } else {
            bad_page = true;
            r = -1;
          }
        }
      } else if ((int64_t)r >= a.num_rows) {
        bad = true;
        r = -1;
      }
      win[tid + i * NT] = r < 0 ? -1 : r;
    }
    lgkm_wait0();
    stage_barrier();
  };
  window_fill();

  // listed row of position p (read from the window), -1 when the key does not count
  auto entry = [&](int p) -> int { return p >= klo && p < khi ? win[p - wbase] : -1; };
  auto row_src = [&](int r) -> const uint8_t* {
    if (XTRA && (r & kExtraRowBit)) {
      const int rx = r & ~kExtraRowBit, pg = rx / a.xPS;
      return a.xcache + (int64_t)pg * a.xpage_bytes + (int64_t)(rx - pg * a.xPS) * kRawRowBytes;
    }
    if (a.flat) return a.cache + (int64_t)r * kRawRowBytes;
    const int pg = r / a.PS;
    return a.cache + (int64_t)pg * a.page_bytes + (int64_t)(r - pg * a.PS) * kRawRowBytes;
  };
  auto scale_src = [&](int r) -> const void* {
    if (r < 0) return a.zero_row;  // a key that does not count: weight 0
    if (XTRA && (r & kExtraRowBit)) {
      if (a.xcache_scale == nullptr) return a.zero_row + kSparseOneOffset;
      const int rx = r & ~kExtraRowBit, pg = rx / a.xPS;
      return a.xcache_scale + (int64_t)pg * a.xcs_page + (rx - pg * a.xPS);
    }
    if (a.cache_scale == nullptr) return a.zero_row + kSparseOneOffset;
    if (a.flat) return a.cache_scale + r;
    const int pg = r / a.PS;
    return a.cache_scale + (int64_t)pg * a.cs_page + (r - pg * a.PS);
  };

  // Loads of stage st into landing buffer rb and scale slot sb, in three steps: the window
  // reads of this lane's entries (issue_read), one load per slot jj (issue_slot) and the
  // stage's mask of counting keys (issue_mask, block-uniform).  Every wave issues exactly
  // kPerWave loads (the spare slots repeat the scale load), so one wait count serves all
  // waves.  The window must cover the stage (issue_window).
  auto issue_window = [&](int st) {  // block-uniform; drains the stage loads when it moves
    const int kbase = st * kStageKeys;
    if (min(kbase + kStageKeys, khi) - 1 >= wbase + kIdxWindow) {
      all_wait0();
      stage_barrier();
      wbase = max(kbase, klo);
      window_fill();
    }
  };
  auto window_covers = [&](int st) { return min(st * kStageKeys + kStageKeys, khi) - 1 < wbase + kIdxWindow; };
  auto slot_of = [&](int jj) { return min(jj * NW + wave, kSlots - 1); };
  auto issue_read = [&](int st, int (&rr)[kPerWave], int& rmask) {
    const int kbase = st * kStageKeys;
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
#pragma unroll
    for (int jj = 0; jj < kPerWave; ++jj) {
      const int J = slot_of(jj);
      rr[jj] = entry(kbase + (J < kRawDma ? (J * 64 + lane_v) / kRawPiecesPerRow : (lane_v & 31)));
    }
    rmask = entry(kbase + (lane_v & 31));
  };
  // FLAT: rows at r * 576 and scales at element r (no page arithmetic)
  auto issue_slot = [&](auto flat, int rb, int sb, int jj, int rj) {
    constexpr bool FLAT = decltype(flat)::value;
    const int J = slot_of(jj);
    const int r = rj;
    if (J < kRawDma) {
      int lane_v = lane;
      asm volatile("" : "+v"(lane_v));
      const int c = J * 64 + lane_v;
      const int piece = c - (c / kRawPiecesPerRow) * kRawPiecesPerRow;
      const uint8_t* row = FLAT ? a.cache + (int64_t)r * kRawRowBytes : row_src(r);
      dma16((r >= 0 ? row : a.zero_row) + piece * 16, raw + rb * kRawStageBytes + J * 1024);
    } else {
      // lanes 32..63 repeat lanes 0..31 (the slot holds 64 floats)
      const void* src = FLAT && r >= 0 && a.cache_scale != nullptr ? (const void*)(a.cache_scale + r) : scale_src(r);
      dma4(src, kscale + sb * 64);
    }
  };
  auto issue_mask = [&](int rmask) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_ballot_w64(lane < 32 && rmask >= 0);
  };
  auto issue = [&](int st, int rb, int sb) -> uint32_t {
    issue_window(st);
    int rr[kPerWave], rmask;
    issue_read(st, rr, rmask);
#pragma unroll
    for (int jj = 0; jj < kPerWave; ++jj) issue_slot(std::false_type(), rb, sb, jj, rr[jj]);
    return issue_mask(rmask);
  };
  // hook steps of the stage compute (value column blocks, when the score registers are
  // free) that take stage k+3's loads: the window reads, then one slot every other step,
  // then the mask
  constexpr bool kHookIssue = kPerWave <= 5;
  constexpr int kIssueRead = 18;

  // landing buffer -> bf16 tile, swizzled like the dense tiles; piece i of this thread is
  // read into wr[i] by take() and converted and stored by put().
  // With 256 threads, thread (r, j) = (tid / 8, tid % 8) widens pieces j + 8i of row r: the
  // source advances by 128 bytes per piece and, as the swizzle only flips the low three
  // bits of a chunk index, each destination chunk by 256 bytes, so three per-thread offsets
  // made once per stage serve every piece.  Other block sizes derive each piece's place
  // from its index.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 wr[kWp];
  constexpr bool kLinear = NT == 256;
  struct WidenGeo {
    int src, dst0, dst1, dstr;  // dstr (ROPE): the chunk of rope values 8j..8j+7
  };
  auto widen_geo = [&]() -> WidenGeo {
    int tid_v = tid;
    asm volatile("" : "+v"(tid_v));
    const int r = tid_v >> 3, j = tid_v & 7, f = swz_mask(r);
    return WidenGeo{r * kRawRowBytes + 16 * j, r * kRowBytes + (((2 * j) ^ f) << 4),
                    r * kRowBytes + (((2 * j + 1) ^ f) << 4), r * kRowBytes + ((64 | (j ^ f)) << 4)};
  };
  // ROPE: eight bf16 rope values of row r of the stage, divided by the row's scale; the
  // thread of the row's first rope piece leaves the scale as used in the stage's slot
  auto put_rope = [&](MLA_LDS uint8_t* d, const u32x4& w, MLA_LDS float* ksl, int r, bool first) {
    const float sg = rope_scale(ksl[r]), inv = 1.f / sg;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __builtin_bit_cast(float, w[i] << 16) * inv;
      const float hi = __builtin_bit_cast(float, w[i] & 0xFFFF0000u) * inv;
      o[i] = (uint32_t)bf16_bits_rne(lo) | ((uint32_t)bf16_bits_rne(hi) << 16);
    }
    *(MLA_LDS u32x4*)d = u32x4{o[0], o[1], o[2], o[3]};
    if (first) {
      ksl[r] = sg;
      ksl[r + 32] = sg;
    }
  };
  auto put_bf16 = [&](MLA_LDS uint8_t* d0, MLA_LDS uint8_t* d1, const u32x4& w) {
    const uint2 b0 = e4m3x4_to_bf16x4(w[0]), b1 = e4m3x4_to_bf16x4(w[1]);
    const uint2 b2 = e4m3x4_to_bf16x4(w[2]), b3 = e4m3x4_to_bf16x4(w[3]);
    *(MLA_LDS u32x4*)d0 = u32x4{b0.x, b0.y, b1.x, b1.y};
    *(MLA_LDS u32x4*)d1 = u32x4{b2.x, b2.y, b3.x, b3.y};
  };
  auto take = [&](const MLA_LDS uint8_t* src, int i, const WidenGeo& wg) {
    if constexpr (kLinear) {
      if (ROPE || i < 4 || (tid & 7) < 4) wr[i] = *(const MLA_LDS u32x4*)(src + wg.src + 128 * i);
    } else {
      // the piece arithmetic is redone per call from an opaque copy of the thread id:
      // hoisted out of the stage loop it would hold registers the stage compute needs
      int tid_v = tid;
      asm volatile("" : "+v"(tid_v));
      const int c = tid_v + i * NT;
      if (i * NT + NT <= kRawPieces || tid + i * NT < kRawPieces) wr[i] = *(const MLA_LDS u32x4*)(src + c * 16);
    }
  };
  // ksl: the stage's scale slot (ROPE only)
  auto put = [&](MLA_LDS uint8_t* dst, int i, const WidenGeo& wg, MLA_LDS float* ksl) {
    if constexpr (kLinear) {
      if (ROPE && i == 4) put_rope(dst + wg.dstr, wr[i], ksl, tid >> 3, (tid & 7) == 0);
      else if (ROPE || i < 4 || (tid & 7) < 4) put_bf16(dst + wg.dst0 + 256 * i, dst + wg.dst1 + 256 * i, wr[i]);
    } else {
      int tid_v = tid;
      asm volatile("" : "+v"(tid_v));
      const int c = tid_v + i * NT;
      if (i * NT + NT <= kRawPieces || tid + i * NT < kRawPieces) {
        const int row = c / kRawPiecesPerRow, piece = c - row * kRawPiecesPerRow;
        MLA_LDS uint8_t* rowp = dst + row * kRowBytes;
        if (ROPE && piece >= 32)
          put_rope(rowp + swz_chunk(row, 64 + piece - 32) * 16, wr[i], ksl, row, piece == 32);
        else
          put_bf16(rowp + swz_chunk(row, 2 * piece) * 16, rowp + swz_chunk(row, 2 * piece + 1) * 16, wr[i]);
      }
    }
  };
  static_assert(!kLinear || kWp == 5, "256 threads: 4.5 (5 with ROPE) pieces each");

  // ---- prologue: stages 0 and 1 in flight, q, then stage 2 issued and stage 0 widened
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
    const uint8_t* qrow = a.q + (int64_t)t * a.q_tok;
    const float qinv = ROPE ? 1.f / rope_scale(a.q_scale != nullptr ? ld_const(a.q_scale + t) : 1.f) : 1.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const uint8_t* qh = qrow + (int64_t)(h0 + 16 * hb + ln) * a.q_head;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ROPE && ks >= 16) {
          // rope values 32(ks - 16) + 8gq .. + 7 (bf16 after the 512 codes), over the scale
          const uint4 w = *(const uint4*)(qh + 512 + 64 * (ks - 16) + 16 * gq);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
          uint32_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = (uint32_t)bf16_bits_rne(__builtin_bit_cast(float, ww[i] << 16) * qinv) |
                   ((uint32_t)bf16_bits_rne(__builtin_bit_cast(float, ww[i] & 0xFFFF0000u) * qinv) << 16);
          qf[hb][ks] = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
        } else {
          const uint2 w = *(const uint2*)(qh + 32 * ks + 8 * gq);
          const uint2 lo = e4m3x4_to_bf16x4(w.x), hi = e4m3x4_to_bf16x4(w.y);
          qf[hb][ks] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
      }
    }
  }
  float q_scale = a.q_scale != nullptr ? ld_const(a.q_scale + t) : 1.f;
  if (ROPE) q_scale = rope_scale(q_scale);
  const float scale_log2 = a.scale_log2 * q_scale;
  all_wait0();
  stage_barrier();
  if (nst > 2) m2 = issue(s_first + 2, 2, 2);
  {
    const WidenGeo wg = widen_geo();
#pragma unroll
    for (int i = 0; i < kWp; ++i) {
      take(raw, i, wg);
      put(tiles, i, wg, kscale);
    }
  }
  lgkm_wait0();

  using Acc = std::conditional_t<HB == 2, WaveAcc2, WaveAcc<HB>>;
  Acc acc;
  if constexpr (HB == 2) wave_acc2_init(acc); else wave_acc_init(acc);

#pragma unroll 1
  for (int k = 0; k < nst; ++k) {
    // stage k+1 has landed (k+2 may be in flight); tile k is whole; every wave is past
    // stage k-1, so its tile and the landing buffer of stage k are free
    if (k + 2 < nst) vm_wait_imm<kPerWave>(); else vm_wait_imm<0>();
    stage_barrier();
    // stage k+3 goes into the landing buffer of stage k (widened during step k-1): from
    // the compute's k-steps when the window covers it, else here
    const bool ahead = k + 3 < nst;
    const bool hook_issue = kHookIssue && a.flat && ahead && window_covers(s_first + k + 3);
    if (ahead && !hook_issue) m3 = issue(s_first + k + 3, (k + 3) % kSpRaw, (k + 3) % kSpScale);
    int rr[kPerWave], rmask = -1;
    const bool next = k + 1 < nst;
    const MLA_LDS uint8_t* wsrc = raw + ((k + 1) % kSpRaw) * kRawStageBytes;
    MLA_LDS uint8_t* wdst = tiles + ((k + 1) % kSpTiles) * kStageBytes;
    MLA_LDS float* wks = kscale + ((k + 1) % kSpScale) * 64;
    WidenGeo wg{0, 0, 0};
    auto hook = [&](int ks) {
      if (hook_issue) {
        const int q = ks - kIssueRead;
        if (q == 0) issue_read(s_first + k + 3, rr, rmask);
        if (q >= 2 && q <= 2 * kPerWave && (q & 1) == 0)
          issue_slot(std::true_type(), (k + 3) % kSpRaw, (k + 3) % kSpScale, q / 2 - 1, rr[q / 2 - 1]);
        if (q == 2 * kPerWave + 1) m3 = issue_mask(rmask);
      }
      if (!next) return;
      if (kLinear && ks == 0) wg = widen_geo();
      if (kTwoPhase) {
        if ((ks & 1) == 0 && ks / 2 < kWp) take(wsrc, ks / 2, wg);
        if ((ks & 1) == 1 && ks / 2 < kWp) put(wdst, ks / 2, wg, wks);
      } else if (ks < kWp) {
        take(wsrc, ks, wg);
        put(wdst, ks, wg, wks);
      }
    };
    // the lane geometry is rebuilt per stage from an opaque lane id: kept across the stage
    // loop it would take registers the compute needs
    int lane_g = lane;
    asm volatile("" : "+v"(lane_g));
    const LaneGeo lg = make_lane_geo(lane_g);
    const MLA_LDS float* ks = kscale + (k % kSpScale) * 64;
    if constexpr (HB == 2)
      stage_compute2<true>(tiles + (k % kSpTiles) * kStageBytes, qf, acc, m0, scale_log2, ks, lg, hook);
    else
      stage_compute<HB, true>(tiles + (k % kSpTiles) * kStageBytes, qf, acc, m0, scale_log2, ks, lg, hook);
    lgkm_wait0();  // the widened tile, before the barrier that hands it to the other waves
    m0 = m1;
    m1 = m2;
    m2 = m3;
  }

  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(a.err, kErrSparseIndex);
  if (__builtin_amdgcn_ballot_w64(bad_page) != 0 && lane == 0) atomicOr(a.err, kErrPageId);
  if constexpr (HB == 2) {
    // every wave is done with the stage buffers before they take the output rows
    stage_barrier();
    stage_epilogue2(acc, lane, h0, t, full, slot, a.H, a.out, a.o_tok, a.o_head, a.part_o, a.part_lse,
                    tiles + wave * 32 * 1024, XTRA ? a.sink : nullptr);
  }
  else
    stage_epilogue<HB>(acc, lane, h0, t, full, slot, a.H, a.out, a.o_tok, a.o_head, a.part_o, a.part_lse,
                       XTRA ? a.sink : nullptr);
}

// SMALL: balanced batch of at most 64 rows, no more rows than work-groups (planned per
// wave, see plan_run).
template <int HB, int NW, bool SMALL, bool DENSE, bool XTRA, bool ROPE>
__global__ __launch_bounds__(NW * 64, 1) void mla_sparse_kernel(const SparseArgs a, const SplitPlan plan) {
  // the widened tiles, then the fp8 landing buffers
  __shared__ __attribute__((aligned(1024))) uint8_t buf_raw[kSpLdsBytes];
  __shared__ __attribute__((aligned(256))) float ksc_raw[kSpScale * 64];
  __shared__ PlanLds L;
  MLA_LDS uint8_t* tiles = (MLA_LDS uint8_t*)buf_raw;
  MLA_LDS uint8_t* land = tiles + kSpTiles * kStageBytes;
  MLA_LDS float* ksc = (MLA_LDS float*)ksc_raw;
  plan_run<NW * 64, SMALL>(
      plan, L,
      [&](PlanLds& l) {
        if constexpr (DENSE) decode_fill<NW * 64>(a, l); else sparse_fill<NW * 64, XTRA>(a, l);
      },
      [&](int t) {
        if constexpr (DENSE) return decode_row_geo(a, t); else return sparse_row_geo<XTRA>(a, t);
      },
      [&](RowGeo* geo, int lane) {
        if constexpr (DENSE) decode_fill_wave(a, geo, lane); else sparse_fill_wave<XTRA>(a, geo, lane);
      },
      [&](int r, const RowGeo& g, int ta, int tc, bool full, int slot) {
        sparse_segment<HB, NW, DENSE, XTRA, ROPE>(a, tiles, land, ksc, (MLA_LDS int*)L.scan, r, g, ta, tc, full, slot);
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
  p.sink = a.sink;
  return p;
}

template <int HB, int NW>
static hipError_t launch_sparse_h(const SparseArgs& a, const SplitPlan& p, hipStream_t stream) {
  const dim3 grid(a.nparts >= 1 ? a.T * a.nparts : a.grid), block(NW * 64);
  const bool small = a.nparts == 0 && a.T <= 64 && a.T <= a.grid && ((!a.dense && !a.shared) || a.B <= 64);
  if (HB == 2 && NW == 4 && small && !a.q_bf16 && a.xidx == nullptr && a.sink == nullptr)
    return launch_fp8mma(a, p, stream);
  if (a.rope) {
    if (a.xidx != nullptr || a.sink != nullptr) return hipErrorInvalidValue;  // refused by the host checks
    if (a.dense) {
      if (small) hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, true, true, false, true>), grid, block, 0, stream, a, p);
      else hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, false, true, false, true>), grid, block, 0, stream, a, p);
    } else {
      if (small) hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, true, false, false, true>), grid, block, 0, stream, a, p);
      else hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, false, false, false, true>), grid, block, 0, stream, a, p);
    }
  } else if (a.dense) {
    if (small) hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, true, true, false, false>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, false, true, false, false>), grid, block, 0, stream, a, p);
  } else if (a.xidx != nullptr || a.sink != nullptr) {
    if (small) hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, true, false, true, false>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, false, false, true, false>), grid, block, 0, stream, a, p);
  } else {
    if (small) hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, true, false, false, false>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_sparse_kernel<HB, NW, false, false, false, false>), grid, block, 0, stream, a, p);
  }
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
