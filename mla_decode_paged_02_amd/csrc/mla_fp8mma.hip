// MLA decode over an fp8 e4m3 latent cache with the scores on fp8 MFMA (gfx950): the dense
// decode over a paged cache and the sparse decode over index lists.
//
// What is computed follows generic_flare_mla_decode_kv_cache_ragged (summary; Args q,
// q_scale_ptr, kv_collection, input_row_offsets, scale, output, d_indices, indices_stride,
// topk_lengths; Parameters mask_str, local_window_size, sparse_mla, fold_shared_index,
// per_token_scale_rope_aware): mla_decode_paged_fp8 and mla_decode_paged_sparse(_shared),
// whose general kernel is mla_sparse.hip.  This kernel serves their balanced split of at
// most 64 rows (and sequences) at 128 heads, without a sink or second stream.  With SPARSE
// the 32 keys of a stage are the rows its 32 list positions name, each gathered by its own
// lane; otherwise they are 32 consecutive positions of the sequence through its page table.
//
// Per work-group (4 waves, one per SIMD) and 32-key stage:
//   scores    wave w computes S^T = K Q^T for heads 32w..32w+31 straight from the e4m3
//             codes: v_mfma_f32_32x32x64_f8f6f4 over the 576 columns (9 k-steps), or with
//             ROPE over the 512 latent columns (8 k-steps) plus v_mfma_f32_32x32x16_bf16 over
//             the 64 bf16 rope columns (4 k-steps) into a second accumulator, so that the
//             logit is scale * (sigma_q sigma_k S_latent + S_rope) exactly;
//   values    the stage's 512 latent columns are widened to bf16 (exact) into a value tile:
//             wave w owns output columns 128w..128w+127 of all heads, O^T += V^T (P sigma_k)^T
//             with the bf16 weights of every head exchanged through LDS (the row scale rides
//             on the weight, so V stays the bare codes and P keeps bf16 precision).
// Step k: the score MFMAs of stage k run with the first value MFMAs of stage k-1 and the
// widening of stage k, and the other value MFMAs of stage k-1 run while the vector units
// turn the scores of stage k into weights, which every wave then publishes for its heads
// in one of two LDS slots; the barrier at the top of the next step makes them visible, so
// a step has one barrier.
//
// Layout of a stage's fp8 rows in LDS: chunk-major, 16-byte chunk c of row r at
// (32 c + r) * 16.  A score operand (lane 32g + i: row i, bytes 64 ks + 32g .. + 31, two
// chunks) is then two reads of 512 contiguous bytes per half-wave, and the stage loads put
// chunk 2J + (lane >> 5) of row lane & 31 at load J: a per-lane constant plus 32 J bytes.
// The operand layout of the fp8 MFMA (lane 32g + i holds 32 k-values of row i of A and of
// column i of B, the halves g disjoint; D as for the bf16 32x32 MFMAs) was checked on
// MI355X against exact products.
#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_plan.h"
#include "mla_rows.h"
#include "mla_stage.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kF8Raw = 3;                 // fp8 stage buffers: scores of k, k+1 landed, k+2 in flight
constexpr int kF8PidWindow = 512;         // page ids of the segment held in LDS
constexpr int kF8PBytes = 4 * 2 * 64 * 16;  // weights: [head block][value k-step][lane] x 16 B
constexpr int kF8VBytes = 32 * kRowBytes;   // one bf16 value tile (rows of 1152 bytes, 1024 used)
constexpr int kF8Loads = 5;               // row loads per wave and stage (the last may repeat one)
constexpr int kF8Scales = 4;              // scale slots: stage k-1 (softmax), k, k+1, k+2 (loading)

template <bool ROPE>
struct F8Geo {
  static constexpr int kRow = ROPE ? 640 : 576;        // bytes of a cache / q row
  static constexpr int kChunks = kRow / 16;            // 40 / 36
  static constexpr int kStage = kStageKeys * kRow;     // 20480 / 18432
  static constexpr int kDma = kStage / 1024;           // 20 / 18 wave-wide loads
  static constexpr int kKs8 = ROPE ? 8 : 9;            // fp8 k-steps of 64 columns
  static_assert(kDma <= 4 * kF8Loads, "every stage load has a wave");
};

struct F8Lds {
  RowGeo geo[256];            // per-wave planning tables (64 rows each)
  int pids[kF8PidWindow];     // page-id window of the segment
  float ksc[kF8Scales][64];   // the stages' row scales (lanes 32..63 repeat 0..31)
};

// LDS swizzle of the bf16 value tile (rows of 72 16-byte chunks, 64 used), the one the
// transposing value reads of mla_decode2.hip were measured conflict-free with.
__device__ __forceinline__ int f8_swz(int r) { return ((r >> 4) & 1) | (((r >> 1) & 1) << 1) | (((r ^ (r >> 2)) & 1) << 2); }

__device__ __forceinline__ void mfma32_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Wait states between the last write of a 16-pass MFMA into the accumulation registers
// and other instructions reading them (24, above the 18 the longest such distance needs):
// these MFMAs are inline assembly, which the compiler's hazard tracking does not see.
__device__ __forceinline__ void fence_o(f32x16 (&o)[4][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]));
#pragma unroll
  for (int cb = 1; cb < 4; ++cb) asm volatile("" : "+a"(o[cb][0]), "+a"(o[cb][1]), "+a"(o[cb][2]), "+a"(o[cb][3]));
}

template <int KPAGES, bool ROPE, bool SPARSE>
__device__ __forceinline__ void fp8mma_segment(const SparseArgs& a, MLA_LDS uint8_t* raw, MLA_LDS uint8_t* vt,
                                               MLA_LDS uint8_t* xbuf, F8Lds& L, int t, const RowGeo& g, int ta,
                                               int tc, bool full, int slot) {
  using G = F8Geo<ROPE>;
  constexpr int NT = 256;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 5, li = lane & 31;
  const int h0 = wave * 32;
  MLA_LDS int* pids = (MLA_LDS int*)L.pids;
  auto ksl = [&](int st) { return (MLA_LDS float*)L.ksc[st % kF8Scales]; };  // scale slot of stage st
  // the weights, rescale factors [4][32] and flags [4] of a stage, in two slots (stage s in
  // slot s & 1), and the epilogue's 1/l [128]
  auto pbuf = [&](int sl) { return xbuf + sl * kF8PBytes; };
  auto alpha_s = [&](int sl) { return (MLA_LDS float*)(xbuf + 2 * kF8PBytes + 512 * sl); };
  auto flag_s = [&](int sl) { return (MLA_LDS int*)(xbuf + 2 * kF8PBytes + 1024 + 16 * sl); };
  MLA_LDS float* inv_s = (MLA_LDS float*)(xbuf + 2 * kF8PBytes + 1024 + 64);

  const int first_tile = __builtin_amdgcn_readfirstlane(g.lo / kTileKeys);
  const int klo = __builtin_amdgcn_readfirstlane(max(g.lo, (first_tile + ta) * kTileKeys));
  const int khi = __builtin_amdgcn_readfirstlane(min(g.hi, (first_tile + tc) * kTileKeys));
  const int s_first = klo / kStageKeys;
  const int nst = (khi - 1) / kStageKeys - s_first + 1;
  const int32_t* pt = a.page_table + (int64_t)__builtin_amdgcn_readfirstlane(g.b) * a.pt_row;
  const int p_last = (khi - 1) / a.PS;
  const int npages32 = (int)min(a.num_rows / a.PS, (int64_t)INT32_MAX);
  // SPARSE: list row g.b of d_indices; list position p of the segment is key p
  const int32_t* ilist = SPARSE ? a.idx + (int64_t)__builtin_amdgcn_readfirstlane(g.b) * a.idx_row : nullptr;
  static_assert(!SPARSE || KPAGES == 0, "the sparse rows are gathered one by one");

  // every wave must be done with the buffers and window of anything before
  all_wait0();
  stage_barrier();

  // ---- query fragments (B operand of S^T = K Q^T), loaded first so that their latency
  // overlaps the window's: lane 32g + i holds q[head h0 + i]
  // bytes 64 ks + 32 g .. + 31 (e4m3), with ROPE also bf16 rope columns 16 kr + 8 g .. + 7
  const uint8_t* qh = a.q + (int64_t)t * a.q_tok + (int64_t)(h0 + li) * a.q_head;
  i32x8 qf[G::kKs8];
#pragma unroll
  for (int ks = 0; ks < G::kKs8; ++ks) {
    const uint4 lo = *(const uint4*)(qh + 64 * ks + 32 * lg);
    const uint4 hi = *(const uint4*)(qh + 64 * ks + 32 * lg + 16);
    qf[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  bf16x8 qr[4];
  if constexpr (ROPE) {
#pragma unroll
    for (int kr = 0; kr < 4; ++kr) qr[kr] = *(const bf16x8*)(qh + 512 + 32 * kr + 16 * lg);
  }

  // ---- page-id window [pbase, pbase + kF8PidWindow) (entries past the segment are -1);
  // SPARSE: the listed rows of list positions [pbase, pbase + kF8PidWindow), checked against
  // the pool as they are stored (-1 past the segment, for negative entries, which are
  // skipped, and for rows past the end of the pool, which are skipped and flagged)
  int pbase = SPARSE ? klo : klo / a.PS;
  int pv[kF8PidWindow / NT];
  bool bad_idx = false;
  auto window_load = [&]() {
#pragma unroll
    for (int i = 0; i < kF8PidWindow / NT; ++i) {
      const int p = pbase + tid + i * NT;
      if (SPARSE)
        pv[i] = p < khi ? ilist[p] : -1;
      else
        pv[i] = p <= p_last ? pt[p] : -1;
    }
  };
  auto window_store = [&]() {
#pragma unroll
    for (int i = 0; i < kF8PidWindow / NT; ++i) {
      int r = pv[i];
      if (SPARSE && (int64_t)r >= a.num_rows) {
        bad_idx = true;
        r = -1;
      }
      pids[tid + i * NT] = SPARSE && r < 0 ? -1 : r;
    }
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
    window_load();
    all_wait0();
    window_store();
    lgkm_wait0();
    stage_barrier();
  }

  bool bad_page = false;
  // page of the stage last looked up, its id, and the id of the page after it (read from
  // the window ahead of need; -1 past the window)
  int lp_last = -1, pid_last = -1, pid_next_v = -1;
  auto stage_page = [&](int st) {
    const int kb0 = st * kStageKeys;  // consecutive stages: the page stays or advances by one
    if (lp_last >= 0 && kb0 >= lp_last * a.PS && kb0 < (lp_last + 1) * a.PS) return pid_last;
    if (lp_last >= 0 && kb0 >= (lp_last + 1) * a.PS && kb0 < (lp_last + 2) * a.PS &&
        lp_last + 1 < pbase + kF8PidWindow) {
      lp_last += 1;
      pid_last = __builtin_amdgcn_readfirstlane(pid_next_v);
    } else {
      const int lp = kb0 / a.PS;
      if (lp >= pbase + kF8PidWindow) window_move(lp);
      lp_last = lp;
      pid_last = __builtin_amdgcn_readfirstlane(pids[lp - pbase]);
    }
    const int nx = lp_last + 1 - pbase;
    pid_next_v = nx < kF8PidWindow ? pids[nx] : -1;
    return pid_last;
  };
  // a stage inside one valid page: the scalar base of its first row, else null
  auto fast_base = [&](int st, int pa) -> const uint8_t* {
    const int kbase = st * kStageKeys;
    if (KPAGES != 0 && kbase >= klo && kbase + kStageKeys <= khi && pa >= 0 && pa < npages32)
      return a.cache + (int64_t)pa * a.page_bytes + (int64_t)((uint32_t)kbase % (uint32_t)a.PS) * G::kRow;
    return nullptr;
  };
  // load jj of this wave: global load J (the spare ones repeat the last, same bytes to the
  // same place); lane -> row lane & 31, chunk 2J + (lane >> 5)
  auto load_j = [&](int jj) { return min(jj * 4 + wave, G::kDma - 1); };
  int lane_c = lane;
  asm volatile("" : "+v"(lane_c));
  const uint32_t doff0 = (uint32_t)((lane_c & 31) * G::kRow + 16 * (lane_c >> 5));
  auto fast_load = [&](const uint8_t* base, MLA_LDS uint8_t* dst, int jj) {
    const int J = load_j(jj);
    dma16_base_nt(base, doff0 + 32 * J, dst + J * 1024);
  };
  // the stage's 32 row scales into its slot (every wave loads the same 32 floats)
  auto scale_src_fast = [&](int st, int pa) -> const void* {
    if (a.cache_scale == nullptr) return a.zero_row + kSparseOneOffset;
    const int kbase = st * kStageKeys;
    return a.cache_scale + (int64_t)pa * a.cs_page + ((uint32_t)kbase % (uint32_t)a.PS) + (lane_c & 31);
  };
  // SPARSE: the place of listed row r (page * PS + slot, or r itself in a flat pool) and of
  // its scale
  auto sparse_row = [&](int r) -> const uint8_t* {
    if (a.flat) return a.cache + (int64_t)r * G::kRow;
    const int pg = r / a.PS;
    return a.cache + (int64_t)pg * a.page_bytes + (int64_t)(r - pg * a.PS) * G::kRow;
  };
  auto sparse_scale = [&](int r) -> const void* {
    if (a.cache_scale == nullptr) return a.zero_row + kSparseOneOffset;
    if (a.flat) return a.cache_scale + r;
    const int pg = r / a.PS;
    return a.cache_scale + (int64_t)pg * a.cs_page + (r - pg * a.PS);
  };
  // pa: the stage's page id when a stage lies in one page (KPAGES), which the window may
  // not hold yet (the prologue issues before it is stored).  Returns the stage's keys that
  // count (SPARSE: the listed ones; else all, the range mask covers the rest).
  auto issue_general = [&](int st, int bi, int pa) -> uint32_t {
    MLA_LDS uint8_t* dst = raw + bi * G::kStage;
    const int kbase = st * kStageKeys;
    if (SPARSE) {
      if (min(kbase + kStageKeys, khi) - 1 >= pbase + kF8PidWindow) window_move(max(kbase, klo));
    } else if (KPAGES == 0) {
      const int lp_hi = (min(kbase + kStageKeys, khi) - 1) / a.PS;
      if (lp_hi >= pbase + kF8PidWindow) window_move(max(kbase, klo) / a.PS);
    }
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
    const int row = lane_v & 31, key = kbase + row;
    const uint8_t* rsrc = nullptr;  // this lane's row, null: the zero row
    const void* ssrc = a.zero_row;  // and its scale (0 for a key that does not count)
    if (SPARSE) {
      const int r = key >= klo && key < khi ? pids[key - pbase] : -1;
      if (r >= 0) {
        rsrc = sparse_row(r);
        ssrc = sparse_scale(r);
      }
    } else if (key >= klo && key < khi) {
      const int lp = key / a.PS;
      const int pid = KPAGES != 0 ? pa : pids[lp - pbase];
      if (pid >= 0 && pid < npages32) {
        rsrc = a.cache + (int64_t)pid * a.page_bytes + (int64_t)(key - lp * a.PS) * G::kRow;
        ssrc = a.cache_scale == nullptr ? (const void*)(a.zero_row + kSparseOneOffset)
                                        : (const void*)(a.cache_scale + (int64_t)pid * a.cs_page + (key - lp * a.PS));
      } else {
        bad_page = true;
      }
    }
#pragma unroll
    for (int jj = 0; jj < kF8Loads; ++jj) {
      const int J = load_j(jj);
      const int c = 2 * J + (lane_v >> 5);
      dma16_nt((rsrc != nullptr ? rsrc : a.zero_row) + 16 * c, dst + J * 1024);
    }
    dma4(ssrc, ksl(st - s_first));
    return SPARSE ? (uint32_t)__builtin_amdgcn_ballot_w64(lane_v < 32 && rsrc != nullptr) : ~0u;
  };
  // SPARSE inside the stage loop: this lane's row and scale sources of stage st (the loads
  // themselves are spread over the next score k-steps) and the stage's keys that count
  struct Gather {
    const uint8_t* row;  // the row's chunk for this lane's half (the zero row when skipped)
    const void* scale;
    uint32_t mask;
  };
  auto gather_prep = [&](int st) -> Gather {
    const int kbase = st * kStageKeys;
    if (min(kbase + kStageKeys, khi) - 1 >= pbase + kF8PidWindow) window_move(max(kbase, klo));
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
    const int key = kbase + (lane_v & 31);
    const int r = key >= klo && key < khi ? pids[key - pbase] : -1;
    Gather gp{a.zero_row + 16 * (lane_v >> 5), a.zero_row, 0u};
    if (r >= 0) {
      gp.row = sparse_row(r) + 16 * (lane_v >> 5);
      gp.scale = sparse_scale(r);
    }
    gp.mask = (uint32_t)__builtin_amdgcn_ballot_w64(lane_v < 32 && r >= 0);
    return gp;
  };
  auto issue = [&](int st, int bi, int pa) -> uint32_t {
    const uint8_t* fb = fast_base(st, pa);
    if (fb == nullptr) return issue_general(st, bi, pa);
#pragma unroll
    for (int jj = 0; jj < kF8Loads; ++jj) fast_load(fb, raw + bi * G::kStage, jj);
    dma4(scale_src_fast(st, pa), ksl(st - s_first));
    return ~0u;
  };

  // ---- prologue: stages 0 and 1 (their page ids by scalar loads, which the full wait
  // covers), the window for the loop, and zeros in the value tile "stage -1" uses
  auto direct_page = [&](int st) { return ld_const(pt + st * kStageKeys / a.PS); };
  const int pa0 = KPAGES != 0 ? direct_page(s_first) : 0;
  const int pa1 = (KPAGES != 0 && nst > 1) ? direct_page(s_first + 1) : 0;
  int pa_n = (KPAGES != 0 && nst > 2) ? direct_page(s_first + 2) : 0;
  // stage "-1" reads a scale slot no load writes: zeros, so its weights are 0 x 0
  for (int i = tid; i < kF8Scales * 64; i += NT) ((MLA_LDS float*)L.ksc)[i] = 0.f;
  lgkm_wait0();
  stage_barrier();
  // the token scale after that wait, which drains the scalar loads too: its latency hides
  // under the stage loads
  const float q_scale = a.q_scale != nullptr ? ld_const(a.q_scale + t) : 1.f;
  const float qsl = a.scale_log2 * q_scale;  // logit units per code product (times sigma_k)
  // keys that count in stages k and k+1 (SPARSE; all otherwise)
  uint32_t msk0 = issue(s_first, 0, pa0), msk1 = ~0u;
  if (nst > 1) msk1 = issue(s_first + 1, 1, pa1);
  if (KPAGES != 0) window_load();
  {
    MLA_LDS uint8_t* z = vt + kF8VBytes;
    for (int i = tid; i < kF8VBytes / 16; i += NT) *(MLA_LDS u32x4*)(z + 16 * i) = u32x4{0, 0, 0, 0};
  }
  all_wait0();
  if (KPAGES != 0) window_store();
  lgkm_wait0();  // made visible to the other waves by the barrier at the loop top

  f32x16 O[4][4];  // O^T tile (column block cb, head block hb), lane 32g+i: head 32hb + i
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      O[cb][hb] = f32x16{};
      asm volatile("" : "+a"(O[cb][hb]));
    }
  float m = -INFINITY, l = 0.f;  // own head h0 + li (lanes i and 32 + i agree on m)
  uint32_t pk[8];                // weights of the last scored stage (bf16 pairs)
  float alpha = 1.f;             // its rescale factor of this head
  int rflag = 0;                 // some head of this wave rescaled at that stage
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = 0;
  // "stage -1": zero weights and no rescale, in slot 1 (visible after the barrier at the
  // loop top)
  {
    MLA_LDS uint8_t* pw = pbuf(1) + wave * 2048 + lane * 16;
    *(MLA_LDS u32x4*)pw = u32x4{0, 0, 0, 0};
    *(MLA_LDS u32x4*)(pw + 1024) = u32x4{0, 0, 0, 0};
    if (lg == 0) alpha_s(1)[wave * 32 + li] = 1.f;
    if (lane == 0) flag_s(1)[wave] = 0;
  }

  // Transposing value reads (the layout of mla_decode2.hip): lane 16G + 4r + q (G = 2g + c)
  // reads row 16kp + 8h + 4g + r, chunk 16w + 4cb + 2c + (q >> 1); four per-lane bases.
  int vb[2][2];
  {
    const int G2 = lane >> 4, gg = G2 >> 1, c = G2 & 1, r = (lane >> 2) & 3, q = lane & 3;
    const int brow = 4 * gg + r;
    const int X = (2 * c + (q >> 1)) ^ f8_swz(brow);
    const int base = brow * kRowBytes + 256 * wave + 8 * (q & 1);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) vb[kp][pp] = base + ((X ^ kp ^ (4 * pp)) << 4);
  }
  // widening: piece p = tid + 256 u (u < 4) is chunk p >> 5 (of the 32 latent chunks) of row
  // p & 31; it becomes bf16 chunks 2c and 2c + 1 of that row of the value tile
  int wdst[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int tid_v = tid;
    asm volatile("" : "+v"(tid_v));
    const int p = tid_v + 256 * u, c = p >> 5, r = p & 31, f = f8_swz(r);
    wdst[u] = r * kRowBytes + ((((2 * c) & ~7) | (((2 * c) ^ f) & 7)) << 4);
  }

  // Step k runs the score MFMAs of stage k with the first value MFMAs of stage k-1 and the
  // widening of stage k's values (phase A), then the other value MFMAs of stage k-1 while
  // the vector units turn the scores of stage k into weights (phase B), and publishes
  // them.  Every step runs the whole stream: at k = 0 the values of "stage -1" are zero
  // weights on the zeroed value tile, and at k = nst the scores of a stale buffer are
  // computed and masked out entirely.
  auto pinv = [](f32x16& v) { asm volatile("" : "+v"(v)); };
  auto pin = [](float& v) { asm volatile("" : "+v"(v)); };
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll 1
  for (int k = 0; k <= nst; ++k) {
    // ---- stage k has landed (stage k+1 may still be in flight)
    if (k < nst) {
      if (k >= 1 && k + 1 < nst) vm_wait_imm<kF8Loads + 1>(); else vm_wait_imm<0>();
    }
    lgkm_wait0();     // this wave's weights of stage k-1 are in LDS
    stage_barrier();  // also: every wave is done with step k-1 (its buffers and weight slot)
    const int kn = k + 2;
    const uint8_t* fb = nullptr;
    int pa_k = 0;
    uint32_t msk2 = ~0u;
    Gather gk{nullptr, nullptr, 0u};  // SPARSE: stage k+2's sources
    if (kn < nst && SPARSE) {
      gk = gather_prep(s_first + kn);
      msk2 = gk.mask;
    } else if (kn < nst) {
      pa_k = pa_n;
      fb = fast_base(s_first + kn, pa_n);
      if (fb == nullptr) msk2 = issue_general(s_first + kn, kn % kF8Raw, pa_n);
      if (KPAGES != 0 && kn + 1 < nst) pa_n = stage_page(s_first + kn + 1);
    }
    MLA_LDS uint8_t* fdst = raw + (kn % kF8Raw) * G::kStage;
    const MLA_LDS uint8_t* rs = raw + (k % kF8Raw) * G::kStage;     // stage k's rows
    const MLA_LDS float* ksp = ksl(k);                               // stage k's scales
    const MLA_LDS uint8_t* vrd = vt + ((k + 1) & 1) * kF8VBytes;    // values of stage k-1
    MLA_LDS uint8_t* vwr = vt + (k & 1) * kF8VBytes;                // values of stage k
    auto kread = [&](int ks) {
      const u32x4 lo = *(const MLA_LDS u32x4*)(rs + ((4 * ks + 2 * lg) * 32 + li) * 16);
      const u32x4 hi = *(const MLA_LDS u32x4*)(rs + ((4 * ks + 2 * lg + 1) * 32 + li) * 16);
      return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto rread = [&](int kr) { return *(const MLA_LDS bf16x8*)(rs + ((32 + 2 * kr + lg) * 32 + li) * 16); };
    auto vread = [&](int kp, int cb) {
      const int o0 = 1152 * 16 * kp + 128 * (cb >> 1), o1 = o0 + 1152 * 8;
      const bf16x4 a0 = ds_read_tr16(vrd + vb[kp][cb & 1] + o0);
      const bf16x4 a1 = ds_read_tr16(vrd + vb[kp][cb & 1] + o1);
      return bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    };
    auto pread = [&](int hb, int kp) {
      return *(const MLA_LDS bf16x8*)(pbuf((k + 1) & 1) + lane * 16 + hb * 2048 + kp * 1024);
    };

    // ---- the weights, rescale factors and flags of stage k-1 (published by every wave at
    // the end of step k-1, visible since the barrier)
    const int slp = (k + 1) & 1;
    bf16x8 vf[8];  // V^T fragment 4kp + cb; at most two live
    vf[0] = vread(0, 0);
    bf16x8 pf0[4], pf1[4];  // P^T (kp, hb)
    {
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      const i32x4 fl = *(const MLA_LDS i32x4*)flag_s(slp);
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pf0[hb] = pread(hb, 0);
      // O holds the values of stages < k-1 relative to the maxima before stage k-1: bring
      // the rescaled heads to their new maxima before stage k-1's values are added
      if ((fl[0] | fl[1] | fl[2] | fl[3]) != 0) {
        fence_o(O);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const float al = fl[hb] != 0 ? alpha_s(slp)[hb * 32 + li] : 1.f;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            O[cb][hb] *= al;
            const int n = 4 * hb + cb + 1;
            if (n < 16)
              asm volatile("" : "+a"(O[cb][hb]), "+a"(O[n & 3][n >> 2]));
            else
              asm volatile("" : "+a"(O[cb][hb]));
          }
        }
        asm volatile("s_nop 4" ::: "memory");
      }
    }
    // value op j = 16kp + 4cb + hb of stage k-1 (and the operand reads it needs next)
    auto pv_op = [&](int j) {
      const int kp = j >> 4, cb = (j >> 2) & 3, hb = j & 3;
      if (hb == 0 && j + 4 < 32) vf[(j >> 2) + 1] = vread((j + 4) >> 4, ((j + 4) >> 2) & 3);
      mfma32_acc(O[cb][hb], vf[4 * kp + cb], kp == 0 ? pf0[hb] : pf1[hb]);
      if (j >= 12 && j < 16) pf1[j - 12] = pread(j - 12, 1);
    };

    // ---- phase A: the score MFMAs of stage k, value ops 0..7 of stage k-1, the widening
    // of stage k's 512 latent columns (piece u: read at k-step u, converted and stored at
    // u + 4), stage k's key scales, and the loads of stage k+2
    f32x16 S, R;
    float ksc[16], kq[16];  // stage k's key scales sigma and sigma * qsl, key 8r + 4g + q at 4r + q
    constexpr int KS = G::kKs8 + (ROPE ? 4 : 0);  // MFMA k-steps of the stage
    static_assert(KS >= 8 && KS > kF8Loads, "room for the value ops, the widening and the loads");
    {
      i32x8 kf[G::kKs8];
      bf16x8 rf8[4];
      u32x4 wr[4];
      kf[0] = kread(0);
      kf[1] = kread(1);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        {
          const int n = i + 2;
          if (n < G::kKs8) kf[n] = kread(n);
          else if (ROPE && n < KS) rf8[n - G::kKs8] = rread(n - G::kKs8);
        }
        if (i < 4) wr[i] = *(const MLA_LDS u32x4*)(rs + (tid + 256 * i) * 16);
        if (i >= 4 && i < 8) {
          const u32x4 w = wr[i - 4];
          const uint2 b0 = e4m3x4_to_bf16x4(w[0]), b1 = e4m3x4_to_bf16x4(w[1]);
          const uint2 b2 = e4m3x4_to_bf16x4(w[2]), b3 = e4m3x4_to_bf16x4(w[3]);
          *(MLA_LDS u32x4*)(vwr + wdst[i - 4]) = u32x4{b0.x, b0.y, b1.x, b1.y};
          // chunk 2c + 1 sits next to chunk 2c: the swizzle flips bits 0..2 of the chunk
          // index by s(r), and 2c ^ s(r) and (2c + 1) ^ s(r) differ in bit 0 only
          *(MLA_LDS u32x4*)(vwr + (wdst[i - 4] ^ 16)) = u32x4{b2.x, b2.y, b3.x, b3.y};
        }
        if (i < 4) {
          typedef float f32x4_t __attribute__((ext_vector_type(4)));
          const f32x4_t v = *(const MLA_LDS f32x4_t*)(ksp + 8 * i + 4 * lg);
          ksc[4 * i] = v.x;
          ksc[4 * i + 1] = v.y;
          ksc[4 * i + 2] = v.z;
          ksc[4 * i + 3] = v.w;
        }
        if (i >= 4 && i < 8) {
#pragma unroll
          for (int e = 4 * (i - 4); e < 4 * (i - 4) + 4; ++e) {
            kq[e] = ksc[e] * qsl;
            pin(kq[e]);
          }
        }
        if (i < G::kKs8) {
          S = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[i], qf[i], i == 0 ? f32x16{} : S, 0, 0, 0, 0, 0, 0);
        } else if constexpr (ROPE) {
          const int kr = i - G::kKs8;
          R = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf8[kr], qr[kr], kr == 0 ? f32x16{} : R, 0, 0, 0);
        }
        if (i < 8) pv_op(i);
        if (i < kF8Loads && fb != nullptr) fast_load(fb, fdst, i);
        if (i == kF8Loads && fb != nullptr) dma4(scale_src_fast(s_first + kn, pa_k), ksl(kn));
        if (SPARSE && kn < nst) {
          if (i < kF8Loads) dma16_nt(gk.row + 32 * load_j(i), fdst + load_j(i) * 1024);
          if (i == kF8Loads) dma4(gk.scale, ksl(kn));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- phase B: value ops 8..31 of stage k-1, with the online softmax of stage k for
    // heads h0 + i (lanes i and 32 + i: keys 8r + 4g + q of register 4r + q) in pinned
    // pieces between them: logits (ops 8..11), running max (9..12), the head's max over
    // both lane halves and the lazy rescale (13..15), one power per op (16..31) and its
    // weight and denominator term one op later.
    // Only a segment's first and last stage (and the stale stage after the last) have keys
    // to mask: the other stages branch around the mask.
    {
      const uint32_t valid = k < nst ? range_bits((s_first + k) * kStageKeys, klo, khi) & msk0 : 0u;
      const bool partial = valid != 0xFFFFFFFFu;
      const uint32_t vbits = valid >> (4 * lg);
      float x[16];
      float lmax = -INFINITY, mx = 0.f, m_new = 0.f, mref = 0.f;
      uint32_t hsw0 = 0, hsw1 = 0;
      float pw[16];  // powers, one op ahead of their weights
      auto weigh = [&](int e) {
        // the weight p sigma_k as rounded for the MFMA; the denominator sums p (the value
        // rows are the bare codes)
        float pe = pw[e];
        pin(pe);
        l += pe;
        const float w = pe * ksc[e];
        if (e & 1) {
          const bf16x2_t w2 = {(__bf16)pw[e - 1], (__bf16)w};
          pk[e >> 1] = __builtin_bit_cast(uint32_t, w2);
          asm volatile("" : "+v"(pk[e >> 1]));
        } else {
          pw[e] = w;  // held until its pair is packed
          pin(pw[e]);
        }
        pin(l);
      };
#pragma unroll
      for (int j = 8; j < 32; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        if (j == 8) {
          pinv(S);
          if (ROPE) pinv(R);
        }
        if (j >= 8 && j < 12) {
#pragma unroll
          for (int e = 4 * (j - 8); e < 4 * (j - 8) + 4; ++e) {
            float v = S[e] * kq[e];
            if (ROPE) v = __builtin_fmaf(R[e], a.scale_log2, v);
            x[e] = v;
          }
          if (partial) {
#pragma unroll
            for (int e = 4 * (j - 8); e < 4 * (j - 8) + 4; ++e) {
              const int row = 8 * (e >> 2) + (e & 3);  // minus 4g, folded into vbits
              x[e] = ((vbits >> row) & 1u) ? x[e] : -INFINITY;
            }
          }
#pragma unroll
          for (int e = 4 * (j - 8); e < 4 * (j - 8) + 4; ++e) pin(x[e]);
        }
        if (j >= 9 && j < 13) {
          const int e0 = 4 * (j - 9);
          pin(lmax);
          lmax = fmaxf(lmax, fmaxf(fmaxf(x[e0], x[e0 + 1]), fmaxf(x[e0 + 2], x[e0 + 3])));
          pin(lmax);
        }
        if (j == 13) {
          const uint32_t bb = __builtin_bit_cast(uint32_t, lmax);
          const auto hsw = __builtin_amdgcn_permlane32_swap(bb, bb, false, false);
          hsw0 = (uint32_t)hsw[0];
          hsw1 = (uint32_t)hsw[1];
          asm volatile("" : "+v"(hsw0), "+v"(hsw1));
        }
        if (j == 14) {
          mx = fmaxf(__builtin_bit_cast(float, hsw0), __builtin_bit_cast(float, hsw1));
          pin(m);
          m_new = mx > m + kRescaleSlack ? mx : m;
          pin(m_new);
        }
        if (j == 15) {
          const float ex = fast_exp2(m - m_new);  // 0 while m is -inf; unused unless m_new != m
          // O is exactly zero while m is -inf: only a finite old maximum needs the rescale
          const uint64_t rf = __builtin_amdgcn_ballot_w64(m_new != m && m != -INFINITY);
          alpha = m_new != m ? ex : 1.f;
          m = m_new;
          mref = m == -INFINITY ? 0.f : m;
          l *= alpha;
          rflag = rf != 0 ? 1 : 0;
          pin(mref);
          pin(l);
        }
        if (j >= 16) {
          const int e = j - 16;
          float a0 = x[e];
          pin(a0);
          pw[e] = fast_exp2(a0 - mref);
          pin(pw[e]);
        }
        if (j >= 17) weigh(j - 17);
        pv_op(j);
      }
      __builtin_amdgcn_sched_barrier(0);
      weigh(15);
    }
    // ---- publish the weights, rescale factor and flag of stage k (own head block) into
    // slot k & 1: every wave is done with that slot's stage k-2 since the barrier above
    {
      MLA_LDS uint8_t* pw = pbuf(k & 1) + wave * 2048 + lane * 16;
      *(MLA_LDS u32x4*)pw = u32x4{pk[0], pk[1], pk[2], pk[3]};
      *(MLA_LDS u32x4*)(pw + 1024) = u32x4{pk[4], pk[5], pk[6], pk[7]};
      if (lg == 0) alpha_s(k & 1)[wave * 32 + li] = alpha;
      if (lane == 0) flag_s(k & 1)[wave] = rflag;
    }
    msk0 = msk1;
    msk1 = msk2;
  }

  if (bad_page) atomicOr(a.err, kErrPageId);
  if (SPARSE && __builtin_amdgcn_ballot_w64(bad_idx) != 0 && lane == 0) atomicOr(a.err, kErrSparseIndex);

  // ---- epilogue: each head's 1/l from its owner, then the wave's 128 columns of every
  // head, normalised, through LDS to contiguous stores
  {
    const uint32_t lb = __builtin_bit_cast(uint32_t, l);
    const auto hsw = __builtin_amdgcn_permlane32_swap(lb, lb, false, false);
    const float l_tot = __builtin_bit_cast(float, (uint32_t)hsw[0]) + __builtin_bit_cast(float, (uint32_t)hsw[1]);
    if (lg == 0) {
      inv_s[h0 + li] = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (!full) a.part_lse[(int64_t)slot * a.H + h0 + li] = l_tot > 0.f ? m + __log2f(l_tot) : -INFINITY;
    }
  }
  fence_o(O);
  lgkm_wait0();
  stage_barrier();  // every wave is done with the stage buffers and has published 1/l
  // two staging areas per wave, [32 heads][256 bytes] each (chunk c of head h at c ^ (h >> 1)),
  // taken in turn: a head block's rows are written while the previous block's are stored
  MLA_LDS uint8_t* st2 = vt + wave * 16384;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    MLA_LDS uint8_t* st = st2 + (hb & 1) * 8192;
    const float inv = inv_s[hb * 32 + li];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x16& o = O[cb][hb];
        const bf16x2_t p0 = {(__bf16)(o[4 * r] * inv), (__bf16)(o[4 * r + 1] * inv)};
        const bf16x2_t p1 = {(__bf16)(o[4 * r + 2] * inv), (__bf16)(o[4 * r + 3] * inv)};
        const uint32_t w0 = __builtin_bit_cast(uint32_t, p0), w1 = __builtin_bit_cast(uint32_t, p1);
        *(MLA_LDS u32x2*)(st + li * 256 + (((4 * cb + r) ^ (li >> 1)) << 4) + 8 * lg) = u32x2{w0, w1};
      }
    lgkm_wait0();
    uint16_t* base = full ? a.out + (int64_t)t * a.o_tok + (int64_t)(hb * 32) * a.o_head
                          : a.part_o + ((int64_t)slot * a.H + hb * 32) * kLatentDim;
    const int64_t hstride = full ? a.o_head : kLatentDim;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int hl = 4 * i + (lane >> 4), c = lane & 15;
      const u32x4 w = *(const MLA_LDS u32x4*)(st + hl * 256 + ((c ^ (hl >> 1)) << 4));
      __builtin_nontemporal_store(w, (u32x4*)(base + hl * hstride + 128 * wave + 8 * c));
    }
  }
}

template <int KPAGES, bool ROPE, bool SPARSE>
__global__ __launch_bounds__(256, 1) void mla_fp8mma_kernel(const SparseArgs a, const SplitPlan plan) {
  __shared__ __attribute__((aligned(1024))) uint8_t raw_b[kF8Raw * F8Geo<true>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t vt_b[2 * kF8VBytes];
  __shared__ __attribute__((aligned(256))) uint8_t xbuf_b[2 * kF8PBytes + 1600];
  __shared__ F8Lds L;
  static_assert(2 * kF8VBytes >= 4 * 16384, "epilogue staging");
  plan_run<256, true>(
      plan, L, [&](F8Lds&) {}, [&](int) { return RowGeo{-1, 0, 0}; },
      [&](RowGeo* geo, int lane) {
        if constexpr (SPARSE) sparse_fill_wave<false>(a, geo, lane); else decode_fill_wave(a, geo, lane);
      },
      [&](int r, const RowGeo& g, int ta, int tc, bool full, int slot) {
        fp8mma_segment<KPAGES, ROPE, SPARSE>(a, (MLA_LDS uint8_t*)raw_b, (MLA_LDS uint8_t*)vt_b, (MLA_LDS uint8_t*)xbuf_b, L,
                                     r, g, ta, tc, full, slot);
      });
}

}  // namespace

// The balanced split of at most 64 rows at 128 heads, for the dense fp8 decode and the
// sparse decode without a sink or second stream (see launch_sparse).
hipError_t launch_fp8mma(const SparseArgs& a, const SplitPlan& p, hipStream_t stream) {
  const dim3 grid(a.grid), block(256);
  const bool kp = a.PS % kStageKeys == 0;
  if (!a.dense) {
    if (a.rope) hipLaunchKernelGGL((mla_fp8mma_kernel<0, true, true>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_fp8mma_kernel<0, false, true>), grid, block, 0, stream, a, p);
  } else if (a.rope) {
    if (kp) hipLaunchKernelGGL((mla_fp8mma_kernel<1, true, false>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_fp8mma_kernel<0, true, false>), grid, block, 0, stream, a, p);
  } else {
    if (kp) hipLaunchKernelGGL((mla_fp8mma_kernel<1, false, false>), grid, block, 0, stream, a, p);
    else hipLaunchKernelGGL((mla_fp8mma_kernel<0, false, false>), grid, block, 0, stream, a, p);
  }
  return hipGetLastError();
}

}  // namespace mla
