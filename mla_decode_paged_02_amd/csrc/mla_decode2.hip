// Dense MLA decode for 128 heads with the value columns split over the waves (gfx950).
//
// What is computed follows generic_flare_mla_decode_kv_cache_ragged (summary; Args q,
// input_row_offsets, scale, output; Parameters mask_str, local_window_size): for each query
// row and head, softmax over the visible cache rows of scale * <q, row>, applied to the
// rows' 512 latent columns.  The result is the one mla_decode.hip computes; this kernel
// serves the balanced split of batches of at most 64 rows and sequences.
//
// Per work-group (4 waves, one per SIMD) and 32-key stage:
//   scores    wave w computes S^T = K Q^T for heads 32w..32w+31 over all 576 columns
//             (v_mfma_f32_32x32x16_bf16, 36 k-steps), runs their online softmax and
//             publishes the bf16 weights P in LDS;
//   values    wave w owns the output columns 128w..128w+127 of all 128 heads:
//             O^T += V^T P^T with V^T fragments of its own columns only (a quarter of
//             the stage) and P^T of every head block read back from LDS.
// Step k runs the score MFMAs of stage k while the vector units turn the scores of stage
// k-1 into weights (the matrix cores issue in order with the vector work, so the softmax
// is spread over the 36 k-steps in short independent pieces); after the weights are
// published, the 32 value MFMAs of stage k-1 follow.  Compared with every wave reading
// all 512 value columns, the transposing LDS reads drop four times; the weights cost an
// 8 KB exchange per stage.
//
// Layouts of v_mfma_f32_32x32x16_bf16 (lane l = 32g + i): A[i][8g..8g+7],
// B[8g..8g+7][i], D[8r + 4g + q][i] in register 4r + q.  Score row n of a stage is key n
// of the stage; the value k-step kp then takes keys 16kp + 8(e / 4) + 4g + (e % 4) as its
// k index 8g + e, which is exactly where the score accumulator left them (registers
// 8kp .. 8kp + 7 of lane 32g + i), so P^T needs no shuffle.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_plan.h"
#include "mla_rows.h"
#include "mla_stage.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kD2Bufs = 4;            // stage buffers: values of k-1, scores of k, k+1, k+2
constexpr int kD2PidWindow = 512;     // page ids of the segment held in LDS
constexpr int kD2PBytes = 4 * 2 * 64 * 16;  // weights: [head block][value k-step][lane] x 16 B
constexpr int kD2ABytes = 1536;       // rescale factors [4][32], flags [4], the epilogue's 1/l [128]
constexpr int kD2DmaPerWave = kDmaPerStage / 4;
constexpr int kD2KAhead = 4;         // score fragments read ahead of their MFMA
static_assert(kDmaPerStage % 4 == 0, "every wave issues the same number of stage loads");

struct D2Lds {
  RowGeo geo[256];          // per-wave planning tables (64 rows each)
  int pids[kD2PidWindow];   // page-id window of the segment
};

// LDS tile layout: rows of 72 16-byte chunks; chunk c of row r is stored at c ^ s(r) within
// its aligned group of 8, with s(r) = r4 | r1 << 1 | (r0 ^ r2) << 2 (r_b: bit b of r).  Of
// the 32768 swizzles that are linear in the five row bits, this is one of the few under
// which, timed on MI355X, both the score reads (lane 32g + i: row i, chunk 2ks + g) and the
// transposing value reads of the 32x32x16 operand layout run at the conflict-free rate;
// the bank models tried before did not predict the measured costs, so the choice rests on
// the timing.  Rows 8 apart share s, rows 16 apart differ in bit 0 only.
__device__ __forceinline__ int d2_swz(int r) { return ((r >> 4) & 1) | (((r >> 1) & 1) << 1) | (((r ^ (r >> 2)) & 1) << 2); }

__device__ __forceinline__ void mfma32_a(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Wait states between the last write of a 16-pass MFMA into the accumulation registers
// and other instructions reading them (24, above the 18 the longest such distance needs):
// these MFMAs are inline assembly, which the compiler's hazard tracking does not see.
__device__ __forceinline__ void mfma32_fence_a(f32x16 (&o)[4][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]));
#pragma unroll
  for (int cb = 1; cb < 4; ++cb) asm volatile("" : "+a"(o[cb][0]), "+a"(o[cb][1]), "+a"(o[cb][2]), "+a"(o[cb][3]));
}

template <int KPAGES>
__device__ __forceinline__ void decode2_segment(const DecodeArgs& a, MLA_LDS uint8_t* tiles, MLA_LDS uint8_t* xbuf,
                                                MLA_LDS int* pids, int t, const RowGeo& g, int ta, int tc, bool full,
                                                int slot) {
  constexpr int NT = 256;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 5, li = lane & 31;
  const int h0 = wave * 32;
  MLA_LDS uint8_t* pbuf = xbuf;                                   // weights
  MLA_LDS float* alpha_s = (MLA_LDS float*)(xbuf + kD2PBytes);    // [4][32]
  MLA_LDS int* flag_s = (MLA_LDS int*)(xbuf + kD2PBytes + 512);   // [4]
  MLA_LDS float* inv_s = (MLA_LDS float*)(xbuf + kD2PBytes + 1024);  // [128], after the loop

  const int first_tile = __builtin_amdgcn_readfirstlane(g.lo / kTileKeys);
  const int klo = __builtin_amdgcn_readfirstlane(max(g.lo, (first_tile + ta) * kTileKeys));
  const int khi = __builtin_amdgcn_readfirstlane(min(g.hi, (first_tile + tc) * kTileKeys));
  const int s_first = klo / kStageKeys;
  const int nst = (khi - 1) / kStageKeys - s_first + 1;
  const int32_t* pt = a.page_table + (int64_t)__builtin_amdgcn_readfirstlane(g.b) * a.pt_row;
  const int p_last = (khi - 1) / a.PS;

  // every wave must be done with the buffers and window of anything before
  all_wait0();
  stage_barrier();

  // ---- page-id window [pbase, pbase + kD2PidWindow) (entries past the segment are -1)
  int pbase = klo / a.PS;
  int pv[kD2PidWindow / NT];
  auto window_load = [&]() {
#pragma unroll
    for (int i = 0; i < kD2PidWindow / NT; ++i) {
      const int p = pbase + tid + i * NT;
      pv[i] = p <= p_last ? pt[p] : -1;
    }
  };
  auto window_store = [&]() {
#pragma unroll
    for (int i = 0; i < kD2PidWindow / NT; ++i) pids[tid + i * NT] = pv[i];
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

  // byte offset of this wave's load jj within a block of 32 consecutive cache rows
  auto dma_off = [&](int jj) -> uint32_t {
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
    const int sl = (jj * 4 + wave) * 64 + lane_v;
    const int row = sl / kRowChunks, c = sl - row * kRowChunks;
    return (uint32_t)(row * kRowBytes + ((c & ~7) | ((c ^ d2_swz(row)) & 7)) * 16);
  };

  bool bad_page = false;
  // page of the stage last looked up, its id, and the id of the page after it (read from
  // the window ahead of need, so a page change costs no wait; -1 past the window)
  int lp_last = -1, pid_last = -1, pid_next_v = -1;
  auto stage_page = [&](int st) {
    const int kb0 = st * kStageKeys;  // consecutive stages: the page stays or advances by one
    if (lp_last >= 0 && kb0 >= lp_last * a.PS && kb0 < (lp_last + 1) * a.PS) return pid_last;
    if (lp_last >= 0 && kb0 >= (lp_last + 1) * a.PS && kb0 < (lp_last + 2) * a.PS &&
        lp_last + 1 < pbase + kD2PidWindow) {
      lp_last += 1;
      pid_last = __builtin_amdgcn_readfirstlane(pid_next_v);
    } else {
      const int lp = kb0 / a.PS;
      if (lp >= pbase + kD2PidWindow) window_move(lp);
      lp_last = lp;
      pid_last = __builtin_amdgcn_readfirstlane(pids[lp - pbase]);
    }
    const int nx = lp_last + 1 - pbase;
    pid_next_v = nx < kD2PidWindow ? pids[nx] : -1;
    return pid_last;
  };
  const int npages32 = (int)min(a.num_pages, (int64_t)INT32_MAX);
  auto fast_base = [&](int st, int pa) -> const uint8_t* {
    const int kbase = st * kStageKeys;
    if (KPAGES != 0 && kbase >= klo && kbase + kStageKeys <= khi && pa >= 0 && pa < npages32)
      return a.cache + (int64_t)pa * a.page_bytes + (int64_t)((uint32_t)kbase % (uint32_t)a.PS) * kRowBytes;
    return nullptr;
  };
  // this lane's byte offset of each of its stage loads (the same for every stage)
  uint32_t doff[kD2DmaPerWave];
#pragma unroll
  for (int jj = 0; jj < kD2DmaPerWave; ++jj) doff[jj] = dma_off(jj);
  auto fast_load = [&](const uint8_t* base, MLA_LDS uint8_t* dst, int jj) {
    dma16_base_nt(base, doff[jj], dst + (jj * 4 + wave) * 1024);
  };
  auto issue_general = [&](int st, int bi, int pa) {
    MLA_LDS uint8_t* dst = tiles + bi * kStageBytes;
    const int kbase = st * kStageKeys;
    const int lpa = kbase / a.PS;
    if (KPAGES == 0) {
      const int lp_hi = (min(kbase + kStageKeys, khi) - 1) / a.PS;
      if (lp_hi >= pbase + kD2PidWindow) window_move(max(kbase, klo) / a.PS);
    }
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
#pragma unroll
    for (int jj = 0; jj < kD2DmaPerWave; ++jj) {
      const int J = jj * 4 + wave;
      const int sl = J * 64 + lane_v;
      const int row = sl / kRowChunks, c = sl - row * kRowChunks;
      const int cg = (c & ~7) | ((c ^ d2_swz(row)) & 7);
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
#pragma unroll
    for (int jj = 0; jj < kD2DmaPerWave; ++jj) fast_load(fb, tiles + bi * kStageBytes, jj);
  };

  // ---- query fragments (B operand of S^T = K Q^T): lane 32g+i holds q[head h0 + i]
  // [16ks + 8g .. + 8]; all ordinary loads land before the stage loop (the stage loads are
  // outside the compiler's wait bookkeeping)
  bf16x8 qf[36];
  {
    const uint16_t* qh = a.q + (int64_t)t * a.q_tok + (int64_t)(h0 + li) * a.q_head + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qf[ks] = *(const bf16x8*)(qh + 16 * ks);
  }

  // ---- prologue: stages 0 and 1 (their page ids by scalar loads, which the full wait
  // covers) and the window for the loop
  auto direct_page = [&](int st) { return ld_const(pt + st * kStageKeys / a.PS); };
  const int pa0 = KPAGES != 0 ? direct_page(s_first) : 0;
  const int pa1 = (KPAGES != 0 && nst > 1) ? direct_page(s_first + 1) : 0;
  int pa_n = (KPAGES != 0 && nst > 2) ? direct_page(s_first + 2) : 0;
  issue(s_first, 0, pa0);
  if (nst > 1) issue(s_first + 1, 1, pa1);
  if (KPAGES != 0) window_load();
  {
    // the values of "stage -1" (zero weights) read the buffer stage 3 will use: zeros
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    MLA_LDS uint8_t* z = tiles + (kD2Bufs - 1) * kStageBytes;
    for (int i = tid; i < kStageBytes / 16; i += NT) *(MLA_LDS u32x4*)(z + 16 * i) = u32x4{0, 0, 0, 0};
  }
  all_wait0();
  if (KPAGES != 0) {
    window_store();
  }
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

  // per-lane LDS offsets: score read of k-step 4j + n at kb[n] + 128 j
  int kb[4];
  {
    const int sw = d2_swz(li);
#pragma unroll
    for (int n = 0; n < 4; ++n) kb[n] = li * kRowBytes + (((2 * n + lg) ^ sw) << 4);
  }
  // Transposing value reads: lane 16G + 4r + q (G = 2g + c) reads row 16kp + 8h + 4g + r,
  // 16-byte chunk 16w + 4cb + 2c + (q >> 1).  Rows 16kp + 8h + (4g + r) differ from 4g + r
  // only in bits 3 and 4, which flip swizzle bit 0 by kp and nothing by h: four per-lane
  // bases cover every read, at vb[kp][cb & 1] + (16kp + 8h) * 1152 + 128 * (cb >> 1).
  int vb[2][2];
  {
    const int G = lane >> 4, gg = G >> 1, c = G & 1, r = (lane >> 2) & 3, q = lane & 3;
    const int brow = 4 * gg + r;
    const int X = (2 * c + (q >> 1)) ^ d2_swz(brow);
    const int base = brow * kRowBytes + 256 * wave + 8 * (q & 1);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) vb[kp][pp] = base + ((X ^ kp ^ (4 * pp)) << 4);
  }

  // Step k scores stage k while the vector units turn the scores of stage k-1 into
  // weights; once every wave has published its weights, it adds the values of stage k-1.
  // Every step runs the whole stream, so it has no branch: at k = 0 no key of "stage -1"
  // is valid (zero weights on the zero-filled buffer), and at k = nst the scores of a
  // stale buffer are computed and dropped.
  f32x16 Sp;  // raw scores of stage k-1
#pragma unroll
  for (int e = 0; e < 16; ++e) Sp[e] = 0.f;
#pragma unroll 1
  for (int k = 0; k <= nst; ++k) {
    // ---- stage k has landed (stage k+1 may still be in flight)
    if (k < nst) {
      if (k >= 1 && k + 1 < nst) vm_wait_imm<kD2DmaPerWave>(); else vm_wait_imm<0>();
    }
    stage_barrier();  // also: every wave is done with the values of stage k-2
    // ---- stage k+2 into the buffer of stage k-2: a stage in one valid page from a scalar
    // base spread over the MFMA stream, any other here
    const int kn = k + 2;
    const uint8_t* fb = nullptr;
    MLA_LDS uint8_t* fdst = tiles + (kn % kD2Bufs) * kStageBytes;
    if (kn < nst) {
      fb = fast_base(s_first + kn, pa_n);
      if (fb == nullptr) issue_general(s_first + kn, kn % kD2Bufs, pa_n);
      if (KPAGES != 0 && kn + 1 < nst) pa_n = stage_page(s_first + kn + 1);
    }

    // per-lane LDS addresses of this step's buffers
    const int bs_off = (k % kD2Bufs) * kStageBytes, bv_off = ((k + kD2Bufs - 1) % kD2Bufs) * kStageBytes;
    int kbs[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) kbs[n] = kb[n] + bs_off;
    int vbs[2][2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) vbs[kp][pp] = vb[kp][pp] + bv_off;
    auto kread = [&](int ks) { return *(const MLA_LDS bf16x8*)(tiles + kbs[ks & 3] + 128 * (ks >> 2)); };
    auto vread = [&](int kp, int cb) {
      const int o0 = 1152 * 16 * kp + 128 * (cb >> 1), o1 = o0 + 1152 * 8;
      const bf16x4 a0 = ds_read_tr16(tiles + vbs[kp][cb & 1] + o0);
      const bf16x4 a1 = ds_read_tr16(tiles + vbs[kp][cb & 1] + o1);
      return bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    };
    auto pread = [&](int hb, int kp) { return *(const MLA_LDS bf16x8*)(pbuf + lane * 16 + hb * 2048 + kp * 1024); };

    // ---- phase A: the 36 score k-steps of stage k on the matrix cores, the online softmax
    // of stage k-1 for heads h0 + i (lanes i and 32 + i: keys 8r + 4g + q of register
    // 4r + q) on the vector units, and the stage loads of stage k+2.  The matrix cores
    // issue in order with the vector work, so each k-step carries only a few independent
    // vector operations: the softmax is spread over the k-steps as a pipeline.
    f32x16 S;
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
    {
      // keys outside the segment (only in its first and last stage, and all of "stage -1")
      // get -inf after scaling; the pipeline then scales by 1
      const uint32_t valid = k == 0 ? 0u : range_bits((s_first + k - 1) * kStageKeys, klo, khi);
      float slx = a.scale_log2;
      if (valid != 0xFFFFFFFFu) {
        const uint32_t vbits = valid >> (4 * lg);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 8 * (e >> 2) + (e & 3);  // minus 4g, folded into vbits
          Sp[e] = ((vbits >> row) & 1u) ? Sp[e] * a.scale_log2 : -INFINITY;
        }
        slx = 1.f;
      }
      float x[16];
      float lmax = -INFINITY, mx = 0.f, m_new = 0.f, ex = 0.f, mref = 0.f;
      uint32_t hsw0 = 0, hsw1 = 0;
      uint64_t rf = 0;
      // pin(v): v is materialised here; with a pin on its inputs before and on its result
      // after, a computation stays in its k-step (the scheduler fences order the pins)
      auto pin = [](float& v) { asm volatile("" : "+v"(v)); };
      auto pinu = [](uint32_t& v) { asm volatile("" : "+v"(v)); };
      bf16x8 kf[36];  // fully unrolled: at most kD2KAhead + 1 live
#pragma unroll
      for (int i = 0; i < kD2KAhead; ++i) kf[i] = kread(i);
#pragma unroll
      for (int i = 0; i < 36; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + kD2KAhead < 36) kf[i + kD2KAhead] = kread(i + kD2KAhead);
        // scale (k-steps 0..7), running maximum (1..8)
        if (i < 8) {
          float s0 = Sp[2 * i], s1 = Sp[2 * i + 1];
          pin(s0);
          pin(s1);
          x[2 * i] = s0 * slx;
          x[2 * i + 1] = s1 * slx;
          pin(x[2 * i]);
          pin(x[2 * i + 1]);
        }
        if (i >= 1 && i <= 8) {
          pin(lmax);
          lmax = fmaxf(lmax, fmaxf(x[2 * i - 2], x[2 * i - 1]));
          pin(lmax);
        }
        // the head's maximum over both lane halves and a lazy rescale once it has grown by
        // more than the slack (the same decision in both lanes of a head); m_new != m is
        // that decision
        if (i == 9) {
          pin(lmax);
          const uint32_t b = __builtin_bit_cast(uint32_t, lmax);
          const auto hsw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
          hsw0 = (uint32_t)hsw[0];
          hsw1 = (uint32_t)hsw[1];
          pinu(hsw0);
          pinu(hsw1);
        }
        if (i == 10) {
          mx = fmaxf(__builtin_bit_cast(float, hsw0), __builtin_bit_cast(float, hsw1));
          pin(mx);
        }
        if (i == 11) {
          pin(m);
          m_new = mx > m + kRescaleSlack ? mx : m;
          pin(m_new);
        }
        if (i == 12) {
          ex = fast_exp2(m - m_new);  // 0 while m is -inf; unused unless m_new != m
          // O is exactly zero while m is -inf: only a finite old maximum needs the rescale
          rf = __builtin_amdgcn_ballot_w64(m_new != m && m != -INFINITY);
          pin(ex);
        }
        if (i == 13) {
          alpha = m_new != m ? ex : 1.f;
          m = m_new;
          mref = m == -INFINITY ? 0.f : m;
          pin(alpha);
          pin(mref);
        }
        if (i == 14) {
          pin(l);
          l *= alpha;
          pin(l);
          rflag = rf != 0 ? 1 : 0;
        }
        // weights, pair p: difference (k-step 14 + p), power (15 + p), rounding (16 + p),
        // and the denominator, which sums the weights as rounded for the MFMA (17 + p)
        if (i >= 14 && i < 22) {
          const int e = 2 * (i - 14);
          x[e] -= mref;
          x[e + 1] -= mref;
          pin(x[e]);
          pin(x[e + 1]);
        }
        if (i >= 15 && i < 23) {
          const int e = 2 * (i - 15);
          x[e] = fast_exp2(x[e]);
          x[e + 1] = fast_exp2(x[e + 1]);
          pin(x[e]);
          pin(x[e + 1]);
        }
        if (i >= 16 && i < 24) {
          const int e = 2 * (i - 16);
          const bf16x2_t pp = {(__bf16)x[e], (__bf16)x[e + 1]};
          pk[e >> 1] = __builtin_bit_cast(uint32_t, pp);
          pinu(pk[e >> 1]);
        }
        if (i >= 17 && i < 25) {
          const int e = 2 * (i - 17);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[e >> 1]), one, l, false);
          pin(l);
        }
        // the compiler's own MFMA: it may move S between registers, and then it knows
        // the wait states a copy of an MFMA result needs
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i], i == 0 ? f32x16{} : S, 0, 0, 0);
        if ((i & 3) == 2 && i / 4 < kD2DmaPerWave) {
          if (fb != nullptr) fast_load(fb, fdst, i / 4);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- publish the weights, rescale factor and flag of stage k-1 (own head block)
    {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      *(MLA_LDS u32x4*)(pbuf + wave * 2048 + lane * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      *(MLA_LDS u32x4*)(pbuf + wave * 2048 + 1024 + lane * 16) = u32x4{pk[4], pk[5], pk[6], pk[7]};
      if (lg == 0) alpha_s[wave * 32 + li] = alpha;
      if (lane == 0) flag_s[wave] = rflag;
    }
    bf16x8 vf[8];  // V^T fragment 4kp + cb; at most two live
    vf[0] = vread(0, 0);
    lgkm_wait0();
    stage_barrier();
    bf16x8 pf0[4], pf1[4];  // P^T (kp, hb)
    {
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      const i32x4 fl = *(const MLA_LDS i32x4*)flag_s;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pf0[hb] = pread(hb, 0);
      // O holds the values of stages < k-1 relative to the maxima before stage k-1: bring
      // the rescaled heads to their new maxima before stage k-1's values are added
      if ((fl[0] | fl[1] | fl[2] | fl[3]) != 0) {
        mfma32_fence_a(O);
        // one tile at a time through ordinary registers: each step is tied to the next
        // tile so the compiler cannot lift all the reads ahead
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const float al = fl[hb] != 0 ? alpha_s[hb * 32 + li] : 1.f;
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

    // ---- phase B: the values of stage k-1, op j = 16kp + 4cb + hb
    {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        const int kp = j >> 4, cb = (j >> 2) & 3, hb = j & 3;
        // the next V^T fragment, one column block ahead
        if (hb == 0 && j + 4 < 32) vf[(j >> 2) + 1] = vread((j + 4) >> 4, ((j + 4) >> 2) & 3);
        mfma32_a(O[cb][hb], vf[4 * kp + cb], kp == 0 ? pf0[hb] : pf1[hb]);
        // kp = 1's weights once kp = 0 is done with each register
        if (j >= 12 && j < 16) pf1[j - 12] = pread(j - 12, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    Sp = S;
  }

  if (bad_page) atomicOr(a.err, kErrPageId);

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
  mfma32_fence_a(O);
  lgkm_wait0();
  stage_barrier();  // every wave is done with the stage buffers and has published 1/l
  // two staging areas per wave, [32 heads][256 bytes] each (chunk c of head h at c ^ (h >> 1)),
  // taken in turn: a head block's rows are written while the previous block's are stored
  MLA_LDS uint8_t* st2 = tiles + wave * 16384;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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

template <int KPAGES>
__global__ __launch_bounds__(256, 1) void mla_decode2_kernel(const DecodeArgs a, const SplitPlan plan) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles_raw[kD2Bufs * kStageBytes];
  __shared__ __attribute__((aligned(256))) uint8_t xbuf_raw[kD2PBytes + kD2ABytes];
  __shared__ D2Lds L;
  static_assert(kD2Bufs * kStageBytes >= 4 * 16384, "epilogue staging");
  MLA_LDS uint8_t* tiles = (MLA_LDS uint8_t*)tiles_raw;
  MLA_LDS uint8_t* xbuf = (MLA_LDS uint8_t*)xbuf_raw;
  plan_run<256, true>(
      plan, L, [&](D2Lds&) {}, [&](int) { return RowGeo{-1, 0, 0}; },
      [&](RowGeo* geo, int lane) { decode_fill_wave(a, geo, lane); },
      [&](int r, const RowGeo& g, int ta, int tc, bool full, int slot) {
        decode2_segment<KPAGES>(a, tiles, xbuf, (MLA_LDS int*)L.pids, r, g, ta, tc, full, slot);
      });
}

}  // namespace

// The balanced split of at most 64 rows and sequences at 128 heads (see launch_decode).
hipError_t launch_decode2(const DecodeArgs& a, const SplitPlan& p, hipStream_t stream) {
  const dim3 grid(a.grid), block(256);
  if (a.PS % kStageKeys == 0) hipLaunchKernelGGL(mla_decode2_kernel<1>, grid, block, 0, stream, a, p);
  else hipLaunchKernelGGL(mla_decode2_kernel<0>, grid, block, 0, stream, a, p);
  return hipGetLastError();
}

}  // namespace mla
