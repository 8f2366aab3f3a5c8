// Ragged MLA prefill with per-head keys (gfx950).
//
// What is computed follows generic_flare_mla_prefill_kv_cache_ragged (summary; Args q, k,
// v, buffer_row_offsets, cache_offsets, input_row_offsets, scale, output): for query row
// t of sequence b and head h, softmax over the sequence's keys i of scale * <q[t,h,:],
// K_i>, with K_i = [k[row_i, h, 0:128] | the rope columns 512..575 of the latent cache row
// at cache position cache_offsets[b] + i] (the rope is shared by all heads), applied to
// v[row_i, h, :].  Query t sits at cache position cache_lens[b] - n_b + t; under the
// causal mask it sees the keys at positions up to its own.
//
// Work-group = (sequence, head, block of 128 queries): four waves of 32 queries.  Keys
// stream through LDS in stages of 32 (no-rope K tile 32 x 128, rope tile 32 x 64, V tile
// 32 x 128, triple buffered) by direct global->LDS loads: each lane's source offset within
// a stage is fixed, so a stage whose keys all count and whose rope rows lie in one page
// costs one scalar base per tensor and five load instructions per wave.  Per wave and
// stage, as in the decode kernels, S^T = K Q^T with the key rows of each MFMA tile permuted
// so the score accumulators are already the P^T operand, an online softmax per query, then
// O^T += V^T P^T with transposing LDS reads.
#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_stage.h"

namespace mla {

constexpr int kPfQ = 128;                    // queries per work-group
constexpr int kPfWaves = 4;                  // 32 queries per wave
constexpr int kPfNT = kPfWaves * 64;
constexpr int kPfKnRow = 256;                // bytes per key row: 128 no-rope columns
constexpr int kPfKrRow = 128;                //                    64 rope columns
constexpr int kPfVRow = 256;                 //                    128 value columns
constexpr int kPfKnStage = kStageKeys * kPfKnRow;
constexpr int kPfKrStage = kStageKeys * kPfKrRow;
constexpr int kPfVStage = kStageKeys * kPfVRow;
constexpr int kPfStage = kPfKnStage + kPfKrStage + kPfVStage;  // 20 KB: [K no-rope | K rope | V]
constexpr int kPfBufs = 3;
constexpr int kPfDma = kPfStage / 1024;      // 20 wave-wide loads per stage
constexpr int kPfDmaPerWave = kPfDma / kPfWaves;
constexpr int kPfPidWindow = 256;            // page ids of the work-group's keys held in LDS
static_assert(kPfDma % kPfWaves == 0 && kPfDmaPerWave == 5, "load slots dealt evenly");

// LDS swizzles: chunk c of row r at position c ^ f(r).  Rows of 256 bytes start on the same
// bank, so the 16 rows of a score read need 16 different 16-byte positions (f over four
// bits); rope rows of 128 bytes alternate bank halves (three bits suffice); the value read
// takes 32-byte chunk pairs of 8 rows, so f keeps pairs together (even values).
__device__ __forceinline__ int pf_kn_swz(int r) { return (((r >> 3) & 3) << 2) | (r & 3); }
__device__ __forceinline__ int pf_kr_swz(int r) { return (((r >> 3) & 3) << 1) | ((r >> 1) & 1); }
__device__ __forceinline__ int pf_v_swz(int r) { return ((((r >> 3) & 1) << 2) | (r & 3)) << 1; }

struct PfAcc {
  f32x4 o[8][2];  // lane 16g+n: O^T[16cb + 4g + i][query 16qb + n of the wave]
  float m[2], l[2];
};

// Sequence and query block of work item j (blocks numbered in sequence order).  Returns
// false when j is past the last block.
__device__ __forceinline__ bool pf_locate(const PrefillArgs& a, int j, int& b, int& qb) {
  int base = 0;
  for (int s = 0; s < a.B; ++s) {
    const int n = (int)ld_const(a.in_off + s + 1) - (int)ld_const(a.in_off + s);
    const int nb = n > 0 ? (n + kPfQ - 1) / kPfQ : 0;
    if (j < base + nb) {
      b = s;
      qb = j - base;
      return true;
    }
    base += nb;
  }
  return false;
}

__global__ __launch_bounds__(kPfNT, 2) void mla_prefill_kernel(const PrefillArgs a, int total_blocks) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles_raw[kPfBufs * kPfStage];
  __shared__ int pids[kPfPidWindow];
  MLA_LDS uint8_t* tiles = (MLA_LDS uint8_t*)tiles_raw;

  // longest work first: the last query blocks (most keys under the causal mask) go out first
  const int w = blockIdx.x;
  const int h = w % a.H;
  const int j = total_blocks - 1 - w / a.H;
  int b, qb;
  if (j < 0 || !pf_locate(a, j, b, qb)) return;
  b = __builtin_amdgcn_readfirstlane(b);
  qb = __builtin_amdgcn_readfirstlane(qb);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, ln = lane & 15;

  const int in0 = (int)ld_const(a.in_off + b), in1 = (int)ld_const(a.in_off + b + 1);
  const int bo0 = (int)ld_const(a.buf_off + b), bo1 = (int)ld_const(a.buf_off + b + 1);
  const int n = in1 - in0, nk = bo1 - bo0;
  const long long co = ld_const(a.cache_off + b);
  const long long L = ld_const(a.cache_lens + b);
  if (nk < 0 || bo0 < 0 || bo1 > a.Tk || n < 0 || in1 > a.Tq) {
    if (tid == 0) atomicOr(a.err, kErrOffsets);
    return;
  }
  const int t0 = qb * kPfQ;                      // first query of the block (local index)
  const int tw = t0 + wave * 32;                 // first query of this wave
  const long long pos0 = L - n;                  // position of local query 0
  // keys [0, key_end) can be visible to some query of the block
  int key_end = nk;
  if (a.mask == kMaskCausal) {
    const long long last = pos0 + min(t0 + kPfQ, n) - 1 - co + 1;
    key_end = (int)max(0LL, min((long long)nk, last));
  }
  const int nst = (key_end + kStageKeys - 1) / kStageKeys;
  const int32_t* pt = a.page_table + (int64_t)b * a.pt_row;

  // ---- page ids of the rope rows: logical pages [lp0, lp0 + kPfPidWindow) in LDS
  const long long lp0 = co / a.PS;
  const long long lp_end = key_end > 0 ? (co + key_end - 1) / a.PS + 1 : lp0;
  for (int i = tid; i < kPfPidWindow; i += kPfNT) {
    const long long lp = lp0 + i;
    pids[i] = lp < lp_end && lp < a.max_pages ? pt[lp] : -1;
  }

  // ---- stage loads.  Wave w takes load slots w + 4i (i = 0..4) of the stage's 20: slots
  // 0..7 the no-rope K rows (4 rows per 1 KB), 8..11 the rope rows (8 per 1 KB), 12..19
  // the V rows; the slot's 1 KB lands at offset 1024 * slot of the stage buffer.
  const int64_t kb = a.k_tok * 2, vb = a.v_tok * 2;   // bytes between key rows
  const uint8_t* kbase = (const uint8_t*)a.k + ((int64_t)bo0 * a.k_tok + (int64_t)h * a.k_head) * 2;
  const uint8_t* vbase = (const uint8_t*)a.v + ((int64_t)bo0 * a.v_tok + (int64_t)h * a.v_head) * 2;
  // row and logical 16-byte chunk of this lane's piece in load i
  auto slot_piece = [&](int i, int lane_v, int& row, int& c) {
    const int G = wave + kPfWaves * i;
    if (i < 2) {
      row = 4 * G + (lane_v >> 4);
      c = (lane_v & 15) ^ pf_kn_swz(row);
    } else if (i == 2) {
      row = 8 * (G - 8) + (lane_v >> 3);
      c = (lane_v & 7) ^ pf_kr_swz(row);
    } else {
      row = 4 * (G - 12) + (lane_v >> 4);
      c = (lane_v & 15) ^ pf_v_swz(row);
    }
  };
  // fixed per-lane source offsets (fast stages): rows relative to the stage's first key
  const bool fast_strides = kb * kStageKeys < (1ll << 31) && vb * kStageKeys < (1ll << 31);
  uint32_t doff[kPfDmaPerWave];
#pragma unroll
  for (int i = 0; i < kPfDmaPerWave; ++i) {
    int row, c;
    slot_piece(i, lane, row, c);
    doff[i] = i < 2 ? (uint32_t)(row * kb + c * 16)
                    : i == 2 ? (uint32_t)(row * kRowBytes + kLatentDim * 2 + c * 16) : (uint32_t)(row * vb + c * 16);
  }
  bool bad = false;
  // page and slot of the first rope row of the next stage to issue (stages are issued in
  // order), advanced by 32 positions per stage without a division
  long long nx_lp = lp0;
  int nx_slot = (int)(co - lp0 * a.PS);
  // the next stage's first K and V rows, advanced by 32 rows per stage
  const uint8_t* nx_k = kbase;
  const uint8_t* nx_v = vbase;
  auto issue = [&](int st, int buf) {
    MLA_LDS uint8_t* dst = tiles + buf * kPfStage;
    const int key0 = st * kStageKeys;
    // the stage's rope rows in one valid page?
    const long long lp = nx_lp;
    const int slot0 = nx_slot;
    nx_slot += kStageKeys;
    while (nx_slot >= a.PS) {
      nx_slot -= a.PS;
      ++nx_lp;
    }
    const uint8_t* kst = nx_k;
    const uint8_t* vst = nx_v;
    nx_k += kb * kStageKeys;
    nx_v += vb * kStageKeys;
    int pid = -1;
    if (lp - lp0 < kPfPidWindow) pid = __builtin_amdgcn_readfirstlane(pids[lp - lp0]);
    const bool fast = fast_strides && key0 + kStageKeys <= key_end && slot0 + kStageKeys <= a.PS && pid >= 0 &&
                      (int64_t)pid < a.num_pages;
    if (fast) {
      const uint8_t* rst = a.cache + (int64_t)pid * a.page_bytes + (int64_t)slot0 * kRowBytes;
#pragma unroll
      for (int i = 0; i < kPfDmaPerWave; ++i)
        dma16_base(i < 2 ? kst : i == 2 ? rst : vst, doff[i], dst + (wave + kPfWaves * i) * 1024);
      return;
    }
    // general stage: per-lane keys, pages and bounds (keys past the visible range and rows
    // of invalid pages read the zero row)
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
#pragma unroll
    for (int i = 0; i < kPfDmaPerWave; ++i) {
      int row, c;
      slot_piece(i, lane_v, row, c);
      const int key = key0 + row;
      const uint8_t* src = a.zero_row + c * 16;
      if (key < key_end) {
        if (i < 2) {
          src = kbase + (int64_t)key * kb + c * 16;
        } else if (i == 2) {
          const long long pos = co + key;
          const long long lpk = pos / a.PS;
          const int pk = lpk - lp0 < kPfPidWindow ? pids[lpk - lp0] : (lpk < a.max_pages ? pt[lpk] : -1);
          if (pk >= 0 && (int64_t)pk < a.num_pages)
            src = a.cache + (int64_t)pk * a.page_bytes + (pos - lpk * a.PS) * kRowBytes + kLatentDim * 2 + c * 16;
          else
            bad = true;
        } else {
          src = vbase + (int64_t)key * vb + c * 16;
        }
      }
      dma16(src, dst + (wave + kPfWaves * i) * 1024);
    }
  };

  // ---- query fragments (B operand of S^T = K Q^T): lane holds q[query][32ks + 8gq .. +8]
  bf16x8 qf[2][6];
#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) {
    const int t = tw + 16 * qb2 + ln;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      qf[qb2][ks] = t < n ? *(const bf16x8*)(a.q + (int64_t)(in0 + t) * a.q_tok + (int64_t)h * a.q_head + 32 * ks + 8 * gq)
                          : bf16x8{};
    }
  }
  // the window is complete before the first stage reads it; all ordinary loads have
  // landed before the stage loads start (their waits are the kernel's own)
  all_wait0();
  __syncthreads();
  if (nst > 0) issue(0, 0);
  if (nst > 1) issue(1, 1);

  PfAcc acc;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) acc.o[cb][0] = acc.o[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc.m[0] = acc.m[1] = -INFINITY;
  acc.l[0] = acc.l[1] = 0.f;

  // per-lane operand geometry (as in the decode kernels)
  const int rowA0 = 8 * (ln >> 2) + (ln & 3), rowA1 = rowA0 + 4;
  const int vr = ln >> 2, vq = lane & 3;
  const int rowV0 = 8 * gq + vr, rowV1 = rowV0 + 4;
  const int vhalf = (vq & 1) * 8;
  // positions of this lane's two queries relative to the cache offset of key 0, clamped
  // so that the per-stage mask arithmetic stays in 32 bits (keys are below 2^24)
  auto rel = [&](long long t) { return (int)max(-(1ll << 30), min(1ll << 30, pos0 + t - co)); };
  int qrel[2];
#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) qrel[qb2] = rel(tw + 16 * qb2 + ln);
  const int wave_q0 = rel(tw);  // relative position of the wave's first query

#pragma unroll 1
  for (int st = 0; st < nst; ++st) {
    // stage st has landed (st+1 may be in flight); every wave is past stage st-1, whose
    // buffer takes stage st+2
    if (st + 1 < nst) vm_wait_imm<kPfDmaPerWave>(); else vm_wait_imm<0>();
    stage_barrier();
    if (st + 2 < nst) issue(st + 2, (st + 2) % kPfBufs);
    const MLA_LDS uint8_t* Kn = tiles + (st % kPfBufs) * kPfStage;
    const MLA_LDS uint8_t* Kr = Kn + kPfKnStage;
    const MLA_LDS uint8_t* V = Kr + kPfKrStage;
    const int kbase_st = st * kStageKeys;

    // S^T = K Q^T: key tiles u = 0, 1 x query blocks (k-steps 0..3 no-rope, 4..5 rope)
    f32x4 s[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) s[u][0] = s[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      bf16x8 k0, k1;
      if (ks < 4) {
        const int c = 4 * ks + gq;
        k0 = *(const MLA_LDS bf16x8*)(Kn + rowA0 * kPfKnRow + (c ^ pf_kn_swz(rowA0)) * 16);
        k1 = *(const MLA_LDS bf16x8*)(Kn + rowA1 * kPfKnRow + (c ^ pf_kn_swz(rowA1)) * 16);
      } else {
        const int c = 4 * (ks - 4) + gq;
        k0 = *(const MLA_LDS bf16x8*)(Kr + rowA0 * kPfKrRow + (c ^ pf_kr_swz(rowA0)) * 16);
        k1 = *(const MLA_LDS bf16x8*)(Kr + rowA1 * kPfKrRow + (c ^ pf_kr_swz(rowA1)) * 16);
      }
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        s[0][qb2] = mfma16x16x32(k0, qf[qb2][ks], s[0][qb2]);
        s[1][qb2] = mfma16x16x32(k1, qf[qb2][ks], s[1][qb2]);
      }
    }

    // masks: key kbase_st + 8gq + j (this lane's keys) against the end of the keys and,
    // under the causal mask, against this lane's query position
    const uint32_t stage_bits = range_bits(kbase_st, 0, key_end);
    const bool all_valid = stage_bits == 0xFFFFFFFFu && (a.mask != kMaskCausal || kbase_st + kStageKeys - 1 <= wave_q0);
    const float ks8[2][4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
    bf16x8 pf[2];
#pragma unroll
    for (int qb2 = 0; qb2 < 2; ++qb2) {
      uint32_t bits = (stage_bits >> (8 * gq)) & 0xFFu;
      if (a.mask == kMaskCausal) {
        const int lim = qrel[qb2] - (kbase_st + 8 * gq) + 1;  // keys j < lim are visible
        const uint32_t cbits = lim <= 0 ? 0u : (lim >= 8 ? 0xFFu : ((1u << lim) - 1u));
        bits &= cbits;
      }
      pf[qb2] = softmax_block<false>(s[0][qb2], s[1][qb2], bits, all_valid, a.scale_log2, ks8, acc.m[qb2],
                                     acc.l[qb2], [&](float alpha) {
#pragma unroll
                                       for (int cb = 0; cb < 8; ++cb) acc.o[cb][qb2] *= alpha;
                                     });
    }

    // O^T += V^T P^T
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int c = 2 * cb + (vq >> 1);
      const bf16x4 a0 = ds_read_tr16(V + rowV0 * kPfVRow + (c ^ pf_v_swz(rowV0)) * 16 + vhalf);
      const bf16x4 a1 = ds_read_tr16(V + rowV1 * kPfVRow + (c ^ pf_v_swz(rowV1)) * 16 + vhalf);
      const bf16x8 vf = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) acc.o[cb][qb2] = mfma16x16x32(vf, pf[qb2], acc.o[cb][qb2]);
    }
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(a.err, kErrPageId);

  // ---- epilogue: out[in0 + t][h][16cb + 4gq + i] = O^T / l (rows with no key: 0)
#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) {
    const float l_tot = wave_sum_xor16_32(acc.l[qb2]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int t = tw + 16 * qb2 + ln;
    if (t < n) {
      uint16_t* orow = a.out + (int64_t)(in0 + t) * a.o_tok + (int64_t)h * a.o_head + 4 * gq;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const f32x4 o = acc.o[cb][qb2];
        const uint32_t lo = (uint32_t)bf16_bits_rne(o[0] * inv) | ((uint32_t)bf16_bits_rne(o[1] * inv) << 16);
        const uint32_t hi = (uint32_t)bf16_bits_rne(o[2] * inv) | ((uint32_t)bf16_bits_rne(o[3] * inv) << 16);
        *(uint2*)(orow + 16 * cb) = make_uint2(lo, hi);
      }
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream, const KernelTimer* timer) {
  // an upper bound of the query blocks: every sequence adds at most one partial block
  const int total_blocks = (a.Tq + kPfQ - 1) / kPfQ + a.B;
  hipError_t e;
  if (timer && (e = hipEventRecord(timer->start, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(mla_prefill_kernel, dim3(total_blocks * a.H), dim3(kPfNT), 0, stream, a, total_blocks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (timer && (e = hipEventRecord(timer->stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
