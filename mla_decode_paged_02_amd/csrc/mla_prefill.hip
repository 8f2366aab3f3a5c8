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
// stream through LDS in stages of 32 (K tile 32 x 192, V tile 32 x 128, double buffered,
// the next stage prefetched into registers while the current one is computed).  Per
// wave and stage, as in the decode kernels, S^T = K Q^T with the key rows of each MFMA
// tile permuted so the score accumulators are already the P^T operand, an online softmax
// per query, then O^T += V^T P^T with transposing LDS reads.
#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_stage.h"

namespace mla {

constexpr int kPfQ = 128;                    // queries per work-group
constexpr int kPfWaves = 4;                  // 32 queries per wave
constexpr int kPfNT = kPfWaves * 64;
constexpr int kPfQkDim = 192, kPfVDim = 128;
constexpr int kPfKRow = kPfQkDim * 2;        // 384 bytes: 16 no-rope chunks + 8 rope chunks
constexpr int kPfVRow = kPfVDim * 2;         // 256 bytes
constexpr int kPfKStage = kStageKeys * kPfKRow;
constexpr int kPfVStage = kStageKeys * kPfVRow;
constexpr int kPfPieces = (kPfKStage + kPfVStage) / 16;   // 1280 sixteen-byte pieces per stage
constexpr int kPfPerThread = kPfPieces / kPfNT;           // 5
static_assert(kPfPieces % kPfNT == 0, "pieces are dealt evenly");

// LDS swizzles (chunk c of row r at position c ^ f(r), an involution within aligned
// groups of 8 (K) or 16 (V) chunks) chosen so the 16 lanes of an MFMA operand read hit
// distinct banks.
__device__ __forceinline__ int pf_kswz(int r) { return ((r >> 1) & 1) | (((r >> 3) & 3) << 1); }
__device__ __forceinline__ int pf_vswz(int r) { return (r & 3) << 1; }

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
  __shared__ __attribute__((aligned(1024))) uint8_t kt_raw[2 * kPfKStage];
  __shared__ __attribute__((aligned(1024))) uint8_t vt_raw[2 * kPfVStage];
  MLA_LDS uint8_t* kt = (MLA_LDS uint8_t*)kt_raw;
  MLA_LDS uint8_t* vt = (MLA_LDS uint8_t*)vt_raw;

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

  // ---- stage loads: 5 sixteen-byte pieces per thread, staged in registers
  bool bad = false;
  uint4 stg[kPfPerThread];
  auto fetch = [&](int st) {
#pragma unroll
    for (int i = 0; i < kPfPerThread; ++i) {
      const int c = tid + i * kPfNT;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < 512) {  // no-rope key columns
        const int row = c >> 4, part = c & 15, key = st * kStageKeys + row;
        if (key < key_end)
          v = *(const uint4*)(a.k + (int64_t)(bo0 + key) * a.k_tok + (int64_t)h * a.k_head + part * 8);
      } else if (c < 768) {  // rope columns of the key's latent cache row
        const int cc = c - 512, row = cc >> 3, part = cc & 7, key = st * kStageKeys + row;
        if (key < key_end) {
          const long long pos = co + key;
          const long long lp = pos / a.PS;
          const int pid = lp < a.max_pages ? pt[lp] : -1;
          if (pid >= 0 && (int64_t)pid < a.num_pages)
            v = *(const uint4*)(a.cache + (int64_t)pid * a.page_bytes + (pos - lp * a.PS) * kRowBytes +
                                 kLatentDim * 2 + part * 16);
          else
            bad = true;
        }
      } else {  // value columns
        const int cc = c - 768, row = cc >> 4, part = cc & 15, key = st * kStageKeys + row;
        if (key < key_end)
          v = *(const uint4*)(a.v + (int64_t)(bo0 + key) * a.v_tok + (int64_t)h * a.v_head + part * 8);
      }
      stg[i] = v;
    }
  };
  auto stash = [&](int buf) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < kPfPerThread; ++i) {
      const int c = tid + i * kPfNT;
      MLA_LDS uint8_t* dst;
      if (c < 512) {
        const int row = c >> 4, part = c & 15;
        dst = kt + buf * kPfKStage + row * kPfKRow + (part ^ pf_kswz(row)) * 16;
      } else if (c < 768) {
        const int cc = c - 512, row = cc >> 3, part = 16 + (cc & 7);
        dst = kt + buf * kPfKStage + row * kPfKRow + (part ^ pf_kswz(row)) * 16;
      } else {
        const int cc = c - 768, row = cc >> 4, part = cc & 15;
        dst = vt + buf * kPfVStage + row * kPfVRow + (part ^ pf_vswz(row)) * 16;
      }
      *(MLA_LDS u32x4*)dst = u32x4{stg[i].x, stg[i].y, stg[i].z, stg[i].w};
    }
  };

  if (nst > 0) fetch(0);

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
  // positions of this lane's two queries (relative to the cache offset of key 0)
  long long qrel[2];
#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) qrel[qb2] = pos0 + (tw + 16 * qb2 + ln) - co;

  if (nst > 0) {
    stash(0);
    __syncthreads();
  }
#pragma unroll 1
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) fetch(st + 1);
    const MLA_LDS uint8_t* K = kt + buf * kPfKStage;
    const MLA_LDS uint8_t* V = vt + buf * kPfVStage;
    const int kbase = st * kStageKeys;

    // S^T = K Q^T: key tiles u = 0, 1 x query blocks
    f32x4 s[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) s[u][0] = s[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      const int c = 4 * ks + gq;
      const bf16x8 k0 = *(const MLA_LDS bf16x8*)(K + rowA0 * kPfKRow + (c ^ pf_kswz(rowA0)) * 16);
      const bf16x8 k1 = *(const MLA_LDS bf16x8*)(K + rowA1 * kPfKRow + (c ^ pf_kswz(rowA1)) * 16);
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        s[0][qb2] = mfma16x16x32(k0, qf[qb2][ks], s[0][qb2]);
        s[1][qb2] = mfma16x16x32(k1, qf[qb2][ks], s[1][qb2]);
      }
    }

    // masks: key kbase + 8gq + j (this lane's keys) against the end of the keys and, under
    // the causal mask, against this lane's query position
    const uint32_t stage_bits = range_bits(kbase, 0, key_end);
    const bool all_valid = stage_bits == 0xFFFFFFFFu &&
                           (a.mask != kMaskCausal || kbase + kStageKeys - 1 <= pos0 + tw - co);
    const float ks8[2][4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
    bf16x8 pf[2];
#pragma unroll
    for (int qb2 = 0; qb2 < 2; ++qb2) {
      uint32_t bits = (stage_bits >> (8 * gq)) & 0xFFu;
      if (a.mask == kMaskCausal) {
        const long long lim = qrel[qb2] - (kbase + 8 * gq) + 1;  // keys j < lim are visible
        const uint32_t cb = lim <= 0 ? 0u : (lim >= 8 ? 0xFFu : ((1u << lim) - 1u));
        bits &= cb;
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
      const bf16x4 a0 = ds_read_tr16(V + rowV0 * kPfVRow + ((2 * cb + (vq >> 1)) ^ pf_vswz(rowV0)) * 16 + vhalf);
      const bf16x4 a1 = ds_read_tr16(V + rowV1 * kPfVRow + ((2 * cb + (vq >> 1)) ^ pf_vswz(rowV1)) * 16 + vhalf);
      const bf16x8 vf = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) acc.o[cb][qb2] = mfma16x16x32(vf, pf[qb2], acc.o[cb][qb2]);
    }

    if (st + 1 < nst) {
      // the other buffer was last read in stage st - 1, before the previous barrier
      stash(buf ^ 1);
      __syncthreads();
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
