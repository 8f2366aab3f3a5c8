// Per-wave compute of one 32-key stage held in LDS, shared by the decode kernels.
//
// A wave owns 16*HB heads of one query row.  With the stage's keys in LDS as bf16 rows of
// 576 (swizzled 16-byte chunks, see swz_chunk):
//   S^T = K Q^T   (16 keys x 16 heads MFMA tiles, 18 k-steps over the 576 columns).  The
//                 keys of each 16-row tile are permuted -- tile u, row m reads key
//                 8*(m/4) + 4u + m%4 -- so that the accumulator layout of S^T (lane 16g+n
//                 holds rows 4g..4g+3, column n) is exactly the operand layout P^T needs:
//                 lane 16g+n holds head n, keys 8g..8g+7;
//   softmax       base-2 online softmax; the running max m is raised only when a stage's
//                 max exceeds it by more than kRescaleSlack, so O and l are rescaled rarely
//                 (the result is the same real number: any offset cancels in O / l);
//   O^T += V^T P^T (512 columns x 16*HB heads, V = the first 512 columns of the same rows),
//                 V^T fragments read with the transposing LDS load.
#pragma once

#include "mla_device.h"

namespace mla {

template <int HB>
struct WaveAcc {
  f32x4 o[32][HB];  // lane 16g+n: O^T[16cb + 4g + i][head 16hb + n]
  float m[HB];      // running max (log2 units)
  float l[HB];      // this lane's share of the softmax denominator
};

// Per-lane constants of the LDS access patterns: byte offsets within a stage.
//   ka[u][p]  score read of key tile u at k-step ks with ks % 2 == p; k-step ks reads at
//             ka[u][ks % 2] + 128 (ks / 2) (the rope k-steps 16, 17 included);
//   va[u][j]  transposing value read of tile u for column block cb with cb % 4 == j, at
//             va[u][j] + 128 (cb / 4).
struct LaneGeo {
  int gq;
  int ka[2][2];
  int va[2][4];
};

__device__ __forceinline__ LaneGeo make_lane_geo(int lane) {
  LaneGeo g;
  g.gq = lane >> 4;
  const int ln = lane & 15;
  const int vq = lane & 3;  // transposing-read coordinates: row 8gq + ln/4, chunk half vq
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ra = 8 * (ln >> 2) + (ln & 3) + 4 * u;  // key row of tile u, MFMA row ln
    const int sa = swz_mask(ra);
#pragma unroll
    for (int p = 0; p < 2; ++p) g.ka[u][p] = ra * kRowBytes + (((4 * p + g.gq) ^ sa) << 4);
    const int rv = 8 * g.gq + (ln >> 2) + 4 * u;
    const int sv = swz_mask(rv);
#pragma unroll
    for (int j = 0; j < 4; ++j) g.va[u][j] = rv * kRowBytes + (((2 * j + (vq >> 1)) ^ sv) << 4) + 8 * (vq & 1);
  }
  return g;
}

template <int HB>
__device__ __forceinline__ void wave_acc_init(WaveAcc<HB>& acc) {
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc.o[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    acc.m[hb] = -INFINITY;
    acc.l[hb] = 0.f;
  }
}

// valid: bit j set when key j of the stage is visible (block-uniform).  kscale (KSCALE
// only): per-key factors of the stage in LDS, applied to the logit and to the value row.
// Online softmax of one 16-row block of a stage (a row is a head in decode, a query in
// prefill): su0 / su1 are the score accumulators of key tiles u = 0, 1 (lane 16g+n: row n,
// keys 8g + 4u + i).  lane_bits: bit j set when key 8g + j counts for this lane's row
// (all_valid: every key of the stage counts for every row).  Returns P^T as the MFMA
// operand (lane 16g+n: row n, keys 8g..8g+7) and updates the running max m (log2 units,
// the same in the four lanes of a row) and this lane's share l of the denominator.
// The common case needs no cross-lane work: the max is only reduced over the four lanes of
// a head when some lane's keys exceed m by more than kRescaleSlack; rescale(alpha) then
// multiplies the block's O by alpha.
template <bool KSCALE, class Rescale>
__device__ __forceinline__ bf16x8 softmax_block(f32x4 su0, f32x4 su1, uint32_t lane_bits, bool all_valid,
                                                float scale_log2, const float (&ks8)[2][4], float& m, float& l,
                                                Rescale rescale) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = su0[i] * scale_log2;
    x[4 + i] = su1[i] * scale_log2;
    if (KSCALE) {
      x[i] *= ks8[0][i];
      x[4 + i] *= ks8[1][i];
    }
  }
  if (!all_valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = ((lane_bits >> j) & 1u) ? x[j] : -INFINITY;
  }
  float lmax = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) lmax = fmaxf(lmax, x[j]);
  if (__builtin_amdgcn_ballot_w64(lmax > m + kRescaleSlack) != 0) {
    const float mx = wave_max_xor16_32(lmax);
    const bool upd = mx > m + kRescaleSlack;  // the same in the four lanes of a head
    const float m_new = upd ? mx : m;
    const float alpha = upd ? fast_exp2(m - m_new) : 1.f;  // 0 while m is -inf
    l *= alpha;
    // O is still exactly zero while m is -inf: only a finite old max needs the multiply
    if (__builtin_amdgcn_ballot_w64(upd && m != -INFINITY) != 0) rescale(alpha);
    m = m_new;
  }
  const float mref = m == -INFINITY ? 0.f : m;  // a head with no visible key so far
  bf16x8 pf;
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = fast_exp2(x[j] - mref);
    pf[j] = (__bf16)(KSCALE ? p[j] * ks8[j >> 2][j & 3] : p[j]);
  }
  if (KSCALE) {
    // the value row is code * scale: the scale is folded into the weight, not into l
#pragma unroll
    for (int j = 0; j < 8; ++j) l += p[j];
  } else {
    // sum the weights as rounded for the MFMA, so a constant V column is reproduced
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int j = 0; j < 8; j += 2) l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pf[j], pf[j + 1]}, one, l, false);
  }
  return pf;
}

// hook(ks) runs after the MFMAs of score k-step ks (0..17) and hook(18 + cb) after those of
// value column block cb (0..31): the caller's slots for work on other stages (their loads,
// their conversion) that runs while the matrix cores work.
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

template <int HB, bool KSCALE, class Hook = NoHook>
__device__ __forceinline__ void stage_compute(const MLA_LDS uint8_t* buf, const bf16x8 (&qf)[HB][18],
                                              WaveAcc<HB>& acc, uint32_t valid, float scale_log2,
                                              const MLA_LDS float* kscale, const LaneGeo& g, Hook hook = Hook()) {
  // ---- S^T = K Q^T, fragments prefetched one k-step ahead
  f32x4 sacc[2][HB];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) sacc[u][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    // Used for 16 and 32 heads (one or two waves, each on a SIMD of its own): the LDS
    // reads are issued just before use and the compiler schedules their waits.
    // Swizzled addresses are formed per read (one xor and one add) rather than kept in
    // registers.
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8 k0 = *(const MLA_LDS bf16x8*)(buf + g.ka[0][ks & 1] + 128 * (ks >> 1));
      const bf16x8 k1 = *(const MLA_LDS bf16x8*)(buf + g.ka[1][ks & 1] + 128 * (ks >> 1));
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        sacc[0][hb] = mfma16x16x32(k0, qf[hb][ks], sacc[0][hb]);
        sacc[1][hb] = mfma16x16x32(k1, qf[hb][ks], sacc[1][hb]);
      }
      __builtin_amdgcn_sched_barrier(0);
      hook(ks);
    }
  }

  // ---- online softmax
  const bool all_valid = valid == 0xFFFFFFFFu;
  float ks8[2][4];
  if (KSCALE) {
    const f32x4 a = *(const MLA_LDS f32x4*)(kscale + 8 * g.gq);
    const f32x4 b = *(const MLA_LDS f32x4*)(kscale + 8 * g.gq + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ks8[0][i] = a[i];
      ks8[1][i] = b[i];
    }
  }
  bf16x8 pf[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
    pf[hb] = softmax_block<KSCALE>(sacc[0][hb], sacc[1][hb], valid >> (8 * g.gq), all_valid, scale_log2, ks8, acc.m[hb],
                                   acc.l[hb], [&](float alpha) {
#pragma unroll
                                     for (int cb = 0; cb < 32; ++cb) acc.o[cb][hb] *= alpha;
                                   });

  // ---- O^T += V^T P^T over the stage's 32 keys
  {
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const bf16x4 a0 = ds_read_tr16(buf + g.va[0][cb & 3] + 128 * (cb >> 2));
      const bf16x4 a1 = ds_read_tr16(buf + g.va[1][cb & 3] + 128 * (cb >> 2));
      const bf16x8 vf = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc.o[cb][hb] = mfma16x16x32(vf, pf[hb], acc.o[cb][hb]);
      hook(18 + cb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The reciprocal of a finished row's softmax denominator: this wave's summed weights l_tot
// (relative to the running max m, log2 units), plus e^sink of the head's sink logit when
// there is one (that weight carries no value).  0 when nothing was weighed.
__device__ __forceinline__ float row_inverse(float l_tot, float m, const float* sink, int h) {
  float den = l_tot;
  if (sink != nullptr) den += fast_exp2(sink[h] * 1.4426950408889634f - m);  // +inf while m is -inf
  return den > 0.f ? 1.f / den : 0.f;
}

// Writes the wave's heads h0 + 16hb + n of row t: final bf16 output, or the normalised
// partial and its log2-sum-exp into `slot` (a split row's sink joins in the combine).
template <int HB>
__device__ __forceinline__ void stage_epilogue(const WaveAcc<HB>& acc, int lane, int h0, int t, bool full,
                                               int slot, int H, uint16_t* out, int64_t o_tok, int64_t o_head,
                                               uint16_t* part_o, float* part_lse, const float* sink) {
  const int gq = lane >> 4, ln = lane & 15;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const float l_tot = wave_sum_xor16_32(acc.l[hb]);
    const int h = h0 + 16 * hb + ln;
    const float inv = full ? row_inverse(l_tot, acc.m[hb], sink, h) : (l_tot > 0.f ? 1.f / l_tot : 0.f);
    // the final row, or a split row's normalised part (bf16 as well) and its log2-sum-exp
    uint16_t* orow = full ? out + (int64_t)t * o_tok + (int64_t)h * o_head + 4 * gq
                          : part_o + ((int64_t)slot * H + h) * kLatentDim + 4 * gq;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const uint32_t lo = (uint32_t)bf16_bits_rne(acc.o[cb][hb][0] * inv) |
                          ((uint32_t)bf16_bits_rne(acc.o[cb][hb][1] * inv) << 16);
      const uint32_t hi = (uint32_t)bf16_bits_rne(acc.o[cb][hb][2] * inv) |
                          ((uint32_t)bf16_bits_rne(acc.o[cb][hb][3] * inv) << 16);
      *(uint2*)(orow + 16 * cb) = make_uint2(lo, hi);
    }
    if (!full && gq == 0) part_lse[(int64_t)slot * H + h] = l_tot > 0.f ? acc.m[hb] + __log2f(l_tot) : -INFINITY;
  }
}

// Bits j (0..31) set for keys base + j that lie in [lo, hi).
__device__ __forceinline__ uint32_t range_bits(int base, int lo, int hi) {
  const int a = max(0, lo - base), b = min(32, hi - base);
  if (b <= a) return 0u;
  const uint32_t upto = b >= 32 ? 0xFFFFFFFFu : ((1u << b) - 1u);
  const uint32_t from = a >= 32 ? 0u : ~((1u << a) - 1u);
  return upto & from;
}


// ---------------------------------------------------------------------------------------
// Wide variant: a wave owns 32 heads (HB = 2), one wave per SIMD.  Each K fragment read
// from LDS then feeds two MFMAs, halving LDS traffic per MFMA compared with 16-head waves.
// O (32 heads x 512 columns, 256 registers per lane) must live in the accumulation
// registers while the score accumulators, Q and the fragments use ordinary ones, so the
// MFMAs are issued through inline assembly with explicit register-file constraints.  The
// compiler does not see inside these statements, so the wait states an MFMA result needs
// before other instructions read it are inserted explicitly (mfma_fence_*): 16 wait
// states cover the longest MFMA-write -> VALU-read distance of the 16x16x32 shapes, and
// ordinary-register inputs written by VALU get two wait states before an MFMA reads them.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void mfma_v_first(f32x4& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a(f32x4& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Orders all later reads of the four score accumulators after enough wait states.
__device__ __forceinline__ void mfma_fence_v4(f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
// Two wait states between VALU writes of MFMA inputs and the MFMA reading them.
__device__ __forceinline__ void valu_fence_v2(bf16x8& a, bf16x8& b) {
  asm volatile("s_nop 1" : "+v"(a), "+v"(b));
}
// Orders later reads of accumulation registers after the MFMAs that wrote them.
template <int N>
__device__ __forceinline__ void mfma_fence_acc(f32x4 (&o)[N]) {
  static_assert(N % 8 == 0, "fenced in groups of eight");
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]),
               "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]));
#pragma unroll
  for (int i = 8; i < N; i += 8)
    asm volatile("" : "+a"(o[i]), "+a"(o[i + 1]), "+a"(o[i + 2]), "+a"(o[i + 3]), "+a"(o[i + 4]),
                 "+a"(o[i + 5]), "+a"(o[i + 6]), "+a"(o[i + 7]));
}

struct WaveAcc2 {
  f32x4 o[64];  // o[2*cb + hb], lane 16g+n: O^T[16cb + 4g + i][head 16hb + n]
  float m[2], l[2];
};

__device__ __forceinline__ void wave_acc2_init(WaveAcc2& acc) {
#pragma unroll
  for (int i = 0; i < 64; ++i) acc.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc.m[0] = acc.m[1] = -INFINITY;
  acc.l[0] = acc.l[1] = 0.f;
}

template <bool KSCALE, class Hook = NoHook>
__device__ __forceinline__ void stage_compute2(const MLA_LDS uint8_t* buf, const bf16x8 (&qf)[2][18],
                                               WaveAcc2& acc, uint32_t valid, float scale_log2,
                                               const MLA_LDS float* kscale, const LaneGeo& g, Hook hook = Hook()) {
  // ---- S^T = K Q^T: 2 key tiles x 2 head blocks.  With one wave per SIMD nothing else
  // hides LDS latency, so K fragments are read kPrefetch k-steps ahead of their MFMAs and
  // scheduling barriers keep the compiler from regrouping the reads.
  constexpr int kPrefetch = 2;
  f32x4 s00, s01, s10, s11;  // s<u><hb>
  {
    auto kread = [&](int u, int ks) {
      return *(const MLA_LDS bf16x8*)(buf + g.ka[u][ks & 1] + 128 * (ks >> 1));
    };
    bf16x8 kf[18][2];  // fully unrolled: only kPrefetch + 1 steps are live at a time
#pragma unroll
    for (int ks = 0; ks < kPrefetch; ++ks) {
      kf[ks][0] = kread(0, ks);
      kf[ks][1] = kread(1, ks);
    }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      if (ks + kPrefetch < 18) {
        kf[ks + kPrefetch][0] = kread(0, ks + kPrefetch);
        kf[ks + kPrefetch][1] = kread(1, ks + kPrefetch);
      }
      if (ks == 0) {
        mfma_v_first(s00, kf[0][0], qf[0][0]);
        mfma_v_first(s10, kf[0][1], qf[0][0]);
        mfma_v_first(s01, kf[0][0], qf[1][0]);
        mfma_v_first(s11, kf[0][1], qf[1][0]);
      } else {
        mfma_v(s00, kf[ks][0], qf[0][ks]);
        mfma_v(s10, kf[ks][1], qf[0][ks]);
        mfma_v(s01, kf[ks][0], qf[1][ks]);
        mfma_v(s11, kf[ks][1], qf[1][ks]);
      }
      hook(ks);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfma_fence_v4(s00, s01, s10, s11);
  }

  // ---- online softmax
  const bool all_valid = valid == 0xFFFFFFFFu;
  float ks8[2][4];
  if (KSCALE) {
    const f32x4 a = *(const MLA_LDS f32x4*)(kscale + 8 * g.gq);
    const f32x4 b = *(const MLA_LDS f32x4*)(kscale + 8 * g.gq + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ks8[0][i] = a[i];
      ks8[1][i] = b[i];
    }
  }
  bf16x8 pf[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
    pf[hb] = softmax_block<KSCALE>(hb == 0 ? s00 : s01, hb == 0 ? s10 : s11, valid >> (8 * g.gq), all_valid, scale_log2,
                                   ks8, acc.m[hb], acc.l[hb], [&](float alpha) {
      // The previous stage's last writes of O were followed by this stage's score MFMAs,
      // far more than the wait states a read needs.  One quad at a time through ordinary
      // registers: each step is tied to the next quad so the compiler cannot lift all the
      // reads ahead and run out of registers.
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        acc.o[2 * cb + hb] *= alpha;
        if (cb + 1 < 32)
          asm volatile("" : "+a"(acc.o[2 * cb + hb]), "+a"(acc.o[2 * cb + 2 + hb]));
        else
          asm volatile("" : "+a"(acc.o[2 * cb + hb]));
      }
    });
  valu_fence_v2(pf[0], pf[1]);

  // ---- O^T += V^T P^T, V^T fragments read kPrefetch column blocks ahead
  {
    auto vread = [&](int u, int cb) { return ds_read_tr16(buf + g.va[u][cb & 3] + 128 * (cb >> 2)); };
    bf16x4 vt[32][2];  // fully unrolled: only kPrefetch + 1 blocks are live at a time
#pragma unroll
    for (int cb = 0; cb < kPrefetch; ++cb) {
      vt[cb][0] = vread(0, cb);
      vt[cb][1] = vread(1, cb);
    }
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      __builtin_amdgcn_sched_barrier(0);
      if (cb + kPrefetch < 32) {
        vt[cb + kPrefetch][0] = vread(0, cb + kPrefetch);
        vt[cb + kPrefetch][1] = vread(1, cb + kPrefetch);
      }
      const bf16x8 vf = {vt[cb][0][0], vt[cb][0][1], vt[cb][0][2], vt[cb][0][3],
                         vt[cb][1][0], vt[cb][1][1], vt[cb][1][2], vt[cb][1][3]};
      mfma_a(acc.o[2 * cb], vf, pf[0]);
      mfma_a(acc.o[2 * cb + 1], vf, pf[1]);
      hook(18 + cb);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Writes the wave's 32 heads h0 .. h0+31 of row t: the final bf16 output, or the split
// row's normalised part (bf16) and its log2-sum-exp into `slot`.  The normalised values go
// through this wave's 32 KB of LDS (`stage`, free once the last stage has been computed)
// so that every store instruction writes one head's 1 KB row contiguously; head rows are
// XOR-swizzled in 16-byte units so the transposing writes spread over the banks.
__device__ __forceinline__ void stage_epilogue2(WaveAcc2& acc, int lane, int h0, int t, bool full, int slot,
                                                int H, uint16_t* out, int64_t o_tok, int64_t o_head,
                                                uint16_t* part_o, float* part_lse, MLA_LDS uint8_t* stage,
                                                const float* sink) {
  mfma_fence_acc(acc.o);
  const int gq = lane >> 4, ln = lane & 15;
  float inv[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float l_tot = wave_sum_xor16_32(acc.l[hb]);
    inv[hb] = full ? row_inverse(l_tot, acc.m[hb], sink, h0 + 16 * hb + ln) : (l_tot > 0.f ? 1.f / l_tot : 0.f);
    if (!full && gq == 0)
      part_lse[(int64_t)slot * H + h0 + 16 * hb + ln] = l_tot > 0.f ? acc.m[hb] + __log2f(l_tot) : -INFINITY;
  }
  // lane 16g+n holds columns 16cb + 4g .. +3 of head 16hb + n
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int hl = 16 * hb + ln;
    MLA_LDS uint8_t* row = stage + hl * 1024;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const f32x4 v = acc.o[2 * cb + hb];
      const uint32_t lo = (uint32_t)bf16_bits_rne(v[0] * inv[hb]) | ((uint32_t)bf16_bits_rne(v[1] * inv[hb]) << 16);
      const uint32_t hi = (uint32_t)bf16_bits_rne(v[2] * inv[hb]) | ((uint32_t)bf16_bits_rne(v[3] * inv[hb]) << 16);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      *(MLA_LDS u32x2*)(row + ((32 * cb + 8 * gq) ^ ((hl & 15) << 4))) = u32x2{lo, hi};
    }
  }
  lgkm_wait0();
  uint16_t* base = full ? out + (int64_t)t * o_tok + (int64_t)h0 * o_head
                        : part_o + ((int64_t)slot * H + h0) * kLatentDim;
  const int64_t hstride = full ? o_head : kLatentDim;
#pragma unroll 4
  for (int hl = 0; hl < 32; ++hl) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = *(const MLA_LDS u32x4*)(stage + hl * 1024 + ((16 * lane) ^ ((hl & 15) << 4)));
    __builtin_nontemporal_store(w, (u32x4*)(base + hl * hstride + 8 * lane));
  }
}

}  // namespace mla
