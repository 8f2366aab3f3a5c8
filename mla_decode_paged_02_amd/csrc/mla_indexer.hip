// FP8 top-k indexer over a paged cache (gfx950).
//
// What is computed follows mla_indexer_ragged_float8_paged (summary; Args output_indices,
// q, q_s, input_row_offsets, k_collection): for query token t of sequence b, the score of
// visible cache row r is the sum over the indexer heads h of the scaled fp8 dot product
//     score(t, r) = sum_h q_s[t, h] * <e4m3(q[t, h, :]), e4m3(k[r, :])> * k_s[r]
// (one k scale per row, granularity head_size); the mask leaves the rows a decode token
// sees (causal, null, sliding window); the top_k highest-scoring rows are returned per
// token, the rest of the row filled with -1.
//
// Readings where the page is silent: the indices are physical rows of the pool (page_id *
// PS + slot), so that they feed the sparse decode's d_indices directly; they are listed by
// descending score, equal scores by ascending logical position.
//
// The sum over heads is linear, so a work-group first folds the token's heads into one
// float32 query row qf[d] = sum_h q_s[t, h] * e4m3(q[t, h, d]) (heads in order), then
// scores every visible row with one dot product of `depth` terms in float32.  Two
// kernels:
//   score:  one work-group per (token, slice of kIdxSlice visible rows) writes each row's
//           64-bit key (order-preserving score bits, then the inverted position, so every
//           key is distinct) to a workspace row of the token;
//   select: one work-group per token loads its keys (at most kIdxMaxKeys) into LDS, a
//           radix select (eight 8-bit digits, most significant first, histograms in LDS)
//           finds the top_k-th largest key, the keys at or above it are compacted, a
//           bitonic sort orders those top_k, and they are written out.
#include <stdint.h>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

constexpr int kIdxThreads = 256;

// The four e4m3 codes of a dword as floats (exact), byte e -> f[e], through the OCP
// conversion the sparse decode uses (e4m3x4_to_bf16x4).
__device__ __forceinline__ void e4m3x4_f32(uint32_t w, float (&f)[4]) {
  const uint2 b = e4m3x4_to_bf16x4(w);
  f[0] = __builtin_bit_cast(float, b.x << 16);
  f[1] = __builtin_bit_cast(float, b.x & 0xFFFF0000u);
  f[2] = __builtin_bit_cast(float, b.y << 16);
  f[3] = __builtin_bit_cast(float, b.y & 0xFFFF0000u);
}

// float -> unsigned key with the same order (larger float, larger key)
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Bitonic sort of n (a power of two) keys in LDS into descending order.
__device__ __forceinline__ void bitonic_desc(uint64_t* v, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int jdist = k >> 1; jdist > 0; jdist >>= 1) {
      for (int i = threadIdx.x; i < n; i += kIdxThreads) {
        const int p = i ^ jdist;
        if (p > i) {
          const uint64_t x = v[i], y = v[p];
          if ((i & k) == 0 ? x < y : x > y) {
            v[i] = y;
            v[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// The token's sequence (binary search of the offsets) and its visible rows [vlo, vhi).
struct TokenRows {
  int b, vlo, vhi;
};

__device__ __forceinline__ TokenRows token_rows(const IndexerArgs& a, int t, bool report) {
  int lo_b = 0, hi_b = a.B;
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if ((int)ld_const(a.offsets + mid) <= t) lo_b = mid; else hi_b = mid;
  }
  TokenRows r{lo_b, 0, 0};
  const int o0 = (int)ld_const(a.offsets + lo_b), o1 = (int)ld_const(a.offsets + lo_b + 1);
  if (t >= o0 && t < o1) {
    long long L = ld_const(a.cache_lens + lo_b);
    const long long Lmax = (long long)a.max_pages * a.PS;
    if (L > Lmax) {
      if (report) atomicOr(a.err, kErrCacheLen);
      L = Lmax;
    }
    if (L < 0) L = 0;
    const int n = o1 - o0, j = t - o0;
    if (a.mask == kMaskNull) {
      r.vhi = (int)L;
    } else {
      const long long pos = L - n + j;
      long long h = pos + 1 < L ? pos + 1 : L;
      if (h < 0) h = 0;
      long long l = 0;
      if (a.mask == kMaskSliding) {
        l = pos - a.window + 1;
        if (l < 0) l = 0;
        if (l > h) l = h;
      }
      r.vlo = (int)l;
      r.vhi = (int)h;
    }
  } else if (report) {
    atomicOr(a.err, kErrOffsets);  // offsets that do not cover this row
  }
  return r;  // vhi - vlo <= max_pages * PS <= kIdxMaxKeys (checked on the host)
}

__global__ __launch_bounds__(kIdxThreads) void mla_indexer_score_kernel(const IndexerArgs a) {
  __shared__ float qf[kIdxMaxDepth];
  const int t = blockIdx.x, tid = threadIdx.x;
  const TokenRows tr = token_rows(a, t, blockIdx.y == 0 && tid == 0);
  const int vlo = tr.vlo, nvis = tr.vhi - tr.vlo, b = tr.b;
  const int i0 = blockIdx.y * kIdxSlice, i1 = min(nvis, i0 + kIdxSlice);
  if (i0 >= i1) return;  // block-uniform, before any barrier

  // ---- heads folded into one float32 query row
  for (int d = tid; d < a.depth; d += kIdxThreads) {
    float acc = 0.f;
    for (int h = 0; h < a.NH; ++h) {
      float f[4];
      e4m3x4_f32(a.q[(int64_t)t * a.q_tok + (int64_t)h * a.q_head + d], f);
      acc += a.q_s[(int64_t)t * a.qs_tok + h] * f[0];
    }
    qf[d] = acc;
  }
  __syncthreads();

  // ---- scores of this slice's rows as distinct keys
  const int32_t* prow = a.page_table + (int64_t)b * a.pt_row;
  uint64_t* krow = a.keys + (int64_t)t * a.keys_row;
  bool bad = false;
  for (int i = i0 + tid; i < i1; i += kIdxThreads) {
    uint64_t key;
    {
      const int pos = vlo + i;
      const int lp = pos / a.PS, slot = pos - lp * a.PS;
      const int pid = prow[lp];
      float s = -INFINITY;
      if (pid >= 0 && (int64_t)pid < a.num_pages) {
        const uint8_t* row = a.k + (int64_t)pid * a.page_bytes + (int64_t)slot * a.depth;
        float acc = 0.f;
        for (int d = 0; d < a.depth; d += 16) {
          const uint4 v = *(const uint4*)(row + d);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float f[4];
            e4m3x4_f32(w[c], f);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += qf[d + 4 * c + e] * f[e];
          }
        }
        const float ks = a.k_s ? a.k_s[(int64_t)pid * a.ks_page + slot] : 1.f;
        s = acc * ks;
        if (s != s) s = -INFINITY;  // a NaN score (NaN data) ranks last
      } else {
        bad = true;
      }
      // the score's order bits, then the inverted position (equal scores: lower first)
      key = ((uint64_t)order_key(s) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)pos);
    }
    krow[i] = key;
  }
  if (bad) atomicOr(a.err, kErrPageId);
}

__global__ __launch_bounds__(kIdxThreads) void mla_indexer_select_kernel(const IndexerArgs a) {
  __shared__ uint64_t keys[kIdxMaxKeys];
  __shared__ uint64_t top[kIdxMaxTopK];
  __shared__ int hist[256];
  __shared__ int wave_tot[kIdxThreads / 64];
  __shared__ int sel_digit, sel_count;
  static_assert(kIdxThreads == 256, "one thread per histogram bin");
  const int t = blockIdx.x, tid = threadIdx.x;
  const TokenRows tr = token_rows(a, t, false);
  const int nvis = tr.vhi - tr.vlo;
  const int32_t* prow = a.page_table + (int64_t)tr.b * a.pt_row;
  const uint64_t* krow = a.keys + (int64_t)t * a.keys_row;
#pragma unroll 4
  for (int i = tid; i < nvis; i += kIdxThreads) keys[i] = krow[i];
  if (tid == 0) sel_count = 0;
  __syncthreads();

  // ---- the nsel largest keys into top[0 .. nsel), unordered
  const int nsel = min(a.top_k, nvis);
  if (nsel == nvis) {
    for (int i = tid; i < nvis; i += kIdxThreads) top[i] = keys[i];
  } else if (nsel > 0) {
    // radix select of the nsel-th largest key: `prefix` holds its digits found so far
    uint64_t prefix = 0;
    int need = nsel;  // how many keys at or above the threshold are still to be placed
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int d = tid; d < 256; d += kIdxThreads) hist[d] = 0;
      __syncthreads();
      const uint64_t hi_mask = shift == 56 ? 0 : ~0ull << (shift + 8);
#pragma unroll 8
      for (int i = tid; i < nvis; i += kIdxThreads) {
        const uint64_t k = keys[i];
        if ((k & hi_mask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 0xFF)], 1);
      }
      __syncthreads();
      {
        // the digit where the count from the top reaches `need`: thread tid takes digit
        // 255 - tid, so a prefix sum over threads is the count of keys with a digit at or
        // above it; the one thread where that count first reaches `need` writes the digit
        const int d = 255 - tid, c = hist[d];
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int up = __shfl_up(incl, off);
          if ((tid & 63) >= off) incl += up;
        }
        if ((tid & 63) == 63) wave_tot[tid >> 6] = incl;
        __syncthreads();
        for (int w = 0; w < (tid >> 6); ++w) incl += wave_tot[w];
        if (c > 0 && incl >= need && incl - c < need) {
          sel_digit = d;
          sel_count = need - (incl - c);  // still needed within digit d
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sel_digit << shift;
      need = sel_count;
      __syncthreads();
    }
    // keys are distinct: exactly nsel keys are >= the threshold `prefix`
    if (tid == 0) sel_count = 0;
    __syncthreads();
    for (int i = tid; i < nvis; i += kIdxThreads) {
      const uint64_t k = keys[i];
      if (k >= prefix) top[atomicAdd(&sel_count, 1)] = k;
    }
  }
  __syncthreads();

  // ---- order them: bitonic sort over the next power of two (padding keys 0 sort last)
  int npow = 1;
  while (npow < nsel) npow <<= 1;
  for (int i = nsel + tid; i < npow; i += kIdxThreads) top[i] = 0;
  __syncthreads();
  bitonic_desc(top, npow);

  // ---- the top_k as physical rows, then -1
  int32_t* orow = a.out + (int64_t)t * a.out_row;
  for (int i = tid; i < a.top_k; i += kIdxThreads) {
    int32_t v = -1;
    if (i < nsel) {
      const int pos = (int)(0xFFFFFFFFu - (uint32_t)(top[i] & 0xFFFFFFFFu));
      const int lp = pos / a.PS, slot = pos - lp * a.PS;
      const int pid = prow[lp];
      v = (pid >= 0 && (int64_t)pid < a.num_pages) ? pid * a.PS + slot : -1;
    }
    orow[i] = v;
  }
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream, const KernelTimer* timer) {
  hipError_t e;
  if (timer && (e = hipEventRecord(timer->start, stream)) != hipSuccess) return e;
  const int slices = (int)((a.keys_row + kIdxSlice - 1) / kIdxSlice);
  hipLaunchKernelGGL(mla_indexer_score_kernel, dim3(a.T, slices > 0 ? slices : 1), dim3(kIdxThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(mla_indexer_select_kernel, dim3(a.T), dim3(kIdxThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (timer && (e = hipEventRecord(timer->stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
