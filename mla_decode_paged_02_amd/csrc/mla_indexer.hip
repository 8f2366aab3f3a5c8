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
// float32 query row qf[d] = sum_h q_s[t, h] * e4m3(q[t, h, d]) (a fixed order), then
// scores every visible row with one dot product of `depth` terms in float32.  Two
// kernels:
//   score:  one work-group per (token, slice of kIdxSlice visible rows) writes each row's
//           64-bit key (order-preserving score bits, then the inverted position, so every
//           key is distinct) to a workspace row of the token;
//   select: one work-group of 1024 threads per token loads its keys (at most
//           kIdxMaxKeys) into LDS; a radix select (eight 8-bit digits, most significant
//           first, histograms in LDS) finds the top_k-th largest key.  Once the bin that
//           holds it has at most kIdxCand keys, one pass moves the keys above that bin to
//           the output list and the bin's keys to a candidate list, and the remaining
//           digits scan the candidates only.  A bitonic sort (in registers and lane
//           shuffles up to distance 64, LDS beyond) orders the top_k, and they are written
//           out.
#include <stdint.h>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

constexpr int kIdxThreads = 256;      // scoring work-group
constexpr int kIdxSelThreads = 1024;  // selection work-group
constexpr int kIdxCand = 1024;        // candidate list of the radix select

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

// The value of lane (lane ^ M): DPP quad permutes for M = 1, 2, a bitmask-mode swizzle
// (lane ^ M within 32 lanes) for M = 4 .. 16, a bpermute for M = 32.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane distance");
  if constexpr (M == 1)
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  else if constexpr (M == 2)
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  else if constexpr (M < 32)
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));  // and 0x1F, xor M
  else
    return (uint32_t)__shfl_xor((unsigned)v, M);
}

// One compare-exchange stage at element distance J (2 .. 64) on the thread's two keys
// (elements e0 and e0 + 1), partners J / 2 lanes away.
template <int J>
__device__ __forceinline__ void lane_stage(uint64_t (&x)[2], int e0, int k) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = e0 + u;
    const uint32_t lo = lane_xor<J / 2>((uint32_t)x[u]), hi = lane_xor<J / 2>((uint32_t)(x[u] >> 32));
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    // the lower element of a descending pair keeps the larger key
    const bool keep_max = ((e & J) == 0) == ((e & k) == 0);
    x[u] = keep_max ? (x[u] > y ? x[u] : y) : (x[u] < y ? x[u] : y);
  }
}

// Bitonic sort of n (a power of two, n <= 2 * kIdxSelThreads) keys in LDS into descending
// order.  Thread tid holds elements 2 tid and 2 tid + 1 in registers: compare-exchange at
// distance 1 stays in the thread, and distances 2 .. 64 pair lanes 1 .. 32 apart within
// the wave (the partner of element e is e ^ jdist, in thread tid ^ jdist / 2), so neither
// needs a barrier.  Distances of 128 and more go through LDS, one barrier per stage.
__device__ __forceinline__ void bitonic_desc(uint64_t* v, int n) {
  static_assert(kIdxMaxTopK <= 2 * kIdxSelThreads, "two keys per thread");
  const int tid = threadIdx.x, e0 = 2 * tid;
  uint64_t x[2] = {0, 0};
  if (e0 < n) {
    x[0] = v[e0];
    x[1] = v[e0 + 1];
  }
  for (int k = 2; k <= n; k <<= 1) {
    if ((k >> 1) >= 128) {
      if (e0 < n) {
        v[e0] = x[0];
        v[e0 + 1] = x[1];
      }
      __syncthreads();
      for (int jdist = k >> 1; jdist >= 128; jdist >>= 1) {
        for (int j = tid; j < (n >> 1); j += kIdxSelThreads) {
          const int i = ((j & ~(jdist - 1)) << 1) | (j & (jdist - 1)), p = i + jdist;
          const uint64_t lo = v[i], hi = v[p];
          if ((i & k) == 0 ? lo < hi : lo > hi) {
            v[i] = hi;
            v[p] = lo;
          }
        }
        __syncthreads();
      }
      if (e0 < n) {
        x[0] = v[e0];
        x[1] = v[e0 + 1];
      }
    }
    switch (min(k >> 1, 64)) {  // distances min(k / 2, 64) down to 2
      case 64: lane_stage<64>(x, e0, k); [[fallthrough]];
      case 32: lane_stage<32>(x, e0, k); [[fallthrough]];
      case 16: lane_stage<16>(x, e0, k); [[fallthrough]];
      case 8: lane_stage<8>(x, e0, k); [[fallthrough]];
      case 4: lane_stage<4>(x, e0, k); [[fallthrough]];
      case 2: lane_stage<2>(x, e0, k); [[fallthrough]];
      default: break;
    }
    if ((e0 & k) == 0 ? x[0] < x[1] : x[0] > x[1]) {
      const uint64_t tmp = x[0];
      x[0] = x[1];
      x[1] = tmp;
    }
  }
  if (e0 < n) {
    v[e0] = x[0];
    v[e0 + 1] = x[1];
  }
  __syncthreads();
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

// NC: 16-byte chunks of a cache row held in registers (depth <= 16 * NC); RF: rows a
// thread has in flight at once.
template <int NC, int RF>
__global__ __launch_bounds__(kIdxThreads) void mla_indexer_score_kernel(const IndexerArgs a) {
  constexpr int R = kIdxSlice / kIdxThreads;  // rows per thread
  static_assert(R % RF == 0, "rows per thread in whole groups");
  __shared__ __align__(16) float qf[kIdxMaxDepth];
  __shared__ float part[kIdxThreads];
  const int t = blockIdx.x, tid = threadIdx.x;
  const TokenRows tr = token_rows(a, t, blockIdx.y == 0 && tid == 0);
  const int vlo = tr.vlo, nvis = tr.vhi - tr.vlo, b = tr.b;
  const int i0 = blockIdx.y * kIdxSlice, i1 = min(nvis, i0 + kIdxSlice);
  if (i0 >= i1) return;  // block-uniform, before any barrier

  // ---- the page ids of this thread's rows (rows i0 + tid + r * kIdxThreads)
  const int32_t* prow = a.page_table + (int64_t)b * a.pt_row;
  int pid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = i0 + tid + r * kIdxThreads;
    pid[r] = i < i1 ? prow[(vlo + i) / a.PS] : 0;
  }

  // ---- heads folded into one float32 query row: G groups of `depth` threads, group g
  // summing heads g, g + G, ...; the groups' sums are then added in group order
  const int G = kIdxThreads / a.depth;
  if (tid < G * a.depth) {
    const int g = tid / a.depth, d = tid - g * a.depth;
    const uint8_t* qt = a.q + (int64_t)t * a.q_tok + d;
    const float* qst = a.q_s + (int64_t)t * a.qs_tok;
    float acc = 0.f;
#pragma unroll 8
    for (int h = g; h < a.NH; h += G) {
      float f[4];
      e4m3x4_f32(qt[(int64_t)h * a.q_head], f);
      acc += qst[h] * f[0];
    }
    part[tid] = acc;
  }
  __syncthreads();
  if (tid < a.depth) {
    float acc = 0.f;
    for (int g = 0; g < G; ++g) acc += part[g * a.depth + tid];
    qf[tid] = acc;
  }
  __syncthreads();

  // ---- scores of this slice's rows as distinct keys, RF rows in flight
  uint64_t* krow = a.keys + (int64_t)t * a.keys_row;
  bool bad = false;
#pragma unroll
  for (int r0 = 0; r0 < R; r0 += RF) {
    uint4 v[RF][NC];
    bool ok[RF];
    int pos[RF];
    float ks[RF];
#pragma unroll
    for (int u = 0; u < RF; ++u) {
      const int i = i0 + tid + (r0 + u) * kIdxThreads;
      pos[u] = vlo + i;
      const int lp = pos[u] / a.PS, slot = pos[u] - lp * a.PS, p = pid[r0 + u];
      ok[u] = p >= 0 && (int64_t)p < a.num_pages;
      if (i < i1 && !ok[u]) bad = true;
      ok[u] = ok[u] && i < i1;
      ks[u] = 1.f;
      if (ok[u]) {
        const uint8_t* row = a.k + (int64_t)p * a.page_bytes + (int64_t)slot * a.depth;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (c * 16 < a.depth) v[u][c] = *(const uint4*)(row + c * 16);
        if (a.k_s) ks[u] = a.k_s[(int64_t)p * a.ks_page + slot];
      }
    }
#pragma unroll
    for (int u = 0; u < RF; ++u) {
      const int i = i0 + tid + (r0 + u) * kIdxThreads;
      if (i >= i1) continue;
      float s = -INFINITY;
      if (ok[u]) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (c * 16 >= a.depth) break;
          const uint32_t w[4] = {v[u][c].x, v[u][c].y, v[u][c].z, v[u][c].w};
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            float f[4];
            e4m3x4_f32(w[e4], f);
            const float4 qv = *(const float4*)&qf[c * 16 + 4 * e4];
            acc += qv.x * f[0];
            acc += qv.y * f[1];
            acc += qv.z * f[2];
            acc += qv.w * f[3];
          }
        }
        s = acc * ks[u];
        if (s != s) s = -INFINITY;  // a NaN score (NaN data) ranks last
      }
      // the score's order bits, then the inverted position (equal scores: lower first)
      krow[i] = ((uint64_t)order_key(s) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)pos[u]);
    }
  }
  if (bad) atomicOr(a.err, kErrPageId);
}

__global__ __launch_bounds__(kIdxSelThreads) void mla_indexer_select_kernel(const IndexerArgs a) {
  __shared__ uint64_t keys[kIdxMaxKeys];
  __shared__ uint64_t top[kIdxMaxTopK];
  __shared__ uint64_t cand[kIdxCand];
  __shared__ int hist[256];
  __shared__ int wave_tot[4];
  __shared__ int sel_digit, sel_count, sel_bin, n_top, n_cand;
  const int t = blockIdx.x, tid = threadIdx.x;
  const TokenRows tr = token_rows(a, t, false);
  const int nvis = tr.vhi - tr.vlo;
  const int32_t* prow = a.page_table + (int64_t)tr.b * a.pt_row;
  const uint64_t* krow = a.keys + (int64_t)t * a.keys_row;
#pragma unroll
  for (int r = 0; r < kIdxMaxKeys / kIdxSelThreads; ++r) {
    const int i = tid + r * kIdxSelThreads;
    if (i < nvis) keys[i] = krow[i];
  }
  if (tid == 0) {
    n_top = 0;
    n_cand = 0;
  }
  __syncthreads();

  // ---- the nsel largest keys into top[0 .. nsel), unordered
  const int nsel = min(a.top_k, nvis);
  if (nsel == nvis) {
    for (int i = tid; i < nvis; i += kIdxSelThreads) top[i] = keys[i];
  } else if (nsel > 0) {
    // radix select of the nsel-th largest key: `prefix` holds its digits found so far,
    // the keys still in play are src[0 .. nsrc)
    uint64_t prefix = 0;
    int need = nsel;  // how many keys at or above the threshold are still to be placed
    const uint64_t* src = keys;
    int nsrc = nvis;
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      const uint64_t hi_mask = shift == 56 ? 0 : ~0ull << (shift + 8);
#pragma unroll 4
      for (int i = tid; i < nsrc; i += kIdxSelThreads) {
        const uint64_t k = src[i];
        if ((k & hi_mask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 0xFF)], 1);
      }
      __syncthreads();
      // the digit where the count from the top reaches `need`: thread tid < 256 takes
      // digit 255 - tid, so a prefix sum over those threads is the count of keys with a
      // digit at or above it; the one thread where that count first reaches `need`
      // writes the digit
      const int d = 255 - tid;
      int c = 0, incl = 0;
      if (tid < 256) {
        c = hist[d];
        incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int up = __shfl_up(incl, off);
          if ((tid & 63) >= off) incl += up;
        }
        if ((tid & 63) == 63) wave_tot[tid >> 6] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < (tid >> 6); ++w) incl += wave_tot[w];
        if (c > 0 && incl >= need && incl - c < need) {
          sel_digit = d;
          sel_count = need - (incl - c);  // still needed within digit d
          sel_bin = c;                    // keys whose digits so far equal the new prefix
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sel_digit << shift;
      need = sel_count;
      const int bin = sel_bin;
      __syncthreads();
      if (src == keys && shift > 0 && bin <= kIdxCand) {
        // keys above the prefix on the digits found are in the top for sure; the keys
        // equal to it there become the candidates for the remaining digits
        const uint64_t m = ~0ull << shift;
#pragma unroll 4
        for (int i = tid; i < nvis; i += kIdxSelThreads) {
          const uint64_t k = keys[i], km = k & m;
          if (km > prefix) top[atomicAdd(&n_top, 1)] = k;
          else if (km == prefix) cand[atomicAdd(&n_cand, 1)] = k;
        }
        __syncthreads();
        src = cand;
        nsrc = bin;
      }
    }
    // keys are distinct: exactly nsel keys are >= the threshold `prefix`, those of
    // src[0 .. nsrc) not yet in top
    for (int i = tid; i < nsrc; i += kIdxSelThreads) {
      const uint64_t k = src[i];
      if (k >= prefix) top[atomicAdd(&n_top, 1)] = k;
    }
  }
  __syncthreads();

  // ---- order them: bitonic sort over the next power of two (padding keys 0 sort last)
  int npow = 1;
  while (npow < nsel) npow <<= 1;
  for (int i = nsel + tid; i < npow; i += kIdxSelThreads) top[i] = 0;
  __syncthreads();
  bitonic_desc(top, npow);

  // ---- the top_k as physical rows, then -1
  int32_t* orow = a.out + (int64_t)t * a.out_row;
  for (int i = tid; i < a.top_k; i += kIdxSelThreads) {
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
  const dim3 sgrid(a.T, slices > 0 ? slices : 1);
  if (a.depth <= 128)
    hipLaunchKernelGGL((mla_indexer_score_kernel<8, 2>), sgrid, dim3(kIdxThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((mla_indexer_score_kernel<16, 1>), sgrid, dim3(kIdxThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(mla_indexer_select_kernel, dim3(a.T), dim3(kIdxSelThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (timer && (e = hipEventRecord(timer->stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
