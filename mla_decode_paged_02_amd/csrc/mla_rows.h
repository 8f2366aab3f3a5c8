// Row geometry of paged decode rows, shared by the dense decode and the dense fp8 path
// of the gathered-row kernel.
//
// Query row t is token j of the n_b tokens of sequence b (input_row_offsets); with L =
// cache_lens[b] rows it sits at position L - n_b + j and sees the keys the mask allows
// (generic_flare_mla_decode_kv_cache_ragged: Args input_row_offsets; Parameters
// mask_str, local_window_size).  The argument block A provides offsets, cache_lens, B,
// T, PS, max_pages, mask, window and the device error word err.
#pragma once

#include "mla_device.h"
#include "mla_plan.h"

namespace mla {

// Visible keys [lo, hi) of query token j of the n tokens of a sequence with L cache rows.
template <class A>
__device__ __forceinline__ void token_range(const A& a, long long L, int n, int j, int& lo, int& hi) {
  if (a.mask == kMaskNull) {
    lo = 0;
    hi = (int)L;
    return;
  }
  const long long pos = L - n + j;
  long long h = pos + 1 < L ? pos + 1 : L;
  if (h < 0) h = 0;
  long long l = 0;
  if (a.mask == kMaskSliding) {
    l = pos - a.window + 1;
    if (l < 0) l = 0;
    if (l > h) l = h;
  }
  lo = (int)l;
  hi = (int)h;
}

template <class A>
__device__ __forceinline__ long long clamp_len(const A& a, long long L, bool report) {
  const long long Lmax = (long long)a.max_pages * a.PS;
  if (L > Lmax) {
    if (report) atomicOr(a.err, kErrCacheLen);
    L = Lmax;
  }
  return L < 0 ? 0 : L;
}

// Geometry of one query row found by binary search of its sequence in the offsets (used
// only for batches with more rows than the planning table holds).
template <class A>
__device__ __forceinline__ RowGeo decode_row_geo(const A& a, int t) {
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int)ld_const(a.offsets + mid) <= t) lo = mid; else hi = mid;
  }
  RowGeo g{lo, 0, 0};
  const int o0 = (int)ld_const(a.offsets + lo), o1 = (int)ld_const(a.offsets + lo + 1);
  const int n = o1 - o0, j = t - o0;
  if (j < 0 || j >= n) {
    g.b = -1;
    return g;
  }
  token_range(a, clamp_len(a, ld_const(a.cache_lens + lo), false), n, j, g.lo, g.hi);
  return g;
}

// Planning table: one thread per sequence writes the geometry of its query rows.
template <int NT, class A>
__device__ __forceinline__ void decode_fill(const A& a, PlanLds& L) {
  for (int t = threadIdx.x; t < a.T; t += NT) L.geo[t] = RowGeo{-1, 0, 0};
  __syncthreads();
  for (int b = threadIdx.x; b < a.B; b += NT) {
    const int o0 = (int)a.offsets[b], o1 = (int)a.offsets[b + 1];
    const long long L0 = a.cache_lens[b];
    if (o1 < o0 || o0 < 0 || o1 > a.T) {
      atomicOr(a.err, kErrOffsets);
      continue;
    }
    const long long Lb = clamp_len(a, L0, true);
    const int n = o1 - o0;
    for (int j = 0; j < n; ++j) {
      RowGeo g{b, 0, 0};
      token_range(a, Lb, n, j, g.lo, g.hi);
      L.geo[o0 + j] = g;
    }
  }
}

// The same geometry written by one wave into its private 64-row table (at most 64 rows and
// 64 sequences): lane b writes the rows of sequence b.
template <class A>
__device__ __forceinline__ void decode_fill_wave(const A& a, RowGeo* geo, int lane) {
  if (lane < a.T) geo[lane] = RowGeo{-1, 0, 0};
  if (lane < a.B) {
    const int o0 = (int)a.offsets[lane], o1 = (int)a.offsets[lane + 1];
    const long long L0 = a.cache_lens[lane];
    if (o1 < o0 || o0 < 0 || o1 > a.T) {
      atomicOr(a.err, kErrOffsets);
    } else {
      const long long Lb = clamp_len(a, L0, true);
      const int n = o1 - o0;
      for (int j = 0; j < n; ++j) {
        RowGeo g{lane, 0, 0};
        token_range(a, Lb, n, j, g.lo, g.hi);
        geo[o0 + j] = g;
      }
    }
  }
}

}  // namespace mla
