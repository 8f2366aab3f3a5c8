// Row geometry of paged decode rows, shared by the dense decode and the dense fp8 path
// of the gathered-row kernel, and of the sparse decode's index lists.
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

// Row t's list positions [0, n): its first min(topk[t], shape[1] of d_indices) entries,
// then (EXT with a second stream) the first min(xtopk[t], its width) entries of its second
// list.
__device__ __forceinline__ int sparse_main_len(const SparseArgs& a, int t) {
  return max(0, min(ld_const(a.topk + t), a.idx_cols));
}
template <bool XTRA>
__device__ __forceinline__ int sparse_len(const SparseArgs& a, int t) {
  int n = sparse_main_len(a, t);
  if (XTRA && a.xidx != nullptr) n += max(0, min(ld_const(a.xtopk + t), a.xidx_cols));
  return n;
}
// Row geometry: b = the row of d_indices / topk_lengths that query row t reads -- t itself,
// or with shared lists (generic_flare_mla_decode_kv_cache_ragged, Parameters
// fold_shared_index) the sequence of t in the input_row_offsets (-1 with no visible entry
// for a row outside them) -- and the list positions [0, n).
template <bool XTRA>
__device__ __forceinline__ RowGeo sparse_row_geo(const SparseArgs& a, int t) {
  if (!a.shared) return RowGeo{t, 0, sparse_len<XTRA>(a, t)};
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int)ld_const(a.offsets + mid) <= t) lo = mid; else hi = mid;
  }
  const int o0 = (int)ld_const(a.offsets + lo), o1 = (int)ld_const(a.offsets + lo + 1);
  if (t < o0 || t >= o1) return RowGeo{-1, 0, 0};
  return RowGeo{lo, 0, sparse_main_len(a, lo)};
}

// Shared lists: sequence b (one thread or lane per sequence) writes the geometry of its
// query rows; malformed offsets set kErrOffsets and leave their rows empty.
__device__ __forceinline__ void sparse_fill_seq(const SparseArgs& a, RowGeo* geo, int b) {
  const int o0 = (int)a.offsets[b], o1 = (int)a.offsets[b + 1];
  if (o1 < o0 || o0 < 0 || o1 > a.T) {
    atomicOr(a.err, kErrOffsets);
    return;
  }
  const int n = sparse_main_len(a, b);
  for (int t = o0; t < o1; ++t) geo[t] = RowGeo{b, 0, n};
}

// The same for one wave's private 64-row table (at most 64 rows and sequences): lane t
// writes row t, or with shared lists lane b the rows of sequence b.
template <bool XTRA>
__device__ __forceinline__ void sparse_fill_wave(const SparseArgs& a, RowGeo* geo, int lane) {
  if (!a.shared) {
    if (lane < a.T) geo[lane] = RowGeo{lane, 0, sparse_len<XTRA>(a, lane)};
  } else {
    if (lane < a.T) geo[lane] = RowGeo{-1, 0, 0};
    if (lane < a.B) sparse_fill_seq(a, geo, lane);
  }
}


}  // namespace mla
