// Work split of the decode kernels over the GPU, shared by the dense and sparse paths.
//
// Every query row's visible keys are cut into 64-key tiles.  Balanced mode: each
// work-group computes the per-row tile counts itself (no host round trip), takes an equal
// run of the concatenated tiles and walks the rows that run touches.  Rows it covers
// completely are written straight to the output; the at most two rows it covers in part
// leave a normalised partial output and its log2-sum-exp in slot 2*gid (the row holding
// the run's first tile) or 2*gid + 1 (the row holding its last tile).  Fixed mode
// (num_partitions = P): work-group gid = (row, part) takes the part-th of P equal tile
// ranges of its row and uses slot gid.
//
// Row geometry (sequence, visible key range) is gathered once per work-group into an LDS
// table by a kernel-specific `fill` step, so the planning costs one round of independent
// global loads rather than chains of dependent ones.
#pragma once

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

struct RowGeo {
  int b;   // sequence (dense) or row (sparse); -1 for a malformed row
  int lo;  // first visible key (or list entry)
  int hi;  // one past the last
};

__device__ __forceinline__ int geo_tiles(const RowGeo& g) {
  return g.hi > g.lo ? (g.hi - 1) / kTileKeys - g.lo / kTileKeys + 1 : 0;
}

constexpr int kPlanMaxRows = 512;  // rows whose geometry the LDS table holds

struct PlanLds {
  RowGeo geo[kPlanMaxRows];
  int scan[1024];
  int found[2];
  int zero[64];  // rows to clear found by this work-group, and their count in zero[63]
};

// Block scan over one chunk: returns the inclusive prefix, sets the chunk total.
template <int NT>
__device__ __forceinline__ int plan_chunk_scan(int v, int* buf, int& chunk_total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < NT; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  chunk_total = buf[NT - 1];
  __syncthreads();
  return incl;
}

// Zero the output row t (rows with no visible key).
template <int NT>
__device__ void plan_zero_row(const SplitPlan& p, int t) {
  const int n16 = p.H * (kLatentDim / 8);
  for (int c = threadIdx.x; c < n16; c += NT) {
    const int h = c / (kLatentDim / 8), c8 = c % (kLatentDim / 8);
    *(uint4*)(p.out + (int64_t)t * p.o_tok + (int64_t)h * p.o_head + c8 * 8) = make_uint4(0, 0, 0, 0);
  }
}

// Runs this work-group's share.
//   fill(L)          block-cooperatively writes L.geo[t] for every row t < p.T (only called
//                    when p.T <= kPlanMaxRows), followed by a block barrier inside plan_run;
//   geo_of(t)        the geometry of one row computed directly (used when p.T is larger);
//   segment(r, g, ta, tc, full, slot) processes tiles [ta, tc) of row r.
template <int NT, class Fill, class GeoOf, class Segment>
__device__ __forceinline__ void plan_run(const SplitPlan& p, PlanLds& L, Fill fill, GeoOf geo_of,
                                         Segment segment) {
  const int gid = blockIdx.x;
  const bool table = p.T <= kPlanMaxRows;
  if (table) {
    fill(L);
    __syncthreads();
  }
  auto row_geo = [&](int t) { return table ? L.geo[t] : geo_of(t); };

  // This work-group's share is the tile run [s, e) of the concatenated rows; r0 is the
  // first row it touches and pre that row's first tile.
  int s = 0, e = 0, r0 = -1, pre = 0;
  if (p.nparts >= 1) {
    const int P = p.nparts;
    const int t = gid / P, part = gid - t * P;
    if (t >= p.T) return;
    const int nt = geo_tiles(row_geo(t));
    const int ta = (int)((long long)part * nt / P), tc = (int)((long long)(part + 1) * nt / P);
    if (ta == tc) {
      if (P == 1) {
        plan_zero_row<NT>(p, t);
      } else {
        for (int h = threadIdx.x; h < p.H; h += NT) p.part_lse[(int64_t)gid * p.H + h] = -INFINITY;
      }
      return;
    }
    r0 = t;  // a run within a single row
    s = ta;
    e = tc;
  } else {
    // per-row tile counts, prefix sums, the row holding tile s (and, for work-group 0,
    // every row's tile range, which the combine kernel reads)
    if (threadIdx.x == 0) {
      L.found[0] = -1;
      L.found[1] = 0;
      L.zero[63] = 0;
    }
    __syncthreads();
    int total = 0;
    if (!table) {
      for (int base = 0; base < p.T; base += NT) {
        const int t = base + threadIdx.x;
        int ctot;
        plan_chunk_scan<NT>(t < p.T ? geo_tiles(geo_of(t)) : 0, L.scan, ctot);
        total += ctot;
      }
    } else {
      for (int t = threadIdx.x; t < p.T; t += NT) total += geo_tiles(L.geo[t]);
      int ctot;
      plan_chunk_scan<NT>(total, L.scan, ctot);
      total = ctot;
    }
    total = __builtin_amdgcn_readfirstlane(total);
    const int W = (total + p.grid - 1) / p.grid;
    s = gid * W;
    e = min(total, s + W);
    if (gid == 0 && threadIdx.x == 0) {
      p.row_meta[0] = total;
      p.row_meta[1] = W;
    }
    int prefix = 0;
    for (int base = 0; base < p.T; base += NT) {
      const int t = base + threadIdx.x;
      const int v = t < p.T ? geo_tiles(row_geo(t)) : 0;
      int ctot;
      const int incl = plan_chunk_scan<NT>(v, L.scan, ctot);
      const int excl = prefix + incl - v;
      if (t < p.T) {
        if (gid == 0) {
          p.row_meta[2 + 2 * t] = excl;
          p.row_meta[3 + 2 * t] = v;
        }
        if (v > 0 && excl <= s && s < excl + v) {
          L.found[0] = t;
          L.found[1] = excl;
        }
        if (v == 0 && t % p.grid == gid) {
          const int slot = atomicAdd(&L.zero[63], 1);
          if (slot < 63) L.zero[slot] = t;
        }
      }
      prefix += ctot;
    }
    __syncthreads();
    // block-uniform values: keep the row walk in scalar registers
    r0 = __builtin_amdgcn_readfirstlane(L.found[0]);
    pre = __builtin_amdgcn_readfirstlane(L.found[1]);
    // rows without visible keys are written as zeros, spread over the work-groups
    const int nzero = __builtin_amdgcn_readfirstlane(L.zero[63]);
    if (nzero <= 63) {
      for (int i = 0; i < nzero; ++i) plan_zero_row<NT>(p, __builtin_amdgcn_readfirstlane(L.zero[i]));
    } else {
      for (int t = gid; t < p.T; t += p.grid)
        if (geo_tiles(row_geo(t)) == 0) plan_zero_row<NT>(p, t);
    }
    if (s >= e || r0 < 0) return;
  }
  // one call site for the segment work, whatever the mode
  const bool fixed = p.nparts >= 1;
  for (int r = r0; r < p.T && pre < e; ++r) {
    RowGeo g = row_geo(r);
    g.b = __builtin_amdgcn_readfirstlane(g.b);
    g.lo = __builtin_amdgcn_readfirstlane(g.lo);
    g.hi = __builtin_amdgcn_readfirstlane(g.hi);
    const int nt = geo_tiles(g);
    if (nt == 0) continue;
    const int run_end = fixed ? nt : pre + nt;
    const int ta = fixed ? s : max(s, pre) - pre;
    const int tc = fixed ? e : min(e, run_end) - pre;
    const bool full = fixed ? p.nparts == 1 : (ta == 0 && tc == nt);
    const int slot = fixed ? gid : (pre <= s ? 2 * gid : 2 * gid + 1);
    segment(r, g, ta, tc, full, slot);
    if (fixed) break;
    pre += nt;
  }
}

}  // namespace mla
