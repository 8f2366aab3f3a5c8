// Work split of the decode kernels over the GPU, shared by the dense and sparse paths.
//
// Every query row's visible keys are cut into 32-key tiles (one stage each).  Each work-group computes the
// per-row tile counts itself (no host round trip).  Three modes:
//   row parts (balanced, when every non-empty row can have a work-group of its own): with
//     S the smallest tile count such that sum_t ceil(nt_t / S) <= grid, row t is cut into
//     P_t = ceil(nt_t / S) near-equal parts, numbered in row order; a work-group takes one
//     part, so it runs one segment with one prologue and one epilogue.  A row in
//     several parts leaves each part's normalised output and log2-sum-exp in the slot of
//     the part's number;
//   stream (balanced, many rows): the concatenated tiles are cut into equal runs; a
//     work-group walks the rows its run touches, writing rows it covers completely and
//     leaving the at most two it covers in part in slot 2*r (the row of run r's first
//     tile) or 2*r + 1 (the row of its last tile);
//   fixed (num_partitions = P): piece t * P + part takes the part-th of P equal tile
//     ranges of row t and uses that slot.
// Pieces are dealt to work-groups by plan_piece.
// Work-group 0 publishes every row's split in row_meta for the combine kernel, which
// merges the parts of split rows by their log2-sum-exps: [0] = mode (0 stream, 1 row
// parts), [1] = tiles per run (stream) or per part (row parts), then per row the pair
// (a, b) of its RowSplit.  Fixed mode needs no table.
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
  int scan[1024];   // planning scratch; reused afterwards as the segments' page-id window
  int found[2];
  int zero[64];  // rows to clear found by this work-group, and their count in zero[63]
  int red[68];   // block sums of the row-parts search, then its row count / total / max
};

// Sum / max over the wave, left in every lane, without LDS traffic: DPP moves combine lane
// pairs (quad_perm 1,0,3,2 and 2,3,0,1), then mirrored halves of 8 and 16 lanes, and the
// gfx950 lane swaps combine the four rows.  Block totals then take one LDS atomic per wave
// (many lanes updating one LDS word serialise).
template <bool MAX>
__device__ __forceinline__ int wave_reduce_i32(int v) {
  auto op = [](int x, int y) { return MAX ? max(x, y) : x + y; };
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  v = op((int)h[0], (int)h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  return op((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int wave_sum_i32(int v) { return wave_reduce_i32<false>(v); }
__device__ __forceinline__ int wave_max_i32(int v) { return wave_reduce_i32<true>(v); }

// Block scan over one chunk of NT values: returns the inclusive prefix, sets the chunk
// total.  Each wave scans its 64 values with lane shifts; wave totals meet in buf.
template <int NT>
__device__ __forceinline__ int plan_chunk_scan(int v, int* buf, int& chunk_total) {
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(v, off);
    if (lane >= off) v += up;
  }
  if (lane == 63) buf[wave] = v;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const int x = buf[w];
    before += w < wave ? x : 0;
    total += x;
  }
  chunk_total = total;
  __syncthreads();  // buf is reused by the next call
  return before + v;
}

// The piece (part, run or fixed part) work-group gid takes.  Pieces are numbered so that
// consecutive ones -- the parts of one row -- go to work-groups that the dispatcher places
// on the same XCD (work-groups are dealt to the eight XCDs round-robin), where they share
// that XCD's L2 for the row's query and page table.  Only the speed depends on this.
__device__ __forceinline__ int plan_piece(int gid, int nwg) {
  if (nwg % 8 != 0) return gid;
  return (gid & 7) * (nwg >> 3) + (gid >> 3);
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

// Where the parts of a split row are (shared with the combine kernel).
struct RowSplit {
  int mode;  // 0 stream: a = the row's first tile in the concatenation, b = tiles per run
             // 1 row parts: a = slot of part 0, b = parts;  2 fixed: a = t * P, b = P
  int a, b;
};

__device__ __forceinline__ int split_count(const RowSplit& rs, int nt) {
  return rs.mode == 0 ? (rs.a + nt - 1) / rs.b - rs.a / rs.b + 1 : rs.b;
}

// The split of row t as the combine kernel sees it; n = 0 when there is nothing to merge.
__device__ __forceinline__ RowSplit row_split(const SplitPlan& p, int t, int& n) {
  if (p.nparts >= 1) {
    n = p.nparts > 1 ? p.nparts : 0;
    return RowSplit{2, t * p.nparts, p.nparts};
  }
  const int mode = p.row_meta[0];
  const RowSplit rs{mode, p.row_meta[2 + 2 * t], mode == 0 ? p.row_meta[1] : p.row_meta[3 + 2 * t]};
  if (mode == 1) {
    n = rs.b > 1 ? rs.b : 0;  // one part: written whole
  } else {
    const int nt = p.row_meta[3 + 2 * t];
    n = nt > 0 && rs.b > 0 ? split_count(rs, nt) : 0;
    if (n == 1) n = 0;  // one run covered the whole row and wrote it
  }
  return rs;
}

// slot of the row's c-th part
__device__ __forceinline__ int split_slot(const RowSplit& rs, int c) {
  if (rs.mode == 0) {
    const int c0 = rs.a / rs.b;  // first run touching the row
    // in run c0 the row holds the run's first tile only if it starts exactly there
    return c == 0 ? (rs.a == c0 * rs.b ? 2 * c0 : 2 * c0 + 1) : 2 * (c0 + c);
  }
  return rs.a + c;
}

// Row-parts planning (see the mode list above), for a batch whose row geometry is in the
// LDS table.  Returns false (before touching any output) when there are more non-empty
// rows than work-groups or no visible key at all; otherwise sets this work-group's tile
// range [s, e) of row r0 (r0 = -1: no part for it), pre = -1, writes row_meta (work-group
// 0) and clears the rows without keys that fall to this work-group.
template <int NT>
__device__ __forceinline__ bool plan_row_parts(const SplitPlan& p, PlanLds& L, int piece, int& s, int& e, int& r0,
                                               int& pre) {
  const int gid = blockIdx.x, tid = threadIdx.x;
  constexpr int kRows = 64;  // red[64..66]: rows with keys, total tiles, largest row
  for (int i = tid; i < 68; i += NT) L.red[i] = 0;
  __syncthreads();
  {
    int rows = 0, total = 0, mx = 0;
    for (int t = tid; t < p.T; t += NT) {
      const int nt = geo_tiles(L.geo[t]);
      rows += nt > 0;
      total += nt;
      mx = max(mx, nt);
    }
    rows = wave_sum_i32(rows);
    total = wave_sum_i32(total);
    mx = wave_max_i32(mx);
    if ((tid & 63) == 0) {
      atomicAdd(&L.red[kRows], rows);
      atomicAdd(&L.red[kRows + 1], total);
      atomicMax(&L.red[kRows + 2], mx);
    }
  }
  __syncthreads();
  const int rows = __builtin_amdgcn_readfirstlane(L.red[kRows]);
  const int total = __builtin_amdgcn_readfirstlane(L.red[kRows + 1]);
  const int maxnt = __builtin_amdgcn_readfirstlane(L.red[kRows + 2]);
  if (rows == 0 || rows > p.grid) return false;

  // Smallest S with sum_t ceil(nt_t / S) <= grid.  It lies in [ceil(total / grid), hi]:
  // every row rounds up by less than one part, so S >= total / (grid - rows) fits, and
  // S = maxnt (one part per row) always fits.  One pass tests the first eight candidates
  // together (one block sum each); a binary search covers a wider bracket.
  const int S0 = max(1, (total + p.grid - 1) / p.grid);
  const int hi = rows < p.grid ? min(maxnt, (total + (p.grid - rows) - 1) / (p.grid - rows)) : maxnt;
  int S = hi;
  {
    // each wave sums its own candidates over all rows (lane = row), so every lane divides
    // by 8 / waves candidates only and no LDS atomics are needed
    constexpr int kWaves = NT / 64;
    constexpr int kPer = kWaves >= 8 ? 1 : 8 / kWaves;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int c[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) c[j] = 0;
    for (int t = tid & 63; t < p.T; t += 64) {
      const int nt = geo_tiles(L.geo[t]);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int Sx = S0 + wave * kPer + j;
        c[j] += (nt + Sx - 1) / Sx;
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      c[j] = wave_sum_i32(c[j]);
      if ((tid & 63) == 0 && wave * kPer + j < 8) L.red[wave * kPer + j] = c[j];
    }
    __syncthreads();
#pragma unroll
    for (int k = 7; k >= 0; --k)
      if (S0 + k <= hi && __builtin_amdgcn_readfirstlane(L.red[k]) <= p.grid) S = S0 + k;
  }
  if (S == hi && S0 + 8 < hi) {
    int trial = 8;  // counters red[8..63]
    auto parts_fit = [&](int Sx) {
      int c = 0;
      for (int t = tid; t < p.T; t += NT) c += (geo_tiles(L.geo[t]) + Sx - 1) / Sx;
      c = wave_sum_i32(c);
      if ((tid & 63) == 0) atomicAdd(&L.red[trial], c);
      __syncthreads();
      const int sum = __builtin_amdgcn_readfirstlane(L.red[trial]);
      ++trial;
      return sum <= p.grid;
    };
    int lo = S0 + 7, up = hi;  // lo fails, up fits
    while (up - lo > 1) {
      const int mid = lo + (up - lo) / 2;
      if (parts_fit(mid)) up = mid; else lo = mid;
    }
    S = up;
  }

  // parts per row, their numbering, this work-group's part, rows to clear
  if (tid == 0) {
    L.found[0] = -1;
    L.found[1] = 0;
    L.zero[63] = 0;
  }
  __syncthreads();
  int prefix = 0;
  for (int base = 0; base < p.T; base += NT) {
    const int t = base + tid;
    const int nt = t < p.T ? geo_tiles(L.geo[t]) : 0;
    const int P = (nt + S - 1) / S;
    int ctot;
    const int incl = plan_chunk_scan<NT>(P, L.scan, ctot);
    const int first = prefix + incl - P;
    if (t < p.T) {
      if (gid == 0) {
        p.row_meta[2 + 2 * t] = first;
        p.row_meta[3 + 2 * t] = P;
      }
      if (P > 0 && first <= piece && piece < first + P) {
        L.found[0] = t;
        L.found[1] = piece - first;
      }
      if (nt == 0 && t % p.grid == gid) {
        const int slot = atomicAdd(&L.zero[63], 1);
        if (slot < 63) L.zero[slot] = t;
      }
    }
    prefix += ctot;
  }
  if (gid == 0 && tid == 0) {
    p.row_meta[0] = 1;  // row-parts mode
    p.row_meta[1] = S;
  }
  __syncthreads();
  const int nzero = __builtin_amdgcn_readfirstlane(L.zero[63]);
  if (nzero <= 63) {
    for (int i = 0; i < nzero; ++i) plan_zero_row<NT>(p, __builtin_amdgcn_readfirstlane(L.zero[i]));
  } else {
    for (int t = gid; t < p.T; t += p.grid)
      if (geo_tiles(L.geo[t]) == 0) plan_zero_row<NT>(p, t);
  }
  r0 = __builtin_amdgcn_readfirstlane(L.found[0]);
  pre = -1;
  if (r0 >= 0) {
    const int part = __builtin_amdgcn_readfirstlane(L.found[1]);
    const int nt = geo_tiles(L.geo[r0]);
    const int P = (nt + S - 1) / S;
    s = (int)((long long)part * nt / P);
    e = (int)((long long)(part + 1) * nt / P);
  }
  return true;
}

// Row-parts planning of a small batch (T <= 64 rows, T <= grid) done by every wave on its
// own: lane t holds row t, so the row sums, the split-size search and the prefix of the
// part counts are wave reductions and a wave scan, with no block barrier.  fill_wave(geo,
// lane) writes rows 0..T-1 of the wave's private table geo (64 entries).  The result is
// the plan plan_row_parts makes (the smallest S that fits, parts numbered in row order);
// a batch without any visible key gets no parts (every row is written as zeros).
template <int NT, class PL, class FillWave>
__device__ __forceinline__ void plan_row_parts_small(const SplitPlan& p, PL& L, int piece, FillWave fill_wave,
                                                     RowGeo& g0, int& s, int& e, int& r0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  RowGeo* wgeo = L.geo + 64 * wave;
  fill_wave(wgeo, lane);
  const RowGeo g = lane < p.T ? wgeo[lane] : RowGeo{-1, 0, 0};
  const int nt = geo_tiles(g);
  const int rows = wave_sum_i32(nt > 0 ? 1 : 0), total = wave_sum_i32(nt), maxnt = wave_max_i32(nt);
  // smallest S in [S0, hi] with sum_t ceil(nt_t / S) <= grid (S0 - 1 never fits, hi does)
  int S = 1;
  if (rows > 0) {
    const int S0 = max(1, (total + p.grid - 1) / p.grid);
    const int hi = rows < p.grid ? min(maxnt, (total + (p.grid - rows) - 1) / (p.grid - rows)) : maxnt;
    int lo = S0 - 1, up = hi;
    while (up - lo > 1) {
      const int mid = lo + (up - lo) / 2;
      if (wave_sum_i32((nt + mid - 1) / mid) <= p.grid) up = mid; else lo = mid;
    }
    S = up;
  }
  const int P = (nt + S - 1) / S;
  int incl = P;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  const int first = incl - P;
  if (blockIdx.x == 0 && wave == 0 && lane < p.T) {
    p.row_meta[2 + 2 * lane] = first;
    p.row_meta[3 + 2 * lane] = P;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    p.row_meta[0] = 1;  // row-parts mode
    p.row_meta[1] = S;
  }
  // rows without keys that fall to this work-group (every wave finds the same ones)
  uint64_t zero = __builtin_amdgcn_ballot_w64(lane < p.T && nt == 0 && lane % p.grid == (int)blockIdx.x);
  while (zero != 0) {
    const int t = __builtin_ctzll(zero);
    zero &= zero - 1;
    plan_zero_row<NT>(p, t);
  }
  const uint64_t mine = __builtin_amdgcn_ballot_w64(P > 0 && first <= piece && piece < first + P);
  r0 = -1;
  if (mine == 0) return;
  r0 = __builtin_ctzll(mine);
  const int part = piece - __builtin_amdgcn_readlane(first, r0);
  const int Pr = __builtin_amdgcn_readlane(P, r0), ntr = __builtin_amdgcn_readlane(nt, r0);
  s = (int)((long long)part * ntr / Pr);
  e = (int)((long long)(part + 1) * ntr / Pr);
  g0 = RowGeo{__builtin_amdgcn_readlane(g.b, r0), __builtin_amdgcn_readlane(g.lo, r0),
              __builtin_amdgcn_readlane(g.hi, r0)};
}

// Runs this work-group's share.
//   fill(L)          block-cooperatively writes L.geo[t] for every row t < p.T (only called
//                    when p.T <= kPlanMaxRows), followed by a block barrier inside plan_run;
//   geo_of(t)        the geometry of one row computed directly (used when p.T is larger);
//   fill_wave        (SMALL) writes one wave's private row table, see plan_row_parts_small;
//   segment(r, g, ta, tc, full, slot) processes tiles [ta, tc) of row r.
// SMALL (chosen by the host for balanced batches of at most 64 rows and 64 sequences, no
// more rows than work-groups) plans per wave and has a single segment call site: the
// general planner is not compiled in, which keeps the stage loop's registers free.
// PL: the kernel's LDS planning block (PlanLds, or with SMALL any block whose geo array
// holds 64 rows per wave).
template <int NT, bool SMALL, class PL, class Fill, class GeoOf, class FillWave, class Segment>
__device__ __forceinline__ void plan_run(const SplitPlan& p, PL& L, Fill fill, GeoOf geo_of, FillWave fill_wave,
                                         Segment segment) {
  const int gid = blockIdx.x;
  const int piece = plan_piece(gid, (int)gridDim.x);
  if constexpr (SMALL) {
    RowGeo g0{0, 0, 0};
    int s0 = 0, e0 = 0, r = -1;
    plan_row_parts_small<NT>(p, L, piece, fill_wave, g0, s0, e0, r);
    if (r >= 0) {
      g0.b = __builtin_amdgcn_readfirstlane(g0.b);
      g0.lo = __builtin_amdgcn_readfirstlane(g0.lo);
      g0.hi = __builtin_amdgcn_readfirstlane(g0.hi);
      segment(r, g0, s0, e0, geo_tiles(g0) == e0 - s0, piece);
    }
    return;
  } else {
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
      const int t = piece / P, part = piece - t * P;
      if (t >= p.T) return;
      const int nt = geo_tiles(row_geo(t));
      const int ta = (int)((long long)part * nt / P), tc = (int)((long long)(part + 1) * nt / P);
      if (ta == tc) {
        if (P == 1) {
          plan_zero_row<NT>(p, t);
        } else {
          for (int h = threadIdx.x; h < p.H; h += NT) p.part_lse[(int64_t)piece * p.H + h] = -INFINITY;
        }
        return;
      }
      r0 = t;  // a run within a single row
      s = ta;
      e = tc;
    } else if (table && plan_row_parts<NT>(p, L, piece, s, e, r0, pre)) {
      // row parts: one segment (or none) per work-group
      if (r0 < 0) return;
    } else {
      // per-row tile counts, prefix sums, the row holding tile s
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
      s = piece * W;
      e = min(total, s + W);
      if (gid == 0 && threadIdx.x == 0) {
        p.row_meta[0] = 0;  // stream mode
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
    // one call site for the segment work, whatever the mode.  Fixed and row-parts modes
    // (pre < 0) run the single tile range [s, e) of row r0 and use slot `piece`.
    const bool fixed = p.nparts >= 1 || pre < 0;
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
      const bool full = p.nparts >= 1 ? p.nparts == 1 : (ta == 0 && tc == nt);
      const int slot = fixed ? piece : (pre <= s ? 2 * piece : 2 * piece + 1);
      segment(r, g, ta, tc, full, slot);
      if (fixed) break;
      pre += nt;
    }
  }
}

}  // namespace mla
