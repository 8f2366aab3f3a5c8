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
//   score:  one work-group per (token, slice of kIdxSlice visible rows) computes each
//           row's 64-bit key (order-preserving score bits, then the inverted position, so
//           every key is distinct) and writes the slice's keys to its part of the token's
//           workspace row grouped by top 8-bit digit, digits descending (a counting sort
//           in LDS), with the size and start of each digit's run;
//   select: one work-group of 1024 threads per token.  The slices' run tables give the
//           threshold's top digit directly; the runs above it are listed and the runs of
//           it are loaded into LDS (the runs below are never read).  A radix select over
//           those keys (8-bit digits, histograms in LDS) follows until all keys of the
//           threshold's bin are needed.  The listed keys are then ordered without a sort
//           network: kIdxBuckets buckets of equal key width between the threshold and
//           the top of the highest non-empty digit, a scan of the bucket counts, and
//           within a bucket a count of the larger keys give each key its output slot.
#include <stdint.h>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

constexpr int kIdxThreads = 256;      // scoring work-group
constexpr int kIdxSelThreads = 1024;  // selection work-group
constexpr int kIdxHistCopies = 4;     // copies of each digit counter in the scoring kernel
constexpr int kFoldHeads = 8;         // heads per fold thread whose q loads go out before the rows
constexpr int kIdxBucketBits = 11;    // buckets of the listing order
constexpr int kIdxBuckets = 1 << kIdxBucketBits;
static_assert(kIdxBuckets % kIdxSelThreads == 0 && kIdxMaxTopK <= kIdxMaxKeys && kIdxMaxTopK % kIdxSelThreads == 0,
              "bucket scan, grouped keys, listed keys per thread");
static_assert(kIdxThreads == 256 && (256 * kIdxHistCopies) % (4 * kIdxThreads) == 0, "one scoring thread per digit");
static_assert(kIdxMaxKeys / kIdxSlice <= kIdxSelThreads / 64, "one selecting wave per key slice");

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

// The token's sequence and its visible rows [vlo, vhi).  The sequence is the last b < B
// with offsets[b] <= t: each lane of a wave tests one offset and a ballot counts them, 64
// offsets per round (non-decreasing offsets; others are caught by the range check below).
// Lane i also loads sequence i's offsets and length, so a batch of at most 64 sequences
// costs one load round trip.
struct TokenRows {
  int b, vlo, vhi;
};

__device__ __forceinline__ TokenRows token_rows(const IndexerArgs& a, int t, bool report) {
  const int lane = (int)(threadIdx.x & 63);
  int below = 0;  // offsets[0 .. B) at or below t
  // lane i also loads sequence i's end offset and length, for a batch of at most 64
  const int i0 = min(lane, a.B - 1);
  const uint32_t own0 = a.offsets[i0], own1 = a.offsets[i0 + 1];
  const int32_t own_len = a.cache_lens[i0];
  for (int base = 0; base < a.B; base += 64) {  // wave-uniform
    const int i = base + lane;
    const uint32_t oi = base == 0 ? own0 : a.offsets[min(i, a.B - 1)];
    below += (int)__popcll(__builtin_amdgcn_ballot_w64(i < a.B && (int64_t)oi <= (int64_t)t));
  }
  const int lo_b = __builtin_amdgcn_readfirstlane(max(below - 1, 0));
  TokenRows r{lo_b, 0, 0};
  int o0, o1;
  long long L;
  if (lo_b < 64) {  // wave-uniform
    o0 = (int)__builtin_amdgcn_readlane((int)own0, lo_b);
    o1 = (int)__builtin_amdgcn_readlane((int)own1, lo_b);
    L = __builtin_amdgcn_readlane(own_len, lo_b);
  } else {
    o0 = (int)ld_const(a.offsets + lo_b);
    o1 = (int)ld_const(a.offsets + lo_b + 1);
    L = ld_const(a.cache_lens + lo_b);
  }
  if (t >= o0 && t < o1) {
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
// thread has in flight at once; PRE: q 4-byte aligned with at most kFoldHeads heads per
// fold thread, so the fold's q loads and the first row group go out together.
template <int NC, int RF, bool PRE>
__global__ __launch_bounds__(kIdxThreads) void mla_indexer_score_kernel(const IndexerArgs a) {
  constexpr int R = kIdxSlice / kIdxThreads;  // rows per thread
  static_assert(R % RF == 0, "rows per thread in whole groups");
  __shared__ __align__(16) float qf[kIdxMaxDepth];
  __shared__ __align__(16) float part[4 * kIdxThreads];  // [group][d] partial sums of the fold
  __shared__ __align__(16) int dcnt[256 * kIdxHistCopies];  // [digit][copy]
  __shared__ __align__(16) uint64_t grouped[kIdxSlice];
  __shared__ int wave_sum[kIdxThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const TokenRows tr = token_rows(a, t, blockIdx.y == 0 && tid == 0);
  const int vlo = tr.vlo, nvis = tr.vhi - tr.vlo, b = tr.b;
  const int i0 = blockIdx.y * kIdxSlice, i1 = min(nvis, i0 + kIdxSlice);
  if (i0 >= i1) return;  // block-uniform, before any barrier
#pragma unroll
  for (int u = 0; u < 256 * kIdxHistCopies / (4 * kIdxThreads); ++u)
    *(int4*)&dcnt[4 * (tid + u * kIdxThreads)] = make_int4(0, 0, 0, 0);

  // ---- the page ids of this thread's rows (rows i0 + tid + r * kIdxThreads)
  const int32_t* prow = a.page_table + (int64_t)b * a.pt_row;
  int pid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = i0 + tid + r * kIdxThreads;
    pid[r] = i < i1 ? prow[(vlo + i) / a.PS] : 0;
  }

  // ---- row groups: RF rows of this thread (rows i0 + tid + (r0 + u) * kIdxThreads),
  // their 16-byte chunks loaded at once, then scored into distinct keys
  uint64_t* krow = a.keys + (int64_t)t * a.keys_row;
  bool bad = false;
  uint64_t key[R];  // row i0 + tid + r * kIdxThreads, if below i1
  struct Rows {
    uint4 v[RF][NC];
    bool ok[RF];
    int pos[RF];
    float ks[RF];
  };
  auto load_rows = [&](int r0, Rows& g) {
#pragma unroll
    for (int u = 0; u < RF; ++u) {
      const int i = i0 + tid + (r0 + u) * kIdxThreads;
      g.pos[u] = vlo + i;
      const int lp = g.pos[u] / a.PS, slot = g.pos[u] - lp * a.PS, p = pid[r0 + u];
      g.ok[u] = p >= 0 && (int64_t)p < a.num_pages;
      if (i < i1 && !g.ok[u]) bad = true;
      g.ok[u] = g.ok[u] && i < i1;
      // no branch around the loads (rows that do not count read the zero row, chunks past
      // the width re-read the last one), so the compiler can count them in its waits
      const int64_t pc = g.ok[u] ? p : 0;
      const uint8_t* row = g.ok[u] ? a.k + pc * a.page_bytes + (int64_t)slot * a.depth : a.zero_row;
      const int nc = a.depth >> 4;
#pragma unroll
      for (int c = 0; c < NC; ++c) g.v[u][c] = *(const uint4*)(row + min(c, nc - 1) * 16);
      const float* sp = g.ok[u] && a.k_s ? a.k_s + pc * a.ks_page + slot : (const float*)a.zero_row;
      g.ks[u] = *sp;  // used (or replaced by 1) when the row is scored
    }
  };
  auto score_rows = [&](int r0, const Rows& g) {
#pragma unroll
    for (int u = 0; u < RF; ++u) {
      const int i = i0 + tid + (r0 + u) * kIdxThreads;
      if (i >= i1) continue;
      float s = -INFINITY;
      if (g.ok[u]) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (c * 16 >= a.depth) break;
          const uint32_t w[4] = {g.v[u][c].x, g.v[u][c].y, g.v[u][c].z, g.v[u][c].w};
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
        s = acc * (a.k_s ? g.ks[u] : 1.f);
        if (s != s) s = -INFINITY;  // a NaN score (NaN data) ranks last
      }
      // the score's order bits, then the inverted position (equal scores: lower first)
      key[r0 + u] = ((uint64_t)order_key(s) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)g.pos[u]);
    }
  };
  Rows first;  // the first row group, in flight during the fold

  // ---- heads folded into one float32 query row, qf[d] = sum_h q_s[h] * q[h, d]: G
  // groups of threads, group g summing heads g, g + G, ...; the groups' sums are then
  // added in group order.  With q 4-byte aligned a thread takes 4 consecutive d of each
  // of its heads (one dword load per head); when a thread has at most kFoldHeads heads
  // their loads go out before those of the first row group, so the fold's wait for them
  // does not also wait for the rows (loads complete in issue order).  Otherwise one d, a
  // byte at a time.
  const float* qst = a.q_s + (int64_t)t * a.qs_tok;
  const bool q4 = (((uintptr_t)a.q | (uintptr_t)a.q_tok | (uintptr_t)a.q_head) & 3) == 0;
  const int G = q4 ? kIdxThreads / (a.depth >> 2) : kIdxThreads / a.depth;
  if constexpr (PRE) {  // q 4-byte aligned and NH <= kFoldHeads * G (checked on the host)
    const int C4 = a.depth >> 2;
    const bool active = tid < G * C4;
    const int g = active ? tid / C4 : 0, c = active ? tid - g * C4 : 0;
    const uint8_t* qt = a.q + (int64_t)t * a.q_tok + 4 * c;
    uint32_t qw[kFoldHeads];
    float qw_s[kFoldHeads];
#pragma unroll
    for (int j = 0; j < kFoldHeads; ++j) {  // heads past NH read head NH - 1 with weight 0
      const int h = min(g + j * G, a.NH - 1);
      qw[j] = *(const uint32_t*)(qt + (int64_t)h * a.q_head);
      qw_s[j] = qst[h];
    }
    load_rows(0, first);
    if (active) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kFoldHeads; ++j) {
        float f[4];
        e4m3x4_f32(qw[j], f);
        const float w = g + j * G < a.NH ? qw_s[j] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += w * f[e];
      }
      *(float4*)&part[g * a.depth + 4 * c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  } else if (q4) {
    const int C4 = a.depth >> 2;
    if (tid < G * C4) {
      const int g = tid / C4, c = tid - g * C4;
      const uint8_t* qt = a.q + (int64_t)t * a.q_tok + 4 * c;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int h = g; h < a.NH; h += G) {
        float f[4];
        e4m3x4_f32(*(const uint32_t*)(qt + (int64_t)h * a.q_head), f);
        const float w = qst[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += w * f[e];
      }
      *(float4*)&part[g * a.depth + 4 * c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  } else {
    if (tid < G * a.depth) {
      const int g = tid / a.depth, d = tid - g * a.depth;
      const uint8_t* qt = a.q + (int64_t)t * a.q_tok + d;
      float acc = 0.f;
#pragma unroll 8
      for (int h = g; h < a.NH; h += G) {
        float f[4];
        e4m3x4_f32(qt[(int64_t)h * a.q_head], f);
        acc += qst[h] * f[0];
      }
      part[tid] = acc;
    }
  }
  __syncthreads();
  if (tid < a.depth) {
    float acc = 0.f;
    for (int g = 0; g < G; ++g) acc += part[g * a.depth + tid];
    qf[tid] = acc;
  }
  __syncthreads();
  if constexpr (!PRE) load_rows(0, first);

  // ---- scores of this slice's rows as distinct keys, RF rows in flight
  score_rows(0, first);
#pragma unroll
  for (int r0 = RF; r0 < R; r0 += RF) {
    Rows g;
    load_rows(r0, g);
    score_rows(r0, g);
  }
  if (bad) atomicOr(a.err, kErrPageId);

  // ---- the slice's keys into krow[i0 .. i1) grouped by top digit, digits descending,
  // and the slice's digit counts: a counting sort whose counters have kIdxHistCopies
  // copies per digit, lane l using copy l % kIdxHistCopies (the keys crowd into a few
  // digits, and lanes of one copy share a counter)
  const int copy = lane % kIdxHistCopies;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (i0 + tid + r * kIdxThreads < i1) atomicAdd(&dcnt[(int)(key[r] >> 56) * kIdxHistCopies + copy], 1);
  __syncthreads();
  {
    // thread tid takes digit 255 - tid: its copies' first slots follow the counts of
    // the higher digits (an exclusive scan in thread order) and of its lower copies
    const int d = 255 - tid;
    int c[kIdxHistCopies], tot = 0;
#pragma unroll
    for (int u = 0; u < kIdxHistCopies; u += 4) {
      const int4 v = *(const int4*)&dcnt[d * kIdxHistCopies + u];
      c[u] = v.x;
      c[u + 1] = v.y;
      c[u + 2] = v.z;
      c[u + 3] = v.w;
      tot += v.x + v.y + v.z + v.w;
    }
    int incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int up = __shfl_up(incl, off);
      if (lane >= off) incl += up;
    }
    if (lane == 63) wave_sum[tid >> 6] = incl;
    __syncthreads();
    int first = incl - tot;
    for (int w = 0; w < (tid >> 6); ++w) first += wave_sum[w];
    uint32_t* hs = a.slice_hist + (int64_t)t * a.hist_row + blockIdx.y * 512;
    hs[d] = (uint32_t)tot;          // keys of digit d
    hs[256 + d] = (uint32_t)first;  // keys of higher digits: where digit d's run starts
#pragma unroll
    for (int u = 0; u < kIdxHistCopies; ++u) {
      dcnt[d * kIdxHistCopies + u] = first;
      first += c[u];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (i0 + tid + r * kIdxThreads < i1) grouped[atomicAdd(&dcnt[(int)(key[r] >> 56) * kIdxHistCopies + copy], 1)] = key[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {  // the grouped slice out in whole rows
    const int j = tid + r * kIdxThreads;
    if (i0 + j < i1) krow[i0 + j] = grouped[j];
  }
}

__global__ __launch_bounds__(kIdxSelThreads) void mla_indexer_select_kernel(const IndexerArgs a) {
  constexpr int NSL = kIdxMaxKeys / kIdxSlice;  // key slices at most, one wave each
  __shared__ __align__(16) uint64_t keys[kIdxMaxKeys];
  __shared__ __align__(16) uint64_t grouped[kIdxMaxTopK];
  __shared__ uint32_t bfirst[kIdxBuckets];
  __shared__ __align__(16) int hist[256];
  __shared__ int wave_tot[kIdxSelThreads / 64], slice_above[NSL], slice_equal[NSL];
  __shared__ uint64_t wave_max[kIdxSelThreads / 64], wave_min[kIdxSelThreads / 64];
  __shared__ int sel_digit, sel_count, sel_bin;
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The scoring kernel's run tables (per slice, the size and start of each top digit's
  // run), loaded before the token's rows are known: thread d < 256 takes digit d of every
  // slice the tables hold (slices past the token's last are masked below).
  uint32_t cnt[NSL], st[NSL];
  if (tid < 256) {
    const int nsl_tab = (int)(a.hist_row / 512);
    const uint32_t* hs = a.slice_hist + (int64_t)t * a.hist_row + tid;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int s2 = min(sl, nsl_tab - 1) * 512;
      cnt[sl] = hs[s2];
      st[sl] = hs[s2 + 256];
    }
  }
  const TokenRows tr = token_rows(a, t, false);
  const int nvis = tr.vhi - tr.vlo;
  const uint64_t* krow = a.keys + (int64_t)t * a.keys_row;
  const int nsel = min(a.top_k, nvis);
#pragma unroll
  for (int u = 0; u < kIdxBuckets / kIdxSelThreads; ++u) bfirst[tid + u * kIdxSelThreads] = 0;
  // ---- The listed keys are keys[nw .. nw + nab) and those of keys[0 .. nw) at or above
  // thr, exactly nsel in all; lo <= each listed key <= hi.
  int nw, nab;
  uint64_t thr, lo, hi;
  if (nsel == nvis) {  // block-uniform: every visible row is listed
    uint64_t mx = 0, mn = ~0ull;
    for (int i = tid; i < nvis; i += kIdxSelThreads) {
      const uint64_t k = krow[i];
      keys[i] = k;
      mx = max(mx, k);
      mn = min(mn, k);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mx = max(mx, (uint64_t)__shfl_xor((unsigned long long)mx, off));
      mn = min(mn, (uint64_t)__shfl_xor((unsigned long long)mn, off));
    }
    if (lane == 0) {
      wave_max[wave] = mx;
      wave_min[wave] = mn;
    }
    __syncthreads();
    hi = 0;
    lo = ~0ull;
    for (int w = 0; w < kIdxSelThreads / 64; ++w) {
      hi = max(hi, wave_max[w]);
      lo = min(lo, wave_min[w]);
    }
    if (nvis == 0) lo = hi = 0;
    nw = 0;
    nab = nvis;
    thr = 0;
  } else {
    // A radix select (8-bit digits, most significant first) finds the threshold:
    // `prefix` holds its digits found so far, `need` how many keys at or above it are
    // still to be listed.
    //
    // First digit, from the run tables.  Thread d < 256 sums digit d over the slices: A
    // keys above it, H of it.  The digit where A < nsel <= A + H is the threshold's.  The
    // highest digit with keys bounds them all from above.
    const int nsl = (nvis + kIdxSlice - 1) / kIdxSlice;  // 1 .. NSL
    if (tid < 256) {
      hist[tid] = 0;
      int A = 0, H = 0;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
        if (sl < nsl) {
          A += (int)st[sl];
          H += (int)cnt[sl];
        }
      if (A < nsel && nsel <= A + H) {  // exactly one digit (distinct keys, 0 < nsel < nvis)
        sel_digit = tid;
        sel_count = nsel - A;
        sel_bin = H;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
          if (sl < nsl) {
            slice_above[sl] = (int)st[sl];
            slice_equal[sl] = (int)cnt[sl];
          }
      }
      const uint64_t nz = __builtin_amdgcn_ballot_w64(H > 0);
      if (lane == 0) wave_tot[wave] = nz ? wave * 64 + 63 - __clzll(nz) : -1;
    }
    __syncthreads();
    uint64_t prefix = (uint64_t)sel_digit << 56;
    int need = sel_count;
    nw = sel_bin;  // keys[0 .. nw): the keys of the first digit
    const int dmax = max(max(wave_tot[0], wave_tot[1]), max(wave_tot[2], wave_tot[3]));
    hi = dmax == 255 ? ~0ull : ((uint64_t)(dmax + 1) << 56) - 1;
    nab = 0;
    for (int sl = 0; sl < nsl; ++sl) nab += slice_above[sl];
    // Wave w takes slice w: its run above the digit goes to keys[nw ..), its run of the
    // digit to keys[0 .. nw) (counting the next digit on the way); the rest is never
    // read.
    if (wave < nsl) {
      int oa = nw, oe = 0;
      for (int w = 0; w < wave; ++w) {
        oa += slice_above[w];
        oe += slice_equal[w];
      }
      const int na = slice_above[wave], n = na + slice_equal[wave];
      // two keys per lane and load (slices start 16-byte aligned: the key row has an even
      // length); a pair past the runs' end re-reads the last even pair, whose second key
      // is still inside the token's key row
      const uint64_t* sk = krow + wave * kIdxSlice;
      ulonglong2 v[kIdxSlice / 128];
#pragma unroll
      for (int u = 0; u < kIdxSlice / 128; ++u)  // all loads in flight
        if (u * 128 < n) v[u] = *(const ulonglong2*)(sk + min(2 * (u * 64 + lane), (n - 1) & ~1));
#pragma unroll
      for (int u = 0; u < kIdxSlice / 128; ++u) {
        if (u * 128 < n) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = 2 * (u * 64 + lane) + e;
            const uint64_t k = e ? v[u].y : v[u].x;
            if (j < na) {
              keys[oa + j] = k;
            } else if (j < n) {
              keys[oe + j - na] = k;
              atomicAdd(&hist[(int)((k >> 48) & 0xFF)], 1);
            }
          }
        }
      }
    }
    __syncthreads();

    // Remaining digits over keys[0 .. nw), until all keys of the threshold's bin are
    // needed; thr is then a lower bound (lower digits zero) with exactly nsel keys at or
    // above it, or the threshold key itself after the last digit.
    thr = prefix;
    if (need < nw) {
      for (int shift = 48;; shift -= 8) {
        if (shift < 48) {  // hist[] was cleared by the previous digit's search
          const uint64_t hi_mask = ~0ull << (shift + 8);
#pragma unroll 4
          for (int i = tid; i < nw; i += kIdxSelThreads) {
            const uint64_t k = keys[i];
            if ((k & hi_mask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 0xFF)], 1);
          }
          __syncthreads();
        }
        // the digit where the count from the top reaches `need`, by wave 0: lane l takes
        // digits 255 - 4 l .. 252 - 4 l, so a prefix sum over the lanes counts the keys
        // at or above each; the digit where that count first reaches `need` is published
        // with the count still needed within it and its size.  The bins are cleared for
        // the next digit as they are read.
        if (wave == 0) {
          const int4 h4 = *(const int4*)&hist[252 - 4 * lane];  // digits 252 - 4 l .. 255 - 4 l
          *(int4*)&hist[252 - 4 * lane] = make_int4(0, 0, 0, 0);
          const int c[4] = {h4.w, h4.z, h4.y, h4.x};            // descending digits
          const int run = c[0] + c[1] + c[2] + c[3];
          int incl = run;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
          }
          int above = incl - run;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (c[u] > 0 && above < need && above + c[u] >= need) {
              sel_digit = 255 - 4 * lane - u;
              sel_count = need - above;
              sel_bin = c[u];
            }
            above += c[u];
          }
        }
        __syncthreads();
        prefix |= (uint64_t)sel_digit << shift;
        need = sel_count;
        const int bin = sel_bin;
        thr = prefix;
        if (need == bin || shift == 0) break;  // all of the bin needed, or prefix exact
      }
    }
    lo = thr;
  }
  const int nall = nw + nab;
  auto listed = [&](int i, uint64_t k) { return i >= nw || k >= thr; };

  // ---- listing order.  Buckets of equal key width between lo and hi, larger keys in
  // higher buckets: a scan from the top bucket gives each bucket's first output slot,
  // and a key's slot is that plus the number of larger keys in its own bucket.  Keys are
  // distinct, so the slots are 0 .. nsel - 1 once each, by descending key.
  const int sh = max(0, 64 - __clzll(hi - lo) - kIdxBucketBits);  // (hi - lo) >> sh < kIdxBuckets
  auto bucket_of = [&](uint64_t k) { return (int)((k - lo) >> sh); };
  for (int i = tid; i < nall; i += kIdxSelThreads) {
    const uint64_t k = keys[i];
    if (listed(i, k)) atomicAdd(&bfirst[bucket_of(k)], 1u);
  }
  __syncthreads();
  {
    // exclusive scan from the top bucket: thread tid holds buckets
    // kIdxBuckets - 1 - BPT * tid - u, u = 0 .. BPT - 1 (descending)
    constexpr int BPT = kIdxBuckets / kIdxSelThreads;
    uint32_t c[BPT], run = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      c[u] = bfirst[kIdxBuckets - 1 - BPT * tid - u];
      run += c[u];
    }
    uint32_t incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t up = __shfl_up(incl, off);
      if (lane >= off) incl += up;
    }
    if (lane == 63) wave_tot[wave] = (int)incl;
    __syncthreads();
    // the waves before this one: an exclusive scan of the 16 wave totals over lanes 0..15
    uint32_t wt = lane < kIdxSelThreads / 64 ? (uint32_t)wave_tot[lane] : 0u, wincl = wt;
#pragma unroll
    for (int off = 1; off < kIdxSelThreads / 64; off <<= 1) {
      const uint32_t up = __shfl_up(wincl, off);
      if (lane >= off) wincl += up;
    }
    uint32_t first = incl - run + (uint32_t)__builtin_amdgcn_readlane((int)(wincl - wt), wave);
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      bfirst[kIdxBuckets - 1 - BPT * tid - u] = first;
      first += c[u];
    }
  }
  __syncthreads();
  // grouped by bucket; afterwards bfirst[b] is the end of bucket b, which is the first
  // slot of bucket b - 1
  for (int i = tid; i < nall; i += kIdxSelThreads) {
    const uint64_t k = keys[i];
    if (listed(i, k)) grouped[atomicAdd(&bfirst[bucket_of(k)], 1u)] = k;
  }
  __syncthreads();

  // ---- the top_k as physical rows in slot order, then -1
  const int32_t* prow = a.page_table + (int64_t)tr.b * a.pt_row;
  int32_t* orow = a.out + (int64_t)t * a.out_row;
  constexpr int OPT = kIdxMaxTopK / kIdxSelThreads;  // listed keys per thread at most
  if (nsel > 0) {                                    // block-uniform
    // both page-id loads in flight before either count (slots past nsel re-read the last
    // key, so there is no branch around the loads)
    uint64_t k[OPT];
    int pid[OPT], slot[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      k[u] = grouped[min(tid + u * kIdxSelThreads, nsel - 1)];
      const int pos = (int)(0xFFFFFFFFu - (uint32_t)(k[u] & 0xFFFFFFFFu));
      const int lp = pos / a.PS;
      slot[u] = pos - lp * a.PS;
      pid[u] = prow[lp];
    }
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      if (tid + u * kIdxSelThreads >= nsel) break;
      const int bk = bucket_of(k[u]);
      const int s0 = bk == kIdxBuckets - 1 ? 0 : (int)bfirst[bk + 1], s1 = (int)bfirst[bk];
      int rank = s0;
      for (int q = s0; q < s1; ++q) rank += grouped[q] > k[u];
      orow[rank] = (pid[u] >= 0 && (int64_t)pid[u] < a.num_pages) ? pid[u] * a.PS + slot[u] : -1;
    }
  }
  for (int i = nsel + tid; i < a.top_k; i += kIdxSelThreads) orow[i] = -1;
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream, const KernelTimer* timer) {
  hipError_t e;
  if (timer && (e = hipEventRecord(timer->start, stream)) != hipSuccess) return e;
  const int slices = (int)((a.keys_row + kIdxSlice - 1) / kIdxSlice);
  const dim3 sgrid(a.T, slices > 0 ? slices : 1);
  const bool q4 = (((uintptr_t)a.q | (uintptr_t)a.q_tok | (uintptr_t)a.q_head) & 3) == 0;
  const bool pre = q4 && a.NH <= kFoldHeads * (kIdxThreads / (a.depth >> 2));
  if (a.depth <= 128) {
    if (pre)
      hipLaunchKernelGGL((mla_indexer_score_kernel<8, 2, true>), sgrid, dim3(kIdxThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((mla_indexer_score_kernel<8, 2, false>), sgrid, dim3(kIdxThreads), 0, stream, a);
  } else {
    if (pre)
      hipLaunchKernelGGL((mla_indexer_score_kernel<16, 1, true>), sgrid, dim3(kIdxThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((mla_indexer_score_kernel<16, 1, false>), sgrid, dim3(kIdxThreads), 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(mla_indexer_select_kernel, dim3(a.T), dim3(kIdxSelThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (timer && (e = hipEventRecord(timer->stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
