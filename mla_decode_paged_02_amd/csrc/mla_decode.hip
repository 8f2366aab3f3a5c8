// Dense MLA decode over a paged bf16 latent cache, and the log-sum-exp combine of
// split-KV partial results (gfx950).
//
// What is computed follows generic_flare_mla_decode_kv_cache_ragged (summary; Args q,
// input_row_offsets, scale, output, num_partitions_in; Parameters mask_str,
// local_window_size): for each query row t and head h, softmax over the visible cache
// rows of scale * <q, row>, applied to the rows' 512 latent columns.
//
// Work split.  A query row's visible keys are cut into 64-key tiles.  In the balanced
// mode every work-group computes the same list of per-row tile counts (one block scan
// over the rows, no host round trip), takes an equal share of the concatenated tiles,
// and walks the rows its share touches: rows it covers completely are written to the
// output directly, the (at most two) rows it covers in part leave a normalised partial
// output and its log2-sum-exp in the workspace, merged afterwards by the combine
// kernel.  With a fixed partition count each row is cut into that many tile ranges.
//
// Per work-group: all heads of one query row (4 waves x 32 heads at H = 128), so each
// cache row is read from HBM exactly once.  Keys stream through LDS in 32-key stages
// (4 buffers, 3 in flight) via direct global->LDS loads; page ids are fetched with
// scalar loads one stage ahead.  Per stage and wave:
//   S^T = K Q^T   32 keys x 32 heads, 18 MFMA k-steps over the 576 columns; the keys
//                 of each 16-row MFMA tile are permuted so that the accumulator layout
//                 of S^T is already the operand layout P^T needs below;
//   softmax       base-2 online softmax with a lazily updated running max (O and l are
//                 rescaled only when the max grows by more than 8 in log2 units);
//   O^T += V^T P^T  512 columns x 32 heads; V^T is read with transposing LDS loads.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

struct RowGeo {
  int b;   // sequence
  int lo;  // first visible key
  int hi;  // one past the last visible key
};

// Visible key range of query row t (binary search of its sequence in the offsets).
__device__ __forceinline__ RowGeo decode_row_geo(const DecodeArgs& a, int t, bool report) {
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int)ld_const(a.offsets + mid) <= t) lo = mid; else hi = mid;
  }
  RowGeo g{lo, 0, 0};
  const int o0 = (int)ld_const(a.offsets + lo), o1 = (int)ld_const(a.offsets + lo + 1);
  const int n = o1 - o0, j = t - o0;
  if (j < 0 || j >= n) {
    if (report) atomicOr(a.err, kErrOffsets);
    return g;
  }
  long long L = ld_const(a.cache_lens + lo);
  const long long Lmax = (long long)a.max_pages * a.PS;
  if (L > Lmax) {
    if (report) atomicOr(a.err, kErrCacheLen);
    L = Lmax;
  }
  if (L < 0) L = 0;
  if (a.mask == kMaskNull) {
    g.hi = (int)L;
    return g;
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
  g.lo = (int)l;
  g.hi = (int)h;
  return g;
}

__device__ __forceinline__ int geo_tiles(const RowGeo& g) {
  return g.hi > g.lo ? (g.hi - 1) / kTileKeys - g.lo / kTileKeys + 1 : 0;
}

// Barrier that also keeps the compiler from moving memory accesses across it, without
// the hardware fence (the waits it needs are stated by the caller).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Block scan over one chunk of rows: returns the inclusive prefix, sets the chunk total.
__device__ __forceinline__ int chunk_scan(int v, int* buf, int& chunk_total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  chunk_total = buf[blockDim.x - 1];
  __syncthreads();
  return incl;
}

template <int NW>
__device__ void zero_row_out(const DecodeArgs& a, int t) {
  const int n16 = a.H * (kLatentDim / 8);
  for (int c = threadIdx.x; c < n16; c += NW * 64) {
    const int h = c / (kLatentDim / 8), c8 = c % (kLatentDim / 8);
    *(uint4*)(a.out + (int64_t)t * a.o_tok + (int64_t)h * a.o_head + c8 * 8) = make_uint4(0, 0, 0, 0);
  }
}

template <int NW>
__device__ void empty_partial(const DecodeArgs& a, int slot) {
  for (int h = threadIdx.x; h < a.H; h += NW * 64) a.part_lse[(int64_t)slot * a.H + h] = -INFINITY;
}

// ---------------------------------------------------------------------------------------
// One row segment: tiles [ta, tc) (relative to the row's first visible tile) of row t.
// KPAGES = 1: PS is a multiple of 32, so a stage lies in one page whose id is fetched with
// a scalar load one stage ahead; KPAGES = 0: any other page size (page ids fetched per
// lane, which serialises the stage loads).
// ---------------------------------------------------------------------------------------
template <int HB, int NW, int KPAGES>
__device__ __forceinline__ void decode_segment(const DecodeArgs& a, MLA_LDS uint8_t* tiles, int t,
                                               const RowGeo& g, int ta, int tc, bool full, int slot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, ln = lane & 15;
  const int h0 = wave * 16 * HB;
  constexpr int kDpw = kDmaPerStage / NW;  // DMA instructions per wave per stage

  // all of these are block-uniform; readfirstlane keeps them (and the page-table
  // addresses derived from them) in scalar registers
  const int first_tile = __builtin_amdgcn_readfirstlane(g.lo / kTileKeys);
  const int klo = __builtin_amdgcn_readfirstlane(max(g.lo, (first_tile + ta) * kTileKeys));
  const int khi = __builtin_amdgcn_readfirstlane(min(g.hi, (first_tile + tc) * kTileKeys));
  const int s_first = klo / kStageKeys;
  const int nst = (khi - 1) / kStageKeys - s_first + 1;
  const int32_t* pt = a.page_table + (int64_t)__builtin_amdgcn_readfirstlane(g.b) * a.pt_row;

  // every wave must be done with the previous segment's buffers
  all_wait0();
  stage_barrier();

  // ---- stage loads
  bool bad_page = false;
  auto stage_pages = [&](int st, int& pa, int& pb) {
    pa = ld_const(pt + st * kStageKeys / a.PS);
    pb = pa;
  };
  auto issue = [&](int st, int bi, int pa, int pb) {
    MLA_LDS uint8_t* dst = tiles + bi * kStageBytes;
    const int kbase = st * kStageKeys;
    const int lpa = kbase / a.PS;
#pragma unroll
    for (int jj = 0; jj < kDpw; ++jj) {
      const int J = jj * NW + wave;
      const int sl = J * 64 + lane;
      const int row = sl / kRowChunks;
      const int cg = swz_chunk(row, sl - row * kRowChunks);
      const int key = kbase + row;
      const uint8_t* src = a.zero_row + cg * 16;
      if (key >= klo && key < khi) {
        int pid, lp;
        if (KPAGES == 0) {
          lp = key / a.PS;
          pid = pt[lp];
        } else {
          lp = lpa;
          pid = pa;
        }
        if (pid >= 0 && (int64_t)pid < a.num_pages)
          src = a.cache + (int64_t)pid * a.page_bytes + (int64_t)(key - lp * a.PS) * kRowBytes + cg * 16;
        else
          bad_page = true;
      }
      dma16(src, dst + J * 1024);
    }
  };

  int pa_n = 0, pb_n = 0;
  const int npro = nst < kNumBuf - 1 ? nst : kNumBuf - 1;
  for (int k = 0; k < npro; ++k) {
    int pa = 0, pb = 0;
    if (KPAGES != 0) stage_pages(s_first + k, pa, pb);
    issue(s_first + k, k, pa, pb);
  }
  if (KPAGES != 0 && kNumBuf - 1 < nst) stage_pages(s_first + kNumBuf - 1, pa_n, pb_n);

  // ---- query fragments: B operand of S^T = K Q^T (lane holds q[h][32ks + 8gq .. +8]).
  // They are loaded after the prologue's LDS loads and waited for completely: the stage
  // loads are invisible to the compiler's wait bookkeeping, so no ordinary vector-memory
  // access may still be in flight, in its view, once the stage loop starts.
  bf16x8 qf[HB][18];
  {
    const uint16_t* qrow = a.q + (int64_t)t * a.q_tok + 8 * gq;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const uint16_t* qh = qrow + (int64_t)(h0 + 16 * hb + ln) * a.q_head;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[hb][ks] = *(const bf16x8*)(qh + 32 * ks);
    }
  }
  all_wait0();

  f32x4 o[32][HB];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) o[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used[HB], l_part[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m_used[hb] = -INFINITY;
    l_part[hb] = 0.f;
  }

  // per-lane LDS addressing that does not depend on the stage
  const int rowA0 = 8 * (ln >> 2) + (ln & 3);  // score tile u = 0 reads this key row
  const int rowA1 = rowA0 + 4;                 // u = 1
  const int xa0 = gq ^ swz_mask(rowA0), xa1 = gq ^ swz_mask(rowA1);
  const int vr = (lane & 15) >> 2, vq = lane & 3;  // transposing-read coordinates
  const int rowV0 = 8 * gq + vr, rowV1 = rowV0 + 4;
  const int xv0 = (vq >> 1) ^ swz_mask(rowV0), xv1 = (vq >> 1) ^ swz_mask(rowV1);
  const int vhalf = (vq & 1) * 8;

  for (int k = 0; k < nst; ++k) {
    // ---- wait for stage k, then refill the buffer stage k-1 used
    {
      // stages issued after stage k and possibly still in flight: k+1 .. k+kNumBuf-2
      static_assert(kNumBuf == 4, "the wait below assumes two younger stages");
      const int younger = KPAGES == 0 ? 0 : min(kNumBuf - 2, nst - 1 - k);
      if (younger >= 2) vm_wait_imm<2 * kDpw>();
      else if (younger == 1) vm_wait_imm<kDpw>();
      else vm_wait_imm<0>();
      stage_barrier();
      const int kn = k + kNumBuf - 1;
      if (kn < nst) {
        if (KPAGES == 0) {
          issue(s_first + kn, kn % kNumBuf, 0, 0);
        } else {
          issue(s_first + kn, kn % kNumBuf, pa_n, pb_n);
          if (kn + 1 < nst) stage_pages(s_first + kn + 1, pa_n, pb_n);
        }
      }
    }

    const MLA_LDS uint8_t* buf = tiles + (k % kNumBuf) * kStageBytes;
    const int kbase = (s_first + k) * kStageKeys;
    const bool stage_full = kbase >= klo && kbase + kStageKeys <= khi;

    // ---- S^T = K Q^T, fragments prefetched one k-step ahead
    f32x4 sacc[2][HB];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) sacc[u][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const MLA_LDS uint8_t* r0 = buf + rowA0 * kRowBytes;
      const MLA_LDS uint8_t* r1 = buf + rowA1 * kRowBytes;
      auto kchunk = [&](int ks, int xa) {
        return ks < 16 ? ((4 * ks) ^ xa) : 64 + ((4 * (ks - 16)) ^ (xa & 7));
      };
      bf16x8 k0 = *(const MLA_LDS bf16x8*)(r0 + kchunk(0, xa0) * 16);
      bf16x8 k1 = *(const MLA_LDS bf16x8*)(r1 + kchunk(0, xa1) * 16);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        bf16x8 n0 = k0, n1 = k1;
        if (ks + 1 < 18) {
          n0 = *(const MLA_LDS bf16x8*)(r0 + kchunk(ks + 1, xa0) * 16);
          n1 = *(const MLA_LDS bf16x8*)(r1 + kchunk(ks + 1, xa1) * 16);
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          sacc[0][hb] = mfma16x16x32(k0, qf[hb][ks], sacc[0][hb]);
          sacc[1][hb] = mfma16x16x32(k1, qf[hb][ks], sacc[1][hb]);
        }
        k0 = n0;
        k1 = n1;
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- online softmax (base 2).  Lane 16gq+ln holds head h0+16hb+ln, keys
    // kbase + 8gq + 4u + i for sacc[u][hb][i].
    bf16x8 pf[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float x[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[u][hb][i] * a.scale_log2;
          if (!stage_full) {
            const int key = kbase + 8 * gq + 4 * u + i;
            v = (key >= klo && key < khi) ? v : -INFINITY;
          }
          x[u][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = wave_max_xor16_32(mx);
      const bool need = mx > m_used[hb] + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = need ? mx : m_used[hb];
        const float alpha = fast_exp2(m_used[hb] - m_new);  // 0 when m_used = -inf
        l_part[hb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) o[cb][hb] *= alpha;
        m_used[hb] = m_new;
      }
      float lsum = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = x[u][i] == -INFINITY ? 0.f : fast_exp2(x[u][i] - m_used[hb]);
          const __bf16 pb = (__bf16)p;
          pf[hb][4 * u + i] = pb;
          lsum += (float)pb;
        }
      l_part[hb] += lsum;
    }

    // ---- O^T += V^T P^T over the stage's 32 keys, V fragments prefetched one block ahead
    {
      const MLA_LDS uint8_t* v0b = buf + rowV0 * kRowBytes + vhalf;
      const MLA_LDS uint8_t* v1b = buf + rowV1 * kRowBytes + vhalf;
      bf16x4 a0 = ds_read_tr16(v0b + ((0 ^ xv0) * 16));
      bf16x4 a1 = ds_read_tr16(v1b + ((0 ^ xv1) * 16));
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        bf16x4 n0 = a0, n1 = a1;
        if (cb + 1 < 32) {
          const int cc = 2 * (cb + 1);
          n0 = ds_read_tr16(v0b + ((cc ^ xv0) * 16));
          n1 = ds_read_tr16(v1b + ((cc ^ xv1) * 16));
        }
        const bf16x8 vf = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[cb][hb] = mfma16x16x32(vf, pf[hb], o[cb][hb]);
        a0 = n0;
        a1 = n1;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if (bad_page) atomicOr(a.err, kErrPageId);

  // ---- epilogue: lane 16gq+ln holds O^T[16cb + 4gq + i][head h0 + 16hb + ln]
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const float l_tot = wave_sum_xor16_32(l_part[hb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int h = h0 + 16 * hb + ln;
    if (full) {
      uint16_t* orow = a.out + (int64_t)t * a.o_tok + (int64_t)h * a.o_head + 4 * gq;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        const uint32_t lo = (uint32_t)bf16_bits_rne(o[cb][hb][0] * inv) |
                            ((uint32_t)bf16_bits_rne(o[cb][hb][1] * inv) << 16);
        const uint32_t hi = (uint32_t)bf16_bits_rne(o[cb][hb][2] * inv) |
                            ((uint32_t)bf16_bits_rne(o[cb][hb][3] * inv) << 16);
        *(uint2*)(orow + 16 * cb) = make_uint2(lo, hi);
      }
    } else {
      float* prow = a.part_o + ((int64_t)slot * a.H + h) * kLatentDim + 4 * gq;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) *(f32x4*)(prow + 16 * cb) = o[cb][hb] * inv;
      if (gq == 0)
        a.part_lse[(int64_t)slot * a.H + h] = l_tot > 0.f ? m_used[hb] + __log2f(l_tot) : -INFINITY;
    }
  }
}

template <int HB, int NW, int KPAGES>
__global__ __launch_bounds__(NW * 64, 1) void mla_decode_kernel(const DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles_raw[kNumBuf * kStageBytes];
  __shared__ int scan[256];
  __shared__ int found[2];
  MLA_LDS uint8_t* tiles = (MLA_LDS uint8_t*)tiles_raw;
  const int gid = blockIdx.x;

  // The work of this work-group is a run of tiles [s, e) over the rows, in row order;
  // r0 is the first row it touches and p its first tile's global index.
  int s = 0, e = 0, r0 = -1, p = 0;
  if (a.nparts >= 1) {
    // fixed partitions: work-group = (row, part)
    const int P = a.nparts;
    const int t = gid / P, part = gid - t * P;
    if (t >= a.T) return;
    const RowGeo g = decode_row_geo(a, t, threadIdx.x == 0);
    const int nt = geo_tiles(g);
    const int ta = (int)((long long)part * nt / P), tc = (int)((long long)(part + 1) * nt / P);
    if (ta == tc) {
      if (P == 1) zero_row_out<NW>(a, t);
      else empty_partial<NW>(a, gid);
      return;
    }
    // express the part as a tile run over a single row
    r0 = t;
    p = 0;
    s = ta;
    e = tc;
  } else {
    // balanced: pass 1, total tiles over all rows
    int total = 0;
    for (int base = 0; base < a.T; base += blockDim.x) {
      const int t = base + threadIdx.x;
      const int v = t < a.T ? geo_tiles(decode_row_geo(a, t, gid == 0)) : 0;
      int ctot;
      chunk_scan(v, scan, ctot);
      total += ctot;
    }
    total = __builtin_amdgcn_readfirstlane(total);
    const int W = (total + a.grid - 1) / a.grid;
    s = gid * W;
    e = min(total, s + W);
    if (gid == 0 && threadIdx.x == 0) {
      a.row_meta[0] = total;
      a.row_meta[1] = W;
    }
    // pass 2: the row holding tile s (and, for work-group 0, every row's tile range)
    if (threadIdx.x == 0) {
      found[0] = -1;
      found[1] = 0;
    }
    __syncthreads();
    int prefix = 0;
    for (int base = 0; base < a.T; base += blockDim.x) {
      const int t = base + threadIdx.x;
      const int v = t < a.T ? geo_tiles(decode_row_geo(a, t, false)) : 0;
      int ctot;
      const int incl = chunk_scan(v, scan, ctot);
      const int excl = prefix + incl - v;
      if (t < a.T) {
        if (gid == 0) {
          a.row_meta[2 + 2 * t] = excl;
          a.row_meta[3 + 2 * t] = v;
        }
        if (v > 0 && excl <= s && s < excl + v) {
          found[0] = t;
          found[1] = excl;
        }
      }
      prefix += ctot;
      __syncthreads();
      if (gid != 0 && found[0] >= 0) break;
    }
    __syncthreads();
    // the values are block-uniform; say so, so that row walking stays in scalar registers
    r0 = __builtin_amdgcn_readfirstlane(found[0]);
    p = __builtin_amdgcn_readfirstlane(found[1]);
    // rows without visible keys are written as zeros, spread over the work-groups
    for (int t = gid; t < a.T; t += a.grid) {
      const RowGeo g = decode_row_geo(a, t, false);
      if (geo_tiles(g) == 0) zero_row_out<NW>(a, t);
    }
    if (s >= e || r0 < 0) return;
  }

  const bool fixed = a.nparts >= 1;
  for (int r = r0; r < a.T && p < e; ++r) {
    const RowGeo g = decode_row_geo(a, r, false);
    const int nt = geo_tiles(g);
    if (nt == 0) continue;
    const int ta = max(s, p) - p, tc = min(e, p + nt) - p;
    bool full;
    int slot;
    if (fixed) {
      full = a.nparts == 1;
      slot = gid;
    } else {
      full = ta == 0 && tc == nt;
      slot = p <= s ? 2 * gid : 2 * gid + 1;
    }
    decode_segment<HB, NW, KPAGES>(a, tiles, r, g, ta, tc, full, slot);
    if (fixed) break;
    p += nt;
  }
}

// ---------------------------------------------------------------------------------------
// Combine: out = sum_c 2^(lse_c - M) O_c / sum_c 2^(lse_c - M), pieces in a fixed order.
// Block = (row, 4 heads); thread = (head, 8 columns).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_combine_kernel(const DecodeArgs a) {
  const int groups = a.H / 4;
  const int t = blockIdx.x / groups, hg = blockIdx.x - t * groups;
  const int h = hg * 4 + (threadIdx.x >> 6), col = (threadIdx.x & 63) * 8;
  int c0, c1, W = 0, p = 0;
  if (a.nparts == 0) {
    W = a.row_meta[1];
    p = a.row_meta[2 + 2 * t];
    const int nt = a.row_meta[3 + 2 * t];
    if (nt == 0 || W == 0) return;
    c0 = p / W;
    c1 = (p + nt - 1) / W;
    if (c0 == c1) return;  // one work-group covered the whole row and wrote it
  } else {
    if (a.nparts == 1) return;
    c0 = 0;
    c1 = a.nparts - 1;
  }
  auto slot_of = [&](int c) {
    if (a.nparts == 0) return c == c0 ? (p == c0 * W ? 2 * c0 : 2 * c0 + 1) : 2 * c;
    return t * a.nparts + c;
  };
  float M = -INFINITY;
  for (int c = c0; c <= c1; ++c) M = fmaxf(M, a.part_lse[(int64_t)slot_of(c) * a.H + h]);
  uint16_t* dst = a.out + (int64_t)t * a.o_tok + (int64_t)h * a.o_head + col;
  if (M == -INFINITY) {
    *(uint4*)dst = make_uint4(0, 0, 0, 0);
    return;
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float den = 0.f;
  for (int c = c0; c <= c1; ++c) {
    const int sl = slot_of(c);
    const float l = a.part_lse[(int64_t)sl * a.H + h];
    if (l == -INFINITY) continue;
    const float w = fast_exp2(l - M);
    den += w;
    const float* src = a.part_o + ((int64_t)sl * a.H + h) * kLatentDim + col;
    const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += w * x0[i];
      acc[4 + i] += w * x1[i];
    }
  }
  const float inv = 1.f / den;
  uint32_t wd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    wd[i] = (uint32_t)bf16_bits_rne(acc[2 * i] * inv) | ((uint32_t)bf16_bits_rne(acc[2 * i + 1] * inv) << 16);
  *(uint4*)dst = make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
size_t decode_slots(int64_t T, int32_t nparts, int32_t grid) {
  return nparts >= 1 ? (size_t)T * (size_t)nparts : 2 * (size_t)grid;
}

template <int HB, int NW>
static hipError_t launch_decode_h(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.nparts >= 1 ? a.T * a.nparts : a.grid), block(NW * 64);
  if (a.PS % kStageKeys == 0)
    hipLaunchKernelGGL((mla_decode_kernel<HB, NW, 1>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((mla_decode_kernel<HB, NW, 0>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, const KernelTimer* timer) {
  hipError_t e;
  if (timer && (e = hipEventRecord(timer->start, stream)) != hipSuccess) return e;
  switch (a.H) {
    case 128: e = launch_decode_h<2, 4>(a, stream); break;
    case 64: e = launch_decode_h<1, 4>(a, stream); break;
    case 32: e = launch_decode_h<1, 2>(a, stream); break;
    case 16: e = launch_decode_h<1, 1>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (timer && (e = hipEventRecord(timer->stop, stream)) != hipSuccess) return e;
  if (a.nparts == 0 || a.nparts > 1) {
    hipLaunchKernelGGL(mla_combine_kernel, dim3(a.T * (a.H / 4)), dim3(256), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace mla
