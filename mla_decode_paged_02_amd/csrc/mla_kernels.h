// Host-visible kernel argument blocks and launch entry points of libmla355.
// Included by the C-ABI layer (validation, workspace) and by the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Workspace header: a zero row (>= 1152 zero bytes) at offset 0, the device error word at
// kHdrErrOffset and the float 1.0 at kSparseOneOffset (the scale of rows without one).
constexpr size_t kHdrErrOffset = 2048;
constexpr size_t kSparseOneOffset = 2064;

// Dense decode over a paged bf16 latent cache.
struct DecodeArgs {
  const uint16_t* q;          // bf16 [T, H, 576]
  int64_t q_tok, q_head;      // element strides
  const uint32_t* offsets;    // [B + 1]
  const int32_t* page_table;  // [B, max_pages]
  int64_t pt_row;             // element stride between page-table rows
  const int32_t* cache_lens;  // [B]
  const uint8_t* cache;       // bf16 [num_pages, PS, 576], rows contiguous
  int64_t page_bytes;         // byte stride between pages
  int64_t num_pages;
  int32_t B, T, H, PS, max_pages;
  float scale_log2;           // scale * log2(e): logits are kept in base-2 units
  int32_t mask, window;
  int32_t nparts;             // 0: balanced split over `grid` work-groups; >= 1: fixed
  int32_t grid;
  uint16_t* out;              // bf16 [T, H, 512]
  int64_t o_tok, o_head;
  uint16_t* part_o;           // bf16 [slots, H, 512] partial outputs (normalised)
  float* part_lse;            // [slots, H] log2-sum-exp of the partials
  int32_t* row_meta;          // [2 + 2T]: the split rows' layout for the combine (mla_plan.h)
  const uint8_t* zero_row;    // >= 1152 zero bytes
  uint32_t* err;              // device error word
};

// Decode over an fp8 e4m3 cache whose rows are gathered one by one: the sparse decode
// (each q row lists physical cache rows to attend to) and, with dense = 1, the dense
// decode over a paged fp8 cache (each q row attends to the visible rows of its sequence,
// found through the page table).
struct SparseArgs {
  const uint8_t* q;           // fp8 e4m3 [T, H, 576] (640 bytes with rope), or bf16 when q_bf16
  int64_t q_tok, q_head;      // element strides
  const float* q_scale;       // [T] or null (= 1)
  const uint8_t* cache;       // fp8 e4m3 [num_pages, PS, 576 or 640 with rope]; a page's rows are contiguous
  int64_t page_bytes;         // byte stride between pages
  const float* cache_scale;   // [num_pages, PS] or null (= 1)
  int64_t cs_page;            // element stride between pages of cache_scale
  int64_t num_rows;           // num_pages * PS: listed rows outside [0, num_rows) are skipped
  int32_t PS;
  int32_t flat;               // 1: row r is at byte r * (576 or 640) and its scale at element r
  const int32_t* idx;         // [T, idx_row] ([B, idx_row] with shared lists)
  int64_t idx_row;            // element stride between index rows
  int32_t idx_cols;           // shape[1] of d_indices (topk is clamped to it)
  const int32_t* topk;        // [T] ([B] with shared lists)
  // shared = 1 ([DEC] Parameters fold_shared_index): idx / topk hold one list per
  // sequence, [B, idx_row] / [B], read by every query row of the sequence (offsets, B)
  int32_t shared;
  // dense = 1: the rows of q row t are the visible positions of its sequence, physical
  // row page_table[b][pos / PS] * PS + pos % PS (idx and topk are unused)
  int32_t dense;
  const uint32_t* offsets;    // [B + 1]
  const int32_t* page_table;  // [B, max_pages]
  int64_t pt_row;             // element stride between page-table rows
  const int32_t* cache_lens;  // [B]
  int32_t B, max_pages, mask, window;
  int32_t T, H;
  int32_t q_bf16;             // 1: q is bf16 (no q_scale)
  int32_t rope;               // 1: q and cache rows are 640-byte rope-aware rows (e4m3 latent, bf16 rope)
  float scale_log2;           // scale * log2(e)
  int32_t nparts;             // 0: balanced; >= 1 fixed
  int32_t grid;
  uint16_t* out;              // bf16 [T, H, 512]
  int64_t o_tok, o_head;
  uint16_t* part_o;
  float* part_lse;
  int32_t* row_meta;
  const uint8_t* zero_row;    // >= 1152 zero bytes
  uint32_t* err;
  // Extended sparse decode only (the kernels' EXT variant): sink logits, and a second
  // stream (xidx null = none) -- row t also attends to the rows its second list names in a
  // second fp8 pool, under the same softmax.  Both pools then hold fewer than 2^30 rows (a
  // second-pool row is marked by kExtraRowBit in the index window).
  const float* sink;          // [H] sink logits (natural-log units), or null
  const int32_t* xidx;        // [T, xidx_row]
  int64_t xidx_row;
  int32_t xidx_cols;
  const int32_t* xtopk;       // [T]
  const uint8_t* xcache;      // fp8 e4m3 [x pages, xPS, 576]
  int64_t xpage_bytes;
  const float* xcache_scale;  // [x pages, xPS] or null (= 1)
  int64_t xcs_page;
  int64_t xnum_rows;
  int32_t xPS;
};
constexpr int32_t kExtraRowBit = 1 << 30;

// Ragged prefill with per-head keys and values.
struct PrefillArgs {
  const uint16_t* q;          // bf16 [Tq, H, 192]
  int64_t q_tok, q_head;
  const uint16_t* k;          // bf16 [Tk, H, 128]
  int64_t k_tok, k_head;
  const uint16_t* v;          // bf16 [Tk, H, 128]
  int64_t v_tok, v_head;
  const uint32_t* buf_off;    // [B + 1]
  const uint32_t* cache_off;  // [B]
  const uint32_t* in_off;     // [B + 1]
  const int32_t* page_table;
  int64_t pt_row;
  const int32_t* cache_lens;
  const uint8_t* cache;       // bf16 latent cache (rope columns 512..575 used)
  int64_t page_bytes;
  int64_t num_pages;
  int32_t B, Tq, Tk, H, PS, max_pages;
  float scale_log2;
  int32_t mask;
  uint16_t* out;              // bf16 [Tq, H, 128]
  int64_t o_tok, o_head;
  const uint8_t* zero_row;    // >= 256 zero bytes (the stage loads of keys that do not count)
  uint32_t* err;
};

// FP8 top-k indexer over a paged cache (mla_indexer.hip).
constexpr int kIdxMaxKeys = 16384;  // visible rows per query token (scores sorted in LDS)
constexpr int kIdxMaxDepth = 256;   // indexer head width
constexpr int kIdxMaxTopK = 2048;
constexpr int kIdxSlice = 1024;     // visible rows a scoring work-group takes
struct IndexerArgs {
  const uint8_t* q;           // fp8 e4m3 [T, NH, depth]
  int64_t q_tok, q_head;      // element strides
  const float* q_s;           // [T, NH] scales
  int64_t qs_tok;
  const uint32_t* offsets;    // [B + 1]
  const int32_t* page_table;  // [B, max_pages]
  int64_t pt_row;
  const int32_t* cache_lens;  // [B]
  const uint8_t* k;           // fp8 e4m3 [num_pages, PS, depth], rows of a page contiguous
  int64_t page_bytes;
  int64_t num_pages;
  const float* k_s;           // [num_pages, PS] row scales or null (= 1)
  int64_t ks_page;
  int32_t B, T, NH, depth, PS, max_pages, mask, window, top_k;
  int32_t* out;               // [T, top_k] physical rows, -1 filled
  int64_t out_row;
  uint64_t* keys;             // workspace [T, keys_row]: the scored rows' sort keys
  int64_t keys_row;           // max_pages * PS rounded up to even (slices 16-byte aligned)
  uint32_t* slice_hist;       // workspace [T, hist_row]: per key slice, the size and start
                              // of each top digit's run of keys
  int64_t hist_row;           // 512 * slices, slices = ceil(keys_row / kIdxSlice)
  uint32_t* err;
  const uint8_t* zero_row;    // >= 256 zero bytes (the workspace header), read in place of rows that do not count
};

// Where the decode kernels put split rows' parts (mla_plan.h).
struct SplitPlan {
  int32_t T, H;
  int32_t nparts;     // 0 = balanced, >= 1 fixed
  int32_t grid;       // work-groups of the balanced mode
  uint16_t* out;      // bf16 [T, H, 512]
  int64_t o_tok, o_head;
  uint16_t* part_o;   // bf16 [slots, H, 512]
  float* part_lse;    // [slots, H]
  int32_t* row_meta;  // [2 + 2T]: the split rows' layout (mla_plan.h)
  const float* sink;  // [H] sink logits merged into split rows' denominators, or null
};

// Workspace needs of the split-KV paths.
size_t decode_slots(int64_t T, int32_t nparts, int32_t grid);
size_t decode_workspace_bytes(int64_t T, int32_t H, int32_t nparts, int32_t grid);

// Optional events bracketing the main kernel of a launch (null = none).
struct KernelTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launchers (return the HIP status of the launches).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, const KernelTimer* timer);
hipError_t launch_combine(const SplitPlan& p, hipStream_t stream);
// The dense decode kernel that splits the value columns over the waves (mla_decode2.hip):
// 128 heads, the balanced split of at most 64 rows and sequences, no more rows than
// work-groups.
hipError_t launch_decode2(const DecodeArgs& a, const SplitPlan& p, hipStream_t stream);
hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream, const KernelTimer* timer);
// The dense fp8 decode kernel with the scores on fp8 MFMA (mla_fp8mma.hip): 128 heads, the
// balanced split of at most 64 rows and sequences, no more rows than work-groups, fp8 q.
hipError_t launch_fp8mma(const SparseArgs& a, const SplitPlan& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream, const KernelTimer* timer);
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream, const KernelTimer* timer);

}  // namespace mla
