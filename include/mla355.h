/*
 * libmla355 -- multi-head latent attention (MLA) over a paged latent KV cache on
 * AMD Instinct MI355X (gfx950).  Plain C ABI: tensors are described by mla_tensor
 * (a device pointer plus element type, shape and element strides); nothing here
 * depends on any framework's types.
 *
 * The operations follow the Modular MAX kernel-library pages, cited by title and
 * section:
 *   generic_flare_mla_decode_kv_cache_ragged  (summary; Parameters mask_str,
 *       local_window_size, sparse_mla; Args q, input_row_offsets, scale, output,
 *       q_scale_ptr, d_indices, indices_stride, topk_lengths, num_partitions_in)
 *   generic_flare_mla_prefill_kv_cache_ragged (summary; Args q, k, v,
 *       buffer_row_offsets, cache_offsets, input_row_offsets, scale, output)
 *   mla_decode_branch_fp8 (summary: the 576-wide query is the projected no-rope part
 *       followed by the rope part; the decode output is in the 512-wide latent space)
 *
 * Common conventions
 *   - Every tensor pointer is a device pointer on the current HIP device and is owned
 *     by the caller, outputs included; the library never frees or reallocates it.
 *   - Strides are in elements.  The innermost dimension must be contiguous (stride 1),
 *     every other stride and every base pointer must be a multiple of 16 bytes.
 *   - A latent cache row is 576 values: columns 0..511 are the latent part (which is
 *     also V), columns 512..575 the rope part.
 *   - cache_lens[b] counts the valid cache rows of sequence b, the rows written for
 *     its current query tokens included; query token j of the n_b tokens of sequence
 *     b sits at cache position cache_lens[b] - n_b + j.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and
 *     return as soon as the work is queued.  Validation uses only the descriptors and
 *     scalars: the library never reads device data on the host.  On any error nothing
 *     is launched and the call returns a status; mla_last_error_message() gives the
 *     detail (per host thread).  Device faults surface at the caller's next
 *     synchronisation.  Out-of-range device data (a page id outside the pool, an index
 *     outside the pool, non-monotone offsets) never causes an out-of-bounds access:
 *     the offending rows contribute nothing and a bit is set in the device error word
 *     read by mla_check_device_errors().
 *   - Workspace (split-KV partial results and the split table) is owned by the
 *     library, one grow-only buffer per (device, stream).  It is allocated on first
 *     use; a call issued while `stream` is capturing a graph must find it already large
 *     enough (see mla_reserve_workspace), else it returns MLA_ERR_WORKSPACE.  Calls on
 *     one stream are ordered, so they may share that stream's workspace.  When a later
 *     call (or mla_reserve_workspace) outside capture needs a larger one, the stream is
 *     synchronised, a new buffer takes over and the old one is retired, not freed:
 *     graphs captured earlier on that stream keep replaying into the old buffer, which
 *     stays allocated until mla_shutdown.  The device error word moves to the new buffer
 *     at that point; errors raised later by replays of such older graphs land in the
 *     retired buffer and are not reported by mla_check_device_errors.
 *   - At most 2^24 query rows per call.
 */
#ifndef MLA355_H_
#define MLA355_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL_ARG = 1,    /* a required pointer or descriptor is NULL */
  MLA_ERR_SHAPE = 2,       /* shapes or strides disagree with each other */
  MLA_ERR_DTYPE = 3,       /* a tensor has the wrong element type */
  MLA_ERR_ALIGNMENT = 4,   /* a base pointer or stride is not 16-byte aligned */
  MLA_ERR_UNSUPPORTED = 5, /* a well-formed request outside what this build implements */
  MLA_ERR_WORKSPACE = 6,   /* workspace could not be allocated, or is too small while capturing */
  MLA_ERR_HIP = 7,         /* a HIP runtime call failed */
  MLA_ERR_VALUE = 8        /* a scalar argument is out of range */
} mla_status;

/* Masking strategy (generic_flare_mla_decode_kv_cache_ragged, Parameters mask_str). */
typedef enum mla_mask {
  MLA_MASK_NULL = 0,                 /* every cache row 0..L-1 is visible */
  MLA_MASK_CAUSAL = 1,               /* rows 0..pos are visible */
  MLA_MASK_SLIDING_WINDOW_CAUSAL = 2 /* rows pos-W+1..pos, W = local_window_size > 0 */
} mla_mask;

typedef enum mla_dtype {
  MLA_DTYPE_BF16 = 0,
  MLA_DTYPE_FP8_E4M3 = 1, /* OCP E4M3 (finite-only "fn" variant), the gfx950 native FP8 */
  MLA_DTYPE_F32 = 2,
  MLA_DTYPE_I32 = 3,
  MLA_DTYPE_U32 = 4
} mla_dtype;

typedef struct mla_tensor {
  void* data;        /* device pointer, caller-owned */
  int32_t dtype;     /* an mla_dtype */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];  /* entries past ndim are ignored */
  int64_t stride[4]; /* element strides; entries past ndim are ignored */
} mla_tensor;

/*
 * Dense MLA decode over a ragged batch against a paged latent cache
 * (generic_flare_mla_decode_kv_cache_ragged: summary; Args q, input_row_offsets,
 * scale, output, num_partitions_in; Parameters mask_str, local_window_size).
 *
 * For every query row t of sequence b and every head h:
 *   s_r = scale * <q[t,h,:], C_b[r,:]> over the visible cache rows r,
 *   out[t,h,:] = sum_r softmax(s)_r * C_b[r, 0:512],
 * where C_b[r] = latent_cache[page_table[b, r / PS], r % PS, :].
 *
 *   q                  bf16 [T, H, 576]; H in {16, 32, 64, 128}
 *   input_row_offsets  u32 [B + 1], off[0] = 0, non-decreasing, off[B] = T
 *   page_table         i32 [B, max_pages]; entries past a sequence's pages are not read
 *   cache_lens         i32 [B]
 *   latent_cache       bf16 [num_pages, PS, 576], PS >= 1, rows contiguous
 *   scale              finite float (usually 1/sqrt(qk head width))
 *   mask, local_window_size   see mla_mask; the window is ignored unless sliding
 *   num_partitions     <= 0: the library balances the work over the whole GPU,
 *                      splitting long rows (split-KV) and merging the pieces by their
 *                      log-sum-exp; >= 1: every query row is split into exactly that
 *                      many key ranges (the graph-capture override), at most 4096
 *   out                bf16 [T, H, 512], written in full (rows with no visible key
 *                      become 0)
 */
mla_status mla_decode_paged(const mla_tensor* q, const mla_tensor* input_row_offsets,
                            const mla_tensor* page_table, const mla_tensor* cache_lens,
                            const mla_tensor* latent_cache, float scale, int32_t mask,
                            int32_t local_window_size, int32_t num_partitions,
                            mla_tensor* out, void* stream);

/*
 * Sparse MLA decode (generic_flare_mla_decode_kv_cache_ragged: Parameters sparse_mla;
 * Args q_scale_ptr, d_indices, indices_stride, topk_lengths, num_partitions_in).
 * Query row t attends only to the cache rows listed in d_indices[t, :], in listed
 * order, with no positional mask: the first topk_lengths[t] entries count, negative
 * entries (the -1 fill) are skipped, duplicates count as often as they are listed.
 * A listed value is a physical row of the pool: page * PS + slot.
 *
 *   q             fp8 e4m3 [T, H, 576] (or bf16, then q_scale must be NULL), or u8
 *                 [T, H, 640] in the rope-aware layout of mla_decode_paged_fp8
 *   q_scale       f32 [T] (one scale per query token, shared by its heads) or NULL = 1
 *   input_row_offsets  u32 [B + 1] (only its shape is checked: index lists are per row)
 *   latent_cache  fp8 e4m3 [num_pages, PS, 576] (a bf16 cache is refused: MLA_ERR_UNSUPPORTED),
 *                 or u8 [num_pages, PS, 640] in the rope-aware layout (Parameters
 *                 per_token_scale_rope_aware; see mla_decode_paged_fp8), q alike
 *   cache_scale   f32 [num_pages, PS] (one scale per cache row) or NULL = 1
 *   d_indices     i32 [T, indices_stride] (row stride = stride[0] >= shape[1])
 *   topk_lengths  i32 [T], values above shape[1] of d_indices are clamped to it
 *   scale, num_partitions, out   as for mla_decode_paged; out is bf16 [T, H, 512]
 */
mla_status mla_decode_paged_sparse(const mla_tensor* q, const mla_tensor* q_scale,
                                   const mla_tensor* input_row_offsets,
                                   const mla_tensor* latent_cache, const mla_tensor* cache_scale,
                                   const mla_tensor* d_indices, const mla_tensor* topk_lengths,
                                   float scale, int32_t num_partitions, mla_tensor* out,
                                   void* stream);

/*
 * Sparse MLA decode with shared index lists (generic_flare_mla_decode_kv_cache_ragged:
 * Parameters sparse_mla, fold_shared_index; the page names a read-once shared-index fold
 * for multi-token decode without a formula, so what follows is this library's reading).
 * Every query token of sequence b (rows input_row_offsets[b] .. input_row_offsets[b+1]-1)
 * attends to sequence b's one list, read by the rules of mla_decode_paged_sparse.  The
 * tokens of a sequence are consecutive work of the split and land on the same XCD, so
 * each listed cache row is fetched from HBM once for all of them and served to the
 * others from that XCD's L2.
 *
 *   q, q_scale, latent_cache, cache_scale, scale, num_partitions, out
 *                      as for mla_decode_paged_sparse
 *   input_row_offsets  u32 [B + 1]: non-decreasing, from 0 to T (read on the device;
 *                      malformed offsets set bit 2 of the device error word and leave
 *                      their rows zero)
 *   d_indices          i32 [B, indices_stride]: one list per sequence
 *   topk_lengths       i32 [B]
 */
mla_status mla_decode_paged_sparse_shared(const mla_tensor* q, const mla_tensor* q_scale,
                                          const mla_tensor* input_row_offsets,
                                          const mla_tensor* latent_cache, const mla_tensor* cache_scale,
                                          const mla_tensor* d_indices, const mla_tensor* topk_lengths,
                                          float scale, int32_t num_partitions, mla_tensor* out,
                                          void* stream);

/*
 * Sparse MLA decode with an attention sink and a second KV stream
 * (generic_flare_mla_decode_kv_cache_ragged: Args attn_sink_ptr, extra_k,
 * extra_d_indices, extra_indices_stride, extra_topk_lengths, extra_scales_ptr; the page
 * names these arguments without a formula, so what follows is this library's reading).
 * Everything mla_decode_paged_sparse takes, plus:
 *
 *   attn_sink          f32 [H] or NULL: one logit per head, shared by every query row of
 *                      the call and not multiplied by `scale`.  It adds e^attn_sink[h] to
 *                      the softmax denominator and nothing to the numerator:
 *                      out[t,h] = sum_r e^{s_r} v_r / (e^{attn_sink[h]} + sum_r e^{s_r}),
 *                      so a row whose lists hold no key gets out = 0.
 *   extra_cache        fp8 e4m3 [extra_pages, extra_PS, 576] or NULL: the second stream's
 *                      pool (rows of a page contiguous)
 *   extra_cache_scale  f32 [extra_pages, extra_PS] or NULL = 1: its row scales
 *   extra_d_indices    i32 [T, extra_stride], row stride = extra_indices_stride: row t's
 *                      second list, physical rows page * extra_PS + slot of extra_cache,
 *                      read by the rules of d_indices (first extra_topk_lengths[t]
 *                      entries, negatives skipped, duplicates counted)
 *   extra_topk_lengths i32 [T]
 *
 * Row t attends to the rows of both lists under one softmax (one set of weights over the
 * union).  extra_cache, extra_d_indices and extra_topk_lengths come together or not at
 * all; with them, each pool must hold fewer than 2^30 rows.  Second-list rows outside
 * extra_cache are skipped and set bit 1 of the device error word.  With neither a sink nor
 * a second stream this is mla_decode_paged_sparse.  A rope-aware (640-byte) q and cache
 * with a sink or a second stream is refused with MLA_ERR_UNSUPPORTED.
 */
mla_status mla_decode_paged_sparse_ext(const mla_tensor* q, const mla_tensor* q_scale,
                                       const mla_tensor* input_row_offsets,
                                       const mla_tensor* latent_cache, const mla_tensor* cache_scale,
                                       const mla_tensor* d_indices, const mla_tensor* topk_lengths,
                                       const mla_tensor* attn_sink, const mla_tensor* extra_cache,
                                       const mla_tensor* extra_cache_scale,
                                       const mla_tensor* extra_d_indices,
                                       const mla_tensor* extra_topk_lengths, float scale,
                                       int32_t num_partitions, mla_tensor* out, void* stream);

/*
 * Dense MLA decode over a paged fp8 e4m3 latent cache
 * (generic_flare_mla_decode_kv_cache_ragged: summary; Args q, q_scale_ptr, kv_collection,
 * input_row_offsets, scale, output, num_partitions_in; Parameters mask_str,
 * local_window_size, per_token_scale_rope_aware).  The same computation as
 * mla_decode_paged, with every value stored as an e4m3 code times a float32 scale: the
 * query's per token (shared by its heads), the cache's per row (all 576 columns).  The
 * codes are widened exactly; the logits and P.V accumulate in fp32 from bf16 operands.
 *
 * Rope-aware layout (per_token_scale_rope_aware; chosen when the cache rows are 640
 * bytes wide, and q must then be too): each 576-wide head row of q and the cache is
 * stored as its 512 latent values in e4m3 followed by its 64 rope values as
 * little-endian bf16, and the token / row scale multiplies the latent codes only.  The
 * rope values enter the logits divided by their scale and multiplied back in fp32, so
 * they carry one extra bf16 rounding; scales of magnitude below 2^-40 are taken as 2^-40
 * for that (their latent part then contributes about nothing, their rope in full).
 *
 *   q                  fp8 e4m3 [T, H, 576], or u8 [T, H, 640] in the rope-aware layout
 *   q_scale            f32 [T] or NULL = 1
 *   input_row_offsets, page_table, cache_lens, mask, local_window_size, scale,
 *   num_partitions, out     as for mla_decode_paged
 *   latent_cache       fp8 e4m3 [num_pages, PS, 576], or u8 [num_pages, PS, 640] in the
 *                      rope-aware layout; rows of a page contiguous, any PS
 *   cache_scale        f32 [num_pages, PS] or NULL = 1
 *
 * Errors as for mla_decode_paged; page ids outside the pool are skipped and set bit 0
 * of the device error word (mla_check_device_errors).
 */
mla_status mla_decode_paged_fp8(const mla_tensor* q, const mla_tensor* q_scale,
                                const mla_tensor* input_row_offsets, const mla_tensor* page_table,
                                const mla_tensor* cache_lens, const mla_tensor* latent_cache,
                                const mla_tensor* cache_scale, float scale, int32_t mask,
                                int32_t local_window_size, int32_t num_partitions,
                                mla_tensor* out, void* stream);

/*
 * FP8 top-k indexer (mla_indexer_ragged_float8_paged: summary; Args output_indices, q,
 * q_s, input_row_offsets, k_collection).  For query token t of sequence b the score of
 * visible cache row r is sum_h q_s[t, h] * <e4m3(q[t, h, :]), e4m3(k[r, :])> * k_scale[r]
 * (scores summed over the heads, one k scale per row); the mask leaves the rows a decode
 * token at position cache_lens[b] - n_b + j sees.  Row t of out_indices receives the
 * top_k highest-scoring visible rows as physical rows of the pool (page_id * PS + slot:
 * the d_indices of mla_decode_paged_sparse), by descending score, equal scores by
 * ascending position, then -1.  Scores are evaluated in float32.
 *
 *   q                  fp8 e4m3 [T, NH, D], D a multiple of 16 up to 256, D contiguous
 *   q_s                f32 [T, NH]
 *   input_row_offsets, page_table, cache_lens, mask, local_window_size
 *                      as for mla_decode_paged; max_pages * PS <= 16384
 *   k_cache            fp8 e4m3 [num_pages, PS, D], rows of a page contiguous, base and
 *                      page stride multiples of 16 bytes
 *   k_scale            f32 [num_pages, PS] or NULL = 1
 *   out_indices        i32 [T, top_k], top_k in [1, 2048], written in full
 *
 * Page ids outside the pool rank last, are never returned and set bit 0 of the device
 * error word.
 */
mla_status mla_indexer_paged_fp8(const mla_tensor* q, const mla_tensor* q_s,
                                 const mla_tensor* input_row_offsets, const mla_tensor* page_table,
                                 const mla_tensor* cache_lens, const mla_tensor* k_cache,
                                 const mla_tensor* k_scale, int32_t mask, int32_t local_window_size,
                                 mla_tensor* out_indices, void* stream);

/*
 * Ragged MLA prefill with per-head keys (generic_flare_mla_prefill_kv_cache_ragged:
 * summary; Args q, k, v, buffer_row_offsets, cache_offsets, input_row_offsets, scale,
 * output).  Key i of sequence b is row buffer_row_offsets[b] + i of k / v at cache
 * position cache_offsets[b] + i; its 192-wide key is [k[row, h, 0:128] | the rope
 * columns 512..575 of its latent cache row], shared rope across heads.
 *
 *   q                   bf16 [Tq, H, 192] = [no-rope 128 | rope 64]; H in {16,...,128}
 *   k, v                bf16 [Tk, H, 128]
 *   buffer_row_offsets  u32 [B + 1] rows of k / v per sequence
 *   cache_offsets       u32 [B]
 *   input_row_offsets   u32 [B + 1] rows of q / out per sequence
 *   page_table, cache_lens, latent_cache   as for mla_decode_paged
 *   mask                MLA_MASK_CAUSAL or MLA_MASK_NULL
 *   out                 bf16 [Tq, H, 128]
 */
mla_status mla_prefill_paged(const mla_tensor* q, const mla_tensor* k, const mla_tensor* v,
                             const mla_tensor* buffer_row_offsets, const mla_tensor* cache_offsets,
                             const mla_tensor* input_row_offsets, const mla_tensor* page_table,
                             const mla_tensor* cache_lens, const mla_tensor* latent_cache,
                             float scale, int32_t mask, mla_tensor* out, void* stream);

/* The split-KV partition count the library's balanced split gives each query row of a
 * dense decode (generic_flare_mla_decode_kv_cache_ragged: Args num_partitions_in, the
 * capturable-graph partition override).  Host only, no device access: the count is
 * planned for `batch` sequences of one query token each whose rows all hold
 * max_pages * page_size visible keys, on the current device's compute units.  Calls with
 * num_partitions <= 0 plan from the actual cache lengths on the device; passing this
 * value as num_partitions instead fixes the split of every row (rows shorter than the
 * longest then get the same number of smaller parts).  Returns 0 when an argument is out
 * of range (batch < 1 or above 2^24, num_heads not in {16, 32, 64, 128}, max_pages or
 * page_size < 1, or max_pages * page_size above 2^30). */
int32_t mla_decode_num_partitions(int64_t batch, int64_t num_heads, int64_t max_pages,
                                  int32_t page_size);

/*
 * mla_decode_paged without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops that forbid hipMalloc.  Same
 * arguments, results and errors as mla_decode_paged; the split-KV workspace is a fixed
 * array of mla_decode_noalloc_scratch_bytes() bytes of device memory that the library
 * holds on each GPU it runs on until the process ends (65.5 MiB: the balanced split of up
 * to 128 heads over up to 256 compute units, or a fixed split of up to 512 part slots of
 * 128 heads, and a split table of up to 2^16 query rows).  A call needing more returns
 * MLA_ERR_WORKSPACE before launching anything.  The call never allocates (no hipMalloc,
 * no hipFree); its first call on a device looks the array up and clears its header with a
 * kernel on `stream` (outside capture it then synchronises `stream` once).  Every call on
 * one GPU shares that array: calls that overlap in time on one GPU (different streams, or
 * graph replays running concurrently) race and must not be issued.  Its device error word
 * is read and cleared by mla_check_device_errors (any stream of the device).
 */
mla_status mla_decode_paged_noalloc(const mla_tensor* q, const mla_tensor* input_row_offsets,
                                    const mla_tensor* page_table, const mla_tensor* cache_lens,
                                    const mla_tensor* latent_cache, float scale, int32_t mask,
                                    int32_t local_window_size, int32_t num_partitions,
                                    mla_tensor* out, void* stream);

/* Size in bytes of the per-GPU array mla_decode_paged_noalloc works in (host only). */
size_t mla_decode_noalloc_scratch_bytes(void);

/* Workspace bytes a decode call with these sizes needs (host only, no device access).
 * num_partitions as in mla_decode_paged; device selects the CU count (-1 = current). */
size_t mla_decode_workspace_bytes(int64_t total_q, int32_t num_heads, int32_t num_partitions,
                                  int32_t device);

/* Workspace bytes an indexer call needs (host only, no device access): total_q query
 * tokens over a page table of max_pages pages of page_size rows.  The call keeps each
 * token's scored keys (8 bytes per row of the table, the row count rounded up to even)
 * and, per 1,024-row slice of it, the size and start of each top-digit run (2 KiB).
 * Reserve this on a stream before capturing an indexer call on it. */
size_t mla_indexer_workspace_bytes(int64_t total_q, int32_t max_pages, int32_t page_size);

/* Grow the workspace of (device, stream) to at least `bytes` (allocates and clears it;
 * not allowed while `stream` is capturing).  device -1 = the current device. */
mla_status mla_reserve_workspace(int32_t device, void* stream, size_t bytes);

/* Synchronise `stream`, read and clear the device error word of (device, stream), and of
 * the device's no-allocation scratch array once mla_decode_paged_noalloc has run there:
 * bit 0 a page id outside [0, num_pages) was met, bit 1 a sparse index outside the
 * pool, bit 2 offsets that decrease or exceed the q rows, bit 3 a cache length above
 * max_pages * PS.  *flags receives the word (0 = clean). */
mla_status mla_check_device_errors(int32_t device, void* stream, uint32_t* flags);

/* Kernel timing for measurement tools.  Enabling creates a ring of 4096 HIP event pairs
 * once (no event is created on a call's path) and restarts the count.  While enabled,
 * every call brackets its main kernel (the attention kernel, not the combine) with the
 * next pair, recorded on the call's stream; calls past the ring's capacity are not timed.
 * mla_profile_read_each synchronises the pairs used since the last read, writes each
 * bracketed launch's milliseconds (up to `capacity` of them, in call order), sets
 * *launches to the number bracketed and starts over; it returns MLA_ERR_WORKSPACE when
 * launches went untimed because the ring was full.  mla_profile_read gives their sum
 * instead.  Leave timing disabled (the default) in graph-captured code.  Host-side
 * bookkeeping only; mla_shutdown destroys the ring. */
mla_status mla_profile_enable(int32_t enable);
mla_status mla_profile_read_each(double* ms_each, int64_t capacity, int64_t* launches);
mla_status mla_profile_read(double* total_ms, int64_t* launches);

/* Free every workspace the library holds (all devices, all streams, retired ones
 * included) and the timing events.  Graphs captured from library calls must not be
 * replayed afterwards. */
void mla_shutdown(void);

const char* mla_status_string(mla_status s);
/* Detail of the last failed call on this host thread ("" if none). */
const char* mla_last_error_message(void);
/* Library version string. */
const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA355_H_ */
