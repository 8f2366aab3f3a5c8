"""Float64 CPU oracle for MLA attention over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The library
(``mla_decode_paged_02_amd``) never does, and this module imports nothing from it:
the two share no code.  Inputs arrive as NumPy arrays in their storage formats
(bfloat16 bit patterns, OCP E4M3 codes) and are widened here, exactly, to float64.

Sources, cited by page title and section (Modular MAX kernel-library API reference):

  [DEC] generic_flare_mla_decode_kv_cache_ragged: summary; Parameters (mask_str,
        sparse_mla); Args (q, input_row_offsets, scale, output, q_scale_ptr,
        d_indices, indices_stride, topk_lengths, num_partitions_in).
  [PRE] generic_flare_mla_prefill_kv_cache_ragged: summary; Parameters (mask_str);
        Args (q, k, v, buffer_row_offsets, cache_offsets, input_row_offsets, scale,
        output).
  [BR]  mla_decode_branch_fp8: summary (q_full = concat(q_nope_proj, q_rope), then
        MLA decode, then the w_uv projection); Args (q, w_uk, w_uv shapes).
  [IDX] mla_indexer_ragged_float8_paged: Args (output_indices, filled with -1 where
        fewer keys are valid; k scales with head_size granularity).

What it computes.  The method is scaled dot-product attention, reached exactly (up to
rounding order) through paging, online softmax and split-KV partitions, so this oracle
is the plain definition written out: gather the visible keys of a query row in logical
order, s = scale * q k^T, p = exp(s - max s), out = sum p v / sum p, and the
log-sum-exp lse = max s + log(sum p).

Readings of points the pages leave open (each also listed in the design notes):

  * cache_lens[b] counts the valid cache rows of sequence b, the rows of the current
    query tokens included; query token j of the n tokens of b sits at position
    L - n + j ([DEC] Args input_row_offsets; the cache is written before attention).
  * Each 576-wide row is [latent (512) | rope (64)] ([BR] summary: concat of the
    projected no-rope part and the rope part, in that order).  The decode output lives
    in the 512-wide latent space that w_uv maps back from ([BR] Args w_uv is
    [num_heads, v_head_dim, kv_latent_dim]), so V = latent columns 0..511.
  * Masks ([DEC] Parameters mask_str): "null" sees keys 0..L-1, "causal" keys
    0..pos, "sliding_window_causal" keys pos-W+1..pos (W = local_window_size;
    parity unpinned for the window width convention).
  * An empty visible set yields out = 0 and lse = -inf (parity unpinned convention).
  * Sparse rows ([DEC] Args d_indices / indices_stride / topk_lengths): row t of
    d_indices lists physical cache rows (page * page_size + slot); only the first
    topk_lengths[t] entries count, negative entries (the -1 fill of [IDX]) and rows
    outside the pool are skipped, listed order and duplicates are kept, and no
    positional mask applies.  Dequantised value = code value * scale; a missing q
    scale means 1.0 ([DEC] Args q_scale_ptr), a missing cache scale likewise.
  * Prefill ([PRE] Args): k holds the per-head no-rope part (128), the 64 rope
    columns of each key come from the paged latent cache (columns 512..575 at the
    key's cache position) and are shared by all heads; v is per head (128).  Key i
    of sequence b is k/v row buffer_row_offsets[b] + i at cache position
    cache_offsets[b] + i; query j is at cache_lens[b] - n_b + j.

  * Rope-aware layout ([DEC] Parameters per_token_scale_rope_aware, which names an
    interleaved FP8+BF16 layout of q and the cache without fixing it): each 576-wide
    head row is stored as 640 bytes, its 512 latent values as E4M3 codes followed by
    its 64 rope values as little-endian bfloat16; the token's (q) or row's (cache)
    float32 scale multiplies the latent codes only, the rope values are taken as
    stored.  V is the dequantised latent part, as above.

  * Shared index lists ([DEC] Parameters fold_shared_index, "read-once shared-index MTP
    fold", with no formula): every query token of sequence b (rows off[b] .. off[b+1]-1
    of input_row_offsets) attends to sequence b's one index list (row b of d_indices,
    its first topk_lengths[b] entries, by the rules above), so the list's rows serve all
    of the sequence's tokens.  The result is the sparse decode with each token given its
    sequence's list.

  * Attention sink and second KV stream ([DEC] Args attn_sink_ptr, extra_k,
    extra_d_indices, extra_indices_stride, extra_topk_lengths, extra_scales_ptr; the
    page names them without a formula): the sink is one logit per head, shared by the
    whole batch and not multiplied by scale, that joins the softmax denominator and
    carries no value; the extra stream is a second index list per query row over a
    second fp8 cache with its own row scales, and the row attends to the rows of both
    lists under one softmax.

Pins: every function here is checked in tests/test_oracle_pins.py against brute
force, closed forms and invariants.  Parity unpinned: the sliding-window width
convention, the empty-set convention, duplicate sparse indices (only their listed
multiplicity is defined by the reading above), and the attention-sink and
extra-stream semantics (the pins check the reading above, which no page fixes).
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 576
LATENT_DIM = 512
ROPE_DIM = 64
PREFILL_NOPE_DIM = 128
PREFILL_V_DIM = 128

MASKS = ("null", "causal", "sliding_window_causal")


# --------------------------------------------------------------------------------------
# storage formats -> float64
# --------------------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen the bits, then to float64."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return u32.view(np.float32).astype(np.float64)


def e4m3_value(code: int) -> float:
    """OCP 8-bit floating point E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits, no infinities, S.1111.111 is NaN, exponent field 0 is subnormal."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man = code & 0x7
    if exp_field == 0xF and man == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp_field - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------------------------------
# the definition of attention for one query row
# --------------------------------------------------------------------------------------

def attend(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
           visible: np.ndarray | None = None, return_probs: bool = False,
           sink: np.ndarray | None = None):
    """softmax(scale * q k^T) v for every query row (a head, or a query of one head).

    q_rows [R, Dk], keys [N, Dk], values [N, Dv] (float64); ``visible`` [R, N] marks
    the keys each row may see (all when None).  Returns out [R, Dv] and lse [R] (the
    natural log of sum_r exp(s_r) over visible keys), plus the probabilities [R, N] on
    request.  A row that sees no key gets out = 0 and lse = -inf.

    ``sink`` [R] (optional): one more logit per row, already in logit units (not scaled),
    that joins the softmax denominator and carries no value ([DEC] Args attn_sink_ptr;
    the reading used here): out = sum_r e^{s_r} v_r / (e^{sink} + sum_r e^{s_r}), and
    lse includes e^{sink}.  A row with no visible key then gets out = 0, lse = sink.
    """
    R = q_rows.shape[0]
    N = keys.shape[0]
    out = np.zeros((R, values.shape[1]))
    lse = np.full(R, -np.inf)
    probs = np.zeros((R, N))
    snk = np.full(R, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64).reshape(R)
    s = float(scale) * (q_rows @ keys.T) if N > 0 else np.zeros((R, 0))
    if visible is not None and N > 0:
        s = np.where(visible, s, -np.inf)
    row_max = s.max(axis=1, initial=-np.inf)
    m = np.maximum(row_max, snk)
    live = ~np.isneginf(m)  # NaN logits propagate; only a row with nothing to weigh is empty
    if live.any():
        ml = m[live]
        p = np.exp(s[live] - ml[:, None])
        l = p.sum(axis=1) + np.exp(snk[live] - ml)
        out[live] = (p @ values) / l[:, None]
        lse[live] = ml + np.log(l)
        probs[live] = p / l[:, None]
    if return_probs:
        return out, lse, probs
    return out, lse


def combine(partials):
    """Merge attention results over disjoint key sets by their log-sum-exp weights.

    partials: iterable of (out [H, Dv], lse [H]).  A part with lse = -inf (no keys)
    carries no weight; if every part is empty the result is zeros and -inf.
    """
    partials = list(partials)
    outs = np.stack([o for o, _ in partials])        # [P, H, Dv]
    lses = np.stack([l for _, l in partials])        # [P, H]
    M = lses.max(axis=0)                             # [H]
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Msafe[None, :]), 0.0)
    wsum = w.sum(axis=0)
    out = np.einsum("ph,phd->hd", w, outs) / np.where(finite, wsum, 1.0)[:, None]
    out[~finite] = 0.0
    lse = np.where(finite, Msafe + np.log(np.where(finite, wsum, 1.0)), -np.inf)
    return out, lse


# --------------------------------------------------------------------------------------
# paging and masking
# --------------------------------------------------------------------------------------

def visible_range(L: int, n: int, j: int, mask: str, window: int = -1):
    """Keys [lo, hi) that query token j (of n) of a sequence with L cache rows sees."""
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    if mask == "null":
        return 0, L
    pos = L - n + j
    hi = max(0, min(pos + 1, L))
    lo = 0
    if mask == "sliding_window_causal" and window is not None and window > 0:
        lo = max(0, pos - window + 1)
    return min(lo, hi), hi


def value_columns(keys: np.ndarray) -> np.ndarray:
    """V of a cache row is its latent part, columns 0..511 (see the header's readings)."""
    return keys[:, :LATENT_DIM]


def logical_rows(cache: np.ndarray, page_table_row: np.ndarray, positions: np.ndarray,
                 page_size: int) -> np.ndarray:
    """Cache rows at logical positions: page page_table_row[pos // PS], slot pos % PS."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[positions // page_size]
    return cache[pages, positions % page_size]


# --------------------------------------------------------------------------------------
# dense decode
# --------------------------------------------------------------------------------------

def decode_paged_f64(q, input_row_offsets, page_table, cache_lens, cache, page_size, scale,
                     mask="causal", window=-1, rows=None):
    """Dense MLA decode on float64 arrays ([DEC] summary and Args).

    q [T, H, 576], cache [num_pages, PS, 576].  Returns (out [R, H, 512], lse [R, H])
    for the requested q rows (all rows by default, in order).
    """
    T, H, _ = q.shape
    off = np.asarray(input_row_offsets, dtype=np.int64)
    rows = list(range(T)) if rows is None else [int(r) for r in rows]
    where = {t: i for i, t in enumerate(rows)}
    out = np.zeros((len(rows), H, LATENT_DIM))
    lse = np.full((len(rows), H), -np.inf)
    for b in range(len(cache_lens)):
        n = int(off[b + 1] - off[b])
        wanted = [j for j in range(n) if int(off[b]) + j in where]
        if not wanted:
            continue
        L = int(cache_lens[b])
        keys = logical_rows(cache, page_table[b], np.arange(L), page_size) if L > 0 \
            else np.zeros((0, HEAD_DIM))
        for j in wanted:
            t = int(off[b]) + j
            lo, hi = visible_range(L, n, j, mask, window)
            k = keys[lo:hi]
            o, l = attend(q[t], k, value_columns(k), scale)
            out[where[t]] = o
            lse[where[t]] = l
    return out, lse


def decode_paged(q_bits, input_row_offsets, page_table, cache_lens, cache_bits, page_size,
                 scale, mask="causal", window=-1, rows=None):
    """Dense MLA decode on bfloat16 storage (bit patterns), evaluated in float64."""
    return decode_paged_f64(bf16_to_f64(q_bits), input_row_offsets, page_table, cache_lens,
                            _LazyBF16(cache_bits), page_size, scale, mask, window, rows)


class _LazyBF16:
    """Widens only the gathered rows of a large bf16 cache (indexing returns float64)."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return bf16_to_f64(self.bits[idx])


# --------------------------------------------------------------------------------------
# sparse decode
# --------------------------------------------------------------------------------------

def sparse_rows(d_indices_row, topk_length, pool_rows):
    """Physical rows that count for one index list ([DEC] Args d_indices, topk_lengths)."""
    listed = np.asarray(d_indices_row[:max(0, int(topk_length))], dtype=np.int64)
    return listed[(listed >= 0) & (listed < pool_rows)]


def decode_sparse_f64(q, input_row_offsets, cache, d_indices, topk_lengths, page_size, scale,
                      rows=None, extra=None, attn_sink=None):
    """Sparse decode on float64 arrays (already dequantised): q [T, H, 576],
    cache [num_pages, PS, 576]; each q row attends to its listed rows, no positional mask.

    extra = (cache2, d_indices2, topk_lengths2, page_size2) (optional): a second KV stream
    ([DEC] Args extra_k, extra_d_indices, extra_indices_stride, extra_topk_lengths; the
    reading used here): row t's second list names rows of cache2 by the same rules, and
    row t attends to the rows of both lists under one softmax.
    attn_sink [H] (optional): one sink logit per head shared by the batch ([DEC] Args
    attn_sink_ptr, read as one weight set for the whole batch), see attend()."""
    T, H, _ = q.shape
    rows = list(range(T)) if rows is None else [int(r) for r in rows]
    pool_rows = cache.shape[0] * page_size
    out = np.zeros((len(rows), H, LATENT_DIM))
    lse = np.full((len(rows), H), -np.inf)
    for i, t in enumerate(rows):
        phys = sparse_rows(d_indices[t], topk_lengths[t], pool_rows)
        k = cache[phys // page_size, phys % page_size]
        if extra is not None:
            cache2, idx2, topk2, ps2 = extra
            phys2 = sparse_rows(idx2[t], topk2[t], cache2.shape[0] * ps2)
            k = np.concatenate([k, cache2[phys2 // ps2, phys2 % ps2]], axis=0)
        out[i], lse[i] = attend(q[t], k, value_columns(k), scale, sink=attn_sink)
    return out, lse


def decode_sparse(q8, q_scale, input_row_offsets, cache8, cache_scale, d_indices, topk_lengths,
                  page_size, scale, rows=None, extra=None, attn_sink=None):
    """Sparse FP8 decode: values are E4M3 code value times the float32 scale of the q
    token / cache row ([DEC] Args q_scale_ptr; [IDX] Args k_collection scales).

    extra = (cache8_2, cache_scale_2, d_indices_2, topk_lengths_2, page_size_2) names the
    second KV stream with its own row scales ([DEC] Args extra_k, extra_scales_ptr,
    extra_d_indices, extra_topk_lengths); attn_sink [H] the sink logits (see
    decode_sparse_f64)."""
    q = e4m3_to_f64(q8)
    if q_scale is not None:
        q = q * np.asarray(q_scale, dtype=np.float64)[:, None, None]
    cache = _LazyE4M3(cache8, cache_scale)
    ex = None
    if extra is not None:
        c8b, csb, idxb, topkb, psb = extra
        ex = (_LazyE4M3(c8b, csb), idxb, topkb, psb)
    return decode_sparse_f64(q, input_row_offsets, cache, d_indices, topk_lengths, page_size,
                             scale, rows, extra=ex, attn_sink=attn_sink)


def decode_paged_fp8(q8, q_scale, input_row_offsets, page_table, cache_lens, cache8, cache_scale,
                     page_size, scale, mask="causal", window=-1, rows=None):
    """Dense MLA decode over a paged FP8 cache ([DEC] Args q_scale_ptr, kv_collection;
    Parameters mask_str, local_window_size, per_token_scale_rope_aware = False): every stored
    value is its E4M3 code value times the float32 scale of its q token (shared by the
    heads) or cache row (all 576 columns); then the dense decode, in float64."""
    q = e4m3_to_f64(q8)
    if q_scale is not None:
        q = q * np.asarray(q_scale, dtype=np.float64)[:, None, None]
    return decode_paged_f64(q, input_row_offsets, page_table, cache_lens, _LazyE4M3(cache8, cache_scale),
                            page_size, scale, mask, window, rows)


def token_lists(input_row_offsets, d_indices_seq, topk_seq):
    """Per-token index lists from per-sequence ones ([DEC] Parameters fold_shared_index):
    token t of sequence b takes row b of the lists and its top-k length."""
    off = np.asarray(input_row_offsets, dtype=np.int64)
    seq_of = np.repeat(np.arange(len(off) - 1), np.diff(off))
    return np.asarray(d_indices_seq)[seq_of], np.asarray(topk_seq)[seq_of]


def decode_sparse_shared(q8, q_scale, input_row_offsets, cache8, cache_scale, d_indices_seq, topk_seq,
                         page_size, scale, rows=None):
    """Sparse FP8 decode where the query tokens of a sequence share its index list
    (d_indices_seq [B, stride], topk_seq [B]); see token_lists."""
    idx, topk = token_lists(input_row_offsets, d_indices_seq, topk_seq)
    return decode_sparse(q8, q_scale, input_row_offsets, cache8, cache_scale, idx, topk, page_size, scale, rows)


ROPE_ROW_BYTES = LATENT_DIM + 2 * ROPE_DIM  # 640


def rope_aware_to_f64(raw, scales):
    """Rows in the rope-aware layout ([DEC] Parameters per_token_scale_rope_aware) to
    float64 [..., 576]: bytes 0..511 are E4M3 latent codes, times the row's scale
    (None = 1); bytes 512..639 are the 64 rope values, little-endian bfloat16, unscaled."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    assert raw.shape[-1] == ROPE_ROW_BYTES, raw.shape
    lat = e4m3_to_f64(raw[..., :LATENT_DIM])
    if scales is not None:
        lat = lat * np.asarray(scales, dtype=np.float64)[..., None]
    rope_bits = np.ascontiguousarray(raw[..., LATENT_DIM:]).view("<u2")
    return np.concatenate([lat, bf16_to_f64(rope_bits)], axis=-1)


class _LazyRopeAware:
    """Dequantises only the gathered rows of a large rope-aware cache."""

    def __init__(self, raw, scales):
        self.raw = raw
        self.scales = scales
        self.shape = raw.shape[:-1] + (HEAD_DIM,)

    def __getitem__(self, idx):
        return rope_aware_to_f64(self.raw[idx], None if self.scales is None else self.scales[idx])


def _rope_aware_q(q_raw, q_scale):
    T, H = q_raw.shape[:2]
    qs = None if q_scale is None else np.broadcast_to(np.asarray(q_scale, dtype=np.float64)[:, None], (T, H))
    return rope_aware_to_f64(q_raw, qs)


def decode_paged_fp8_rope_aware(q_raw, q_scale, input_row_offsets, page_table, cache_lens, cache_raw,
                                cache_scale, page_size, scale, mask="causal", window=-1, rows=None):
    """Dense MLA decode with q [T, H, 640] and the paged cache [pages, PS, 640] in the
    rope-aware layout (see rope_aware_to_f64; q_scale [T] per token, cache_scale
    [pages, PS] per row), then the dense decode in float64."""
    q = _rope_aware_q(q_raw, q_scale)
    return decode_paged_f64(q, input_row_offsets, page_table, cache_lens, _LazyRopeAware(cache_raw, cache_scale),
                            page_size, scale, mask, window, rows)


def decode_sparse_rope_aware(q_raw, q_scale, input_row_offsets, cache_raw, cache_scale, d_indices,
                             topk_lengths, page_size, scale, rows=None):
    """Sparse decode ([DEC] Parameters sparse_mla) over a rope-aware cache."""
    q = _rope_aware_q(q_raw, q_scale)
    return decode_sparse_f64(q, input_row_offsets, _LazyRopeAware(cache_raw, cache_scale), d_indices,
                             topk_lengths, page_size, scale, rows)


# --------------------------------------------------------------------------------------
# FP8 top-k indexer
# --------------------------------------------------------------------------------------

def indexer_scores(q8_t, q_s_t, k8_rows, k_scale_rows):
    """Scores of one query token against cache rows ([IDX] summary: the FP8 product of q
    and the cached k with their scales, summed over all heads):
    score[r] = sum_h q_s[h] * <e4m3(q[h]), e4m3(k[r])> * k_scale[r], in float64."""
    q = e4m3_to_f64(q8_t)                               # [NH, D]
    k = e4m3_to_f64(k8_rows)                            # [R, D]
    per_head = k @ q.T                                  # [R, NH]
    s = per_head @ np.asarray(q_s_t, dtype=np.float64)  # sum over heads
    if k_scale_rows is not None:
        s = s * np.asarray(k_scale_rows, dtype=np.float64)
    return s


def rank_order(scores, positions):
    """Indices that sort the scored rows for the top-k: descending score, equal scores by
    ascending logical position (the reading of [IDX] Args output_indices used here)."""
    return np.lexsort((np.asarray(positions), -np.asarray(scores, dtype=np.float64)))


def indexer_paged_fp8(q8, q_s, input_row_offsets, page_table, cache_lens, k8, k_scale, page_size,
                      top_k, mask="causal", window=-1, return_scores=False):
    """FP8 top-k indexer over a paged cache ([IDX] summary and Args output_indices, q, q_s,
    input_row_offsets, k_collection).  Query token j of sequence b scores the rows its
    mask leaves visible (the decode visibility); row t of the result holds the top_k
    highest-scoring rows, as physical rows page_id * PS + slot, by descending score and
    equal scores by ascending position, then -1.  With return_scores, also the visible
    logical positions and their scores per row."""
    T = q8.shape[0]
    off = np.asarray(input_row_offsets, dtype=np.int64)
    out = np.full((T, top_k), -1, dtype=np.int64)
    seen = []
    for b in range(len(cache_lens)):
        n = int(off[b + 1] - off[b])
        L = int(cache_lens[b])
        for j in range(n):
            t = int(off[b]) + j
            lo, hi = visible_range(L, n, j, mask, window)
            pos = np.arange(lo, hi, dtype=np.int64)
            pages = np.asarray(page_table[b], dtype=np.int64)[pos // page_size]
            slots = pos % page_size
            ks = None if k_scale is None else k_scale[pages, slots]
            sc = indexer_scores(q8[t], q_s[t], k8[pages, slots], ks) if len(pos) else np.zeros(0)
            take = rank_order(sc, pos)[:top_k]
            out[t, :len(take)] = pages[take] * page_size + slots[take]
            seen.append((t, pos, sc))
    return (out, seen) if return_scores else out


class _LazyE4M3:
    """Dequantises only the gathered rows of a large E4M3 cache."""

    def __init__(self, codes, scales):
        self.codes = codes
        self.scales = scales
        self.shape = codes.shape

    def __getitem__(self, idx):
        v = e4m3_to_f64(self.codes[idx])
        if self.scales is not None:
            v = v * np.asarray(self.scales[idx], dtype=np.float64)[..., None]
        return v


# --------------------------------------------------------------------------------------
# ragged prefill
# --------------------------------------------------------------------------------------

def prefill_paged_f64(q, k, v, buffer_row_offsets, cache_offsets, input_row_offsets, page_table,
                      cache_lens, cache, page_size, scale, mask="causal", rows=None, heads=None):
    """Ragged MLA prefill on float64 arrays ([PRE] summary and Args).

    q [Tq, H, 192] = [no-rope 128 | rope 64], k [Tk, H, 128], v [Tk, H, 128],
    cache [num_pages, PS, 576] supplies rope columns 512..575.  Returns out
    [R, H', 128] for the requested q rows and heads (all by default).
    """
    Tq, H, _ = q.shape
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    rows = list(range(Tq)) if rows is None else [int(r) for r in rows]
    where = {t: i for i, t in enumerate(rows)}
    in_off = np.asarray(input_row_offsets, dtype=np.int64)
    bro = np.asarray(buffer_row_offsets, dtype=np.int64)
    out = np.zeros((len(rows), len(heads), PREFILL_V_DIM))
    for b in range(len(cache_lens)):
        n = int(in_off[b + 1] - in_off[b])
        wanted = [j for j in range(n) if int(in_off[b]) + j in where]
        if not wanted:
            continue
        nk = int(bro[b + 1] - bro[b])
        L = int(cache_lens[b])
        apos = int(cache_offsets[b]) + np.arange(nk)                   # cache position of key i
        rope = logical_rows(cache, page_table[b], apos, page_size)[:, LATENT_DIM:]   # [nk, 64]
        qpos = np.array([L - n + j for j in wanted])                   # positions of the queries
        if mask == "null":
            vis = np.ones((len(wanted), nk), dtype=bool)
        elif mask == "causal":
            vis = apos[None, :] <= qpos[:, None]
        else:
            raise ValueError(f"prefill mask {mask!r} not covered")
        qrows = [int(in_off[b]) + j for j in wanted]
        dst = [where[t] for t in qrows]
        for hi, h in enumerate(heads):
            kf = np.concatenate([k[bro[b]:bro[b] + nk, h, :], rope], axis=1)   # [nk, 192]
            vh = v[bro[b]:bro[b] + nk, h, :]
            qh = np.stack([q[t, h] for t in qrows])                           # [n', 192]
            o, _ = attend(qh, kf, vh, scale, visible=vis)
            out[dst, hi] = o
    return out


def prefill_paged(q_bits, k_bits, v_bits, buffer_row_offsets, cache_offsets, input_row_offsets,
                  page_table, cache_lens, cache_bits, page_size, scale, mask="causal", rows=None,
                  heads=None):
    """Ragged MLA prefill on bfloat16 storage, evaluated in float64."""
    return prefill_paged_f64(_LazyBF16(q_bits), _LazyBF16(k_bits), _LazyBF16(v_bits),
                             buffer_row_offsets, cache_offsets, input_row_offsets, page_table,
                             cache_lens, _LazyBF16(cache_bits), page_size, scale, mask, rows, heads)
