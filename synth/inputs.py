"""Seeded synthetic inputs for MLA attention over a paged latent cache.

This module only draws random numbers, rounds them to their storage formats and lays
them out the way the kernels and the oracle read them: a paged cache, a page table,
ragged row offsets and sparse row-index lists.  It performs none of the attention
arithmetic, so the CPU oracle and the GPU path consume exactly the same bytes without
sharing any part of the method.

Storage layouts (row-major, little-endian; "bf16" arrays hold raw bfloat16 bit
patterns as uint16, "e4m3" arrays hold OCP FP8 E4M3 codes as uint8):

  q                  bf16  [T, H, 576]       cols 0..511 latent, 512..575 rope
  latent_cache       bf16  [num_pages, PS, 576]
  page_table         int32 [B, max_pages]    entries past a sequence's pages are -1
  cache_lens         int32 [B]               valid cache rows, current tokens included
  input_row_offsets  uint32 [B + 1]          q rows of sequence b are [off[b], off[b+1])
  rope-aware q8 / cache8  uint8 [..., 640]   512 e4m3 latent codes, then 64 bf16 rope
                                             values (little-endian); see rope_aware()

Draws: a Generator seeded with ``seed`` gives, in this order, the lengths / top-k
counts, the page permutation and the sparse index lists; the large value arrays come
from child streams of SeedSequence([seed, tag]) with tag 1 = q, 2 = cache, 3 = prefill
k, 4 = prefill v, 11 / 12 = rope-aware q / cache rope values (split into a fixed number of chunks, so the bytes never depend on
the host's thread count).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 576       # latent (512) + rope (64)
LATENT_DIM = 512
ROPE_DIM = 64
PREFILL_QK_DIM = 192  # per-head no-rope (128) + rope (64)
PREFILL_V_DIM = 128
PREFILL_NOPE_DIM = 128

BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F

__all__ = [
    "HEAD_DIM", "LATENT_DIM", "ROPE_DIM", "PREFILL_QK_DIM", "PREFILL_V_DIM",
    "PREFILL_NOPE_DIM", "BF16_NAN_BITS", "E4M3_NAN_CODE", "default_scale", "rope_aware",
    "bf16_bits", "e4m3_codes", "DecodeCase", "SparseCase", "PrefillCase",
    "make_decode_case", "make_sparse_case", "make_shared_sparse_case", "make_prefill_case", "config_case",
    "CONFIG_DESCRIPTIONS", "algorithmic_bytes", "algorithmic_flops",
    "IndexerCase", "make_indexer_case", "indexer_config",
]


def default_scale() -> float:
    """1/sqrt(192) rounded to float32 (the un-absorbed q/k head width of 128 + 64)."""
    return float(np.float32(1.0 / math.sqrt(192.0)))


# --------------------------------------------------------------------------------------
# storage-format encoders (input preparation only)
# --------------------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # uint32 wrap-around can only happen for NaN bit patterns, which are replaced below
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_NAN_BITS
    return rounded


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Encode float32 values (|x| <= 448) as OCP E4M3 codes via torch's float8_e4m3fn cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _quantise_rows(x: np.ndarray, axis) -> tuple[np.ndarray, np.ndarray]:
    """Per-row absmax scaling to the E4M3 range: scale = amax/448 (1 for all-zero rows)."""
    amax = np.max(np.abs(x), axis=axis, keepdims=True)
    sc = (amax / np.float32(448.0)).astype(np.float32)
    sc = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
    codes = e4m3_codes(np.clip(x / sc, -448.0, 448.0))
    return codes, np.squeeze(sc, axis=axis).astype(np.float32)


_CHUNKS = 16  # fixed split of large draws, so the bytes do not depend on the host


def _normal_bf16(seed, tag, shape, std=1.0, as_bits=True):
    """N(0, std^2) float32 draws of ``shape``, rounded to bf16 bits (or kept as float32).

    Large arrays are split along the leading axis into a fixed number of chunks, each
    drawn from its own child stream of SeedSequence([seed, tag]) and filled in parallel.
    """
    from concurrent.futures import ThreadPoolExecutor

    shape = tuple(int(d) for d in shape)
    out = np.empty(shape, dtype=np.uint16 if as_bits else np.float32)
    if out.size == 0:
        return out
    n0 = shape[0]
    step = -(-n0 // _CHUNKS)
    bounds = [(i, min(n0, i + step)) for i in range(0, n0, step)]
    children = np.random.SeedSequence([int(seed), int(tag)]).spawn(len(bounds))

    def fill(k):
        a, b = bounds[k]
        x = np.random.default_rng(children[k]).standard_normal((b - a,) + shape[1:], dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[a:b] = bf16_bits(x) if as_bits else x

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range(len(bounds))))
    return out


def _normal_e4m3_rows(seed, tag, shape):
    """N(0,1) draws of ``shape`` quantised to E4M3 with one float32 scale per last-axis row.

    Uses the same chunked child streams as ``_normal_bf16`` (identical draws for a given
    seed, tag and shape); returns (codes uint8 [shape], scales float32 [shape[:-1]]).
    """
    from concurrent.futures import ThreadPoolExecutor

    shape = tuple(int(d) for d in shape)
    codes = np.empty(shape, dtype=np.uint8)
    scales = np.empty(shape[:-1], dtype=np.float32)
    n0 = shape[0]
    step = -(-n0 // _CHUNKS)
    bounds = [(i, min(n0, i + step)) for i in range(0, n0, step)]
    children = np.random.SeedSequence([int(seed), int(tag)]).spawn(len(bounds))

    def fill(k):
        a, b = bounds[k]
        x = np.random.default_rng(children[k]).standard_normal((b - a,) + shape[1:], dtype=np.float32)
        codes[a:b], scales[a:b] = _quantise_rows(x, axis=len(shape) - 1)

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range(len(bounds))))
    return codes, scales


# --------------------------------------------------------------------------------------
# paging helpers (layout only)
# --------------------------------------------------------------------------------------

def _page_layout(rng, lens, page_size, spare_pages, shuffle, max_pages=None):
    """Assign physical pages to each sequence's logical pages from a seeded permutation."""
    lens = np.asarray(lens, dtype=np.int64)
    npages = (lens + page_size - 1) // page_size
    total = int(npages.sum()) + int(spare_pages)
    perm = rng.permutation(total).astype(np.int32) if shuffle else np.arange(total, dtype=np.int32)
    width = int(max(1, npages.max() if len(npages) else 1))
    if max_pages is not None:
        assert max_pages >= width
        width = int(max_pages)
    table = np.full((len(lens), width), -1, dtype=np.int32)
    cur = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[cur:cur + n]
        cur += n
    spare = perm[cur:]
    return table, total, spare


def _poison_unused(cache, table, lens, page_size, spare, poison):
    """Fill page-tail slots and unreferenced pages with NaN (bf16) or the E4M3 NaN code."""
    for b, L in enumerate(np.asarray(lens)):
        n = (int(L) + page_size - 1) // page_size
        if n and L % page_size:
            cache[table[b, n - 1], L % page_size:, :] = poison
    for p in spare:
        cache[p] = poison


# --------------------------------------------------------------------------------------
# dense decode
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeCase:
    name: str
    q: np.ndarray | None           # uint16 [T, H, 576] (None for an fp8 case)
    input_row_offsets: np.ndarray  # uint32 [B + 1]
    page_table: np.ndarray         # int32 [B, max_pages]
    cache_lens: np.ndarray         # int32 [B]
    latent_cache: np.ndarray | None  # uint16 [num_pages, PS, 576] (None for an fp8 case)
    page_size: int
    scale: float
    mask: str = "causal"
    window: int = -1
    # fp8 cases: E4M3 codes with one float32 scale per q token / cache row
    q8: np.ndarray | None = None           # uint8 [T, H, 576]
    q_scale: np.ndarray | None = None      # float32 [T]
    cache8: np.ndarray | None = None       # uint8 [num_pages, PS, 576]
    cache_scale: np.ndarray | None = None  # float32 [num_pages, PS]

    @property
    def fp8(self) -> bool:
        return self.q8 is not None

    @property
    def batch(self) -> int:
        return int(self.cache_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int((self.q8 if self.fp8 else self.q).shape[0])

    @property
    def num_heads(self) -> int:
        return int((self.q8 if self.fp8 else self.q).shape[1])


def make_decode_case(seed, lens, num_heads, page_size, q_per_seq=1, mask="causal",
                     window=-1, tail="normal", spare_pages=0, shuffle=True,
                     q_std=1.0, cache_std=1.0, max_pages=None, fp8=False, name="decode"):
    """Dense decode inputs.  ``lens`` is a sequence or a callable rng -> lengths.

    fp8: q and cache as E4M3 codes of the same N(0,1) draws, with one float32 scale per q
    token (absmax over its heads) and per cache row (absmax over its 576 values)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens(rng) if callable(lens) else lens, dtype=np.int32)
    B = len(lens)
    n_q = np.broadcast_to(np.asarray(q_per_seq, dtype=np.int64), (B,))
    offsets = np.zeros(B + 1, dtype=np.uint32)
    offsets[1:] = np.cumsum(n_q)
    T = int(offsets[-1])
    table, total, spare = _page_layout(rng, lens, page_size, spare_pages, shuffle, max_pages)
    if fp8:
        qf = _normal_bf16(seed, 1, (T, num_heads, HEAD_DIM), q_std, as_bits=False)
        q8, q_scale = _quantise_rows(qf, axis=(1, 2))
        del qf
        c8, c_scale = _normal_e4m3_rows(seed, 2, (total, page_size, HEAD_DIM))
        if tail == "nan":
            _poison_unused(c8, table, lens, page_size, spare, np.uint8(E4M3_NAN_CODE))
            _poison_unused(c_scale[..., None], table, lens, page_size, spare, np.float32(np.nan))
        return DecodeCase(name=name, q=None, input_row_offsets=offsets, page_table=table,
                          cache_lens=lens, latent_cache=None, page_size=page_size,
                          scale=default_scale(), mask=mask, window=window, q8=q8,
                          q_scale=q_scale, cache8=c8, cache_scale=c_scale)
    q = _normal_bf16(seed, 1, (T, num_heads, HEAD_DIM), q_std)
    cache = _normal_bf16(seed, 2, (total, page_size, HEAD_DIM), cache_std)
    if tail == "nan":
        _poison_unused(cache, table, lens, page_size, spare, np.uint16(BF16_NAN_BITS))
    return DecodeCase(name=name, q=q, input_row_offsets=offsets, page_table=table,
                      cache_lens=lens, latent_cache=cache, page_size=page_size,
                      scale=default_scale(), mask=mask, window=window)


def rope_aware(case, seed):
    """The same fp8 case (DecodeCase or SparseCase) in the rope-aware layout: every 576-wide
    q head and cache row becomes 640 bytes, its first 512 E4M3 codes (scales unchanged)
    followed by 64 bfloat16 values (little-endian) drawn N(0,1).  Cache rows whose first
    code is the NaN code (poisoned slots) get NaN rope values too."""
    def convert(codes, tag):
        lead = codes.shape[:-1]
        rope = _normal_bf16(seed, tag, lead + (ROPE_DIM,))
        bad = codes[..., 0] == E4M3_NAN_CODE
        rope[bad] = BF16_NAN_BITS
        out = np.empty(lead + (LATENT_DIM + 2 * ROPE_DIM,), dtype=np.uint8)
        out[..., :LATENT_DIM] = codes[..., :LATENT_DIM]
        out[..., LATENT_DIM:] = rope.astype("<u2").view(np.uint8).reshape(lead + (2 * ROPE_DIM,))
        return out
    return dataclasses.replace(case, name=case.name + "-rope", q8=convert(case.q8, 11),
                               cache8=convert(case.cache8, 12))


# --------------------------------------------------------------------------------------
# sparse fp8 decode
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class SparseCase:
    name: str
    q8: np.ndarray                 # uint8 E4M3 [T, H, 576]
    q_scale: np.ndarray | None     # float32 [T] (one scale per q token) or None (= 1.0)
    input_row_offsets: np.ndarray  # uint32 [B + 1]
    cache8: np.ndarray             # uint8 E4M3 [num_pages, PS, 576]
    cache_scale: np.ndarray | None  # float32 [num_pages, PS] (one per cache row) or None
    d_indices: np.ndarray          # int32 [T, indices_stride], physical rows, -1 padded
    topk_lengths: np.ndarray       # int32 [T]
    page_size: int
    scale: float
    page_table: np.ndarray | None = None  # the logical->physical map the indices came from
    rows_per_seq: int = 0

    @property
    def total_q(self) -> int:
        return int(self.q8.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q8.shape[1])


def make_sparse_case(seed, batch, num_heads, rows_per_seq, page_size, topk_range,
                     n_index, poison=False, spare_pages=0, with_scales=True, name="sparse"):
    """Sparse decode inputs: E4M3 q and cache with float32 per-token / per-row scales.

    Each sequence owns ``rows_per_seq`` cache rows; its index list holds ``n_index``
    distinct logical positions drawn without replacement, translated to physical rows
    (page * PS + slot); entries at or past ``topk_lengths[b]`` are set to -1.
    """
    rng = np.random.default_rng(seed)
    lo, hi = topk_range
    topk = rng.integers(lo, hi, endpoint=True, size=batch).astype(np.int32)
    lens = np.full(batch, rows_per_seq, dtype=np.int32)
    table, total, spare = _page_layout(rng, lens, page_size, spare_pages, True)
    qf = _normal_bf16(seed, 1, (batch, num_heads, HEAD_DIM), as_bits=False)
    if with_scales:
        q8, q_scale = _quantise_rows(qf, axis=(1, 2))      # one scale per q token
        c8, c_scale = _normal_e4m3_rows(seed, 2, (total, page_size, HEAD_DIM))
    else:
        q8, q_scale = e4m3_codes(np.clip(qf, -448, 448)), None
        cf = _normal_bf16(seed, 2, (total, page_size, HEAD_DIM), as_bits=False)
        c8, c_scale = e4m3_codes(np.clip(cf, -448, 448)), None
        del cf
    del qf
    idx = np.full((batch, n_index), -1, dtype=np.int32)
    for b in range(batch):
        pos = rng.choice(rows_per_seq, n_index, replace=False)
        phys = table[b, pos // page_size].astype(np.int64) * page_size + pos % page_size
        idx[b] = phys.astype(np.int32)
        idx[b, topk[b]:] = -1
    if poison:
        listed = np.zeros(total * page_size, dtype=bool)
        for b in range(batch):
            rows = idx[b, :topk[b]]
            listed[rows[rows >= 0]] = True
        flat = c8.reshape(total * page_size, HEAD_DIM)
        flat[~listed] = E4M3_NAN_CODE
        if c_scale is not None:
            c_scale.reshape(-1)[~listed] = np.float32(np.nan)
    offsets = np.arange(batch + 1, dtype=np.uint32)
    return SparseCase(name=name, q8=q8, q_scale=q_scale, input_row_offsets=offsets,
                      cache8=c8, cache_scale=c_scale, d_indices=idx, topk_lengths=topk,
                      page_size=page_size, scale=default_scale(), page_table=table,
                      rows_per_seq=rows_per_seq)


def make_shared_sparse_case(seed, n_tokens, num_heads, rows_per_seq, page_size, topk_range, n_index,
                            name="shared"):
    """Sparse inputs with one index list per sequence shared by its query tokens: the
    lists, cache and scales of make_sparse_case(seed, len(n_tokens), ...), and q drawn for
    sum(n_tokens) tokens (with its per-token scales) from seed + 1.  input_row_offsets
    gives the tokens of each sequence; d_indices / topk_lengths have one row per sequence."""
    B, T = len(n_tokens), int(sum(n_tokens))
    base = make_sparse_case(seed, B, num_heads, rows_per_seq, page_size, topk_range, n_index, name=name)
    tok = make_sparse_case(seed + 1, T, num_heads, 64, 16, (1, 1), 1, name=name + "-q")
    off = np.zeros(B + 1, dtype=np.uint32)
    off[1:] = np.cumsum(n_tokens)
    return dataclasses.replace(base, q8=tok.q8, q_scale=tok.q_scale, input_row_offsets=off)


# --------------------------------------------------------------------------------------
# FP8 top-k indexer
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class IndexerCase:
    name: str
    q8: np.ndarray                 # uint8 E4M3 [T, NH, D]
    q_s: np.ndarray                # float32 [T, NH] (one scale per token and head)
    input_row_offsets: np.ndarray  # uint32 [B + 1]
    page_table: np.ndarray         # int32 [B, max_pages]
    cache_lens: np.ndarray         # int32 [B]
    k8: np.ndarray                 # uint8 E4M3 [num_pages, PS, D]
    k_scale: np.ndarray            # float32 [num_pages, PS] (one per cache row)
    page_size: int
    top_k: int
    mask: str = "causal"
    window: int = -1

    @property
    def total_q(self) -> int:
        return int(self.q8.shape[0])


def make_indexer_case(seed, lens, num_heads, depth, page_size, top_k, q_per_seq=1, mask="causal",
                      window=-1, name="indexer"):
    """Indexer inputs: N(0,1) draws quantised to E4M3, q scaled per (token, head) and the
    cache per row (absmax / 448), in a shuffled page pool."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens(rng) if callable(lens) else lens, dtype=np.int32)
    B = len(lens)
    n_q = np.broadcast_to(np.asarray(q_per_seq, dtype=np.int64), (B,))
    offsets = np.zeros(B + 1, dtype=np.uint32)
    offsets[1:] = np.cumsum(n_q)
    T = int(offsets[-1])
    table, total, _ = _page_layout(rng, lens, page_size, 0, True)
    q8, q_s = _normal_e4m3_rows(seed, 5, (T, num_heads, depth))
    k8, k_scale = _normal_e4m3_rows(seed, 6, (total, page_size, depth))
    return IndexerCase(name=name, q8=q8, q_s=q_s, input_row_offsets=offsets, page_table=table,
                       cache_lens=lens, k8=k8, k_scale=k_scale, page_size=page_size, top_k=top_k,
                       mask=mask, window=window)


def indexer_config():
    """The indexer in front of the sparse workload C4: 32 sequences of 16384 cache rows,
    one query token each, 64 indexer heads of width 128, top 2048 (seed 355005)."""
    return make_indexer_case(355_005, [16384] * 32, 64, 128, 64, 2048, name="X4")


# --------------------------------------------------------------------------------------
# ragged prefill
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillCase:
    name: str
    q: np.ndarray                   # uint16 [Tq, H, 192]
    k: np.ndarray                   # uint16 [Tk, H, 128]  (per-head no-rope part)
    v: np.ndarray                   # uint16 [Tk, H, 128]
    buffer_row_offsets: np.ndarray  # uint32 [B + 1] rows of k / v per sequence
    cache_offsets: np.ndarray       # uint32 [B] cache position of each sequence's k row 0
    input_row_offsets: np.ndarray   # uint32 [B + 1] rows of q / out per sequence
    page_table: np.ndarray          # int32 [B, max_pages]
    cache_lens: np.ndarray          # int32 [B]
    latent_cache: np.ndarray        # uint16 [num_pages, PS, 576] (rope = cols 512..575)
    page_size: int
    scale: float
    mask: str = "causal"

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])


def make_prefill_case(seed, new_lens, prefix_lens, num_heads, page_size, mask="causal",
                      shuffle=True, name="prefill"):
    """Ragged prefill: sequence b appends new_lens[b] tokens after prefix_lens[b] cached ones.

    k / v hold every key of the sequence (prefix + new), cache_offsets are 0, and the
    paged latent cache supplies the shared rope columns for all of them.
    """
    rng = np.random.default_rng(seed)
    new_lens = np.asarray(new_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    total_lens = (new_lens + prefix_lens).astype(np.int32)
    B = len(new_lens)
    in_off = np.zeros(B + 1, dtype=np.uint32)
    in_off[1:] = np.cumsum(new_lens)
    buf_off = np.zeros(B + 1, dtype=np.uint32)
    buf_off[1:] = np.cumsum(total_lens)
    table, total, _ = _page_layout(rng, total_lens, page_size, 0, shuffle)
    Tq, Tk = int(in_off[-1]), int(buf_off[-1])
    q = _normal_bf16(seed, 1, (Tq, num_heads, PREFILL_QK_DIM))
    cache = _normal_bf16(seed, 2, (total, page_size, HEAD_DIM))
    k = _normal_bf16(seed, 3, (Tk, num_heads, PREFILL_NOPE_DIM))
    v = _normal_bf16(seed, 4, (Tk, num_heads, PREFILL_V_DIM))
    return PrefillCase(name=name, q=q, k=k, v=v, buffer_row_offsets=buf_off,
                       cache_offsets=np.zeros(B, dtype=np.uint32), input_row_offsets=in_off,
                       page_table=table, cache_lens=total_lens, latent_cache=cache,
                       page_size=page_size, scale=default_scale(), mask=mask)


# --------------------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------------------

CONFIG_DESCRIPTIONS = {
    0: "tiny decode: B=2, H=16, cache lens {37,100}, page 16, causal",
    1: "batch decode: B=64, H=128, cache lens U[1024,4096], page 64, causal",
    2: "long-context split-KV decode: B=8, H=128, lens {32768 x4, 65536 x4}, page 64",
    3: "ragged causal prefill: new {512,1024,2048,3968} after {0,256,0,1024}, H=128, page 64",
    4: "sparse fp8 decode: B=32, H=128, 16384 rows/seq, 2048 indices, top-k U[1024,2048]",
}


def config_case(k: int, **overrides):
    """Full-size inputs of workload k (seed 355000 + k)."""
    seed = 355_000 + k
    if k == 0:
        return make_decode_case(seed, [37, 100], 16, 16, name="C0", **overrides)
    if k == 1:
        return make_decode_case(
            seed, lambda rng: rng.integers(1024, 4096, endpoint=True, size=64), 128, 64,
            name="C1", **overrides)
    if k == 2:
        return make_decode_case(seed, [32768] * 4 + [65536] * 4, 128, 64, name="C2", **overrides)
    if k == 3:
        return make_prefill_case(seed, [512, 1024, 2048, 3968], [0, 256, 0, 1024], 128, 64,
                                 name="C3", **overrides)
    if k == 4:
        return make_sparse_case(seed, 32, 128, 16384, 64, (1024, 2048), 2048, name="C4", **overrides)
    raise ValueError(f"no workload {k}")


# --------------------------------------------------------------------------------------
# what the method must read (for bandwidth figures)
# --------------------------------------------------------------------------------------

def algorithmic_bytes(case) -> int:
    """Bytes the method must read: every visible cache row once, plus q (and its scales)."""
    if isinstance(case, DecodeCase):
        rows = 0
        off = case.input_row_offsets.astype(np.int64)
        for b in range(case.batch):
            L = int(case.cache_lens[b])
            n = int(off[b + 1] - off[b])
            if n == 0:
                continue
            # union of the keys seen by the sequence's q rows, each read once
            lo = 0
            if case.mask == "sliding_window_causal" and case.window > 0:
                lo = max(0, (L - n) - case.window + 1)
            rows += max(0, L - lo)
        if case.fp8:
            # 576 (all e4m3) or 640 (rope-aware) bytes per row, plus its scale
            row_bytes = int(case.cache8.shape[-1]) + (4 if case.cache_scale is not None else 0)
            qb = case.q8.size + (case.q_scale.size * 4 if case.q_scale is not None else 0)
            return rows * row_bytes + qb
        return rows * HEAD_DIM * 2 + case.q.size * 2
    if isinstance(case, SparseCase):
        # every list's rows once (a list shared by a sequence's tokens is read once)
        listed = int(sum(int(np.count_nonzero(case.d_indices[r, :case.topk_lengths[r]] >= 0))
                         for r in range(case.d_indices.shape[0])))
        row_bytes = int(case.cache8.shape[-1]) + (4 if case.cache_scale is not None else 0)
        qb = case.q8.size + (case.q_scale.size * 4 if case.q_scale is not None else 0)
        return listed * row_bytes + qb
    if isinstance(case, PrefillCase):
        return (case.q.size + case.k.size + case.v.size) * 2 + int(case.cache_lens.sum()) * ROPE_DIM * 2
    if isinstance(case, IndexerCase):
        rows = 0
        off = case.input_row_offsets.astype(np.int64)
        for b in range(len(case.cache_lens)):
            L = int(case.cache_lens[b])
            n = int(off[b + 1] - off[b])
            if n == 0:
                continue
            lo = max(0, (L - n) - case.window + 1) if case.mask == "sliding_window_causal" else 0
            rows += max(0, L - lo)
        depth = case.q8.shape[2]
        return rows * (depth + 4) + case.q8.size + case.q_s.size * 4
    raise TypeError(type(case))


def algorithmic_flops(case) -> int:
    """2*H*(576+512) per visible (key, q row) pair for decode; 2*H*(192+128) for prefill."""
    if isinstance(case, DecodeCase):
        H = case.num_heads
        off = case.input_row_offsets.astype(np.int64)
        pairs = 0
        for b in range(case.batch):
            L = int(case.cache_lens[b])
            n = int(off[b + 1] - off[b])
            for j in range(n):
                pos = L - n + j
                if case.mask == "null":
                    pairs += L
                else:
                    hi = min(pos + 1, L)
                    lo = 0 if case.mask == "causal" else max(0, pos - case.window + 1)
                    pairs += max(0, hi - lo)
        return pairs * 2 * H * (HEAD_DIM + LATENT_DIM)
    if isinstance(case, SparseCase):
        per_list = [int(np.count_nonzero(case.d_indices[r, :case.topk_lengths[r]] >= 0))
                    for r in range(case.d_indices.shape[0])]
        if case.d_indices.shape[0] == case.total_q:
            listed = sum(per_list)
        else:  # shared lists: each token of sequence b attends to list b
            listed = int(sum(n * c for n, c in zip(np.diff(case.input_row_offsets.astype(np.int64)), per_list)))
        return listed * 2 * case.num_heads * (HEAD_DIM + LATENT_DIM)
    if isinstance(case, PrefillCase):
        H = case.num_heads
        pairs = 0
        off = case.input_row_offsets.astype(np.int64)
        for b in range(len(case.cache_lens)):
            L = int(case.cache_lens[b])
            n = int(off[b + 1] - off[b])
            # query j sits at L - n + j and sees keys 0..L-n+j under the causal mask
            pairs += n * (L - n) + n * (n + 1) // 2 if case.mask == "causal" else n * L
        return pairs * 2 * H * (PREFILL_QK_DIM + PREFILL_V_DIM)
    if isinstance(case, IndexerCase):
        NH, depth = case.q8.shape[1], case.q8.shape[2]
        off = case.input_row_offsets.astype(np.int64)
        pairs = 0
        for b in range(len(case.cache_lens)):
            L = int(case.cache_lens[b])
            n = int(off[b + 1] - off[b])
            for jj in range(n):
                pos = L - n + jj
                hi = L if case.mask == "null" else min(pos + 1, L)
                lo = max(0, pos - case.window + 1) if case.mask == "sliding_window_causal" else 0
                pairs += max(0, hi - lo)
        return pairs * 2 * NH * depth
    raise TypeError(type(case))
