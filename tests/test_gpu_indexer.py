"""FP8 top-k indexer on the GPU (through the C ABI) against the float64 oracle, and the
indexer chained into the sparse decode.

Selection is an integer result decided by floating-point scores: the kernel decides on
float32 scores, the oracle on float64 ones.  Rows whose scores lie within the float32
error band of the k-th score are equally valid choices at the boundary, so the check is:
the -1 fill and the number of valid entries exact; every entry a distinct visible row;
every chosen row scoring at least the k-th score minus the band; every visible row
scoring above the k-th score plus the band chosen; the listed order non-increasing within
the band; and at most 1% of the listed rows different from the oracle's list."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import FP8_TOL, compare, f32_dev, i32_dev, need_gpu, to_f64, u8_dev
from synth import indexer_config, make_indexer_case

pytestmark = pytest.mark.gpu


def run_indexer(m, c, table=None):
    import torch
    out = m.indexer_paged_fp8(u8_dev(c.q8), f32_dev(c.q_s), i32_dev(c.input_row_offsets),
                              i32_dev(c.page_table if table is None else table), i32_dev(c.cache_lens),
                              u8_dev(c.k8), f32_dev(c.k_scale), c.top_k, mask=c.mask,
                              local_window_size=c.window)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64)


def score_band(c, t, pos):
    """float32 error band of row t's scores: (heads + width) * 2^-24 times the largest
    sum of absolute products, with a factor 4 of margin."""
    q = np.abs(O.e4m3_to_f64(c.q8[t])) * c.q_s[t][:, None].astype(np.float64)   # [NH, D]
    qa = q.sum(axis=0)
    b = np.searchsorted(c.input_row_offsets.astype(np.int64), t, side="right") - 1
    ps = c.page_size
    pages = c.page_table[b][pos // ps].astype(np.int64)
    k = np.abs(O.e4m3_to_f64(c.k8[pages, pos % ps])) * c.k_scale[pages, pos % ps][:, None]
    bound = float((k @ qa).max(initial=0.0))
    NH, D = c.q8.shape[1], c.q8.shape[2]
    return 4.0 * (NH + D) * 2.0 ** -24 * bound


def check_indexer(got, c, what):
    want, seen = O.indexer_paged_fp8(c.q8, c.q_s, c.input_row_offsets, c.page_table, c.cache_lens, c.k8,
                                     c.k_scale, c.page_size, c.top_k, c.mask, c.window, return_scores=True)
    ps = c.page_size
    differ = 0
    for t, pos, sc in seen:
        b = np.searchsorted(c.input_row_offsets.astype(np.int64), t, side="right") - 1
        k = min(c.top_k, len(pos))
        row = got[t]
        assert np.all(row[k:] == -1), f"{what} row {t}: entries past {k} not -1"
        sel = row[:k]
        assert np.all(sel >= 0), f"{what} row {t}: fewer than {k} entries"
        assert len(np.unique(sel)) == k, f"{what} row {t}: repeated rows"
        # physical row -> logical position through this sequence's page table
        phys_of_pos = c.page_table[b][pos // ps].astype(np.int64) * ps + pos % ps
        where = {int(p): i for i, p in enumerate(phys_of_pos)}
        idx = np.array([where.get(int(r), -1) for r in sel])
        assert np.all(idx >= 0), f"{what} row {t}: a row that is not visible"
        if k == 0:
            continue
        band = score_band(c, t, pos)
        kth = np.sort(sc)[::-1][k - 1]
        chosen = sc[idx]
        assert chosen.min() >= kth - band, f"{what} row {t}: a row below the k-th score by more than {band}"
        assert np.all(np.diff(chosen) <= band), f"{what} row {t}: order not descending"
        # every visible row scoring clearly above the k-th must have been chosen
        clear = np.flatnonzero(sc > kth + band)
        missing = np.setdiff1d(clear, idx)
        assert missing.size == 0, f"{what} row {t}: {missing.size} rows above the k-th score plus the band left out"
        differ += int(np.count_nonzero(sel != want[t][:k]))
    return differ


@pytest.mark.parametrize("ps", [16, 64])
@pytest.mark.parametrize("mask,window", [("causal", -1), ("null", -1), ("sliding_window_causal", 40)])
def test_indexer_small(ps, mask, window):
    m = need_gpu()
    c = make_indexer_case(41, [1, 37, 100, 700, 64, 300], 8, 64, ps, 48, q_per_seq=[1, 2, 1, 3, 1, 2],
                          mask=mask, window=window, name="idx-small")
    differ = check_indexer(run_indexer(m, c), c, f"PS={ps} {mask}")
    listed = sum(min(c.top_k, hi - lo) for hi, lo in _visible_counts(c))
    print(f"[parity] indexer PS={ps} {mask}: {differ} of {listed} listed rows differ from the oracle's order",
          flush=True)
    # rows that differ are boundary choices within the float32 band (checked above); at
    # most 1% of the listed rows may be such choices
    assert differ <= max(1, listed // 100)


def _visible_counts(c):
    """(hi, lo) of every query row's visible range, from the oracle's reading."""
    off = c.input_row_offsets.astype(np.int64)
    res = []
    for b, L in enumerate(c.cache_lens):
        n = int(off[b + 1] - off[b])
        for j in range(n):
            lo, hi = O.visible_range(int(L), n, j, c.mask, c.window)
            res.append((hi, lo))
    return res


def test_indexer_full_size():
    """The indexer in front of C4: 32 sequences x 16384 rows, 64 heads of 128, top 2048."""
    m = need_gpu()
    c = indexer_config()
    got = run_indexer(m, c)
    differ = check_indexer(got, c, "X4")
    total = c.total_q * c.top_k
    print(f"[parity] indexer X4: {differ} of {total} listed rows differ from the oracle's order", flush=True)
    assert differ <= total // 100


def test_indexer_bad_page_is_flagged():
    m = need_gpu()
    c = make_indexer_case(42, [200, 300], 4, 32, 64, 16, name="idx-bad")
    table = c.page_table.copy()
    table[1, 2] = 10_000_000
    m.check_device_errors()
    got = run_indexer(m, c, table=table)
    assert m.check_device_errors() & 1
    pool = c.k8.shape[0] * c.page_size
    assert np.all((got == -1) | ((got >= 0) & (got < pool)))


def test_indexer_feeds_sparse_decode():
    """Indexer -> sparse decode on the GPU against oracle indexer -> oracle sparse decode."""
    import torch
    from synth import make_decode_case
    m = need_gpu()
    lens, H, ps, top_k = [1500, 2048, 700, 1999], 32, 64, 256
    idx_case = make_indexer_case(43, lens, 16, 64, ps, top_k, name="chain-idx")
    dec = make_decode_case(43, lens, H, ps, fp8=True, name="chain-dec")
    # the decode cache shares the indexer's page table (same pool geometry)
    dec.page_table = idx_case.page_table
    npages = idx_case.k8.shape[0]
    assert dec.cache8.shape[0] == npages
    got_idx = m.indexer_paged_fp8(u8_dev(idx_case.q8), f32_dev(idx_case.q_s), i32_dev(idx_case.input_row_offsets),
                                  i32_dev(idx_case.page_table), i32_dev(idx_case.cache_lens), u8_dev(idx_case.k8),
                                  f32_dev(idx_case.k_scale), top_k)
    topk_len = i32_dev(np.full(len(lens), top_k, dtype=np.int32))
    out = m.decode_paged_sparse(u8_dev(dec.q8), f32_dev(dec.q_scale), i32_dev(dec.input_row_offsets),
                                u8_dev(dec.cache8), f32_dev(dec.cache_scale), got_idx, topk_len, dec.scale)
    torch.cuda.synchronize()
    want_idx = O.indexer_paged_fp8(idx_case.q8, idx_case.q_s, idx_case.input_row_offsets, idx_case.page_table,
                                   idx_case.cache_lens, idx_case.k8, idx_case.k_scale, ps, top_k)
    want, _ = O.decode_sparse(dec.q8, dec.q_scale, dec.input_row_offsets, dec.cache8, dec.cache_scale,
                              want_idx.astype(np.int32), np.full(len(lens), top_k, dtype=np.int32), ps, dec.scale)
    compare(to_f64(out), want, FP8_TOL, "indexer -> sparse decode")


@pytest.mark.parametrize("num_heads,depth", [(3, 16), (5, 48), (64, 128), (7, 208), (2, 256), (48, 256)])
def test_indexer_widths(num_heads, depth):
    """Head widths from 16 to 256 (rows held in registers in 8 or 16 chunks) and head counts
    that leave some fold groups empty, or give a fold thread more heads than it preloads
    (48 heads of 256); lengths over several 1024-row slices, top_k below, at and above the
    visible count."""
    m = need_gpu()
    c = make_indexer_case(44 + depth, [1, 1023, 1024, 2500, 4097], num_heads, depth, 64, 1024,
                          q_per_seq=[1, 2, 1, 3, 1], name=f"idx-w{depth}")
    differ = check_indexer(run_indexer(m, c), c, f"NH={num_heads} D={depth}")
    total = c.total_q * c.top_k
    print(f"[parity] indexer NH={num_heads} D={depth}: {differ} of {total} listed rows differ", flush=True)
    assert differ <= max(total // 100, 8)


def test_indexer_malformed_offsets_are_flagged():
    """Offsets that decrease set bit 2 of the device error word; a token no sequence's
    offsets cover gets an empty list (-1), every entry is still -1 or a row of the pool,
    and a token past the malformed entry gets the same list as with valid offsets."""
    m = need_gpu()
    c = make_indexer_case(48, [500, 700, 900, 1100], 8, 128, 64, 256, q_per_seq=1, name="idx-off")
    good = run_indexer(m, c)
    m.check_device_errors()  # clear
    bad_off = c.input_row_offsets.copy()
    bad_off[2] = 0  # [0, 1, 0, 3, 4]: sequence 1 would end before it starts
    import torch
    out = m.indexer_paged_fp8(u8_dev(c.q8), f32_dev(c.q_s), i32_dev(bad_off), i32_dev(c.page_table),
                              i32_dev(c.cache_lens), u8_dev(c.k8), f32_dev(c.k_scale), c.top_k, mask=c.mask,
                              local_window_size=c.window)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64)
    assert m.check_device_errors() & 4
    pool_rows = c.k8.shape[0] * c.page_size
    assert np.all((got == -1) | ((got >= 0) & (got < pool_rows)))
    assert np.all(got[0] == -1)  # token 0: no offsets pair covers it
    assert np.array_equal(got[3], good[3])


def test_indexer_unaligned_q():
    """q as a view into rows one byte wider (head stride D + 1, not a multiple of 4 bytes):
    the head fold reads it a byte at a time instead of a dword; the result meets the same
    checks over sequences of several 1024-row slices."""
    import torch
    m = need_gpu()
    c = make_indexer_case(47, [700, 2500, 1024], 8, 128, 64, 512, q_per_seq=[1, 2, 1], name="idx-uq")
    T, NH, D = c.q8.shape
    wide = torch.zeros((T, NH, D + 1), dtype=torch.uint8, device="cuda")
    wide[:, :, :D] = u8_dev(c.q8)
    q_view = wide[:, :, :D]
    assert q_view.stride(1) % 4 != 0
    out = m.indexer_paged_fp8(q_view, f32_dev(c.q_s), i32_dev(c.input_row_offsets), i32_dev(c.page_table),
                              i32_dev(c.cache_lens), u8_dev(c.k8), f32_dev(c.k_scale), c.top_k, mask=c.mask,
                              local_window_size=c.window)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64)
    differ = check_indexer(got, c, "unaligned q")
    assert differ <= max(c.total_q * c.top_k // 100, 8)
    aligned = run_indexer(m, c)
    assert check_indexer(aligned, c, "aligned q") <= max(c.total_q * c.top_k // 100, 8)


@pytest.mark.parametrize("top_k", [1, 700, 2048])
def test_indexer_ties_exact(top_k):
    """Cache rows drawn from three patterns with one shared scale: scores tie exactly in
    float32 and in float64, so the order within a tie is decided by position alone (lower
    first) and the result equals the oracle's entry for entry.  Groups of thousands of equal
    scores keep the radix bin of the threshold large through the score digits."""
    m = need_gpu()
    c = make_indexer_case(45, [5000, 16384, 3001], 4, 64, 64, top_k, q_per_seq=[1, 1, 2], name="idx-ties")
    rng = np.random.default_rng(4545)
    pats = c.k8[0, :3].copy()
    c.k8 = pats[rng.integers(0, 3, size=c.k8.shape[:2])]
    c.k_scale = np.full_like(c.k_scale, 0.0078125)
    got = run_indexer(m, c)
    want = O.indexer_paged_fp8(c.q8, c.q_s, c.input_row_offsets, c.page_table, c.cache_lens, c.k8,
                               c.k_scale, c.page_size, c.top_k, c.mask, c.window)
    assert np.array_equal(got, want.astype(np.int64)), \
        f"top_k={top_k}: {int(np.count_nonzero(got != want))} entries differ from the oracle"
    print(f"[parity] indexer ties top_k={top_k}: exact", flush=True)


@pytest.mark.parametrize("mask,window", [("causal", -1), ("sliding_window_causal", 1500)])
def test_indexer_many_tokens_per_sequence(mask, window):
    """128 query tokens per sequence (512 in all): each token sees its own causal or
    sliding range, one selection work-group per token; the 128-row sequence has tokens that
    see fewer rows than top_k."""
    m = need_gpu()
    c = make_indexer_case(46, [4000, 2500, 128, 3333], 8, 64, 64, 512, q_per_seq=128, mask=mask,
                          window=window, name="idx-many")
    differ = check_indexer(run_indexer(m, c), c, f"many tokens {mask}")
    total = c.total_q * c.top_k
    print(f"[parity] indexer 512 tokens {mask}: {differ} of {total} listed rows differ", flush=True)
    assert differ <= max(total // 100, 8)
