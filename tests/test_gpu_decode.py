"""Dense decode on the GPU (through the C ABI) against the float64 oracle."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import BF16_TOL, bits_of, compare, decode_on_gpu, need_gpu, to_f64
from synth import config_case, make_decode_case

pytestmark = pytest.mark.gpu


def oracle_of(case, rows=None):
    out, _ = O.decode_paged(case.q, case.input_row_offsets, case.page_table, case.cache_lens,
                            case.latent_cache, case.page_size, case.scale, case.mask, case.window,
                            rows=rows)
    return out


def test_c0_tiny():
    m = need_gpu()
    case = config_case(0)
    got = decode_on_gpu(m, case)
    compare(to_f64(got), oracle_of(case), BF16_TOL, "C0 balanced")
    for P in (1, 2, 3, 7):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), oracle_of(case), BF16_TOL, f"C0 P={P}")


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("ps", [16, 64, 32])
def test_ragged_small(H, ps):
    m = need_gpu()
    case = make_decode_case(100 + H + ps, [1, 63, 64, 65, 200, 333, 1000], H, ps, name="ragged")
    want = oracle_of(case)
    for P in (0, 1, 3):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), want, BF16_TOL, f"H={H} PS={ps} P={P}")


@pytest.mark.parametrize("ps", [128, 256])
def test_large_pages(ps):
    """Pages holding several 32-key stages: consecutive stages reuse one page id."""
    m = need_gpu()
    case = make_decode_case(140 + ps, [1, 31, 33, 255, 257, 700, 1500], 128, ps, name="large-pages")
    want = oracle_of(case)
    for P in (0, 1, 3):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), want, BF16_TOL, f"PS={ps} P={P}")


@pytest.mark.parametrize("mask,window", [("null", -1), ("causal", -1), ("sliding_window_causal", 50)])
def test_multi_token_masks(mask, window):
    m = need_gpu()
    case = make_decode_case(7, [40, 130, 300, 700], 32, 64, q_per_seq=[1, 3, 2, 4], mask=mask,
                            window=window, name="mtp")
    want = oracle_of(case)
    for P in (0, 2):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), want, BF16_TOL, f"{mask} P={P}")


def test_c1_batch_decode():
    m = need_gpu()
    case = config_case(1)
    want = oracle_of(case)
    for P in (0, 1, 3, 7):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), want, BF16_TOL, f"C1 P={P}")


def test_c2_long_context_split():
    m = need_gpu()
    case = config_case(2)
    want = oracle_of(case)
    for P in (0, 1, 7, 64):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), want, BF16_TOL, f"C2 P={P}")


@pytest.mark.parametrize("ps,lens,mask", [(16, [20011, 300], "causal"), (64, [70001, 5000], "causal"),
                                           (16, [21000], "sliding_window_causal")])
def test_page_window_refill(ps, lens, mask):
    """One segment longer than the kernel's 1024-entry page-id window, so the window is
    refilled inside the stage loop: PS=16 (per-key page lookups) and PS=64 (one page per
    stage), whole rows at num_partitions=1 and the library's own split
    (generic_flare_mla_decode_kv_cache_ragged, Args num_partitions_in)."""
    m = need_gpu()
    window = 19000 if mask == "sliding_window_causal" else -1
    case = make_decode_case(300 + ps, lens, 16, ps, mask=mask, window=window, name="window-refill")
    assert max(lens) // ps > 1024
    want = oracle_of(case)
    for P in (1, 0, 2):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), want, BF16_TOL,
                f"PS={ps} lens={lens} {mask} P={P}")


def test_page_permutation_bitwise():
    """Physical page placement never changes the bits of the result."""
    m = need_gpu()
    case = make_decode_case(11, [100, 777, 1500], 128, 64, name="perm")
    a = bits_of(decode_on_gpu(m, case))
    rng = np.random.default_rng(5)
    npages = case.latent_cache.shape[0]
    perm = rng.permutation(npages)           # new physical id of old page p is perm[p]
    cache2 = np.empty_like(case.latent_cache)
    cache2[perm] = case.latent_cache
    table2 = np.where(case.page_table >= 0, perm[np.maximum(case.page_table, 0)], -1).astype(np.int32)
    b = bits_of(decode_on_gpu(m, case, table=table2, cache=cache2))
    assert np.array_equal(a, b)


def test_one_key_is_value_row():
    m = need_gpu()
    case = make_decode_case(12, [1, 1, 1], 128, 64, name="onekey")
    got = bits_of(decode_on_gpu(m, case))
    for b in range(3):
        v = case.latent_cache[case.page_table[b, 0], 0, :512]
        assert np.array_equal(got[b], np.broadcast_to(v, got[b].shape))


def test_nan_poisoned_tails_and_spare_pages():
    m = need_gpu()
    clean = make_decode_case(13, [37, 100, 1000, 64], 64, 64, spare_pages=3, name="clean")
    dirty = make_decode_case(13, [37, 100, 1000, 64], 64, 64, spare_pages=3, tail="nan", name="dirty")
    a = bits_of(decode_on_gpu(m, clean))
    b = decode_on_gpu(m, dirty)
    assert np.all(np.isfinite(to_f64(b)))
    assert np.array_equal(a, bits_of(b))


def test_deterministic_runs():
    m = need_gpu()
    case = config_case(1)
    a = bits_of(decode_on_gpu(m, case))
    for _ in range(2):
        assert np.array_equal(a, bits_of(decode_on_gpu(m, case)))


def test_batch_permutation_fixed_partitions_bitwise():
    """With a fixed partition count each row's split depends only on that row."""
    m = need_gpu()
    case = make_decode_case(14, [300, 1200, 64, 2000], 128, 64, name="bperm")
    a = bits_of(decode_on_gpu(m, case, num_partitions=3))
    perm = [2, 0, 3, 1]
    case2 = make_decode_case(14, [300, 1200, 64, 2000], 128, 64, name="bperm")
    case2.q = case.q[perm]
    case2.cache_lens = case.cache_lens[perm]
    case2.page_table = case.page_table[perm]
    b = bits_of(decode_on_gpu(m, case2, num_partitions=3))
    assert np.array_equal(b, a[perm])


def test_empty_rows_are_zero():
    m = need_gpu()
    case = make_decode_case(15, [0, 50, 0, 130], 16, 16, name="empty")
    got = to_f64(decode_on_gpu(m, case))
    want = oracle_of(case)
    compare(got, want, BF16_TOL, "empty rows")
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    for P in (1, 4):
        got = to_f64(decode_on_gpu(m, case, num_partitions=P))
        assert np.all(got[0] == 0) and np.all(got[2] == 0)


def test_no_visible_key_at_all():
    """A batch whose every row is empty: every output row is written as zeros (over a NaN
    filled buffer), balanced and fixed splits alike."""
    import torch
    m = need_gpu()
    case = make_decode_case(16, [0, 0, 0], 32, 16, name="all-empty")
    for P in (0, 1, 3):
        out = torch.full((case.q.shape[0], 32, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        got = to_f64(decode_on_gpu(m, case, num_partitions=P, out=out))
        assert np.all(got == 0), f"P={P}"


def test_bad_page_id_is_flagged_not_faulted():
    m = need_gpu()
    case = make_decode_case(16, [100, 200], 16, 64, name="badpid")
    table = case.page_table.copy()
    table[1, 1] = 10_000_000      # far outside the pool
    m.check_device_errors()       # clear
    got = decode_on_gpu(m, case, table=table)
    assert np.all(np.isfinite(to_f64(got)))
    assert m.check_device_errors() & 1


@pytest.mark.parametrize("nrows", [300, 600])
def test_many_rows_stream_split(nrows):
    """More non-empty rows than work-groups: the stream split instead of row parts (and,
    past the planning table's 512 rows, the per-row geometry search)."""
    m = need_gpu()
    rng = np.random.default_rng(nrows)
    lens = [int(x) for x in rng.integers(1, 400, nrows)]
    case = make_decode_case(200 + nrows, lens, 16, 64, name="many")
    compare(to_f64(decode_on_gpu(m, case)), oracle_of(case), BF16_TOL, f"{nrows} rows")


@pytest.mark.parametrize("T,H,ps,max_len", [(8192, 16, 16, 48), (2048, 128, 64, 300)])
def test_large_batch_sampled_rows(T, H, ps, max_len):
    """Thousands of one-token sequences (lengths U[1, max_len]): far more rows than the
    planning table and the work-groups, so each work-group streams many rows.  The whole
    output is finite; the first, the last and 96 random rows are checked against the
    oracle row by row."""
    m = need_gpu()
    rng = np.random.default_rng(T + H)
    lens = [int(x) for x in rng.integers(1, max_len + 1, T)]
    case = make_decode_case(300 + H, lens, H, ps, name="large-batch")
    got = to_f64(decode_on_gpu(m, case))
    assert np.all(np.isfinite(got))
    rows = sorted(set([0, T - 1] + [int(r) for r in rng.choice(T, 96, replace=False)]))
    compare(got[rows], oracle_of(case, rows=rows), BF16_TOL, f"{T} rows x {H} heads (sampled)")


def test_row_parts_mixed_rows():
    """Row parts with empty, one-tile and long rows side by side."""
    m = need_gpu()
    case = make_decode_case(17, [0, 1, 64, 65, 0, 5000, 130, 9000, 0, 3], 128, 64, name="mixed")
    got = to_f64(decode_on_gpu(m, case))
    compare(got, oracle_of(case), BF16_TOL, "mixed rows")
    assert np.all(got[0] == 0) and np.all(got[4] == 0) and np.all(got[8] == 0)


def test_alternating_shapes_reuse_workspace():
    """Split rows are merged through per-row arrival counters that every launch leaves
    cleared: calls of different shapes and split modes on one stream stay exact."""
    m = need_gpu()
    big = config_case(1)
    small = make_decode_case(18, [5000, 3, 700], 64, 64, name="alt")
    a = bits_of(decode_on_gpu(m, big))
    raw = decode_on_gpu(m, small)
    compare(to_f64(raw), oracle_of(small), BF16_TOL, "alt small")
    b = bits_of(raw)
    b5 = bits_of(decode_on_gpu(m, small, num_partitions=5))
    for P in (0, 5, 0, 2, 5):
        got = bits_of(decode_on_gpu(m, small, num_partitions=P))
        if P == 0:
            assert np.array_equal(got, b)
        elif P == 5:
            assert np.array_equal(got, b5)
        assert np.array_equal(bits_of(decode_on_gpu(m, big)), a)


@pytest.mark.parametrize("n_tok", [2, 4])
def test_c1_multi_token(n_tok):
    """The C1 batch with 2 or 4 query tokens per sequence (causal within the new tokens):
    every row matches the oracle, balanced and fixed splits alike."""
    m = need_gpu()
    case = config_case(1, q_per_seq=n_tok)
    want = oracle_of(case)
    for P in (0, 3):
        compare(to_f64(decode_on_gpu(m, case, num_partitions=P)), want, BF16_TOL, f"C1 x{n_tok} P={P}")
