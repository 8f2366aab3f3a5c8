"""Sparse fp8 decode on the GPU (through the C ABI) against the float64 oracle."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import (BF16_TOL, FP8_TOL, bf16_dev, bits_of, compare, f32_dev, i32_dev, need_gpu,
                      to_f64, u8_dev)
from synth import config_case, make_sparse_case
from synth.inputs import bf16_bits

pytestmark = pytest.mark.gpu


def oracle_of(case, d_indices=None, topk=None, rows=None):
    out, _ = O.decode_sparse(case.q8, case.q_scale, case.input_row_offsets, case.cache8,
                             case.cache_scale,
                             case.d_indices if d_indices is None else d_indices,
                             case.topk_lengths if topk is None else topk,
                             case.page_size, case.scale, rows=rows)
    return out


def sparse_on_gpu(m, case, num_partitions=0, d_indices=None, topk=None, cache8=None,
                  cache_scale="case", q=None, q_scale="case"):
    import torch
    qd = u8_dev(case.q8) if q is None else q
    if q_scale == "case":
        q_scale = f32_dev(case.q_scale) if case.q_scale is not None else None
    if cache_scale == "case":
        cache_scale = f32_dev(case.cache_scale) if case.cache_scale is not None else None
    if cache8 is None:
        cache8 = case.cache8
    cd = cache8 if isinstance(cache8, torch.Tensor) else u8_dev(cache8)
    res = m.decode_paged_sparse(
        qd, q_scale, i32_dev(case.input_row_offsets), cd,
        cache_scale, i32_dev(case.d_indices if d_indices is None else d_indices),
        i32_dev(case.topk_lengths if topk is None else topk), case.scale,
        num_partitions=num_partitions)
    torch.cuda.synchronize()
    return res


def test_c4_sparse_fp8():
    m = need_gpu()
    case = config_case(4)
    want = oracle_of(case)
    for P in (0, 1, 3):
        compare(to_f64(sparse_on_gpu(m, case, num_partitions=P)), want, FP8_TOL, f"C4 P={P}")


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("ps", [16, 64])
def test_sparse_small(H, ps):
    m = need_gpu()
    case = make_sparse_case(300 + H + ps, 5, H, 700, ps, (1, 300), 300, name="sp-small")
    want = oracle_of(case)
    for P in (0, 1, 3):
        compare(to_f64(sparse_on_gpu(m, case, num_partitions=P)), want, FP8_TOL, f"H={H} PS={ps} P={P}")


@pytest.mark.parametrize("B,H,rows_per_seq,n_index", [(1024, 16, 256, 128), (600, 128, 128, 64)])
def test_many_rows_sampled(B, H, rows_per_seq, n_index):
    """Hundreds to a thousand one-token rows with lists of 0 .. n_index entries: more rows
    than work-groups.  The whole output is finite and rows with an empty list are zero; the
    first, the last and 96 random rows are checked against the oracle row by row, with the
    library's split and with a fixed split of 2."""
    m = need_gpu()
    case = make_sparse_case(500 + H, B, H, rows_per_seq, 64, (0, n_index), n_index, name="sp-many")
    rng = np.random.default_rng(B)
    rows = sorted(set([0, B - 1] + [int(r) for r in rng.choice(B, 96, replace=False)]))
    want = oracle_of(case, rows=rows)
    empty = np.flatnonzero(case.topk_lengths == 0)
    for P in (0, 2):
        got = to_f64(sparse_on_gpu(m, case, num_partitions=P))
        assert np.all(np.isfinite(got))
        assert np.all(got[empty] == 0.0)
        compare(got[rows], want, FP8_TOL, f"{B} rows x {H} heads P={P} (sampled)")


def test_long_lists_window_refill():
    """64 one-token rows at 128 heads whose lists hold up to 8192 entries, drawn with
    repetition from 1024 rows of each sequence, one in 16 skipped: the library's split gives
    each work-group segments of about 2000 list positions, so the window of listed rows the
    balanced-batch kernel holds (512 positions) is refilled inside its segments.  Four rows
    are compared with the oracle; the whole output is finite."""
    m = need_gpu()
    case = make_sparse_case(79, 64, 128, 1024, 64, (1024, 1024), 1024, name="sp-long")
    rng = np.random.default_rng(79)
    n = 8192
    idx = np.empty((64, n), np.int32)
    for b in range(64):
        idx[b] = case.d_indices[b][rng.integers(0, 1024, size=n)]
        idx[b, rng.random(n) < 1 / 16] = -1
    topk = rng.integers(6000, n, endpoint=True, size=64).astype(np.int32)
    rows = [0, 17, 40, 63]
    want = oracle_of(case, d_indices=idx, topk=topk, rows=rows)
    m.check_device_errors()
    got = to_f64(sparse_on_gpu(m, case, d_indices=idx, topk=topk))
    assert m.check_device_errors() == 0
    assert np.all(np.isfinite(got))
    compare(got[rows], want, FP8_TOL, "long lists (sampled)")


# 128 heads: the balanced-batch fp8-MFMA kernel; the other head counts: the general kernel
@pytest.mark.parametrize("H", [64, 128])
def test_index_list_semantics(H):
    """Duplicates count twice, negative entries are skipped, entries past topk are never
    read (even when they name rows outside the pool), topk is clamped to the list width,
    and an empty list gives zeros -- none of this raises the device error bit."""
    m = need_gpu()
    case = make_sparse_case(41, 5, H, 512, 64, (100, 100), 120, name="sp-sem")
    idx = case.d_indices.copy()
    topk = case.topk_lengths.copy()
    idx[0, 10] = idx[0, 3]          # duplicate
    idx[0, 20] = -1                 # hole inside the counted prefix
    idx[1, 5] = -7                  # any negative entry is skipped
    idx[2, 100:] = 2 ** 30          # garbage past topk is never read
    topk[3] = 10_000                # clamped to the 120 listed columns
    idx[3, 100:] = idx[3, :20]
    topk[4] = 0                     # nothing to attend to
    m.check_device_errors()
    got = to_f64(sparse_on_gpu(m, case, d_indices=idx, topk=topk))
    assert m.check_device_errors() == 0
    compare(got, oracle_of(case, d_indices=idx, topk=topk), FP8_TOL, "index semantics")
    assert np.all(got[4] == 0)


@pytest.mark.parametrize("H", [32, 128])
def test_out_of_pool_index_is_flagged_and_skipped(H):
    m = need_gpu()
    case = make_sparse_case(42, 3, H, 256, 64, (60, 60), 64, name="sp-oob")
    idx = case.d_indices.copy()
    idx[1, 7] = 1 << 29              # inside topk, outside the pool
    m.check_device_errors()
    got = to_f64(sparse_on_gpu(m, case, d_indices=idx))
    assert m.check_device_errors() & 2
    compare(got, oracle_of(case, d_indices=idx), FP8_TOL, "out-of-pool skipped")


def test_poisoned_unlisted_rows_bitwise():
    """Rows no list names (NaN codes, NaN scales) never reach the result."""
    m = need_gpu()
    clean = make_sparse_case(43, 4, 128, 1024, 64, (200, 400), 400, name="sp-clean")
    dirty = make_sparse_case(43, 4, 128, 1024, 64, (200, 400), 400, poison=True, name="sp-dirty")
    a = bits_of(sparse_on_gpu(m, clean))
    b = sparse_on_gpu(m, dirty)
    assert np.all(np.isfinite(to_f64(b)))
    assert np.array_equal(a, bits_of(b))


def test_without_scales():
    m = need_gpu()
    case = make_sparse_case(44, 3, 128, 600, 16, (100, 250), 250, with_scales=False, name="sp-noscale")
    compare(to_f64(sparse_on_gpu(m, case)), oracle_of(case), FP8_TOL, "no scales")


def test_bf16_query():
    """A bf16 query (no token scale) against the fp8 cache."""
    m = need_gpu()
    case = make_sparse_case(45, 3, 64, 600, 64, (100, 250), 250, name="sp-bf16q")
    qf = O.e4m3_to_f64(case.q8) * case.q_scale[:, None, None]
    qb = bf16_bits(qf.astype(np.float32))
    got = to_f64(sparse_on_gpu(m, case, q=bf16_dev(qb), q_scale=None))
    cache = O.e4m3_to_f64(case.cache8) * case.cache_scale[..., None]
    want, _ = O.decode_sparse_f64(O.bf16_to_f64(qb), case.input_row_offsets, cache, case.d_indices,
                                  case.topk_lengths, case.page_size, case.scale)
    compare(got, want, BF16_TOL, "bf16 q")


def test_list_order_does_not_matter():
    m = need_gpu()
    case = make_sparse_case(46, 4, 128, 900, 64, (300, 500), 500, name="sp-order")
    idx = case.d_indices.copy()
    rng = np.random.default_rng(9)
    for t in range(idx.shape[0]):
        k = int(case.topk_lengths[t])
        idx[t, :k] = idx[t, :k][rng.permutation(k)]
    a = to_f64(sparse_on_gpu(m, case))
    b = to_f64(sparse_on_gpu(m, case, d_indices=idx))
    compare(b, a, FP8_TOL, "permuted lists")


def test_sparse_deterministic():
    m = need_gpu()
    case = make_sparse_case(47, 8, 128, 2048, 64, (500, 1000), 1000, name="sp-det")
    a = bits_of(sparse_on_gpu(m, case))
    for _ in range(2):
        assert np.array_equal(a, bits_of(sparse_on_gpu(m, case)))


@pytest.mark.parametrize("H", [64, 128])
def test_strided_pages_and_scales(H):
    """Pages and scale rows with padding between them (views of larger buffers) take the
    general loader, which derives each row's page and slot by division."""
    import torch
    m = need_gpu()
    case = make_sparse_case(77, 4, H, 700, 16, (100, 300), 300, name="sp-strided")
    NP, PS = case.cache8.shape[0], case.page_size
    big = torch.full((NP, PS + 3, 576), 0x7F, dtype=torch.uint8, device="cuda:0")  # NaN padding
    big[:, :PS] = u8_dev(case.cache8)
    sc = torch.full((NP, PS + 4), float("nan"), dtype=torch.float32, device="cuda:0")
    sc[:, :PS] = f32_dev(case.cache_scale)
    got = to_f64(sparse_on_gpu(m, case, cache8=big[:, :PS], cache_scale=sc[:, :PS]))
    compare(got, oracle_of(case), FP8_TOL, "strided pages and scales")
    flat = bits_of(sparse_on_gpu(m, case))
    assert np.array_equal(bits_of(sparse_on_gpu(m, case, cache8=big[:, :PS], cache_scale=sc[:, :PS])), flat)


@pytest.mark.parametrize("H", [16, 128])
def test_empty_lists(H):
    """Rows whose lists are empty (top-k 0) or hold only skipped entries are zero; a batch
    with no listed row at all writes every row as zeros (over a NaN filled buffer)."""
    import torch
    m = need_gpu()
    case = make_sparse_case(78, 4, H, 300, 16, (50, 120), 120, name="sp-empty")
    topk = case.topk_lengths.copy()
    topk[1] = 0
    idx = case.d_indices.copy()
    idx[2, :] = -1
    got = to_f64(sparse_on_gpu(m, case, topk=topk, d_indices=idx))
    compare(got, oracle_of(case, d_indices=idx, topk=topk), FP8_TOL, "empty lists")
    assert np.all(got[1] == 0) and np.all(got[2] == 0)
    zero = np.zeros_like(case.topk_lengths)
    for P in (0, 1, 3):
        out = torch.full((4, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        qd = u8_dev(case.q8)
        res = m.decode_paged_sparse(qd, f32_dev(case.q_scale), i32_dev(case.input_row_offsets),
                                    u8_dev(case.cache8), f32_dev(case.cache_scale), i32_dev(case.d_indices),
                                    i32_dev(zero), case.scale, num_partitions=P, out=out)
        torch.cuda.synchronize()
        assert np.all(to_f64(res) == 0), f"P={P}"
