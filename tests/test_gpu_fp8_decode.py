"""Dense decode over a paged fp8 cache on the GPU (through the C ABI) against the float64
oracle: the C1 batch at full size, ragged small cases over head counts, page sizes and
masks, NaN-poisoned page tails, and a page id outside the pool."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import FP8_TOL, bits_of, compare, decode_fp8_on_gpu, need_gpu, to_f64
from synth import config_case, make_decode_case

pytestmark = pytest.mark.gpu


def oracle_of(case):
    out, _ = O.decode_paged_fp8(case.q8, case.q_scale, case.input_row_offsets, case.page_table,
                                case.cache_lens, case.cache8, case.cache_scale, case.page_size,
                                case.scale, case.mask, case.window)
    return out


def test_fp8_c1_batch():
    m = need_gpu()
    case = config_case(1, fp8=True)
    want = oracle_of(case)
    for P in (0, 3):
        compare(to_f64(decode_fp8_on_gpu(m, case, num_partitions=P)), want, FP8_TOL, f"fp8 C1 P={P}")


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("ps", [16, 64, 48])
def test_fp8_ragged_small(H, ps):
    m = need_gpu()
    case = make_decode_case(31, [1, 37, 100, 700, 64], H, ps, fp8=True, name="fp8-small")
    want = oracle_of(case)
    for P in (0, 2):
        compare(to_f64(decode_fp8_on_gpu(m, case, num_partitions=P)), want, FP8_TOL, f"H={H} PS={ps} P={P}")


@pytest.mark.parametrize("mask,window", [("null", -1), ("causal", -1), ("sliding_window_causal", 50)])
def test_fp8_multi_token_masks(mask, window):
    m = need_gpu()
    case = make_decode_case(32, [40, 130, 300, 700], 32, 64, q_per_seq=[1, 3, 2, 4], mask=mask,
                            window=window, fp8=True, name="fp8-mtp")
    want = oracle_of(case)
    compare(to_f64(decode_fp8_on_gpu(m, case)), want, FP8_TOL, f"fp8 {mask}")


def test_fp8_nan_poisoned_tails_bitwise():
    """Page tails and spare pages hold the E4M3 NaN code with NaN scales: never read."""
    m = need_gpu()
    clean = make_decode_case(33, [37, 100, 1000, 64], 64, 64, spare_pages=3, fp8=True, name="clean")
    dirty = make_decode_case(33, [37, 100, 1000, 64], 64, 64, spare_pages=3, tail="nan", fp8=True,
                             name="dirty")
    a = bits_of(decode_fp8_on_gpu(m, clean))
    b = decode_fp8_on_gpu(m, dirty)
    assert np.all(np.isfinite(to_f64(b)))
    assert np.array_equal(a, bits_of(b))


def test_fp8_bad_page_id_is_flagged_not_faulted():
    m = need_gpu()
    case = make_decode_case(34, [100, 200], 16, 64, fp8=True, name="fp8-badpid")
    table = case.page_table.copy()
    table[1, 1] = 10_000_000      # far outside the pool
    m.check_device_errors()       # clear
    got = decode_fp8_on_gpu(m, case, table=table)
    assert np.all(np.isfinite(to_f64(got)))
    assert m.check_device_errors() & 1
