"""The rope-aware interleaved layout (640-byte q heads and cache rows: 512 E4M3 latent codes
then 64 bf16 rope values, the scale on the codes only) through mla_decode_paged_fp8 and
mla_decode_paged_sparse on the GPU, against the float64 oracle: the C1 batch at full size,
ragged small cases over head counts (both widening layouts of the kernel), page sizes, masks
and fixed splits, zero scales, NaN-poisoned page tails, and the sparse C4-type batch."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import FP8_TOL, bits_of, compare, decode_fp8_on_gpu, f32_dev, i32_dev, need_gpu, to_f64, u8_dev
from synth import config_case, make_decode_case, make_sparse_case, rope_aware

pytestmark = pytest.mark.gpu


def dense_oracle(case, rows=None):
    out, _ = O.decode_paged_fp8_rope_aware(case.q8, case.q_scale, case.input_row_offsets, case.page_table,
                                           case.cache_lens, case.cache8, case.cache_scale, case.page_size,
                                           case.scale, case.mask, case.window, rows=rows)
    return out


def sparse_oracle(case, rows=None):
    out, _ = O.decode_sparse_rope_aware(case.q8, case.q_scale, case.input_row_offsets, case.cache8,
                                        case.cache_scale, case.d_indices, case.topk_lengths, case.page_size,
                                        case.scale, rows=rows)
    return out


def sparse_on_gpu(m, case, num_partitions=0):
    import torch
    q_scale = f32_dev(case.q_scale) if case.q_scale is not None else None
    c_scale = f32_dev(case.cache_scale) if case.cache_scale is not None else None
    res = m.decode_paged_sparse(u8_dev(case.q8), q_scale, i32_dev(case.input_row_offsets), u8_dev(case.cache8),
                                c_scale, i32_dev(case.d_indices), i32_dev(case.topk_lengths), case.scale,
                                num_partitions=num_partitions)
    torch.cuda.synchronize()
    return res


def test_rope_aware_c1_batch_sampled_rows():
    """The C1 batch (B=64, H=128, lens U[1024,4096], PS=64) in the rope-aware layout, in the
    library's split and a fixed one; twelve rows spread over the batch against the oracle."""
    m = need_gpu()
    case = rope_aware(config_case(1, fp8=True), 1401)
    rows = np.linspace(0, case.total_q - 1, 12).astype(int)
    want = dense_oracle(case, rows=rows)
    for P in (0, 3):
        got = to_f64(decode_fp8_on_gpu(m, case, num_partitions=P))
        compare(got[rows], want[rows] if want.shape[0] == case.total_q else want, FP8_TOL, f"rope C1 P={P}")


@pytest.mark.parametrize("H", [16, 64, 128])
@pytest.mark.parametrize("ps", [16, 64])
def test_rope_aware_ragged_small(H, ps):
    m = need_gpu()
    case = rope_aware(make_decode_case(1410 + H + ps, [1, 37, 100, 700, 64], H, ps, fp8=True, name="rope-small"),
                      1411)
    want = dense_oracle(case)
    for P in (0, 2, 5):
        compare(to_f64(decode_fp8_on_gpu(m, case, num_partitions=P)), want, FP8_TOL, f"H={H} PS={ps} P={P}")


@pytest.mark.parametrize("mask,window", [("null", -1), ("causal", -1), ("sliding_window_causal", 40)])
def test_rope_aware_multi_token_masks(mask, window):
    m = need_gpu()
    case = rope_aware(make_decode_case(1420, [90, 300, 513], 128, 64, q_per_seq=3, mask=mask, window=window,
                                       fp8=True, name="rope-mtp"), 1421)
    compare(to_f64(decode_fp8_on_gpu(m, case)), dense_oracle(case), FP8_TOL, f"rope {mask}")


def test_rope_aware_zero_scales():
    """Zero row and token scales: the latent part of such a row or token drops out, its
    rope part still counts (the kernel takes scales below 2^-40 as 2^-40 on both sides of
    its rope quotient); token 1 meets zero-scale rows with both sides at the floor."""
    m = need_gpu()
    case = rope_aware(make_decode_case(1430, [40, 200, 77], 128, 16, fp8=True, name="rope-zero"), 1431)
    cs = case.cache_scale.copy()
    cs.reshape(-1)[::7] = 0.0
    qs = case.q_scale.copy()
    qs[1] = 0.0
    case.cache_scale, case.q_scale = cs, qs
    compare(to_f64(decode_fp8_on_gpu(m, case)), dense_oracle(case), FP8_TOL, "rope zero scales")


def test_rope_aware_poisoned_tails_bitwise():
    """NaN codes and NaN rope values in the unused slots of every last page change nothing."""
    m = need_gpu()
    base = make_decode_case(1440, [33, 100, 5], 64, 16, fp8=True, name="rope-clean", spare_pages=2)
    clean = rope_aware(base, 1441)
    poisoned = rope_aware(make_decode_case(1440, [33, 100, 5], 64, 16, fp8=True, tail="nan", spare_pages=2,
                                           name="rope-poison"), 1441)
    a = bits_of(decode_fp8_on_gpu(m, clean))
    b = bits_of(decode_fp8_on_gpu(m, poisoned))
    assert np.array_equal(a, b)
    compare(to_f64(decode_fp8_on_gpu(m, clean)), dense_oracle(clean), FP8_TOL, "rope clean")


def test_rope_aware_sparse_c4_type():
    """The C4 shape (B=32, H=128, 2048 listed rows, top-k U[1024,2048]) in the rope-aware
    layout, every element against the oracle."""
    m = need_gpu()
    case = rope_aware(config_case(4), 1450)
    want = sparse_oracle(case)
    for P in (0, 3):
        compare(to_f64(sparse_on_gpu(m, case, num_partitions=P)), want, FP8_TOL, f"rope C4 P={P}")


@pytest.mark.parametrize("H", [16, 128])
def test_rope_aware_sparse_small(H):
    m = need_gpu()
    case = rope_aware(make_sparse_case(1460 + H, 5, H, 700, 16, (1, 300), 300, name="rope-sp"), 1461)
    want = sparse_oracle(case)
    for P in (0, 1, 3):
        compare(to_f64(sparse_on_gpu(m, case, num_partitions=P)), want, FP8_TOL, f"rope sparse H={H} P={P}")
