"""mla_decode_paged_noalloc (the dense decode whose split-KV workspace is a fixed per-GPU
array, for callers that cannot allocate) against mla_decode_paged: two calls in a row,
the second smaller, each bit-equal to the allocating entry point and within the bf16
tolerance of the float64 oracle; a call needing more than the array is refused."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import BF16_TOL, bf16_dev, bits_of, compare, i32_dev, need_gpu, to_f64
from synth import config_case, make_decode_case

pytestmark = pytest.mark.gpu


def _dev(case):
    return dict(q=bf16_dev(case.q), off=i32_dev(case.input_row_offsets), pt=i32_dev(case.page_table),
                lens=i32_dev(case.cache_lens), cache=bf16_dev(case.latent_cache))


def _both(m, case, num_partitions):
    import torch
    d = _dev(case)
    T, H = case.total_q, case.q.shape[1]
    out_a = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    out_b.fill_(float("nan"))
    m.decode_paged(d["q"], d["off"], d["pt"], d["lens"], d["cache"], case.scale, mask=case.mask,
                   local_window_size=case.window, num_partitions=num_partitions, out=out_a)
    m.decode_paged_noalloc(d["q"], d["off"], d["pt"], d["lens"], d["cache"], case.scale, mask=case.mask,
                           local_window_size=case.window, num_partitions=num_partitions, out=out_b)
    torch.cuda.synchronize()
    return out_a, out_b


def test_noalloc_matches_decode_paged_twice():
    m = need_gpu()
    want_err = m.check_device_errors()  # start from a clean error word
    assert want_err in (0, want_err)
    first = config_case(1)  # 64 rows x 128 heads, the balanced split
    second = make_decode_case(71, [1, 37, 100, 700, 2000], 128, 64, q_per_seq=[1, 2, 1, 1, 3],
                              name="noalloc-small")
    for case, parts, what in ((first, 0, "C1 balanced"), (second, 3, "small batch, 3 partitions")):
        a, b = _both(m, case, parts)
        assert np.array_equal(bits_of(a), bits_of(b)), f"{what}: no-alloc output differs from mla_decode_paged"
        want, _ = O.decode_paged(case.q, case.input_row_offsets, case.page_table, case.cache_lens,
                                 case.latent_cache, case.page_size, case.scale, case.mask, case.window)
        compare(to_f64(b), want, BF16_TOL, f"no-alloc {what}")
    assert m.check_device_errors() == 0


def test_noalloc_refuses_more_than_its_array():
    import torch
    m = need_gpu()
    case = make_decode_case(72, [100] * 64, 128, 64, name="noalloc-big")
    d = _dev(case)
    out = torch.empty((64, 128, 512), dtype=torch.bfloat16, device="cuda")
    # 64 rows x 100 partitions = 6400 part slots of 128 KiB: far above the array
    with pytest.raises(m.MlaError) as e:
        m.decode_paged_noalloc(d["q"], d["off"], d["pt"], d["lens"], d["cache"], case.scale, num_partitions=100,
                               out=out)
    assert e.value.status == 6
    assert m.decode_workspace_bytes(64, 128, 100) > m.decode_noalloc_scratch_bytes()
