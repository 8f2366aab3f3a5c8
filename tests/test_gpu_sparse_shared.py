"""Sparse decode with shared per-sequence index lists (mla_decode_paged_sparse_shared) on
the GPU against the float64 oracle: the C4 batch with 2 query tokens per sequence, ragged
token counts with an empty sequence, every head count, fixed splits, the equality with the
per-token entry point given replicated lists, and malformed offsets."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import FP8_TOL, bits_of, compare, f32_dev, i32_dev, need_gpu, to_f64, u8_dev
from synth import make_sparse_case

pytestmark = pytest.mark.gpu


def shared_case(seed, n_tokens, H, rows_per_seq=2048, ps=64, topk_range=(200, 600), n_index=600):
    """A sparse case with one list per sequence and len(n_tokens) sequences; the q rows are
    redrawn for sum(n_tokens) tokens from the same generator."""
    B = len(n_tokens)
    base = make_sparse_case(seed, B, H, rows_per_seq, ps, topk_range, n_index, name="shared")
    T = int(sum(n_tokens))
    tok = make_sparse_case(seed + 1, T, H, 64, 16, (1, 1), 1, name="shared-q")
    off = np.zeros(B + 1, dtype=np.uint32)
    off[1:] = np.cumsum(n_tokens)
    return dict(q8=tok.q8, q_scale=tok.q_scale, off=off, cache8=base.cache8, c_scale=base.cache_scale,
                idx=base.d_indices, topk=base.topk_lengths, ps=ps, scale=base.scale)


def oracle_of(c):
    out, _ = O.decode_sparse_shared(c["q8"], c["q_scale"], c["off"], c["cache8"], c["c_scale"], c["idx"],
                                    c["topk"], c["ps"], c["scale"])
    return out


def shared_on_gpu(m, c, num_partitions=0, off=None):
    import torch
    res = m.decode_paged_sparse_shared(u8_dev(c["q8"]), f32_dev(c["q_scale"]),
                                       i32_dev(c["off"] if off is None else off), u8_dev(c["cache8"]),
                                       f32_dev(c["c_scale"]), i32_dev(c["idx"]), i32_dev(c["topk"]), c["scale"],
                                       num_partitions=num_partitions)
    torch.cuda.synchronize()
    return res


def test_c4_two_tokens_per_sequence():
    m = need_gpu()
    c = shared_case(1500, [2] * 32, 128, rows_per_seq=16384, topk_range=(1024, 2048), n_index=2048)
    want = oracle_of(c)
    for P in (0, 3):
        compare(to_f64(shared_on_gpu(m, c, num_partitions=P)), want, FP8_TOL, f"shared C4x2 P={P}")


@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_ragged_tokens(H):
    m = need_gpu()
    c = shared_case(1510 + H, [1, 3, 0, 4, 2], H)
    want = oracle_of(c)
    for P in (0, 1, 3):
        compare(to_f64(shared_on_gpu(m, c, num_partitions=P)), want, FP8_TOL, f"shared H={H} P={P}")


def test_many_sequences_use_the_general_planner():
    """More than 64 sequences: the block planner (not the per-wave one) fills the rows."""
    m = need_gpu()
    c = shared_case(1520, [1, 2, 3] * 30, 32, rows_per_seq=512, topk_range=(10, 200), n_index=200)
    compare(to_f64(shared_on_gpu(m, c)), oracle_of(c), FP8_TOL, "shared 90 sequences")


def test_equals_per_token_lists_bitwise():
    """The same computation as mla_decode_paged_sparse given each token its sequence's list."""
    import torch
    m = need_gpu()
    c = shared_case(1530, [2, 1, 3], 128)
    idx, topk = O.token_lists(c["off"], c["idx"], c["topk"])
    per_token = m.decode_paged_sparse(u8_dev(c["q8"]), f32_dev(c["q_scale"]), i32_dev(c["off"]), u8_dev(c["cache8"]),
                                      f32_dev(c["c_scale"]), i32_dev(idx), i32_dev(topk), c["scale"])
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(per_token), bits_of(shared_on_gpu(m, c)))


@pytest.mark.parametrize("H", [64, 128])
def test_malformed_offsets_are_flagged(H):
    """Offsets that decrease set bit 2 of the device error word; the rows they cover stay
    zero and every other row is still right (128 heads: the balanced-batch fp8-MFMA
    kernel; 64: the general kernel)."""
    m = need_gpu()
    c = shared_case(1540, [2, 2, 2], H)
    bad = c["off"].copy()
    bad[2] = 1  # sequence 1 would end before it starts
    m.check_device_errors()       # clear
    got = to_f64(shared_on_gpu(m, c, off=bad))
    assert m.check_device_errors() & 4
    good = dict(c, off=c["off"])
    want = oracle_of(good)
    compare(got[4:], want[4:], FP8_TOL, "rows after the malformed sequence")
