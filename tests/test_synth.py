"""Seeded input generator: determinism, layout invariants and the recorded workloads."""
import hashlib
import json
import os

import numpy as np
import pytest

from synth import (config_case, make_decode_case, make_sparse_case, algorithmic_bytes,
                   algorithmic_flops, bf16_bits)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("k", range(5))
def test_workload_bytes_are_recorded(k):
    with open(os.path.join(GOLDEN, "synth_checksums.json")) as f:
        want = json.load(f)[f"C{k}"]
    case = config_case(k)
    for field, digest in want.items():
        got = hashlib.sha256(np.ascontiguousarray(getattr(case, field)).tobytes()).hexdigest()
        assert got == digest, field


def test_same_seed_same_bytes_other_seed_differs():
    a = make_decode_case(7, [30, 70], 4, 16)
    b = make_decode_case(7, [30, 70], 4, 16)
    c = make_decode_case(8, [30, 70], 4, 16)
    assert np.array_equal(a.latent_cache, b.latent_cache) and np.array_equal(a.q, b.q)
    assert not np.array_equal(a.latent_cache, c.latent_cache)


def test_page_table_is_a_permutation():
    c = config_case(1)
    npages = (c.cache_lens + c.page_size - 1) // c.page_size
    used = np.concatenate([c.page_table[b, :n] for b, n in enumerate(npages)])
    assert len(np.unique(used)) == len(used) == c.latent_cache.shape[0]
    for b, n in enumerate(npages):
        assert np.all(c.page_table[b, n:] == -1)
    assert 1024 <= c.cache_lens.min() and c.cache_lens.max() <= 4096


def test_c0_c3_shapes():
    c0 = config_case(0)
    assert list(c0.cache_lens) == [37, 100] and c0.q.shape == (2, 16, 576)
    assert c0.latent_cache.shape == (10, 16, 576) and c0.page_table.shape == (2, 7)
    c3 = config_case(3)
    assert list(c3.input_row_offsets) == [0, 512, 1536, 3584, 7552]
    assert list(c3.buffer_row_offsets) == [0, 512, 1792, 3840, 8832]
    assert list(c3.cache_lens) == [512, 1280, 2048, 4992]
    assert c3.q.shape == (7552, 128, 192) and c3.k.shape == (8832, 128, 128)


def test_sparse_indices_layout():
    s = make_sparse_case(3, 4, 8, 1024, 64, (100, 200), 256)
    pool = s.cache8.shape[0] * s.page_size
    for t in range(4):
        k = s.topk_lengths[t]
        head = s.d_indices[t, :k]
        assert np.all((head >= 0) & (head < pool)) and len(np.unique(head)) == k
        assert np.all(s.d_indices[t, k:] == -1)
        # every listed row belongs to sequence t's pages
        own = set(int(p) for p in s.page_table[t])
        assert all(int(r) // s.page_size in own for r in head)
    assert s.q_scale.shape == (4,) and s.cache_scale.shape == s.cache8.shape[:2]


def test_nan_tail_poison():
    c = make_decode_case(9, [5, 20], 2, 16, tail="nan", spare_pages=2)
    bits = c.latent_cache
    p_last = c.page_table[0, 0]
    assert np.all(bits[p_last, 5:] == 0x7FC0) and not np.any(bits[p_last, :5] == 0x7FC0)


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, np.inf, np.nan], dtype=np.float32)
    assert list(bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F80, 0x7FC0]


def test_algorithmic_sizes_c1():
    c = config_case(1)
    assert algorithmic_bytes(c) == int(c.cache_lens.sum()) * 1152 + 64 * 128 * 576 * 2
    assert algorithmic_flops(c) == int(c.cache_lens.sum()) * 2 * 128 * 1088
