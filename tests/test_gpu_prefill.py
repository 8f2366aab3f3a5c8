"""Ragged prefill on the GPU (through the C ABI) against the float64 oracle."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import BF16_TOL, bf16_dev, bits_of, compare, i32_dev, need_gpu, to_f64
from synth import config_case, make_prefill_case

pytestmark = pytest.mark.gpu


def oracle_of(case, rows=None, heads=None, **over):
    c = dict(q=case.q, k=case.k, v=case.v, bro=case.buffer_row_offsets, co=case.cache_offsets,
             inoff=case.input_row_offsets, pt=case.page_table, lens=case.cache_lens,
             cache=case.latent_cache, mask=case.mask)
    c.update(over)
    return O.prefill_paged(c["q"], c["k"], c["v"], c["bro"], c["co"], c["inoff"], c["pt"], c["lens"],
                           c["cache"], case.page_size, case.scale, c["mask"], rows=rows, heads=heads)


def prefill_on_gpu(m, case, **over):
    import torch
    c = dict(q=case.q, k=case.k, v=case.v, bro=case.buffer_row_offsets, co=case.cache_offsets,
             inoff=case.input_row_offsets, pt=case.page_table, lens=case.cache_lens,
             cache=case.latent_cache, mask=case.mask)
    c.update(over)
    res = m.prefill_paged(bf16_dev(c["q"]), bf16_dev(c["k"]), bf16_dev(c["v"]), i32_dev(c["bro"]),
                          i32_dev(c["co"]), i32_dev(c["inoff"]), i32_dev(c["pt"]), i32_dev(c["lens"]),
                          bf16_dev(c["cache"]), case.scale, mask=c["mask"])
    torch.cuda.synchronize()
    return res


def test_c3_prefill_every_row_16_heads():
    """The full C3 batch on the GPU; every one of its 7552 query rows is compared with the
    oracle for 16 heads spread over the 128 (every eighth).  The float64 oracle of all 128
    heads takes minutes on the host; 16 heads cover every query block of every sequence
    and every head position within a wave's 32-head group modulo 8."""
    m = need_gpu()
    case = config_case(3)
    got = to_f64(prefill_on_gpu(m, case))
    heads = list(range(0, 128, 8))
    want = oracle_of(case, heads=heads)
    compare(got[:, heads], want, BF16_TOL, "C3 all rows, 16 heads")
    assert np.all(np.isfinite(got))


def test_rope_pages_past_the_window():
    """A sequence whose keys span more than the kernel's 256-entry rope page window
    (PS=16, 4600 keys = 288 pages): stages past it look their page ids up in the page
    table directly."""
    m = need_gpu()
    case = make_prefill_case(66, [300, 40], [4300, 100], 16, 16, name="pf-window")
    assert (300 + 4300) // 16 > 256
    for mask in ("causal", "null"):
        compare(to_f64(prefill_on_gpu(m, case, mask=mask)), oracle_of(case, mask=mask), BF16_TOL,
                f"rope window fallback {mask}")


@pytest.mark.parametrize("H", [16, 64])
@pytest.mark.parametrize("ps", [16, 64])
@pytest.mark.parametrize("mask", ["causal", "null"])
def test_prefill_small(H, ps, mask):
    m = need_gpu()
    case = make_prefill_case(500 + H + ps, [1, 100, 130, 257], [0, 5, 64, 300], H, ps, mask=mask,
                             name="pf-small")
    compare(to_f64(prefill_on_gpu(m, case)), oracle_of(case), BF16_TOL, f"H={H} PS={ps} {mask}")


@pytest.mark.parametrize("mask", ["causal", "null"])
def test_prefill_many_short_sequences(mask):
    """300 sequences of 0 .. 40 new tokens after 0 .. 199 cached ones: hundreds of small
    query blocks launched longest-first, many sequences without new tokens."""
    m = need_gpu()
    rng = np.random.default_rng(65)
    new = [int(x) for x in rng.integers(0, 41, 300)]
    prefix = [int(x) for x in rng.integers(0, 200, 300)]
    case = make_prefill_case(65, new, prefix, 16, 16, mask=mask, name="pf-many")
    compare(to_f64(prefill_on_gpu(m, case)), oracle_of(case), BF16_TOL, f"300 short sequences {mask}")


def test_keys_of_new_tokens_only():
    """k / v hold only the new tokens, cache_offsets place them after the cached prefix."""
    m = need_gpu()
    new, prefix = [40, 200, 129], [17, 0, 300]
    case = make_prefill_case(61, new, prefix, 32, 64, name="pf-co")
    bro = case.buffer_row_offsets.astype(int)
    keep = np.concatenate([np.arange(bro[b] + prefix[b], bro[b + 1]) for b in range(len(new))])
    k2, v2 = case.k[keep], case.v[keep]
    bro2 = np.zeros(len(new) + 1, dtype=np.uint32)
    bro2[1:] = np.cumsum(new)
    co2 = np.asarray(prefix, dtype=np.uint32)
    got = to_f64(prefill_on_gpu(m, case, k=k2, v=v2, bro=bro2, co=co2))
    compare(got, oracle_of(case, k=k2, v=v2, bro=bro2, co=co2), BF16_TOL, "new-token keys")


def test_empty_sequence_in_batch():
    m = need_gpu()
    case = make_prefill_case(62, [50, 0, 70], [10, 40, 0], 16, 16, name="pf-empty")
    compare(to_f64(prefill_on_gpu(m, case)), oracle_of(case), BF16_TOL, "empty sequence")


def test_bad_rope_page_is_flagged_not_faulted():
    m = need_gpu()
    case = make_prefill_case(63, [64, 64], [0, 64], 16, 64, name="pf-bad")
    pt = case.page_table.copy()
    pt[1, 0] = 1 << 28
    m.check_device_errors()
    got = to_f64(prefill_on_gpu(m, case, pt=pt))
    assert m.check_device_errors() & 1
    assert np.all(np.isfinite(got))


def test_prefill_deterministic():
    m = need_gpu()
    case = make_prefill_case(64, [300, 513], [0, 100], 64, 64, name="pf-det")
    a = bits_of(prefill_on_gpu(m, case))
    assert np.array_equal(a, bits_of(prefill_on_gpu(m, case)))
