"""Sparse fp8 decode with an attention sink and a second KV stream on the GPU (through the
C ABI mla_decode_paged_sparse_ext) against the float64 oracle.

generic_flare_mla_decode_kv_cache_ragged, Args attn_sink_ptr, extra_k, extra_d_indices,
extra_indices_stride, extra_topk_lengths, extra_scales_ptr.  The page names these without
a formula; the oracle implements the reading (one sink logit per head in the softmax
denominator; one softmax over the rows of both lists), so parity here is parity with that
reading, which no page pins."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from gpu_util import FP8_TOL, bits_of, compare, f32_dev, i32_dev, need_gpu, to_f64, u8_dev
from synth import config_case, make_sparse_case

pytestmark = pytest.mark.gpu


def sink_logits(seed, H):
    """Sink logits of the size of a row's log-sum-exp (so the sink takes a real share),
    with one head at -inf (no sink) and one far above (nearly all weight on the sink)."""
    rng = np.random.default_rng(seed)
    s = rng.uniform(4.0, 10.0, H).astype(np.float32)
    s[0] = -np.inf
    s[min(1, H - 1)] = 40.0
    return s


def second_stream(seed, T, ps, rows, width, topk_range):
    """A second fp8 pool and per-row lists into it (a sparse case of its own)."""
    c = make_sparse_case(seed, T, 16, rows, ps, topk_range, width, name="extra")
    return c.cache8, c.cache_scale, c.d_indices, c.topk_lengths, ps


def oracle_of(case, extra=None, sink=None):
    out, _ = O.decode_sparse(case.q8, case.q_scale, case.input_row_offsets, case.cache8, case.cache_scale,
                             case.d_indices, case.topk_lengths, case.page_size, case.scale, extra=extra,
                             attn_sink=None if sink is None else sink.astype(np.float64))
    return out


def ext_on_gpu(m, case, extra=None, sink=None, num_partitions=0, extra_cache=None):
    import torch
    ex = {}
    if extra is not None:
        c8, cs, idx, tk, _ = extra
        ex = dict(extra_cache=u8_dev(c8 if extra_cache is None else extra_cache),
                  extra_cache_scale=None if cs is None else f32_dev(cs),
                  extra_d_indices=i32_dev(idx), extra_topk_lengths=i32_dev(tk))
    res = m.decode_paged_sparse_ext(
        u8_dev(case.q8), f32_dev(case.q_scale), i32_dev(case.input_row_offsets), u8_dev(case.cache8),
        f32_dev(case.cache_scale), i32_dev(case.d_indices), i32_dev(case.topk_lengths), case.scale,
        attn_sink=None if sink is None else f32_dev(sink), num_partitions=num_partitions, **ex)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("what", ["sink", "extra", "both"])
@pytest.mark.parametrize("H,ps", [(16, 16), (128, 64)])
def test_sparse_ext_small(what, H, ps):
    m = need_gpu()
    case = make_sparse_case(400 + H + ps, 6, H, 700, ps, (1, 300), 300, name="ext-small")
    extra = second_stream(401 + H, 6, 32, 500, 200, (0, 200)) if what != "sink" else None
    sink = sink_logits(402, H) if what != "extra" else None
    want = oracle_of(case, extra, sink)
    for P in (0, 1, 3):
        compare(to_f64(ext_on_gpu(m, case, extra, sink, P)), want, FP8_TOL, f"{what} H={H} PS={ps} P={P}")


def test_c4_with_sink_and_second_stream():
    """C4 (32 rows x 128 heads, top-k U[1024, 2048] of 2048) with sink logits and a second
    stream of up to 512 rows per query row from a 64 K-row second pool (page size 64)."""
    m = need_gpu()
    case = config_case(4)
    extra = second_stream(403, case.total_q, 64, 2048, 512, (0, 512))
    sink = sink_logits(404, 128)
    want = oracle_of(case, extra, sink)
    for P in (0, 1, 3):
        compare(to_f64(ext_on_gpu(m, case, extra, sink, P)), want, FP8_TOL, f"C4 + sink + second stream P={P}")


def test_without_sink_or_rows_is_the_plain_sparse_decode():
    """A sink of -inf everywhere, or a second stream whose lists count no row, gives the
    same bits as mla_decode_paged_sparse on the same split (num_partitions 3: one kernel
    serves all three).  With the library's split the plain decode of this batch runs the
    balanced-batch fp8-MFMA kernel: it agrees with them within the fp8 tolerance, and the
    two extended forms still agree bit for bit."""
    m = need_gpu()
    case = make_sparse_case(405, 8, 128, 1000, 64, (1, 500), 500, name="ext-plain")
    import torch
    c8, cs, idx, tk, ps = second_stream(406, 8, 16, 200, 50, (0, 50))
    for P in (3, 0):
        plain = m.decode_paged_sparse(u8_dev(case.q8), f32_dev(case.q_scale), i32_dev(case.input_row_offsets),
                                      u8_dev(case.cache8), f32_dev(case.cache_scale), i32_dev(case.d_indices),
                                      i32_dev(case.topk_lengths), case.scale, num_partitions=P)
        torch.cuda.synchronize()
        b = ext_on_gpu(m, case, sink=np.full(128, -np.inf, dtype=np.float32), num_partitions=P)
        c = ext_on_gpu(m, case, extra=(c8, cs, idx, np.zeros_like(tk), ps), num_partitions=P)
        assert np.array_equal(bits_of(b), bits_of(c))
        if P:
            assert np.array_equal(bits_of(plain), bits_of(b))
        else:
            compare(to_f64(b), to_f64(plain), FP8_TOL, "extended forms vs plain, library split")


def test_second_stream_poison_and_bad_rows():
    """Second-pool rows that are not listed, or listed past extra_topk_lengths, are never
    read (NaN-poisoned: bitwise-equal output); a listed row outside the second pool is
    skipped and sets bit 1 of the device error word."""
    m = need_gpu()
    case = make_sparse_case(407, 5, 64, 800, 64, (10, 400), 400, name="ext-poison")
    c8, cs, idx, tk, ps = second_stream(408, 5, 16, 300, 120, (5, 100))
    sink = sink_logits(409, 64)
    clean = bits_of(ext_on_gpu(m, case, (c8, cs, idx, tk, ps), sink))
    listed = np.zeros(c8.shape[0] * ps, dtype=bool)
    for t in range(5):
        r = idx[t, :tk[t]]
        listed[r[r >= 0]] = True
    p8, pcs = c8.copy(), cs.copy()
    p8.reshape(-1, 576)[~listed] = 0x7F
    pcs.reshape(-1)[~listed] = np.nan
    poisoned = bits_of(ext_on_gpu(m, case, (p8, pcs, idx, tk, ps), sink))
    assert np.array_equal(clean, poisoned)
    m.check_device_errors()
    bad = idx.copy()
    bad[2, 0] = c8.shape[0] * ps + 5
    tk2 = tk.copy()
    tk2[2] = max(1, tk2[2])
    got = to_f64(ext_on_gpu(m, case, (c8, cs, bad, tk2, ps), sink))
    assert m.check_device_errors() & 2
    assert np.all(np.isfinite(got))
    want = oracle_of(case, (c8, cs, bad, tk2, ps), sink)
    compare(got, want, FP8_TOL, "second stream with a row outside its pool")
