"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin fails.

Each mutant patches one oracle function for the duration of the test; the pins then
run against the mutated oracle and at least one of them must raise.
"""
import numpy as np
import pytest

import oracle.mla_oracle as O
from oracle_pins import ALL_PINS

_attend = O.attend
_visible = O.visible_range
_rows = O.logical_rows
_sparse_rows = O.sparse_rows
_rank_order = O.rank_order
_decode_sparse_f64 = O.decode_sparse_f64


def m_scale_dropped(mp):
    mp.setattr(O, "attend", lambda q, k, v, scale, *a, **kw: _attend(q, k, v, 1.0, *a, **kw))


def m_values_shifted(mp):
    mp.setattr(O, "value_columns", lambda keys: keys[:, 64:])


def m_causal_off_by_one(mp):
    def vr(L, n, j, mask, window=-1):
        lo, hi = _visible(L, n, j, mask, window)
        return (lo, max(lo, hi - 1)) if mask != "null" else (lo, hi)
    mp.setattr(O, "visible_range", vr)


def m_token_order_reversed(mp):
    mp.setattr(O, "visible_range", lambda L, n, j, mask, window=-1: _visible(L, n, n - 1 - j, mask, window))


def m_page_slot_swapped(mp):
    def rows(cache, table_row, positions, page_size):
        positions = np.asarray(positions, dtype=np.int64)
        pages = np.asarray(table_row, dtype=np.int64)[positions % page_size]
        return cache[pages, np.minimum(positions // page_size, page_size - 1)]
    mp.setattr(O, "logical_rows", rows)


def m_combine_unweighted(mp):
    def comb(parts):
        parts = list(parts)
        return np.mean([o for o, _ in parts], axis=0), np.max([l for _, l in parts], axis=0)
    mp.setattr(O, "combine", comb)


def m_no_max_subtraction(mp):
    def att(q, keys, values, scale, visible=None, return_probs=False):
        R = q.shape[0]
        if keys.shape[0] == 0:
            return _attend(q, keys, values, scale, visible, return_probs)
        s = scale * (q @ keys.T)
        if visible is not None:
            s = np.where(visible, s, -np.inf)
        with np.errstate(over="ignore", invalid="ignore"):
            p = np.exp(s)
            l = p.sum(axis=1)
            out = (p @ values) / l[:, None]
            lse = np.log(l)
        return (out, lse, p / l[:, None]) if return_probs else (out, lse)
    mp.setattr(O, "attend", att)


def m_softmax_over_heads(mp):
    def att(q, keys, values, scale, visible=None, return_probs=False):
        if keys.shape[0] == 0 or q.shape[0] == 1:
            # a softmax over a single row is the same either way; break it another way
            out, lse, *rest = _attend(q, keys, values, scale, visible, True)
            return (out * 0.999, lse, *rest) if return_probs else (out * 0.999, lse)
        s = scale * (q @ keys.T)
        m = s.max(axis=0)
        p = np.exp(s - m[None, :])
        l = p.sum(axis=0)
        pn = p / l[None, :]
        out = pn @ values
        lse = m.max() + np.log(l.sum()) + np.zeros(q.shape[0])
        return (out, lse, pn) if return_probs else (out, lse)
    mp.setattr(O, "attend", att)


def m_lse_without_max(mp):
    def att(q, keys, values, scale, visible=None, return_probs=False):
        r = list(_attend(q, keys, values, scale, visible, True))
        o, lse, p = r
        s = scale * (q @ keys.T) if keys.shape[0] else np.zeros((q.shape[0], 1))
        lse = np.where(np.isfinite(lse), lse - s.max(axis=1), lse)
        return (o, lse, p) if return_probs else (o, lse)
    mp.setattr(O, "attend", att)


def m_e4m3_bias8(mp):
    def val(code):
        code = int(code) & 0xFF
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 7
        if e == 15 and m == 7:
            return float("nan")
        if e == 0:
            return sign * (m / 8.0) * 2.0 ** (1 - 8)
        return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)
    mp.setattr(O, "E4M3_TABLE", np.array([val(c) for c in range(256)]))


def m_sparse_ignores_topk(mp):
    mp.setattr(O, "sparse_rows", lambda row, topk, pool: _sparse_rows(row, len(row), pool))


def m_sparse_keeps_pads(mp):
    def sr(row, topk, pool):
        listed = np.asarray(row[:max(0, int(topk))], dtype=np.int64)
        return np.where(listed < 0, 0, listed)
    mp.setattr(O, "sparse_rows", sr)


def m_prefill_rope_at_query(mp):
    """Rope taken from the wrong cache rows (shifted by one position)."""
    def rows(cache, table_row, positions, page_size):
        positions = np.asarray(positions, dtype=np.int64)
        shifted = np.minimum(positions + 1, positions.max(initial=0))
        return _rows(cache, table_row, shifted, page_size)
    mp.setattr(O, "logical_rows", rows)


def m_bf16_low_half(mp):
    def dec(bits):
        u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
        return (u32 << np.uint32(15)).view(np.float32).astype(np.float64)
    mp.setattr(O, "bf16_to_f64", dec)


def m_indexer_unweighted_heads(mp):
    """The head scores summed without their q_s weights."""
    def scores(q8_t, q_s_t, k8_rows, k_scale_rows):
        s = (O.e4m3_to_f64(k8_rows) @ O.e4m3_to_f64(q8_t).T).sum(axis=1)
        return s if k_scale_rows is None else s * np.asarray(k_scale_rows, dtype=np.float64)
    mp.setattr(O, "indexer_scores", scores)


def m_indexer_ties_reversed(mp):
    """Equal scores ranked by descending position."""
    mp.setattr(O, "rank_order", lambda sc, pos: np.lexsort((-np.asarray(pos), -np.asarray(sc, dtype=np.float64))))


def m_sink_dropped(mp):
    mp.setattr(O, "attend", lambda q, k, v, scale, visible=None, return_probs=False, sink=None:
               _attend(q, k, v, scale, visible, return_probs))


def m_sink_scaled(mp):
    """The sink logit multiplied by the attention scale like a dot product."""
    def att(q, k, v, scale, visible=None, return_probs=False, sink=None):
        return _attend(q, k, v, scale, visible, return_probs, None if sink is None else np.asarray(sink) * scale)
    mp.setattr(O, "attend", att)


def m_sink_in_numerator(mp):
    """The sink treated as a key whose value row is all ones."""
    def att(q, k, v, scale, visible=None, return_probs=False, sink=None):
        if sink is None:
            return _attend(q, k, v, scale, visible, return_probs)
        R = q.shape[0]
        s = scale * (q @ k.T) if k.shape[0] else np.zeros((R, 0))
        snk = np.asarray(sink, dtype=np.float64)
        m = np.maximum(s.max(axis=1, initial=-np.inf), snk)
        p = np.exp(s - m[:, None])
        ps = np.exp(snk - m)
        l = p.sum(axis=1) + ps
        out = (p @ v + ps[:, None]) / l[:, None]
        lse = m + np.log(l)
        return (out, lse, p / l[:, None]) if return_probs else (out, lse)
    mp.setattr(O, "attend", att)


def m_extra_stream_ignored(mp):
    mp.setattr(O, "decode_sparse_f64", lambda *a, extra=None, **kw: _decode_sparse_f64(*a, extra=None, **kw))


def m_extra_reads_main_cache(mp):
    """The second list's rows looked up in the main cache."""
    def dsp(q, off, cache, idx, topk, ps, scale, rows=None, extra=None, attn_sink=None):
        if extra is not None:
            extra = (cache, extra[1], extra[2], ps)
        return _decode_sparse_f64(q, off, cache, idx, topk, ps, scale, rows, extra=extra, attn_sink=attn_sink)
    mp.setattr(O, "decode_sparse_f64", dsp)


_rope_aware = O.rope_aware_to_f64


def m_rope_scaled(mp):
    """The row scale applied to the rope values as well."""
    def f(raw, scales):
        v = _rope_aware(raw, None)
        return v if scales is None else v * np.asarray(scales, dtype=np.float64)[..., None]
    mp.setattr(O, "rope_aware_to_f64", f)


def m_rope_big_endian(mp):
    """The rope values read with their bytes swapped."""
    def f(raw, scales):
        raw = np.array(raw, dtype=np.uint8, copy=True)
        r = raw[..., 512:].reshape(raw.shape[:-1] + (64, 2))
        raw[..., 512:] = r[..., ::-1].reshape(raw.shape[:-1] + (128,))
        return _rope_aware(raw, scales)
    mp.setattr(O, "rope_aware_to_f64", f)


def m_rope_unscaled_latent(mp):
    """The latent codes left without their scale."""
    mp.setattr(O, "rope_aware_to_f64", lambda raw, scales: _rope_aware(raw, None))


_token_lists = O.token_lists


def m_shared_lists_by_token(mp):
    """Token t takes list row t (clamped) instead of its sequence's row."""
    def tl(off, idx, topk):
        T = int(np.asarray(off)[-1])
        r = np.minimum(np.arange(T), len(topk) - 1)
        return np.asarray(idx)[r], np.asarray(topk)[r]
    mp.setattr(O, "token_lists", tl)


def m_shared_lists_first_token_only(mp):
    """Only the first token of each sequence sees the list; the others see none."""
    def tl(off, idx, topk):
        i, k = _token_lists(off, idx, topk)
        k = k.copy()
        first = np.asarray(off, dtype=np.int64)[:-1]
        keep = np.zeros(len(k), dtype=bool)
        keep[first[first < len(k)]] = True
        k[~keep] = 0
        return i, k
    mp.setattr(O, "token_lists", tl)


MUTANTS = [m_scale_dropped, m_values_shifted, m_causal_off_by_one, m_token_order_reversed,
           m_page_slot_swapped, m_combine_unweighted, m_no_max_subtraction, m_softmax_over_heads,
           m_lse_without_max, m_e4m3_bias8, m_sparse_ignores_topk, m_sparse_keeps_pads,
           m_prefill_rope_at_query, m_bf16_low_half,
           m_indexer_unweighted_heads, m_indexer_ties_reversed, m_sink_dropped, m_sink_scaled,
           m_sink_in_numerator, m_extra_stream_ignored, m_extra_reads_main_cache,
           m_rope_scaled, m_rope_big_endian, m_rope_unscaled_latent, m_shared_lists_by_token,
           m_shared_lists_first_token_only]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_some_pin_catches(mutant, monkeypatch):
    mutant(monkeypatch)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"{mutant.__name__}: no pin failed"
