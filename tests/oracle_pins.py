"""Pins for the CPU oracle: each function checks the oracle against something other than
itself (brute force on tiny inputs, closed forms, invariants, format definitions) and
raises AssertionError on failure.  They are collected as tests by test_oracle_pins.py
and re-run under planted mistakes by test_oracle_mutants.py.

Every oracle call goes through the module object ``O`` so that a patched function is
the one that runs.
"""
import math
import os

import numpy as np

import oracle.mla_oracle as O
from brute import attention_row, decode_contiguous

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
D = 576
DV = 512
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


# --------------------------------------------------------------------------------------
# tiny-input builders (layout only)
# --------------------------------------------------------------------------------------

def page_up(seq_keys, page_size, rng, spare=2, fill=np.nan):
    """Scatter contiguous per-sequence rows into a shuffled page pool; unused slots = fill."""
    npages = [-(-len(k) // page_size) for k in seq_keys]
    total = sum(npages) + spare
    perm = rng.permutation(total)
    width = max(1, max(npages))
    cache = np.full((total, page_size, seq_keys[0].shape[1]), fill)
    table = np.full((len(seq_keys), width), -1, dtype=np.int32)
    cur = 0
    for b, keys in enumerate(seq_keys):
        for j in range(npages[b]):
            pid = int(perm[cur])
            cur += 1
            table[b, j] = pid
            chunk = keys[j * page_size:(j + 1) * page_size]
            cache[pid, :len(chunk)] = chunk
    lens = np.array([len(k) for k in seq_keys], dtype=np.int32)
    return cache, table, lens


def offsets_of(n_tokens):
    off = np.zeros(len(n_tokens) + 1, dtype=np.uint32)
    off[1:] = np.cumsum(n_tokens)
    return off


def tiny_decode(seed=1, lens=(5, 37, 20), n_tokens=(1, 3, 2), H=2, page_size=16, q_std=1.0):
    rng = np.random.default_rng(seed)
    seq_keys = [rng.standard_normal((L, D)) for L in lens]
    T = sum(n_tokens)
    q = rng.standard_normal((T, H, D)) * q_std
    cache, table, lens_arr = page_up(seq_keys, page_size, rng)
    return dict(q=q, seq_keys=seq_keys, cache=cache, table=table, lens=lens_arr,
                off=offsets_of(n_tokens), n_tokens=list(n_tokens), page_size=page_size)


def run_dense(c, mask="causal", window=-1, scale=SCALE, table=None, cache=None):
    return O.decode_paged_f64(c["q"], c["off"], c["table"] if table is None else table,
                              c["lens"], c["cache"] if cache is None else cache,
                              c["page_size"], scale, mask, window)


def close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(same_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), "non-finite mismatch"
    assert diff.max(initial=0.0) <= tol, f"max diff {diff.max()} > {tol}"


# --------------------------------------------------------------------------------------
# P1: brute force on contiguous (unpaged) keys
# --------------------------------------------------------------------------------------

def pin_p1_dense_causal():
    c = tiny_decode()
    out, lse = run_dense(c, "causal")
    bo, bl = decode_contiguous(c["q"].tolist(), [k.tolist() for k in c["seq_keys"]],
                               c["n_tokens"], SCALE, "causal")
    close(out, bo, 1e-12)
    close(lse, bl, 1e-12)


def pin_p1_dense_null():
    c = tiny_decode(seed=2, lens=(9, 17), n_tokens=(2, 1), page_size=4)
    out, lse = run_dense(c, "null")
    bo, bl = decode_contiguous(c["q"].tolist(), [k.tolist() for k in c["seq_keys"]],
                               c["n_tokens"], SCALE, "null")
    close(out, bo, 1e-12)
    close(lse, bl, 1e-12)


def pin_p1_dense_sliding():
    c = tiny_decode(seed=3, lens=(12, 30), n_tokens=(3, 2), page_size=8)
    out, lse = run_dense(c, "sliding_window_causal", window=5)
    bo, bl = decode_contiguous(c["q"].tolist(), [k.tolist() for k in c["seq_keys"]],
                               c["n_tokens"], SCALE, "sliding_window_causal", window=5)
    close(out, bo, 1e-12)
    close(lse, bl, 1e-12)


def _torch_e4m3(codes):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def tiny_sparse(seed=4, H=2, page_size=8, pages=5, T=3, stride=9):
    rng = np.random.default_rng(seed)
    # finite E4M3 codes only (exclude the two NaN codes)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    cache8 = rng.choice(finite, size=(pages, page_size, D)).astype(np.uint8)
    q8 = rng.choice(finite[(finite & 0x78) < 0x50], size=(T, H, D)).astype(np.uint8)  # |q| <= 8
    q_scale = rng.uniform(0.001, 0.01, size=T).astype(np.float32)
    c_scale = rng.uniform(0.001, 0.01, size=(pages, page_size)).astype(np.float32)
    rows = pages * page_size
    idx = np.full((T, stride), -1, dtype=np.int32)
    topk = np.array([7, 1, 9], dtype=np.int32)[:T]
    for t in range(T):
        idx[t] = rng.integers(0, rows, size=stride)
    idx[0, 2] = -1            # a pad inside the counted prefix is skipped
    idx[2, 3] = idx[2, 5]     # a duplicate counts twice
    return dict(q8=q8, q_scale=q_scale, cache8=cache8, c_scale=c_scale, idx=idx, topk=topk,
                page_size=page_size, off=np.arange(T + 1, dtype=np.uint32))


def pin_p1_sparse():
    s = tiny_sparse()
    out, lse = O.decode_sparse(s["q8"], s["q_scale"], s["off"], s["cache8"], s["c_scale"],
                               s["idx"], s["topk"], s["page_size"], SCALE)
    ps = s["page_size"]
    qv = _torch_e4m3(s["q8"]) * s["q_scale"].astype(np.float64)[:, None, None]
    cv = _torch_e4m3(s["cache8"]) * s["c_scale"].astype(np.float64)[:, :, None]
    for t in range(len(s["topk"])):
        keys = []
        for i in range(int(s["topk"][t])):
            r = int(s["idx"][t, i])
            if r < 0:
                continue
            keys.append(cv[r // ps, r % ps].tolist())
        for h in range(qv.shape[1]):
            o, l = attention_row(qv[t, h].tolist(), keys, [k[:DV] for k in keys], SCALE)
            close(out[t, h], o, 1e-12)
            close(lse[t, h], l, 1e-12)


def pin_p1_dense_fp8():
    """Dense fp8 decode against brute force on contiguous keys, dequantised independently
    (torch's float8_e4m3fn widening times the row / token scales); the pool's unused
    slots hold the NaN code with a NaN scale and must never be read."""
    rng = np.random.default_rng(21)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    lens, n_tokens, H, ps = (13, 30), (2, 3), 2, 8
    seq_codes = [rng.choice(finite, size=(L, D)).astype(np.uint8) for L in lens]
    seq_scales = [rng.uniform(0.001, 0.01, size=L).astype(np.float32) for L in lens]
    T = sum(n_tokens)
    q8 = rng.choice(finite[(finite & 0x78) < 0x50], size=(T, H, D)).astype(np.uint8)
    q_scale = rng.uniform(0.001, 0.01, size=T).astype(np.float32)
    npages = [-(-L // ps) for L in lens]
    total = sum(npages) + 2
    perm = rng.permutation(total)
    cache8 = np.full((total, ps, D), 0x7F, dtype=np.uint8)
    c_scale = np.full((total, ps), np.nan, dtype=np.float32)
    table = np.full((len(lens), max(npages)), -1, dtype=np.int32)
    cur = 0
    for b, L in enumerate(lens):
        for j in range(npages[b]):
            pid = int(perm[cur])
            cur += 1
            table[b, j] = pid
            n = min(ps, L - j * ps)
            cache8[pid, :n] = seq_codes[b][j * ps:j * ps + n]
            c_scale[pid, :n] = seq_scales[b][j * ps:j * ps + n]
    off = offsets_of(n_tokens)
    qv = _torch_e4m3(q8) * q_scale.astype(np.float64)[:, None, None]
    keys = [(_torch_e4m3(seq_codes[b]) * seq_scales[b].astype(np.float64)[:, None]).tolist() for b in range(2)]
    for mask, window in (("causal", -1), ("sliding_window_causal", 4), ("null", -1)):
        out, lse = O.decode_paged_fp8(q8, q_scale, off, table, np.array(lens, dtype=np.int32), cache8, c_scale,
                                      ps, SCALE, mask, window)
        bo, bl = decode_contiguous(qv.tolist(), keys, list(n_tokens), SCALE, mask, window)
        close(out, bo, 1e-12)
        close(lse, bl, 1e-12)


def _torch_bf16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float32).numpy().astype(np.float64)


def _rope_rows(rng, n, finite):
    """n rope-aware rows (640 bytes: 512 E4M3 codes, then 64 bf16 rope values) with their
    independent float64 reading: torch's e4m3 widening times the scale, torch's bf16."""
    codes = rng.choice(finite, size=(n, 512)).astype(np.uint8)
    rope = (rng.standard_normal((n, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    raw = np.concatenate([codes, rope.astype("<u2").view(np.uint8).reshape(n, 128)], axis=1)
    return raw, codes, rope


def pin_rope_aware_row_layout():
    """One hand-built row: the latent codes sit at bytes 0..511 and take the scale, the
    rope values are little-endian bf16 at bytes 512..639 and do not."""
    raw = np.zeros((1, 640), dtype=np.uint8)
    raw[0, 0] = 0x38          # E4M3 1.0
    raw[0, 511] = 0xC0        # E4M3 -2.0
    raw[0, 512:514] = (0x80, 0x3F)  # bf16 0x3F80 = 1.0, low byte first
    raw[0, 638:640] = (0x40, 0xC0)  # bf16 0xC040 = -3.0
    got = O.rope_aware_to_f64(raw, np.array([0.25], dtype=np.float32))
    want = np.zeros((1, 576))
    want[0, 0], want[0, 511], want[0, 512], want[0, 575] = 0.25, -0.5, 1.0, -3.0
    close(got, want, 0.0)


def pin_rope_aware_dense_fp8():
    """Dense decode over a rope-aware cache against brute force on contiguous keys read
    independently; one cache row has scale 0, which silences its latent part only.  The
    pool's unused slots hold NaN codes and NaN scales and must never be read."""
    rng = np.random.default_rng(41)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    small = finite[(finite & 0x78) < 0x50]
    lens, n_tokens, H, ps = (11, 26), (2, 3), 2, 8
    T = sum(n_tokens)
    seq = [_rope_rows(rng, L, finite) for L in lens]
    scales = [rng.uniform(0.001, 0.01, size=L).astype(np.float32) for L in lens]
    scales[1][4] = 0.0
    qraw, qcodes, qrope = _rope_rows(rng, T * H, small)
    qraw, qcodes, qrope = qraw.reshape(T, H, 640), qcodes.reshape(T, H, 512), qrope.reshape(T, H, 64)
    q_scale = rng.uniform(0.01, 0.1, size=T).astype(np.float32)
    npages = [-(-L // ps) for L in lens]
    total = sum(npages) + 2
    perm = rng.permutation(total)
    cache = np.full((total, ps, 640), 0xFF, dtype=np.uint8)
    c_scale = np.full((total, ps), np.nan, dtype=np.float32)
    table = np.full((len(lens), max(npages)), -1, dtype=np.int32)
    cur = 0
    for b, L in enumerate(lens):
        for j in range(npages[b]):
            pid = int(perm[cur])
            cur += 1
            table[b, j] = pid
            n = min(ps, L - j * ps)
            cache[pid, :n] = seq[b][0][j * ps:j * ps + n]
            c_scale[pid, :n] = scales[b][j * ps:j * ps + n]
    off = offsets_of(n_tokens)
    qv = np.concatenate([_torch_e4m3(qcodes) * q_scale.astype(np.float64)[:, None, None], _torch_bf16(qrope)], axis=2)
    keys = [np.concatenate([_torch_e4m3(seq[b][1]) * scales[b].astype(np.float64)[:, None], _torch_bf16(seq[b][2])],
                           axis=1).tolist() for b in range(2)]
    for mask, window in (("causal", -1), ("sliding_window_causal", 5), ("null", -1)):
        out, lse = O.decode_paged_fp8_rope_aware(qraw, q_scale, off, table, np.array(lens, dtype=np.int32), cache,
                                                 c_scale, ps, SCALE, mask, window)
        bo, bl = decode_contiguous(qv.tolist(), keys, list(n_tokens), SCALE, mask, window)
        close(out, bo, 1e-12)
        close(lse, bl, 1e-12)


def pin_rope_aware_sparse():
    """Sparse decode over a rope-aware cache against attention_row on the listed rows."""
    rng = np.random.default_rng(42)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    small = finite[(finite & 0x78) < 0x50]
    H, ps, pages, T, stride = 2, 8, 4, 3, 7
    raw, codes, rope = _rope_rows(rng, pages * ps, finite)
    c_scale = rng.uniform(0.001, 0.01, size=pages * ps).astype(np.float32)
    qraw, qcodes, qrope = _rope_rows(rng, T * H, small)
    q_scale = rng.uniform(0.01, 0.1, size=T).astype(np.float32)
    idx = rng.integers(0, pages * ps, size=(T, stride)).astype(np.int32)
    idx[1, 0] = -1
    topk = np.array([5, 3, 7], dtype=np.int32)
    out, lse = O.decode_sparse_rope_aware(qraw.reshape(T, H, 640), q_scale, np.arange(T + 1, dtype=np.uint32),
                                          raw.reshape(pages, ps, 640), c_scale.reshape(pages, ps), idx, topk, ps,
                                          SCALE)
    kv = np.concatenate([_torch_e4m3(codes) * c_scale.astype(np.float64)[:, None], _torch_bf16(rope)], axis=1)
    qv = np.concatenate([_torch_e4m3(qcodes).reshape(T, H, 512) * q_scale.astype(np.float64)[:, None, None],
                         _torch_bf16(qrope).reshape(T, H, 64)], axis=2)
    for t in range(T):
        keys = [kv[int(r)].tolist() for r in idx[t, :topk[t]] if r >= 0]
        for h in range(H):
            o, l = attention_row(qv[t, h].tolist(), keys, [k[:DV] for k in keys], SCALE)
            close(out[t, h], o, 1e-12)
            close(lse[t, h], l, 1e-12)


def pin_shared_index_lists():
    """Query tokens sharing their sequence's list, against attention_row over that list:
    3 sequences with 2, 1 and 3 tokens, lists of different lengths with a pad inside."""
    rng = np.random.default_rng(43)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    small = finite[(finite & 0x78) < 0x50]
    H, ps, pages, stride = 2, 8, 5, 9
    n_tokens = (2, 1, 3)
    off = offsets_of(n_tokens)
    T, B = int(off[-1]), len(n_tokens)
    cache8 = rng.choice(finite, size=(pages, ps, D)).astype(np.uint8)
    c_scale = rng.uniform(0.001, 0.01, size=(pages, ps)).astype(np.float32)
    q8 = rng.choice(small, size=(T, H, D)).astype(np.uint8)
    q_scale = rng.uniform(0.001, 0.01, size=T).astype(np.float32)
    idx = rng.integers(0, pages * ps, size=(B, stride)).astype(np.int32)
    idx[2, 1] = -1
    topk = np.array([6, 2, 9], dtype=np.int32)
    out, lse = O.decode_sparse_shared(q8, q_scale, off, cache8, c_scale, idx, topk, ps, SCALE)
    kv = _torch_e4m3(cache8).reshape(pages * ps, D) * c_scale.reshape(-1).astype(np.float64)[:, None]
    qv = _torch_e4m3(q8) * q_scale.astype(np.float64)[:, None, None]
    t = 0
    for b, n in enumerate(n_tokens):
        keys = [kv[int(r)].tolist() for r in idx[b, :topk[b]] if r >= 0]
        for _ in range(n):
            for h in range(H):
                o, l = attention_row(qv[t, h].tolist(), keys, [k[:DV] for k in keys], SCALE)
                close(out[t, h], o, 1e-12)
                close(lse[t, h], l, 1e-12)
            t += 1


def pin_p1_indexer():
    """The indexer against scalar brute force: scores by plain loops over heads and
    columns with math.fsum (torch's e4m3 widening), selection by a full sort of
    (-score, position), physical rows through the page table, -1 fill."""
    rng = np.random.default_rng(22)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    NH, Dk, ps, top_k = 3, 16, 4, 6
    lens, n_tokens = (9, 3), (2, 1)
    pages_needed = [-(-L // ps) for L in lens]
    total = sum(pages_needed) + 1
    k8 = rng.choice(finite, size=(total, ps, Dk)).astype(np.uint8)
    k_scale = rng.uniform(0.5, 2.0, size=(total, ps)).astype(np.float32)
    perm = rng.permutation(total)
    table = np.full((2, max(pages_needed)), -1, dtype=np.int32)
    cur = 0
    for b in range(2):
        for j in range(pages_needed[b]):
            table[b, j] = perm[cur]
            cur += 1
    T = sum(n_tokens)
    q8 = rng.choice(finite, size=(T, NH, Dk)).astype(np.uint8)
    q_s = rng.uniform(0.5, 2.0, size=(T, NH)).astype(np.float32)
    off = offsets_of(n_tokens)
    for mask, window in (("causal", -1), ("null", -1), ("sliding_window_causal", 3)):
        got = O.indexer_paged_fp8(q8, q_s, off, table, np.array(lens, dtype=np.int32), k8, k_scale, ps, top_k,
                                  mask, window)
        qv, kv = _torch_e4m3(q8), _torch_e4m3(k8)
        t = 0
        for b, L in enumerate(lens):
            n = n_tokens[b]
            for j in range(n):
                pos_t = L - n + j
                vis = []
                for r in range(L):
                    if mask != "null" and r > pos_t:
                        continue
                    if mask == "sliding_window_causal" and r <= pos_t - window:
                        continue
                    pg, sl = int(table[b, r // ps]), r % ps
                    sc = math.fsum(float(q_s[t, h]) * math.fsum(qv[t, h, d] * kv[pg, sl, d] for d in range(Dk))
                                   for h in range(NH)) * float(k_scale[pg, sl])
                    vis.append((-sc, r, pg * ps + sl))
                vis.sort()
                want = [v[2] for v in vis[:top_k]] + [-1] * (top_k - min(top_k, len(vis)))
                assert list(got[t]) == want, (mask, t, list(got[t]), want)
                t += 1


def _paged_rows(k_rows, ps, rng, spare=1):
    """Scatter the logical rows of each sequence over a shuffled pool of pages of ps rows."""
    npages = [-(-len(k) // ps) for k in k_rows]
    total = sum(npages) + spare
    perm = rng.permutation(total)
    pool = np.zeros((total, ps, k_rows[0].shape[1]), dtype=np.uint8)
    table = np.full((len(k_rows), max(npages)), -1, dtype=np.int32)
    cur = 0
    for b, rows in enumerate(k_rows):
        for j in range(npages[b]):
            table[b, j] = perm[cur]
            chunk = rows[j * ps:(j + 1) * ps]
            pool[perm[cur], :len(chunk)] = chunk
            cur += 1
    return pool, table


def pin_p1_indexer_head_weights():
    """The per-head weights q_s decide the order ([IDX] Args q_s): codes of moderate size
    (|value| in [0.5, 2)) and q_s log-uniform over 1e-2..1e2, so that the unweighted head
    sum ranks the rows differently (checked here); the oracle must match scalar brute
    force, loops over heads and columns with math.fsum on torch's e4m3 widening."""
    rng = np.random.default_rng(23)
    moderate = np.array([c for c in range(256) if ((c >> 3) & 0xF) in (6, 7)], dtype=np.uint8)
    NH, Dk, ps, top_k = 4, 16, 4, 5
    lens, n_tokens = (23, 14), (1, 2)
    k_rows = [rng.choice(moderate, size=(L, Dk)).astype(np.uint8) for L in lens]
    k8, table = _paged_rows(k_rows, ps, rng)
    k_scale = rng.uniform(0.5, 2.0, size=k8.shape[:2]).astype(np.float32)
    T = sum(n_tokens)
    q8 = rng.choice(moderate, size=(T, NH, Dk)).astype(np.uint8)
    q_s = (10.0 ** rng.uniform(-2.0, 2.0, size=(T, NH))).astype(np.float32)
    off = offsets_of(n_tokens)
    qv, kv = _torch_e4m3(q8), _torch_e4m3(k8)
    got = O.indexer_paged_fp8(q8, q_s, off, table, np.array(lens, dtype=np.int32), k8, k_scale, ps, top_k,
                              "causal", -1)
    weights_matter = False
    t = 0
    for b, L in enumerate(lens):
        n = n_tokens[b]
        for j in range(n):
            pos_t = L - n + j
            weighted, unweighted = [], []
            for r in range(pos_t + 1):
                pg, sl = int(table[b, r // ps]), r % ps
                dots = [math.fsum(qv[t, h, d] * kv[pg, sl, d] for d in range(Dk)) for h in range(NH)]
                ks = float(k_scale[pg, sl])
                weighted.append((-math.fsum(float(q_s[t, h]) * dots[h] for h in range(NH)) * ks, r, pg * ps + sl))
                unweighted.append((-math.fsum(dots) * ks, r, pg * ps + sl))
            weighted.sort()
            unweighted.sort()
            want = [v[2] for v in weighted[:top_k]]
            weights_matter |= want != [v[2] for v in unweighted[:top_k]]
            assert list(got[t]) == want, (t, list(got[t]), want)
            t += 1
    assert weights_matter, "the inputs must make the head weights change the top-k"


def pin_indexer_exact_ties():
    """Equal scores rank by ascending logical position (the reading of [IDX] Args
    output_indices).  Sequence 0: every row identical, so the top-k are the first k
    visible positions.  Sequence 1: three rows of a high-scoring pattern at positions
    {2, 5, 9}, the rest of one low-scoring pattern; top 5 = those three, then positions 0
    and 1.  Expectations are written out by construction, through the page table."""
    rng = np.random.default_rng(24)
    Dk, ps, top_k = 16, 4, 5
    one = 0x38  # e4m3 code of 1.0
    hi_row = np.full(Dk, one, dtype=np.uint8)
    lo_row = np.zeros(Dk, dtype=np.uint8)
    lo_row[0] = one
    seq0 = np.tile(hi_row, (13, 1))
    seq1 = np.tile(lo_row, (11, 1))
    seq1[[2, 5, 9]] = hi_row
    k8, table = _paged_rows([seq0, seq1], ps, rng)
    k_scale = np.ones(k8.shape[:2], dtype=np.float32)
    q8 = np.full((3, 2, Dk), one, dtype=np.uint8)
    q_s = np.array([[1.0, 0.5]] * 3, dtype=np.float32)
    off = offsets_of((2, 1))
    lens = np.array([13, 11], dtype=np.int32)

    def phys(b, positions):
        return [int(table[b, p // ps]) * ps + p % ps for p in positions]

    got = O.indexer_paged_fp8(q8, q_s, off, table, lens, k8, k_scale, ps, top_k, "causal", -1)
    assert list(got[0]) == phys(0, [0, 1, 2, 3, 4])      # token at position 11
    assert list(got[1]) == phys(0, [0, 1, 2, 3, 4])      # token at position 12
    assert list(got[2]) == phys(1, [2, 5, 9, 0, 1])
    got = O.indexer_paged_fp8(q8, q_s, off, table, lens, k8, k_scale, ps, top_k, "sliding_window_causal", 4)
    assert list(got[0]) == phys(0, [8, 9, 10, 11]) + [-1]
    assert list(got[2]) == phys(1, [9, 7, 8, 10]) + [-1]


def tiny_sparse_extra(seed=30, H=2, T=3):
    """A sparse case with a second KV stream (its own fp8 pool, page size and row scales)
    and per-head sink logits."""
    rng = np.random.default_rng(seed)
    base = tiny_sparse(seed=seed, H=H, T=T)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    pages2, ps2, stride2 = 3, 4, 6
    cache8_2 = rng.choice(finite, size=(pages2, ps2, D)).astype(np.uint8)
    c_scale_2 = rng.uniform(0.001, 0.01, size=(pages2, ps2)).astype(np.float32)
    idx2 = rng.integers(0, pages2 * ps2, size=(T, stride2)).astype(np.int32)
    idx2[1, 0] = -1                       # a pad inside the counted prefix is skipped
    topk2 = np.array([4, 0, 6], dtype=np.int32)[:T]
    sink = rng.normal(0.0, 2.0, size=H)
    base.update(cache8_2=cache8_2, c_scale_2=c_scale_2, idx2=idx2, topk2=topk2, ps2=ps2, sink=sink)
    return base


def _run_sparse_extra(c, extra=True, sink=True):
    ex = (c["cache8_2"], c["c_scale_2"], c["idx2"], c["topk2"], c["ps2"]) if extra else None
    return O.decode_sparse(c["q8"], c["q_scale"], c["off"], c["cache8"], c["c_scale"], c["idx"], c["topk"],
                           c["page_size"], SCALE, extra=ex, attn_sink=c["sink"] if sink else None)


def pin_p1_sparse_extra_stream_and_sink():
    """Sparse decode with a second KV stream and sink logits against scalar brute force:
    the keys of a row are its listed main rows then its listed extra rows (each widened by
    torch's e4m3 conversion times its own pool's row scale), one softmax over all of them
    plus e^sink[h] in the denominator."""
    c = tiny_sparse_extra()
    out, lse = _run_sparse_extra(c)
    qv = _torch_e4m3(c["q8"]) * c["q_scale"][:, None, None].astype(np.float64)
    kv1 = _torch_e4m3(c["cache8"]) * c["c_scale"][..., None].astype(np.float64)
    kv2 = _torch_e4m3(c["cache8_2"]) * c["c_scale_2"][..., None].astype(np.float64)
    ps, ps2 = c["page_size"], c["ps2"]
    for t in range(qv.shape[0]):
        keys = []
        for i in range(int(c["topk"][t])):
            r = int(c["idx"][t, i])
            if 0 <= r < kv1.shape[0] * ps:
                keys.append(kv1[r // ps, r % ps].tolist())
        for i in range(int(c["topk2"][t])):
            r = int(c["idx2"][t, i])
            if 0 <= r < kv2.shape[0] * ps2:
                keys.append(kv2[r // ps2, r % ps2].tolist())
        for h in range(qv.shape[1]):
            bo, bl = attention_row(qv[t, h].tolist(), keys, [k[:DV] for k in keys], SCALE,
                                   sink=float(c["sink"][h]), dv=DV)
            close(out[t, h], bo, 1e-12)
            close(lse[t, h], bl, 1e-12)


def pin_sink_at_minus_infinity_is_no_sink():
    """A sink logit of -inf adds e^-inf = 0: exactly the result without a sink."""
    c = tiny_sparse_extra(seed=31)
    c["sink"] = np.full_like(c["sink"], -np.inf)
    a = _run_sparse_extra(c)
    b = _run_sparse_extra(c, sink=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def pin_sink_one_key_closed_form():
    """One key of logit s and a sink s*: out = v / (1 + e^(s* - s)), lse = log(e^s + e^s*)
    (the sink never enters the numerator and is not multiplied by scale)."""
    rng = np.random.default_rng(32)
    q = rng.standard_normal((1, 3, D))
    key = rng.standard_normal((1, 1, D))
    sink = np.array([-1.5, 0.3, 4.0])
    out, lse = O.decode_sparse_f64(q, np.array([0, 1], np.uint32), key, np.array([[0]], np.int32),
                                   np.array([1], np.int32), 1, SCALE, attn_sink=sink)
    s = SCALE * (q[0] @ key[0, 0])
    want = key[0, 0, :DV][None, :] / (1.0 + np.exp(sink - s))[:, None]
    close(out[0], want, 1e-14)
    close(lse[0], np.logaddexp(s, sink), 1e-13)
    # no key at all: the sink takes all the weight
    out0, lse0 = O.decode_sparse_f64(q, np.array([0, 1], np.uint32), key, np.array([[-1]], np.int32),
                                     np.array([1], np.int32), 1, SCALE, attn_sink=sink)
    assert np.all(out0 == 0.0)
    close(lse0[0], sink, 0.0)


def pin_sink_is_a_zero_valued_part():
    """Adding a sink equals merging the sink-free result with a part of output 0 and
    log-sum-exp sink (the split-KV merge of generic_flare_mla_decode_kv_cache_ragged)."""
    c = tiny_sparse_extra(seed=33)
    with_sink = _run_sparse_extra(c)
    without = _run_sparse_extra(c, sink=False)
    for t in range(with_sink[0].shape[0]):
        o, l = O.combine([(without[0][t], without[1][t]),
                          (np.zeros_like(without[0][t]), np.asarray(c["sink"], dtype=np.float64))])
        close(with_sink[0][t], o, 1e-13)
        close(with_sink[1][t], l, 1e-12)


def pin_extra_stream_is_one_merged_pool():
    """A second stream equals one stream over a pool that holds both caches' rows (page
    size 1, the extra rows placed after the main ones, their indices shifted by the main
    pool's row count), without reference to the merge algebra."""
    c = tiny_sparse_extra(seed=34)
    got = _run_sparse_extra(c)
    ps, ps2 = c["page_size"], c["ps2"]
    n1 = c["cache8"].shape[0] * ps
    pool = np.concatenate([c["cache8"].reshape(-1, 1, D), c["cache8_2"].reshape(-1, 1, D)])
    scales = np.concatenate([c["c_scale"].reshape(-1, 1), c["c_scale_2"].reshape(-1, 1)])
    T = c["idx"].shape[0]
    width = c["idx"].shape[1] + c["idx2"].shape[1]
    idx = np.full((T, width), -1, dtype=np.int32)
    topk = np.zeros(T, dtype=np.int32)
    for t in range(T):
        a = [int(x) for x in c["idx"][t, :c["topk"][t]]]
        b = [int(x) + n1 if x >= 0 else -1 for x in c["idx2"][t, :c["topk2"][t]]]
        idx[t, :len(a) + len(b)] = a + b
        topk[t] = len(a) + len(b)
    want = O.decode_sparse(c["q8"], c["q_scale"], c["off"], pool, scales, idx, topk, 1, SCALE,
                           attn_sink=c["sink"])
    close(got[0], want[0], 1e-13)
    close(got[1], want[1], 1e-12)


def pin_extra_stream_is_combine_of_streams():
    """Attention over both lists equals the log-sum-exp merge of attention over each list
    alone (P8 algebra on a key partition)."""
    c = tiny_sparse_extra(seed=35)
    both = _run_sparse_extra(c, sink=False)
    main = _run_sparse_extra(c, extra=False, sink=False)
    c2 = dict(c, cache8=c["cache8_2"], c_scale=c["c_scale_2"], idx=c["idx2"], topk=c["topk2"], page_size=c["ps2"])
    other = _run_sparse_extra(c2, extra=False, sink=False)
    for t in range(both[0].shape[0]):
        o, l = O.combine([(main[0][t], main[1][t]), (other[0][t], other[1][t])])
        close(both[0][t], o, 1e-13)
        close(both[1][t], l, 1e-12)


def tiny_prefill(seed=5, new=(3, 4), prefix=(0, 2), H=2, page_size=4):
    rng = np.random.default_rng(seed)
    total = [a + b for a, b in zip(new, prefix)]
    seq_cache = [rng.standard_normal((L, D)) for L in total]
    cache, table, lens = page_up(seq_cache, page_size, rng)
    Tq, Tk = sum(new), sum(total)
    q = rng.standard_normal((Tq, H, 192))
    k = rng.standard_normal((Tk, H, 128))
    v = rng.standard_normal((Tk, H, 128))
    return dict(q=q, k=k, v=v, bro=offsets_of(total), cofs=np.zeros(len(new), dtype=np.uint32),
                ino=offsets_of(new), table=table, lens=lens, cache=cache, seq_cache=seq_cache,
                page_size=page_size, new=list(new), total=total)


def run_prefill(p, mask="causal", **kw):
    return O.prefill_paged_f64(p["q"], p["k"], p["v"], p["bro"], p["cofs"], p["ino"], p["table"],
                               p["lens"], p["cache"], p["page_size"], SCALE, mask, **kw)


def pin_p1_prefill():
    p = tiny_prefill()
    out = run_prefill(p)
    H = p["q"].shape[1]
    t = 0
    for b, n in enumerate(p["new"]):
        L = p["total"][b]
        k0 = int(p["bro"][b])
        for j in range(n):
            pos = L - n + j
            for h in range(H):
                keys, vals = [], []
                for i in range(L):
                    if i > pos:
                        continue
                    keys.append(list(p["k"][k0 + i, h]) + list(p["seq_cache"][b][i, 512:576]))
                    vals.append(list(p["v"][k0 + i, h]))
                o, _ = attention_row(list(p["q"][t, h]), keys, vals, SCALE)
                close(out[t, h], o, 1e-12)
            t += 1


# --------------------------------------------------------------------------------------
# P2, P14: layout invariances
# --------------------------------------------------------------------------------------

def pin_p2_page_permutation():
    c = tiny_decode(seed=6)
    out1, lse1 = run_dense(c)
    cache2, table2, _ = page_up(c["seq_keys"], c["page_size"], np.random.default_rng(99), spare=5)
    out2, lse2 = run_dense(c, table=table2, cache=cache2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def pin_p14_batch_permutation():
    c = tiny_decode(seed=7, lens=(5, 37, 20, 11), n_tokens=(1, 1, 1, 1))
    out, lse = run_dense(c)
    perm = [2, 0, 3, 1]
    keys2 = [c["seq_keys"][i] for i in perm]
    cache2, table2, lens2 = page_up(keys2, c["page_size"], np.random.default_rng(5))
    out2, lse2 = O.decode_paged_f64(c["q"][perm], c["off"], table2, lens2, cache2,
                                    c["page_size"], SCALE, "causal")
    assert np.array_equal(out2, out[perm]) and np.array_equal(lse2, lse[perm])


# --------------------------------------------------------------------------------------
# P3 - P7: closed forms
# --------------------------------------------------------------------------------------

def pin_p3_one_key():
    c = tiny_decode(seed=8, lens=(1, 1), n_tokens=(1, 1), page_size=16)
    out, lse = run_dense(c)
    for b in range(2):
        assert np.array_equal(out[b], np.broadcast_to(c["seq_keys"][b][0, :DV], out[b].shape))
        s = SCALE * (c["q"][b] @ c["seq_keys"][b][0])
        close(lse[b], s, 1e-12)


def pin_p4_normalisation():
    rng = np.random.default_rng(9)
    qh = rng.standard_normal((3, D))
    keys = rng.standard_normal((40, D))
    _, _, p = O.attend(qh, keys, O.value_columns(keys), SCALE, return_probs=True)
    close(p.sum(axis=1), np.ones(3), 1e-14)
    assert np.all(p >= 0)
    const = keys.copy()
    const[:, :DV] = 0.625
    out, _ = O.attend(qh, const, O.value_columns(const), SCALE)
    close(out, np.full((3, DV), 0.625), 1e-14)


def pin_p5_zero_scale_is_mean():
    c = tiny_decode(seed=10, lens=(5, 37, 20), n_tokens=(1, 3, 2))
    out, _ = run_dense(c, scale=0.0)
    t = 0
    for b, keys in enumerate(c["seq_keys"]):
        n = c["n_tokens"][b]
        for j in range(n):
            vis = keys[:len(keys) - n + j + 1, :DV]
            close(out[t], np.broadcast_to(vis.mean(axis=0), out[t].shape), 1e-13)
            t += 1
    c["q"] = np.zeros_like(c["q"])
    out0, _ = run_dense(c)
    close(out0[0], np.broadcast_to(c["seq_keys"][0][:, :DV].mean(axis=0), out0[0].shape), 1e-13)


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()[:2]
                vals[k] = v
    return vals


def pin_p6_two_keys():
    g = _golden("two_key_example.txt")
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    keys = np.zeros((2, D))
    keys[0, 0], keys[1, 0] = 2.0, 1.0
    vals = np.zeros((2, DV))
    vals[0, 0], vals[1, 1] = 1.0, 1.0
    out, lse = O.attend(q, keys, vals, 1.0)
    close(out[0, 0], float(g["p0"]), 1e-15)
    close(out[0, 1], float(g["p1"]), 1e-15)
    close(out[0, 2:], np.zeros(DV - 2), 0.0)
    close(lse[0], float(g["lse"]), 1e-15)
    # random two-key case against the logistic closed form
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, D))
    keys = rng.standard_normal((2, D))
    out, _ = O.attend(q, keys, O.value_columns(keys), SCALE)
    for h in range(2):
        s0 = SCALE * math.fsum(q[h] * keys[0])
        s1 = SCALE * math.fsum(q[h] * keys[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        close(out[h], w0 * keys[0, :DV] + (1.0 - w0) * keys[1, :DV], 1e-13)


def pin_p7_rope_shift():
    c = tiny_decode(seed=12, lens=(13, 21), n_tokens=(1, 2))
    j = 512 + 17
    for keys in c["seq_keys"]:
        keys[:, j] = 1.5
    cache, table, _ = page_up(c["seq_keys"], c["page_size"], np.random.default_rng(3))
    outs, lses = [], []
    for a in (0.0, 2.5):
        q = c["q"].copy()
        q[:, :, j] = a
        o, l = O.decode_paged_f64(q, c["off"], table, c["lens"], cache, c["page_size"], SCALE)
        outs.append(o)
        lses.append(l)
    close(outs[0], outs[1], 1e-12)
    close(lses[1] - lses[0], np.full(lses[0].shape, SCALE * 2.5 * 1.5), 1e-12)


# --------------------------------------------------------------------------------------
# P8: split-KV algebra
# --------------------------------------------------------------------------------------

def pin_p8_split_combine():
    rng = np.random.default_rng(13)
    qh = rng.standard_normal((4, D))
    keys = rng.standard_normal((70, D))
    full_o, full_l = O.attend(qh, keys, O.value_columns(keys), SCALE)
    for cuts in ([0, 70], [0, 1, 70], [0, 23, 23, 50, 70], [0, 5, 9, 64, 69, 70]):
        parts = [O.attend(qh, keys[a:b], O.value_columns(keys[a:b]), SCALE)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        o, l = O.combine(parts)
        close(o, full_o, 1e-12)
        close(l, full_l, 1e-12)
    o, l = O.combine([O.attend(qh, keys[:0], O.value_columns(keys[:0]), SCALE)] * 2)
    close(o, np.zeros_like(full_o), 0.0)
    assert np.all(np.isneginf(l))


# --------------------------------------------------------------------------------------
# P9: absorbed decode equals un-absorbed prefill
# --------------------------------------------------------------------------------------

def pin_p9_absorption():
    """Projecting q's no-rope part through w_uk and the latent output through w_uv turns
    MLA decode over the latent cache into ordinary attention with per-head k = w_uk^T c
    and v = w_uv c (mla_decode_branch_fp8 summary and Args w_uk / w_uv)."""
    rng = np.random.default_rng(14)
    H, N = 3, 11
    latent = rng.standard_normal((N, 512))
    rope = rng.standard_normal((N, 64))
    w_uk = rng.standard_normal((H, 512, 128)) / math.sqrt(512)
    w_uv = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    q_nope = rng.standard_normal((H, 128))
    q_rope = rng.standard_normal((H, 64))
    rows = np.concatenate([latent, rope], axis=1)
    cache, table, lens = page_up([rows], 4, rng)
    q_abs = np.concatenate([np.einsum("hln,hn->hl", w_uk, q_nope), q_rope], axis=1)[None]
    raw, _ = O.decode_paged_f64(q_abs, offsets_of([1]), table, lens, cache, 4, SCALE, "causal")
    dec = np.einsum("hvl,hl->hv", w_uv, raw[0])
    k = np.einsum("hln,il->ihn", w_uk, latent)
    v = np.einsum("hvl,il->ihv", w_uv, latent)
    q_pre = np.concatenate([q_nope, q_rope], axis=1)[None]
    pre = O.prefill_paged_f64(q_pre, k, v, offsets_of([N]), np.zeros(1, np.uint32), offsets_of([1]),
                              table, lens, cache, 4, SCALE, "causal")
    close(pre[0], dec, 1e-10)


# --------------------------------------------------------------------------------------
# P10: masks
# --------------------------------------------------------------------------------------

def pin_p10_masks():
    c = tiny_decode(seed=15, lens=(5, 37, 20), n_tokens=(1, 1, 1))
    oc, lc = run_dense(c, "causal")
    on, ln = run_dense(c, "null")
    assert np.array_equal(oc, on) and np.array_equal(lc, ln)
    p = tiny_prefill(seed=16, new=(4, 3), prefix=(0, 2))
    out = run_prefill(p, "causal")
    assert np.array_equal(out[0], p["v"][0])                 # first query of a fresh sequence
    out_null = run_prefill(p, "null")
    last = [int(p["ino"][b + 1]) - 1 for b in range(2)]
    close(out[last], out_null[last], 1e-14)


# --------------------------------------------------------------------------------------
# P11, P12: sparse semantics
# --------------------------------------------------------------------------------------

def pin_p11_sparse_is_dense():
    c = tiny_decode(seed=17, lens=(37, 20), n_tokens=(1, 1), page_size=8)
    ps = c["page_size"]
    stride = 40
    idx = np.full((2, stride), -1, dtype=np.int32)
    topk = np.zeros(2, dtype=np.int32)
    for b in range(2):
        L = int(c["lens"][b])
        pos = np.arange(L)
        idx[b, :L] = c["table"][b, pos // ps] * ps + pos % ps
        topk[b] = L
    so, sl = O.decode_sparse_f64(c["q"], c["off"], c["cache"], idx, topk, ps, SCALE)
    do, dl = run_dense(c, "null")
    assert np.array_equal(so, do) and np.array_equal(sl, dl)
    # a subset equals dense attention over a cache holding only those rows, listed order
    rng = np.random.default_rng(18)
    sub = [rng.choice(int(c["lens"][b]), size=7, replace=False) for b in range(2)]
    idx2 = np.full((2, 9), -1, dtype=np.int32)
    for b in range(2):
        idx2[b, :7] = c["table"][b, sub[b] // ps] * ps + sub[b] % ps
    so2, _ = O.decode_sparse_f64(c["q"], c["off"], c["cache"], idx2, np.array([7, 7]), ps, SCALE)
    packed = [c["seq_keys"][b][sub[b]] for b in range(2)]
    cache3, table3, lens3 = page_up(packed, 4, rng)
    do2, _ = O.decode_paged_f64(c["q"], c["off"], table3, lens3, cache3, 4, SCALE, "null")
    close(so2, do2, 1e-13)


def pin_p12_sparse_poison():
    s = tiny_sparse(seed=19)
    args = (s["off"],)
    out, lse = O.decode_sparse(s["q8"], s["q_scale"], s["off"], s["cache8"], s["c_scale"],
                               s["idx"], s["topk"], s["page_size"], SCALE)
    assert np.all(np.isfinite(out))
    ps = s["page_size"]
    listed = np.zeros(s["cache8"].shape[0] * ps, dtype=bool)
    for t in range(len(s["topk"])):
        r = s["idx"][t, :s["topk"][t]]
        listed[r[r >= 0]] = True
    c8 = s["cache8"].copy().reshape(-1, D)
    cs = s["c_scale"].copy().reshape(-1)
    c8[~listed] = 0x7F
    cs[~listed] = np.nan
    out2, lse2 = O.decode_sparse(s["q8"], s["q_scale"], *args, c8.reshape(s["cache8"].shape),
                                 cs.reshape(s["c_scale"].shape), s["idx"], s["topk"], ps, SCALE)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    idx3 = s["idx"].copy()
    for t in range(len(s["topk"])):
        idx3[t, s["topk"][t]:] = np.flatnonzero(~listed)[:idx3.shape[1] - s["topk"][t]]
    out3, _ = O.decode_sparse(s["q8"], s["q_scale"], *args, s["cache8"], s["c_scale"], idx3,
                              s["topk"], ps, SCALE)
    assert np.array_equal(out, out3)


# --------------------------------------------------------------------------------------
# P13: storage formats
# --------------------------------------------------------------------------------------

def pin_p13_e4m3():
    import torch
    g = _golden("e4m3_ocp_points.txt")
    for code, val in g.items():
        got = O.e4m3_to_f64(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])


def pin_p13_bf16():
    import torch
    g = _golden("bf16_points.txt")
    for bits, val in g.items():
        got = O.bf16_to_f64(np.array([int(bits, 16)], dtype=np.uint16))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val), (bits, got, val)
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = O.bf16_to_f64(allbits)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])


# --------------------------------------------------------------------------------------
# numerics: large logits stay finite and exact
# --------------------------------------------------------------------------------------

def pin_large_logits():
    c = tiny_decode(seed=20, lens=(9, 14), n_tokens=(1, 1), q_std=400.0)
    out, lse = run_dense(c)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert np.max(lse) > 800.0  # exp of such logits overflows float64
    bo, bl = decode_contiguous(c["q"].tolist(), [k.tolist() for k in c["seq_keys"]],
                               c["n_tokens"], SCALE, "causal")
    close(out, bo, 1e-11)
    close(lse, bl, 1e-11)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
