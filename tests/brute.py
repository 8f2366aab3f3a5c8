"""Brute-force attention in plain Python scalar loops, for tiny inputs.

Independent of the oracle: contiguous (unpaged) keys and values given as Python lists,
its own masking loop, math.fsum for every sum, and exp with the row maximum subtracted
(the same real number as exp(s)/sum exp(s), written so large logits stay finite).
"""
import math


def attention_row(q_vec, keys, vals, scale, sink=None, dv=None):
    """One head: q_vec [D], keys [N][D], vals [N][Dv] -> (out [Dv], lse).

    sink: an optional extra logit that adds e^sink to the denominator (and to the
    log-sum-exp) and nothing to the numerator.  dv: the value width when keys is empty."""
    dv = len(vals[0]) if vals else (dv or 0)
    logits = [scale * math.fsum(a * b for a, b in zip(q_vec, k)) for k in keys]
    terms = logits + ([sink] if sink is not None else [])
    if not terms or max(terms) == -math.inf:
        return [0.0] * dv, -math.inf
    top = max(terms)
    w = [math.exp(x - top) for x in logits]
    tot = math.fsum(w + ([math.exp(sink - top)] if sink is not None else []))
    out = [math.fsum(w[r] * vals[r][c] for r in range(len(keys))) / tot for c in range(dv)]
    return out, top + math.log(tot)


def decode_contiguous(q_rows, seq_keys, n_tokens, scale, mask, window=-1, value_width=512):
    """q_rows[t][h][d]; seq_keys[b] = contiguous list of that sequence's cache rows.

    Query token j of the n tokens of sequence b sits at position len(keys) - n + j.
    Returns out[t][h][c] and lse[t][h].
    """
    out, lse = [], []
    t = 0
    for b, keys in enumerate(seq_keys):
        L = len(keys)
        for j in range(n_tokens[b]):
            pos = L - n_tokens[b] + j
            vis = []
            for r in range(L):
                if mask == "causal" and r > pos:
                    continue
                if mask == "sliding_window_causal" and (r > pos or r <= pos - window):
                    continue
                vis.append(r)
            ks = [keys[r] for r in vis]
            vs = [keys[r][:value_width] for r in vis]
            o_t, l_t = [], []
            for h in range(len(q_rows[t])):
                o, l = attention_row(q_rows[t][h], ks, vs, scale)
                o_t.append(o)
                l_t.append(l)
            out.append(o_t)
            lse.append(l_t)
            t += 1
    return out, lse
