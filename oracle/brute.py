"""Brute-force window definition of a compressed row -- TEST INFRASTRUCTURE.

Pure Python, float64, tiny sizes only.  It knows nothing of plans, state
buffers, chunks or ragged batches: given a request's whole token sequence it
pools the row that closes at length ``s`` straight from the positions the
window covers.  It is the definition the chunked oracle is checked against.

Definition (c4.cuh page, c4_forward; compressor_v2.py page,
_compress_forward_c128_fallback):
  * ratio 4: the window holds the 8 positions s-8 .. s-1.  The first four
    (the previous block) contribute the kv-overlap and score-overlap quarters
    of their row, the last four the kv and score quarters.  Positions before
    the start of the sequence (only when s == 4) are left out.
  * ratio 128: the window holds the 128 positions s-128 .. s-1, each giving
    the kv and score halves of its row.
  * each channel d: t_i = score_i[d] + ape[i][d];
    out[d] = sum_i exp(t_i) kv_i[d] / sum_i exp(t_i)  (shifted by max t_i).
"""
from __future__ import annotations

import math


def window_entries(cr, hd, s):
    """List of (position, kv column offset, score column offset, ape row) for the row closing at s."""
    if cr == 4:
        ents = []
        for i in range(8):
            pos = s - 8 + i
            if pos < 0:
                continue
            if i < 4:
                ents.append((pos, 0, 2 * hd, i))
            else:
                ents.append((pos, hd, 3 * hd, i))
        return ents
    if cr == 128:
        return [(s - 128 + i, 0, hd, i) for i in range(128)]
    raise ValueError(cr)


def pooled_row(cr, hd, seq, ape, s):
    """Pool the compressed row that closes at length s (s % cr == 0, s >= cr).

    seq[pos][col] is the request's full kv/score sequence as floats,
    ape[i][d] the score bias."""
    assert s % cr == 0 and s >= cr
    ents = window_entries(cr, hd, s)
    out = []
    for d in range(hd):
        t = [seq[p][sc + d] + ape[i][d] for (p, _, sc, i) in ents]
        v = [seq[p][kc + d] for (p, kc, _, _) in ents]
        m = max(t)
        w = [math.exp(x - m) for x in t]
        out.append(sum(wi * vi for wi, vi in zip(w, v)) / sum(w))
    return out
