"""Drive a sequence of prefill chunks and decode steps through a back end.

A back end is any object with the five calls (plan_prefill, compress, write,
plan_decode, decode) in the oracle's numpy calling convention; the CPU
oracle is one, the HIP library (wrapped for numpy) is the other.  The driver
records every emitted compressed row as {(request, seq_len): row} so that a
test can compare it with the brute-force window over the whole sequence.
"""
from __future__ import annotations

import numpy as np

WINDOW = {4: 8, 128: 128}


def nan_state(num_rows, R, dtype):
    if dtype == "bf16":
        return np.full((num_rows, R), 0x7FC0, np.uint16)
    return np.full((num_rows, R), np.nan, np.float32)


def run_chunked(backend, cr, hd, dtype, seqs, chunks, decode_steps, state_index, num_slots, ape, state=None,
                swa=None, start=None):
    """seqs[b]: the request's whole input sequence [L_b, R]; chunks[b]: list of extend lengths
    (prefill rounds, request b takes part in round r if it has an r-th chunk); then
    ``decode_steps`` single-token steps for every request.  Returns (emitted, state).

    With ``swa`` = dict(req_to_token, full_to_swa, swa_page_size, ring_size, num_state_rows) the
    plans come from the SWA-paged planners and state_index holds the request pool indices.
    ``start[b]`` (default 0) is a prefix of request b already held in the state (prefix reuse)."""
    B = len(seqs)
    R = seqs[0].shape[1]
    W = WINDOW[cr]
    if state is None:
        rows = swa["num_state_rows"] if swa else num_slots * W
        state = nan_state(rows, R, dtype)
    length = list(start) if start is not None else [0] * B
    emitted = {}
    rounds = max(len(c) for c in chunks)
    for r in range(rounds):
        active = [b for b in range(B) if r < len(chunks[b])]
        if not active:
            continue
        e = np.array([chunks[b][r] for b in active], np.int32)
        s = np.array([length[b] + chunks[b][r] for b in active], np.int32)
        idx = np.array([state_index[b] for b in active], np.int32)
        inp = np.concatenate([seqs[b][length[b]:length[b] + chunks[b][r]] for b in active])
        num_q = int(e.sum())
        cap_c = min(num_q, num_q // cr + len(active))
        if swa:
            cap_w = min(num_q, len(active) * (W - 1) + (4 * (num_q // swa["swa_page_size"] + len(active))
                                                        if cr == 4 else 0))
            pc, pw, counts, st = backend.plan_prefill_swa(cr, s, e, idx, swa["req_to_token"], swa["full_to_swa"],
                                                          swa["swa_page_size"], swa["ring_size"], state.shape[0],
                                                          num_q, cap_c, cap_w)
            assert st == 0, st
        else:
            cap_w = min(num_q, len(active) * (W - 1))
            pc, pw, counts = backend.plan_prefill(cr, s, e, idx, state.shape[0], num_q, cap_c, cap_w)
        assert counts[2] == 0, counts
        out, err = backend.compress(cr, hd, state, inp, ape, pc, int(counts[0]))
        assert err == 0
        state = backend.write(cr, hd, state, inp, pw, int(counts[1]))
        # map each record back to its request through the ragged offsets
        base = np.concatenate([[0], np.cumsum(e)])
        recs = np.ascontiguousarray(pc[: counts[0]]).view("<u4").reshape(-1, 4)
        for k in range(int(counts[0])):
            seq_len = int(recs[k, 0])
            ragged = int(recs[k, 1]) & 0xFFFFFF
            a = int(np.searchsorted(base, ragged, side="right") - 1)
            key = (active[a], seq_len)
            assert key not in emitted, key
            emitted[key] = out[k].copy()
        for b in active:
            length[b] += chunks[b][r]
    for _ in range(decode_steps):
        s = np.array([length[b] + 1 for b in range(B)], np.int32)
        idx = np.asarray(state_index, np.int32)
        inp = np.stack([seqs[b][length[b]] for b in range(B)])
        if swa:
            pd, status = backend.plan_decode_swa(cr, s, idx, swa["req_to_token"], swa["full_to_swa"],
                                                 swa["swa_page_size"], swa["ring_size"], state.shape[0])
        else:
            pd, status = backend.plan_decode(cr, s, idx, state.shape[0])
        assert status == 0
        out, state, err = backend.decode(cr, hd, state, inp, ape, pd)
        assert err == 0
        for b in range(B):
            if s[b] % cr == 0:
                key = (b, int(s[b]))
                assert key not in emitted, key
                emitted[key] = out[b].copy()
            else:
                assert np.all(out[b] == 0), "non-boundary decode row must be zero"
            length[b] += 1
    return emitted, state


class Pages:
    """A caller's page table: one 4-row page per (request, block), allocated on first use."""

    def __init__(self, rng, n):
        self.free = list(rng.permutation(n))
        self.table = {}

    def __call__(self, b, block, allocate=True):
        if block < 0:
            return -1
        key = (b, block)
        if key not in self.table:
            if not allocate:
                return -1
            self.table[key] = int(self.free.pop())
        return self.table[key]


def _chunk_pages(pages, b, s, e):
    p0 = s - e
    last = (s // 4) * 4
    lsp = pages(b, (p0 - 1) // 4) if p0 > 0 else -1
    lfp = pages(b, (p0 - 1) // 4 - 1) if p0 > 4 else -1
    wfp = pages(b, last // 4 - 1)
    idx = pages(b, last // 4)
    return idx, (lfp, lsp, wfp, last)


def run_chunked_page4(backend, rng, hd, dtype, seqs, chunks, decode_steps, ape, n_pages):
    """Ratio 4 over caller-allocated pages: every block of every request gets a page of its own
    (from a shuffled pool of n_pages); chunks and decode steps as in run_chunked.
    Returns (emitted, state)."""
    B = len(seqs)
    R = 4 * hd
    state = nan_state(n_pages * 4, R, dtype)
    pages = Pages(rng, n_pages)
    length = [0] * B
    emitted = {}
    for r in range(max(len(c) for c in chunks)):
        active = [b for b in range(B) if r < len(chunks[b])]
        e = np.array([chunks[b][r] for b in active], np.int32)
        s = np.array([length[b] + chunks[b][r] for b in active], np.int32)
        idx, bundle = zip(*[_chunk_pages(pages, b, int(sb), int(eb)) for b, sb, eb in zip(active, s, e)])
        inp = np.concatenate([seqs[b][length[b]:length[b] + chunks[b][r]] for b in active])
        num_q = int(e.sum())
        cap_c = min(num_q, num_q // 4 + len(active))
        cap_w = min(num_q, len(active) * 7)
        pc, pw, counts, status = backend.plan_prefill_page4(s, e, idx, bundle, state.shape[0], num_q, cap_c, cap_w)
        assert counts[2] == 0 and status == 0, (counts, status)
        out, err = backend.compress(4, hd, state, inp, ape, pc, int(counts[0]))
        assert err == 0
        state = backend.write(4, hd, state, inp, pw, int(counts[1]))
        base = np.concatenate([[0], np.cumsum(e)])
        recs = np.ascontiguousarray(pc[: counts[0]]).view("<u4").reshape(-1, 4)
        for k in range(int(counts[0])):
            a_ = int(np.searchsorted(base, int(recs[k, 1]) & 0xFFFFFF, side="right") - 1)
            emitted[(active[a_], int(recs[k, 0]))] = out[k].copy()
        for b in active:
            length[b] += chunks[b][r]
    for _ in range(decode_steps):
        s = np.array([length[b] + 1 for b in range(B)], np.int32)
        idx = [pages(b, (int(s[b]) - 1) // 4) for b in range(B)]
        prev = [pages(b, (int(s[b]) - 1) // 4 - 1) for b in range(B)]
        pd, status = backend.plan_decode_page4(s, idx, prev, state.shape[0])
        assert status == 0
        inp = np.stack([seqs[b][length[b]] for b in range(B)])
        out, state, err = backend.decode(4, hd, state, inp, ape, pd)
        assert err == 0
        for b in range(B):
            if s[b] % 4 == 0:
                emitted[(b, int(s[b]))] = out[b].copy()
            length[b] += 1
    return emitted, state


class OracleBackend:
    """The CPU oracle in the driver's calling convention."""

    def __init__(self, oracle):
        self.o = oracle

    def plan_prefill(self, cr, s, e, idx, rows, num_q, cap_c, cap_w):
        return self.o.plan_prefill(cr, s, e, idx, rows, num_q, cap_c, cap_w)

    def compress(self, cr, hd, state, inp, ape, pc, num_c):
        return self.o.compress(cr, hd, state, inp, ape, pc, num_c)

    def write(self, cr, hd, state, inp, pw, num_w):
        state = state.copy()
        assert self.o.write(cr, hd, state, inp, pw, num_w) == 0
        return state

    def plan_decode(self, cr, s, idx, rows):
        return self.o.plan_decode(cr, s, idx, rows)

    def plan_prefill_swa(self, *a):
        return self.o.plan_prefill_swa(*a)

    def plan_decode_swa(self, *a):
        return self.o.plan_decode_swa(*a)

    def plan_prefill_page4(self, *a):
        return self.o.plan_prefill_page4(*a)

    def plan_decode_page4(self, *a):
        return self.o.plan_decode_page4(*a)

    def decode(self, cr, hd, state, inp, ape, pd):
        state = state.copy()
        out, err = self.o.decode(cr, hd, state, inp, ape, pd)
        return out, state, err


class OnlineBackend:
    """The online ratio-128 state behind the same calls: plans are the ordinary ratio-128 plans
    over 128 virtual rows per slot; ``state`` is [slots, 3, hd] (m, l, acc).  ``inner`` provides
    plan_prefill / plan_decode and compress_online / write_online / decode_online; the fold of the
    tail tokens needs ``ape``, which the state-buffer write does not take."""

    def __init__(self, inner, ape):
        self.inner = inner
        self.ape = ape

    def plan_prefill(self, cr, s, e, idx, rows, num_q, cap_c, cap_w):
        return self.inner.plan_prefill(cr, s, e, idx, rows * 128, num_q, cap_c, cap_w)

    def plan_decode(self, cr, s, idx, rows):
        return self.inner.plan_decode(cr, s, idx, rows * 128)

    def compress(self, cr, hd, state, inp, ape, pc, num_c):
        return self.inner.compress_online(hd, state, inp, ape, pc, num_c)

    def write(self, cr, hd, state, inp, pw, num_w):
        st, err = self.inner.write_online(hd, state, inp, self.ape, pw, num_w)
        assert err == 0
        return st

    def decode(self, cr, hd, state, inp, ape, pd):
        return self.inner.decode_online(hd, state, inp, ape, pd)


class OracleOnline:
    """The oracle's online functions in OnlineBackend's ``inner`` convention."""

    def __init__(self, oracle):
        self.o = oracle

    def plan_prefill(self, *a):
        return self.o.plan_prefill(*a)

    def plan_decode(self, *a):
        return self.o.plan_decode(*a)

    def compress_online(self, hd, state, inp, ape, pc, num_c):
        return self.o.compress_online(hd, state, inp, ape, pc, num_c)

    def write_online(self, hd, state, inp, ape, pw, num_w):
        return self.o.write_online(hd, state, inp, ape, pw, num_w)

    def decode_online(self, hd, state, inp, ape, pd):
        return self.o.decode_online(hd, state, inp, ape, pd)


def as_float(a, dtype):
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


def random_split(rng, L, max_chunks, min_len=1):
    """Split L tokens into at most max_chunks positive pieces."""
    n = int(rng.integers(1, max_chunks, endpoint=True))
    n = min(n, L)
    if n == 1:
        return [L]
    cuts = np.sort(rng.choice(np.arange(1, L), size=n - 1, replace=False))
    pieces = np.diff(np.concatenate([[0], cuts, [L]]))
    return [int(x) for x in pieces]
