"""The benchmark's accounting, on the CPU: the algorithmic bytes it divides by kernel time, counted
row by row from the oracle's plans, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
from sparse_attention_kv_plan_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _row_seq_lens(w):
    cap_c, cap_w = oracle.capacities(w.cr, w.B, w.num_q)
    pc, _, counts = oracle.plan_prefill(w.cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                        w.num_q, cap_c, cap_w)
    return pc[: counts[0]].view("<u4").reshape(-1, 4)[:, 0].astype(np.int64)


def _window_bytes_by_hand(cr, hd, esize, seqs):
    """Each row: the kv and score halves of every window entry that takes part (a first ratio-4
    block has no previous block), the fp32 output row, the record; the ape table once."""
    W = 8 if cr == 4 else 128
    total = W * hd * esize
    for s in seqs:
        entries = 4 if (cr == 4 and s == 4) else W
        total += entries * (hd * esize + hd * esize) + hd * 4 + 16
    return total


def test_pool_bytes_of_the_mixed_prefill():
    for cr, rows, expect in [(4, 31448, 580160896), (128, 973, 257205456)]:
        w = wl.mixed_prefill(cr, with_tensors=False)
        seqs = _row_seq_lens(w)
        assert len(seqs) == rows and not np.any(seqs == 4)  # no first block in this batch
        got = bench.algorithmic_bytes_compress(cr, 512, 2, seqs)
        assert got == _window_bytes_by_hand(cr, 512, 2, seqs) == expect


def test_pool_bytes_count_a_first_block_as_four_entries():
    w = wl.c4_prefill_1x64(with_tensors=False)  # prefix 0: the first row closes the first block
    seqs = _row_seq_lens(w)
    assert len(seqs) == 16 and seqs[0] == 4 and np.all(seqs[1:] > 4)
    got = bench.algorithmic_bytes_compress(4, 128, 4, seqs)
    assert got == _window_bytes_by_hand(4, 128, 4, seqs)
    assert got == 15 * (8 * 2 * 128 * 4 + 512 + 16) + (4 * 2 * 128 * 4 + 512 + 16) + 8 * 128 * 4


def test_decode_bytes_by_hand():
    for w in (wl.c4_decode_b256(with_tensors=False), wl.c128_decode_b1024(with_tensors=False)):
        R = (4 if w.cr == 4 else 2) * w.hd
        W = 8 if w.cr == 4 else 128
        total = W * w.hd * 2
        for s in w.seq_lens:
            total += 2 * R * 2 + w.hd * 4 + 16  # the new row read and stored, the output row, the record
            if s % w.cr == 0:  # the window's entries other than the new token, from the state
                total += (3 if (w.cr == 4 and s == 4) else W - 1) * 2 * w.hd * 2
        assert bench.algorithmic_bytes_decode(w.cr, w.hd, 2, w.seq_lens) == total


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, timeout=300)
    assert r.returncode == 2 and r.stdout == b""
    assert b"one GPU" in r.stderr


def test_cpu_baseline_slices_cover_the_work_once():
    """The all-cores oracle leg hands each thread a slice of records or requests: the slices are
    disjoint, in order, and cover the whole range (an empty range gives no slice)."""
    for n in (0, 1, 7, 16, 31448):
        for parts in (1, 3, 8, 16, 64):
            sl = bench._slices(n, parts)
            assert len(sl) <= max(1, parts)
            covered = [k for a, b in sl for k in range(a, b)] if n < 100 else None
            if covered is not None:
                assert covered == list(range(n))
            assert all(b > a for a, b in sl) and (not sl or (sl[0][0] == 0 and sl[-1][1] == n))
            assert all(sl[i][1] == sl[i + 1][0] for i in range(len(sl) - 1))
