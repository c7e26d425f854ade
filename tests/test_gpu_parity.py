"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Bars: plans, counts, padding and state buffers bit-exact; pooled rows within
|err| <= 1e-5 + 1e-5 |ref| for fp32 inputs (float64 arithmetic on the GPU)
and <= 2e-2 for bf16 inputs (fp32 arithmetic on the GPU); float64 in the
oracle.  Output rows past
num_c must stay untouched (checked against a NaN fill, bitwise).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import kvc  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402
from tests.chunked import OracleBackend, as_float, nan_state, random_split, run_chunked  # noqa: E402

pytestmark = pytest.mark.gpu

W = {4: 8, 128: 128}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_backend import GpuBackend
    return GpuBackend()


def assert_pool_close(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    tol = (1e-5 + 1e-5 * np.abs(ref)) if dtype == "f32" else np.full_like(ref, 2e-2)
    bad = err > tol
    assert not bad.any(), "%s: %d elements out of tolerance, max err %.3g" % (what, bad.sum(), err.max())


def _plans_equal(g, o):
    gpc, gpw, gcounts = g
    opc, opw, ocounts = o
    assert gcounts.tolist() == ocounts.tolist()
    assert np.array_equal(gpc, opc), "C records differ"
    assert np.array_equal(gpw, opw), "W records differ"


# --------------------------------------------------------------------------
# planners
# --------------------------------------------------------------------------

def _random_plan_case(rng, cr):
    B = int(np.exp(rng.uniform(0, np.log(1024.5))))
    B = max(1, min(1024, B))
    kind = rng.integers(0, 3)
    prefix = rng.integers(0, 5000, size=B)
    if kind == 0:      # general ragged batch
        e = rng.integers(1, 600, size=B)
    elif kind == 1:    # uniform extends (multi-token prediction shape)
        e = np.full(B, int(rng.integers(1, 33)))
    else:              # uniform but long: takes the general path
        e = np.full(B, int(rng.integers(33, 300)))
    idx = rng.permutation(1024)[:B]
    return B, prefix + e, e, idx


@pytest.mark.parametrize("cr", [4, 128])
def test_plan_prefill_fuzz(gpu, cr):
    rng = np.random.default_rng(11 + cr)
    for case in range(60):
        B, s, e, idx = _random_plan_case(rng, cr)
        num_q = int(e.sum())
        cap_c, cap_w = oracle.capacities(cr, B, num_q)
        cap_c += int(rng.integers(0, 5))
        cap_w += int(rng.integers(0, 5))
        say("plan_prefill cr=%d case=%d B=%d num_q=%d" % (cr, case, B, num_q))
        g = gpu.plan_prefill(cr, s, e, idx, 1024 * W[cr], num_q, cap_c, cap_w)
        o = oracle.plan_prefill(cr, s, e, idx, 1024 * W[cr], num_q, cap_c, cap_w)
        _plans_equal(g, o)


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 31, 32, 33])
@pytest.mark.parametrize("cr", [4, 128])
def test_plan_prefill_uniform_extend(gpu, cr, E):
    s, e, idx = wl.mixed_prefill_lens(uniform_extend=E)
    num_q = int(e.sum())
    cap_c, cap_w = oracle.capacities(cr, 64, num_q)
    say("plan_prefill uniform cr=%d E=%d" % (cr, E))
    _plans_equal(gpu.plan_prefill(cr, s, e, idx, 64 * W[cr], num_q, cap_c, cap_w),
                 oracle.plan_prefill(cr, s, e, idx, 64 * W[cr], num_q, cap_c, cap_w))


def test_plan_prefill_errors(gpu):
    cases = [
        (4, [3, 8], [4, 4], [0, 1], 16, 8, 6, 8),      # extend > seq_len
        (4, [8, 8], [0, 8], [0, 1], 16, 8, 6, 8),      # extend == 0
        (4, [8, 8], [4, 4], [0, 1], 16, 9, 6, 8),      # sum != num_q
        (4, [8, 8], [4, 4], [0, 2], 16, 8, 6, 8),      # index out of range
        (4, [8, 8], [4, 4], [-1, 0], 16, 8, 6, 8),     # negative index
        (4, [64], [64], [0], 8, 64, 15, 8),            # C capacity
        (4, [64], [64], [0], 8, 64, 16, 6),            # W capacity
        (128, [300, 130], [300, 5], [1, 0], 256, 305, 2, 46),   # C capacity, ratio 128
        (128, [300, 130], [300, 5], [1, 0], 256, 305, 3, 45),   # W capacity, ratio 128
        (128, [300, 130], [300, 5], [1, 0], 256, 305, 0, 0),    # zero capacities
        (128, [300, 130], [300, 5], [1, 0], 256, 305, 3, 46),   # exactly enough
        (4, [2 ** 31 - 1], [5], [0], 8, 5, 5, 5),       # very long sequence
        (4, [8, 8, 8], [4, 4, 4], [2, 0, 2], 24, 12, 9, 12),   # two requests on one ring
        (128, [130, 5], [2, 5], [1, 1], 256, 7, 4, 7),          # two requests on one page
        (4, [8, 8], [4, 4], [2, 2], 16, 8, 6, 8),               # repeated index out of range: index error only
        (4, [6, 6, 6], [2, 2, 2], [1, 0, 1], 24, 6, 6, 6),      # duplicate on the uniform-extend path
    ]
    for c in cases:
        say("plan_prefill errors", c)
        _plans_equal(gpu.plan_prefill(*c), oracle.plan_prefill(*c))


@pytest.mark.parametrize("cr", [4, 128])
def test_plan_prefill_duplicate_slots(gpu, cr):
    """Batches of up to 1024 requests in which one or several state slots are repeated anywhere in
    the batch (or not at all): the planner flags exactly the batches the oracle flags, with the
    same counts and all-invalid records; the uniform-extend path included."""
    rng = np.random.default_rng(900 + cr)
    for case in range(24):
        B = int(rng.choice([2, 3, 64, 1000, 1024]))
        e = np.full(B, 2) if case % 3 == 0 else rng.integers(1, 40, size=B)
        s = (rng.integers(0, 400, size=B) + e).astype(np.int32)
        e = e.astype(np.int32)
        slots = B + 8
        idx = rng.permutation(slots)[:B].astype(np.int32)
        kind = case % 4
        if kind == 1:    # one repeat, at two random places
            i, j = rng.choice(B, size=2, replace=False)
            idx[j] = idx[i]
        elif kind == 2:  # many repeats
            k = max(1, B // 10)
            idx[rng.choice(B, size=k, replace=False)] = idx[rng.choice(B, size=k)]
        elif kind == 3:  # first and last
            idx[-1] = idx[0]
        num_q = int(e.sum())
        cap_c, cap_w = oracle.capacities(cr, B, num_q)
        args = (cr, s, e, idx, slots * W[cr], num_q, cap_c, cap_w)
        o = oracle.plan_prefill(*args)
        assert bool(o[2][2] & kvc.DERR_DUPLICATE) == (len(set(idx.tolist())) < B)
        _plans_equal(gpu.plan_prefill(*args), o)


@pytest.mark.parametrize("cr", [4, 128])
def test_plan_prefill_golden(gpu, cr):
    import json
    import os
    name = "plan_c4_prefill_two_requests.json" if cr == 4 else "plan_c128_prefill_two_requests.json"
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", name)))
    pc, pw, counts = gpu.plan_prefill(cr, g["seq_lens"], g["extend_lens"], g["state_index"], 4 * W[cr],
                                      g["num_q"], 16, 256)
    assert oracle.unpack_c(pc[: counts[0]]).tolist() == g["plan_c"]
    assert counts[2] == 0


def test_plan_decode(gpu):
    rng = np.random.default_rng(3)
    for cr in (4, 128):
        for B in (1, 7, 256, 1024, 1025, 4096, 65536):
            s = rng.integers(1, 1 << 20, size=B)
            idx = rng.permutation(max(B, 70000))[:B]
            rows = max(B, 70000) * W[cr]
            say("plan_decode cr=%d B=%d" % (cr, B))
            g = gpu.plan_decode(cr, s, idx, rows)
            o = oracle.plan_decode(cr, s, idx, rows)
            assert g[1] == o[1] == 0 and np.array_equal(g[0], o[0])
        # bad requests are invalid one by one
        s = np.array([5, 0, 9, -3, 12], np.int32)
        idx = np.array([0, 1, 2, 3, 9], np.int32)
        g = gpu.plan_decode(cr, s, idx, 5 * W[cr])
        o = oracle.plan_decode(cr, s, idx, 5 * W[cr])
        assert g[1] == o[1] == (kvc.DERR_EXTEND | kvc.DERR_INDEX) and np.array_equal(g[0], o[0])


# --------------------------------------------------------------------------
# write / compress / decode on oracle-built plans
# --------------------------------------------------------------------------

SHAPES = [(4, 128, "f32"), (4, 512, "bf16"), (4, 256, "bf16"), (4, 128, "bf16"), (4, 512, "f32"), (4, 256, "f32"),
          (128, 512, "bf16"), (128, 128, "f32"), (128, 256, "f32"), (128, 128, "bf16"), (128, 512, "f32"),
          (128, 256, "bf16")]


@pytest.mark.parametrize("cr,hd,dtype", SHAPES)
def test_prefill_compress_and_write(gpu, cr, hd, dtype):
    rng = np.random.default_rng(hd + cr + (dtype == "bf16"))
    for trial in range(3):
        B = int(rng.integers(1, 9))
        w = wl.random_prefill(rng, cr, hd, dtype, B, prefix_hi=3 * W[cr], extend_lo=1,
                              extend_hi=3 * W[cr] if trial < 2 else 700, num_slots=B + 3)
        cap_c, cap_w = oracle.capacities(cr, B, w.num_q)
        pc, pw, counts = oracle.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                             w.num_q, cap_c + 2, cap_w + 2)
        say("compress cr=%d hd=%d %s trial=%d B=%d num_q=%d num_c=%d" % (cr, hd, dtype, trial, B, w.num_q,
                                                                         counts[0]))
        ref, err = oracle.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
        got, gerr = gpu.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
        assert err == gerr == 0
        n = int(counts[0])
        assert_pool_close(got[:n], ref[:n], dtype, "compress")
        assert np.all(np.isnan(got[n:])), "rows past num_c must be untouched"
        st_o = w.state.copy()
        assert oracle.write(cr, hd, st_o, w.input, pw, counts[1]) == 0
        st_g = gpu.write(cr, hd, w.state, w.input, pw, counts[1])
        assert np.array_equal(st_g.view(np.uint8), st_o.view(np.uint8)), "state differs after write"


@pytest.mark.parametrize("cr,hd,dtype", SHAPES)
def test_decode(gpu, cr, hd, dtype):
    rng = np.random.default_rng(7 * hd + cr)
    for trial in range(3):
        B = int(rng.integers(1, 300))
        w = wl.random_decode(rng, cr, hd, dtype, B, prefix_hi=3 * W[cr], num_slots=B + 2)
        if trial == 2:  # every request on a boundary, including the first block
            w.seq_lens = (rng.integers(1, 4, size=B) * cr).astype(np.int32)
        pd, status = oracle.plan_decode(cr, w.seq_lens, w.state_index, w.num_state_rows)
        say("decode cr=%d hd=%d %s trial=%d B=%d boundaries=%d" % (cr, hd, dtype, trial, B,
                                                                   int((w.seq_lens % cr == 0).sum())))
        st_o = w.state.copy()
        ref, err = oracle.decode(cr, hd, st_o, w.input, w.ape, pd)
        got, st_g, gerr = gpu.decode(cr, hd, w.state, w.input, w.ape, pd)
        assert err == gerr == 0
        assert_pool_close(got, ref, dtype, "decode")
        nb = w.seq_lens % cr != 0
        assert np.all(got[nb] == 0.0)
        assert np.array_equal(st_g.view(np.uint8), st_o.view(np.uint8)), "state differs after decode"


def _scale_scores(a, cr, hd, dtype, factor):
    """Multiply the score columns of input or state rows (|kv ov|kv|sc ov|sc| for ratio 4, |kv|sc| for
    ratio 128) by factor, staying in the storage dtype."""
    x = as_float(a, dtype).astype(np.float32)
    lo = 2 * hd if cr == 4 else hd
    x[:, lo:] *= np.float32(factor)
    return wl.to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("cr", [4, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_magnitude_scores(gpu, cr, dtype):
    """Scores of size ~1e30: exp of an unshifted score overflows, so the pool is finite only
    because the window maximum is subtracted first; the weights are then one-hot up to
    rounding, and the rows must still match the float64 oracle."""
    hd = 128
    rng = np.random.default_rng(40 + cr + (dtype == "bf16"))
    B = 6
    w = wl.random_prefill(rng, cr, hd, dtype, B, prefix_hi=3 * W[cr], extend_lo=1, extend_hi=3 * W[cr],
                          num_slots=B + 1)
    w.input = _scale_scores(w.input, cr, hd, dtype, 1e30)
    w.state = _scale_scores(w.state, cr, hd, dtype, 1e30)
    cap_c, cap_w = oracle.capacities(cr, B, w.num_q)
    pc, pw, counts = oracle.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                         w.num_q, cap_c, cap_w)
    say("large scores cr=%d %s num_c=%d" % (cr, dtype, counts[0]))
    ref, err = oracle.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
    got, gerr = gpu.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
    assert err == gerr == 0
    n = int(counts[0])
    assert n > 0
    assert_pool_close(got[:n], ref[:n], dtype, "compress, large scores")
    d = wl.random_decode(rng, cr, hd, dtype, 64, prefix_hi=3 * W[cr], num_slots=65)
    d.seq_lens = (rng.integers(1, 4, size=64) * cr).astype(np.int32)  # every request pools
    d.input = _scale_scores(d.input, cr, hd, dtype, 1e30)
    d.state = _scale_scores(d.state, cr, hd, dtype, 1e30)
    pd, status = oracle.plan_decode(cr, d.seq_lens, d.state_index, d.num_state_rows)
    ref, err = oracle.decode(cr, hd, d.state.copy(), d.input, d.ape, pd)
    got, _, gerr = gpu.decode(cr, hd, d.state, d.input, d.ape, pd)
    assert status == err == gerr == 0
    assert_pool_close(got, ref, dtype, "decode, large scores")


def _scale_all(a, dtype, factor):
    """Every column of input, state or ape rows times factor, in the storage dtype."""
    x = as_float(a, dtype).astype(np.float32) * np.float32(factor)
    return wl.to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("cr", [4, 128])
@pytest.mark.parametrize("scale", [3.0, 30.0, 1000.0])
def test_fp32_bar_at_large_input_scales(gpu, cr, scale):
    """fp32 inputs (kv, scores and ape) 3, 30 and 1000 times the configs' size, prefill and decode,
    at the fp32 bar 1e-5 + 1e-5 |ref|.  At these sizes two nearly equal leading weights on
    kv values of opposite sign leave |ref| small while the terms are large, so the bar asks for
    weights correct to a few parts in 1e8 of the kv spread: the pool's float64 arithmetic for
    fp32 inputs gives that for any finite input with |kv| up to 2^30."""
    rng = np.random.default_rng([77, cr, int(scale)])
    for hd in (128, 512):
        B = 8
        w = wl.random_prefill(rng, cr, hd, "f32", B, prefix_hi=3 * W[cr], extend_lo=1, extend_hi=3 * W[cr],
                              num_slots=B + 2)
        w.input, w.state, w.ape = (_scale_all(x, "f32", scale) for x in (w.input, w.state, w.ape))
        cap_c, cap_w = oracle.capacities(cr, B, w.num_q)
        pc, pw, counts = oracle.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                             w.num_q, cap_c, cap_w)
        say("fp32 x%g cr=%d hd=%d num_c=%d" % (scale, cr, hd, counts[0]))
        ref, err = oracle.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
        got, gerr = gpu.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
        n = int(counts[0])
        assert err == gerr == 0 and n > 0
        assert_pool_close(got[:n], ref[:n], "f32", "compress x%g" % scale)
        d = wl.random_decode(rng, cr, hd, "f32", 96, prefix_hi=3 * W[cr], num_slots=97)
        d.seq_lens = (rng.integers(1, 4, size=96) * cr).astype(np.int32)  # every request pools
        d.input, d.state, d.ape = (_scale_all(x, "f32", scale) for x in (d.input, d.state, d.ape))
        pd, status = oracle.plan_decode(cr, d.seq_lens, d.state_index, d.num_state_rows)
        ref, err = oracle.decode(cr, hd, d.state.copy(), d.input, d.ape, pd)
        got, _, gerr = gpu.decode(cr, hd, d.state, d.input, d.ape, pd)
        assert status == err == gerr == 0
        assert_pool_close(got, ref, "f32", "decode x%g" % scale)


@pytest.mark.parametrize("cr,s,e,expect", [
    (4, [2, 7], [2, 2], (0, 4)),   # no row closes: no C records, the tokens are written
    (128, [128], [128], (1, 0)),   # the chunk closes exactly one block: one row, nothing written
    (4, [1], [1], (0, 1)),         # a single token
])
def test_empty_record_sets(gpu, cr, s, e, expect):
    """Chunks whose C or W set is empty, planned with capacities equal to the counts (so zero-size
    plan buffers): the planner, the pool and the write match the oracle and touch nothing else."""
    hd, B, num_q = 128, len(s), int(sum(e))
    w = wl.prefill_workload("empty", cr, hd, "f32", s, e, list(range(B)), B, [77, cr])
    cap_c, cap_w = expect
    say("empty record sets cr=%d s=%s e=%s" % (cr, s, e))
    g = gpu.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows, num_q, cap_c, cap_w)
    o = oracle.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows, num_q, cap_c, cap_w)
    _plans_equal(g, o)
    pc, pw, counts = o
    assert tuple(counts[:2]) == expect and counts[2] == 0
    got, gerr = gpu.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
    ref, err = oracle.compress(cr, hd, w.state, w.input, w.ape, pc, counts[0])
    assert gerr == err == 0
    if counts[0] == 0:
        assert got.shape[0] == 0
    else:
        assert_pool_close(got, ref, "f32", "compress")
    st_o = w.state.copy()
    assert oracle.write(cr, hd, st_o, w.input, pw, counts[1]) == 0
    st_g = gpu.write(cr, hd, w.state, w.input, pw, counts[1])
    assert np.array_equal(st_g.view(np.uint8), st_o.view(np.uint8))
    if counts[1] == 0:
        assert np.array_equal(st_g.view(np.uint8), w.state.view(np.uint8)), "a write with no records changed the state"


def test_decode_maximum_batch(gpu):
    """Ratio-4 decode at the largest batch the ABI takes (65 536 requests, hd 128 bf16, a 512 MiB
    state): every pooled row against the oracle, the whole state bit for bit."""
    rng = np.random.default_rng(65536)
    B, hd, cr = 65536, 128, 4
    R = 4 * hd

    def bf16_bits(n):  # finite bf16 values in [0.5, 1) with random signs, drawn quickly
        return (rng.integers(0, 1 << 7, size=n, dtype=np.uint16) | np.uint16(0x3F00)
                | (rng.integers(0, 2, size=n, dtype=np.uint16) << np.uint16(15))).astype(np.uint16)

    s = rng.integers(1, 4097, size=B).astype(np.int32)
    idx = rng.permutation(B).astype(np.int32)
    state = bf16_bits(B * 8 * R).reshape(B * 8, R)
    inp = bf16_bits(B * R).reshape(B, R)
    ape = wl.to_bf16_bits((0.1 * rng.standard_normal((8, hd))).astype(np.float32))
    pd, status = oracle.plan_decode(cr, s, idx, B * 8)
    assert status == 0
    say("decode maximum batch B=%d boundaries=%d" % (B, int((s % cr == 0).sum())))
    st_o = state.copy()
    ref, err = oracle.decode(cr, hd, st_o, inp, ape, pd)
    got, st_g, gerr = gpu.decode(cr, hd, state, inp, ape, pd)
    assert err == gerr == 0
    assert_pool_close(got, ref, "bf16", "decode at the maximum batch")
    assert np.all(got[s % cr != 0] == 0.0)
    assert np.array_equal(st_g, st_o), "state differs after decode"


@pytest.mark.parametrize("B,hd,layout,listed", [
    (4100, 128, "random", False), (16384, 512, "random", False), (40000, 128, "random", False),
    (16384, 128, "clustered", False), (40000, 128, "clustered", False),
    (16384, 512, "random", True), (32768, 512, "random", True), (65536, 128, "random", True),
    (16384, 128, "clustered", True), (40000, 128, "clustered", True)])
def test_decode_c128_large_batches(gpu, B, hd, layout, listed):
    """Ratio-128 decode at large batches.  Without the planner's boundary list the pool workgroups
    rank the closing requests of each range of 1024 requests over 8 (up to 32 768 requests) or 4
    slots; with it (planned on the GPU, records checked against the oracle's) they take every
    P-th entry.  Above 16 384 requests the slices are 128 channels wide at bf16.  16 384 and
    32 768 at hd 512 bf16 are the bench sweep's launch shapes.  Closing requests sit at random
    places, or in one contiguous run across several ranges (every rank slot then pools many).
    The whole batch runs on the GPU from device-drawn inputs (a state of up to 8 GiB).  The
    oracle then pools every closing request and 256 others, each from a copy of its own page, and
    every state row is checked: each new token's row holds its input row bit for bit, and no
    other row changes."""
    cr, Wn = 128, 128
    R = 2 * hd
    dev = gpu.device
    rng = np.random.default_rng(B + hd + (layout == "clustered"))
    s = rng.integers(1, 65537, size=B).astype(np.int64)
    if layout == "clustered":  # a run of 1500 neighbours all closing a block, across range edges
        s[s % cr == 0] += 1
        close = np.arange(700, 2200)
    else:  # more closing requests at random places
        close = rng.choice(B, size=max(8, B // 64), replace=False)  # the first block among them
    s[close] = rng.integers(1, 512, size=len(close)) * 128
    s[close[0]] = 128
    s = s.astype(np.int32)
    idx = rng.permutation(B).astype(np.int32)
    g = torch.Generator(device=dev)
    g.manual_seed(B * 7 + hd)
    state = torch.randn((B * Wn, R), generator=g, device=dev).to(torch.bfloat16)
    inp = torch.randn((B, R), generator=g, device=dev).to(torch.bfloat16)
    ape = (0.1 * torch.randn((Wn, hd), generator=g, device=dev)).to(torch.bfloat16)
    pd, status = oracle.plan_decode(cr, s, idx, B * Wn)
    assert status == 0
    closing = np.nonzero(s % cr == 0)[0]
    others = rng.choice(np.nonzero(s % cr != 0)[0], size=256, replace=False)
    sample = np.concatenate([closing, others])
    pages = state.view(B, Wn, R)[torch.from_numpy(idx[sample].astype(np.int64)).to(dev)].contiguous()
    pristine = state.clone()
    say("decode c128 large batch B=%d hd=%d %s closing=%d list=%s" % (B, hd, layout, len(closing), listed))
    out = torch.full((B, hd), float("nan"), dtype=torch.float32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    bl = None
    pd_dev = torch.from_numpy(pd).to(dev)
    if listed:
        pd_dev = torch.zeros_like(pd_dev)
        bl = kvc.boundary_list(B, dev)
        kvc.plan_decode(cr, torch.from_numpy(s).to(dev), torch.from_numpy(idx).to(dev), B * Wn, pd_dev, st,
                        boundaries=bl)
        assert int(st.item()) == 0 and np.array_equal(pd_dev.cpu().numpy(), pd)
        lst = bl.cpu().numpy()
        n_c = len(closing)
        order = np.argsort(lst[0:2 * n_c:2])  # the list's order is not fixed
        assert lst[2 * B] == n_c and np.array_equal(lst[0:2 * n_c:2][order], closing)
        assert np.array_equal(lst[1:2 * n_c:2][order], oracle.unpack_d(pd)[closing, 2])
    kvc.decode(cr, hd, state, inp, ape, pd_dev, out, st, boundaries=bl)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    loc = torch.from_numpy(idx.astype(np.int64) * Wn + (s.astype(np.int64) - 1) % Wn).to(dev)
    assert torch.equal(state[loc].view(torch.int16), inp.view(torch.int16)), "new tokens' rows"
    state[loc] = pristine[loc]
    assert torch.equal(state.view(torch.int16), pristine.view(torch.int16)), "a row other than a new token's changed"
    del state, pristine
    n = len(sample)
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    pd_c, status = oracle.plan_decode(cr, s[sample], np.arange(n, dtype=np.int32), n * Wn)
    ref, err = oracle.decode(cr, hd, bits(pages.view(n * Wn, R)), bits(inp[torch.from_numpy(sample).to(dev)]),
                             bits(ape), pd_c)
    assert status == err == 0
    got = out[torch.from_numpy(sample).to(dev)].cpu().numpy().astype(np.float64)
    assert_pool_close(got, ref, "bf16", "decode c128 B=%d" % B)
    assert np.all(got[len(closing):] == 0.0)


def test_first_block_never_reads_masked_rows(gpu):
    """Block 0 of ratio 4: the overlap entries precede the sequence and must not be loaded.
    The state is NaN and the ragged rows before the request hold +-inf; a read of either
    would show up in the output."""
    hd = 128
    rng = np.random.default_rng(5)
    # request 0 fills ragged rows 0..5 with infinities; request 1 starts a sequence at row 6
    inp = rng.standard_normal((6 + 4, 4 * hd)).astype(np.float32)
    inp[:6] = np.inf
    s, e, idx = [6, 4], [6, 4], [1, 0]
    pc, pw, counts = oracle.plan_prefill(4, s, e, idx, 16, 10, 4, 14)
    C = oracle.unpack_c(pc[: counts[0]])
    ape = rng.standard_normal((8, hd)).astype(np.float32)
    state = nan_state(16, 4 * hd, "f32")
    got, gerr = gpu.compress(4, hd, state, inp, ape, pc, counts[0])
    ref, err = oracle.compress(4, hd, state, inp, ape, pc, counts[0])
    k = [int(r[1]) for r in C].index(9)
    assert gerr == err == 0 and np.all(np.isfinite(got[k]))
    assert_pool_close(got[k:k + 1], ref[k:k + 1], "f32", "first block")
    # decode of the first block too
    pd, _ = oracle.plan_decode(4, [4], [0], 8)
    st = nan_state(8, 4 * hd, "f32")
    st[0:3] = inp[6:9]  # positions 0..2 already in the ring
    out, st_g, gerr = gpu.decode(4, hd, st, inp[9:10], ape, pd)
    ref, _ = oracle.decode(4, hd, st.copy(), inp[9:10], ape, pd)
    assert gerr == 0 and np.all(np.isfinite(out))
    assert_pool_close(out, ref, "f32", "first block decode")


def test_consumer_record_errors(gpu):
    hd = 128
    inp = np.zeros((4, 4 * hd), np.float32)
    st = np.zeros((8, 4 * hd), np.float32)
    bad_w = np.zeros((1, 8), np.uint8)
    bad_w.view("<u4")[0, 0] = 9
    counts = torch.tensor([0, 1, 0, 0], dtype=torch.int32, device="cuda")
    from tests.gpu_backend import to_dev
    st_d = to_dev(st)
    kvc.write(4, hd, st_d, to_dev(inp), to_dev(bad_w), counts)
    assert int(counts[3].item()) == oracle.write(4, hd, st.copy(), inp, bad_w, 1) == kvc.DERR_RECORD
    assert torch.count_nonzero(st_d).item() == 0
    bad_c = np.zeros((1, 16), np.uint8)
    bad_c.view("<u4")[0] = [8, 3 | (2 << 24), 0, 5]
    got, gerr = gpu.compress(4, hd, st, inp, np.zeros((8, hd), np.float32), bad_c, 1)
    _, err = oracle.compress(4, hd, st, inp, np.zeros((8, hd), np.float32), bad_c, 1)
    assert gerr == err == kvc.DERR_RECORD and np.all(np.isnan(got))
    bad_d = np.zeros((1, 16), np.uint8)
    bad_d.view("<i4")[0] = [8, 99, 0, 1]
    out, st_g, gerr = gpu.decode(4, hd, st, inp[:1], np.zeros((8, hd), np.float32), bad_d)
    ref, oerr = oracle.decode(4, hd, st.copy(), inp[:1], np.zeros((8, hd), np.float32), bad_d)
    assert gerr == oerr == kvc.DERR_RECORD and np.all(out == 0) and np.array_equal(st_g, st)


# --------------------------------------------------------------------------
# end to end: chunked prefill + decode, GPU against the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cr,dtype", [(4, "bf16"), (4, "f32"), (128, "bf16")])
def test_chunked_prefill_then_decode(gpu, cr, dtype):
    rng = np.random.default_rng(21 + cr)
    hd = 128
    B = 5
    R = wl.ROW_MULT[cr] * hd
    decode_steps = 12 if cr == 4 else 140
    seqs, chunks = [], []
    for b in range(B):
        L = int(rng.integers(1, 5 * W[cr]))
        x = rng.standard_normal((L + decode_steps, R)).astype(np.float32)
        seqs.append(wl.to_bf16_bits(x) if dtype == "bf16" else x)
        chunks.append(random_split(rng, L, 5))
    ape_f = (0.1 * rng.standard_normal((W[cr], hd))).astype(np.float32)
    ape = wl.to_bf16_bits(ape_f) if dtype == "bf16" else ape_f
    idx = rng.permutation(7)[:B]
    say("chunked cr=%d %s chunks=%s" % (cr, dtype, chunks))
    em_o, st_o = run_chunked(OracleBackend(oracle), cr, hd, dtype, seqs, chunks, decode_steps, idx, 7, ape)
    em_g, st_g = run_chunked(gpu, cr, hd, dtype, seqs, chunks, decode_steps, idx, 7, ape)
    assert sorted(em_o) == sorted(em_g)
    for k in em_o:
        assert_pool_close(em_g[k][None], em_o[k][None], dtype, str(k))
    assert np.array_equal(st_g.view(np.uint8), st_o.view(np.uint8))


# --------------------------------------------------------------------------
# the named workloads at full size, GPU plans feeding GPU kernels
# --------------------------------------------------------------------------

def _run_prefill_pipeline(w):
    """GPU: plan -> compress -> write, all through the C ABI, in the launch order the bench uses."""
    from tests.gpu_backend import to_dev
    cr, hd = w.cr, w.hd
    plan_c, plan_w, counts = kvc.alloc_prefill_plan(cr, w.B, w.num_q)
    state = to_dev(w.state)
    inp = to_dev(w.input)
    ape = to_dev(w.ape)
    out = torch.full((plan_c.shape[0], hd), float("nan"), dtype=torch.float32, device="cuda")
    kvc.plan_prefill(cr, to_dev(w.seq_lens), to_dev(w.extend_lens), to_dev(w.state_index), w.num_state_rows,
                     w.num_q, plan_c, plan_w, counts)
    kvc.compress(cr, hd, state, inp, ape, plan_c, counts, out)
    kvc.write(cr, hd, state, inp, plan_w, counts)
    torch.cuda.synchronize()
    return (plan_c.cpu().numpy(), plan_w.cpu().numpy(), counts.cpu().numpy(), out.cpu().numpy(),
            state.cpu().numpy())


@pytest.mark.parametrize("name", ["c4_prefill_1x64", "c128_prefill_4req", "mixed_c4", "mixed_c128", "mixed_c4_e2",
                                  "mixed_c128_e2"])
def test_named_prefill_workloads(gpu, name):
    w = {"c4_prefill_1x64": lambda: wl.c4_prefill_1x64(), "c128_prefill_4req": lambda: wl.c128_prefill_4req(),
         "mixed_c4": lambda: wl.mixed_prefill(4), "mixed_c128": lambda: wl.mixed_prefill(128),
         "mixed_c4_e2": lambda: wl.mixed_prefill(4, uniform_extend=2),
         "mixed_c128_e2": lambda: wl.mixed_prefill(128, uniform_extend=2)}[name]()
    say("workload %s: B=%d num_q=%d" % (w.name, w.B, w.num_q))
    pc, pw, counts, out, state = _run_prefill_pipeline(w)
    cap_c, cap_w = oracle.capacities(w.cr, w.B, w.num_q)
    opc, opw, ocounts = oracle.plan_prefill(w.cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                            w.num_q, cap_c, cap_w)
    assert counts.tolist() == ocounts.tolist() and counts[2] == 0 and counts[3] == 0
    assert np.array_equal(pc, opc) and np.array_equal(pw, opw)
    n = int(counts[0])
    ref, err = oracle.compress(w.cr, w.hd, w.state, w.input, w.ape, opc, n)
    assert err == 0
    assert_pool_close(out[:n], ref[:n], w.dtype, w.name)
    st_o = w.state.copy()
    oracle.write(w.cr, w.hd, st_o, w.input, opw, int(ocounts[1]))
    assert np.array_equal(state.view(np.uint8), st_o.view(np.uint8))
    if name == "c4_prefill_1x64":
        assert n == 16 and counts[1] == 4


@pytest.mark.parametrize("name", ["c4_decode_b256", "c128_decode_b1024"])
def test_named_decode_workloads(gpu, name):
    from tests.gpu_backend import to_dev
    w = wl.c4_decode_b256() if name == "c4_decode_b256" else wl.c128_decode_b1024()
    say("workload %s: B=%d boundaries=%d" % (w.name, w.B, int((w.seq_lens % w.cr == 0).sum())))
    plan_d = torch.empty((w.B, kvc.D_BYTES), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    state = to_dev(w.state)
    out = torch.full((w.B, w.hd), float("nan"), dtype=torch.float32, device="cuda")
    kvc.plan_decode(w.cr, to_dev(w.seq_lens), to_dev(w.state_index), w.num_state_rows, plan_d, status)
    kvc.decode(w.cr, w.hd, state, to_dev(w.input), to_dev(w.ape), plan_d, out, status)
    torch.cuda.synchronize()
    opd, ostatus = oracle.plan_decode(w.cr, w.seq_lens, w.state_index, w.num_state_rows)
    assert int(status.item()) == ostatus == 0
    assert np.array_equal(plan_d.cpu().numpy(), opd)
    st_o = w.state.copy()
    ref, err = oracle.decode(w.cr, w.hd, st_o, w.input, w.ape, opd)
    assert err == 0
    assert_pool_close(out.cpu().numpy(), ref, w.dtype, w.name)
    assert np.array_equal(state.cpu().numpy().view(np.uint8), st_o.view(np.uint8))


def test_plan_prefill_maximum_size(gpu):
    """1024 requests and 2^24 - 1 tokens: ragged ids use all 24 bits of the C record."""
    for cr in (4, 128):
        rng = np.random.default_rng(99 + cr)
        e = np.full(1024, 16384, np.int64)
        e[-1] = (1 << 24) - 1 - int(e[:-1].sum())
        prefix = rng.integers(0, 1 << 20, size=1024)
        s = prefix + e
        idx = rng.permutation(1024)
        num_q = int(e.sum())
        assert num_q == (1 << 24) - 1
        cap_c, cap_w = oracle.capacities(cr, 1024, num_q)
        say("plan_prefill maximum size cr=%d cap_c=%d" % (cr, cap_c))
        g = gpu.plan_prefill(cr, s, e, idx, 1024 * W[cr], num_q, cap_c, cap_w)
        o = oracle.plan_prefill(cr, s, e, idx, 1024 * W[cr], num_q, cap_c, cap_w)
        _plans_equal(g, o)
        last = oracle.unpack_c(g[0][g[2][0] - 1: g[2][0]])[0]
        assert last[1] > (1 << 23)  # the high ragged-id bits are in use


def test_prefill_chunk_under_graph_capture(gpu):
    """A whole prefill chunk (plan, compress, write) captured in a HIP graph and replayed: every
    replay matches the eager run.  Nothing in the path syncs, allocates or memsets."""
    from tests.gpu_backend import to_dev
    rng = np.random.default_rng(17)
    w = wl.random_prefill(rng, 4, 512, "bf16", 8, prefix_hi=500, extend_lo=1, extend_hi=700, num_slots=12)
    s_d, e_d, i_d = to_dev(w.seq_lens), to_dev(w.extend_lens), to_dev(w.state_index)
    inp, ape = to_dev(w.input), to_dev(w.ape)
    state0 = to_dev(w.state)
    plan_c, plan_w, counts = kvc.alloc_prefill_plan(4, w.B, w.num_q)
    state = state0.clone()
    out = torch.zeros((plan_c.shape[0], w.hd), dtype=torch.float32, device="cuda")

    def chunk():
        kvc.plan_prefill(4, s_d, e_d, i_d, w.num_state_rows, w.num_q, plan_c, plan_w, counts)
        kvc.compress_c4(w.hd, state, inp, ape, plan_c, counts, out)
        kvc.write(4, w.hd, state, inp, plan_w, counts)

    chunk()
    torch.cuda.synchronize()
    ref_out, ref_state, ref_counts = out.clone(), state.clone(), counts.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        state.copy_(state0)
        with torch.cuda.graph(g, stream=side):
            chunk()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        say("graph replay", rep)
        state.copy_(state0)
        out.zero_()
        counts.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(counts, ref_counts)
        assert torch.equal(out, ref_out)
        assert torch.equal(state, ref_state)
