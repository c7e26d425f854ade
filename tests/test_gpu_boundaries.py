"""GPU tests of the ratio-128 boundary list.

kvc_plan_decode and kvc_plan_decode_swa can write, beside the decode records, the list of the
requests whose new token closes a block (valid records with seq_len % 128 == 0), each with the
page its window is read from, and their count; kvc_decode_c128 then pools from the list instead of
scanning the records.  The list is not part of the method and its order is not fixed, so what is
unique about it is compared bit for bit with the oracle's records: the count, the set of requests
(each once), each request's page, the untouched entries past the count.  Decodes with and without
the list must give the same rows and state bit for bit, and both match the oracle (bars as in
test_gpu_parity.py).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import kvc  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402
from tests.gpu_backend import to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu
SENT = 0x5A5A5A5A  # fill of the list before planning: entries past the count must keep it


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def expected_list(pd):
    """(requests, pages) of the records that pool: invalid records carry seq_len 0xFFFFFFFF."""
    d = oracle.unpack_d(pd)
    b = np.nonzero(d[:, 0] % 128 == 0)[0]
    return b, d[b, 2]


def check_list(bl, pd, what):
    B = pd.shape[0]
    b, page = expected_list(pd)
    n = len(b)
    assert bl.shape == (2 * B + 2,)
    assert bl[2 * B] == n and bl[2 * B + 1] == 0, "%s: count %d, expected %d" % (what, bl[2 * B], n)
    req, pg = bl[0:2 * n:2], bl[1:2 * n:2]
    order = np.argsort(req, kind="stable")
    assert np.array_equal(req[order], b), "%s: requests differ" % what
    assert np.array_equal(pg[order], page), "%s: pages differ" % what
    assert np.all(bl[2 * n:2 * B] == SENT), "%s: entries past the count were written" % what
    return n


def gpu_plan(dev, s, idx, rows):
    B = len(s)
    pd = torch.full((B, kvc.D_BYTES), 0x5A, dtype=torch.uint8, device=dev)
    bl = torch.full((2 * B + 2,), SENT, dtype=torch.int32, device=dev)
    st = torch.full((1,), -7, dtype=torch.int32, device=dev)
    kvc.plan_decode(128, to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(idx, np.int32)), int(rows), pd, st,
                    boundaries=bl)
    return pd, bl, int(st.item())


def decode_pair(dev, hd, state, inp, ape, pd, bl):
    """kvc_decode_c128 without and with the list on copies of the same state."""
    res = []
    for lst in (None, bl):
        st = to_dev(state)
        out = torch.full((pd.shape[0], hd), float("nan"), dtype=torch.float32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        kvc.decode_c128(hd, st, to_dev(inp), to_dev(ape), pd, out, status, boundaries=lst)
        res.append((out.cpu().numpy().astype(np.float64), to_host(st, state), int(status.item())))
    return res


def assert_pool_close(got, ref, dtype, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), what
    tol = (1e-5 + 1e-5 * np.abs(ref)) if dtype == "f32" else np.full_like(ref, 2e-2)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), "%s: %d elements out of tolerance" % (what, bad.sum())


@pytest.mark.parametrize("B", [1, 7, 300, 1024, 1025, 4100, 65536])
def test_plan_decode_boundary_list(dev, B):
    """Random lengths with one request in 8 closing a block, plus requests that get invalid records
    (seq_len <= 0, a state index out of range), some of them on a boundary length."""
    rng = np.random.default_rng(900 + B)
    slots = B + 5
    s = rng.integers(1, 1 << 20, size=B)
    close = rng.random(B) < 1 / 8
    s[close] = rng.integers(1, 8192, size=int(close.sum())) * 128
    idx = rng.permutation(slots)[:B]
    if B > 2:
        bad = rng.choice(B, size=max(1, B // 40), replace=False)
        s[bad[::2]] = rng.choice([0, -128, -5], size=len(bad[::2]))
        idx[bad[1::2]] = slots + 3
        s[bad[1::2]] = 256  # a boundary length on a bad index: no entry
    say("plan_decode boundary list B=%d closing=%d" % (B, int(close.sum())))
    pd, bl, status = gpu_plan(dev, s, idx, slots * 128)
    opd, ostatus = oracle.plan_decode(128, s, idx, slots * 128)
    assert status == ostatus and np.array_equal(pd.cpu().numpy(), opd)
    check_list(bl.cpu().numpy(), opd, "B=%d" % B)


@pytest.mark.parametrize("B,kind", [(4096, "all"), (5000, "all"), (65536, "all"), (5000, "none")])
def test_plan_decode_boundary_list_extremes(dev, B, kind):
    """Every request closes a block (the list holds the whole batch: every planner thread then has a
    closing request in each of up to 64 passes, past the 4 it keeps in registers), or none does
    (count 0)."""
    rng = np.random.default_rng(17)
    s = rng.integers(1, 600, size=B) * 128 + (0 if kind == "all" else rng.integers(1, 128, size=B))
    idx = rng.permutation(B)
    pd, bl, status = gpu_plan(dev, s, idx, B * 128)
    opd, _ = oracle.plan_decode(128, s, idx, B * 128)
    assert status == 0 and np.array_equal(pd.cpu().numpy(), opd)
    assert check_list(bl.cpu().numpy(), opd, kind) == (B if kind == "all" else 0)


def test_plan_decode_swa_boundary_list(dev):
    rng = np.random.default_rng(640)
    for B in (1, 33, 1024, 5000):
        stride = 3000
        r2t, f2s, _ = wl.swa_tables(rng, stride, B + 3, 128, stride=stride)
        rows = (B + 3) * 128
        s = rng.integers(1, stride + 1, size=B)
        close = rng.random(B) < 1 / 4
        s[close] = rng.integers(1, stride // 128 + 1, size=int(close.sum())) * 128
        rid = rng.permutation(B + 3)[:B]
        say("plan_decode_swa boundary list B=%d" % B)
        pd = torch.full((B, kvc.D_BYTES), 0x5A, dtype=torch.uint8, device=dev)
        bl = torch.full((2 * B + 2,), SENT, dtype=torch.int32, device=dev)
        st = torch.full((1,), -7, dtype=torch.int32, device=dev)
        kvc.plan_decode_swa(128, to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(rid, np.int32)),
                            to_dev(np.asarray(r2t, np.int32)), to_dev(np.asarray(f2s, np.int32)), 128, 128, rows,
                            pd, st, boundaries=bl)
        opd, ostatus = oracle.plan_decode_swa(128, s, rid, r2t, f2s, 128, 128, rows)
        assert int(st.item()) == ostatus == 0 and np.array_equal(pd.cpu().numpy(), opd)
        check_list(bl.cpu().numpy(), opd, "swa B=%d" % B)


@pytest.mark.parametrize("hd,dtype", [(512, "bf16"), (128, "f32"), (256, "f32"), (128, "bf16"), (512, "f32"),
                                      (256, "bf16")])
def test_decode_c128_with_list(dev, hd, dtype):
    rng = np.random.default_rng(31 * hd + (dtype == "bf16"))
    for trial in range(3):
        B = int(rng.integers(1, 300))
        w = wl.random_decode(rng, 128, hd, dtype, B, prefix_hi=3 * 128, num_slots=B + 2)
        if trial == 2:  # every request on a boundary, including the first block
            w.seq_lens = (rng.integers(1, 4, size=B) * 128).astype(np.int32)
        pd, bl, status = gpu_plan(dev, w.seq_lens, w.state_index, w.num_state_rows)
        opd, ostatus = oracle.plan_decode(128, w.seq_lens, w.state_index, w.num_state_rows)
        assert status == ostatus == 0 and np.array_equal(pd.cpu().numpy(), opd)
        n = check_list(bl.cpu().numpy(), opd, "trial %d" % trial)
        say("decode c128 with list hd=%d %s trial=%d B=%d boundaries=%d" % (hd, dtype, trial, B, n))
        (g0, s0, e0), (g1, s1, e1) = decode_pair(dev, hd, w.state, w.input, w.ape, pd, bl)
        st_o = w.state.copy()
        ref, err = oracle.decode(128, hd, st_o, w.input, w.ape, opd)
        assert err == e0 == e1 == 0
        assert np.array_equal(g0.view(np.uint64), g1.view(np.uint64)), "rows differ with the list"
        assert np.array_equal(s0.view(np.uint8), s1.view(np.uint8)), "state differs with the list"
        assert_pool_close(g1, ref, dtype, "decode with the list")
        assert np.array_equal(s1.view(np.uint8), st_o.view(np.uint8)), "state differs from the oracle's"


def test_decode_c128_list_errors(dev):
    """A list that does not match the records: a count above the batch is clamped, entries outside the
    batch or the state are skipped and reported, and a negative count pools nothing (the closing
    requests' rows are then left as they were)."""
    hd, B = 128, 200
    rng = np.random.default_rng(77)
    w = wl.random_decode(rng, 128, hd, "bf16", B, prefix_hi=3 * 128, num_slots=B + 2)
    w.seq_lens[:5] = 128 * np.arange(1, 6)
    pd, bl, _ = gpu_plan(dev, w.seq_lens, w.state_index, w.num_state_rows)
    good = bl.clone()
    n = int(good[2 * B].item())
    assert 5 <= n <= B - 3
    (ref, st_ref, _), _ = decode_pair(dev, hd, w.state, w.input, w.ape, pd, good)
    closing = np.nonzero(w.seq_lens % 128 == 0)[0]
    for what, edit, expect in [
        ("count above the batch", lambda t: t.__setitem__(2 * B, 3 * B), kvc.DERR_RECORD),
        ("bad entries", lambda t: (t.__setitem__(slice(2 * n, 2 * n + 4), torch.tensor([B + 3, 0, 0, 1 << 30],
                                                                                       dtype=torch.int32)),
                                   t.__setitem__(2 * B, n + 2)), kvc.DERR_RECORD),
        ("negative count", lambda t: t.__setitem__(2 * B, -4), 0),
    ]:
        bad = good.clone()
        edit(bad)
        st = to_dev(w.state)
        out = torch.full((B, hd), float("nan"), dtype=torch.float32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        say("decode c128 list error case: %s" % what)
        kvc.decode_c128(hd, st, to_dev(w.input), to_dev(w.ape), pd, out, status, boundaries=bad)
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(to_host(st, w.state).view(np.uint8), st_ref.view(np.uint8)), what
        if what == "negative count":
            assert int(status.item()) == 0
            assert np.all(np.isnan(got[closing])), what
            rest = np.setdiff1d(np.arange(B), closing)
            assert np.array_equal(got[rest], ref[rest]), what
        else:
            # a count above the batch reads every entry of the list: those past the real count hold
            # the fill the planner left, a request outside the batch, and are reported too
            assert int(status.item()) == expect, what
            assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), what


def test_random_boundary_lists(dev):
    """60 random batches (up to 8192 requests, hd 128-512, bf16 or fp32): closing requests at random,
    in one cluster or strided, at fractions from none to all, with invalid records among them.  The
    list against the oracle's records, and the decode with and without it bit for bit."""
    for case in range(60):
        rng = np.random.default_rng([41, case])
        B = int(np.exp(rng.uniform(0, np.log(8192))))
        hd = int(rng.choice([128, 256, 512]))
        dtype = str(rng.choice(["bf16", "f32"]))
        s = rng.integers(1, 65537, size=B)
        s[s % 128 == 0] += 1
        nb = int(round(float(rng.choice([0.0, 1 / 128, 1 / 16, 0.5, 1.0])) * B))
        if nb:
            kind = int(rng.integers(0, 3))
            if kind == 0:
                close = rng.choice(B, size=nb, replace=False)
            elif kind == 1:
                first = int(rng.integers(0, B - nb + 1))
                close = np.arange(first, first + nb)
            else:
                close = (np.arange(nb) * max(1, B // nb)) % B
            s[close] = rng.integers(1, 512, size=len(close)) * 128
        slots = B + 2
        idx = rng.permutation(slots)[:B]
        if B > 8:
            bad = rng.choice(B, size=B // 8, replace=False)
            s[bad[::2]] = 0
            idx[bad[1::2]] = slots + 5
        say("random boundary list case %d B=%d hd=%d %s closing=%d" % (case, B, hd, dtype, nb))
        pd, bl, status = gpu_plan(dev, s, idx, slots * 128)
        opd, ostatus = oracle.plan_decode(128, s, idx, slots * 128)
        assert status == ostatus and np.array_equal(pd.cpu().numpy(), opd)
        check_list(bl.cpu().numpy(), opd, "case %d" % case)
        R = 2 * hd
        g = torch.Generator(device=dev)
        g.manual_seed(case)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        state0 = torch.randn((slots * 128, R), generator=g, device=dev).to(tdt)
        inp = torch.randn((B, R), generator=g, device=dev).to(tdt)
        ape = (0.1 * torch.randn((128, hd), generator=g, device=dev)).to(tdt)
        res = []
        for lst in (None, bl):
            state = state0.clone()
            out = torch.full((B, hd), float("nan"), dtype=torch.float32, device=dev)
            st = torch.zeros(1, dtype=torch.int32, device=dev)
            kvc.decode_c128(hd, state, inp, ape, pd, out, st, boundaries=lst)
            res.append((out.view(torch.int32).cpu(), state.view(torch.int16).cpu(), int(st.item())))
        assert res[0][2] == res[1][2]
        assert torch.equal(res[0][0], res[1][0]), "case %d: rows differ with the list" % case
        assert torch.equal(res[0][1], res[1][1]), "case %d: state differs with the list" % case


def test_decode_c128_with_swa_list(dev):
    """The list from kvc_plan_decode_swa feeds kvc_decode_c128: rows and state equal bit for bit to the
    decode without it, and the rows match the oracle's decode of the oracle's SWA records."""
    rng = np.random.default_rng(655)
    hd, B, stride = 256, 600, 1024
    r2t, f2s, _ = wl.swa_tables(rng, stride, B + 3, 128, stride=stride)
    rows = (B + 3) * 128
    s = rng.integers(1, stride + 1, size=B)
    close = rng.random(B) < 1 / 4
    s[close] = rng.integers(1, stride // 128 + 1, size=int(close.sum())) * 128
    rid = rng.permutation(B + 3)[:B]
    pd = torch.empty((B, kvc.D_BYTES), dtype=torch.uint8, device=dev)
    bl = torch.full((2 * B + 2,), SENT, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    kvc.plan_decode_swa(128, to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(rid, np.int32)),
                        to_dev(np.asarray(r2t, np.int32)), to_dev(np.asarray(f2s, np.int32)), 128, 128, rows,
                        pd, st, boundaries=bl)
    opd, ostatus = oracle.plan_decode_swa(128, s, rid, r2t, f2s, 128, 128, rows)
    assert int(st.item()) == ostatus == 0 and np.array_equal(pd.cpu().numpy(), opd)
    n = check_list(bl.cpu().numpy(), opd, "swa")
    say("decode c128 with an SWA list B=%d boundaries=%d" % (B, n))
    R = 2 * hd
    state = wl.to_bf16_bits(rng.standard_normal((rows, R)).astype(np.float32))
    inp = wl.to_bf16_bits(rng.standard_normal((B, R)).astype(np.float32))
    ape = wl.to_bf16_bits((0.1 * rng.standard_normal((128, hd))).astype(np.float32))
    (g0, s0, e0), (g1, s1, e1) = decode_pair(dev, hd, state, inp, ape, pd, bl)
    st_o = state.copy()
    ref, err = oracle.decode(128, hd, st_o, inp, ape, opd)
    assert err == e0 == e1 == 0
    assert np.array_equal(g0.view(np.uint64), g1.view(np.uint64)), "rows differ with the list"
    assert np.array_equal(s0.view(np.uint8), s1.view(np.uint8)), "state differs with the list"
    assert_pool_close(g1, ref, "bf16", "SWA decode with the list")
    assert np.array_equal(s1.view(np.uint8), st_o.view(np.uint8)), "state differs from the oracle's"


def test_decode_step_with_list_under_graph_capture(dev):
    """plan_decode with the boundary list, then decode_c128 from it, captured in a HIP graph and
    replayed: every replay matches the eager run (the list's count word included).  The planner
    takes its entries from an LDS counter, so nothing needs clearing between steps."""
    rng = np.random.default_rng(23)
    hd, B = 512, 3000
    w = wl.random_decode(rng, 128, hd, "bf16", B, prefix_hi=3 * 128, num_slots=B + 2)
    w.seq_lens[rng.choice(B, size=B // 10, replace=False)] = 128 * 2
    s_d, i_d = to_dev(w.seq_lens), to_dev(w.state_index)
    inp, ape, state0 = to_dev(w.input), to_dev(w.ape), to_dev(w.state)
    pd = torch.empty((B, kvc.D_BYTES), dtype=torch.uint8, device=dev)
    bl = kvc.boundary_list(B, dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.zeros((B, hd), dtype=torch.float32, device=dev)
    state = state0.clone()

    def step():
        kvc.plan_decode(128, s_d, i_d, w.num_state_rows, pd, st, boundaries=bl)
        kvc.decode_c128(hd, state, inp, ape, pd, out, st, boundaries=bl)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), state.clone(), int(bl[2 * B].item()), int(st.item()))
    assert ref[3] == 0 and ref[2] == int((w.seq_lens % 128 == 0).sum())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        state.copy_(state0)
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        say("decode step graph replay", rep)
        state.copy_(state0)
        out.fill_(float("nan"))
        bl.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(bl[2 * B].item()) == ref[2] and int(st.item()) == 0
        assert torch.equal(out.view(torch.int32), ref[0].view(torch.int32))
        assert torch.equal(state.view(torch.int16), ref[1].view(torch.int16))


def test_binding_rejects_bad_lists(dev):
    """The binding refuses a boundary list for ratio 4, one shorter than 2 * batch + 2 entries, and one
    that is not int32, before anything is enqueued."""
    B = 16
    s = to_dev(np.full(B, 128, np.int32))
    idx = to_dev(np.arange(B, dtype=np.int32))
    pd = torch.empty((B, kvc.D_BYTES), dtype=torch.uint8, device=dev)
    for cr, bl in ((4, kvc.boundary_list(B, dev)), (128, torch.zeros(2 * B + 1, dtype=torch.int32, device=dev)),
                   (128, torch.zeros(2 * B + 2, dtype=torch.int64, device=dev))):
        with pytest.raises(kvc.KvcError):
            kvc.plan_decode(cr, s, idx, B * 128, pd, None, boundaries=bl)
    state = torch.zeros((B * 128, 256), dtype=torch.bfloat16, device=dev)
    inp = torch.zeros((B, 256), dtype=torch.bfloat16, device=dev)
    ape = torch.zeros((128, 128), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((B, 128), dtype=torch.float32, device=dev)
    with pytest.raises(kvc.KvcError):
        kvc.decode(4, 128, state, inp, ape, pd, out, None, boundaries=kvc.boundary_list(B, dev))
    with pytest.raises(kvc.KvcError):
        kvc.decode_c128(128, state, inp, ape, pd, out, None, boundaries=torch.zeros(2 * B, dtype=torch.int32,
                                                                                     device=dev))
