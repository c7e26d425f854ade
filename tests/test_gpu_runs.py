"""GPU parity of the ratio-128 run list (kvc_plan_prefill's `runs` output) and of the online state
update that reads it (kvc_write_c128_online with `runs`).

The list is integer work and is compared bit for bit with the list read off the oracle's W records:
request b's run is its W records (the ones on its slot's page), given by the first record's
ragged row and write location and the record count; a request without W records, and every request
of a plan with an error, has an all-zero entry.  The slots written from the list are compared with
the oracle's write_online under the same bars as the scan path, and with the scan path's bit for bit
(both fold a run by the same path for its length).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import kvc  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402
from tests.test_gpu_online import _slots, assert_slots_close  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.load()
    return torch.device("cuda")


def to_dev(a, dev):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)


def expected_runs(pw, num_w, idx):
    """The run list read off the oracle's W records: per request, the records on its page."""
    w = oracle.unpack_w(pw[:num_w]).astype(np.int64) if num_w else np.zeros((0, 2), np.int64)
    out = np.zeros((len(idx), 4), np.int32)
    for b, slot in enumerate(np.asarray(idx, np.int64)):
        k = np.nonzero(w[:, 1] // 128 == slot)[0]
        if len(k) == 0:
            continue
        # the records of one request are consecutive, with consecutive rows and positions
        assert np.array_equal(k, np.arange(k[0], k[0] + len(k)))
        assert np.array_equal(w[k, 0] - w[k[0], 0], np.arange(len(k)))
        assert np.array_equal(w[k, 1] - w[k[0], 1], np.arange(len(k)))
        out[b] = (w[k[0], 0], w[k[0], 1], len(k), 0)
    return out


def gpu_plan(s, e, idx, rows, num_q, dev, cap=None):
    B = len(s)
    cap_c, cap_w = cap if cap is not None else oracle.capacities(128, B, num_q)
    pc, pw, counts = kvc.alloc_prefill_plan(128, B, num_q, dev, cap_c=cap_c, cap_w=cap_w)
    runs = kvc.run_list(B, dev)
    runs.fill_(0x5A5A5A5A)  # every entry must be written
    kvc.plan_prefill(128, to_dev(np.asarray(s, np.int32), dev), to_dev(np.asarray(e, np.int32), dev),
                     to_dev(np.asarray(idx, np.int32), dev), int(rows), int(num_q), pc, pw, counts, runs=runs)
    return pc, pw, counts, runs


def check_list(s, e, idx, rows, num_q, dev, what):
    B = len(s)
    cap_c, cap_w = oracle.capacities(128, B, num_q)
    opc, opw, oc = oracle.plan_prefill(128, np.asarray(s, np.int32), np.asarray(e, np.int32),
                                       np.asarray(idx, np.int32), rows, num_q, cap_c, cap_w)
    pc, pw, counts, runs = gpu_plan(s, e, idx, rows, num_q, dev)
    got = runs.cpu().numpy()
    assert counts.cpu().tolist() == oc.tolist(), what
    assert np.array_equal(pw.cpu().numpy(), opw), what
    want = expected_runs(opw, int(oc[1]), idx) if oc[2] == 0 else np.zeros((B, 4), np.int32)
    assert np.array_equal(got, want), "%s: %d entries differ" % (what, int((got != want).any(axis=1).sum()))
    return got


def test_run_list_random_batches(dev):
    rng = np.random.default_rng(4401)
    for trial in range(12):
        B = int(rng.choice([1, 7, 64, 333, 1024]))
        prefix = rng.integers(0, 70000, size=B)
        e = rng.integers(1, 600, size=B)
        s = prefix + e
        # some requests end exactly on a block boundary: no W records, an all-zero entry
        end = rng.random(B) < 0.2
        s[end] = np.maximum(128, (s[end] // 128) * 128)
        e = np.minimum(e, s)
        num_q = int(e.sum())
        idx = rng.permutation(B + 9)[:B]
        say("run list trial=%d B=%d num_q=%d block ends=%d" % (trial, B, num_q, int((s % 128 == 0).sum())))
        got = check_list(s, e, idx, (B + 9) * 128, num_q, dev, "trial %d" % trial)
        assert np.all(got[s % 128 == 0] == 0)


def test_run_list_uniform_extends(dev):
    """The planner's equal-extend path (every extend the same E <= 32), as when a few tokens per
    request are verified at once."""
    rng = np.random.default_rng(4402)
    for B, E in ((64, 2), (1000, 1), (17, 32), (1024, 4)):
        s = rng.integers(E, 9000, size=B)
        e = np.full(B, E)
        idx = rng.permutation(B)
        say("run list uniform B=%d E=%d" % (B, E))
        check_list(s, e, idx, B * 128, B * E, dev, "uniform B=%d E=%d" % (B, E))


def test_run_list_on_plan_errors_is_all_zero(dev):
    rng = np.random.default_rng(4403)
    B = 40
    s = rng.integers(200, 5000, size=B)
    e = rng.integers(1, 150, size=B)
    idx = rng.permutation(B + 3)[:B]
    cases = {"duplicate slot": (s, e, np.where(np.arange(B) == 7, idx[3], idx), kvc.DERR_DUPLICATE),
             "slot out of range": (s, e, np.where(np.arange(B) == 5, B + 3, idx), kvc.DERR_INDEX),
             "extend above length": (s, np.where(np.arange(B) == 2, s + 1, e), idx, kvc.DERR_EXTEND)}
    for name, (s_, e_, idx_, bit) in cases.items():
        num_q = int(np.asarray(e_).sum())
        say("run list error case: %s" % name)
        _, _, counts, runs = gpu_plan(s_, e_, idx_, (B + 3) * 128, num_q, dev)
        c = counts.cpu().tolist()
        assert c[2] & bit and c[0] == c[1] == 0, name
        assert not runs.cpu().numpy().any(), name
    # more W records than the capacity: a capacity error, and no run either
    num_q = int(e.sum())
    say("run list error case: capacity")
    _, _, counts, runs = gpu_plan(s, e, idx, (B + 3) * 128, num_q, dev, cap=(num_q, 3))
    assert counts.cpu().tolist()[2] & kvc.DERR_CAPACITY and not runs.cpu().numpy().any()


SHAPES = [(512, "bf16"), (128, "f32"), (256, "bf16"), (512, "f32")]


def _inputs(rng, num_q, hd, dtype):
    x = rng.standard_normal((num_q, 2 * hd)).astype(np.float32)
    a = (0.1 * rng.standard_normal((128, hd))).astype(np.float32)
    if dtype == "bf16":
        return wl.to_bf16_bits(x), wl.to_bf16_bits(a)
    return x, a


def write_with_runs(hd, slots, inp, ape, s, e, idx, rows, dev):
    """The slots after the write from the run list, and after the write that scans the W records."""
    pc, pw, counts, runs = gpu_plan(s, e, idx, rows, int(np.asarray(e).sum()), dev)
    st = to_dev(np.asarray(slots, np.float32), dev)
    st_scan = st.clone()
    inp_d, ape_d = to_dev(inp, dev), to_dev(ape, dev)
    kvc.write_c128_online(hd, st, inp_d, ape_d, pw, counts, runs=runs)
    kvc.write_c128_online(hd, st_scan, inp_d, ape_d, pw, counts)
    return st.cpu().numpy(), st_scan.cpu().numpy(), counts.cpu().numpy(), pw.cpu().numpy()


@pytest.mark.parametrize("hd,dtype", SHAPES)
def test_write_from_run_list(hd, dtype, dev):
    """Random chunks (runs that continue a block and runs that start one) and the run shapes of the
    scan path's test: every record a run of its own, runs of 1-3, 2-40 and 127 records."""
    rng = np.random.default_rng(4500 + hd + (dtype == "bf16"))
    cases = []
    for trial in range(3):
        B = int(rng.integers(1, 12))
        prefix = rng.integers(0, 400, size=B)
        e = rng.integers(1, 300 if trial < 2 else 700, size=B)
        cases.append(("random %d" % trial, prefix + e, e))
    for name, r in (("runs of 1", np.ones(160, np.int64)), ("runs of 1 to 3", rng.integers(1, 4, size=120)),
                    ("runs of 2 to 40", rng.integers(2, 41, size=40)), ("runs of 127", np.full(6, 127))):
        B = len(r)
        p0 = np.array([int(rng.integers(0, 128 - x)) if x < 127 else 0 for x in r]) + 128 * rng.integers(0, 3, B)
        cases.append((name, p0 + r, r))
    for name, s, e in cases:
        B = len(s)
        slots_n = B + 5
        idx = rng.permutation(slots_n)[:B]
        num_q = int(e.sum())
        inp, ape = _inputs(rng, num_q, hd, dtype)
        slots = _slots(rng, slots_n, hd)
        cap_c, cap_w = oracle.capacities(128, B, num_q)
        _, opw, oc = oracle.plan_prefill(128, s.astype(np.int32), e.astype(np.int32), idx.astype(np.int32),
                                         slots_n * 128, num_q, cap_c, cap_w)
        say("write from run list %s hd=%d %s B=%d num_w=%d" % (name, hd, dtype, B, oc[1]))
        st_o, err = oracle.write_online(hd, slots, inp, ape, opw, int(oc[1]))
        assert err == 0
        st_g, st_scan, c, pw = write_with_runs(hd, slots, inp, ape, s, e, idx, slots_n * 128, dev)
        assert c[2] == 0 and c[3] == 0, name
        touched = np.unique(oracle.unpack_w(opw[: oc[1]])[:, 1] // 128)
        assert_slots_close(st_g, st_o, touched, "write " + name)
        # the same two fold paths as the scan: the same bits
        assert np.array_equal(st_g.view(np.uint32), st_scan.view(np.uint32)), name
        untouched = np.setdiff1d(np.arange(slots_n), touched)
        assert np.array_equal(st_g[untouched].view(np.uint32), slots[untouched].view(np.uint32)), name


def test_write_from_run_list_full_size(dev):
    """The mixed prefill (64 requests, 125 792 tokens), bf16, hd 512: the slots written from the
    list equal the oracle's, and the scan path's bit for bit."""
    w = wl.mixed_prefill(128)
    hd = w.hd
    rng = np.random.default_rng(4601)
    slots = _slots(rng, w.B, hd)
    say("write from run list, full size: B=%d num_q=%d" % (w.B, w.num_q))
    pc, pw, counts, runs = gpu_plan(w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows, w.num_q, dev)
    inp, ape = to_dev(w.input, dev), to_dev(w.ape, dev)
    st_l = to_dev(slots, dev)
    st_s = to_dev(slots, dev)
    kvc.write_c128_online(hd, st_l, inp, ape, pw, counts, runs=runs)
    kvc.write_c128_online(hd, st_s, inp, ape, pw, counts)
    c = counts.cpu().numpy()
    assert c[2] == 0 and c[3] == 0
    opw = pw.cpu().numpy()
    assert np.array_equal(runs.cpu().numpy(), expected_runs(opw, int(c[1]), w.state_index))
    st_o, err = oracle.write_online(hd, slots, w.input, w.ape, opw, int(c[1]))
    assert err == 0
    touched = np.unique(oracle.unpack_w(opw[: c[1]])[:, 1] // 128)
    got = st_l.cpu().numpy()
    assert_slots_close(got, st_o, touched, "list")
    assert np.array_equal(got.view(np.uint32), st_s.cpu().numpy().view(np.uint32)), "list vs scan"


def test_online_chunk_with_run_list_under_graph_capture(dev):
    """plan_prefill with the run list, the online pool and the write from the list, captured in a
    HIP graph and replayed: every replay matches the eager chain bit for bit."""
    rng = np.random.default_rng(4801)
    hd, B = 512, 48
    prefix = rng.integers(0, 2000, size=B)
    e = rng.integers(1, 400, size=B)
    s = prefix + e
    num_q = int(e.sum())
    idx = rng.permutation(B + 4)[:B]
    inp_h, ape_h = _inputs(rng, num_q, hd, "bf16")
    inp, ape = to_dev(inp_h, dev), to_dev(ape_h, dev)
    slots0 = to_dev(_slots(rng, B + 4, hd), dev)
    s_d, e_d, i_d = (to_dev(np.asarray(x, np.int32), dev) for x in (s, e, idx))
    pc, pw, counts = kvc.alloc_prefill_plan(128, B, num_q, dev)
    runs = kvc.run_list(B, dev)
    out = torch.zeros((pc.shape[0], hd), dtype=torch.float32, device=dev)
    slots = slots0.clone()

    def chunk():
        kvc.plan_prefill(128, s_d, e_d, i_d, (B + 4) * 128, num_q, pc, pw, counts, runs=runs)
        kvc.compress_c128_online(hd, slots, inp, ape, pc, counts, out)
        kvc.write_c128_online(hd, slots, inp, ape, pw, counts, runs=runs)

    chunk()
    torch.cuda.synchronize()
    ref = (out.clone(), slots.clone(), runs.clone(), counts.clone())
    assert ref[3].tolist()[2:] == [0, 0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        slots.copy_(slots0)
        with torch.cuda.graph(g, stream=side):
            chunk()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        say("online chunk graph replay", rep)
        slots.copy_(slots0)
        out.fill_(float("nan"))
        runs.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(counts, ref[3]) and torch.equal(runs, ref[2])
        n = int(ref[3][0])  # rows past num_c are not written
        assert torch.equal(out[:n].view(torch.int32), ref[0][:n].view(torch.int32))
        assert torch.equal(slots.view(torch.int32), ref[1].view(torch.int32))


def test_write_from_run_list_errors(dev):
    """Entries the kernel cannot honour set KVC_DERR_RECORD and leave every slot untouched; a plan
    without W records (counts[1] == 0) writes nothing."""
    hd = 128
    rng = np.random.default_rng(4701)
    slots = _slots(rng, 2, hd)
    inp = to_dev(np.ones((8, 2 * hd), np.float32), dev)
    ape = to_dev(np.zeros((128, hd), np.float32), dev)
    pw = torch.zeros((8, kvc.W_BYTES), dtype=torch.uint8, device=dev)
    bad = {"slot out of range": (0, 5 * 128, 2), "past the block": (0, 127, 2), "rows past num_q": (6, 3, 3),
           "negative location": (0, -128, 1), "negative length": (0, 0, -1)}
    for name, (ragged, loc, n) in bad.items():
        runs = torch.tensor([[ragged, loc, n, 0]], dtype=torch.int32, device=dev)
        counts = torch.tensor([0, 8, 0, 0], dtype=torch.int32, device=dev)
        st = to_dev(slots, dev)
        kvc.write_c128_online(hd, st, inp, ape, pw, counts, runs=runs)
        assert counts.cpu().tolist()[3] == kvc.DERR_RECORD, name
        assert np.array_equal(st.cpu().numpy().view(np.uint32), slots.view(np.uint32)), name
    runs = torch.tensor([[0, 128, 3, 0]], dtype=torch.int32, device=dev)
    counts = torch.tensor([0, 0, 0, 0], dtype=torch.int32, device=dev)
    st = to_dev(slots, dev)
    kvc.write_c128_online(hd, st, inp, ape, pw, counts, runs=runs)
    assert counts.cpu().tolist() == [0, 0, 0, 0]
    assert np.array_equal(st.cpu().numpy().view(np.uint32), slots.view(np.uint32))


def test_binding_rejects_bad_run_lists(dev):
    s = torch.tensor([130], dtype=torch.int32, device=dev)
    e = torch.tensor([3], dtype=torch.int32, device=dev)
    idx = torch.tensor([0], dtype=torch.int32, device=dev)
    pc, pw, counts = kvc.alloc_prefill_plan(4, 1, 3, dev)
    with pytest.raises(kvc.KvcError):  # ratio 4 has no run list
        kvc.plan_prefill(4, s, e, idx, 8, 3, pc, pw, counts, runs=kvc.run_list(1, dev))
    pc, pw, counts = kvc.alloc_prefill_plan(128, 1, 3, dev)
    wrong_rows = torch.zeros((2, 4), dtype=torch.int32, device=dev)  # a list for two requests
    flat = torch.zeros(4, dtype=torch.int32, device=dev)
    wide = torch.zeros((1, 4), dtype=torch.int64, device=dev)
    strided = torch.zeros((1, 8), dtype=torch.int32, device=dev)[:, ::2]  # every other int32
    for bad in (wrong_rows, flat, wide, strided):
        with pytest.raises(kvc.KvcError):
            kvc.plan_prefill(128, s, e, idx, 128, 3, pc, pw, counts, runs=bad)
    for bad in (flat, wide, strided):  # the write takes the batch from the list itself
        with pytest.raises(kvc.KvcError):
            kvc.write_c128_online(128, torch.zeros((1, 3, 128), device=dev), torch.zeros((3, 256), device=dev),
                                  torch.zeros((128, 128), device=dev), pw, counts, runs=bad)
