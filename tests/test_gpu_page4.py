"""GPU parity of the ratio-4 planners over caller-allocated 4-row pages (Page4Align).

Plans, counts and status words are compared with the oracle byte for byte;
the chunked run (GPU plans feeding the GPU compress, write and decode) is
compared with the oracle's chunked run: pooled rows at the pool bars, the
state buffer bit for bit.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402
from tests.chunked import OracleBackend, Pages, random_split, run_chunked_page4  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_backend import GpuBackend
    return GpuBackend()


def _bundles(rng, s, e, n_pages, pages=None):
    """Pages for one chunk of every request: a fresh page for every block it touches."""
    pages = pages or Pages(rng, n_pages)
    idx, bundle = [], []
    for b in range(len(s)):
        p0, last = int(s[b] - e[b]), (int(s[b]) // 4) * 4
        idx.append(pages(b, last // 4))
        bundle.append((pages(b, (p0 - 1) // 4 - 1) if p0 > 4 else -1, pages(b, (p0 - 1) // 4) if p0 > 0 else -1,
                       pages(b, last // 4 - 1), last))
    return np.array(idx, np.int32), np.array(bundle, np.int32)


def _same(g, o):
    gpc, gpw, gc, gst = g
    opc, opw, oc, ost = o
    assert gc.tolist() == oc.tolist() and gst == ost, (gc, oc, gst, ost)
    assert np.array_equal(gpc, opc), "C records differ"
    assert np.array_equal(gpw, opw), "W records differ"


@pytest.mark.parametrize("kind", ["general", "uniform"])
def test_plan_prefill_page4_fuzz(gpu, kind):
    rng = np.random.default_rng(1100 + (kind == "uniform"))
    for case in range(40):
        B = int(rng.integers(1, 200))
        prefix = rng.integers(0, 3000, size=B)
        e = np.full(B, int(rng.integers(1, 33))) if kind == "uniform" else rng.integers(1, 400, size=B)
        s = (prefix + e).astype(np.int32)
        e = e.astype(np.int32)
        num_q = int(e.sum())
        n_pages = int((s // 4 + 3).sum()) + 8
        idx, bundle = _bundles(rng, s, e, n_pages)
        cap_c, cap_w = oracle.capacities(4, B, num_q)
        args = (s, e, idx, bundle, n_pages * 4, num_q, cap_c + 3, cap_w + 3)
        _same(gpu.plan_prefill_page4(*args), oracle.plan_prefill_page4(*args))


def test_plan_page4_errors(gpu):
    rng = np.random.default_rng(1200)
    B = 16
    s = rng.integers(9, 300, size=B).astype(np.int32)
    e = np.minimum(s, rng.integers(1, 60, size=B)).astype(np.int32)
    num_q = int(e.sum())
    n_pages = int((s // 4 + 3).sum())
    idx, bundle = _bundles(rng, s, e, n_pages)
    cap_c, cap_w = oracle.capacities(4, B, num_q)
    # a bad page index: plan error
    bad_idx = idx.copy()
    bad_idx[3] = n_pages
    args = (s, e, bad_idx, bundle, n_pages * 4, num_q, cap_c, cap_w)
    _same(gpu.plan_prefill_page4(*args), oracle.plan_prefill_page4(*args))
    # two requests on one page: plan error
    dup_idx = idx.copy()
    dup_idx[9] = dup_idx[2]
    args = (s, e, dup_idx, bundle, n_pages * 4, num_q, cap_c, cap_w)
    o = oracle.plan_prefill_page4(*args)
    assert o[2][2] == 32
    _same(gpu.plan_prefill_page4(*args), o)
    # bad bundle pages that records read or write: those records only
    bad = bundle.copy()
    bad[2, 1] = -3          # load_second_page
    bad[5, 0] = n_pages     # load_first_page
    bad[7, 2] = n_pages + 9  # write_first_page
    args = (s, e, idx, bad, n_pages * 4, num_q, cap_c, cap_w)
    o = oracle.plan_prefill_page4(*args)
    _same(gpu.plan_prefill_page4(*args), o)
    # decode: previous pages are checked only where they are read
    sd = np.array([4, 5, 8, 12, 16, 17], np.int32)
    pidx = np.arange(6, dtype=np.int32)
    prev = np.array([-1, -1, 99, 7, -1, -1], np.int32)
    for pr in (prev, np.abs(prev) % 10):
        g = gpu.plan_decode_page4(sd, pidx, pr, 40)
        o = oracle.plan_decode_page4(sd, pidx, pr, 40)
        assert g[1] == o[1] and np.array_equal(g[0], o[0])


def test_page4_wrappers_check_buffer_sizes(gpu):
    """A record buffer shorter than the batch, a table of the wrong length or an int64 table is
    refused by the binding before anything is launched (a short plan_d would take device writes
    past its end)."""
    from sparse_attention_kv_plan_amd import kvc
    from tests.gpu_backend import to_dev
    i32 = lambda a: to_dev(np.asarray(a, np.int32))  # noqa: E731
    s, idx, prev = i32([5, 8, 12]), i32([0, 1, 2]), i32([-1, 3, 4])
    short_d = torch.zeros((2, kvc.D_BYTES), dtype=torch.uint8, device="cuda")
    with pytest.raises(kvc.KvcError, match="plan_d"):
        kvc.plan_decode_page4(s, idx, prev, 40, short_d)
    pd = torch.zeros((3, kvc.D_BYTES), dtype=torch.uint8, device="cuda")
    with pytest.raises(kvc.KvcError, match="one entry per request"):
        kvc.plan_decode_page4(s, idx[:2], prev, 40, pd)
    with pytest.raises(kvc.KvcError, match="int32"):
        kvc.plan_decode_page4(s, idx.long(), prev, 40, pd)
    e = i32([5, 8, 12])
    bundle = i32(np.zeros((3, 4)))
    pc, pw, counts = kvc.alloc_prefill_plan(4, 3, 25, "cuda")
    with pytest.raises(kvc.KvcError, match="one entry per request"):
        kvc.plan_prefill_page4(s, e[:2], idx, bundle, 40, 25, pc, pw, counts)
    with pytest.raises(kvc.KvcError, match="plan_c"):
        kvc.plan_prefill_page4(s, e, idx, bundle, 40, 25, pc.view(-1), pw, counts)
    with pytest.raises(kvc.KvcError, match="int32"):
        kvc.plan_prefill_page4(s, e, idx, bundle, 40, 25, pc, pw, counts.long())
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,hd", [("bf16", 512), ("f32", 128)])
def test_page4_chunked_prefill_then_decode(gpu, dtype, hd):
    rng = np.random.default_rng(1300 + hd)
    B, steps = 5, 11
    seqs, chunks = [], []
    for _ in range(B):
        L = int(rng.integers(1, 120))
        x = rng.standard_normal((L + steps, 4 * hd)).astype(np.float32)
        seqs.append(wl.to_bf16_bits(x) if dtype == "bf16" else x)
        chunks.append(random_split(rng, L, 6))
    a = (0.1 * rng.standard_normal((8, hd))).astype(np.float32)
    ape = wl.to_bf16_bits(a) if dtype == "bf16" else a
    say("page4 chunked %s hd=%d" % (dtype, hd))
    ref, st_o = run_chunked_page4(OracleBackend(oracle), np.random.default_rng(5), hd, dtype, seqs, chunks, steps, ape,
                                  n_pages=300)
    got, st_g = run_chunked_page4(gpu, np.random.default_rng(5), hd, dtype, seqs, chunks, steps, ape, n_pages=300)
    assert set(got) == set(ref)
    for key in ref:
        g, r = np.asarray(got[key], np.float64), np.asarray(ref[key], np.float64)
        tol = (1e-5 + 1e-5 * np.abs(r)) if dtype == "f32" else 2e-2
        assert np.all(np.abs(g - r) <= tol), key
    assert np.array_equal(np.asarray(st_g).view(np.uint8), np.asarray(st_o).view(np.uint8)), "state differs"


def test_plan_prefill_page4_full_size(gpu):
    """The mixed prefill's 64 requests (125 792 tokens) with a page for every block."""
    w = wl.mixed_prefill(4, with_tensors=False)
    rng = np.random.default_rng(1400)
    n_pages = int((w.seq_lens // 4 + 3).sum())
    idx, bundle = _bundles(rng, w.seq_lens, w.extend_lens, n_pages)
    cap_c, cap_w = oracle.capacities(4, w.B, w.num_q)
    args = (w.seq_lens, w.extend_lens, idx, bundle, n_pages * 4, w.num_q, cap_c, cap_w)
    g, o = gpu.plan_prefill_page4(*args), oracle.plan_prefill_page4(*args)
    _same(g, o)
    assert o[2][0] > 30000 and o[2][2] == 0
