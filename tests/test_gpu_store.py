"""GPU parity of the norm + rotary embedding + bf16 store step against the oracle.

Both the standalone calls (float32 rows already in HBM) and the calls fused
into the prefill pools are compared with the oracle (float64).  Bar, per
stored channel: |gpu - ref| <= 2^-7 |ref| + 2^-12 max|ref row|.  The store
rounds an fp32 value to bf16 (8 significand bits: half an ulp is at most
2^-8 of the value), and the fp32 value itself is off by ~1e-6 relative, so
one bf16 ulp (2^-7) bounds the rounded result.  The absolute term covers
channels near zero, whose error is the fp32 error of the row: pooling error
(~1e-6 of the largest kv, for the fused calls) enlarged by the norm's
1 / rms, and cancellation inside a rotated pair.  The GPU pools read the
same input bits as the oracle, so the bar is the same for bf16 and fp32
inputs.
Which cache rows are written is compared exactly: the cache starts filled
with 0xFFFF, a bit pattern the store never produces.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import kvc  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu

W = {4: 8, 128: 128}
UNTOUCHED = 0xFFFF


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.load()
    return "cuda"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _store_tensors(si, hd):
    cache = torch.full((si.num_cache_rows, hd), -1, dtype=torch.int16, device="cuda")  # 0xFFFF
    return dev(si.norm_weight), dev(si.freqs_cis) if si.freqs_cis.size else None, dev(si.out_loc), cache


def _cache_host(cache):
    return cache.cpu().numpy().view(np.uint16)


def assert_store_close(bits, ref, what=""):
    """bits: uint16 [rows, hd] from the GPU; ref: float64 [rows, hd], NaN rows = not stored."""
    stored_ref = ~np.isnan(ref).all(axis=1)
    stored_gpu = ~(bits == UNTOUCHED).all(axis=1)
    assert np.array_equal(stored_ref, stored_gpu), "%s: stored rows differ (%d vs %d)" % (
        what, stored_ref.sum(), stored_gpu.sum())
    assert not (bits[stored_gpu] == UNTOUCHED).any(), what
    got = wl.bf16_bits_to_f32(bits[stored_gpu]).astype(np.float64)
    r = ref[stored_ref]
    assert np.isfinite(got).all(), what
    tol = 2.0 ** -7 * np.abs(r) + 2.0 ** -12 * np.abs(r).max(axis=1, keepdims=True)
    err = np.abs(got - r)
    bad = err > tol
    assert not bad.any(), "%s: %d channels out of tolerance, max err %.3g" % (what, bad.sum(), err.max())


def _prefill_case(rng, cr, B, extend_hi):
    s = rng.integers(1, 4 * W[cr], size=B) + rng.integers(0, extend_hi, size=B)
    e = np.minimum(s, rng.integers(1, extend_hi + 1, size=B))
    num_q = int(e.sum())
    cap_c, cap_w = oracle.capacities(cr, B, num_q)
    pc, pw, counts = oracle.plan_prefill(cr, s, e, rng.permutation(B), B * W[cr], num_q, cap_c + 3, cap_w)
    return s, e, num_q, pc, pw, counts


STORE_SHAPES = [(4, 512, 64), (128, 512, 64), (4, 128, 64), (128, 128, 128), (4, 256, 8), (128, 256, 0),
                (4, 128, 0), (128, 512, 512)]


@pytest.mark.parametrize("cr,hd,rope_dim", STORE_SHAPES)
def test_norm_rope_store_prefill(gpu, cr, hd, rope_dim):
    rng = np.random.default_rng(100 + cr + hd + rope_dim)
    for trial in range(3):
        B = int(rng.integers(1, 12))
        s, e, num_q, pc, _, counts = _prefill_case(rng, cr, B, 3 * W[cr] if trial < 2 else 900)
        n = int(counts[0])
        say("store prefill cr=%d hd=%d rope=%d trial=%d num_q=%d num_c=%d" % (cr, hd, rope_dim, trial, num_q, n))
        rows = (rng.standard_normal((pc.shape[0], hd)) * rng.uniform(0.05, 4, size=(pc.shape[0], 1))).astype(
            np.float32)
        si = wl.store_inputs(rng, hd, rope_dim, int(s.max()) + 1, num_q)
        ref, err = oracle.store_prefill(cr, rows, pc, n, si.norm_weight, si.eps, si.freqs_cis, si.out_loc,
                                        np.full((si.num_cache_rows, hd), np.nan))
        assert err == 0
        w, f, loc, cache = _store_tensors(si, hd)
        cnt = dev(np.array([n, 0, 0, 0], np.int32))
        kvc.norm_rope_store_prefill(cr, dev(rows), dev(pc), cnt, w, si.eps, f, loc, cache)
        assert int(cnt[3].item()) == 0
        assert_store_close(_cache_host(cache), ref, "store prefill")


@pytest.mark.parametrize("cr,hd,rope_dim", STORE_SHAPES)
def test_norm_rope_store_decode(gpu, cr, hd, rope_dim):
    rng = np.random.default_rng(200 + cr + hd + rope_dim)
    for trial in range(3):
        B = int(rng.integers(1, 600))
        s = rng.integers(1, 4 * cr, size=B).astype(np.int32)
        if trial == 1:
            s = (rng.integers(1, 4, size=B) * cr).astype(np.int32)  # all on a boundary, first block included
        pd, status = oracle.plan_decode(cr, s, rng.permutation(B), B * W[cr])
        assert status == 0
        pd[rng.random(B) < 0.1] = 0xFF  # invalid records store nothing
        say("store decode cr=%d hd=%d rope=%d trial=%d B=%d" % (cr, hd, rope_dim, trial, B))
        rows = rng.standard_normal((B, hd)).astype(np.float32)
        si = wl.store_inputs(rng, hd, rope_dim, 4 * cr, B)
        ref, err = oracle.store_decode(cr, rows, pd, si.norm_weight, si.eps, si.freqs_cis, si.out_loc,
                                       np.full((si.num_cache_rows, hd), np.nan))
        assert err == 0
        w, f, loc, cache = _store_tensors(si, hd)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        kvc.norm_rope_store_decode(cr, dev(rows), dev(pd), w, si.eps, f, loc, cache, st)
        assert int(st.item()) == 0
        assert_store_close(_cache_host(cache), ref, "store decode")


FUSED_SHAPES = [(4, 512, "bf16", 64), (4, 128, "f32", 64), (4, 512, "f32", 64), (4, 256, "bf16", 0),
                (4, 128, "bf16", 128), (128, 512, "bf16", 64), (128, 128, "f32", 8), (128, 256, "bf16", 256),
                (128, 512, "f32", 0)]


@pytest.mark.parametrize("cr,hd,dtype,rope_dim", FUSED_SHAPES)
def test_compress_norm_rope_store(gpu, cr, hd, dtype, rope_dim):
    """The fused pool + store against the oracle's pool followed by its store, and against
    the GPU's own two-call sequence (pool into float32 rows, then the standalone store)."""
    rng = np.random.default_rng(300 + cr + hd + rope_dim + (dtype == "bf16"))
    for trial in range(3):
        B = int(rng.integers(1, 9))
        w = wl.random_prefill(rng, cr, hd, dtype, B, prefix_hi=3 * W[cr], extend_lo=1,
                              extend_hi=3 * W[cr] if trial < 2 else 700, num_slots=B + 3)
        cap_c, cap_w = oracle.capacities(cr, B, w.num_q)
        pc, _, counts = oracle.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                            w.num_q, cap_c + 2, cap_w)
        n = int(counts[0])
        say("fused cr=%d hd=%d %s rope=%d trial=%d num_q=%d num_c=%d" % (cr, hd, dtype, rope_dim, trial, w.num_q,
                                                                          n))
        pooled, err = oracle.compress(cr, hd, w.state, w.input, w.ape, pc, n)
        assert err == 0
        si = wl.store_inputs(rng, hd, rope_dim, int(w.seq_lens.max()) + 1, w.num_q)
        ref, err = oracle.store_prefill(cr, pooled.astype(np.float32), pc, n, si.norm_weight, si.eps,
                                        si.freqs_cis, si.out_loc, np.full((si.num_cache_rows, hd), np.nan))
        assert err == 0
        wt, f, loc, cache = _store_tensors(si, hd)
        cnt = dev(np.array([n, 0, 0, 0], np.int32))
        state, inp, ape, pcd = dev(w.state), dev(w.input), dev(w.ape), dev(pc)
        kvc.compress_norm_rope_store(cr, hd, state, inp, ape, pcd, cnt, wt, si.eps, f, loc, cache)
        assert int(cnt[3].item()) == 0
        fused = _cache_host(cache)
        assert_store_close(fused, ref, "fused")
        # the two-call GPU sequence pools to the same bits and normalises with another
        # summation order: the stored values differ by at most one bf16 ulp
        out = torch.full((pc.shape[0], hd), float("nan"), dtype=torch.float32, device="cuda")
        kvc.compress(cr, hd, state, inp, ape, pcd, cnt, out)
        cache2 = torch.full_like(cache, -1)
        kvc.norm_rope_store_prefill(cr, out, pcd, cnt, wt, si.eps, f, loc, cache2)
        two = _cache_host(cache2)
        assert np.array_equal(fused == UNTOUCHED, two == UNTOUCHED)
        m = fused != UNTOUCHED
        a = wl.bf16_bits_to_f32(fused[m]).astype(np.float64)
        b = wl.bf16_bits_to_f32(two[m]).astype(np.float64)
        assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-6), "fused vs two calls"


def test_store_errors(gpu):
    """Records whose key, location or position is out of range are skipped and reported."""
    hd, cr, rope_dim = 128, 4, 64
    rng = np.random.default_rng(9)
    fields = [(8, 0, 0, 0, 0), (12, 1, 0, 0, 0), (16, 2, 0, 0, 0), (64, 3, 0, 0, 0), (20, 4, 0, 0, 0)]
    pc = np.full((6, 16), 0xFF, np.uint8)
    for k, (s, rag, blen, rp0, rp1) in enumerate(fields):
        pc[k] = np.array([s, rag | (blen << 24), rp0, rp1], np.uint32).view(np.uint8)
    rows = rng.standard_normal((6, hd)).astype(np.float32)
    # ragged 1 -> location 99, outside the 8-row cache; ragged 3 closes at 64 -> position 60,
    # beyond the 40-row table.  First with out_loc cut to 2 entries: ragged 2..4 have no entry.
    out_loc = np.array([0, 99, 5, 6, 3], np.int32)
    freqs = wl.rope_table(40, rope_dim)
    wgt = np.ones(hd, np.float32)
    ref, err = oracle.store_prefill(cr, rows, pc, 5, wgt, 1e-6, freqs, out_loc[:2], np.full((8, hd), np.nan))
    assert err == kvc.DERR_RECORD
    cache = torch.full((8, hd), -1, dtype=torch.int16, device="cuda")
    cnt = dev(np.array([5, 0, 0, 0], np.int32))
    kvc.norm_rope_store_prefill(cr, dev(rows), dev(pc), cnt, dev(wgt), 1e-6, dev(freqs), dev(out_loc[:2]), cache)
    assert int(cnt[3].item()) == kvc.DERR_RECORD
    assert_store_close(_cache_host(cache), ref, "errors")
    # the same out_loc with all five entries: only the location and the position are bad
    ref, err = oracle.store_prefill(cr, rows, pc, 5, wgt, 1e-6, freqs, out_loc, np.full((8, hd), np.nan))
    assert err == kvc.DERR_RECORD
    cache.fill_(-1)
    cnt = dev(np.array([5, 0, 0, 0], np.int32))
    kvc.norm_rope_store_prefill(cr, dev(rows), dev(pc), cnt, dev(wgt), 1e-6, dev(freqs), dev(out_loc), cache)
    assert int(cnt[3].item()) == kvc.DERR_RECORD
    bits = _cache_host(cache)
    assert_store_close(bits, ref, "errors 2")
    assert (~(bits == UNTOUCHED).all(axis=1)).sum() == 3
    # decode: status word
    pd = np.zeros((3, 16), np.uint8)
    for b, s in enumerate([8, 8, 12]):
        pd[b, :4] = np.array([s], np.uint32).view(np.uint8)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache.fill_(-1)
    kvc.norm_rope_store_decode(cr, dev(rows[:3]), dev(pd), dev(wgt), 1e-6, dev(freqs), dev(np.array([1, 99, 2],
                               np.int32)), cache, st)
    assert int(st.item()) == kvc.DERR_RECORD
    bits = _cache_host(cache)
    assert [int(~(bits[r] == UNTOUCHED).all()) for r in range(8)] == [0, 1, 1, 0, 0, 0, 0, 0]


@pytest.mark.parametrize("cr", [4, 128])
def test_fused_store_record_errors(gpu, cr):
    """The fused kernels report bad store targets in counts[3] and store nothing for them."""
    hd = 512
    rng = np.random.default_rng(40 + cr)
    w = wl.random_prefill(rng, cr, hd, "bf16", 4, prefix_hi=2 * W[cr], extend_lo=W[cr], extend_hi=3 * W[cr],
                          num_slots=7)
    cap_c, cap_w = oracle.capacities(cr, 4, w.num_q)
    pc, _, counts = oracle.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows, w.num_q,
                                        cap_c, cap_w)
    n = int(counts[0])
    assert n >= 2
    si = wl.store_inputs(rng, hd, 64, int(w.seq_lens.max()) + 1, w.num_q)
    rag = oracle.unpack_c(pc[:n])[:, 1]
    si.out_loc[rag[0]] = si.num_cache_rows + 5  # outside the cache
    wt, f, loc, cache = _store_tensors(si, hd)
    cnt = dev(np.array([n, 0, 0, 0], np.int32))
    kvc.compress_norm_rope_store(cr, hd, dev(w.state), dev(w.input), dev(w.ape), dev(pc), cnt, wt, si.eps, f, loc,
                                 cache)
    assert int(cnt[3].item()) == kvc.DERR_RECORD
    bits = _cache_host(cache)
    stored = ~(bits == UNTOUCHED).all(axis=1)
    assert stored.sum() == n - 1
    assert stored[si.out_loc[rag[1:]]].all()


# --------------------------------------------------------------------------
# the named workloads at full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cr", [4, 128])
def test_mixed_prefill_fused_store_full_size(gpu, cr):
    """64 requests, 125,792 tokens: GPU plan -> fused pool + store, against the oracle's pool + store."""
    w = wl.mixed_prefill(cr)
    say("fused store workload %s: B=%d num_q=%d" % (w.name, w.B, w.num_q))
    plan_c, plan_w, counts = kvc.alloc_prefill_plan(cr, w.B, w.num_q)
    kvc.plan_prefill(cr, dev(w.seq_lens), dev(w.extend_lens), dev(w.state_index), w.num_state_rows, w.num_q,
                     plan_c, plan_w, counts)
    rng = np.random.default_rng(1005)
    si = wl.store_inputs(rng, w.hd, 64, int(w.seq_lens.max()) + 1, w.num_q)
    wt, f, loc, cache = _store_tensors(si, w.hd)
    kvc.compress_norm_rope_store(cr, w.hd, dev(w.state), dev(w.input), dev(w.ape), plan_c, counts, wt, si.eps, f,
                                 loc, cache)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert c[2] == 0 and c[3] == 0
    pc = plan_c.cpu().numpy()
    n = int(c[0])
    pooled, err = oracle.compress(cr, w.hd, w.state, w.input, w.ape, pc, n)
    assert err == 0
    ref, err = oracle.store_prefill(cr, pooled.astype(np.float32), pc, n, si.norm_weight, si.eps, si.freqs_cis,
                                    si.out_loc, np.full((si.num_cache_rows, w.hd), np.nan))
    assert err == 0
    assert_store_close(_cache_host(cache), ref, w.name)


@pytest.mark.parametrize("cr", [4, 128])
def test_mixed_prefill_standalone_store_full_size(gpu, cr):
    """64 requests, 125,792 tokens: GPU plan -> GPU pool into fp32 rows -> standalone store (the
    launch that gives each lane group several rows), against the oracle's store of the same fp32
    rows; every other cache row stays untouched."""
    w = wl.mixed_prefill(cr)
    say("standalone store workload %s: B=%d num_q=%d" % (w.name, w.B, w.num_q))
    plan_c, plan_w, counts = kvc.alloc_prefill_plan(cr, w.B, w.num_q)
    kvc.plan_prefill(cr, dev(w.seq_lens), dev(w.extend_lens), dev(w.state_index), w.num_state_rows, w.num_q,
                     plan_c, plan_w, counts)
    rows = torch.full((plan_c.shape[0], w.hd), float("nan"), dtype=torch.float32, device="cuda")
    kvc.compress(cr, w.hd, dev(w.state), dev(w.input), dev(w.ape), plan_c, counts, rows)
    rng = np.random.default_rng(2005 + cr)
    si = wl.store_inputs(rng, w.hd, 64, int(w.seq_lens.max()) + 1, w.num_q)
    wt, f, loc, cache = _store_tensors(si, w.hd)
    kvc.norm_rope_store_prefill(cr, rows, plan_c, counts, wt, si.eps, f, loc, cache)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert c[2] == 0 and c[3] == 0
    n = int(c[0])
    ref, err = oracle.store_prefill(cr, rows.cpu().numpy(), plan_c.cpu().numpy(), n, si.norm_weight, si.eps,
                                    si.freqs_cis, si.out_loc, np.full((si.num_cache_rows, w.hd), np.nan))
    assert err == 0
    assert_store_close(_cache_host(cache), ref, w.name)


@pytest.mark.parametrize("name", ["c4_decode_b256", "c128_decode_b1024"])
def test_decode_store_full_size(gpu, name):
    w = wl.c4_decode_b256() if name == "c4_decode_b256" else wl.c128_decode_b1024()
    say("decode store workload %s: B=%d" % (w.name, w.B))
    plan_d = torch.empty((w.B, kvc.D_BYTES), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    state = dev(w.state)
    out = torch.empty((w.B, w.hd), dtype=torch.float32, device="cuda")
    kvc.plan_decode(w.cr, dev(w.seq_lens), dev(w.state_index), w.num_state_rows, plan_d, status)
    kvc.decode(w.cr, w.hd, state, dev(w.input), dev(w.ape), plan_d, out, status)
    rng = np.random.default_rng(1003)
    si = wl.store_inputs(rng, w.hd, 64, int(w.seq_lens.max()) + 1, w.B)
    wt, f, loc, cache = _store_tensors(si, w.hd)
    kvc.norm_rope_store_decode(w.cr, out, plan_d, wt, si.eps, f, loc, cache, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref, err = oracle.store_decode(w.cr, out.cpu().numpy(), plan_d.cpu().numpy(), si.norm_weight, si.eps,
                                   si.freqs_cis, si.out_loc, np.full((si.num_cache_rows, w.hd), np.nan))
    assert err == 0
    assert_store_close(_cache_host(cache), ref, name)


DECODE_FUSED = [(512, "bf16", 64), (128, "f32", 64), (512, "f32", 64), (256, "bf16", 0), (128, "bf16", 128)]


@pytest.mark.parametrize("hd,dtype,rope_dim", DECODE_FUSED)
def test_decode_c4_norm_rope_store(gpu, hd, dtype, rope_dim):
    """The fused ratio-4 decode + store against the oracle's decode followed by its store; the
    state after the step is compared bit for bit."""
    rng = np.random.default_rng(400 + hd + rope_dim + (dtype == "bf16"))
    for trial in range(3):
        B = int(rng.integers(1, 300))
        w = wl.random_decode(rng, 4, hd, dtype, B, prefix_hi=24, num_slots=B + 2)
        if trial == 2:  # every request closes a block, the first block included
            w.seq_lens = (rng.integers(1, 4, size=B) * 4).astype(np.int32)
        pd, status = oracle.plan_decode(4, w.seq_lens, w.state_index, w.num_state_rows)
        assert status == 0
        say("fused decode hd=%d %s rope=%d trial=%d B=%d boundaries=%d" % (hd, dtype, rope_dim, trial, B,
                                                                           int((w.seq_lens % 4 == 0).sum())))
        st_o = w.state.copy()
        pooled, err = oracle.decode(4, hd, st_o, w.input, w.ape, pd)
        assert err == 0
        si = wl.store_inputs(rng, hd, rope_dim, int(w.seq_lens.max()) + 1, B)
        ref, err = oracle.store_decode(4, pooled.astype(np.float32), pd, si.norm_weight, si.eps, si.freqs_cis,
                                       si.out_loc, np.full((si.num_cache_rows, hd), np.nan))
        assert err == 0
        wt, f, loc, cache = _store_tensors(si, hd)
        state = dev(w.state)
        stt = torch.zeros(1, dtype=torch.int32, device="cuda")
        kvc.decode_c4_norm_rope_store(hd, state, dev(w.input), dev(w.ape), dev(pd), wt, si.eps, f, loc, cache, stt)
        assert int(stt.item()) == 0
        assert_store_close(_cache_host(cache), ref, "fused decode")
        got_state = state.cpu().numpy()
        assert np.array_equal(got_state.view(np.uint8), st_o.view(np.uint8)), "state differs after the step"


def test_decode_c4_norm_rope_store_bad_target(gpu):
    """A boundary request whose location is out of range: its token still reaches the state,
    its row is not stored, and the status word says so."""
    hd = 512
    rng = np.random.default_rng(77)
    w = wl.random_decode(rng, 4, hd, "bf16", 16, prefix_hi=24, num_slots=18)
    w.seq_lens = (rng.integers(1, 4, size=16) * 4).astype(np.int32)
    pd, _ = oracle.plan_decode(4, w.seq_lens, w.state_index, w.num_state_rows)
    st_o = w.state.copy()
    pooled, _ = oracle.decode(4, hd, st_o, w.input, w.ape, pd)
    si = wl.store_inputs(rng, hd, 64, int(w.seq_lens.max()) + 1, 16)
    si.out_loc[5] = si.num_cache_rows  # one past the end
    ref, err = oracle.store_decode(4, pooled.astype(np.float32), pd, si.norm_weight, si.eps, si.freqs_cis, si.out_loc,
                                   np.full((si.num_cache_rows, hd), np.nan))
    assert err == kvc.DERR_RECORD
    wt, f, loc, cache = _store_tensors(si, hd)
    state = dev(w.state)
    stt = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.decode_c4_norm_rope_store(hd, state, dev(w.input), dev(w.ape), dev(pd), wt, si.eps, f, loc, cache, stt)
    assert int(stt.item()) == kvc.DERR_RECORD
    assert_store_close(_cache_host(cache), ref, "bad target")
    assert np.array_equal(state.cpu().numpy().view(np.uint8), st_o.view(np.uint8))


def test_decode_c4_norm_rope_store_full_size(gpu):
    """256 requests, prefixes up to 32768: the fused step against decode + standalone store on the GPU
    and against the oracle."""
    w = wl.c4_decode_b256()
    say("fused decode store workload %s: B=%d" % (w.name, w.B))
    plan_d = torch.empty((w.B, kvc.D_BYTES), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.plan_decode(4, dev(w.seq_lens), dev(w.state_index), w.num_state_rows, plan_d, status)
    si = wl.store_inputs(np.random.default_rng(1013), w.hd, 64, int(w.seq_lens.max()) + 1, w.B)
    wt, f, loc, cache = _store_tensors(si, w.hd)
    state = dev(w.state)
    kvc.decode_c4_norm_rope_store(w.hd, state, dev(w.input), dev(w.ape), plan_d, wt, si.eps, f, loc, cache, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    pd = plan_d.cpu().numpy()
    st_o = w.state.copy()
    pooled, err = oracle.decode(4, w.hd, st_o, w.input, w.ape, pd)
    assert err == 0
    ref, err = oracle.store_decode(4, pooled.astype(np.float32), pd, si.norm_weight, si.eps, si.freqs_cis,
                                   si.out_loc, np.full((si.num_cache_rows, w.hd), np.nan))
    assert err == 0
    assert_store_close(_cache_host(cache), ref, w.name)
    assert np.array_equal(state.cpu().numpy().view(np.uint8), st_o.view(np.uint8))


def test_store_paths_under_graph_capture(gpu):
    """A prefill chunk with the fused store (plan, pool + store, write) and a fused ratio-4 decode step,
    captured in one HIP graph and replayed: every replay matches the eager run bit for bit."""
    rng = np.random.default_rng(23)
    w = wl.random_prefill(rng, 4, 512, "bf16", 8, prefix_hi=500, extend_lo=1, extend_hi=700, num_slots=12)
    d = wl.random_decode(rng, 4, 512, "bf16", 64, prefix_hi=40, num_slots=64)
    s_d, e_d, i_d = dev(w.seq_lens), dev(w.extend_lens), dev(w.state_index)
    inp, ape, state0 = dev(w.input), dev(w.ape), dev(w.state)
    d_inp, d_ape, d_state0 = dev(d.input), dev(d.ape), dev(d.state)
    plan_c, plan_w, counts = kvc.alloc_prefill_plan(4, w.B, w.num_q)
    plan_d = torch.empty((d.B, kvc.D_BYTES), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    si = wl.store_inputs(rng, 512, 64, int(max(w.seq_lens.max(), d.seq_lens.max())) + 1, max(w.num_q, d.B))
    wt, f, loc, cache = _store_tensors(si, 512)
    state, d_state = state0.clone(), d_state0.clone()

    def step():
        kvc.plan_prefill(4, s_d, e_d, i_d, w.num_state_rows, w.num_q, plan_c, plan_w, counts)
        kvc.compress_norm_rope_store(4, 512, state, inp, ape, plan_c, counts, wt, si.eps, f, loc, cache)
        kvc.write(4, 512, state, inp, plan_w, counts)
        kvc.plan_decode(4, dev_d_seq, dev_d_idx, d.num_state_rows, plan_d, status)
        kvc.decode_c4_norm_rope_store(512, d_state, d_inp, d_ape, plan_d, wt, si.eps, f, loc[:d.B], cache, status)

    dev_d_seq, dev_d_idx = dev(d.seq_lens), dev(d.state_index)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (cache, state, d_state, counts, status)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        say("store graph replay", rep)
        state.copy_(state0)
        d_state.copy_(d_state0)
        cache.fill_(-1)
        counts.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((cache, state, d_state, counts, status), ref):
            assert torch.equal(got, want)


STORE_FUZZ_CASES = 120


def store_fuzz_case(rng):
    """One random store case (the four calls in turn: standalone prefill and decode stores, the
    fused prefill pools, the fused ratio-4 decode); checks the GPU against the oracle."""
    kind = str(rng.choice(["prefill", "decode", "fused", "fused_decode"]))
    cr = 4 if kind == "fused_decode" else int(rng.choice([4, 128]))
    hd = int(rng.choice([128, 256, 512]))
    dtype = str(rng.choice(["f32", "bf16"]))
    rope_dim = int(rng.choice([0, 8, 64, hd // 2, hd]))
    eps = float(rng.choice([1e-6, 1e-3, 0.0]))
    label = "store fuzz %s cr=%d hd=%d %s rope=%d eps=%g" % (kind, cr, hd, dtype, rope_dim, eps)
    if kind in ("prefill", "fused"):
        B = int(rng.integers(1, 10))
        w = wl.random_prefill(rng, cr, hd, dtype, B, prefix_hi=3 * W[cr], extend_lo=1,
                              extend_hi=int(rng.choice([3 * W[cr], 700])), num_slots=B + 2)
        cap_c, cap_w = oracle.capacities(cr, B, w.num_q)
        pc, _, counts = oracle.plan_prefill(cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                            w.num_q, cap_c + int(rng.integers(0, 3)), cap_w)
        n = int(counts[0])
        si = wl.store_inputs(rng, hd, rope_dim, int(w.seq_lens.max()) + 1, w.num_q, eps=eps)
        if kind == "prefill":
            rows = (rng.standard_normal((pc.shape[0], hd)) * rng.uniform(0.05, 4, size=(pc.shape[0], 1))).astype(
                np.float32)
        else:
            pooled, err = oracle.compress(cr, hd, w.state, w.input, w.ape, pc, n)
            assert err == 0
            rows = np.zeros((pc.shape[0], hd), np.float32)
            rows[:n] = pooled[:n]
        say("%s B=%d num_c=%d" % (label, B, n))
        ref, err = oracle.store_prefill(cr, rows, pc, n, si.norm_weight, si.eps, si.freqs_cis, si.out_loc,
                                        np.full((si.num_cache_rows, hd), np.nan))
        assert err == 0
        wt, f, loc, cache = _store_tensors(si, hd)
        cnt = dev(np.array([n, 0, 0, 0], np.int32))
        if kind == "prefill":
            kvc.norm_rope_store_prefill(cr, dev(rows), dev(pc), cnt, wt, si.eps, f, loc, cache)
        else:
            kvc.compress_norm_rope_store(cr, hd, dev(w.state), dev(w.input), dev(w.ape), dev(pc), cnt, wt, si.eps,
                                         f, loc, cache)
        assert int(cnt[3].item()) == 0, label
        assert_store_close(_cache_host(cache), ref, label)
        return
    B = int(rng.integers(1, 400))
    w = wl.random_decode(rng, cr, hd, dtype, B, prefix_hi=3 * cr, num_slots=B + 2)
    pd, status = oracle.plan_decode(cr, w.seq_lens, w.state_index, w.num_state_rows)
    assert status == 0
    si = wl.store_inputs(rng, hd, rope_dim, int(w.seq_lens.max()) + 1, B, eps=eps)
    say("%s B=%d boundaries=%d" % (label, B, int((w.seq_lens % cr == 0).sum())))
    wt, f, loc, cache = _store_tensors(si, hd)
    stt = torch.zeros(1, dtype=torch.int32, device="cuda")
    if kind == "decode":
        rows = rng.standard_normal((B, hd)).astype(np.float32)
        ref, err = oracle.store_decode(cr, rows, pd, si.norm_weight, si.eps, si.freqs_cis, si.out_loc,
                                       np.full((si.num_cache_rows, hd), np.nan))
        assert err == 0
        kvc.norm_rope_store_decode(cr, dev(rows), dev(pd), wt, si.eps, f, loc, cache, stt)
    else:
        st_o = w.state.copy()
        pooled, err = oracle.decode(4, hd, st_o, w.input, w.ape, pd)
        assert err == 0
        ref, err = oracle.store_decode(4, pooled.astype(np.float32), pd, si.norm_weight, si.eps, si.freqs_cis,
                                       si.out_loc, np.full((si.num_cache_rows, hd), np.nan))
        assert err == 0
        state = dev(w.state)
        kvc.decode_c4_norm_rope_store(hd, state, dev(w.input), dev(w.ape), dev(pd), wt, si.eps, f, loc, cache, stt)
        assert np.array_equal(state.cpu().numpy().view(np.uint8), st_o.view(np.uint8)), label
    assert int(stt.item()) == 0, label
    assert_store_close(_cache_host(cache), ref, label)


def test_random_store_cases(gpu):
    for case in range(STORE_FUZZ_CASES):
        store_fuzz_case(np.random.default_rng([2026, case]))
