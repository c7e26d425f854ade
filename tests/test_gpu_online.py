"""GPU parity of the online ratio-128 state against the oracle.

Slots are compared through what they mean: m within fp32 rounding of the
scores, and l, acc after rescaling to the oracle's m (a slot is determined up
to that shift), within 1e-5 relative.  Pooled rows use the pool bars of the
paged path: 1e-5 + 1e-5 |ref| for fp32 inputs, 2e-2 for bf16 inputs.  The
chunked runs from NaN-filled slots check that no slot is read before it is
written; the full-size run checks the online pool against the paged pool on
the same window contents.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import kvc  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402
from tests.chunked import OnlineBackend, OracleOnline, random_split, run_chunked  # noqa: E402

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


def assert_pool_close(got, ref, dtype, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all(), what
    tol = (1e-5 + 1e-5 * np.abs(ref)) if dtype == "f32" else np.full_like(ref, 2e-2)
    err = np.abs(got - ref)
    assert (err <= tol).all(), "%s: %d out of tolerance, max err %.3g" % (what, (err > tol).sum(), err.max())


def assert_slots_close(got, ref, rows, what=""):
    g, r = np.asarray(got, np.float64)[rows], np.asarray(ref, np.float64)[rows]
    assert np.isfinite(g).all(), what
    np.testing.assert_allclose(g[:, 0], r[:, 0], rtol=1e-6, atol=1e-6, err_msg=what + " m")
    f = np.exp(g[:, 0] - r[:, 0])  # rescale the GPU's sums to the oracle's maximum
    np.testing.assert_allclose(g[:, 1] * f, r[:, 1], rtol=1e-5, err_msg=what + " l")
    np.testing.assert_allclose(g[:, 2] * f, r[:, 2], rtol=1e-5, atol=1e-5 * np.abs(r[:, 1]).max(),
                               err_msg=what + " acc")


def _slots(rng, n, hd):
    s = np.empty((n, 3, hd), np.float32)
    s[:, 0] = rng.standard_normal((n, hd)) * 2
    s[:, 1] = rng.uniform(0.5, 40, size=(n, hd))
    s[:, 2] = rng.standard_normal((n, hd)) * s[:, 1]
    return s


SHAPES = [(512, "bf16"), (128, "f32"), (256, "bf16"), (512, "f32"), (128, "bf16")]


@pytest.mark.parametrize("hd,dtype", SHAPES)
def test_online_compress_and_write(gpu, hd, dtype):
    rng = np.random.default_rng(600 + hd + (dtype == "bf16"))
    for trial in range(3):
        B = int(rng.integers(1, 9))
        prefix = rng.integers(0, 400, size=B)
        e = rng.integers(1, 300 if trial < 2 else 700, size=B)
        s = (prefix + e).astype(np.int32)
        num_q = int(e.sum())
        idx = rng.permutation(B + 3)[:B].astype(np.int32)
        x = rng.standard_normal((num_q, 2 * hd)).astype(np.float32)
        inp = wl.to_bf16_bits(x) if dtype == "bf16" else x
        a = (0.1 * rng.standard_normal((128, hd))).astype(np.float32)
        ape = wl.to_bf16_bits(a) if dtype == "bf16" else a
        slots = _slots(rng, B + 3, hd)
        cap_c, cap_w = oracle.capacities(128, B, num_q)
        pc, pw, counts = oracle.plan_prefill(128, s, e, idx, (B + 3) * 128, num_q, cap_c + 2, cap_w + 2)
        say("online cr=128 hd=%d %s trial=%d B=%d num_q=%d num_c=%d num_w=%d" % (hd, dtype, trial, B, num_q,
                                                                                  counts[0], counts[1]))
        ref, err = oracle.compress_online(hd, slots, inp, ape, pc, counts[0])
        assert err == 0
        got, gerr = gpu.compress_online(hd, slots, inp, ape, pc, counts[0])
        assert gerr == 0
        n = int(counts[0])
        assert_pool_close(got[:n], ref[:n], dtype, "compress")
        assert np.isnan(got[n:]).all(), "rows past num_c must be untouched"
        st_o, err = oracle.write_online(hd, slots, inp, ape, pw, counts[1])
        assert err == 0
        st_g, gerr = gpu.write_online(hd, slots, inp, ape, pw, counts[1])
        assert gerr == 0
        touched = np.unique(oracle.unpack_w(pw[: counts[1]])[:, 1] // 128)
        assert_slots_close(st_g, st_o, touched, "write")
        untouched = np.setdiff1d(np.arange(B + 3), touched)
        assert np.array_equal(st_g[untouched].view(np.uint32), slots[untouched].view(np.uint32))


@pytest.mark.parametrize("hd,dtype", SHAPES)
def test_online_decode(gpu, hd, dtype):
    rng = np.random.default_rng(700 + hd + (dtype == "bf16"))
    for trial in range(3):
        B = int(rng.integers(1, 400))
        s = rng.integers(1, 600, size=B).astype(np.int32)
        if trial == 2:
            s = (rng.integers(1, 4, size=B) * 128).astype(np.int32)
        idx = rng.permutation(B).astype(np.int32)
        x = rng.standard_normal((B, 2 * hd)).astype(np.float32)
        inp = wl.to_bf16_bits(x) if dtype == "bf16" else x
        a = (0.1 * rng.standard_normal((128, hd))).astype(np.float32)
        ape = wl.to_bf16_bits(a) if dtype == "bf16" else a
        slots = _slots(rng, B, hd)
        pd, status = oracle.plan_decode(128, s, idx, B * 128)
        assert status == 0
        pd[rng.random(B) < 0.05] = 0xFF
        say("online decode hd=%d %s trial=%d B=%d" % (hd, dtype, trial, B))
        ref, st_o, err = oracle.decode_online(hd, slots, inp, ape, pd)
        got, st_g, gerr = gpu.decode_online(hd, slots, inp, ape, pd)
        assert err == gerr == 0
        assert_pool_close(got, ref, dtype, "decode")
        valid = oracle.unpack_d(pd)[:, 0].astype(np.int64) != 0xFFFFFFFF
        assert np.all(got[~valid] == 0) and np.all(got[valid & (s % 128 != 0)] == 0)
        assert_slots_close(st_g, st_o, idx[valid], "decode")


@pytest.mark.parametrize("hd,dtype", [(512, "bf16"), (128, "f32")])
def test_online_write_run_shapes(gpu, hd, dtype):
    """The state update where runs are short and many (every record a run of its own, so a
    32-record group holds up to 32 runs), where runs cross group boundaries, where a run fills a
    block up to its last open position (127 records) and where it continues a block that began
    in an earlier chunk: slots equal the oracle's, untouched slots stay bit-identical."""
    rng = np.random.default_rng(900 + hd)
    cases = {
        "runs of 1": np.ones(160, np.int64),
        "runs of 1 to 3": rng.integers(1, 4, size=120),
        "runs of 2 to 40": rng.integers(2, 41, size=40),
        "runs of 127": np.full(6, 127),
    }
    for name, runs in cases.items():
        B = len(runs)
        # a run is the chunk's positions after the block's last completed position: prefix p0 % 128 + run <= 127
        p0 = np.array([int(rng.integers(0, 128 - r)) if r < 127 else 0 for r in runs]) + 128 * rng.integers(0, 3, B)
        e = runs.astype(np.int32)
        s = (p0 + e).astype(np.int32)
        num_q = int(e.sum())
        slots_n = B + 5
        idx = rng.permutation(slots_n)[:B].astype(np.int32)
        x = rng.standard_normal((num_q, 2 * hd)).astype(np.float32)
        inp = wl.to_bf16_bits(x) if dtype == "bf16" else x
        a = (0.1 * rng.standard_normal((128, hd))).astype(np.float32)
        ape = wl.to_bf16_bits(a) if dtype == "bf16" else a
        slots = _slots(rng, slots_n, hd)
        cap_c, cap_w = oracle.capacities(128, B, num_q)
        pc, pw, counts = oracle.plan_prefill(128, s, e, idx, slots_n * 128, num_q, cap_c, cap_w)
        assert counts[2] == 0 and counts[1] == num_q, name  # every new token is written: no block closes
        say("online write %s hd=%d %s B=%d num_w=%d" % (name, hd, dtype, B, counts[1]))
        st_o, err = oracle.write_online(hd, slots, inp, ape, pw, counts[1])
        st_g, gerr = gpu.write_online(hd, slots, inp, ape, pw, counts[1])
        assert err == gerr == 0, name
        assert_slots_close(st_g, st_o, idx, "write " + name)
        untouched = np.setdiff1d(np.arange(slots_n), idx)
        assert np.array_equal(st_g[untouched].view(np.uint32), slots[untouched].view(np.uint32)), name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_online_chunked_prefill_then_decode(gpu, dtype):
    """Random chunkings and decode steps from NaN slots: the GPU emits the oracle's rows."""
    rng = np.random.default_rng(800 + (dtype == "bf16"))
    hd, B, steps = 128, 5, 140
    seqs, chunks = [], []
    for _ in range(B):
        L = int(rng.integers(1, 700))
        x = rng.standard_normal((L + steps, 2 * hd)).astype(np.float32)
        seqs.append(wl.to_bf16_bits(x) if dtype == "bf16" else x)
        chunks.append(random_split(rng, L, 5))
    a = (0.1 * rng.standard_normal((128, hd))).astype(np.float32)
    ape = wl.to_bf16_bits(a) if dtype == "bf16" else a
    idx = rng.permutation(7)[:B]
    nan_slots = np.full((7, 3, hd), np.nan)
    ref, _ = run_chunked(OnlineBackend(OracleOnline(oracle), ape), 128, hd, dtype, seqs, chunks, steps, idx, 7, ape,
                         state=nan_slots)
    got, _ = run_chunked(OnlineBackend(gpu, ape), 128, hd, dtype, seqs, chunks, steps, idx, 7, ape,
                         state=nan_slots.astype(np.float32))
    assert set(got) == set(ref)
    for key in ref:
        assert_pool_close(got[key], ref[key], dtype, str(key))


def test_online_record_errors(gpu):
    hd = 128
    inp = np.ones((8, 2 * hd), np.float32)
    ape = np.zeros((128, hd), np.float32)
    slots = _slots(np.random.default_rng(1), 2, hd)
    pc = np.full((2, 16), 0xFF, np.uint8)
    pc[0] = np.array([130, 3 | (125 << 24), 7, 7], np.uint32).view(np.uint8)  # continues slot 7 of 2
    out, err = gpu.compress_online(hd, slots, inp, ape, pc, 1)
    assert err == kvc.DERR_RECORD and np.isnan(out).all()
    pc[0] = np.array([200, 3 | (200 << 24), 0, 0], np.uint32).view(np.uint8)  # buffer_len above 127
    out, err = gpu.compress_online(hd, slots, inp, ape, pc, 1)
    assert err == kvc.DERR_RECORD and np.isnan(out).all()
    pw = np.zeros((2, 8), np.uint8)
    pw[0] = np.array([0, 5 * 128], np.uint32).view(np.uint8)
    pw[1] = np.array([1, 5 * 128 + 1], np.uint32).view(np.uint8)
    st, err = gpu.write_online(hd, slots, inp, ape, pw, 2)
    assert err == kvc.DERR_RECORD and np.array_equal(st.view(np.uint32), slots.view(np.uint32))
    pd = np.zeros((1, 16), np.uint8)
    pd[0] = np.array([5, 9 * 128 + 4, 9, 9], np.uint32).view(np.uint8)
    out, st, err = gpu.decode_online(hd, slots, inp[:1], ape, pd)
    assert err == kvc.DERR_RECORD and np.all(out == 0)


def test_online_matches_paged_pool_full_size(gpu):
    """The mixed prefill (64 requests, 125 792 tokens), ratio 128: slots built from the paged state's
    rows before each request's chunk; the online pool equals the paged pool on the same windows,
    and the written slots equal the oracle's."""
    from tests.gpu_backend import to_dev
    w = wl.mixed_prefill(128)
    hd = w.hd
    say("online full size: B=%d num_q=%d" % (w.B, w.num_q))
    state_f = (w.state.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ape_f = (w.ape.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    slots = np.full((w.B, 3, hd), np.nan, np.float32)
    for b in range(w.B):
        p0 = int(w.seq_lens[b] - w.extend_lens[b])
        q = p0 % 128
        if q == 0:
            continue
        rows = state_f[w.state_index[b] * 128 + np.arange(q)]
        t = rows[:, hd:] + ape_f[:q]
        m = t.max(axis=0)
        e = np.exp(t - m)
        slots[w.state_index[b]] = np.stack([m, e.sum(axis=0), (e * rows[:, :hd]).sum(axis=0)])
    plan_c, plan_w, counts = kvc.alloc_prefill_plan(128, w.B, w.num_q)
    kvc.plan_prefill(128, to_dev(w.seq_lens), to_dev(w.extend_lens), to_dev(w.state_index), w.num_state_rows,
                     w.num_q, plan_c, plan_w, counts)
    st_d, inp, ape = to_dev(slots), to_dev(w.input), to_dev(w.ape)
    out_online = torch.full((plan_c.shape[0], hd), float("nan"), dtype=torch.float32, device="cuda")
    out_paged = torch.full_like(out_online, float("nan"))
    kvc.compress_c128_online(hd, st_d, inp, ape, plan_c, counts, out_online)
    kvc.compress(128, hd, to_dev(w.state), inp, ape, plan_c, counts, out_paged)
    kvc.write_c128_online(hd, st_d, inp, ape, plan_w, counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert c[2] == 0 and c[3] == 0
    n = int(c[0])
    a, b = out_online[:n].cpu().numpy(), out_paged[:n].cpu().numpy()
    assert np.all(np.abs(a - b) <= 1e-5 + 1e-5 * np.abs(b)), "online vs paged pool"
    pc, pw = plan_c.cpu().numpy(), plan_w.cpu().numpy()
    ref, err = oracle.compress_online(hd, slots, w.input, w.ape, pc, n)
    assert err == 0
    assert_pool_close(a, ref[:n], "bf16", "online vs oracle")
    st_o, err = oracle.write_online(hd, slots, w.input, w.ape, pw, int(c[1]))
    assert err == 0
    touched = np.unique(oracle.unpack_w(pw[: c[1]])[:, 1] // 128)
    assert_slots_close(st_d.cpu().numpy(), st_o, touched, "write")
