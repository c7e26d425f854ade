"""GPU parity on random chunkings: ratio, head_dim, dtype, batch, the split of every request into
prefill chunks and the number of decode steps all drawn from a fixed seed; for the per-request
ring and page, and for the SWA-paged rings, the online ratio-128 slots and the caller's 4-row
pages.  Every emitted row is
compared with the oracle's (fp32 bar 1e-5 + 1e-5 |ref|, bf16 bar 2e-2) and the state buffer after
the last step bit for bit.

Inputs of either dtype take scores and values of the configs' size and 2, 3 and 30 times larger
(fp32: the pool runs in float64, so the bar holds at every scale; bf16: bar 2e-2)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402
from tests.chunked import (OnlineBackend, OracleBackend, OracleOnline, random_split, run_chunked,  # noqa: E402
                           run_chunked_page4)

pytestmark = pytest.mark.gpu

W = {4: 8, 128: 128}
CASES = 300


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.gpu_backend import GpuBackend
    return GpuBackend()


def _case(rng):
    cr = int(rng.choice([4, 128]))
    hd = int(rng.choice([128, 256, 512]))
    dtype = str(rng.choice(["f32", "bf16"]))
    B = int(rng.integers(1, 25 if cr == 4 else 9))
    R = wl.ROW_MULT[cr] * hd
    decode_steps = int(rng.integers(0, 2 * W[cr] + 4)) if cr == 4 else int(rng.integers(0, 160))
    seqs, chunks = [], []
    for _ in range(B):
        L = int(rng.integers(1, 6 * W[cr] if cr == 4 else 3 * W[cr]))
        scale = float(rng.choice([1.0, 2.0, 3.0, 30.0]))
        x = (scale * rng.standard_normal((L + decode_steps, R))).astype(np.float32)
        seqs.append(wl.to_bf16_bits(x) if dtype == "bf16" else x)
        chunks.append(random_split(rng, L, int(rng.integers(1, 7))))
    ape_f = (0.1 * rng.standard_normal((W[cr], hd))).astype(np.float32)
    ape = wl.to_bf16_bits(ape_f) if dtype == "bf16" else ape_f
    slots = B + int(rng.integers(0, 4))
    idx = rng.permutation(slots)[:B]
    return cr, hd, dtype, seqs, chunks, decode_steps, idx, slots, ape


def test_random_chunkings_match_the_oracle(gpu):
    for case in range(CASES):
        cr, hd, dtype, seqs, chunks, decode_steps, idx, slots, ape = _case(np.random.default_rng([2024, case]))
        print("fuzz case %d: ratio %d hd %d %s B=%d decode=%d chunks per request %s" %
              (case, cr, hd, dtype, len(seqs), decode_steps, [len(c) for c in chunks]), flush=True)
        em_o, st_o = run_chunked(OracleBackend(oracle), cr, hd, dtype, seqs, chunks, decode_steps, idx, slots, ape)
        em_g, st_g = run_chunked(gpu, cr, hd, dtype, seqs, chunks, decode_steps, idx, slots, ape)
        assert sorted(em_o) == sorted(em_g), case
        for k in em_o:
            g, o = em_g[k].astype(np.float64), em_o[k].astype(np.float64)
            tol = (1e-5 + 1e-5 * np.abs(o)) if dtype == "f32" else 2e-2
            assert np.all(np.isfinite(g)) and np.all(np.abs(g - o) <= tol), (case, k, float(np.abs(g - o).max()))
        assert np.array_equal(st_g.view(np.uint8), st_o.view(np.uint8)), case


VARIANT_CASES = 150


def _close(g, o, dtype, what):
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    tol = (1e-5 + 1e-5 * np.abs(o)) if dtype == "f32" else 2e-2
    assert np.all(np.isfinite(g)) and np.all(np.abs(g - o) <= tol), (what, float(np.abs(g - o).max()))


def _seqs(rng, B, l_hi, steps, R, dtype):
    seqs, chunks = [], []
    for _ in range(B):
        L = int(rng.integers(1, l_hi))
        x = rng.standard_normal((L + steps, R)).astype(np.float32)
        seqs.append(wl.to_bf16_bits(x) if dtype == "bf16" else x)
        chunks.append(random_split(rng, L, int(rng.integers(1, 7))))
    return seqs, chunks


def _ape(rng, n, hd, dtype):
    a = (0.1 * rng.standard_normal((n, hd))).astype(np.float32)
    return wl.to_bf16_bits(a) if dtype == "bf16" else a


def test_random_chunkings_of_the_other_state_mappings(gpu):
    for case in range(VARIANT_CASES):
        rng = np.random.default_rng([2025, case])
        kind = str(rng.choice(["swa", "online", "page4"]))
        hd = int(rng.choice([128, 256, 512]))
        dtype = str(rng.choice(["f32", "bf16"]))
        if kind == "swa":
            cr = int(rng.choice([4, 128]))
            if cr == 4:
                sps = int(rng.choice([8, 16, 32, 64, 128]))
                ring = int(rng.choice([r for r in (8, 16, 32) if sps % r == 0]))
            else:
                sps, ring = int(rng.choice([128, 256, 512])), 128
            B, steps = int(rng.integers(1, 7)), int(rng.integers(0, 20 if cr == 4 else 140))
            seqs, chunks = _seqs(rng, B, 6 * sps if cr == 4 else 600, steps, wl.ROW_MULT[cr] * hd, dtype)
            stride = max(len(x) for x in seqs) + 4
            r2t, f2s, num_pages = wl.swa_tables(rng, stride, B + 2, sps, stride=stride)
            rows = num_pages * ring if cr == 4 else (B + 2) * 128
            swa = dict(req_to_token=r2t, full_to_swa=f2s, swa_page_size=sps, ring_size=ring, num_state_rows=rows)
            ape, idx = _ape(rng, W[cr], hd, dtype), rng.permutation(B + 2)[:B]
            print("fuzz case %d: SWA ratio %d hd %d %s page %d ring %d B=%d decode=%d" %
                  (case, cr, hd, dtype, sps, ring, B, steps), flush=True)
            em_o, st_o = run_chunked(OracleBackend(oracle), cr, hd, dtype, seqs, chunks, steps, idx, 0, ape, swa=swa)
            em_g, st_g = run_chunked(gpu, cr, hd, dtype, seqs, chunks, steps, idx, 0, ape, swa=swa)
            assert sorted(em_o) == sorted(em_g), case
            for k in em_o:
                _close(em_g[k], em_o[k], dtype, (case, k))
            assert np.array_equal(st_g.view(np.uint8), st_o.view(np.uint8)), case
        elif kind == "online":
            B, steps = int(rng.integers(1, 7)), int(rng.integers(0, 150))
            slots = B + 2
            seqs, chunks = _seqs(rng, B, 600, steps, 2 * hd, dtype)
            ape, idx = _ape(rng, 128, hd, dtype), rng.permutation(slots)[:B]
            print("fuzz case %d: online ratio 128 hd %d %s B=%d decode=%d" % (case, hd, dtype, B, steps), flush=True)
            nan_slots = np.full((slots, 3, hd), np.nan)
            ref, _ = run_chunked(OnlineBackend(OracleOnline(oracle), ape), 128, hd, dtype, seqs, chunks, steps, idx,
                                 slots, ape, state=nan_slots)
            got, _ = run_chunked(OnlineBackend(gpu, ape), 128, hd, dtype, seqs, chunks, steps, idx, slots, ape,
                                 state=nan_slots.astype(np.float32))
            assert set(got) == set(ref), case
            for k in ref:
                _close(got[k], ref[k], dtype, (case, k))
        else:
            B, steps = int(rng.integers(1, 9)), int(rng.integers(0, 20))
            seqs, chunks = _seqs(rng, B, 120, steps, 4 * hd, dtype)
            ape, pseed = _ape(rng, 8, hd, dtype), int(rng.integers(0, 1 << 30))
            n_pages = int(sum(len(x) for x in seqs) // 4 + 4 * B + 8)
            print("fuzz case %d: 4-row pages hd %d %s B=%d decode=%d pages=%d" % (case, hd, dtype, B, steps, n_pages),
                  flush=True)
            ref, st_o = run_chunked_page4(OracleBackend(oracle), np.random.default_rng(pseed), hd, dtype, seqs, chunks,
                                          steps, ape, n_pages=n_pages)
            got, st_g = run_chunked_page4(gpu, np.random.default_rng(pseed), hd, dtype, seqs, chunks, steps, ape,
                                          n_pages=n_pages)
            assert set(got) == set(ref), case
            for k in ref:
                _close(got[k], ref[k], dtype, (case, k))
            assert np.array_equal(np.asarray(st_g).view(np.uint8), np.asarray(st_o).view(np.uint8)), case
