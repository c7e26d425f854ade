"""GPU parity on random chunkings: ratio, head_dim, dtype, batch, the split of every request into
prefill chunks and the number of decode steps all drawn from a fixed seed.  Every emitted row is
compared with the oracle's (fp32 bar 1e-5 + 1e-5 |ref|, bf16 bar 2e-2) and the state buffer after
the last step bit for bit.

fp32 inputs keep scores of the configs' size (standard deviation 1 or 2): the score + ape sum and
its exponent are formed in fp32, so a weight carries a relative error of about |score| * 2^-24 and
a row whose terms nearly cancel can miss the absolute 1e-5 once scores reach tens.  bf16 inputs
also take scores and values 3 and 30 times larger (bar 2e-2)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import workloads as wl  # noqa: E402
from tests.chunked import OracleBackend, random_split, run_chunked  # noqa: E402

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
        scale = float(rng.choice([1.0, 2.0])) if dtype == "f32" else float(rng.choice([1.0, 3.0, 30.0]))
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
