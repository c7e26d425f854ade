"""The pools and the write at the largest chunk the ABI takes: 1024 requests and 2^24 - 1 tokens.

Ragged ids then use all 24 bits of a C record, and input offsets pass 2^34 elements (ratio 4 at
head_dim 256 and ratio 128 at head_dim 512, bf16: 32 GiB of input each), so every row address must
be formed in 64 bits.  The inputs are drawn on the device; a sample of records (the highest ragged
ids, random ones, and the first record of random requests, which reads the state) is checked
against the oracle on just the rows each one reads, and a sample of W records against the rows
they copy.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sparse_attention_kv_plan_amd import kvc  # noqa: E402

pytestmark = pytest.mark.gpu

W = {4: 8, 128: 128}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.load()
    return torch.device("cuda")


@pytest.mark.parametrize("cr,hd", [(4, 256), (128, 512)])
def test_compress_and_write_at_maximum_token_count(dev, cr, hd):
    rng = np.random.default_rng(7700 + cr)
    B, win = 1024, W[cr]
    e = np.full(B, 16384, np.int64)
    e[-1] = (1 << 24) - 1 - int(e[:-1].sum())
    prefix = rng.integers(0, 1 << 20, size=B)
    s = prefix + e
    idx = rng.permutation(B)
    num_q = int(e.sum())
    R = (4 if cr == 4 else 2) * hd
    say("max tokens cr=%d hd=%d num_q=%d input %.1f GiB" % (cr, hd, num_q, num_q * R * 2 / 2**30))
    gen = torch.Generator(device=dev)
    gen.manual_seed(cr)
    inp = torch.randn((num_q, R), generator=gen, device=dev, dtype=torch.bfloat16)
    state = torch.randn((B * win, R), generator=gen, device=dev, dtype=torch.bfloat16)
    ape = (0.1 * torch.randn((win, hd), generator=gen, device=dev)).to(torch.bfloat16)
    state_h = state.view(torch.int16).cpu().numpy().view(np.uint16)
    ape_h = ape.view(torch.int16).cpu().numpy().view(np.uint16)

    i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32)).to(dev)  # noqa: E731
    pc, pw, counts = kvc.alloc_prefill_plan(cr, B, num_q, dev)
    kvc.plan_prefill(cr, i32(s), i32(e), i32(idx), B * win, num_q, pc, pw, counts)
    out = torch.empty((pc.shape[0], hd), dtype=torch.float32, device=dev)
    kvc.compress(cr, hd, state, inp, ape, pc, counts, out)
    torch.cuda.synchronize()
    c = counts.cpu().tolist()
    assert c[2] == 0 and c[3] == 0, c
    n_c, n_w = c[0], c[1]

    # the sample of C records
    recs = oracle.unpack_c(pc[:n_c].cpu().numpy()).astype(np.int64)  # seq_len, ragged, blen, rp0, rp1
    ragged = recs[:, 1]
    first_of = np.searchsorted(ragged, np.concatenate([[0], np.cumsum(e)[:-1]]))  # each request's first record
    sel = np.unique(np.concatenate([
        np.arange(n_c - 48, n_c),                              # the highest ragged ids
        rng.choice(n_c, size=48, replace=False),
        first_of[rng.choice(B, size=32, replace=False)],       # first records: the window starts in the state
    ]))
    assert ragged[sel].max() > (1 << 23) and (recs[sel, 2] > 0).any()
    # a compact input holding only the rows each sampled record reads: record m's window entry i is
    # input row ragged - (win - 1) + i, put at row m * win + i
    rows = (ragged[sel][:, None] - (win - 1) + np.arange(win)[None, :]).clip(0, num_q - 1)
    mini = inp[torch.from_numpy(rows.reshape(-1)).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    plan = pc[torch.from_numpy(sel).to(dev)].cpu().numpy().copy()
    words = plan.view(np.uint32).reshape(-1, 4)
    words[:, 1] = (np.arange(len(sel)) * win + win - 1).astype(np.uint32) | (words[:, 1] & 0xFF000000)
    ref, err = oracle.compress(cr, hd, state_h, mini, ape_h, plan, len(sel))
    assert err == 0
    got = out[torch.from_numpy(sel).to(dev)].cpu().numpy().astype(np.float64)
    bad = np.abs(got - ref) > 2e-2
    assert not bad.any(), "%d of %d values out of the bf16 bar, max err %.3g" % (bad.sum(), bad.size,
                                                                                   np.abs(got - ref).max())

    # the write: a sample of W records (the last ones and random ones) copies its input row
    kvc.write(cr, hd, state, inp, pw, counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist()[3] == 0
    wrec = oracle.unpack_w(pw[:n_w].cpu().numpy()).astype(np.int64)  # ragged, write_loc
    wsel = np.unique(np.concatenate([np.arange(max(0, n_w - 64), n_w), rng.choice(n_w, size=min(n_w, 512),
                                                                                   replace=False)]))
    assert wrec[wsel, 0].max() > (1 << 23)
    src = inp[torch.from_numpy(wrec[wsel, 0]).to(dev)]
    dst = state[torch.from_numpy(wrec[wsel, 1]).to(dev)]
    assert torch.equal(src.view(torch.int16), dst.view(torch.int16))
    del inp, state, out
    torch.cuda.empty_cache()
