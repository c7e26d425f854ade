"""Pins of the oracle's norm + rotary embedding + store step.

* worked examples derived by hand from the pages (tests/golden/);
* the norm is torch's RMSNorm and the rotation is a complex product
  (torch, float64, CPU), on records that the oracle's own planner emits;
* invariants: with unit weights the stored row's mean square is
  ms / (ms + eps) whatever the rotation (a rotation keeps every pair's norm);
* which rows are stored: every valid C record at out_loc[ragged_id], only the
  decode records that close a block, nothing else touched;
* error bits for locations, positions and ragged ids out of range.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ERR_RECORD = 16


def _golden():
    with open(os.path.join(GOLDEN, "store_worked_examples.json")) as f:
        return json.load(f)


def _pack_c(fields, invalid=0):
    out = np.full((len(fields) + invalid, 16), 0xFF, np.uint8)
    for k, (s, rag, blen, rp0, rp1) in enumerate(fields):
        words = np.array([s, rag | (blen << 24), rp0, rp1], dtype=np.uint32)
        out[k] = words.view(np.uint8)
    return out


def _pack_d(seq_lens):
    out = np.zeros((len(seq_lens), 16), np.uint8)
    for b, s in enumerate(seq_lens):
        out[b, :4] = np.array([s], np.uint32).view(np.uint8)
    return out


def _table(max_pos, pairs, at):
    t = np.full((max_pos, pairs, 2), np.nan, np.float32)
    for p, v in at.items():
        t[int(p)] = v
    return t


def _expected_cache(n, hd, stored):
    c = np.full((n, hd), np.nan)
    for loc, row in stored.items():
        c[int(loc)] = row
    return c


def test_worked_example_decode():
    g = _golden()["decode_c4"]
    hd = len(g["norm_weight"])
    freqs = _table(g["max_position"], 2, g["freqs_at"])
    cache, err = oracle.store_decode(g["compress_ratio"], np.array(g["rows"], np.float32), _pack_d(g["seq_lens"]),
                                     g["norm_weight"], g["eps"], freqs, g["out_loc"],
                                     np.full((g["num_cache_rows"], hd), np.nan))
    assert err == 0
    np.testing.assert_array_equal(cache, _expected_cache(g["num_cache_rows"], hd, g["stored"]))


def test_worked_example_eps():
    g = _golden()["eps"]
    cache, err = oracle.store_decode(g["compress_ratio"], np.array(g["rows"], np.float32), _pack_d(g["seq_lens"]),
                                     g["norm_weight"], g["eps"], np.zeros((0, 0, 2), np.float32), g["out_loc"],
                                     np.full((1, 2), np.nan))
    assert err == 0
    np.testing.assert_array_equal(cache, _expected_cache(1, 2, g["stored"]))


def test_worked_example_prefill():
    g = _golden()["prefill_c128"]
    hd = len(g["norm_weight"])
    plan = _pack_c(g["plan_c"], g["invalid_records"])
    out_loc = np.full(g["num_loc"], -1, np.int32)  # any other lookup would be an error
    for r, loc in g["out_loc_at"].items():
        out_loc[int(r)] = loc
    freqs = _table(g["max_position"], 1, g["freqs_at"])
    cache, err = oracle.store_prefill(g["compress_ratio"], np.array(g["rows"], np.float32), plan, len(plan),
                                      g["norm_weight"], g["eps"], freqs, out_loc,
                                      np.full((g["num_cache_rows"], hd), np.nan))
    assert err == 0
    np.testing.assert_allclose(cache, _expected_cache(g["num_cache_rows"], hd, g["stored"]), rtol=0, atol=1e-7)


# --------------------------------------------------------------------------
# against torch (float64, CPU): RMSNorm, then the complex product
# --------------------------------------------------------------------------

def _freqs(rng, max_pos, rope_dim):
    theta = rng.uniform(-np.pi, np.pi, size=(max_pos, rope_dim // 2))
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)


def _torch_reference(rows, w, eps, freqs, pos, rope_dim):
    x = torch.from_numpy(rows.astype(np.float64))
    y = torch.nn.functional.rms_norm(x, (x.shape[1],), torch.from_numpy(w.astype(np.float64)), eps)
    if rope_dim:
        hd = x.shape[1]
        f = torch.from_numpy(freqs.astype(np.float64))[torch.from_numpy(pos)]
        z = torch.view_as_complex(y[:, hd - rope_dim:].contiguous().view(len(pos), rope_dim // 2, 2))
        y[:, hd - rope_dim:] = torch.view_as_real(z * torch.view_as_complex(f.contiguous())).reshape(len(pos), -1)
    return y.numpy()


@pytest.mark.parametrize("cr,hd,rope_dim,eps", [(4, 512, 64, 1e-6), (128, 512, 64, 1e-6), (4, 128, 128, 1e-5),
                                                (128, 128, 0, 0.5), (4, 256, 8, 1e-6)])
def test_prefill_matches_torch_rms_norm_and_complex_rotation(cr, hd, rope_dim, eps):
    rng = np.random.default_rng(7 + cr + hd + rope_dim)
    B = 6
    s = rng.integers(1, 700, size=B)
    e = np.minimum(s, rng.integers(1, 400, size=B))
    num_q = int(e.sum())
    cap_c, cap_w = oracle.capacities(cr, B, num_q)
    pc, _, counts = oracle.plan_prefill(cr, s, e, rng.permutation(B), B * (8 if cr == 4 else 128), num_q, cap_c,
                                        cap_w)
    n = int(counts[0])
    assert n > 0
    f = oracle.unpack_c(pc[:n])
    rows = (rng.standard_normal((cap_c, hd)) * rng.uniform(0.1, 3.0, size=(cap_c, 1))).astype(np.float32)
    w = rng.uniform(0.5, 1.5, size=hd).astype(np.float32)
    max_pos = int(s.max())
    freqs = _freqs(rng, max_pos, rope_dim)
    out_loc = rng.permutation(num_q + 5)[:num_q].astype(np.int32)
    cache, err = oracle.store_prefill(cr, rows, pc, n, w, eps, freqs, out_loc, np.full((num_q + 5, hd), np.nan))
    assert err == 0
    pos = np.maximum(f[:, 0].astype(np.int64) - cr, 0)
    ref = _torch_reference(rows[:n], w, eps, freqs, pos, rope_dim)
    locs = out_loc[f[:, 1]]
    np.testing.assert_allclose(cache[locs], ref, rtol=1e-12, atol=1e-12)
    untouched = np.setdiff1d(np.arange(num_q + 5), locs)
    assert np.isnan(cache[untouched]).all()


@pytest.mark.parametrize("cr", [4, 128])
def test_decode_stores_only_rows_that_close_a_block(cr):
    rng = np.random.default_rng(30 + cr)
    B = 64
    s = rng.integers(1, 3 * cr, size=B)
    s[:4] = [cr, 2 * cr, cr + 1, 4]  # the first block (position 0) and a non-boundary
    idx = rng.permutation(B)
    pd, status = oracle.plan_decode(cr, s, idx, B * (8 if cr == 4 else 128))
    assert status == 0
    hd, rope_dim = 128, 32
    rows = rng.standard_normal((B, hd)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, size=hd).astype(np.float32)
    freqs = _freqs(rng, 3 * cr, rope_dim)
    out_loc = rng.permutation(B).astype(np.int32)
    cache, err = oracle.store_decode(cr, rows, pd, w, 1e-6, freqs, out_loc, np.full((B, hd), np.nan))
    assert err == 0
    boundary = s % cr == 0
    assert boundary.any() and (~boundary).any()
    ref = _torch_reference(rows[boundary], w, 1e-6, freqs, np.maximum(s[boundary] - cr, 0), rope_dim)
    np.testing.assert_allclose(cache[out_loc[boundary]], ref, rtol=1e-12, atol=1e-12)
    assert np.isnan(cache[out_loc[~boundary]]).all()


def test_unit_weight_mean_square_closed_form():
    """With w = 1 the row's mean square becomes ms / (ms + eps); the rotation keeps every
    pair's norm, so this holds over the whole row, rotated channels included."""
    rng = np.random.default_rng(5)
    hd, B = 512, 16
    rows = (rng.standard_normal((B, hd)) * rng.uniform(0.01, 10, size=(B, 1))).astype(np.float32)
    eps = 0.25
    freqs = _freqs(rng, 1000, 64)
    s = rng.integers(1, 200, size=B) * 4
    cache, err = oracle.store_decode(4, rows, _pack_d(s), np.ones(hd, np.float32), eps, freqs,
                                     np.arange(B, dtype=np.int32), np.full((B, hd), np.nan))
    assert err == 0
    ms = (rows.astype(np.float64) ** 2).mean(axis=1)
    # the table's (cos, sin) are fp32, so |cis|^2 = 1 only to about 2^-22: that bounds the
    # rotated channels' deviation; a wrong norm is off by orders of magnitude more
    np.testing.assert_allclose((cache ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-6)
    # the un-rotated part is the plain scaled row
    np.testing.assert_allclose(cache[:, :hd - 64], rows[:, :hd - 64] / np.sqrt(ms + eps)[:, None], rtol=1e-12)
    # each rotated pair keeps its norm
    pre = rows[:, hd - 64:].astype(np.float64).reshape(B, 32, 2) / np.sqrt(ms + eps)[:, None, None]
    post = cache[:, hd - 64:].reshape(B, 32, 2)
    np.testing.assert_allclose(np.hypot(post[..., 0], post[..., 1]), np.hypot(pre[..., 0], pre[..., 1]), rtol=1e-6)


# --------------------------------------------------------------------------
# errors
# --------------------------------------------------------------------------

def test_errors_skip_only_the_bad_record():
    hd = 8
    rows = np.ones((4, hd), np.float32)
    w = np.ones(hd, np.float32)
    freqs = np.tile(np.array([1, 0], np.float32), (10, 1, 1)).reshape(10, 1, 2)
    plan = _pack_c([(8, 0, 0, 0, 0), (12, 1, 0, 0, 0), (16, 2, 0, 0, 0), (64, 3, 0, 0, 0)])
    # record 1: location outside the cache; record 2: ragged id outside out_loc; record 3: position 60 >= 10
    cache, err = oracle.store_prefill(4, rows, plan, 4, w, 0.0, freqs, np.array([0, 9], np.int32),
                                      np.full((4, hd), np.nan))
    assert err == ERR_RECORD
    assert np.isfinite(cache[0]).all() and np.isnan(cache[1:]).all()
    # each kind of bad record alone, so that no other record sets the error bit: a location one
    # past the last cache row, a ragged id one past out_loc, a position one past the table
    for recs, out_loc in (([(8, 0, 0, 0, 0), (12, 1, 0, 0, 0)], [0, 4]),
                          ([(8, 0, 0, 0, 0), (12, 2, 0, 0, 0)], [0, 1]),
                          ([(8, 0, 0, 0, 0), (14, 1, 0, 0, 0)], [0, 1])):
        cache, err = oracle.store_prefill(4, rows, _pack_c(recs), 2, w, 0.0, freqs, np.array(out_loc, np.int32),
                                          np.full((4, hd), np.nan))
        assert err == ERR_RECORD, (recs, out_loc)
        assert np.isfinite(cache[0]).all() and np.isnan(cache[1:]).all(), (recs, out_loc)
    # without rotated channels the position is not looked up
    cache, err = oracle.store_prefill(4, rows[:, :6], _pack_c([(64, 0, 0, 0, 0)]), 1, w[:6], 0.0,
                                      np.zeros((0, 0, 2), np.float32), np.array([1], np.int32),
                                      np.full((2, 6), np.nan))
    assert err == 0 and np.isfinite(cache[1]).all()
    # decode: an invalid record stores nothing and is no error
    pd = _pack_d([8, 8])
    pd[1] = 0xFF
    cache, err = oracle.store_decode(4, rows[:2], pd, w, 0.0, freqs, np.array([1, 0], np.int32),
                                     np.full((2, hd), np.nan))
    assert err == 0 and np.isfinite(cache[1]).all() and np.isnan(cache[0]).all()
