"""CPU oracle for the KV-compressor hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``sparse_attention_kv_plan_amd``) never imports it, and the two
share no code: the arithmetic lives in ``kvc_oracle.c`` (plain C, float64) and
in ``brute.py`` (pure Python, tiny sizes only).

Every function takes and returns numpy arrays.  bf16 tensors travel as
``uint16`` bit patterns; plan records travel as ``uint8`` byte arrays of
16 (C, D) or 8 (W) bytes per record.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB = os.path.join(_HERE, "libkvc_oracle.so")

C_BYTES, W_BYTES, D_BYTES = 16, 8, 16
WINDOW = {4: 8, 128: 128}
ROW_MULT = {4: 4, 128: 2}  # row width of a kv/score row, in units of head_dim


def build(force: bool = True) -> str:
    """Compile kvc_oracle.c with gcc (no fast-math) into libkvc_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        # KVC_ORACLE_LIB lets the mutation test load a deliberately broken copy
        path = os.environ.get("KVC_ORACLE_LIB")
        if path is None:
            path = _LIB
            if not os.path.exists(path):
                build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        lib.oracle_plan_prefill.argtypes = [I, I, I, P, P, P, L, P, I, P, I, P]
        lib.oracle_plan_decode.argtypes = [I, I, P, P, L, P, P]
        lib.oracle_compress.argtypes = [I, I, I, P, L, P, I, P, P, I, P]
        lib.oracle_write.argtypes = [I, I, I, P, L, P, I, P, I]
        lib.oracle_decode.argtypes = [I, I, I, P, L, P, P, P, I, P]
        lib.oracle_plan_prefill_swa.argtypes = [I, I, I, P, P, P, P, L, L, P, L, I, I, L, P, I, P, I, P, P]
        lib.oracle_plan_decode_swa.argtypes = [I, I, P, P, P, L, L, P, L, I, I, L, P, P]
        D = ctypes.c_double
        lib.oracle_store_prefill.argtypes = [I, I, I, P, P, I, P, D, P, L, P, L, P, L]
        lib.oracle_store_decode.argtypes = [I, I, I, P, P, I, P, D, P, L, P, L, P, L]
        lib.oracle_compress_online.argtypes = [I, I, P, L, P, I, P, P, I, P]
        lib.oracle_plan_prefill_page4.argtypes = [I, I, P, P, P, P, L, P, I, P, I, P, P]
        lib.oracle_plan_decode_page4.argtypes = [I, P, P, P, L, P, P]
        lib.oracle_write_online.argtypes = [I, I, P, L, P, I, P, P, I]
        lib.oracle_decode_online.argtypes = [I, I, P, L, P, P, P, I, P]
        for f in ("oracle_plan_prefill", "oracle_plan_decode", "oracle_compress", "oracle_write",
                  "oracle_decode", "oracle_plan_prefill_swa", "oracle_plan_decode_swa", "oracle_store_prefill",
                  "oracle_store_decode", "oracle_compress_online", "oracle_write_online", "oracle_decode_online",
                  "oracle_plan_prefill_page4", "oracle_plan_decode_page4"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _elem(a):
    """Return (contiguous array, is_bf16) for a bf16 (uint16 bits) or fp32 array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, 1
    if a.dtype == np.float32:
        return a, 0
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32, got %s" % a.dtype)


class OracleError(ValueError):
    pass


def plan_prefill(cr, seq_lens, extend_lens, state_index, num_state_rows, num_q, cap_c, cap_w):
    """Build the prefill plan.  Returns (plan_c bytes [cap_c,16], plan_w bytes [cap_w,8], counts[4])."""
    s, e, idx = _i32(seq_lens), _i32(extend_lens), _i32(state_index)
    pc = np.zeros((max(cap_c, 0), C_BYTES), np.uint8)
    pw = np.zeros((max(cap_w, 0), W_BYTES), np.uint8)
    counts = np.zeros(4, np.int32)
    rc = _load().oracle_plan_prefill(cr, len(s), num_q, _ptr(s), _ptr(e), _ptr(idx), int(num_state_rows),
                                     _ptr(pc), cap_c, _ptr(pw), cap_w, _ptr(counts))
    if rc != 0:
        raise OracleError("oracle_plan_prefill rejected its arguments")
    return pc, pw, counts


def plan_decode(cr, seq_lens, state_index, num_state_rows):
    """Build the decode plan.  Returns (plan_d bytes [B,16], status)."""
    s, idx = _i32(seq_lens), _i32(state_index)
    pd = np.zeros((len(s), D_BYTES), np.uint8)
    status = np.zeros(1, np.int32)
    rc = _load().oracle_plan_decode(cr, len(s), _ptr(s), _ptr(idx), int(num_state_rows), _ptr(pd), _ptr(status))
    if rc != 0:
        raise OracleError("oracle_plan_decode rejected its arguments")
    return pd, int(status[0])


def compress(cr, hd, state, inp, ape, plan_c, num_c, out=None):
    """Pool the first num_c C records.  state [rows, R], inp [num_q, R], ape [W, hd].

    Returns (out float64 [len(plan_c), hd] -- rows not pooled are NaN unless
    ``out`` is given --, error bits)."""
    state, sb = _elem(state)
    inp, ib = _elem(inp)
    ape, ab = _elem(ape)
    assert sb == ib == ab
    pc = np.ascontiguousarray(plan_c, dtype=np.uint8)
    if out is None:
        out = np.full((max(pc.shape[0], 1), hd), np.nan, np.float64)
    err = _load().oracle_compress(cr, ib, hd, _ptr(state), state.shape[0], _ptr(inp), inp.shape[0], _ptr(ape),
                                  _ptr(pc), int(num_c), _ptr(out))
    return out[: pc.shape[0]], err


def write(cr, hd, state, inp, plan_w, num_w):
    """Scatter the first num_w W records into ``state`` in place.  Returns error bits."""
    inp, ib = _elem(inp)
    assert state.flags.c_contiguous
    _, sb = _elem(state)
    assert sb == ib
    pw = np.ascontiguousarray(plan_w, dtype=np.uint8)
    return _load().oracle_write(cr, ib, hd, _ptr(state), state.shape[0], _ptr(inp), inp.shape[0], _ptr(pw),
                                int(num_w))


def decode(cr, hd, state, inp, ape, plan_d):
    """Fused decode, in place on ``state``.  Returns (out float64 [B, hd], error bits)."""
    inp, ib = _elem(inp)
    ape, ab = _elem(ape)
    assert state.flags.c_contiguous
    _, sb = _elem(state)
    assert sb == ib == ab
    pd = np.ascontiguousarray(plan_d, dtype=np.uint8)
    B = pd.shape[0]
    out = np.full((B, hd), np.nan, np.float64)  # every row is the oracle's own: pooled or zero
    err = _load().oracle_decode(cr, ib, hd, _ptr(state), state.shape[0], _ptr(inp), _ptr(ape), _ptr(pd), B,
                                _ptr(out))
    return out, err


def plan_prefill_swa(cr, seq_lens, extend_lens, req_pool_indices, req_to_token, full_to_swa, swa_page_size,
                     ring_size, num_state_rows, num_q, cap_c, cap_w):
    """SWA-paged prefill plan.  req_to_token: int32 [num_reqs, stride]; full_to_swa: int32 [num_full].
    Returns (plan_c, plan_w, counts[4], status)."""
    s, e, rid = _i32(seq_lens), _i32(extend_lens), _i32(req_pool_indices)
    r2t = _i32(req_to_token)
    f2s = _i32(full_to_swa)
    pc = np.zeros((max(cap_c, 0), C_BYTES), np.uint8)
    pw = np.zeros((max(cap_w, 0), W_BYTES), np.uint8)
    counts = np.zeros(4, np.int32)
    status = np.zeros(1, np.int32)
    rc = _load().oracle_plan_prefill_swa(cr, len(s), num_q, _ptr(s), _ptr(e), _ptr(rid), _ptr(r2t), r2t.shape[1],
                                         r2t.shape[0], _ptr(f2s), f2s.shape[0], swa_page_size, ring_size,
                                         int(num_state_rows), _ptr(pc), cap_c, _ptr(pw), cap_w, _ptr(counts),
                                         _ptr(status))
    if rc != 0:
        raise OracleError("oracle_plan_prefill_swa rejected its arguments")
    return pc, pw, counts, int(status[0])


def plan_decode_swa(cr, seq_lens, req_pool_indices, req_to_token, full_to_swa, swa_page_size, ring_size,
                    num_state_rows):
    """SWA-paged decode plan.  Returns (plan_d, status)."""
    s, rid = _i32(seq_lens), _i32(req_pool_indices)
    r2t = _i32(req_to_token)
    f2s = _i32(full_to_swa)
    pd = np.zeros((len(s), D_BYTES), np.uint8)
    status = np.zeros(1, np.int32)
    rc = _load().oracle_plan_decode_swa(cr, len(s), _ptr(s), _ptr(rid), _ptr(r2t), r2t.shape[1], r2t.shape[0],
                                        _ptr(f2s), f2s.shape[0], swa_page_size, ring_size, int(num_state_rows),
                                        _ptr(pd), _ptr(status))
    if rc != 0:
        raise OracleError("oracle_plan_decode_swa rejected its arguments")
    return pd, int(status[0])


_GUARD_ROWS = 16
_GUARD = -3.0e300  # a value no stored row holds


def _store(fn, cr, rows, plan, n, norm_weight, eps, freqs_cis, out_loc, cache):
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    hd = rows.shape[1]
    w = np.ascontiguousarray(norm_weight, dtype=np.float32)
    freqs = np.ascontiguousarray(freqs_cis, dtype=np.float32)
    rope_dim = 0 if freqs.size == 0 else freqs.shape[1] * 2
    freqs = freqs.reshape(-1, max(rope_dim, 1)) if freqs.size else freqs
    loc = _i32(out_loc)
    cache = np.asarray(cache, dtype=np.float64)
    rows_c = cache.shape[0]
    # guard rows after the cache: a store past its last row shows up here instead of in other memory
    buf = np.full((rows_c + _GUARD_ROWS, hd), _GUARD)
    buf[:rows_c] = cache
    plan = np.ascontiguousarray(plan, dtype=np.uint8)
    err = fn(cr, hd, rope_dim, _ptr(rows), _ptr(plan), int(n), _ptr(w), float(eps), _ptr(freqs),
             freqs.shape[0] if freqs.size else 0, _ptr(loc), loc.size, _ptr(buf), rows_c)
    if not np.all(buf[rows_c:] == _GUARD):
        raise AssertionError("the store wrote past the last cache row")
    return buf[:rows_c], err


def store_prefill(cr, rows, plan_c, num_c, norm_weight, eps, freqs_cis, out_loc, cache):
    """Norm + rotary embedding + store of prefill compressed rows (float64).

    rows: float32 [>= num_c, hd], row k belonging to C record k; freqs_cis:
    float32 [max_position, rope_dim / 2, 2] (cos, sin), rope_dim = 0 when
    empty; out_loc: int32 per ragged token; cache: float [rows, hd], copied.
    Returns (cache with the stored rows replaced, error bits)."""
    return _store(_load().oracle_store_prefill, cr, rows, plan_c, num_c, norm_weight, eps, freqs_cis, out_loc, cache)


def store_decode(cr, rows, plan_d, norm_weight, eps, freqs_cis, out_loc, cache):
    """Decode variant: rows [B, hd], out_loc int32 per request; only records
    whose seq_len closes a block are stored."""
    plan_d = np.ascontiguousarray(plan_d, dtype=np.uint8)
    return _store(_load().oracle_store_decode, cr, rows, plan_d, plan_d.shape[0], norm_weight, eps, freqs_cis,
                  out_loc, cache)


def _online_state(state, hd):
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    if st.ndim != 3 or st.shape[1:] != (3, hd):
        raise ValueError("online state must be [slots, 3, hd] (m, l, acc)")
    return st


def compress_online(hd, state, inp, ape, plan_c, num_c):
    """Ratio-128 pool with the online state: state [slots, 3, hd] (m, l, acc) float64.
    Returns (out float64 [cap_c, hd] (NaN where untouched), error bits)."""
    inp, bf = _elem(inp)
    ape, _ = _elem(ape)
    st = _online_state(state, hd)
    plan_c = np.ascontiguousarray(plan_c, dtype=np.uint8)
    out = np.full((max(plan_c.shape[0], 1), hd), np.nan)
    err = _load().oracle_compress_online(bf, hd, _ptr(st), st.shape[0], _ptr(inp), inp.shape[0], _ptr(ape),
                                         _ptr(plan_c), int(num_c), _ptr(out))
    return out[: plan_c.shape[0]], err


def write_online(hd, state, inp, ape, plan_w, num_w):
    """Fold each request's W records into its slot.  Returns (new state, error bits)."""
    inp, bf = _elem(inp)
    ape, _ = _elem(ape)
    st = _online_state(state, hd)
    plan_w = np.ascontiguousarray(plan_w, dtype=np.uint8)
    err = _load().oracle_write_online(bf, hd, _ptr(st), st.shape[0], _ptr(inp), inp.shape[0], _ptr(ape),
                                      _ptr(plan_w), int(num_w))
    return st, err


def decode_online(hd, state, inp, ape, plan_d):
    """Decode step with the online state.  Returns (out float64 [B, hd], new state, error bits)."""
    inp, bf = _elem(inp)
    ape, _ = _elem(ape)
    st = _online_state(state, hd)
    plan_d = np.ascontiguousarray(plan_d, dtype=np.uint8)
    B = plan_d.shape[0]
    out = np.zeros((B, hd))
    err = _load().oracle_decode_online(bf, hd, _ptr(st), st.shape[0], _ptr(inp), _ptr(ape), _ptr(plan_d), B,
                                       _ptr(out))
    return out, st, err


def plan_prefill_page4(seq_lens, extend_lens, page_index, bundle, num_state_rows, num_q, cap_c, cap_w):
    """Ratio-4 prefill plan over caller-allocated 4-row pages.  bundle: int32 [B, 4] =
    (load_first_page, load_second_page, write_first_page, last_position).
    Returns (plan_c, plan_w, counts, status)."""
    s, e, idx = _i32(seq_lens), _i32(extend_lens), _i32(page_index)
    bnd = np.ascontiguousarray(np.asarray(bundle, np.int32).reshape(-1, 4))
    B = s.size
    pc = np.zeros((cap_c, C_BYTES), np.uint8)
    pw = np.zeros((cap_w, W_BYTES), np.uint8)
    counts = np.zeros(4, np.int32)
    status = np.zeros(1, np.int32)
    rc = _load().oracle_plan_prefill_page4(B, int(num_q), _ptr(s), _ptr(e), _ptr(idx), _ptr(bnd),
                                           int(num_state_rows), _ptr(pc), int(cap_c), _ptr(pw), int(cap_w),
                                           _ptr(counts), _ptr(status))
    if rc < 0:
        raise ValueError("bad host arguments")
    return pc, pw, counts, int(status[0])


def plan_decode_page4(seq_lens, page_index, prev_page, num_state_rows):
    """Ratio-4 decode plan over caller-allocated pages: page_index[b] takes the new token,
    prev_page[b] holds the window's overlap block.  Returns (plan_d, status)."""
    s, idx, prev = _i32(seq_lens), _i32(page_index), _i32(prev_page)
    pd = np.zeros((s.size, D_BYTES), np.uint8)
    status = np.zeros(1, np.int32)
    rc = _load().oracle_plan_decode_page4(s.size, _ptr(s), _ptr(idx), _ptr(prev), int(num_state_rows), _ptr(pd),
                                          _ptr(status))
    if rc < 0:
        raise ValueError("bad host arguments")
    return pd, int(status[0])


def capacities_swa(cr, B, num_q, swa_page_size):
    """Capacities that always suffice for the SWA-paged plan (ratio 4 adds page-tail writes)."""
    cap_w = B * (WINDOW[cr] - 1) + (4 * (num_q // swa_page_size + B) if cr == 4 else 0)
    return min(num_q, num_q // cr + B), min(num_q, cap_w)


# --------------------------------------------------------------------------
# record helpers (byte layout as documented in kvc_oracle.c)
# --------------------------------------------------------------------------

def unpack_c(plan_c):
    """Decode C records -> int64 array [n, 5]: seq_len, ragged_id, buffer_len, read_page_0, read_page_1."""
    w = np.ascontiguousarray(plan_c, np.uint8).view("<u4").reshape(-1, 4).astype(np.int64)
    out = np.empty((w.shape[0], 5), np.int64)
    out[:, 0] = w[:, 0]
    out[:, 1] = w[:, 1] & 0xFFFFFF
    out[:, 2] = w[:, 1] >> 24
    out[:, 3] = w[:, 2].astype(np.uint32).view(np.int32)
    out[:, 4] = w[:, 3].astype(np.uint32).view(np.int32)
    return out


def unpack_w(plan_w):
    """Decode W records -> int64 array [n, 2]: ragged_id, write_loc."""
    w = np.ascontiguousarray(plan_w, np.uint8).view("<u4").reshape(-1, 2)
    return np.stack([w[:, 0].astype(np.int64), w[:, 1].view(np.int32).astype(np.int64)], axis=1)


def unpack_d(plan_d):
    """Decode D records -> int64 array [n, 4]: seq_len, write_loc, read_page_0, read_page_1."""
    w = np.ascontiguousarray(plan_d, np.uint8).view("<u4").reshape(-1, 4)
    out = w.view(np.int32).astype(np.int64)
    out[:, 0] = w[:, 0].astype(np.int64)
    return out


def capacities(cr, B, num_q):
    """Capacities that always suffice: every C or W record fits."""
    return min(num_q, num_q // cr + B), min(num_q, B * (WINDOW[cr] - 1))
