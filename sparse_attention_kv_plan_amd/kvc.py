"""ctypes binding of libkvc.so (include/kvc.h): argument marshalling only.

Every call takes torch CUDA tensors, passes their device pointers and the
current HIP stream to the C entry point of the same name, and raises
``KvcError`` when the library returns a non-zero code.  All computation runs
in the library's HIP kernels; there is no fallback: if libkvc.so is missing
or cannot be loaded, ``load()`` raises.

Plan records are carried as uint8 tensors of 16 (C, D) or 8 (W) bytes per
record; bf16 tensors may be passed as torch.bfloat16 or as int16/uint16 bit
patterns.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libkvc.so")
HEADER = os.path.join(ROOT, "include", "kvc.h")

KVC_OK, KVC_EINVAL, KVC_EHIP = 0, -1, -2
KVC_F32, KVC_BF16 = 0, 1
DERR_EXTEND, DERR_NUMQ, DERR_INDEX, DERR_CAPACITY, DERR_RECORD, DERR_DUPLICATE = 1, 2, 4, 8, 16, 32
WINDOW = {4: 8, 128: 128}
ROW_MULT = {4: 4, 128: 2}
C_BYTES, W_BYTES, D_BYTES = 16, 8, 16

_lib = None


class KvcError(RuntimeError):
    pass


def load(build_if_missing: bool = False):
    """Load libkvc.so.  With build_if_missing, compile it first when absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise KvcError("libkvc.so is not built (python -m sparse_attention_kv_plan_amd.build)")
        from sparse_attention_kv_plan_amd import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    sig = {
        "kvc_plan_prefill": [I, I, I, P, P, P, L, P, I, P, I, P, P, P],
        "kvc_plan_decode": [I, I, P, P, L, P, P, P, P],
        "kvc_write": [I, I, I, P, L, P, I, P, I, P, P],
        "kvc_compress_c4": [I, I, P, L, P, I, P, P, I, P, P, P],
        "kvc_compress_c128": [I, I, P, L, P, I, P, P, I, P, P, P],
        "kvc_decode_c4": [I, I, P, L, P, P, P, I, P, P, P],
        "kvc_decode_c128": [I, I, P, L, P, P, P, P, I, P, P, P],
        "kvc_plan_prefill_swa": [I, I, I, P, P, P, P, L, L, P, L, I, I, L, P, I, P, I, P, P, P],
        "kvc_plan_decode_swa": [I, I, P, P, P, L, L, P, L, I, I, L, P, P, P, P],
        "kvc_norm_rope_store_prefill": [I, I, P, P, I, P, P, P],
        "kvc_norm_rope_store_decode": [I, I, P, P, I, P, P, P],
        "kvc_compress_c4_norm_rope_store": [I, I, P, L, P, I, P, P, I, P, P, P],
        "kvc_compress_c128_norm_rope_store": [I, I, P, L, P, I, P, P, I, P, P, P],
        "kvc_decode_c4_norm_rope_store": [I, I, P, L, P, P, P, I, P, P, P],
        "kvc_compress_c128_online": [I, I, P, L, P, I, P, P, I, P, P, P],
        "kvc_plan_prefill_page4": [I, I, P, P, P, P, L, P, I, P, I, P, P, P],
        "kvc_plan_decode_page4": [I, P, P, P, L, P, P, P],
        "kvc_write_c128_online": [I, I, P, L, P, I, P, P, I, P, P, I, P],
        "kvc_decode_c128_online": [I, I, P, L, P, P, P, I, P, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.kvc_strerror.argtypes = [ctypes.c_int]
    lib.kvc_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions():
    """Names of the functions declared in include/kvc.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvc_\w+)\s*\(", text, re.M)))


def strerror(code: int) -> str:
    return load().kvc_strerror(code).decode()


def _check(rc: int, what: str):
    if rc != KVC_OK:
        raise KvcError("%s: %s (%d)" % (what, strerror(rc), rc))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t) -> int:
    if t.dtype == torch.float32:
        return KVC_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return KVC_BF16
    raise KvcError("unsupported element type %s" % t.dtype)


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise KvcError("tensors must be contiguous CUDA tensors")


def _i32(*ts):
    """Lengths, indices, tables, counts and status words are int32 in the ABI: an int64 tensor
    would be read as pairs of int32 words, giving wrong (often in-range) values silently."""
    for t in ts:
        if t is not None and t.dtype != torch.int32:
            raise KvcError("index, length, count and status tensors must be int32, got %s" % t.dtype)


def _shape(t, rows_at_least, cols, what):
    """The library cannot see device buffer sizes: check them before handing pointers over."""
    if t.dim() != 2 or t.shape[0] < rows_at_least or t.shape[1] != cols:
        raise KvcError("%s must be [>= %d, %d], got %s" % (what, rows_at_least, cols, tuple(t.shape)))


def _rows(cr, head_dim, state, inp):
    R = ROW_MULT[cr] * head_dim
    _shape(state, 0, R, "state")
    _shape(inp, 0, R, "input")
    if state.element_size() != inp.element_size():
        raise KvcError("state and input must share a dtype")


# --------------------------------------------------------------------------
# allocation helpers (torch owns the memory)
# --------------------------------------------------------------------------

def capacities(cr: int, batch: int, num_q: int):
    """Record capacities that always suffice for a prefill chunk."""
    return min(num_q, num_q // cr + batch), min(num_q, batch * (WINDOW[cr] - 1))


def alloc_prefill_plan(cr: int, batch: int, num_q: int, device="cuda", cap_c=None, cap_w=None):
    cc, cw = capacities(cr, batch, num_q)
    cap_c = cc if cap_c is None else cap_c
    cap_w = cw if cap_w is None else cap_w
    plan_c = torch.empty((cap_c, C_BYTES), dtype=torch.uint8, device=device)
    plan_w = torch.empty((cap_w, W_BYTES), dtype=torch.uint8, device=device)
    counts = torch.empty(4, dtype=torch.int32, device=device)
    return plan_c, plan_w, counts


# --------------------------------------------------------------------------
# the C entry points
# --------------------------------------------------------------------------

def plan_prefill(cr, seq_lens, extend_lens, state_index, num_state_rows, num_q, plan_c, plan_w, counts,
                 stream=None, runs=None):
    """runs: None, or for ratio 128 an int32 [batch, 4] tensor (run_list()) that receives each
    request's run of W records for kvc_write_c128_online."""
    _i32(seq_lens, extend_lens, state_index, counts, runs)
    _dev(seq_lens, extend_lens, state_index, plan_c, plan_w, counts, runs)
    B = seq_lens.numel()
    if extend_lens.numel() != B or state_index.numel() != B or counts.numel() < 4:
        raise KvcError("seq_lens, extend_lens, state_index must have one entry per request; counts 4")
    _shape(plan_c, 0, C_BYTES, "plan_c")
    _shape(plan_w, 0, W_BYTES, "plan_w")
    _runs(cr, runs, B)
    rc = load().kvc_plan_prefill(cr, seq_lens.numel(), num_q, _p(seq_lens), _p(extend_lens), _p(state_index),
                                 num_state_rows, _p(plan_c), plan_c.shape[0], _p(plan_w), plan_w.shape[0],
                                 _p(counts), _p(runs), _stream(stream))
    _check(rc, "kvc_plan_prefill")


def run_list(batch, device):
    """An int32 [batch, 4] buffer for the ratio-128 run list of a prefill chunk (see kvc_plan_prefill)."""
    return torch.empty((batch, 4), dtype=torch.int32, device=device)


def _runs(cr, runs, batch):
    if runs is not None and (cr != 128 or tuple(runs.shape) != (batch, 4) or not runs.is_contiguous()):
        raise KvcError("the run list is for ratio 128 and must be a contiguous int32 [batch, 4] tensor")


def boundary_list(batch, device):
    """An int32 buffer for the ratio-128 boundary list of a decode batch (see kvc_plan_decode)."""
    return torch.empty(2 * batch + 2, dtype=torch.int32, device=device)


def _boundaries(cr, boundaries, batch):
    _i32(boundaries)
    _dev(boundaries)
    if boundaries is not None and (cr != 128 or boundaries.numel() < 2 * batch + 2):
        raise KvcError("the boundary list is for ratio 128 and needs 2 * batch + 2 int32 entries")


def plan_decode(cr, seq_lens, state_index, num_state_rows, plan_d, status=None, stream=None, boundaries=None):
    _i32(seq_lens, state_index, status)
    _dev(seq_lens, state_index, plan_d, status)
    if state_index.numel() != seq_lens.numel():
        raise KvcError("seq_lens and state_index must have one entry per request")
    _shape(plan_d, seq_lens.numel(), D_BYTES, "plan_d")
    _boundaries(cr, boundaries, seq_lens.numel())
    rc = load().kvc_plan_decode(cr, seq_lens.numel(), _p(seq_lens), _p(state_index), num_state_rows, _p(plan_d),
                                _p(boundaries), _p(status), _stream(stream))
    _check(rc, "kvc_plan_decode")


def capacities_swa(cr: int, batch: int, num_q: int, swa_page_size: int):
    """Record capacities that always suffice for an SWA-paged prefill chunk (ratio 4 adds up to
    4 page-tail writes per SWA page)."""
    cap_w = batch * (WINDOW[cr] - 1) + (4 * (num_q // swa_page_size + batch) if cr == 4 else 0)
    return min(num_q, num_q // cr + batch), min(num_q, cap_w)


def plan_prefill_swa(cr, seq_lens, extend_lens, req_pool_indices, req_to_token, full_to_swa, swa_page_size,
                     ring_size, num_state_rows, num_q, plan_c, plan_w, counts, status=None, stream=None):
    """req_to_token: int32 [num_reqs, stride]; full_to_swa: int32 [num_full]."""
    _i32(seq_lens, extend_lens, req_pool_indices, req_to_token, full_to_swa, counts, status)
    _dev(seq_lens, extend_lens, req_pool_indices, req_to_token, full_to_swa, plan_c, plan_w, counts, status)
    B = seq_lens.numel()
    if extend_lens.numel() != B or req_pool_indices.numel() != B or counts.numel() < 4 or req_to_token.dim() != 2:
        raise KvcError("one length and one request slot per request, counts 4, req_to_token 2-D")
    _shape(plan_c, 0, C_BYTES, "plan_c")
    _shape(plan_w, 0, W_BYTES, "plan_w")
    rc = load().kvc_plan_prefill_swa(cr, B, num_q, _p(seq_lens), _p(extend_lens), _p(req_pool_indices),
                                     _p(req_to_token), req_to_token.shape[1], req_to_token.shape[0],
                                     _p(full_to_swa), full_to_swa.numel(), swa_page_size, ring_size, num_state_rows,
                                     _p(plan_c), plan_c.shape[0], _p(plan_w), plan_w.shape[0], _p(counts),
                                     _p(status), _stream(stream))
    _check(rc, "kvc_plan_prefill_swa")


def plan_decode_swa(cr, seq_lens, req_pool_indices, req_to_token, full_to_swa, swa_page_size, ring_size,
                    num_state_rows, plan_d, status=None, stream=None, boundaries=None):
    _i32(seq_lens, req_pool_indices, req_to_token, full_to_swa, status)
    _dev(seq_lens, req_pool_indices, req_to_token, full_to_swa, plan_d, status)
    if req_pool_indices.numel() != seq_lens.numel() or req_to_token.dim() != 2:
        raise KvcError("one request slot per request, req_to_token 2-D")
    _shape(plan_d, seq_lens.numel(), D_BYTES, "plan_d")
    _boundaries(cr, boundaries, seq_lens.numel())
    rc = load().kvc_plan_decode_swa(cr, seq_lens.numel(), _p(seq_lens), _p(req_pool_indices), _p(req_to_token),
                                    req_to_token.shape[1], req_to_token.shape[0], _p(full_to_swa),
                                    full_to_swa.numel(), swa_page_size, ring_size, num_state_rows, _p(plan_d),
                                    _p(boundaries), _p(status), _stream(stream))
    _check(rc, "kvc_plan_decode_swa")


def plan_prefill_page4(seq_lens, extend_lens, page_index, bundle, num_state_rows, num_q, plan_c, plan_w, counts,
                       status=None, stream=None):
    """Ratio-4 prefill plan over caller-allocated 4-row pages; bundle: int32 [batch, 4]."""
    _i32(seq_lens, extend_lens, page_index, bundle, counts, status)
    _dev(seq_lens, extend_lens, page_index, bundle, plan_c, plan_w, counts, status)
    B = seq_lens.numel()
    if tuple(bundle.shape) != (B, 4):
        raise KvcError("bundle must be int32 [batch, 4]")
    if extend_lens.numel() != B or page_index.numel() != B or counts.numel() < 4:
        raise KvcError("seq_lens, extend_lens, page_index must have one entry per request; counts 4")
    _shape(plan_c, 0, C_BYTES, "plan_c")
    _shape(plan_w, 0, W_BYTES, "plan_w")
    rc = load().kvc_plan_prefill_page4(B, num_q, _p(seq_lens), _p(extend_lens), _p(page_index), _p(bundle),
                                       num_state_rows, _p(plan_c), plan_c.shape[0], _p(plan_w), plan_w.shape[0],
                                       _p(counts), _p(status), _stream(stream))
    _check(rc, "kvc_plan_prefill_page4")


def plan_decode_page4(seq_lens, page_index, prev_page, num_state_rows, plan_d, status=None, stream=None):
    _i32(seq_lens, page_index, prev_page, status)
    _dev(seq_lens, page_index, prev_page, plan_d, status)
    if page_index.numel() != seq_lens.numel() or prev_page.numel() != seq_lens.numel():
        raise KvcError("seq_lens, page_index and prev_page must have one entry per request")
    _shape(plan_d, seq_lens.numel(), D_BYTES, "plan_d")
    rc = load().kvc_plan_decode_page4(seq_lens.numel(), _p(seq_lens), _p(page_index), _p(prev_page), num_state_rows,
                                      _p(plan_d), _p(status), _stream(stream))
    _check(rc, "kvc_plan_decode_page4")


def write(cr, head_dim, state, inp, plan_w, counts, stream=None):
    _i32(counts)
    _dev(state, inp, plan_w, counts)
    _rows(cr, head_dim, state, inp)
    _shape(plan_w, 0, W_BYTES, "plan_w")
    rc = load().kvc_write(cr, _dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), inp.shape[0], _p(plan_w),
                          plan_w.shape[0], _p(counts), _stream(stream))
    _check(rc, "kvc_write")


def compress_c4(head_dim, state, inp, ape, plan_c, counts, out, stream=None):
    _i32(counts)
    _dev(state, inp, ape, plan_c, counts, out)
    _rows(4, head_dim, state, inp)
    _shape(ape, WINDOW[4], head_dim, "ape")
    _shape(plan_c, 0, C_BYTES, "plan_c")
    _shape(out, plan_c.shape[0], head_dim, "out")
    if out.dtype != torch.float32 or ape.element_size() != inp.element_size():
        raise KvcError("out must be float32 and ape share the input dtype")
    rc = load().kvc_compress_c4(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), inp.shape[0], _p(ape),
                                _p(plan_c), plan_c.shape[0], _p(counts), _p(out), _stream(stream))
    _check(rc, "kvc_compress_c4")


def compress_c128(head_dim, state, inp, ape, plan_c, counts, out, stream=None):
    _i32(counts)
    _dev(state, inp, ape, plan_c, counts, out)
    _rows(128, head_dim, state, inp)
    _shape(ape, WINDOW[128], head_dim, "ape")
    _shape(plan_c, 0, C_BYTES, "plan_c")
    _shape(out, plan_c.shape[0], head_dim, "out")
    if out.dtype != torch.float32 or ape.element_size() != inp.element_size():
        raise KvcError("out must be float32 and ape share the input dtype")
    rc = load().kvc_compress_c128(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), inp.shape[0],
                                  _p(ape), _p(plan_c), plan_c.shape[0], _p(counts), _p(out), _stream(stream))
    _check(rc, "kvc_compress_c128")


def compress(cr, head_dim, state, inp, ape, plan_c, counts, out, stream=None):
    (compress_c4 if cr == 4 else compress_c128)(head_dim, state, inp, ape, plan_c, counts, out, stream)


# --------------------------------------------------------------------------
# norm + rotary embedding + bf16 store of the compressed rows
# --------------------------------------------------------------------------

class StoreArgs(ctypes.Structure):
    """kvc_store_args of include/kvc.h."""
    _fields_ = [("norm_weight", ctypes.c_void_p), ("freqs_cis", ctypes.c_void_p), ("out_loc", ctypes.c_void_p),
                ("cache", ctypes.c_void_p), ("num_loc", ctypes.c_int64), ("max_position", ctypes.c_int64),
                ("num_cache_rows", ctypes.c_int64), ("eps", ctypes.c_float), ("rope_dim", ctypes.c_int32)]


def store_args(head_dim, norm_weight, eps, freqs_cis, out_loc, cache):
    """Pack the store parameters.  norm_weight: float32 [head_dim]; freqs_cis:
    float32 [max_position, rope_dim / 2, 2] (cos, sin), or None for no rotated
    channels; out_loc: int32 [num_loc]; cache: bf16 (or 16-bit bits) [rows, head_dim]."""
    _dev(norm_weight, freqs_cis, out_loc, cache)
    if norm_weight.dtype != torch.float32 or norm_weight.numel() != head_dim:
        raise KvcError("norm_weight must be float32 [%d]" % head_dim)
    if out_loc.dtype != torch.int32 or out_loc.dim() != 1:
        raise KvcError("out_loc must be a 1-D int32 tensor")
    _shape(cache, 0, head_dim, "cache")
    if cache.element_size() != 2:
        raise KvcError("cache must hold bf16 rows")
    if freqs_cis is None or freqs_cis.numel() == 0:
        rope_dim, max_pos, fptr = 0, 0, None
    else:
        if freqs_cis.dtype != torch.float32 or freqs_cis.dim() != 3 or freqs_cis.shape[2] != 2:
            raise KvcError("freqs_cis must be float32 [max_position, rope_dim / 2, 2]")
        rope_dim, max_pos, fptr = 2 * freqs_cis.shape[1], freqs_cis.shape[0], freqs_cis.data_ptr()
    return StoreArgs(norm_weight.data_ptr(), fptr, out_loc.data_ptr(), cache.data_ptr(), out_loc.numel(), max_pos,
                     cache.shape[0], float(eps), rope_dim)


def norm_rope_store_prefill(cr, rows, plan_c, counts, norm_weight, eps, freqs_cis, out_loc, cache, stream=None):
    """Store row k of rows (float32 [cap_c, hd]) for every valid C record k < counts[0]."""
    _i32(counts)
    _dev(rows, plan_c, counts)
    hd = rows.shape[1]
    _shape(plan_c, 0, C_BYTES, "plan_c")
    _shape(rows, plan_c.shape[0], hd, "rows")
    if rows.dtype != torch.float32:
        raise KvcError("rows must be float32")
    st = store_args(hd, norm_weight, eps, freqs_cis, out_loc, cache)
    rc = load().kvc_norm_rope_store_prefill(cr, hd, _p(rows), _p(plan_c), plan_c.shape[0], _p(counts),
                                            ctypes.byref(st), _stream(stream))
    _check(rc, "kvc_norm_rope_store_prefill")


def norm_rope_store_decode(cr, rows, plan_d, norm_weight, eps, freqs_cis, out_loc, cache, status=None, stream=None):
    """Store row b of rows (float32 [batch, hd]) for every D record that closes a block."""
    _i32(status)
    _dev(rows, plan_d, status)
    hd = rows.shape[1]
    _shape(plan_d, 1, D_BYTES, "plan_d")
    _shape(rows, plan_d.shape[0], hd, "rows")
    if rows.dtype != torch.float32:
        raise KvcError("rows must be float32")
    st = store_args(hd, norm_weight, eps, freqs_cis, out_loc, cache)
    rc = load().kvc_norm_rope_store_decode(cr, hd, _p(rows), _p(plan_d), plan_d.shape[0], _p(status),
                                           ctypes.byref(st), _stream(stream))
    _check(rc, "kvc_norm_rope_store_decode")


def compress_norm_rope_store(cr, head_dim, state, inp, ape, plan_c, counts, norm_weight, eps, freqs_cis, out_loc,
                             cache, stream=None):
    """Pool, norm, rotate and store in one kernel (kvc_compress_c{4,128}_norm_rope_store)."""
    _i32(counts)
    _dev(state, inp, ape, plan_c, counts)
    _rows(cr, head_dim, state, inp)
    _shape(ape, WINDOW[cr], head_dim, "ape")
    _shape(plan_c, 0, C_BYTES, "plan_c")
    if ape.element_size() != inp.element_size():
        raise KvcError("ape must share the input dtype")
    st = store_args(head_dim, norm_weight, eps, freqs_cis, out_loc, cache)
    fn = load().kvc_compress_c4_norm_rope_store if cr == 4 else load().kvc_compress_c128_norm_rope_store
    rc = fn(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), inp.shape[0], _p(ape), _p(plan_c),
            plan_c.shape[0], _p(counts), ctypes.byref(st), _stream(stream))
    _check(rc, "kvc_compress_c%d_norm_rope_store" % cr)


def decode_c4_norm_rope_store(head_dim, state, inp, ape, plan_d, norm_weight, eps, freqs_cis, out_loc, cache,
                              status=None, stream=None):
    """Ratio-4 decode with the store step in one kernel (kvc_decode_c4_norm_rope_store)."""
    _i32(status)
    _dev(state, inp, ape, plan_d, status)
    _rows(4, head_dim, state, inp)
    _shape(ape, WINDOW[4], head_dim, "ape")
    _shape(plan_d, 1, D_BYTES, "plan_d")
    _shape(inp, plan_d.shape[0], 4 * head_dim, "input")
    if ape.element_size() != inp.element_size():
        raise KvcError("ape must share the input dtype")
    st = store_args(head_dim, norm_weight, eps, freqs_cis, out_loc, cache)
    rc = load().kvc_decode_c4_norm_rope_store(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), _p(ape),
                                              _p(plan_d), plan_d.shape[0], _p(status), ctypes.byref(st),
                                              _stream(stream))
    _check(rc, "kvc_decode_c4_norm_rope_store")


# --------------------------------------------------------------------------
# online ratio-128 state: slots float32 [num_slots, 3, hd] (m, l, acc)
# --------------------------------------------------------------------------

def _online_state(state, head_dim):
    if state.dtype != torch.float32 or state.dim() != 3 or tuple(state.shape[1:]) != (3, head_dim):
        raise KvcError("online state must be float32 [slots, 3, %d]" % head_dim)


def compress_c128_online(head_dim, state, inp, ape, plan_c, counts, out, stream=None):
    _i32(counts)
    _dev(state, inp, ape, plan_c, counts, out)
    _online_state(state, head_dim)
    _shape(inp, 0, 2 * head_dim, "input")
    _shape(ape, WINDOW[128], head_dim, "ape")
    _shape(plan_c, 0, C_BYTES, "plan_c")
    _shape(out, plan_c.shape[0], head_dim, "out")
    if out.dtype != torch.float32 or ape.element_size() != inp.element_size():
        raise KvcError("out must be float32 and ape share the input dtype")
    rc = load().kvc_compress_c128_online(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), inp.shape[0],
                                         _p(ape), _p(plan_c), plan_c.shape[0], _p(counts), _p(out), _stream(stream))
    _check(rc, "kvc_compress_c128_online")


def write_c128_online(head_dim, state, inp, ape, plan_w, counts, stream=None, runs=None):
    """runs: None (the runs are found in plan_w), or the run list the chunk's plan_prefill wrote."""
    _i32(counts, runs)
    _dev(state, inp, ape, plan_w, counts, runs)
    _online_state(state, head_dim)
    _shape(inp, 0, 2 * head_dim, "input")
    _shape(ape, WINDOW[128], head_dim, "ape")
    _shape(plan_w, 0, W_BYTES, "plan_w")
    if ape.element_size() != inp.element_size():
        raise KvcError("ape must share the input dtype")
    batch = 0
    if runs is not None:
        batch = runs.shape[0] if runs.dim() == 2 else -1
        _runs(128, runs, batch)
    rc = load().kvc_write_c128_online(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), inp.shape[0],
                                      _p(ape), _p(plan_w), plan_w.shape[0], _p(counts), _p(runs), batch,
                                      _stream(stream))
    _check(rc, "kvc_write_c128_online")


def decode_c128_online(head_dim, state, inp, ape, plan_d, out, status=None, stream=None):
    _i32(status)
    _dev(state, inp, ape, plan_d, out, status)
    _online_state(state, head_dim)
    _shape(plan_d, 1, D_BYTES, "plan_d")
    _shape(inp, plan_d.shape[0], 2 * head_dim, "input")
    _shape(ape, WINDOW[128], head_dim, "ape")
    _shape(out, plan_d.shape[0], head_dim, "out")
    if out.dtype != torch.float32 or ape.element_size() != inp.element_size():
        raise KvcError("out must be float32 and ape share the input dtype")
    rc = load().kvc_decode_c128_online(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), _p(ape),
                                       _p(plan_d), plan_d.shape[0], _p(status), _p(out), _stream(stream))
    _check(rc, "kvc_decode_c128_online")


def decode_c4(head_dim, state, inp, ape, plan_d, out, status=None, stream=None):
    _i32(status)
    _dev(state, inp, ape, plan_d, out, status)
    _rows(4, head_dim, state, inp)
    _shape(plan_d, 0, D_BYTES, "plan_d")
    B = plan_d.shape[0]
    _shape(inp, B, ROW_MULT[4] * head_dim, "input")
    _shape(ape, WINDOW[4], head_dim, "ape")
    _shape(out, B, head_dim, "out")
    if out.dtype != torch.float32 or ape.element_size() != inp.element_size():
        raise KvcError("out must be float32 and ape share the input dtype")
    rc = load().kvc_decode_c4(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), _p(ape), _p(plan_d),
                              plan_d.shape[0], _p(status), _p(out), _stream(stream))
    _check(rc, "kvc_decode_c4")


def decode_c128(head_dim, state, inp, ape, plan_d, out, status=None, stream=None, boundaries=None):
    """boundaries: the list kvc_plan_decode (or _swa) wrote with plan_d, or None."""
    _i32(status)
    _dev(state, inp, ape, plan_d, out, status)
    _rows(128, head_dim, state, inp)
    _shape(plan_d, 0, D_BYTES, "plan_d")
    B = plan_d.shape[0]
    _shape(inp, B, ROW_MULT[128] * head_dim, "input")
    _shape(ape, WINDOW[128], head_dim, "ape")
    _shape(out, B, head_dim, "out")
    _boundaries(128, boundaries, B)
    if out.dtype != torch.float32 or ape.element_size() != inp.element_size():
        raise KvcError("out must be float32 and ape share the input dtype")
    rc = load().kvc_decode_c128(_dtype(inp), head_dim, _p(state), state.shape[0], _p(inp), _p(ape), _p(plan_d),
                                _p(boundaries), plan_d.shape[0], _p(status), _p(out), _stream(stream))
    _check(rc, "kvc_decode_c128")


def decode(cr, head_dim, state, inp, ape, plan_d, out, status=None, stream=None, boundaries=None):
    if cr == 4:
        if boundaries is not None:
            raise KvcError("the boundary list is for ratio 128")
        decode_c4(head_dim, state, inp, ape, plan_d, out, status, stream)
    else:
        decode_c128(head_dim, state, inp, ape, plan_d, out, status, stream, boundaries)
