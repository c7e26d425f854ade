"""Seeded synthetic workloads for the KV compressor (inputs only).

This module draws lengths, state indices, kv/score inputs, ``ape`` and the
initial state buffer.  It holds none of the compressor's arithmetic: no plan,
no window, no softmax.  Tests and the benchmark feed the same host arrays to
the HIP library and to the CPU oracle.

Recipe (all draws from ``numpy.random.default_rng``):
  * lengths and state indices come from ``default_rng(seed)``, in the order
    lengths, then indices (a permutation of the available rings / pages,
    first B taken);
  * each compressor's tensors come from ``default_rng([seed, ratio])`` in the
    order input, ape, state; normals are float32 ``standard_normal`` scaled by
    the stated standard deviation; a tensor is drawn in chunks of 8192 rows,
    chunk k from the k-th child seed that the tensor's generator spawns;
  * bf16 tensors are the float32 draws rounded to nearest-even bf16 and are
    carried as uint16 bit patterns; fp32 tensors are carried as float32.
  * "uniform in [a, b]" means integers with both ends included.

Layouts: a row of the ratio-4 input/state is ``|kv overlap|kv|score overlap|
score|`` (4 x head_dim), a row of the ratio-128 input/state is ``|kv|score|``
(2 x head_dim).  The state buffer is a flat ``[num_state_rows, row]`` array:
ratio 4 gives each ring 8 rows, ratio 128 gives each page 128 rows.
"""
from __future__ import annotations

import concurrent.futures
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

WINDOW = {4: 8, 128: 128}
ROW_MULT = {4: 4, 128: 2}
CHUNK_ROWS = 8192


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return the uint16 bit patterns."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    return _round_in_place(u)


def _round_in_place(u: np.ndarray) -> np.ndarray:
    """u: float32 bit patterns (modified).  Returns the bf16 patterns (nearest, ties to even)."""
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_rows(rng, rows, cols, col_sigma, dtype):
    """[rows, cols] normals, column c scaled by col_sigma[c]; float32 or bf16 bits.

    Row chunk k (CHUNK_ROWS rows) is drawn from its own child generator
    ``default_rng(rng_seed.spawn)``: the values do not depend on how many
    threads draw them."""
    out = np.empty((rows, cols), np.uint16 if dtype == "bf16" else np.float32)
    sig = np.broadcast_to(np.asarray(col_sigma, np.float32), (cols,))
    scale = None if np.all(sig == 1.0) else np.ascontiguousarray(sig)
    nchunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    seeds = rng.bit_generator.seed_seq.spawn(max(nchunks, 1)) if hasattr(rng.bit_generator, "seed_seq") \
        else rng.bit_generator._seed_seq.spawn(max(nchunks, 1))

    def fill(k):
        r0, r1 = k * CHUNK_ROWS, min(rows, (k + 1) * CHUNK_ROWS)
        x = np.random.default_rng(seeds[k]).standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale is not None:
            x *= scale
        if dtype == "bf16":
            out[r0:r1] = _round_in_place(x.view(np.uint32))
        else:
            out[r0:r1] = x

    if nchunks > 1:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(nchunks)))
    elif nchunks == 1:
        fill(0)
    return out


@dataclass
class Workload:
    name: str
    cr: int                      # compress ratio, 4 or 128
    hd: int                      # head_dim
    dtype: str                   # "bf16" or "f32"
    kind: str                    # "prefill" or "decode"
    seq_lens: np.ndarray         # int32 [B]
    state_index: np.ndarray      # int32 [B]
    num_state_rows: int
    input: Optional[np.ndarray] = None   # [num_q or B, row]
    ape: Optional[np.ndarray] = None     # [W, hd]
    state: Optional[np.ndarray] = None   # [num_state_rows, row]
    extend_lens: Optional[np.ndarray] = None  # int32 [B] (prefill)
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_q(self) -> int:
        return int(self.extend_lens.sum()) if self.kind == "prefill" else self.B

    @property
    def row(self) -> int:
        return ROW_MULT[self.cr] * self.hd

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def fill_tensors(w: Workload, rng, kv_sigma=1.0, score_sigma=1.0, ape_sigma=0.1, state_sigma=1.0,
                 state_fill: Optional[float] = None) -> Workload:
    """Draw input, ape and state for a workload whose lengths/indices are set."""
    hd, R = w.hd, w.row
    sig = np.empty(R, np.float32)
    if w.cr == 4:
        sig[: 2 * hd] = kv_sigma
        sig[2 * hd:] = score_sigma
    else:
        sig[:hd] = kv_sigma
        sig[hd:] = score_sigma
    w.input = _normal_rows(rng, w.num_q, R, sig, w.dtype)
    w.ape = _normal_rows(rng, WINDOW[w.cr], hd, np.float32(ape_sigma), w.dtype)
    if state_fill is None:
        w.state = _normal_rows(rng, w.num_state_rows, R, np.float32(state_sigma), w.dtype)
    else:
        v = np.full((w.num_state_rows, R), state_fill, np.float32)
        w.state = to_bf16_bits(v) if w.dtype == "bf16" else v
    return w


def prefill_workload(name, cr, hd, dtype, seq_lens, extend_lens, state_index, num_slots, tensor_seed,
                     score_sigma=1.0, state_fill=None, with_tensors=True) -> Workload:
    """num_slots = number of rings (ratio 4) or pages (ratio 128) in the state buffer."""
    w = Workload(name=name, cr=cr, hd=hd, dtype=dtype, kind="prefill",
                 seq_lens=np.asarray(seq_lens, np.int32), extend_lens=np.asarray(extend_lens, np.int32),
                 state_index=np.asarray(state_index, np.int32), num_state_rows=num_slots * WINDOW[cr])
    if with_tensors:
        fill_tensors(w, np.random.default_rng(tensor_seed), score_sigma=score_sigma, state_fill=state_fill)
    return w


def decode_workload(name, cr, hd, dtype, seq_lens, state_index, num_slots, tensor_seed, state_fill=None,
                    with_tensors=True) -> Workload:
    w = Workload(name=name, cr=cr, hd=hd, dtype=dtype, kind="decode",
                 seq_lens=np.asarray(seq_lens, np.int32), state_index=np.asarray(state_index, np.int32),
                 num_state_rows=num_slots * WINDOW[cr])
    if with_tensors:
        fill_tensors(w, np.random.default_rng(tensor_seed), state_fill=state_fill)
    return w


# --------------------------------------------------------------------------
# the named workloads: small ratio-4 prefill, ratio-128 prefill, the two decode
# batches and the mixed chunked prefill
# --------------------------------------------------------------------------

def c4_prefill_1x64(with_tensors=True):
    """c4 prefill, 1 request, prefix 0, extend 64, fp32, head_dim 128."""
    seed = 1001
    return prefill_workload("c4 prefill 1x64 fp32 hd128", 4, 128, "f32", [64], [64], [0], 1, [seed, 4],
                            with_tensors=with_tensors)


def c128_prefill_4req(with_tensors=True):
    """c128 prefill, 4 requests, prefix 0, extends uniform in [1, 2048], bf16, head_dim 512."""
    seed = 1002
    rng = np.random.default_rng(seed)
    e = rng.integers(1, 2048, size=4, endpoint=True)
    idx = rng.permutation(4)
    return prefill_workload("c128 prefill 4 req e~U[1,2048] bf16 hd512", 128, 512, "bf16", e, e, idx, 4,
                            [seed, 128], score_sigma=2.0, with_tensors=with_tensors)


def c4_decode_b256(with_tensors=True):
    """c4 decode, batch 256, prefixes uniform in [1, 32768], bf16, head_dim 512."""
    seed = 1003
    rng = np.random.default_rng(seed)
    prefix = rng.integers(1, 32768, size=256, endpoint=True)
    idx = rng.permutation(256)
    return decode_workload("c4 decode B256 bf16 hd512", 4, 512, "bf16", prefix + 1, idx, 256, [seed, 4],
                           with_tensors=with_tensors)


def c128_decode_b1024(with_tensors=True):
    """c128 decode, batch 1024, prefixes uniform in [1, 65536], bf16, head_dim 512."""
    seed = 1004
    rng = np.random.default_rng(seed)
    prefix = rng.integers(1, 65536, size=1024, endpoint=True)
    idx = rng.permutation(1024)
    return decode_workload("c128 decode B1024 bf16 hd512", 128, 512, "bf16", prefix + 1, idx, 1024, [seed, 128],
                           with_tensors=with_tensors)


def mixed_prefill_lens(uniform_extend: Optional[int] = None):
    seed = 1005
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, 65536, size=64, endpoint=True)
    if uniform_extend is None:
        e = rng.integers(1, 4096, size=64, endpoint=True)
    else:
        e = np.full(64, uniform_extend, np.int64)
    idx = rng.permutation(64)
    return prefix + e, e, idx


def mixed_prefill(cr, uniform_extend: Optional[int] = None, with_tensors=True):
    """Mixed chunked prefill, 64 requests, prefixes in [0, 65536], extends in [1, 4096] (or all equal).

    The same lengths and indices serve ratio 4 and ratio 128."""
    s, e, idx = mixed_prefill_lens(uniform_extend)
    tag = "mixed" if uniform_extend is None else "uniform e=%d" % uniform_extend
    seed = [1005, cr] if uniform_extend is None else [1005, cr, uniform_extend]
    return prefill_workload("c%d %s prefill 64 req bf16 hd512" % (cr, tag), cr, 512, "bf16", s, e, idx, 64,
                            seed, with_tensors=with_tensors)


def random_prefill(rng, cr, hd, dtype, B, prefix_hi, extend_lo, extend_hi, num_slots=None, state_fill=None):
    """A random ragged prefill batch for tests (prefixes uniform in [0, prefix_hi])."""
    prefix = rng.integers(0, prefix_hi, size=B, endpoint=True)
    e = rng.integers(extend_lo, extend_hi, size=B, endpoint=True)
    num_slots = num_slots or B
    idx = rng.permutation(num_slots)[:B]
    w = prefill_workload("random", cr, hd, dtype, prefix + e, e, idx, num_slots, None, with_tensors=False)
    return fill_tensors(w, rng, state_fill=state_fill)


def random_decode(rng, cr, hd, dtype, B, prefix_hi, num_slots=None, state_fill=None):
    prefix = rng.integers(0, prefix_hi, size=B, endpoint=True)
    num_slots = num_slots or B
    idx = rng.permutation(num_slots)[:B]
    w = decode_workload("random", cr, hd, dtype, prefix + 1, idx, num_slots, None, with_tensors=False)
    return fill_tensors(w, rng, state_fill=state_fill)


# --------------------------------------------------------------------------
# SWA-paged state: index tables (inputs of the SWA planners)
# --------------------------------------------------------------------------

def swa_tables(rng, max_len, num_reqs, swa_page_size, stride=None):
    """Index tables of a paged sliding-window pool, as a serving system would hold them.

    req_to_token[rid, pos] is the token's slot in the full KV cache (a random
    permutation of all num_reqs * stride slots); full_to_swa[slot] is its slot
    in the SWA pool: each (request, pos // swa_page_size) gets its own SWA page,
    drawn from a shuffled pool, and the token sits at page * swa_page_size +
    pos % swa_page_size.  Returns (req_to_token int32 [num_reqs, stride],
    full_to_swa int32 [num_reqs * stride], number of SWA pages)."""
    stride = stride or max_len
    pages_per_req = (stride + swa_page_size - 1) // swa_page_size
    num_pages = num_reqs * pages_per_req
    page_of = rng.permutation(num_pages).reshape(num_reqs, pages_per_req)
    full = rng.permutation(num_reqs * stride).astype(np.int64).reshape(num_reqs, stride)
    pos = np.arange(stride)
    swa = page_of[:, pos // swa_page_size] * swa_page_size + pos % swa_page_size
    f2s = np.empty(num_reqs * stride, np.int64)
    f2s[full.ravel()] = swa.ravel()
    return full.astype(np.int32), f2s.astype(np.int32), int(num_pages)


@dataclass
class StoreInputs:
    """Inputs of the norm / rotary / store step that follows the pool."""
    norm_weight: np.ndarray  # float32 [hd]
    eps: float
    freqs_cis: np.ndarray    # float32 [max_position, rope_dim / 2, 2] (cos, sin)
    out_loc: np.ndarray      # int32 [num_loc], distinct cache rows
    num_cache_rows: int


def rope_table(max_position: int, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """A rotary table as a caller would pass it: angle p * base^(-2k / rope_dim)
    for position p and pair k, stored as float32 (cos, sin)."""
    if rope_dim == 0:
        return np.zeros((0, 0, 2), np.float32)
    inv = base ** (-np.arange(0, rope_dim, 2, dtype=np.float64) / rope_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def store_inputs(rng, hd: int, rope_dim: int, max_position: int, num_loc: int, spare_rows: int = 7,
                 eps: float = 1e-6) -> StoreInputs:
    """Norm weight ~ N(1, 0.1); out_loc = the first num_loc entries of a
    permutation of num_loc + spare_rows cache rows (all distinct)."""
    w = (1.0 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    rows = num_loc + spare_rows
    loc = rng.permutation(rows)[:num_loc].astype(np.int32)
    return StoreInputs(w, eps, rope_table(max_position, rope_dim), loc, rows)
