"""Benchmark of the KV-compressor hot path on one MI355X.

One step is one pass of the whole path over the named workloads, all through
the C ABI on one HIP stream:
  * ratio-4 mixed chunked prefill: 64 requests, prefixes in [0, 65536],
    extends in [1, 4096] (~131k tokens), bf16, head_dim 512:
    kvc_plan_prefill -> kvc_compress_c4 -> kvc_write;
  * ratio-128 prefill over the same ragged batch:
    kvc_plan_prefill -> kvc_compress_c128 -> kvc_write;
  * ratio-4 decode, batch 256: kvc_plan_decode -> kvc_decode_c4;
  * ratio-128 decode, batch 1024: kvc_plan_decode -> kvc_decode_c128.
Inputs are synthetic (seeded normals), resident in HBM before timing starts.

value = tokens consumed per second (each compressor pass counts its tokens,
decode one token per request), over K steps run back to back.  The roofline
object reports the dominant kernel (kvc_compress_c4 on the prefill batch):
algorithmic bytes per launch divided by its average duration, timed with HIP
events on the launch stream over the timed region ("cache": "warm"), and its
cold-cache time beside it.  After the timed region, untimed passes give:
  * every launch's time and algorithmic GB/s (step_rows, f_rows);
  * the four kernels of the step with cold caches: before each launch the
    state is restored from a pristine copy and then 1 GiB is read (cold_us,
    cold_frac);
  * each named workload as its own chain (configs): the ratio-4 prefill of one
    64-token request (fp32, head_dim 128) and the ratio-128 prefill of four
    requests, plan -> compress -> write; the two decode batches, plan ->
    decode; launched one by one and as a replayed HIP graph;
  * the decode step as a replayed HIP graph, and the step on four streams;
  * same-box bandwidth ceilings: 16-byte-vector streams over 1 GiB (a copy,
    8 reads per write, reads only) from probe/libstream_probe.so, and the
    dominant kernel's GB/s as a fraction of the copy and of the 8:1 stream.
cpu_baseline times the float64 C oracle over the same step on the host cores
(all this process may use, up to 16, then one).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--sweep]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "compressed tokens/s and achieved HBM GB/s (% of peak), c4 & c128 prefill+decode"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=7)
    ap.add_argument("--sweep", action="store_true",
                    help="also time the compress and decode kernels over growing workloads (reported under "
                         "'sweep')")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device to device 5 times (calibrates the HBM byte counters), then "
                         "time plain one-read-one-write streams of 128 MiB to 1 GiB")
    return ap.parse_args()


# Sources of the dominant kernel: the traffic figure is only reported while they are
# unchanged since the counters in TRAFFIC_FILE were taken.
KERNEL_SOURCES = ["sparse_attention_kv_plan_amd/csrc/kvc_compress.hip", "sparse_attention_kv_plan_amd/csrc/kvc_pool.hpp",
                  "sparse_attention_kv_plan_amd/csrc/kvc_device.hpp", "sparse_attention_kv_plan_amd/csrc/kvc_store.hpp"]
TRAFFIC_FILE = "profiles/compress_c4_mixed_prefill_traffic.md"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or None.

    The summary holds lines "key: value"; it is used only if its source hash matches."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|", "`")):
                k, v = line.split(":", 1)
                kv[k.strip().lstrip("-* ").strip()] = v.strip().strip("`")
    if kv.get("kernel source hash") != kernel_source_hash():
        return None
    try:
        return int(float(kv["HBM bytes per launch"]))
    except (KeyError, ValueError):
        return None


def copy_probe():
    """A 1 GiB device-to-device copy, 5 times (the byte counters' calibration: every byte is read once
    and written once), then the plain streams that bound a kernel reading as many bytes as it writes,
    128 MiB to 1 GiB each way: torch's copy (the runtime's blit kernel) and torch's elementwise negation
    (a vector kernel, one read and one write per element), warm (back to back) and cold (1 GiB read
    between launches), medians of 20."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    print(json.dumps({"copy_probe_bytes": n, "copies": 5, "ms_per_copy": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
    flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    streams = []
    for mib in (128, 256, 512, 1024):
        m = mib << 20
        s64, d64 = src[:m].view(torch.int64), dst[:m].view(torch.int64)
        for kind, f in (("copy_", lambda: d64.copy_(s64)), ("neg", lambda: torch.neg(s64, out=d64))):
            for cold in (False, True):
                ts = []
                for _ in range(22):
                    if cold:
                        flush_caches(flush)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    f()
                    e1.record()
                    ts.append((e0, e1))
                torch.cuda.synchronize()
                us = float(np.median([x.elapsed_time(y) for x, y in ts[2:]])) * 1e3
                streams.append({"MiB_each_way": mib, "kernel": kind, "cache": "cold" if cold else "warm",
                                "us": round(us, 2), "GBps": round(2 * m / (us * 1e-6) / 1e9, 1)})
    print(json.dumps({"read1_write1_streams": streams}), flush=True)


def algorithmic_bytes_compress(cr, hd, esize, seq_lens_of_rows):
    """Bytes the pool must move: every kv and score element of the kept window entries once,
    the fp32 output row, the 16-byte record; ape once per launch."""
    W = 8 if cr == 4 else 128
    kept = np.where((cr == 4) & (seq_lens_of_rows == 4), 4, W)
    per_row = kept * 2 * hd * esize + hd * 4 + 16
    return int(per_row.sum()) + W * hd * esize


def algorithmic_bytes_store(hd, rope_dim, rows):
    """Bytes the standalone store must move: the fp32 row in, the bf16 row out, the record, the
    out_loc entry and the row of the rotary table; the norm weight once per launch."""
    return rows * (hd * 4 + hd * 2 + 16 + 4 + rope_dim * 4) + hd * 4


def algorithmic_bytes_fused_store(cr, hd, esize, seq_lens_of_rows, rope_dim):
    """The pool's bytes with the bf16 row, the out_loc entry and the table row in place of the fp32 row."""
    rows = len(seq_lens_of_rows)
    return (algorithmic_bytes_compress(cr, hd, esize, seq_lens_of_rows) + rows * (hd * 2 + 4 + rope_dim * 4 - hd * 4)
            + hd * 4)


def algorithmic_bytes_decode(cr, hd, esize, seq_lens):
    """Bytes a fused decode must move: the new row in and out of the state, the fp32 output row and
    the record per request; on a boundary the window's other entries (3 of them at seq_len 4 for
    ratio 4) from the state; ape once."""
    R = (4 if cr == 4 else 2) * hd
    W = 8 if cr == 4 else 128
    s = np.asarray(seq_lens, np.int64)
    boundary = s % cr == 0
    others = np.where((cr == 4) & (s == 4), 3, W - 1)
    per = 2 * R * esize + hd * 4 + 16 + np.where(boundary, others * 2 * hd * esize, 0)
    return int(per.sum()) + W * hd * esize


def algorithmic_bytes_plan_prefill(B, cap_c, cap_w):
    """Bytes a prefill planner must move: three int32 per request in, every record slot out (records
    and their invalid padding), the four counters."""
    return 12 * B + 16 * cap_c + 8 * cap_w + 16


def algorithmic_bytes_plan_decode(B, n_list=None):
    """Bytes a decode planner must move: two int32 per request in, one 16-byte record out, and with
    a ratio-128 boundary list its n_list entries and the count (8 bytes each)."""
    return 8 * B + 16 * B + (0 if n_list is None else 8 * n_list + 8)


def algorithmic_bytes_write(cr, hd, esize, num_w):
    """Bytes the state write must move: each written input row read once and stored once, plus its
    8-byte record."""
    R = (4 if cr == 4 else 2) * hd
    return num_w * (2 * R * esize + 8)


def algorithmic_bytes_store_decode(hd, rope_dim, seq_lens, cr):
    """Bytes the standalone decode store must move: every record; for a request that closes a block
    the fp32 row in, the bf16 row out, its out_loc entry and rotary row; the norm weight once."""
    boundary = int((np.asarray(seq_lens, np.int64) % cr == 0).sum())
    return len(seq_lens) * 16 + boundary * (hd * 4 + hd * 2 + 4 + rope_dim * 4) + hd * 4


def algorithmic_bytes_fused_decode_store(hd, esize, seq_lens, rope_dim):
    """Ratio-4 decode with the store fused: the decode's bytes with the boundary rows stored as bf16
    (plus out_loc and the rotary row) instead of every fp32 output row."""
    s = np.asarray(seq_lens, np.int64)
    boundary = s % 4 == 0
    others = np.where(s == 4, 3, 7)
    per = 2 * 4 * hd * esize + 16 + np.where(boundary, others * 2 * hd * esize + hd * 2 + 4 + rope_dim * 4, 0)
    return int(per.sum()) + 8 * hd * esize + hd * 4


def algorithmic_bytes_online(hd, esize, blen_of_rows, write_runs, decode_seq_lens):
    """The online ratio-128 calls.  Pool: per row the (128 - buffer_len) input entries, the slot's
    partial when buffer_len > 0, the fp32 row and the record; ape once.  State update: per run of n
    tokens the n rows and records, the old slot when the run continues a block, the new slot; ape
    once.  Decode: per request its row and record, the old slot unless it starts a block, the new
    slot and the fp32 output row; ape once."""
    slot = 3 * hd * 4
    blen = np.asarray(blen_of_rows, np.int64)
    pool = int(((128 - blen) * 2 * hd * esize + np.where(blen > 0, slot, 0) + hd * 4 + 16).sum())
    write = sum(n * (2 * hd * esize + 8) + (slot if cont else 0) + slot for n, cont in write_runs)
    s = np.asarray(decode_seq_lens, np.int64)
    fresh = (s - 1) % 128 == 0
    dec = int((2 * hd * esize + 16 + np.where(fresh, 0, slot) + slot + hd * 4).sum())
    ape = 128 * hd * esize
    return pool + ape, write + ape, dec + ape


def sweep(torch, kvc, dev, P4, P128, to_dev):
    """Extra, labelled results: kernel time and algorithmic GB/s as the work grows (prefill: the first
    k requests of the mixed batch; decode: batches with device-generated inputs), warm and with cold
    caches (1 GiB read before every launch, untimed).  Each decode batch also times a plain stream of
    the same algorithmic bytes (torch's elementwise negation, half of them read and half written) under
    the same two conditions; of_stream is the stream's time over the decode's."""
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device=dev)

    def med_us(f, n=10, cold=False):
        ts = []
        for _ in range(n + 2):
            if cold:
                flush_caches(flush_buf)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return round(float(np.median([a.elapsed_time(b) for a, b in ts[2:]])) * 1e3, 2)

    out = {"prefill": [], "decode": []}
    for P in (P4, P128):
        w = P.w
        for k in (1, 4, 16, 32, 64):
            nq = int(w.extend_lens[:k].sum())
            pc, pw, cnt = kvc.alloc_prefill_plan(w.cr, k, nq, dev)
            kvc.plan_prefill(w.cr, to_dev(w.seq_lens[:k]), to_dev(w.extend_lens[:k]), to_dev(w.state_index[:k]),
                             w.num_state_rows, nq, pc, pw, cnt)
            o = torch.empty((pc.shape[0], w.hd), dtype=torch.float32, device=dev)
            inp = P.inp[:nq]
            us = med_us(lambda: kvc.compress(w.cr, w.hd, P.state, inp, P.ape, pc, cnt, o))
            n = int(cnt[0].item())
            seqs = pc[:n].cpu().numpy().view("<u4").reshape(-1, 4)[:, 0].astype(np.int64)
            nbytes = algorithmic_bytes_compress(w.cr, w.hd, w.esize, seqs)
            cold_us = med_us(lambda: kvc.compress(w.cr, w.hd, P.state, inp, P.ape, pc, cnt, o), cold=True)
            out["prefill"].append({"ratio": w.cr, "requests": k, "tokens": nq, "rows": n, "us": us,
                                   "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "cold_us": cold_us,
                                   "cold_GBps": round(nbytes / (cold_us * 1e-6) / 1e9, 1)})
    hd = 512
    for cr, batches in ((4, (256, 1024, 4096, 16384, 65536)), (128, (1024, 4096, 16384, 32768))):
        R, W = (4 if cr == 4 else 2) * hd, (8 if cr == 4 else 128)
        for B in batches:
            rng = np.random.default_rng(5000 + cr + B)
            seq = (rng.integers(1, 65537, size=B) + 1).astype(np.int32)
            idx = rng.permutation(B).astype(np.int32)
            gen = torch.Generator(device=dev)
            gen.manual_seed(int(B) * 131 + cr)
            state = torch.randn((B * W, R), generator=gen, device=dev, dtype=torch.bfloat16)
            inp = torch.randn((B, R), generator=gen, device=dev, dtype=torch.bfloat16)
            ape = torch.randn((W, hd), generator=gen, device=dev, dtype=torch.bfloat16) * 0.1
            plan_d = torch.empty((B, kvc.D_BYTES), dtype=torch.uint8, device=dev)
            status = torch.zeros(1, dtype=torch.int32, device=dev)
            o = torch.empty((B, hd), dtype=torch.float32, device=dev)
            bl = kvc.boundary_list(B, dev) if cr == 128 else None
            kvc.plan_decode(cr, to_dev(seq), to_dev(idx), B * W, plan_d, status, boundaries=bl)
            us = med_us(lambda: kvc.decode(cr, hd, state, inp, ape, plan_d, o, status, boundaries=bl))
            cold_us = med_us(lambda: kvc.decode(cr, hd, state, inp, ape, plan_d, o, status, boundaries=bl), cold=True)
            # ratio 128 without the list: the pool workgroups rank the closing requests themselves
            scan_us = med_us(lambda: kvc.decode(cr, hd, state, inp, ape, plan_d, o, status)) if cr == 128 else None
            assert int(status.item()) == 0
            nbytes = algorithmic_bytes_decode(cr, hd, 2, seq)
            del state, inp
            # the ceiling at this size: a plain stream moving the same bytes, half read and half written
            half = max(nbytes // 16, 1)
            src = torch.ones(half, dtype=torch.int64, device=dev)
            dst = torch.empty_like(src)
            s_us = med_us(lambda: torch.neg(src, out=dst))
            s_cold = med_us(lambda: torch.neg(src, out=dst), cold=True)
            del src, dst
            out["decode"].append({"ratio": cr, "batch": B, "boundaries": int((seq % cr == 0).sum()), "us": us,
                                  "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "cold_us": cold_us,
                                  "cold_GBps": round(nbytes / (cold_us * 1e-6) / 1e9, 1),
                                  "stream_us": s_us, "stream_cold_us": s_cold,
                                  "of_stream": round(s_us / us, 3), "cold_of_stream": round(s_cold / cold_us, 3),
                                  "no_list_us": scan_us})
    del flush_buf
    torch.cuda.empty_cache()
    return out


def time_chain(torch, stream, named, n=50, warm=5):
    """Times of a chain of launches on `stream`: `named` is a list of (name, fn) run in order.  Each
    launch alone, bracketed by a pair of events (median over n; a pair adds a few microseconds of
    stream time, so a launch-bound kernel reads long), and the chain as the time of n chains run
    back to back divided by n.  Returns ({name: us}, chain_us)."""
    for _ in range(warm):
        for _, f in named:
            f()
    per = {name: [] for name, _ in named}
    for _ in range(n):
        for name, f in named:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            per[name].append((a, b))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        for _, f in named:
            f()
    b.record(stream)
    torch.cuda.synchronize()
    med = lambda pairs: round(float(np.median([x.elapsed_time(y) for x, y in pairs])) * 1e3, 2)  # noqa: E731
    return {name: med(v) for name, v in per.items()}, round(a.elapsed_time(b) * 1e3 / n, 2)


def time_graph(torch, stream, fns, n=100):
    """The chain `fns` captured once as a HIP graph (on a side stream) and replayed n times back to
    back on `stream`: the time per replay, without host launch gaps.  The chains hold no memset."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for f in fns:
                f()
    stream.wait_stream(side)
    for _ in range(5):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1e3 / n, 2)


def flush_caches(flush):
    """Read a 1 GiB buffer (untimed): afterwards L2 and the 256 MB last-level cache hold only its clean
    lines.  A flush by writing would leave up to 256 MB of dirty lines that the next kernel has to
    write back to HBM on its own time."""
    flush.sum(dtype=flush.dtype)


PROBE_KINDS = (("copy", 0, 2.0), ("read8_write1", 1, 1.125), ("read", 2, 1.0))  # name, kind, bytes moved per src byte


def load_stream_probe():
    """probe/libstream_probe.so: plain 16-byte-vector streams (copy, 8 reads per write, read only) that
    give the same-box bandwidth ceilings.  Built by the package's build step beside libkvc.so."""
    import ctypes

    import torch  # noqa: F401  (first: the library then binds to the HIP runtime torch has loaded)
    from sparse_attention_kv_plan_amd import build as hip_build
    if not os.path.exists(hip_build.PROBE_LIB):
        raise RuntimeError("%s is not built (python -m sparse_attention_kv_plan_amd.build)" % hip_build.PROBE_LIB)
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    lib.stream_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_void_p]
    lib.stream_probe.restype = ctypes.c_int
    return lib


def stream_ceilings(torch, stream, n=10):
    """Same-box bandwidth ceilings, measured beside the kernels (outside the timed step): 16-byte-vector
    streams over a 1 GiB source, with ordinary and with streaming (non-temporal) loads, warm (back to
    back) and cold (1 GiB read before each launch, untimed), medians of n launches on `stream`.  "copy"
    reads and writes every byte; "read8_write1" writes one vector per 8 read (the ratio-4 pool's mix of
    about 8 bytes in per byte out); "read" writes nothing.  GB/s count read plus written bytes.
    Back-to-back copies run slower than cold ones (each inherits the previous one's dirty lines in the
    last-level cache), so the ceiling of a stream is its best over both load kinds and both cache states.
    Returns (all entries, {name: that best GB/s})."""
    lib = load_stream_probe()
    m = 1 << 30
    src = torch.full((m // 8,), 0x0101010101010101, dtype=torch.int64, device=stream.device)
    dst = torch.empty_like(src)
    flush = torch.ones(1 << 27, dtype=torch.int64, device=stream.device)
    entries, best = [], {}
    for name, kind, per_byte in PROBE_KINDS:
        for nt in (0, 1):
            def launch():
                rc = lib.stream_probe(kind, nt, src.data_ptr(), m, dst.data_ptr(), m, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError("stream_probe(%d, %d) returned %d" % (kind, nt, rc))
            launch()
            for cold in (False, True):
                ts = []
                for _ in range(n + 2):
                    if cold:
                        flush_caches(flush)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    launch()
                    b.record(stream)
                    ts.append((a, b))
                torch.cuda.synchronize()
                us = float(np.median([a.elapsed_time(b) for a, b in ts[2:]])) * 1e3
                gbps = round(per_byte * m / (us * 1e-6) / 1e9, 1)
                entries.append({"stream": name, "loads": "nontemporal" if nt else "ordinary",
                                "cache": "cold" if cold else "warm", "us": round(us, 2), "GBps": gbps})
                best[name] = max(best.get(name, 0.0), gbps)
    del src, dst, flush
    return entries, best


def cold_times(torch, stream, cases, n=20):
    """Median time of each launch with cold caches: before every timed launch the state it reads or
    writes is restored from its pristine copy, then 1 GiB is read, so neither L2 nor the last-level
    cache holds any of its operands (both untimed).  cases: list of (name, fn, restore)."""
    flush = torch.ones(1 << 27, dtype=torch.int64, device=stream.device)
    out = {}
    for name, f, restore in cases:
        pairs = []
        for _ in range(n + 2):
            restore()
            flush_caches(flush)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            pairs.append((a, b))
        torch.cuda.synchronize()
        out[name] = round(float(np.median([a.elapsed_time(b) for a, b in pairs[2:]])) * 1e3, 2)
    del flush
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU: the compressor has no multi-GPU path in this library "
              "(requests shard across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_kv_plan_amd import kvc
    from sparse_attention_kv_plan_amd import workloads as wl

    kvc.load(build_if_missing=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    t0 = time.time()
    log("generating workloads ...")
    p4, p128 = wl.mixed_prefill(4), wl.mixed_prefill(128)
    d4, d128 = wl.c4_decode_b256(), wl.c128_decode_b1024()
    log("workloads ready in %.1f s: prefill num_q=%d, decode B=%d/%d" % (time.time() - t0, p4.num_q, d4.B, d128.B))

    class Prefill:
        def __init__(self, w):
            self.w = w
            self.s, self.e, self.idx = to_dev(w.seq_lens), to_dev(w.extend_lens), to_dev(w.state_index)
            self.inp, self.ape, self.state = to_dev(w.input), to_dev(w.ape), to_dev(w.state)
            self.pristine = self.state.clone()
            self.plan_c, self.plan_w, self.counts = kvc.alloc_prefill_plan(w.cr, w.B, w.num_q, dev)
            self.out = torch.empty((self.plan_c.shape[0], w.hd), dtype=torch.float32, device=dev)

        def restore(self):
            self.state.copy_(self.pristine)

        def plan(self):
            kvc.plan_prefill(self.w.cr, self.s, self.e, self.idx, self.w.num_state_rows, self.w.num_q,
                             self.plan_c, self.plan_w, self.counts)

        def compress(self):
            kvc.compress(self.w.cr, self.w.hd, self.state, self.inp, self.ape, self.plan_c, self.counts, self.out)

        def write(self):
            kvc.write(self.w.cr, self.w.hd, self.state, self.inp, self.plan_w, self.counts)

    class Decode:
        def __init__(self, w):
            self.w = w
            self.s, self.idx = to_dev(w.seq_lens), to_dev(w.state_index)
            self.inp, self.ape, self.state = to_dev(w.input), to_dev(w.ape), to_dev(w.state)
            self.pristine = self.state.clone()
            self.plan_d = torch.empty((w.B, kvc.D_BYTES), dtype=torch.uint8, device=dev)
            self.status = torch.zeros(1, dtype=torch.int32, device=dev)
            self.out = torch.empty((w.B, w.hd), dtype=torch.float32, device=dev)
            # ratio 128: the planner's boundary list feeds the decode's pool workgroups
            self.bl = kvc.boundary_list(w.B, dev) if w.cr == 128 else None

        def plan(self):
            kvc.plan_decode(self.w.cr, self.s, self.idx, self.w.num_state_rows, self.plan_d, self.status,
                            boundaries=self.bl)

        def decode(self):
            kvc.decode(self.w.cr, self.w.hd, self.state, self.inp, self.ape, self.plan_d, self.out, self.status,
                       boundaries=self.bl)

        def restore(self):
            self.state.copy_(self.pristine)

    P4, P128, D4, D128 = Prefill(p4), Prefill(p128), Decode(d4), Decode(d128)

    # SWA-paged planners over the same requests (timed in the breakdown pass only): SWA pages of
    # 128 tokens, ratio-4 rings of 8 rows, ratio-128 rings of 128 rows; each workload gets index
    # tables sized to its own requests
    def swa_tables_dev(w, seed):
        rng = np.random.default_rng(seed)
        r2t, f2s, npages = wl.swa_tables(rng, int(w.seq_lens.max()), w.B, 128)
        rows = npages * 8 if w.cr == 4 else w.B * 128
        return to_dev(r2t), to_dev(f2s), rows, to_dev(rng.permutation(w.B).astype(np.int32))

    class SwaPrefill:
        def __init__(self, w, seed):
            self.w = w
            self.r2t, self.f2s, self.rows, self.rid = swa_tables_dev(w, seed)
            self.s, self.e = to_dev(w.seq_lens), to_dev(w.extend_lens)
            cc, cw = kvc.capacities_swa(w.cr, w.B, w.num_q, 128)
            self.pc, self.pw, self.counts = kvc.alloc_prefill_plan(w.cr, w.B, w.num_q, dev, cap_c=cc, cap_w=cw)
            self.status = torch.zeros(1, dtype=torch.int32, device=dev)

        def plan(self):
            kvc.plan_prefill_swa(self.w.cr, self.s, self.e, self.rid, self.r2t, self.f2s, 128,
                                 8 if self.w.cr == 4 else 128, self.rows, self.w.num_q, self.pc, self.pw,
                                 self.counts, self.status)

    class SwaDecode:
        def __init__(self, w, seed):
            self.w = w
            self.r2t, self.f2s, self.rows, self.rid = swa_tables_dev(w, seed)
            self.s = to_dev(w.seq_lens)
            self.pd = torch.empty((w.B, kvc.D_BYTES), dtype=torch.uint8, device=dev)
            self.status = torch.zeros(1, dtype=torch.int32, device=dev)

        def plan(self):
            kvc.plan_decode_swa(self.w.cr, self.s, self.rid, self.r2t, self.f2s, 128, 8 if self.w.cr == 4 else 128,
                                self.rows, self.pd, self.status)

    # ratio 4 over caller-allocated 4-row pages (Page4Align): a page for every block of every request
    class Page4:
        def __init__(self, P, D, seed):
            rng = np.random.default_rng(seed)
            w, d = P.w, D.w
            p0 = (w.seq_lens - w.extend_lens).astype(np.int64)
            last = (w.seq_lens // 4) * 4
            n_pages = int((w.seq_lens // 4 + 4).sum() + (d.seq_lens // 4 + 4).sum())
            perm = rng.permutation(n_pages).astype(np.int32)
            base = np.concatenate([[0], np.cumsum(w.seq_lens // 4 + 4)])[:-1]  # request b's pages: base[b] + block

            def page(b, blk):
                return np.where(blk >= 0, perm[base[b] + np.maximum(blk, 0)], -1)

            b_ = np.arange(w.B)
            bundle = np.stack([page(b_, (p0 - 1) // 4 - 1) * (p0 > 4) - (p0 <= 4),
                               page(b_, (p0 - 1) // 4) * (p0 > 0) - (p0 <= 0),
                               page(b_, last // 4 - 1), last], axis=1).astype(np.int32)
            self.w, self.rows = w, n_pages * 4
            self.s, self.e = to_dev(w.seq_lens), to_dev(w.extend_lens)
            self.idx, self.bundle = to_dev(page(b_, last // 4).astype(np.int32)), to_dev(bundle)
            self.pc, self.pw, self.counts = kvc.alloc_prefill_plan(4, w.B, w.num_q, dev)
            self.status = torch.zeros(1, dtype=torch.int32, device=dev)
            # decode: the new token's page and the page before it, from the pages the prefill requests left
            dpages = perm[n_pages - 2 * d.B:]
            self.ds = to_dev(d.seq_lens)
            self.didx, self.dprev = to_dev(dpages[: d.B].copy()), to_dev(dpages[d.B:].copy())
            self.pd = torch.empty((d.B, kvc.D_BYTES), dtype=torch.uint8, device=dev)

        def plan(self):
            kvc.plan_prefill_page4(self.s, self.e, self.idx, self.bundle, self.rows, self.w.num_q, self.pc, self.pw,
                                   self.counts, self.status)

        def plan_decode(self):
            kvc.plan_decode_page4(self.ds, self.didx, self.dprev, self.rows, self.pd, self.status)

    PG4 = Page4(P4, D4, 2404)

    SP4, SP128, SD4 = SwaPrefill(p4, 2004), SwaPrefill(p128, 2128), SwaDecode(d4, 2003)
    swa_launches = [("plan_prefill_swa c4", SP4.plan), ("plan_prefill_swa c128", SP128.plan),
                    ("plan_decode_swa c4", SD4.plan), ("plan_prefill_page4", PG4.plan),
                    ("plan_decode_page4", PG4.plan_decode)]

    # norm + rotary + bf16 store of the compressed rows (breakdown pass only): rotary on the last 64
    # channels, one cache row per ragged token (prefill) or request (decode)
    class Store:
        def __init__(self, X, n, seed):
            self.X, w = X, X.w
            si = wl.store_inputs(np.random.default_rng(seed), w.hd, 64, int(w.seq_lens.max()) + 1, n)
            self.wt, self.f, self.loc = to_dev(si.norm_weight), to_dev(si.freqs_cis), to_dev(si.out_loc)
            self.cache = torch.empty((si.num_cache_rows, w.hd), dtype=torch.int16, device=dev)
            self.eps = si.eps

        def fused(self):
            X, w = self.X, self.X.w
            kvc.compress_norm_rope_store(w.cr, w.hd, X.state, X.inp, X.ape, X.plan_c, X.counts, self.wt, self.eps,
                                         self.f, self.loc, self.cache)

        def prefill(self):
            X = self.X
            kvc.norm_rope_store_prefill(X.w.cr, X.out, X.plan_c, X.counts, self.wt, self.eps, self.f, self.loc,
                                        self.cache)

        def decode(self):
            X = self.X
            kvc.norm_rope_store_decode(X.w.cr, X.out, X.plan_d, self.wt, self.eps, self.f, self.loc, self.cache,
                                       X.status)

        def fused_decode(self):
            X = self.X
            kvc.decode_c4_norm_rope_store(X.w.hd, X.state, X.inp, X.ape, X.plan_d, self.wt, self.eps, self.f,
                                          self.loc, self.cache, X.status)

    # the online ratio-128 state (breakdown pass only): one fp32 slot of (m, l, acc) per request
    # instead of a 128-row page, driven by the same plans
    class Online:
        def __init__(self, X, n, seed):
            self.X, w = X, X.w
            gen = torch.Generator(device=dev)
            gen.manual_seed(seed)
            self.slots = torch.randn((n, 3, w.hd), generator=gen, device=dev, dtype=torch.float32)
            self.slots[:, 1].abs_().add_(1.0)  # running sums are positive
            self.runs = None
            if hasattr(X, "plan_w"):  # a prefill chunk: plan it once more with the run list for the write
                self.runs = kvc.run_list(w.B, dev)
                self.plan_runs()

        def plan_runs(self):
            X, w = self.X, self.X.w
            kvc.plan_prefill(128, X.s, X.e, X.idx, w.num_state_rows, w.num_q, X.plan_c, X.plan_w, X.counts,
                             runs=self.runs)

        def compress(self):
            X, w = self.X, self.X.w
            kvc.compress_c128_online(w.hd, self.slots, X.inp, X.ape, X.plan_c, X.counts, X.out)

        def write(self):
            X, w = self.X, self.X.w
            kvc.write_c128_online(w.hd, self.slots, X.inp, X.ape, X.plan_w, X.counts, runs=self.runs)

        def write_scan(self):
            X, w = self.X, self.X.w
            kvc.write_c128_online(w.hd, self.slots, X.inp, X.ape, X.plan_w, X.counts)

        def decode(self):
            X, w = self.X, self.X.w
            kvc.decode_c128_online(w.hd, self.slots, X.inp, X.ape, X.plan_d, X.out, X.status)

    OP128, OD128 = Online(P128, p128.B, 4128), Online(D128, d128.B, 4129)
    online_launches = [("plan_prefill c128 runs", OP128.plan_runs), ("compress_c128_online", OP128.compress),
                       ("write_c128_online", OP128.write), ("write_c128_online scan", OP128.write_scan),
                       ("decode_c128_online", OD128.decode)]

    # the uniform-extend variant of the mixed batch (every extend 2, the multi-token-prediction shape):
    # the planner's equal-extend path, timed in the breakdown pass only
    M4, M128 = Prefill(wl.mixed_prefill(4, uniform_extend=2)), Prefill(wl.mixed_prefill(128, uniform_extend=2))
    OM128 = Online(M128, M128.w.B, 4130)  # the online state after the same chunk: 64 runs of 2 tokens
    mtp_launches = [("plan_prefill c4 e=2", M4.plan), ("compress_c4 e=2", M4.compress), ("write c4 e=2", M4.write),
                    ("plan_prefill c128 e=2", M128.plan), ("compress_c128 e=2", M128.compress),
                    ("write c128 e=2", M128.write), ("write_c128_online e=2", OM128.write),
                    ("write_c128_online scan e=2", OM128.write_scan)]

    ST4, ST128 = Store(P4, p4.num_q, 3004), Store(P128, p128.num_q, 3128)
    SD4S, SD128S = Store(D4, d4.B, 3003), Store(D128, d128.B, 3129)
    store_launches = [("compress_c4_norm_rope_store", ST4.fused), ("norm_rope_store_prefill c4", ST4.prefill),
                      ("compress_c128_norm_rope_store", ST128.fused),
                      ("norm_rope_store_prefill c128", ST128.prefill),
                      ("norm_rope_store_decode c4", SD4S.decode), ("norm_rope_store_decode c128", SD128S.decode),
                      ("decode_c4_norm_rope_store", SD4S.fused_decode)]

    launches = [("plan_prefill c4", P4.plan), ("compress_c4", P4.compress), ("write c4", P4.write),
                ("plan_prefill c128", P128.plan), ("compress_c128", P128.compress), ("write c128", P128.write),
                ("plan_decode c4", D4.plan), ("decode_c4", D4.decode),
                ("plan_decode c128", D128.plan), ("decode_c128", D128.decode)]
    dominant = "compress_c4"
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for name, f in launches:
            if ev is not None and name == dominant:
                ev[0].record(stream)
                f()
                ev[1].record(stream)
            else:
                f()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ----
    # the dominant kernel is bracketed by events on every EVENT_EVERY-th step (a bracketed step runs
    # about 13 us longer, so the pairs are kept few: 20 samples at K = 200)
    EVENT_EVERY = 10
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range((args.steps + EVENT_EVERY - 1) // EVENT_EVERY)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(kev[k // EVENT_EVERY] if k % EVENT_EVERY == 0 else None)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    dom_us = float(np.mean([a.elapsed_time(b) for a, b in kev])) * 1e3

    # per-kernel breakdown (separate, untimed pass; events around every launch), with the
    # SWA-paged planners of the same requests and the store step after the pool
    extra = swa_launches + store_launches + online_launches + mtp_launches
    bev = {name: [] for name, _ in launches + extra}
    for _ in range(5):
        for name, f in launches + extra:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            bev[name].append((a, b))
    torch.cuda.synchronize()
    kernels_us = {n: round(float(np.median([a.elapsed_time(b) for a, b in v])) * 1e3, 2) for n, v in bev.items()}

    # decode step alone (plan + fused decode for both ratios), eager and as a replayed HIP graph:
    # small launch-bound kernels, where the graph removes the launch gaps
    def decode_step():
        for name, f in launches[6:]:
            f()

    def per_call_ms(f, n=200):
        for _ in range(10):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    decode_us = {"eager": round(per_call_ms(decode_step) * 1e3, 2),
                 "graph": time_graph(torch, stream, [f for _, f in launches[6:]], n=200)}

    # The same step with its four chains on four streams (default priority).  The chains share no
    # buffer, so they are joined only at the two ends of the loop: a join in every step costs more
    # than the overlap saves.  Reported beside the headline, which stays on one stream so that the
    # dominant kernel's event time is its own.
    chain_streams = [stream] + [torch.cuda.Stream() for _ in range(3)]
    chains = [launches[0:3], launches[3:6], launches[6:8], launches[8:10]]

    def chains_once():
        for st, chain in zip(chain_streams, chains):
            with torch.cuda.stream(st):
                for _, f in chain:
                    f()

    for _ in range(10):
        chains_once()
    torch.cuda.synchronize()
    oa, ob = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    oa.record(stream)
    for st in chain_streams[1:]:
        st.wait_event(oa)
    for _ in range(args.steps):
        chains_once()
    for st in chain_streams[1:]:
        joined = torch.cuda.Event()
        joined.record(st)
        stream.wait_event(joined)
    ob.record(stream)
    torch.cuda.synchronize()
    overlap_ms = oa.elapsed_time(ob) / args.steps

    # the four kernels of the step with cold caches: state restored and 1 GiB read before every
    # launch (untimed); the headline loop above runs its steps back to back ("warm")
    cold = cold_times(torch, stream, [("compress_c4", P4.compress, P4.restore),
                                      ("compress_c128", P128.compress, P128.restore),
                                      ("decode_c4", D4.decode, D4.restore),
                                      ("decode_c128", D128.decode, D128.restore)])
    ceil_all, ceil = stream_ceilings(torch, stream)

    # the other named workloads, each timed as its own chain: the small ratio-4 prefill (1 request,
    # 64 tokens, fp32, head_dim 128) and the ratio-128 prefill of 4 requests (plan -> compress ->
    # write), and the two decode batches of the step (plan -> fused decode)
    configs = {}
    for name, w in (("c4_prefill_1x64", wl.c4_prefill_1x64()), ("c128_prefill_4req", wl.c128_prefill_4req())):
        X = Prefill(w)
        per, chain_us = time_chain(torch, stream, [("plan", X.plan), ("compress", X.compress), ("write", X.write)])
        graph_us = time_graph(torch, stream, [X.plan, X.compress, X.write])
        c = X.counts.cpu().tolist()
        assert c[2] == 0 and c[3] == 0, (name, c)
        seqs = X.plan_c[: c[0]].cpu().numpy().view("<u4").reshape(-1, 4)[:, 0].astype(np.int64)
        cb = algorithmic_bytes_compress(w.cr, w.hd, w.esize, seqs)
        wb = algorithmic_bytes_write(w.cr, w.hd, w.esize, c[1])
        configs[name] = {"tokens": w.num_q, "rows": c[0], "writes": c[1], "dtype": "f32" if w.esize == 4 else "bf16",
                         "head_dim": w.hd, "plan_us": per["plan"], "compress_us": per["compress"],
                         "write_us": per["write"], "chain_us": chain_us, "graph_chain_us": graph_us,
                         "tokens_per_s": round(w.num_q / (chain_us * 1e-6), 1),
                         "graph_tokens_per_s": round(w.num_q / (graph_us * 1e-6), 1),
                         "compress_bytes": cb, "compress_GBps": round(cb / (per["compress"] * 1e-6) / 1e9, 1),
                         "write_bytes": wb, "bound": "launch"}
        del X
    for name, D in (("c4_decode_b256", D4), ("c128_decode_b1024", D128)):
        per, chain_us = time_chain(torch, stream, [("plan", D.plan), ("decode", D.decode)])
        graph_us = time_graph(torch, stream, [D.plan, D.decode])
        db = algorithmic_bytes_decode(D.w.cr, D.w.hd, D.w.esize, D.w.seq_lens)
        configs[name] = {"tokens": D.w.B, "rows": int((D.w.seq_lens % D.w.cr == 0).sum()), "dtype": "bf16",
                         "head_dim": D.w.hd, "plan_us": per["plan"], "decode_us": per["decode"],
                         "chain_us": chain_us, "graph_chain_us": graph_us,
                         "tokens_per_s": round(D.w.B / (chain_us * 1e-6), 1),
                         "graph_tokens_per_s": round(D.w.B / (graph_us * 1e-6), 1),
                         "decode_bytes": db, "decode_GBps": round(db / (per["decode"] * 1e-6) / 1e9, 1),
                         "bound": "launch"}

    # sanity: no device-side errors, plans as sized
    for P in (P4, P128, M4, M128):
        c = P.counts.cpu().tolist()
        assert c[2] == 0 and c[3] == 0, ("device error", c)
    for D in (D4, D128):
        assert int(D.status.item()) == 0
    for S in (ST4, ST128):
        assert int(S.X.counts[3].item()) == 0
    for S in (SP4, SP128):
        c = S.counts.cpu().tolist()
        assert c[2] == 0 and int(S.status.item()) == 0, ("SWA plan error", c)
    assert int(SD4.status.item()) == 0
    assert int(PG4.counts[2].item()) == 0 and int(PG4.status.item()) == 0, "page-4 plan error"

    n_c4 = int(P4.counts[0].item())
    rows_seq = P4.plan_c[:n_c4].cpu().numpy().view("<u4").reshape(-1, 4)[:, 0].astype(np.int64)
    dom_bytes = algorithmic_bytes_compress(4, p4.hd, p4.esize, rows_seq)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    # the store step after the pool: fused into the pool vs pool into fp32 rows + standalone store
    store_step = {"rope_dim": 64}
    for cr, P, w in ((4, P4, p4), (128, P128, p128)):
        n = int(P.counts[0].item())
        seqs = P.plan_c[:n].cpu().numpy().view("<u4").reshape(-1, 4)[:, 0].astype(np.int64)
        fused_us = kernels_us["compress_c%d_norm_rope_store" % cr]
        two_us = kernels_us["compress_c%d" % cr] + kernels_us["norm_rope_store_prefill c%d" % cr]
        fb = algorithmic_bytes_fused_store(cr, w.hd, w.esize, seqs, 64)
        sb = algorithmic_bytes_store(w.hd, 64, n)
        store_step["c%d" % cr] = {
            "rows": n, "fused_us": fused_us, "pool_then_store_us": round(two_us, 2),
            "fused_GBps": round(fb / (fused_us * 1e-6) / 1e9, 1), "fused_bytes": fb,
            "store_only_GBps": round(sb / (kernels_us["norm_rope_store_prefill c%d" % cr] * 1e-6) / 1e9, 1),
            "store_only_bytes": sb}

    # every launch of the step against its bound: the pools stream HBM; the planners, the writes (a
    # few MB of rows behind a record load) and the fused decodes are chains of dependent loads
    def row_entry(name, nbytes, bound):
        us = kernels_us[name]
        gbps = nbytes / (us * 1e-6) / 1e9
        r = {"us": us, "bytes": int(nbytes), "GBps": round(gbps, 1), "frac": round(gbps / 8000.0, 4),
             "bound": bound}
        if name in cold:
            r["cold_us"] = cold[name]
            r["cold_frac"] = round(nbytes / (cold[name] * 1e-6) / 1e9 / 8000.0, 4)
        return r

    step_rows = {}
    for cr, P, w in ((4, P4, p4), (128, P128, p128)):
        c = P.counts.cpu().tolist()
        seqs = P.plan_c[: c[0]].cpu().numpy().view("<u4").reshape(-1, 4)[:, 0].astype(np.int64)
        step_rows["plan_prefill c%d" % cr] = row_entry(
            "plan_prefill c%d" % cr, algorithmic_bytes_plan_prefill(w.B, P.plan_c.shape[0], P.plan_w.shape[0]),
            "latency")
        step_rows["compress_c%d" % cr] = row_entry(
            "compress_c%d" % cr, algorithmic_bytes_compress(cr, w.hd, w.esize, seqs), "hbm")
        step_rows["write c%d" % cr] = row_entry(
            "write c%d" % cr, algorithmic_bytes_write(cr, w.hd, w.esize, c[1]), "latency")
    for cr, D, w in ((4, D4, d4), (128, D128, d128)):
        n_list = int((w.seq_lens % 128 == 0).sum()) if cr == 128 else None
        step_rows["plan_decode c%d" % cr] = row_entry(
            "plan_decode c%d" % cr, algorithmic_bytes_plan_decode(w.B, n_list), "latency")
        step_rows["decode_c%d" % cr] = row_entry(
            "decode_c%d" % cr, algorithmic_bytes_decode(cr, w.hd, w.esize, w.seq_lens), "latency")

    # the launches of the "next" rows against their bounds (breakdown-pass times): the store after the
    # pool, the online ratio-128 state, and the planners of the SWA-paged and Page4Align mappings
    f_rows = {}
    for cr, P, w in ((4, P4, p4), (128, P128, p128)):
        c = P.counts.cpu().tolist()
        seqs = P.plan_c[: c[0]].cpu().numpy().view("<u4").reshape(-1, 4)[:, 0].astype(np.int64)
        f_rows["compress_c%d_norm_rope_store" % cr] = row_entry(
            "compress_c%d_norm_rope_store" % cr, algorithmic_bytes_fused_store(cr, w.hd, w.esize, seqs, 64), "hbm")
        sb = algorithmic_bytes_store(w.hd, 64, c[0])  # 105 MB for ratio 4, 3 MB (latency-bound) for 128
        f_rows["norm_rope_store_prefill c%d" % cr] = row_entry("norm_rope_store_prefill c%d" % cr, sb,
                                                               "hbm" if sb > 50e6 else "latency")
    for cr, w in ((4, d4), (128, d128)):
        f_rows["norm_rope_store_decode c%d" % cr] = row_entry(
            "norm_rope_store_decode c%d" % cr, algorithmic_bytes_store_decode(w.hd, 64, w.seq_lens, cr), "latency")
    f_rows["decode_c4_norm_rope_store"] = row_entry(
        "decode_c4_norm_rope_store", algorithmic_bytes_fused_decode_store(d4.hd, d4.esize, d4.seq_lens, 64), "latency")
    c = P128.counts.cpu().tolist()
    rec_c = P128.plan_c[: c[0]].cpu().numpy().view("<u4").reshape(-1, 4)
    blen = (rec_c[:, 1] >> 24).astype(np.int64)
    rec_w = P128.plan_w[: c[1]].cpu().numpy().view("<u4").reshape(-1, 2).astype(np.int64)
    runs, k = [], 0
    while k < len(rec_w):  # a run: consecutive records of one slot and consecutive positions
        j = k + 1
        while (j < len(rec_w) and rec_w[j, 1] // 128 == rec_w[k, 1] // 128
               and rec_w[j, 1] - rec_w[k, 1] == j - k and rec_w[j, 0] - rec_w[k, 0] == j - k):
            j += 1
        runs.append((j - k, rec_w[k, 1] % 128 > 0))
        k = j
    ob = algorithmic_bytes_online(p128.hd, p128.esize, blen, runs, d128.seq_lens)
    f_rows["compress_c128_online"] = row_entry("compress_c128_online", ob[0], "hbm")
    f_rows["plan_prefill c128 runs"] = row_entry(
        "plan_prefill c128 runs", algorithmic_bytes_plan_prefill(p128.B, P128.plan_c.shape[0], P128.plan_w.shape[0])
        + 16 * p128.B, "latency")
    # with the run list the write reads one 16-byte entry per request instead of the 8-byte W records
    f_rows["write_c128_online"] = row_entry("write_c128_online", ob[1] - 8 * c[1] + 16 * p128.B, "latency")
    f_rows["write_c128_online scan"] = row_entry("write_c128_online scan", ob[1], "latency")
    f_rows["decode_c128_online"] = row_entry("decode_c128_online", ob[2], "latency")
    for name, P, w in (("plan_prefill_swa c4", SP4, p4), ("plan_prefill_swa c128", SP128, p128),
                       ("plan_prefill_page4", PG4, p4)):
        f_rows[name] = row_entry(name, algorithmic_bytes_plan_prefill(w.B, P.pc.shape[0], P.pw.shape[0]), "latency")
    f_rows["plan_decode_swa c4"] = row_entry("plan_decode_swa c4", algorithmic_bytes_plan_decode(d4.B), "latency")
    f_rows["plan_decode_page4"] = row_entry("plan_decode_page4", algorithmic_bytes_plan_decode(d4.B) + 4 * d4.B,
                                            "latency")

    tokens = p4.num_q + p128.num_q + d4.B + d128.B
    value = tokens / (ms_per_step * 1e-3)
    # the compressed rows one step emits: every C record of both prefills and every decode request
    # that closes a block
    rows = (int(P4.counts[0].item()) + int(P128.counts[0].item()) + int((d4.seq_lens % 4 == 0).sum())
            + int((d128.seq_lens % 128 == 0).sum()))

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "c4+c128 mixed chunked prefill (64 req, prefix U[0,65536], extend U[1,4096], "
                        "%d tokens, head_dim 512) + c4 decode B=256 + c128 decode B=1024" % p4.num_q,
            "prefill_tokens": p4.num_q,
            "decode_batch": [d4.B, d128.B],
            "head_dim": 512,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_us, 2),
            "cache": "warm",
            "cold_us": cold[dominant],
            "cold_frac": round(dom_bytes / (cold[dominant] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            # same-box ceilings (16-byte-vector streams over 1 GiB, the best of their four timings): a
            # copy moves as many bytes in as out, the pool's mix about 8 in per 1 out
            "copy_ceiling": ceil["copy"],
            "of_copy_ceiling": round(achieved / ceil["copy"], 4),
            "mix_ceiling": ceil["read8_write1"],
            "of_mix_ceiling": round(achieved / ceil["read8_write1"], 4),
        },
        "stream_ceilings": ceil_all,
        "configs": configs,
        "kernels_us": kernels_us,
        "step_rows": step_rows,
        "f_rows": f_rows,
        "compressed_rows": {"per_step": rows, "per_s": round(rows / (ms_per_step * 1e-3), 1)},
        "decode_step_us": decode_us,
        "overlapped_step": {"streams": 4, "ms_per_step": round(overlap_ms, 4),
                            "tokens_per_s": round((p4.num_q + p128.num_q + d4.B + d128.B) / (overlap_ms * 1e-3), 1)},
        "store_step": store_step,
        "wall_s_timed": round(wall, 3),
    }

    if args.sweep:
        log("sweep ...")
        result["sweep"] = sweep(torch, kvc, dev, P4, P128, to_dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p4, p128, d4, d128, tokens, args.cpu_reps)

    print(json.dumps(result), flush=True)


def cpu_model():
    """The host CPU from /proc/cpuinfo: its model name, with the family / model / stepping numbers
    (a virtual machine may show only a generic name) and the logical CPUs the host lists."""
    fields, n = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k = k.strip()
                if k == "processor":
                    n += 1
                elif k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v.strip()
    except OSError:
        pass
    name = fields.get("model name") or platform.processor() or "unknown"
    nums = ", ".join("%s %s" % (k, fields[k]) for k in ("cpu family", "model", "stepping") if k in fields)
    return "%s (%s%s%d logical CPUs)" % (name, nums, "; " if nums else "", n or (os.cpu_count() or 0))


def _slices(n, parts):
    """[lo, hi) bounds splitting range(n) into at most `parts` nearly equal pieces."""
    parts = max(1, min(parts, n))
    cuts = [n * k // parts for k in range(parts + 1)]
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def cpu_baseline(p4, p128, d4, d128, tokens, reps):
    """The float64 C oracle over one whole step (same workloads, host copies), in two legs: all the
    cores this process may use (up to 16), then one core.  Each leg runs the unchanged oracle calls:
    the plan on one thread, the pool over slices of C records, the write over slices of W records
    (after every pool slice), and each decode over slices of requests, the slices on a thread pool
    (the oracle's C calls release the interpreter lock)."""
    import concurrent.futures

    import oracle

    oracle.build(force=False)
    model = cpu_model()

    def one_step(ex, parts):
        """The oracle calls of one step, timed; the state copies that give each run a fresh state
        (the write and the decodes change it in place) are made before the clock starts."""
        fresh = {id(w): w.state.copy() for w in (p4, p128, d4, d128)}

        def run(fn, n, *args):
            futs = [ex.submit(fn, a, b, *args) for a, b in _slices(n, parts)]
            for f in futs:
                f.result()

        t = time.perf_counter()
        for w in (p4, p128):
            cap_c, cap_w = oracle.capacities(w.cr, w.B, w.num_q)
            pc, pw, counts = oracle.plan_prefill(w.cr, w.seq_lens, w.extend_lens, w.state_index, w.num_state_rows,
                                                 w.num_q, cap_c, cap_w)
            run(lambda a, b: oracle.compress(w.cr, w.hd, w.state, w.input, w.ape, pc[a:b], b - a), int(counts[0]))
            st = fresh[id(w)]
            run(lambda a, b: oracle.write(w.cr, w.hd, st, w.input, pw[a:b], b - a), int(counts[1]))
        for w in (d4, d128):
            pd, _ = oracle.plan_decode(w.cr, w.seq_lens, w.state_index, w.num_state_rows)
            st = fresh[id(w)]
            run(lambda a, b: oracle.decode(w.cr, w.hd, st, w.input[a:b], w.ape, pd[a:b]), w.B)
        return time.perf_counter() - t

    legs = []
    for threads in (min(len(os.sched_getaffinity(0)), 16), 1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            times = [one_step(ex, threads) for _ in range(reps)]
        sec = float(np.median(times))
        legs.append({"threads": threads, "value": round(tokens / sec, 1), "s_per_step": round(sec, 4),
                     "runs": reps})
    best = legs[0]
    return {"value": best["value"], "unit": "tokens/s", "cores": best["threads"], "kind": "oracle",
            "model": model, "one_core": legs[1],
            "sample": "the whole bench step (both mixed prefills, both decode batches), float64 C oracle, "
                      "median of %d runs per leg: %d threads %.3f s per step, 1 thread %.3f s per step; %s"
                      % (reps, best["threads"], best["s_per_step"], legs[1]["s_per_step"], model)}


if __name__ == "__main__":
    main()
