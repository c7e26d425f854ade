"""The benchmark's same-box bandwidth streams (probe/libstream_probe.so).

CPU: the library loads, its tiles are what the kernels cover, and bad arguments are refused before
any HIP call.  GPU: each stream computes what it claims (a copy copies, the 8:1 stream writes the xor
of its 8 reads, the read stream writes nothing), so the ceilings it gives move the bytes they count.
"""
import ctypes
import errno
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_attention_kv_plan_amd import build as hip_build  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hip_build.PROBE_LIB):
        hip_build.build()
    lib = bench.load_stream_probe()
    lib.stream_probe_tile.argtypes = [ctypes.c_int]
    lib.stream_probe_tile.restype = ctypes.c_int64
    return lib


def test_tiles(lib):
    # 256 threads x 16 bytes x (reads per write x vectors per thread)
    assert [lib.stream_probe_tile(k) for k in range(3)] == [16384, 32768, 65536]
    assert lib.stream_probe_tile(3) == -errno.EINVAL


def test_bad_arguments_are_refused_before_any_launch(lib):
    p, q = 1 << 20, 1 << 21  # aligned stand-ins: refused on the host before they could be used
    bad = [
        (3, 0, p, 16384, q, 16384),          # no such kind
        (0, 0, 0, 16384, q, 16384),          # null source
        (0, 0, p, 16384, 0, 16384),          # null destination
        (0, 0, p + 8, 16384, q, 16384),      # misaligned source
        (0, 0, p, 16384, q + 4, 16384),      # misaligned destination
        (0, 0, p, 0, q, 16384),              # empty
        (0, 0, p, 16384 + 16, q, 32768),     # not a whole tile
        (0, 0, p, 32768, q, 16384),          # copy destination too small
        (1, 1, p, 65536, q, 8191),           # 8:1 destination below an eighth
        (2, 0, p, 65536, q, 4095),           # read-only destination below a sixteenth
    ]
    for args in bad:
        assert lib.stream_probe(*args, None) == -errno.EINVAL, args


def test_kinds_table_matches_the_bytes_counted():
    assert [(n, k) for n, k, _ in bench.PROBE_KINDS] == [("copy", 0), ("read8_write1", 1), ("read", 2)]
    assert [b for _, _, b in bench.PROBE_KINDS] == [2.0, 1.0 + 1 / 8, 1.0]


@pytest.mark.gpu
def test_streams_compute_what_they_claim(lib):
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    n = 3 * 65536  # bytes: three tiles of the largest kind
    rng = np.random.default_rng(7)
    host = rng.integers(0, 2**32, size=n // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(dev)
    for nt in (0, 1):
        dst = torch.zeros(n // 4, dtype=torch.int32, device=dev)
        assert lib.stream_probe(0, nt, src.data_ptr(), n, dst.data_ptr(), n, stream.cuda_stream) == 0
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy().view(np.uint32), host)

        dst = torch.zeros(n // 4, dtype=torch.int32, device=dev)
        assert lib.stream_probe(1, nt, src.data_ptr(), n, dst.data_ptr(), n // 8, stream.cuda_stream) == 0
        torch.cuda.synchronize()
        # vector v (16 bytes) of workgroup g, thread t: xor over r of src vector (g*8 + r)*256 + t
        vec = host.reshape(-1, 4)
        want = np.bitwise_xor.reduce(vec.reshape(-1, 8, 256, 4), axis=1).reshape(-1)
        got = dst.cpu().numpy().view(np.uint32)
        assert np.array_equal(got[: n // 32], want) and not got[n // 32:].any()

        same = torch.full((n // 4,), 0x5a5a5a5a, dtype=torch.int32, device=dev)
        dst = torch.zeros(n // 4, dtype=torch.int32, device=dev)
        assert lib.stream_probe(2, nt, same.data_ptr(), n, dst.data_ptr(), n // 16, stream.cuda_stream) == 0
        torch.cuda.synchronize()
        assert not dst.cpu().numpy().any()  # 16 equal vectors xor to zero: nothing written

        dst = torch.zeros(n // 4, dtype=torch.int32, device=dev)
        assert lib.stream_probe(2, nt, src.data_ptr(), n, dst.data_ptr(), n // 16, stream.cuda_stream) == 0
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(vec.reshape(-1, 16, 256, 4), axis=1).reshape(-1)
        got = dst.cpu().numpy().view(np.uint32)
        assert np.array_equal(got[: n // 64], want) and not got[n // 64:].any()
