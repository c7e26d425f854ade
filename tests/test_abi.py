"""The C-ABI library loads and exports every symbol include/kvc.h declares.

CPU only: no compute call is made.  The host argument checks run before any
HIP call, so calls with bad host arguments return KVC_EINVAL here too.
"""
import ctypes
import subprocess

import pytest

from sparse_attention_kv_plan_amd import kvc


@pytest.fixture(scope="module")
def lib():
    return kvc.load(build_if_missing=True)


def test_header_declares_the_boundary():
    assert kvc.header_functions() == sorted([
        "kvc_plan_prefill", "kvc_plan_decode", "kvc_write", "kvc_compress_c4", "kvc_compress_c128",
        "kvc_decode_c4", "kvc_decode_c128", "kvc_strerror", "kvc_plan_prefill_swa", "kvc_plan_decode_swa"])


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", kvc.LIB_PATH]).decode()
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in kvc.header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else of ours leaks out of the library
    assert sorted(n for n in exported if n.startswith("kvc")) == kvc.header_functions()


def test_strerror(lib):
    assert kvc.strerror(0) == "ok"
    for code in (-1, -2, 1, 2, 4, 8, 16):
        assert kvc.strerror(code) and "unknown" not in kvc.strerror(code)
    assert "unknown" in kvc.strerror(12345)


def test_host_argument_checks_reject_without_enqueueing(lib):
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    E = kvc.KVC_EINVAL
    # ratio, batch, num_q, capacities, row count
    assert lib.kvc_plan_prefill(5, 1, 1, p, p, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_plan_prefill(4, 0, 1, p, p, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_plan_prefill(4, 1025, 2000, p, p, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_plan_prefill(4, 2, 1, p, p, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1 << 24, p, p, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1, p, p, p, 8, p, -1, p, 1, p, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1, p, p, p, -8, p, 1, p, 1, p, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1, None, p, p, 8, p, 1, p, 1, p, None) == E
    misaligned = ctypes.c_void_p(p.value + 4)
    assert lib.kvc_plan_prefill(4, 1, 1, p, p, p, 8, misaligned, 1, p, 1, p, None) == E
    assert lib.kvc_plan_decode(3, 1, p, p, 8, p, None, None) == E
    assert lib.kvc_plan_decode(4, 0, p, p, 8, p, None, None) == E
    assert lib.kvc_plan_decode(4, 65537, p, p, 8, p, None, None) == E
    # dtype and head_dim
    assert lib.kvc_write(4, 2, 128, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_write(4, 1, 64, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_compress_c4(1, 96, p, 8, p, 1, p, p, 1, p, p, None) == E
    assert lib.kvc_compress_c128(3, 128, p, 8, p, 1, p, p, 1, p, p, None) == E
    assert lib.kvc_compress_c4(1, 128, p, 8, p, 1, misaligned, p, 1, p, p, None) == E
    assert lib.kvc_decode_c4(1, 128, p, 8, p, p, p, 0, None, p, None) == E
    assert lib.kvc_decode_c128(1, 128, p, 8, p, p, None, 1, None, p, None) == E
    # SWA planners: page size not a multiple of the ring, ratio-4 ring of 4, ratio-128 ring of 256
    L = ctypes.c_int64
    assert lib.kvc_plan_prefill_swa(4, 1, 8, p, p, p, p, L(64), L(1), p, L(64), 12, 8, L(8), p, 4, p, 8, p,
                                    None, None) == E
    assert lib.kvc_plan_prefill_swa(4, 1, 8, p, p, p, p, L(64), L(1), p, L(64), 16, 4, L(8), p, 4, p, 8, p,
                                    None, None) == E
    assert lib.kvc_plan_decode_swa(128, 1, p, p, p, L(64), L(1), p, L(64), 256, 256, L(256), p, None, None) == E
    assert lib.kvc_plan_decode_swa(4, 1, p, p, p, L(0), L(1), p, L(64), 16, 8, L(8), p, None, None) == E
    # empty work is a no-op that needs no device
    assert lib.kvc_compress_c4(1, 128, p, 8, p, 1, p, p, 0, p, p, None) == kvc.KVC_OK
    assert lib.kvc_write(128, 1, 512, p, 8, p, 1, p, 0, p, None) == kvc.KVC_OK
