"""The C-ABI library loads and exports every symbol include/kvc.h declares.

CPU only: no compute call is made.  The host argument checks run before any
HIP call, so calls with bad host arguments return KVC_EINVAL here too.
"""
import ctypes
import os
import subprocess

import pytest

from sparse_attention_kv_plan_amd import kvc


@pytest.fixture(scope="module")
def lib():
    return kvc.load(build_if_missing=True)


def test_header_declares_the_boundary():
    assert kvc.header_functions() == sorted([
        "kvc_plan_prefill", "kvc_plan_decode", "kvc_write", "kvc_compress_c4", "kvc_compress_c128",
        "kvc_decode_c4", "kvc_decode_c128", "kvc_strerror", "kvc_plan_prefill_swa", "kvc_plan_decode_swa",
        "kvc_norm_rope_store_prefill", "kvc_norm_rope_store_decode", "kvc_compress_c4_norm_rope_store",
        "kvc_compress_c128_norm_rope_store", "kvc_decode_c4_norm_rope_store", "kvc_compress_c128_online",
        "kvc_write_c128_online", "kvc_decode_c128_online", "kvc_plan_prefill_page4", "kvc_plan_decode_page4"])


def test_store_args_layout_matches_the_header(tmp_path):
    """The ctypes mirror of kvc_store_args has the C compiler's size and offsets."""
    src = tmp_path / "layout.c"
    fields = [f[0] for f in kvc.StoreArgs._fields_]
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "kvc.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(kvc_store_args));\n'
                   + "".join('  printf("%%zu\\n", offsetof(kvc_store_args, %s));\n' % f for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.dirname(kvc.HEADER), "-o", str(exe), str(src)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    assert got[0] == ctypes.sizeof(kvc.StoreArgs)
    assert got[1:] == [getattr(kvc.StoreArgs, f).offset for f in fields]


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
    for code in (-1, -2, 1, 2, 4, 8, 16, 32):
        assert kvc.strerror(code) and "unknown" not in kvc.strerror(code)
    assert "unknown" in kvc.strerror(12345)


def test_host_argument_checks_reject_without_enqueueing(lib):
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    E = kvc.KVC_EINVAL
    # ratio, batch, num_q, capacities, row count
    assert lib.kvc_plan_prefill(5, 1, 1, p, p, p, 8, p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill(4, 0, 1, p, p, p, 8, p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill(4, 1025, 2000, p, p, p, 8, p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill(4, 2, 1, p, p, p, 8, p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1 << 24, p, p, p, 8, p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1, p, p, p, 8, p, -1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1, p, p, p, -8, p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill(4, 1, 1, None, p, p, 8, p, 1, p, 1, p, None, None) == E
    misaligned = ctypes.c_void_p(p.value + 4)
    assert lib.kvc_plan_prefill(4, 1, 1, p, p, p, 8, misaligned, 1, p, 1, p, None, None) == E
    # the run list: ratio 128 only, 16-byte aligned
    assert lib.kvc_plan_prefill(4, 1, 1, p, p, p, 8, p, 1, p, 1, p, p, None) == E
    assert lib.kvc_plan_prefill(128, 1, 1, p, p, p, 128, p, 1, p, 1, p, misaligned, None) == E
    assert lib.kvc_plan_decode(3, 1, p, p, 8, p, None, None, None) == E
    assert lib.kvc_plan_decode(4, 0, p, p, 8, p, None, None, None) == E
    assert lib.kvc_plan_decode(4, 65537, p, p, 8, p, None, None, None) == E
    # the boundary list: ratio 128 only, 8-byte aligned
    assert lib.kvc_plan_decode(4, 1, p, p, 8, p, p, None, None) == E
    assert lib.kvc_plan_decode(128, 1, p, p, 128, p, misaligned, None, None) == E
    # dtype and head_dim
    assert lib.kvc_write(4, 2, 128, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_write(4, 1, 64, p, 8, p, 1, p, 1, p, None) == E
    assert lib.kvc_compress_c4(1, 96, p, 8, p, 1, p, p, 1, p, p, None) == E
    assert lib.kvc_compress_c128(3, 128, p, 8, p, 1, p, p, 1, p, p, None) == E
    assert lib.kvc_compress_c4(1, 128, p, 8, p, 1, misaligned, p, 1, p, p, None) == E
    assert lib.kvc_decode_c4(1, 128, p, 8, p, p, p, 0, None, p, None) == E
    assert lib.kvc_decode_c128(1, 128, p, 8, p, p, None, None, 1, None, p, None) == E
    assert lib.kvc_decode_c128(1, 128, p, 128, p, p, p, misaligned, 1, None, p, None) == E
    # SWA planners: page size not a multiple of the ring, ratio-4 ring of 4, ratio-128 ring of 256
    L = ctypes.c_int64
    assert lib.kvc_plan_prefill_swa(4, 1, 8, p, p, p, p, L(64), L(1), p, L(64), 12, 8, L(8), p, 4, p, 8, p,
                                    None, None) == E
    assert lib.kvc_plan_prefill_swa(4, 1, 8, p, p, p, p, L(64), L(1), p, L(64), 16, 4, L(8), p, 4, p, 8, p,
                                    None, None) == E
    assert lib.kvc_plan_decode_swa(128, 1, p, p, p, L(64), L(1), p, L(64), 256, 256, L(256), p, None, None,
                                   None) == E
    assert lib.kvc_plan_decode_swa(4, 1, p, p, p, L(0), L(1), p, L(64), 16, 8, L(8), p, None, None, None) == E
    assert lib.kvc_plan_decode_swa(4, 1, p, p, p, L(64), L(1), p, L(64), 16, 8, L(8), p, p, None, None) == E
    # norm / rotary / store parameters
    def st(**kw):
        a = dict(norm_weight=p.value, freqs_cis=p.value, out_loc=p.value, cache=p.value, num_loc=4, max_position=8,
                 num_cache_rows=4, eps=1e-6, rope_dim=64)
        a.update(kw)
        return ctypes.byref(kvc.StoreArgs(**a))
    store_p = lib.kvc_norm_rope_store_prefill
    for bad in (dict(rope_dim=12), dict(rope_dim=136), dict(rope_dim=-8), dict(eps=-1.0), dict(eps=float("nan")),
                dict(eps=float("inf")), dict(norm_weight=None), dict(cache=misaligned.value), dict(num_loc=-1),
                dict(max_position=-1), dict(freqs_cis=None)):
        assert store_p(4, 128, p, p, 1, p, st(**bad), None) == E, bad
    assert store_p(4, 128, p, p, 1, p, None, None) == E
    assert store_p(4, 96, p, p, 1, p, st(), None) == E
    assert store_p(4, 128, p, p, 0, p, st(rope_dim=0, freqs_cis=None), None) == kvc.KVC_OK
    assert lib.kvc_norm_rope_store_decode(128, 128, p, p, 0, None, st(), None) == E
    assert lib.kvc_norm_rope_store_decode(128, 128, p, misaligned, 1, None, st(), None) == E
    assert lib.kvc_compress_c4_norm_rope_store(1, 128, p, 8, p, 1, p, p, 1, p, None, None) == E
    assert lib.kvc_compress_c128_norm_rope_store(1, 128, p, 8, p, 1, p, p, 1, p, st(rope_dim=4), None) == E
    assert lib.kvc_compress_c4_norm_rope_store(1, 128, p, 8, p, 1, p, p, 0, p, st(), None) == kvc.KVC_OK
    assert lib.kvc_decode_c4_norm_rope_store(1, 128, p, 8, p, p, p, 1, None, None, None) == E
    assert lib.kvc_decode_c4_norm_rope_store(1, 128, p, 8, p, p, p, 1, None, st(rope_dim=20), None) == E
    assert lib.kvc_decode_c4_norm_rope_store(1, 128, p, 8, p, p, p, 0, None, st(), None) == E
    # page-4 planners: batch, token count, bundle alignment
    assert lib.kvc_plan_prefill_page4(0, 1, p, p, p, p, L(64), p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill_page4(2, 1, p, p, p, p, L(64), p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_prefill_page4(1, 1, p, p, p, misaligned, L(64), p, 1, p, 1, p, None, None) == E
    assert lib.kvc_plan_decode_page4(0, p, p, p, L(64), p, None, None) == E
    assert lib.kvc_plan_decode_page4(1, p, p, p, L(64), misaligned, None, None) == E
    # online ratio-128 state: head_dim, slot count, alignment, batch
    assert lib.kvc_compress_c128_online(1, 96, p, 2, p, 1, p, p, 1, p, p, None) == E
    assert lib.kvc_compress_c128_online(1, 128, p, -1, p, 1, p, p, 1, p, p, None) == E
    assert lib.kvc_compress_c128_online(1, 128, misaligned, 2, p, 1, p, p, 1, p, p, None) == E
    assert lib.kvc_write_c128_online(1, 128, p, 2, p, 1, p, misaligned, 1, p, None, 0, None) == E
    # with a run list: 16-byte aligned, 1 <= batch <= 1024 (checked before the empty-plan shortcut)
    assert lib.kvc_write_c128_online(1, 128, p, 2, p, 1, p, p, 1, p, misaligned, 1, None) == E
    assert lib.kvc_write_c128_online(1, 128, p, 2, p, 1, p, p, 0, p, p, 0, None) == E
    assert lib.kvc_write_c128_online(1, 128, p, 2, p, 1, p, p, 0, p, p, 1025, None) == E
    assert lib.kvc_decode_c128_online(1, 128, p, 2, p, p, p, 0, None, p, None) == E
    assert lib.kvc_compress_c128_online(1, 128, p, 2, p, 1, p, p, 0, p, p, None) == kvc.KVC_OK
    assert lib.kvc_write_c128_online(1, 128, p, 2, p, 1, p, p, 0, p, None, 0, None) == kvc.KVC_OK
    assert lib.kvc_write_c128_online(1, 128, p, 2, p, 1, p, p, 0, p, p, 1, None) == kvc.KVC_OK
    # empty work is a no-op that needs no device
    assert lib.kvc_compress_c4(1, 128, p, 8, p, 1, p, p, 0, p, p, None) == kvc.KVC_OK
    assert lib.kvc_write(128, 1, 512, p, 8, p, 1, p, 0, p, None) == kvc.KVC_OK


def test_binding_rejects_host_tensors():
    """A host tensor's pointer must never reach a kernel: every wrapper checks that its tensors are
    contiguous device tensors before calling the library (the check runs before any HIP call)."""
    torch = pytest.importorskip("torch")
    kvc.load(build_if_missing=True)
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    hd = 128
    st4, in4 = torch.zeros((8, 4 * hd)), torch.zeros((8, 4 * hd))
    st128, in128 = torch.zeros((128, 2 * hd)), torch.zeros((128, 2 * hd))
    pc, pw, pd = (torch.zeros((4, kvc.C_BYTES), dtype=torch.uint8), torch.zeros((4, kvc.W_BYTES), dtype=torch.uint8),
                  torch.zeros((1, kvc.D_BYTES), dtype=torch.uint8))
    ape4, ape128, out = torch.zeros((8, hd)), torch.zeros((128, hd)), torch.zeros((4, hd))
    wgt, cache = torch.ones(hd), torch.zeros((4, hd), dtype=torch.bfloat16)
    slots = torch.zeros((1, 3, hd))
    calls = [
        lambda: kvc.plan_prefill(4, i32(1), i32(1), i32(1), 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_decode(4, i32(1), i32(1), 8, pd),
        lambda: kvc.plan_prefill_page4(i32(1), i32(1), i32(1), torch.zeros((1, 4), dtype=torch.int32), 8, 1, pc, pw,
                                       i32(4)),
        lambda: kvc.plan_decode_page4(i32(1), i32(1), i32(1), 8, pd),
        lambda: kvc.write(4, hd, st4, in4, pw, i32(4)),
        lambda: kvc.compress_c4(hd, st4, in4, ape4, pc, i32(4), out),
        lambda: kvc.compress_c128(hd, st128, in128, ape128, pc, i32(4), out),
        lambda: kvc.decode_c4(hd, st4, in4, ape4, pd, out),
        lambda: kvc.decode_c128(hd, st128, in128, ape128, pd, out),
        lambda: kvc.norm_rope_store_prefill(4, out, pc, i32(4), wgt, 1e-6, None, i32(4), cache),
        lambda: kvc.compress_norm_rope_store(4, hd, st4, in4, ape4, pc, i32(4), wgt, 1e-6, None, i32(4), cache),
        lambda: kvc.compress_c128_online(hd, slots, in128, ape128, pc, i32(4), out),
        lambda: kvc.write_c128_online(hd, slots, in128, ape128, pw, i32(4)),
        lambda: kvc.decode_c128_online(hd, slots, in128, ape128, pd, out),
    ]
    for call in calls:
        with pytest.raises(kvc.KvcError, match="CUDA"):
            call()


def test_binding_rejects_non_int32_index_tensors():
    """Lengths, indices, tables, counts and status words are int32 in the ABI: an int64 tensor would
    be read as pairs of int32 words.  Every wrapper refuses one before a pointer reaches the library
    (the check runs before the device check, so it is seen here on host tensors)."""
    torch = pytest.importorskip("torch")
    kvc.load(build_if_missing=True)
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    i64 = lambda n: torch.zeros(n, dtype=torch.int64)  # noqa: E731
    hd = 128
    st4, in4 = torch.zeros((8, 4 * hd)), torch.zeros((8, 4 * hd))
    st128, in128 = torch.zeros((128, 2 * hd)), torch.zeros((128, 2 * hd))
    pc, pw, pd = (torch.zeros((4, kvc.C_BYTES), dtype=torch.uint8), torch.zeros((4, kvc.W_BYTES), dtype=torch.uint8),
                  torch.zeros((1, kvc.D_BYTES), dtype=torch.uint8))
    ape4, ape128, out = torch.zeros((8, hd)), torch.zeros((128, hd)), torch.zeros((4, hd))
    slots = torch.zeros((1, 3, hd))
    b4 = torch.zeros((1, 4), dtype=torch.int32)
    r2t, f2s = torch.zeros((1, 16), dtype=torch.int32), i32(16)
    calls = [
        lambda: kvc.plan_prefill(4, i64(1), i32(1), i32(1), 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_prefill(4, i32(1), i64(1), i32(1), 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_prefill(4, i32(1), i32(1), i64(1), 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_prefill(4, i32(1), i32(1), i32(1), 8, 1, pc, pw, i64(4)),
        lambda: kvc.plan_decode(4, i32(1), i64(1), 8, pd),
        lambda: kvc.plan_decode(4, i32(1), i32(1), 8, pd, i64(1)),
        lambda: kvc.plan_prefill_swa(4, i32(1), i32(1), i64(1), r2t, f2s, 16, 8, 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_prefill_swa(4, i32(1), i32(1), i32(1), r2t.long(), f2s, 16, 8, 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_prefill_swa(4, i32(1), i32(1), i32(1), r2t, f2s.long(), 16, 8, 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_decode_swa(4, i32(1), i32(1), r2t, f2s.long(), 16, 8, 8, pd),
        lambda: kvc.plan_prefill_page4(i32(1), i32(1), i64(1), b4, 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_prefill_page4(i32(1), i32(1), i32(1), b4.long(), 8, 1, pc, pw, i32(4)),
        lambda: kvc.plan_decode_page4(i32(1), i32(1), i64(1), 8, pd),
        lambda: kvc.write(4, hd, st4, in4, pw, i64(4)),
        lambda: kvc.compress_c4(hd, st4, in4, ape4, pc, i64(4), out),
        lambda: kvc.compress_c128(hd, st128, in128, ape128, pc, i64(4), out),
        lambda: kvc.decode_c4(hd, st4, in4, ape4, pd, out, i64(1)),
        lambda: kvc.decode_c128(hd, st128, in128, ape128, pd, out, i64(1)),
        lambda: kvc.compress_c128_online(hd, slots, in128, ape128, pc, i64(4), out),
        lambda: kvc.write_c128_online(hd, slots, in128, ape128, pw, i64(4)),
        lambda: kvc.decode_c128_online(hd, slots, in128, ape128, pd, out, i64(1)),
    ]
    for k, call in enumerate(calls):
        with pytest.raises(kvc.KvcError, match="int32"):
            call()
