"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of kvc_oracle.c (a dropped
term, an off-by-one, a wrong sign, a swapped operand or page), builds it with
gcc on the CPU, and runs the pin suite against it in a subprocess.  The suite
must fail for every mutant; the unmodified oracle passes it (test_oracle_pins).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvc_oracle.c")

MUTANTS = [
    ("buffer_len off by one", "const int64_t in_chunk = (j + 1 < W) ? j + 1 : W;",
     "const int64_t in_chunk = (j < W) ? j : W;"),
    ("page alternation dropped", "if (cr == 4) return idx * 2 + ((pos / 4) & 1);", "if (cr == 4) return idx * 2;"),
    ("overlap block not kept", "const int64_t first_w = last_c - (cr == 4 ? 4 : 0);",
     "const int64_t first_w = last_c;"),
    ("read page 0 taken at pos",
     "put_u32(r + 4, (uint32_t)ragged | ((uint32_t)blen << 24));\n          put_u32(r + 8, as_u32((int32_t)page_of(cr, idx, pos0)));",
     "put_u32(r + 4, (uint32_t)ragged | ((uint32_t)blen << 24));\n          put_u32(r + 8, as_u32((int32_t)page_of(cr, idx, pos)));"),
    ("decode read page 0 taken at the new token",
     "put_u32(r + 4, as_u32((int32_t)loc_of(cr, idx, pos1)));\n    put_u32(r + 8, as_u32((int32_t)page_of(cr, idx, pos0)));",
     "put_u32(r + 4, as_u32((int32_t)loc_of(cr, idx, pos1)));\n    put_u32(r + 8, as_u32((int32_t)page_of(cr, idx, pos1)));"),
    ("kv quarters swapped", "e.kv_col = (i < 4) ? 0 : hd;", "e.kv_col = (i < 4) ? hd : 0;"),
    ("score quarters swapped", "e.sc_col = (i < 4) ? 2 * hd : 3 * hd;", "e.sc_col = (i < 4) ? 3 * hd : 2 * hd;"),
    ("ragged window off by one", "e.row = ragged - 7 + i;", "e.row = ragged - 8 + i;"),
    ("c128 ragged window off by one", "e.row = ragged - 127 + i;", "e.row = ragged - 126 + i;"),
    ("ape rows reversed", "t[n] = sc + widen(ape, is_bf16, i, hd, d);",
     "t[n] = sc + widen(ape, is_bf16, W - 1 - i, hd, d);"),
    ("ape dropped", "t[n] = sc + widen(ape, is_bf16, i, hd, d);", "t[n] = sc;"),
    ("first-block mask dropped", "  const int first = (cr == 4 && seq_len == 4) ? 4 : 0;\n  for (int64_t d",
     "  const int first = 0;\n  for (int64_t d"),
    ("softmax sign flipped", "const double w = exp(t[i] - m);", "const double w = exp(m - t[i]);"),
    ("ragged base not advanced", "ragged_base += e;", "ragged_base += 0;"),
    ("overlap page used for current block", "e.row = (i < 4) ? rp0 * 4 + i : rp1 * 4 + (i - 4);",
     "e.row = (i < 4) ? rp0 * 4 + i : rp0 * 4 + (i - 4);"),
    ("write location one position late", "put_u32(r + 4, as_u32((int32_t)loc_of(cr, idx, pos)));",
     "put_u32(r + 4, as_u32((int32_t)loc_of(cr, idx, pos + 1)));"),
    ("decode token slot off by one", "const int64_t pos1 = s - 1; /* the new token */",
     "const int64_t pos1 = s; /* the new token */"),
    ("decode pools before writing",
     "    memcpy((uint8_t*)state + (size_t)(wl * R * esz), (const uint8_t*)input + (size_t)((int64_t)b * R * esz),\n"
     "           (size_t)(R * esz));\n    if (boundary) pool_row(cr, is_bf16, hd, src, seq_len, state, input, ape, o);",
     "    if (boundary) pool_row(cr, is_bf16, hd, src, seq_len, state, input, ape, o);\n"
     "    memcpy((uint8_t*)state + (size_t)(wl * R * esz), (const uint8_t*)input + (size_t)((int64_t)b * R * esz),\n"
     "           (size_t)(R * esz));"),
    ("compress trigger shifted", "if ((pos + 1) % cr == 0) {", "if (pos % cr == 0) {"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0].replace(" ", "_") for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found exactly once: %r" % old
    mutated = tmp_path / "kvc_oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libkvc_oracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(lib), str(mutated), "-lm"])
    env = dict(os.environ, KVC_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    assert r.returncode != 0, "pins did not catch mutant '%s':\n%s" % (name, r.stdout.decode()[-2000:])
