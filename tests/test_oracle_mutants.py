"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of kvc_oracle.c (a dropped
term, an off-by-one, a wrong sign, a swapped operand or page), builds it with
gcc on the CPU, and runs the pin suite against it in a subprocess.  The suite
must fail for every mutant; the unmodified oracle passes it (test_oracle_pins).
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvc_oracle.c")

MUTANTS = [
    ("buffer_len off by one", "const int64_t in_chunk = (j + 1 < W) ? j + 1 : W;",
     "const int64_t in_chunk = (j < W) ? j : W;", 0),
    ("SWA buffer_len off by one", "const int64_t in_chunk = (j + 1 < W) ? j + 1 : W;",
     "const int64_t in_chunk = (j < W) ? j : W;", 1),
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
    ("ragged base not advanced", "ragged_base += e;", "ragged_base += 0;", 0),
    ("SWA ragged base not advanced", "ragged_base += e;", "ragged_base += 0;", 1),
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
    ("compress trigger shifted", "if ((pos + 1) % cr == 0) {", "if (pos % cr == 0) {", 0),
    ("SWA compress trigger shifted", "if ((pos + 1) % cr == 0) {", "if (pos % cr == 0) {", 1),
    ("SWA page-tail writes dropped", "const int page_tail = (cr == 4) && (pos % swa_page_size >= swa_page_size - cr);",
     "const int page_tail = 0;"),
    ("SWA ring slot taken modulo the page size", "row = (swa / sps) * ring + swa % ring;",
     "row = (swa / sps) * ring + (swa % sps) % ring + ((swa % sps) >= ring ? 1 : 0);"),
    ("SWA ring of the wrong page", "row = (swa / sps) * ring + swa % ring;", "row = (swa / ring) * ring + swa % ring;"),
    ("SWA decode reads the overlap block from the new token's page",
     "put_u32(r + 8, as_u32((int32_t)(row0 / cr)));", "put_u32(r + 8, as_u32((int32_t)(row1 / cr)));"),
    ("rotation sin sign flipped",
     "y[base + 2 * k] = re * c - im * s;\n    y[base + 2 * k + 1] = re * s + im * c;",
     "y[base + 2 * k] = re * c + im * s;\n    y[base + 2 * k + 1] = -re * s + im * c;"),
    ("rotated channels at the head of the row", "const int64_t base = hd - rope_dim;", "const int64_t base = 0;"),
    ("rotary pairs split in halves", "const double re = y[base + 2 * k], im = y[base + 2 * k + 1];",
     "const double re = y[base + k], im = y[base + k + rope_dim / 2];"),
    ("norm eps dropped", "sqrt(ss / (double)hd + eps)", "sqrt(ss / (double)hd)"),
    ("norm over the sum, not the mean", "sqrt(ss / (double)hd + eps)", "sqrt(ss + eps)"),
    ("norm weight dropped", "y[d] = (double)x[d] * inv * (double)w[d];", "y[d] = (double)x[d] * inv;"),
    ("rotary position one late", "int64_t pos = (int64_t)seq_len - cr;", "int64_t pos = (int64_t)seq_len - cr + 1;"),
    ("table row stride halved", "freqs + pos * rope_dim : NULL", "freqs + pos * (rope_dim / 2) : NULL"),
    ("decode stores rows that close no block",
     "if (seq_len == 0xFFFFFFFFu || seq_len % (uint32_t)cr != 0) continue;", "if (seq_len == 0xFFFFFFFFu) continue;"),
    ("prefill location by record, not ragged id", "x + (size_t)k * hd, seq_len, ragged,", "x + (size_t)k * hd, seq_len, k,"),
    ("store location range unchecked", "if (loc < 0 || loc >= num_cache_rows) return ERR_RECORD;",
     "if (loc < 0) return ERR_RECORD;"),
    ("online fold drops the sum rescale", "*l = *l * a + b;",
     "*l = *l + b;"),
    ("online fold drops the weighted-sum rescale", "*acc = *acc * a + kv * b;",
     "*acc = *acc + kv * b;"),
    ("online compress ignores the partial in the slot", "      if (blen > 0) {\n        const double* s = state + slot * 3 * hd;",
     "      if (0) {\n        const double* s = state + slot * 3 * hd;"),
    ("online write always starts a fresh block", "int fresh = p0 == 0;",
     "int fresh = 1;"),
    ("online write takes ape by run index", "widen(ape, is_bf16, p0 + i, hd, d)",
     "widen(ape, is_bf16, i, hd, d)"),
    ("online decode never starts a fresh block", "fold(&m, &l, &acc, pos % 128 == 0, t,",
     "fold(&m, &l, &acc, 0, t,"),
    ("online decode emits one token early", "if (seq_len % 128 == 0) o[d] = acc / l;",
     "if (pos % 128 == 0) o[d] = acc / l;"),
    ("online write merges runs of different slots", "get_i32(plan_w + (size_t)(k + n) * 8 + 4) / 128 == slot",
     "1"),
    ("online compress window off by one", "        const int64_t row = ragged - 127 + i;\n        const double t",
     "        const int64_t row = ragged - 126 + i;\n        const double t"),
    ("online compress accepts buffer_len above 127", "    if (blen > 127 || (blen > 0 && (slot < 0",
     "    if ((blen > 0 && (slot < 0"),
    ("duplicate state slots accepted", "      if (idx[c] == idx[b]) return 1;", "      if (0) return 1;"),
    ("duplicate state slots compared with the next request only", "    for (int c = b + 1; c < B; ++c)",
     "    for (int c = b + 1; c < B && c < b + 2; ++c)"),
    ("page4 overlap entries always from the first load page", "rp0 = blen <= 4 ? lsp : lfp;",
     "rp0 = lfp;"),
    ("page4 overlap threshold off by one", "rp0 = blen <= 4 ? lsp : lfp;",
     "rp0 = blen < 4 ? lsp : lfp;"),
    ("page4 write split at the wrong position", "const int64_t page = pos < last ? wfp : page_index[b];",
     "const int64_t page = pos <= last ? wfp : page_index[b];"),
    ("page4 writes only the current block", "const int64_t first_w = (s / 4) * 4 - 4;",
     "const int64_t first_w = (s / 4) * 4;"),
    ("page4 decode slot one late", "put_u32(r + 4, as_u32((int32_t)(page * 4 + (s - 1) % 4)));",
     "put_u32(r + 4, as_u32((int32_t)(page * 4 + s % 4)));"),
    ("page4 decode overlap from the page of the new token", "put_u32(r + 8, as_u32((int32_t)prev));",
     "put_u32(r + 8, as_u32((int32_t)page));"),
    ("C padding written as zeros",
     "if (cap_c > num_c) memset(plan_c + (size_t)num_c * 16, 0xFF, (size_t)(cap_c - num_c) * 16);",
     "if (cap_c > num_c) memset(plan_c + (size_t)num_c * 16, 0x00, (size_t)(cap_c - num_c) * 16);", 0),
    ("W padding written as zeros",
     "if (cap_w > num_w) memset(plan_w + (size_t)num_w * 8, 0xFF, (size_t)(cap_w - num_w) * 8);",
     "if (cap_w > num_w) memset(plan_w + (size_t)num_w * 8, 0x00, (size_t)(cap_w - num_w) * 8);", 0),
    ("counts kept after a planner error", "  if (err) {\n    num_c = 0;\n    num_w = 0;\n  } else {",
     "  if (err) {\n  } else {", 0),
    ("capacity check off by one", "if (num_c > cap_c || num_w > cap_w) err |= ERR_CAPACITY;",
     "if (num_c >= cap_c || num_w > cap_w) err |= ERR_CAPACITY;", 0),
    ("extend beyond seq_len accepted", "if (e <= 0 || e > s) err |= ERR_EXTEND;", "if (e <= 0) err |= ERR_EXTEND;", 0),
    ("decode leaves rows that close no block unwritten",
     "    for (int d = 0; d < hd; ++d) o[d] = 0.0;\n    if (seq_len == 0xFFFFFFFFu) continue;",
     "    if (seq_len == 0xFFFFFFFFu) continue;"),
    ("softmax max not subtracted", "const double w = exp(t[i] - m);", "const double w = exp(t[i]);"),
    ("write copies half a row",
     "    memcpy((uint8_t*)state + (size_t)(loc * R * esz), (const uint8_t*)input + (size_t)((int64_t)ragged * R * esz),\n"
     "           (size_t)(R * esz));",
     "    memcpy((uint8_t*)state + (size_t)(loc * R * esz), (const uint8_t*)input + (size_t)((int64_t)ragged * R * esz),\n"
     "           (size_t)(R * esz / 2));"),
    ("ratio 128 keeps an overlap block too", "const int64_t first_w = last_c - (cr == 4 ? 4 : 0);",
     "const int64_t first_w = last_c - 4;"),
    ("ape row by kept-entry count", "t[n] = sc + widen(ape, is_bf16, i, hd, d);",
     "t[n] = sc + widen(ape, is_bf16, n, hd, d);"),
    ("first-block mask also on the second block", "const int first = (cr == 4 && seq_len == 4) ? 4 : 0;\n  for (int64_t d",
     "const int first = (cr == 4 && seq_len <= 8) ? 4 : 0;\n  for (int64_t d"),
    ("ratio-4 entries before the chunk read from the input",
     "static entry_src c4_entry(int i, int64_t blen, int64_t ragged, int64_t rp0, int64_t rp1, int64_t hd) {\n  entry_src e;\n  if (i < blen) {",
     "static entry_src c4_entry(int i, int64_t blen, int64_t ragged, int64_t rp0, int64_t rp1, int64_t hd) {\n  entry_src e;\n  if (i < blen && 0) {"),
]


def _plant(src, old, new, nth):
    """Replace the nth occurrence of old (or the only one when nth is None)."""
    if nth is None:
        assert src.count(old) == 1, "mutation site not found exactly once: %r" % old
        return src.replace(old, new)
    at = -1
    for _ in range(nth + 1):
        at = src.index(old, at + 1)
    return src[:at] + new + src[at + len(old):]


PIN_FILES = ["test_oracle_pins.py", "test_oracle_swa_pins.py", "test_oracle_store_pins.py",
             "test_oracle_online_pins.py", "test_oracle_page4_pins.py"]


def _run_pins_against(mutant, workdir):
    """Build the mutant oracle and run the pin suite on it; returns (exit code, output tail)."""
    name, old, new = mutant[:3]
    nth = mutant[3] if len(mutant) > 3 else None
    d = os.path.join(workdir, name.replace(" ", "_").replace("'", ""))
    os.makedirs(d)
    mutated = os.path.join(d, "kvc_oracle_mutant.c")
    with open(mutated, "w") as f:
        f.write(_plant(open(SRC).read(), old, new, nth))
    lib = os.path.join(d, "libkvc_oracle_mutant.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", lib, mutated, "-lm"])
    env = dict(os.environ, KVC_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                       [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    return r.returncode, r.stdout.decode(errors="replace")[-2000:]


class _PinRuns:
    """Pin runs of the mutants, one process each.  In a plain pytest run every mutant is started
    at once on a pool of workers; under pytest-xdist (which already spreads the cases over its
    workers) a case runs its own mutant when it asks for it."""

    def __init__(self, workdir, prefetch):
        self.workdir = workdir
        workers = max(1, min(8, len(os.sched_getaffinity(0)))) if prefetch else 1
        self.ex = concurrent.futures.ThreadPoolExecutor(max_workers=workers)
        self.futures = {}
        if prefetch:
            for m in MUTANTS:
                self._submit(m)

    def _submit(self, mutant):
        if mutant[0] not in self.futures:
            self.futures[mutant[0]] = self.ex.submit(_run_pins_against, mutant, self.workdir)
        return self.futures[mutant[0]]

    def result(self, mutant):
        return self._submit(mutant).result()


@pytest.fixture(scope="module")
def pin_runs(tmp_path_factory):
    runs = _PinRuns(str(tmp_path_factory.mktemp("mutants")), prefetch="PYTEST_XDIST_WORKER" not in os.environ)
    yield runs
    runs.ex.shutdown(wait=True, cancel_futures=True)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0].replace(" ", "_") for m in MUTANTS])
def test_pins_catch_mutant(pin_runs, mutant):
    code, tail = pin_runs.result(mutant)
    assert code != 0, "pins did not catch mutant '%s':\n%s" % (mutant[0], tail)
