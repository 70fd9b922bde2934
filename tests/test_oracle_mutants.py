"""The oracle's pins catch plausible mistakes in the oracle (CPU only).

Each mutant is a copy of oracle/pc_oracle.c with one slip planted in it (a
dropped term, a wrong rounding rule, a swapped index, a wrong offset).  It is
compiled to a separate library and the pin suite is run against it in a
child process; every mutant must make at least one pin fail.  Every mutant
stays within the buffers the oracle is given.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pc_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

sys.path.insert(0, ROOT)
from oracle import build as obuild  # noqa: E402

MUTANTS = {
    "accumulator starts at +0": [("float acc = -0.0f;", "float acc = 0.0f;")],
    "ties rounded away from zero": [("rest > 0x8000u || (rest == 0x8000u && (keep & 1u))", "rest >= 0x8000u")],
    "ties rounded to odd": [("(rest == 0x8000u && (keep & 1u))", "(rest == 0x8000u && !(keep & 1u))")],
    "truncation instead of rounding": [("keep += 1u;", "keep += 0u;")],
    "infinity taken for NaN": [("if (mag > 0x7F800000u)", "if (mag >= 0x7F800000u)")],
    "NaN keeps its payload": [("return (uint16_t)0x7FC0u; /* any NaN */", "return (uint16_t)((u >> 16) | 0x40u);")],
    "fold order ignored": [("int r = order ? order[j] : j;", "int r = j;")],
    "fold order reversed": [("int r = order ? order[j] : j;", "int r = order ? order[n - 1 - j] : n - 1 - j;")],
    "last rank dropped": [("for (int j = 0; j < n; ++j) {\n        int r = order", "for (int j = 0; j < n - 1; ++j) {\n        int r = order")],
    "widen by the wrong shift": [("((uint32_t)h) << 16", "((uint32_t)h) << 15")],
    "LL pack halves swapped": [("(uint64_t)src[2 * j] | ((uint64_t)src[2 * j + 1] << 16)", "(uint64_t)src[2 * j + 1] | ((uint64_t)src[2 * j] << 16)")],
    "LL seq in the low word": [("dst[j] = data | ((uint64_t)seq << 32);", "dst[j] = (data << 32) | seq;")],
    "LL consume halves swapped": [("(lines[r][j] >> (16 * h))", "(lines[r][j] >> (16 * (1 - h)))")],
    "LL ready if any rank is current": [("int ready = 1;", "int ready = 0;"), ("!= seq) ready = 0;", "== seq) ready = 1;")],
    "LL bitmap MSB-first": [("bitmap[j / 64] |= (uint64_t)1 << (j % 64);", "bitmap[j / 64] |= (uint64_t)1 << (63 - j % 64);")],
    "LL stale lines folded": [("if (!ready) continue;", "if (0) continue;")],
    "twoshot copy-out skips rank 0": [("if (r != s) memcpy(", "if (r != s && r != 0) memcpy(")],
    "twoshot owner slice mis-indexed": [("uint16_t* owner = outs[s] + (size_t)s * slice;", "uint16_t* owner = outs[s] + (size_t)(n - 1 - s) * slice;")],
    "all-gather payload offset": [("memcpy(out + item * 128, rec + 8, 128);", "memcpy(out + item * 128, rec, 128);")],
    "all-gather record stride": [("const uint8_t* rec = shards[r] + 136 * b;", "const uint8_t* rec = shards[r] + 128 * b;")],
    "all-gather header low word only": [("if (header != seq) continue;", "if ((uint32_t)header != (uint32_t)seq) continue;")],
    "all-gather output transposed": [("size_t item = (size_t)r * blocks + b;", "size_t item = (size_t)b * n + r;")],
    "validation compares each flag": [("for (int r = 0; r < n; ++r) folded += flags[r][b];\n        ok[b] = folded == (uint32_t)n * flag;", "int each = 1;\n        for (int r = 0; r < n; ++r) { folded += flags[r][b]; each &= flags[r][b] == flag; }\n        ok[b] = each;")],
    "validation without the rank count": [("ok[b] = folded == (uint32_t)n * flag;", "ok[b] = folded == flag;")],
    "validation reads tile 0's flags": [("folded += flags[r][b];", "folded += flags[r][0];")],
    "validation writes rejected tiles": [("        ok[b] = folded == (uint32_t)n * flag;\n        if (!ok[b]) continue;", "        ok[b] = folded == (uint32_t)n * flag;")],
    "sentinel not substituted": [("dst[i] = src[i] == ORC_SENTINEL ? (uint16_t)ORC_CANON_NAN : src[i];", "dst[i] = src[i];")],
    "sentinel checked on first element only": [("for (size_t e = 8 * p; e < 8 * p + 8; ++e)\n                if (slots[r][e] == ORC_SENTINEL) ready = 0;", "for (size_t e = 8 * p; e < 8 * p + 1; ++e)\n                if (slots[r][e] == ORC_SENTINEL) ready = 0;")],
    "sentinel slots not re-armed": [("for (size_t e = 8 * p; e < 8 * p + 8; ++e) slots[r][e] = (uint16_t)ORC_SENTINEL;", "for (size_t e = 8 * p; e < 8 * p; ++e) slots[r][e] = (uint16_t)ORC_SENTINEL;")],
    "sentinel re-arms unready packs": [("        if (!ready) continue;\n        bitmap[p / 64]", "        if (!ready) { for (int r = 0; r < n; ++r) slots[r][8 * p] = (uint16_t)ORC_SENTINEL; continue; }\n        bitmap[p / 64]")],
}


def mutate(text, edits):
    for old, new in edits:
        assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
        text = text.replace(old, new)
    return text


def run_mutant(name, edits, tmp):
    src = mutate(open(SRC).read(), edits)
    tag = "".join(c if c.isalnum() else "_" for c in name)
    cfile = os.path.join(tmp, tag + ".c")
    lib = os.path.join(tmp, tag + ".so")
    with open(cfile, "w") as f:
        f.write(src)
    subprocess.run(["gcc", *obuild.CFLAGS, cfile, "-o", lib], check=True, capture_output=True)
    env = dict(os.environ, PC_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


@pytest.mark.slow
def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda kv: run_mutant(kv[0], kv[1], tmp), MUTANTS.items()))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants not caught by any pin: " + ", ".join(n for n, _ in survivors)
    for n, rc, out in results:
        assert rc == 1, (n, rc, out)   # a test failure, not a crash or collection error
