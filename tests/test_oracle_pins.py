"""The oracle against facts fixed outside itself (CPU only).

Every pin in ``oracle_pins.py`` must hold for the oracle as built, and every
mistake planted in a mutated copy of the oracle's C source must make at least
one pin fail -- so a plausible slip anywhere in the oracle (a dropped term, a
wrong index, a transposed operand, an off-by-one boundary) cannot pass
unnoticed.  The mutants are compiled from text edits of
``oracle/hisparse_oracle.c`` into a temporary directory; the oracle itself is
never modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

from oracle.oracle import SRC, build_oracle
import oracle_pins




@pytest.mark.parametrize("name", list(oracle_pins.ALL_PINS))
def test_pin_holds(orc_lib, name):
    fails = oracle_pins.ALL_PINS[name](orc_lib)
    assert not fails, "\n".join(fails[:10])


# (label, exact text in the oracle source, replacement): one planted mistake each
MUTANTS = [
    ("victim from MRU end", "int32_t v = N[m];", "int32_t v = N[nN - 1 - m];"),
    ("misses in descending index", "int32_t i = misses[m];", "int32_t i = misses[M - 1 - m];"),
    ("hits placed before untouched slots",
     "    for (int32_t k = M; k < nN; ++k)\n        lru[j++] = N[k];\n    for (int32_t k = 0; k < nH; ++k)\n        lru[j++] = H[k];",
     "    for (int32_t k = 0; k < nH; ++k)\n        lru[j++] = H[k];\n    for (int32_t k = M; k < nN; ++k)\n        lru[j++] = N[k];"),
    ("loaded slots placed before hits",
     "    for (int32_t k = 0; k < nH; ++k)\n        lru[j++] = H[k];\n    for (int32_t k = 0; k < M; ++k)\n        lru[j++] = N[k];",
     "    for (int32_t k = 0; k < M; ++k)\n        lru[j++] = N[k];\n    for (int32_t k = 0; k < nH; ++k)\n        lru[j++] = H[k];"),
    ("hit order reversed", "        lru[j++] = H[k];", "        lru[j++] = H[nH - 1 - k];"),
    ("loaded slots left at the LRU end",
     "    for (int32_t k = M; k < nN; ++k)\n        lru[j++] = N[k];\n    for (int32_t k = 0; k < nH; ++k)\n        lru[j++] = H[k];\n    for (int32_t k = 0; k < M; ++k)\n        lru[j++] = N[k];",
     "    for (int32_t k = 0; k < nN; ++k)\n        lru[j++] = N[k];\n    for (int32_t k = 0; k < nH; ++k)\n        lru[j++] = H[k];"),
    ("newest token not special", "} else if (t == L - 1) {", "} else if (0) {"),
    ("fast path boundary off by one", "    if (L <= B) {\n        for", "    if (L < B) {\n        for"),
    ("newest row boundary off by one", "    if (L <= B)\n        return L - 1;", "    if (L < B)\n        return L - 1;"),
    ("copies the neighbouring host row",
     "memcpy(hot_req + (int64_t)v * rb, host_req + (int64_t)t * rb, (size_t)rb);",
     "memcpy(hot_req + (int64_t)v * rb, host_req + (int64_t)(t > 0 ? t - 1 : t + 1) * rb, (size_t)rb);"),
    ("plan pair transposed", "plan_pos[m] = t;\n        plan_slot[m] = v;", "plan_pos[m] = v;\n        plan_slot[m] = t;"),
    ("resident tier missing", "    if (resident) {", "    if (0) {"),
    ("admission identity boundary", "tok[s] = (L0 <= B) ? s : -1;", "tok[s] = (L0 < B) ? s : -1;"),
    ("hit not recorded", "is_hit[s] = 1;", "is_hit[s] = 0;"),
    ("slot map not updated on miss", "        tok[v] = t;\n", "        (void)0;\n"),
    ("backup from the wrong row",
     "               hot + ((int64_t)r * (B + 1) + row) * rb, (size_t)rb);",
     "               hot + ((int64_t)r * (B + 1) + (row == B ? B - 1 : row)) * rb, (size_t)rb);"),
    ("backup to the wrong position",
     "memcpy(host + ((int64_t)r * max_seq + (L - 1)) * rb,",
     "memcpy(host + ((int64_t)r * max_seq + (L > 1 ? L - 2 : 0)) * rb,"),
    ("replay reads the slot as position",
     "                   host + ((int64_t)r * max_seq + t) * rb, (size_t)rb);",
     "                   host + ((int64_t)r * max_seq + v) * rb, (size_t)rb);"),
    ("admission fill skips row 0", "for (int32_t p = 0; p < L0; ++p)", "for (int32_t p = 1; p < L0; ++p)"),
    ("padding resolved as position", "            out[i] = -1;                    /* padding */",
     "            out[i] = t + 1;                 /* padding */"),
    ("duplicate top-k accepted", "if (t < -1 || t >= L || seen[t]) {", "if (t < -1 || t >= L) {"),
    ("resident row: page and offset swapped", "res_row[i] = (int64_t)phys * page_size + t % page_size;",
     "res_row[i] = (int64_t)(t % page_size) * page_size + phys;"),
    ("resident entry left in the hot tiers", "hot_row[i] = -1;                 /* leaves the hot tiers untouched */",
     "(void)0;"),
    ("hot rows not shifted into the caller's view", "v = hot_base + out[i];", "v = out[i];"),
    ("page looked up by offset", "int32_t pg = t / page_size;", "int32_t pg = t % page_size;"),
    ("page past the table taken as resident", "int32_t phys = pg < max_pages ? block_row[pg] : -1;",
     "int32_t phys = pg < max_pages ? block_row[pg] : 0;"),
    ("physical page 0 not resident", "if (phys >= 0) {\n            res_row", "if (phys > 0) {\n            res_row"),
    ("hot base of request 0 used for all", "hot_row_base + (int64_t)r * (B + 1),", "hot_row_base,"),
    ("page transfer not cut at the pool end", "        if (rows > page_size)\n            rows = page_size;",
     "        rows = page_size;"),
    ("mirror skipped", "        if (mp >= 0)\n            memcpy(mirror", "        if (mp > 0)\n            memcpy(mirror"),
    ("host page ignores the request", "memcpy(host + ((int64_t)r * max_seq + (int64_t)hp * page_size) * rb, from,",
     "memcpy(host + ((int64_t)hp * page_size) * rb, from,"),
    ("source page offset dropped", "const uint8_t* from = src + (int64_t)sp * page_size * rb;",
     "const uint8_t* from = src;"),
]


@pytest.fixture(scope="module")
def oracle_source():
    with open(SRC) as f:
        return f.read()


_RUN_PINS = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from oracle.oracle import load_oracle
import oracle_pins
lib = load_oracle({lib!r})
for name, pin in oracle_pins.ALL_PINS.items():
    try:
        fails = pin(lib)
    except Exception as e:
        fails = [repr(e)]
    if fails:
        print("caught by", name, ":", fails[0][:200])
        sys.exit(3)
sys.exit(0)
"""


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(oracle_source, label, old, new):
    """Each mutant runs the pins in a child process: a pin failing, an oracle
    error or a crash of the mutant (a planted overrun can abort) all count as
    caught; only a clean pass of every pin does not."""
    assert oracle_source.count(old) == 1, f"mutation site for '{label}' not found exactly once"
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests_dir)
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(oracle_source.replace(old, new))
        lib = build_oracle(src=src, out=os.path.join(d, "libmutant.so"), extra_flags=["-I", os.path.dirname(SRC)])
        code = _RUN_PINS.format(root=root, tests=tests_dir, lib=lib)
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
        assert res.returncode != 0, f"planted mistake '{label}' passed every pin"
