"""The oracle's pins must catch plausible mistakes in the oracle itself. Each case below
plants one (a dropped term, a wrong index, layout or sign, an off-by-one, a wrong rounding
rule) in a copy of oracle/oracle.c, builds it with gcc, and runs the oracle's pin tests
against that copy in a separate process (ORACLE_LIBRARY). The case passes when at least
one pin fails. The real oracle.c is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_attention.py", "tests/test_oracle_paging.py",
        "tests/test_oracle_blocksize.py", "tests/test_oracle_fp8.py",
        "tests/test_oracle_prefill.py"]

# (name, text in oracle.c, replacement); the text must occur exactly once
MUTANTS = [
    ("softmax sum without the max shift",
     "        s[t] = exp(s[t] - m);\n        l += s[t];",
     "        l += exp(s[t]);\n        s[t] = exp(s[t] - m);"),
    ("weights not normalised", "double p = s[t] / l;", "double p = s[t];"),
    ("scale dropped", "s[t] = scale * dot;", "s[t] = dot;"),
    ("V layout transposed", "return ((blk * Hkv + g) * d + i) * bs + t;",
     "return ((blk * Hkv + g) * bs + t) * d + i;"),
    ("block index with a fixed 16-token block", "int64_t blk = table_row[t / bs];",
     "int64_t blk = table_row[t / 16];"),
    ("interleaved GQA head mapping", "        int g = h / G;\n        int64_t n = seq_lens[b];",
     "        int g = h % Hkv;\n        int64_t n = seq_lens[b];"),
    ("partition one token short", "int64_t t0 = p * P, t1 = t0 + P < n ? t0 + P : n;",
     "int64_t t0 = p * P, t1 = t0 + P - 1 < n ? t0 + P - 1 : n;"),
    ("merge weights without the partition sums",
     "double w = exp(m[r * max_parts + p] - M) * l[r * max_parts + p];",
     "double w = exp(m[r * max_parts + p] - M);"),
    ("causal mask excludes the query's own position",
     "oracle_attend(o, NULL, NULL, qq, K, V, pos + 1, d, scale);",
     "oracle_attend(o, NULL, NULL, qq, K, V, pos, d, scale);"),
    ("e4m3 ties not to even", "if (dd < best_d || (dd == best_d && (c & 1) == 0 && (best & 1) == 1)) {",
     "if (dd < best_d) {"),
    ("e4m3 subnormal exponent", "if (e == 0) v = ldexp((double)m, -9);",
     "if (e == 0) v = ldexp((double)m, -10);"),
    ("fp16 exponent bias", "else v = ldexp((double)(0x400 | f), e - 25);",
     "else v = ldexp((double)(0x400 | f), e - 24);"),
    ("V rows from the key input", "memcpy(vdst, vsrc, (size_t)e);", "memcpy(vdst, ksrc, (size_t)e);"),
]


def _run_pins(source: str, tmp_path):
    """Build source as the oracle library and run the pin tests against it."""
    c = tmp_path / "oracle_copy.c"
    c.write_text(source)
    so = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-shared",
                    "-fPIC", "-o", str(so), str(c), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIBRARY=str(so))
    return subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    """The control: the same build and run of the unmodified source passes, so a mutant's
    failure comes from its mutation."""
    r = _run_pins(open(SRC).read(), tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {name}"
    r = _run_pins(src.replace(old, new), tmp_path)
    assert r.returncode == 1, (f"no pin caught '{name}' (pytest exit {r.returncode}):\n"
                               + r.stdout[-2000:])
