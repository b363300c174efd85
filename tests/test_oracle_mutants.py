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


# The pool model (oracle/allocator.py), Python: each mutant runs in a copy of the tree's
# oracle, workloads and tests, so the real file is never touched. Its pins are the
# oracle's own tests (worked examples, invariants), not the comparisons with the C++ pool.
ALLOC_PINS = ["tests/test_oracle_allocator.py", "tests/test_oracle_prefix.py",
              "tests/test_oracle_blocksize.py"]
ALLOC_MUTANTS = [
    ("free queue taken from the back", "blk = self.free.popleft()", "blk = self.free.pop()"),
    ("freed blocks pushed to the front",
     "self.free.append(blk)      # keeps its key until popped again",
     "self.free.appendleft(blk)"),
    ("a new block one token early", "while len(blocks) * self.bs < length + n_tokens:",
     "while len(blocks) * self.bs <= length + n_tokens:"),
    ("slot offset counted from the block's end",
     "slots = [blocks[pos // self.bs] * self.bs + pos % self.bs",
     "slots = [blocks[pos // self.bs] * self.bs + (self.bs - 1 - pos % self.bs)"),
    ("shared blocks freed with their first owner",
     "            self.ref[blk] -= 1\n            if self.ref[blk] == 0:",
     "            self.ref[blk] -= 1\n            if self.ref[blk] <= 1:"),
    ("bytes per token without K and V", "return 2 * num_layers * num_kv_heads * head_dim * elem_bytes",
     "return num_layers * num_kv_heads * head_dim * elem_bytes"),
    ("copy-on-write block not counted", "need = -(-(length + n_tokens) // self.bs) - len(blocks) + int(cow)",
     "need = -(-(length + n_tokens) // self.bs) - len(blocks)"),
    ("prefix key of the block alone, not the chain",
     "key = (self.salt[sid], tuple(toks[:(j + 1) * self.bs]))",
     "key = (self.salt[sid], tuple(toks[j * self.bs:(j + 1) * self.bs]))"),
]


def _copy_tree(dst):
    import shutil
    for d in ("oracle", "workloads", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("__pycache__", "*.tmp"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst)


def _run_alloc_pins(old, new, tmp_path):
    dst = tmp_path / "tree"
    _copy_tree(str(dst))
    f = dst / "oracle" / "allocator.py"
    if old is not None:
        src = f.read_text()
        assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
        f.write_text(src.replace(old, new))
    env = {k: v for k, v in os.environ.items() if k != "ORACLE_LIBRARY"}
    return subprocess.run([sys.executable, "-m", "pytest", *ALLOC_PINS, "-x", "-q", "-m",
                           "not gpu", "-p", "no:cacheprovider"], cwd=str(dst), env=env,
                          capture_output=True, text=True, timeout=600)


def test_unmodified_pool_model_copy_passes_the_pins(tmp_path):
    r = _run_alloc_pins(None, None, tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", ALLOC_MUTANTS, ids=[m[0] for m in ALLOC_MUTANTS])
def test_pins_catch_planted_pool_model_mistake(name, old, new, tmp_path):
    r = _run_alloc_pins(old, new, tmp_path)
    assert r.returncode == 1, (f"no pin caught '{name}' (pytest exit {r.returncode}):\n"
                               + r.stdout[-2000:])
