"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch each one.  This guards the pins themselves: a pin set that a
dropped term or a swapped index survives would not prove the oracle right."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pa_oracle.cpp")

# (name, exact source text, planted replacement, pin tests expected to catch it)
MUTATIONS = [
    ("kv head = h % hkv", "h / G, hkv, d, bs, nb, scale, dtype);",
     "h % hkv, hkv, d, bs, nb, scale, dtype);", "brute_force or head_groups"),
    ("scale dropped", "s[j] = scale * acc;", "s[j] = acc;", "brute_force"),
    ("slot offset shifted", "((static_cast<int64_t>(b) * bs + j % bs) * hkv + g) * d",
     "((static_cast<int64_t>(b) * bs + (j + 1) % bs) * hkv + g) * d", "brute_force"),
    ("K and V swapped in gather", "v_out[static_cast<int64_t>(j) * d + e] = widen(value_cache",
     "v_out[static_cast<int64_t>(j) * d + e] = widen(key_cache", "brute_force"),
    ("f16 exponent bias off by one", "static_cast<int>(expo) - 25", "static_cast<int>(expo) - 24",
     "f16_widen"),
    ("bf16 narrowing truncates", "const double r = std::nearbyint(units);\n    // r may",
     "const double r = std::trunc(units);\n    // r may", "bf16_narrow or f16_narrow"),
    ("merge weight dropped", "num = num + wp[p] * accp", "num = num + accp", "partitioned"),
    ("cache write offset", "const int64_t dst = (b * bs + o) * row;",
     "const int64_t dst = (o * bs + b) * row;", "cache_write or workload"),
    ("int8 scale over 128", "const float sc = a / 127.0f;", "const float sc = a / 128.0f;",
     "int8_quantize"),
    ("int8 codes truncated", "std::nearbyint(widen(x[e], dtype) / sc)",
     "std::trunc(widen(x[e], dtype) / sc)", "int8_quantize"),
    ("int8 scale index [blk][off][g]", "const int64_t sdst = (blk * hkv + g) * bs + off;",
     "const int64_t sdst = (blk * bs + off) * hkv + g;", "int8_cache_write or int8_decode"),
    ("int8 dequant drops the scale", "ks * static_cast<float>(key_cache[row + e])",
     "static_cast<float>(key_cache[row + e])", "int8_decode"),
    ("prefill position one early", "const int32_t pos = context_lens[i] - n + (row - query_start[i]);",
     "const int32_t pos = context_lens[i] - n + (row - query_start[i]) - 1;", "prefill"),
    ("prefill kv head h % hkv", "h / G /* kv head */", "h % hkv /* kv head */", "prefill"),
    ("int8 V scale from K", "const float vs = value_scale[(blk * hkv + g) * bs + off];",
     "const float vs = key_scale[(blk * hkv + g) * bs + off];", "int8_decode"),
]


@pytest.mark.parametrize("name,old,new,selector", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, selector):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for '{name}' not found exactly once"
    mutant = tmp_path / "pa_oracle.cpp"
    mutant.write_text(src.replace(old, new))
    (tmp_path / "pa_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "pa_oracle.h")).read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
                    "-pthread", str(mutant), "-o", str(lib)], check=True)
    env = dict(os.environ, PA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", selector],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"planted mistake '{name}' survived the pins:\n{r.stdout[-2000:]}"


MODEL_SRC = os.path.join(ROOT, "oracle", "allocator_model.py")

# (name, exact source text, planted replacement, occurrences of the anchor)
MODEL_MUTATIONS = [
    ("prefix key not chained", "key = tuple(tokens[: (i + 1) * bs])",
     "key = tuple(tokens[i * bs: (i + 1) * bs])", 2),
    ("last-token block reused", "range((len(tokens) - 1) // bs if tokens else 0)",
     "range(len(tokens) // bs)", 1),
    ("hit left in the pool", "self.free_blocks.remove(b)", "pass", 1),
    ("handed-out block stays cached", "        self._forget(block)\n", "        pass\n", 1),
    ("free in table order", "reversed(self.tables.get(seq_id, []))",
     "self.tables.get(seq_id, [])", 1),
    ("pool check ignores hits", "taken_from_pool = fresh + sum(", "taken_from_pool = fresh + 0 * sum(", 1),
    ("duplicate key overwritten", "                if key not in self.cached:\n",
     "                if True:\n", 1),
]


@pytest.mark.parametrize("name,old,new,count", MODEL_MUTATIONS, ids=[m[0] for m in MODEL_MUTATIONS])
def test_planted_model_mistake_is_caught(tmp_path, name, old, new, count):
    src = open(MODEL_SRC).read()
    assert src.count(old) == count, f"mutation anchor for '{name}' not found {count} time(s)"
    mutant = tmp_path / "allocator_model.py"
    mutant.write_text(src.replace(old, new))
    env = dict(os.environ, PA_ALLOC_MODEL_PATH=str(mutant))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_prefix_cache_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"planted mistake '{name}' survived the pins:\n{r.stdout[-2000:]}"
