"""The oracle against its pins, and planted mistakes against the same pins."""
import json
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_holds(pin, oracle_lib):
    pin(oracle_lib)


# Each planted mistake: (name, exact text in oracle.c, replacement).  The
# replacement is applied once to a copy of the source, compiled with the same
# flags, and every pin is run on that copy; at least one must fail.
MUTANTS = [
    ("dropped-scale", "z[i] = sc * dot;", "z[i] = dot;"),
    ("wrong-slot", "(t % bs)) * D;", "((t + 1) % bs)) * D;"),
    ("wrong-block-entry", "block_tables[(int64_t)s * table_stride + t / bs];",
     "block_tables[(int64_t)s * table_stride + (t / bs) / 2];"),
    ("kv-head-0", "g = (int)(pair % Hkv);", "g = 0 * (int)(pair % Hkv);"),
    ("gqa-interleaved", "const int h = g * G + hh;\n            const uint16_t* qh",
     "const int h = hh * Hkv + g;\n            const uint16_t* qh"),
    ("k-as-v", "acc[d] += w * Vc[(int64_t)i * D + d];", "acc[d] += w * Kc[(int64_t)i * D + d];"),
    ("no-normalise", "Z += w;", "Z += 1.0;"),
    ("f16-exponent-bias", "e - 25);", "e - 24);"),
    ("bf16-fraction", "(double)(f + 128), e - 134", "(double)(f + 127), e - 134"),
    ("drop-last-token", "for (int i = 0; i < n; ++i) {\n                const double w",
     "for (int i = 0; i < n - 1; ++i) {\n                const double w"),
    ("lse-no-log", "m + log(Z);", "m + Z;"),
    ("wrong-sign-score", "z[i] = sc * dot;", "z[i] = -sc * dot;"),
    ("q-head-of-kv", "q + ((int64_t)s * Hq + h) * D;", "q + ((int64_t)s * Hq + g) * D;"),
    ("range-off-by-one", "const int n = hi > lo ? hi - lo : 0;", "const int n = hi > lo ? hi - lo - (lo > 0) : 0;"),
    ("fp8-exponent-bias", "(double)(f + 8), e - 10);", "(double)(f + 8), e - 9);"),
    ("fp8-subnormal", "ldexp((double)f, -9);", "ldexp((double)f, -10);"),
    ("fp8-scale-transposed", "k_scale, b * Hkv + g);", "k_scale, g * num_blocks + b);"),
    ("fp8-v-with-k-scale", "kv_dtype, v_scale, b * Hkv + g);", "kv_dtype, k_scale, b * Hkv + g);"),
    ("fp8-ties-odd", "(c & 1) == 0", "(c & 1) == 1"),
    ("fp8-quant-scale", "amax / 448.0f", "amax / 480.0f"),
    ("fp8-quant-tail", "if (i < ntok * D) {", "if (i <= ntok * D) {"),
    ("prefill-no-causal-mask", "lens[r] = n - m + i + 1;", "lens[r] = n;"),
    ("prefill-position-from-start", "lens[r] = n - m + i + 1;", "lens[r] = i + 1;"),
    ("prefill-first-table-row", "block_tables + (int64_t)s * table_stride,", "block_tables + (int64_t)0 * table_stride,"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    so = oracle.compile_c(str(path), str(tmp_path / f"lib_{name}.so"))
    # Run the pins in a child process so that a mutant cannot take pytest down.
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import json, sys, oracle\n"
        "from tests import oracle_pins as P\n"
        f"lib = oracle.OracleLib({so!r})\n"
        "failed = []\n"
        "for pin in P.ALL_PINS:\n"
        "    try:\n"
        "        pin(lib)\n"
        "    except (AssertionError, ValueError):\n"
        "        failed.append(pin.__name__)\n"
        "print(json.dumps(failed))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, f"mutant {name} crashed instead of failing a pin:\n{r.stderr[-2000:]}"
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, f"planted mistake {name} passed every pin"
