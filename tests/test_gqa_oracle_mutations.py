"""Plants plausible mistakes in a temporary copy of the GQA decode-attention
oracle (on the CPU) and checks that its pins catch every one of them."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gqa_oracle.c")

MUTATIONS = {
    "wrong KV head": ("const int g = h / G;", "const int g = h % HKV;"),
    "scale dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "not normalised": ("out[(size_t)h * D + d] = L > 0 ? acc / den : 0.0;",
                       "out[(size_t)h * D + d] = L > 0 ? acc : 0.0;"),
    "V read token-major": ("return (((size_t)(j / GQA_BLOCK) * HKV + g) * D + d) * GQA_BLOCK + (size_t)(j % GQA_BLOCK);",
                           "return (((size_t)(j / GQA_BLOCK) * HKV + g) * GQA_BLOCK + (size_t)(j % GQA_BLOCK)) * D + d;"),
    "K blocks without the head stride": (
        "return (((size_t)(j / GQA_BLOCK) * HKV + g) * GQA_BLOCK + (size_t)(j % GQA_BLOCK)) * D + d;\n}\n/* V",
        "return (((size_t)(j / GQA_BLOCK) + g) * GQA_BLOCK + (size_t)(j % GQA_BLOCK)) * D + d;\n}\n/* V"),
    "tail of the last block attended": ("for (int j = 0; j < L; ++j) {\n      double dot",
                                        "for (int j = 0; j < ((L + 31) / 32) * 32; ++j) {\n      double dot"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    a, b = MUTATIONS[name]
    src = open(SRC).read()
    assert a in src, f"mutation anchor missing: {name}"
    (tmp_path / "m.c").write_text(src.replace(a, b))
    lib = str(tmp_path / "lib.so")
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
                           "-fPIC", "-o", lib, str(tmp_path / "m.c"), "-lm"])
    env = dict(os.environ, GQA_ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_gqa_oracle_pins.py"),
                        "-q", "-x", "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0, f"no pin caught: {name}\n{r.stdout[-2000:]}"
