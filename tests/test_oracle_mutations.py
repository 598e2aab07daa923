"""Plants plausible mistakes in a temporary copy of the oracle (on the CPU) and
checks that the oracle's pins catch every one of them."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_q4_oracle.c")

MUTATIONS = {
    "nibble order swapped": ("int q = (k & 1) ? (byte >> 4) : (byte & 15);",
                             "int q = (k & 1) ? (byte & 15) : (byte >> 4);"),
    "bias dropped": ("float v = fmaf((float)q, s, b);", "float v = (float)q * s;"),
    "gate/up rows swapped": ("const float* wg = wgu + (size_t)j * H;\n      const float* wu = wgu + (size_t)(I + j) * H;",
                             "const float* wu = wgu + (size_t)j * H;\n      const float* wg = wgu + (size_t)(I + j) * H;"),
    "silu sign flipped": ("(1.0 + exp(-(double)gf))", "(1.0 + exp((double)gf))"),
    "shared expert left out of combine": ("double acc = has_shared ? (double)y[(R + t) * H + n] : 0.0;",
                                          "double acc = 0.0;"),
    "ties to the upper expert": ("l[e] > l[best]", "l[e] >= l[best]"),
    "wrong quant group index": ("scales[(size_t)n * (K / 64) + k / 64]",
                                "scales[(size_t)n * (K / 64) + (k / 64 + 1) % (K / 64)]"),
    "unstable scatter": ("int p = cursor[ids[r]]++;",
                         "int p = offsets[ids[r]+1] - 1 - (cursor[ids[r]]++ - offsets[ids[r]]);"),
    "weights not renormalized": ("if (norm_topk) {", "if (!norm_topk) {"),
    "logit sum reversed": ("for (int h = 0; h < H; ++h) {\n        float p", "for (int h = H - 1; h >= 0; --h) {\n        float p"),
    "logit summed in 64-column blocks": (
        "      float acc = 0.0f;\n      for (int h = 0; h < H; ++h) {\n"
        "        float p = bf16_to_f32(x[(size_t)t * H + h]) * bf16_to_f32(wr[(size_t)e * H + h]);\n"
        "        acc = acc + p;\n      }\n",
        "      float acc = 0.0f, blk = 0.0f;\n      for (int h = 0; h < H; ++h) {\n"
        "        float p = bf16_to_f32(x[(size_t)t * H + h]) * bf16_to_f32(wr[(size_t)e * H + h]);\n"
        "        blk = blk + p;\n        if (h % 64 == 63 || h == H - 1) { acc = acc + blk; blk = 0.0f; }\n      }\n"),
    "logit accumulated in fp64": ("      float acc = 0.0f;\n      for (int h = 0; h < H; ++h) {",
                                  "      double acc = 0.0;\n      for (int h = 0; h < H; ++h) {"),
    "row token index wrong": ("row_token[r] = sorted_idx[offsets[e] + r] / K;",
                              "row_token[r] = sorted_idx[offsets[e] + r] % T;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    a, b = MUTATIONS[name]
    src = open(SRC).read()
    assert a in src, f"mutation anchor missing: {name}"
    d = tmp_path
    (d / "m.c").write_text(src.replace(a, b))
    shutil.copy(os.path.join(ROOT, "oracle", "moe_q4_oracle.h"), d)
    lib = str(d / "lib.so")
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
                           "-fPIC", "-o", lib, str(d / "m.c"), "-lm"])
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-q", "-x", "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0, f"no pin caught: {name}\n{r.stdout[-2000:]}"
