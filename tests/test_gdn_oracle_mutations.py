"""Plants plausible mistakes in a temporary copy of the Gated DeltaNet scan
oracle (on the CPU) and checks that its pins catch every one of them."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTATIONS = {
    "gate not applied to the recall": ("        recall *= a;\n", ""),
    "write strength dropped": ("const double c = b * (vi - recall);", "const double c = (vi - recall);"),
    "delta sign flipped": ("const double c = b * (vi - recall);", "const double c = b * (recall - vi);"),
    "state not decayed": ("row[j] = a * row[j] + c * kk[j];", "row[j] = row[j] + c * kk[j];"),
    "output reads the key": ("out += row[j] * qq[j];", "out += row[j] * kk[j];"),
    "wrong key head": ("const int hk = hv / group;", "const int hk = hv % HK;"),
    "initial state ignored": ("state_in ? (double)state_in[(size_t)hv * DV * DK + i] : 0.0", "0.0"),
    "recall from the updated row": (
        "        double recall = 0.0;\n        for (int j = 0; j < DK; ++j) recall += row[j] * kk[j];\n"
        "        recall *= a;\n",
        "        for (int j = 0; j < DK; ++j) row[j] = a * row[j];\n"
        "        double recall = 0.0;\n        for (int j = 0; j < DK; ++j) recall += row[j] * kk[j];\n"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    a, b = MUTATIONS[name]
    src = open(SRC).read()
    assert a in src, f"mutation anchor missing: {name}"
    (tmp_path / "m.c").write_text(src.replace(a, b))
    lib = str(tmp_path / "lib.so")
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
                           "-fPIC", "-o", lib, str(tmp_path / "m.c")])
    env = dict(os.environ, GDN_ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_gdn_oracle_pins.py"),
                        "-q", "-x", "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0, f"no pin caught: {name}\n{r.stdout[-2000:]}"
