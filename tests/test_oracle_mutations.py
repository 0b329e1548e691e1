"""The oracle's pins catch plausible mistakes: each case below plants one mistake in a copy of
oracle/oracle.c (a decode bias, a nibble order, a rounding mode, a sign, a row swap, a dropped
weight, an unstable sort, a tie order, a transposed index), builds that copy with the oracle's
own gcc flags, and runs the pin tests meant to catch it against the copy (NVFP4_ORACLE_LIB).
Each must fail. The same copy without a mutation must pass, so a failure comes from the mistake
and not from the harness. CPU only; the mutants run four at a time."""
import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = ROOT / "oracle" / "oracle.c"

# (name, text in oracle.c, replacement, pin test files that must catch it)
MUTANTS = [
    ("E2M1 exponent bias", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)", ["test_oracle_formats.py"]),
    ("E2M1 subnormal step", "(e == 0) ? 0.5 * m", "(e == 0) ? 1.0 * m", ["test_oracle_formats.py"]),
    ("E4M3 exponent bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)", ["test_oracle_formats.py"]),
    ("fp16 rounding truncates", "double n = rint(ldexp(a, 10 - e));", "double n = floor(ldexp(a, 10 - e));",
     ["test_oracle_formats.py"]),
    ("code nibble order", "int code = (k & 1) ? (byte >> 4) : (byte & 15);",
     "int code = (k & 1) ? (byte & 15) : (byte >> 4);", ["test_oracle_gemm.py"]),
    ("SiLU sign", "return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));", ["test_oracle_formats.py"]),
    ("MoE up row = gate row (layout 0)", "return w->layout ? 2 * i + 1 : w->I + i;", "return w->layout ? 2 * i + 1 : i;",
     ["test_oracle_gemm.py"]),
    ("per-token MoE drops the slot weight", "o[n] += wk * y;", "o[n] += y;", ["test_oracle_gemm.py"]),
    ("grouped MoE skips SiLU", "hj[i] = silu(g) * u;", "hj[i] = g * u;", ["test_oracle_gemm.py"]),
    ("grouped MoE transposes W2", "acc += w2[n * I + i] * hj[i];", "acc += w2[i * K + n] * hj[i];",
     ["test_oracle_gemm.py"]),
    ("plan scatter not stable", "    for (int64_t p = 0; p < P; ++p) {\n        int32_t id = ids[p];\n        if (id >= 0 && id < E) {",
     "    for (int64_t p = P - 1; p >= 0; --p) {\n        int32_t id = ids[p];\n        if (id >= 0 && id < E) {",
     ["test_oracle_plan.py"]),
    ("plan row tiles one row short", "for (int32_t r = 0; r < counts[e]; r += (int32_t)BM) {",
     "for (int32_t r = 0; r < counts[e] - 1; r += (int32_t)BM) {", ["test_oracle_plan.py"]),
    ("router tie order", "    if (a != b) return a > b;\n    return ia < ib;", "    if (a != b) return a > b;\n    return ia > ib;",
     ["test_oracle_route.py"]),
    ("shared gate sign", "sigma[m] = 1.0 / (1.0 + exp(-z));", "sigma[m] = 1.0 / (1.0 + exp(z));",
     ["test_oracle_shared.py"]),
    ("FP8 channel scale dropped", "row[k] = orc_e4m3(codes[n * K + k]) * (double)chscale[n];",
     "row[k] = orc_e4m3(codes[n * K + k]);", ["test_oracle_fp8.py"]),
    ("gated MLP up row (layout 1)", "weight_row(c13, s13, g13, 2 * I, K, 0, layout ? 2 * i + 1 : I + i, ur);",
     "weight_row(c13, s13, g13, 2 * I, K, 0, layout ? 2 * i : I + i, ur);", ["test_oracle_mlp.py"]),
]


def _build(text: str, out: pathlib.Path):
    c = out.with_suffix(".c")
    c.write_text(text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-o", str(out), str(c), "-lm"], check=True, capture_output=True)


def _run_pins(lib: pathlib.Path, files) -> int:
    env = dict(os.environ, NVFP4_ORACLE_LIB=str(lib))
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + [str(ROOT / "tests" / f) for f in files]
    return subprocess.run(cmd, env=env, cwd=str(ROOT), capture_output=True, timeout=600).returncode


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_pins_catch_planted_oracle_mistakes(tmp_path):
    base = SRC.read_text()
    for name, old, new, _ in MUTANTS:
        assert base.count(old) == 1, f"mutation site of '{name}' not found exactly once in oracle.c"
    clean = tmp_path / "clean.so"
    _build(base, clean)

    def one(i):
        name, old, new, files = MUTANTS[i]
        lib = tmp_path / f"mutant{i}.so"
        _build(base.replace(old, new), lib)
        return name, _run_pins(lib, files)

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        control = ex.submit(_run_pins, clean, ["test_oracle_formats.py", "test_oracle_gemm.py", "test_oracle_fp8.py",
                                               "test_oracle_mlp.py", "test_oracle_route.py", "test_oracle_shared.py"])
        results = list(ex.map(one, range(len(MUTANTS))))
        assert control.result() == 0, "the unmutated copy must pass the pins"
    survived = [name for name, rc in results if rc != 1]  # 1: tests ran and failed
    assert not survived, f"mutants not caught by their pins: {survived}"
