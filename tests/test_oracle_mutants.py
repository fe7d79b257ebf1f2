"""The oracle's pins catch plausible mistakes: each case below plants one
mistake (a sign, a dropped term, a wrong index or bound, a wrong rounding)
in a private copy of the oracle, rebuilds it, and runs the pin tests against
the copy, which must fail; an edit that leaves the arithmetic alone must
pass.  CPU only; the repository's oracle is never modified."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

# (name, file, old text, new text, pin test file)
BATCHED = "test_oracle.py"
SEGMENTS = "test_oracle_segments.py"
COSTFIT = "test_oracle_costfit.py"
C = "adaln_oracle.c"
PY = "costfit.py"
MUTANTS = [
    ("shift sign", C, "+ shift[b * D + d];", "- shift[b * D + d];", BATCHED),
    ("(1 + scale) dropped", C, "y[row * D + d] = xhat * (1.0 + scale[b * D + d])",
     "y[row * D + d] = xhat * (scale[b * D + d])", BATCHED),
    ("eps outside the root", C, "*rstd_out = 1.0 / sqrt(var + eps);",
     "*rstd_out = 1.0 / (sqrt(var) + eps);", BATCHED),
    ("unbiased variance", C, "double var = sq / (double)D;",
     "double var = sq / (double)(D - 1);", BATCHED),
    ("dx without the xhat term", C,
     "\n                dx[row * D + d] = r[row] * (g - c1 - xhat * c2);",
     "\n                dx[row * D + d] = r[row] * (g - c1);", BATCHED),
    ("dscale of g instead of dy", C,
     "                    for (int64_t j = 0; j < nd; ++j) {\n"
     "                        int64_t d = d0 + j;\n"
     "                        double g = dy[row * D + d];",
     "                    for (int64_t j = 0; j < nd; ++j) {\n"
     "                        int64_t d = d0 + j;\n"
     "                        double g = dy[row * D + d] * (1.0 + scale[b * D + d]);",
     BATCHED),
    ("dshift stores dscale", C, "dshift[b * D + d0 + j] = acc_h[j];",
     "dshift[b * D + d0 + j] = acc_s[j];", BATCHED),
    ("bucket batch not at least 1", C, "return b > 1 ? b : 1;", "return b;",
     BATCHED),
    ("memory bound off by one", C, "int64_t mem_bound = m_mem / S;",
     "int64_t mem_bound = m_mem / (S + 1);", BATCHED),
    ("segment modulation index ignored", C,
     "return mod ? (int64_t)mod[s] : s;", "return s;", SEGMENTS),
    ("segment dscale from the other vectors", C,
     "if (seg_mod_of(mod, s) != m)", "if (seg_mod_of(mod, s) == m)", SEGMENTS),
    ("segment dx sums without scale", C,
     "double g = gr[d] * (1.0 + scale[m * D + d]);\n"
     "                    double xhat = (xr[d] - mu[row]) * r[row];\n"
     "                    sum_g += g;",
     "double g = gr[d];\n"
     "                    double xhat = (xr[d] - mu[row]) * r[row];\n"
     "                    sum_g += g;", SEGMENTS),
    ("cost model exponent p - 1", PY,
     "return a + b * np.asarray(B, float) * np.asarray(S, float) ** p",
     "return a + b * np.asarray(B, float) * np.asarray(S, float) ** (p - 1)",
     COSTFIT),
    ("fit residual without B", PY,
     "return t - (a + bs * (B * S ** p) / scale)",
     "return t - (a + bs * (S ** p) / scale)", COSTFIT),
    ("bucket rule rounds up", PY, "q = math.floor(m_comp / math.pow(float(S), p))",
     "q = math.ceil(m_comp / math.pow(float(S), p))", COSTFIT),
    ("compute bound without the integer batch", PY,
     "return float(m_mem // s_ref) * math.pow(float(s_ref), p)",
     "return float(m_mem / s_ref) * math.pow(float(s_ref), p)", COSTFIT),
    ("compute bound at the next batch", PY,
     "return float(m_mem // s_ref) * math.pow(float(s_ref), p)",
     "return float(m_mem // s_ref + 1) * math.pow(float(s_ref), p)", COSTFIT),
]
CONTROLS = [
    ("comment only (C)", C, "/* Forward: y = xhat", "/* forward: y = xhat",
     BATCHED),
    ("comment only (Python)", PY, '"""Predicted step time a + b * B * S^p."""',
     '"""Predicted step time."""', COSTFIT),
]


def _mutant(tmp_path, file, old, new):
    root = tmp_path / "m"
    dst = root / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("*.so", "*.tmp",
                                                  "__pycache__"))
    path = dst / file
    src = path.read_text()
    # a case that does not apply exactly once would test nothing
    assert src.count(old) == 1, f"{old!r} occurs {src.count(old)} times"
    path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                    str(dst / "adaln_oracle.c"), str(dst / "check_rows.c"),
                    "-o", str(dst / "liboracle.so"), "-lm"], check=True)
    return root


def _pins(root, test_file):
    env = dict(os.environ, PYTHONPATH=f"{root}{os.pathsep}{ROOT}")
    where = subprocess.run(
        [sys.executable, "-c", "import oracle; print(oracle.__file__)"],
        cwd=root, env=env, capture_output=True, text=True, check=True)
    assert where.stdout.strip().startswith(str(root)), where.stdout
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         "-c", os.devnull, "--rootdir", str(root),
         os.path.join(TESTS, test_file)],
        cwd=root, env=env, capture_output=True, text=True, timeout=600)
    return res.returncode, res.stdout[-400:]


@pytest.fixture(scope="module", autouse=True)
def _gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")


@pytest.mark.parametrize("name,file,old,new,pins", MUTANTS,
                         ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_the_pins(tmp_path, name, file, old, new, pins):
    rc, out = _pins(_mutant(tmp_path, file, old, new), pins)
    assert rc == 1, f"{name}: the pins did not catch it\n{out}"


@pytest.mark.parametrize("name,file,old,new,pins", CONTROLS,
                         ids=[m[0] for m in CONTROLS])
def test_harmless_edit_passes_the_pins(tmp_path, name, file, old, new, pins):
    rc, out = _pins(_mutant(tmp_path, file, old, new), pins)
    assert rc == 0, f"{name}: control failed\n{out}"
