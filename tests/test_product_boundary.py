"""The product path's boundary, on the CPU: the package never imports or loads
the oracle, the binding raises when the HIP library is missing (no CPU
fallback), and bench.py measures one GPU only."""

import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_prefill_amd")


def _run(code, timeout=120):
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                          timeout=timeout)


def test_package_sources_do_not_import_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n == "oracle" or n.startswith("oracle.") for n in names), (f, names)


def test_native_sources_do_not_reference_the_oracle():
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f)).read()
        assert "s2o_oracle" not in text and "oracle/" not in text, f


def test_importing_the_package_loads_no_oracle_module():
    r = _run("import sys\n"
             "import long_context_prefill_amd as s2o\n"
             "from long_context_prefill_amd import synth, profile_summary\n"
             "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]\n"
             "assert not bad, bad\n"
             "print('ok')\n")
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


def test_binding_raises_when_the_library_is_missing():
    r = _run("from long_context_prefill_amd import _lib as L\n"
             "L._lib = None\n"
             "L.LIB_PATH = '/nonexistent/libs2o.so'\n"
             "try:\n"
             "    L.list_entries(L.problem(1, 1, 1, 256, 64, 0, 128, 64, 64))\n"
             "except ImportError as e:\n"
             "    print('raised:', e)\n"
             "else:\n"
             "    print('no error')\n")
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "no CPU fallback" in r.stdout, r.stdout


@pytest.mark.parametrize("n", [2, 8])
def test_bench_measures_one_gpu_only(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and r.stdout == "", (r.returncode, r.stdout)
    assert "measures one GPU" in r.stderr
