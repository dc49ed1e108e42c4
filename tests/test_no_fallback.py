"""The product path has no fallback: without the HIP library every call raises, and the package never
imports the oracle (CPU; each check runs in a fresh interpreter so nothing is already loaded)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(code):
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_missing_library_raises():
    r = _run(
        "import numpy as np\n"
        "from lut_logits_amd import binding\n"
        "binding.LIB_PATH = '/nonexistent/librq_lut.so'\n"
        "import lut_logits_amd as la\n"
        "try:\n"
        "    la.packed10_codes_bytes(10, 2, 12)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('no error')\n")
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "is not built" in r.stdout, r.stdout


def test_package_does_not_import_the_oracle():
    r = _run(
        "import sys\n"
        "import lut_logits_amd, lut_logits_amd.binding, lut_logits_amd.formats, lut_logits_amd.synth\n"
        "import lut_logits_amd.composite\n"
        "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))\n")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "[]", r.stdout
