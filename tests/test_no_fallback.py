"""The product path has no CPU fallback: with the shared library missing, the
binding raises instead of computing anything, and the package never imports
the oracle."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_PROBE = r"""
import sys
sys.path.insert(0, %r)
import int8_group_quantized_amd.binding as B
B._LIB_PATH = "/nonexistent/libqgemm.so"
B._lib = None
import int8_group_quantized_amd as q
try:
    q.lib()
except RuntimeError as e:
    print("raised:", e)
else:
    print("no error")
print("oracle imported:", any(m == "oracle" or m.startswith("oracle.") for m in sys.modules))
"""


def test_missing_library_raises_and_oracle_is_not_imported():
    r = subprocess.run([sys.executable, "-c", _PROBE % ROOT], capture_output=True, text=True,
                       timeout=300, cwd="/")
    assert r.returncode == 0, r.stderr
    assert "raised: libqgemm.so is not built" in r.stdout
    assert "oracle imported: False" in r.stdout


def test_package_sources_do_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "int8_group_quantized_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_oracle_does_not_reference_the_product():
    odir = os.path.join(ROOT, "oracle")
    for f in os.listdir(odir):
        if f.endswith(".py"):
            text = open(os.path.join(odir, f)).read()
            assert "int8_group_quantized_amd" not in text, f
            assert "libqgemm" not in text, f
