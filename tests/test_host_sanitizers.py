"""tests/test_abi.py and tests/test_oracle.py again, against host-only builds with
AddressSanitizer and UndefinedBehaviorSanitizer: the C ABI's host code (gdn_api.cpp:
argument validation, the transaction planner, the offset and size arithmetic) linked
with launch stubs that refuse as the real launchers do without a GPU, and the C oracle.
Both are loaded in place of the regular builds (GDN_LIBRARY, GDN_ORACLE_LIBRARY) by a
child pytest with the ASan runtime preloaded; any sanitizer finding aborts it."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc and g++")
def test_validation_and_oracle_are_clean_under_asan_and_ubsan(tmp_path):
    import oracle
    from gateddeltanet_linear_attention_amd import sanitize
    lib = sanitize.build(str(tmp_path))
    olib = oracle.build(force=True, out=str(tmp_path / "libgdn_oracle.so"), sanitize=True)
    env = dict(os.environ, GDN_LIBRARY=lib, GDN_ORACLE_LIBRARY=olib, LD_PRELOAD=sanitize.runtime_preload(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_oracle.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-6000:] + "\n" + r.stderr[-6000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    assert " passed" in r.stdout, out
