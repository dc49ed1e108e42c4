"""The CPU suite once more under AddressSanitizer and UndefinedBehaviorSanitizer: the host code of
librq_lut.so (every argument check, workspace query and planner reached without a GPU) and the oracle,
both rebuilt with the sanitizers (tests/sanitize_run.py). A sanitizer report fails this test and is
printed."""
import os
import shutil

import pytest

import sanitize_run


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc to build the sanitizer library")
def test_cpu_suite_under_asan_ubsan():
    me = os.path.relpath(__file__, sanitize_run.ROOT)
    rc = sanitize_run.run(["tests", "--ignore", me, "-x"])
    assert rc == 0, f"CPU suite under ASan/UBSan exited with {rc} (86: ASan report, 87: UBSan report, " \
                    f"88: a report was written)"
