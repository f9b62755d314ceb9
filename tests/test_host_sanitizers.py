"""The C-ABI tests and the oracle pins under host ASan + UBSan (CPU only).

See tests/host_sanitizers.py for the two instrumented builds.  A sanitizer
report ends its process with a non-zero status, so each run must exit 0 and
print no report.
"""
import pytest

from tests import host_sanitizers as hs

REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _clean(res):
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-6000:]
    for r in REPORTS:
        assert r not in text, text[-6000:]
    return text


@pytest.mark.slow
def test_library_host_code_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libgdn_san.so")
    hs.build_library(lib)
    text = _clean(hs.run_library_tests(lib))
    assert " passed" in text


@pytest.mark.slow
def test_oracle_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    hs.build_oracle(lib)
    text = _clean(hs.run_oracle_pins(lib))
    assert "pins" in text
