"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer
(host side): a host-only driver calls every entry point with invalid arguments; each call
must be refused with the expected status and no sanitizer may report anything. No GPU is
touched."""
import shutil

import pytest


def test_validation_under_host_sanitizers():
    if shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    from io_aware_exact_21_amd import sanitize_build as sb
    sb.build_sanitized()
    r = sb.run_driver()
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "refused as expected" in r.stdout
