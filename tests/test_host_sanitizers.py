"""Every host-only path of libdszero.so (argument validation of each entry
point, the layout and partition routines, the status strings) run from a C
program against a copy of the library built with the host AddressSanitizer
and UndefinedBehaviorSanitizer.  No GPU is used: every device entry point is
called with arguments it rejects before any device work."""
import os
import subprocess

import pytest

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "host_checks")


def test_host_paths_under_address_and_undefined_behaviour_sanitizers():
    if not os.path.exists(EXE):
        pytest.skip("host-sanitizer build not available (built by __graft_entry__.build())")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all host paths ok" in r.stdout
