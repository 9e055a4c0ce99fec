"""Shared pytest configuration: the ``gpu`` marker and import paths."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # FA_TEST_REVERSE_ORDER=1 runs every test with the library's workgroups
    # taking their work items in reverse order (the race-check switch); all
    # parity results must hold in that order too.
    if os.environ.get("FA_TEST_REVERSE_ORDER") == "1":
        import io_aware_exact_10_amd as fa
        fa.fa_debug_reverse_order(1)
