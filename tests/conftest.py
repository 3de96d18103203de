import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test")


# max|err| / RMS of every floating-point parity check, printed at the end of the run
MARGINS = []


def pytest_terminal_summary(terminalreporter):
    if MARGINS:
        terminalreporter.write_line("parity margins (max|err| / RMS(ref), tolerance):")
        for label, v, t in MARGINS:
            terminalreporter.write_line(f"  {label:40s} {v:.3e}  tol {t:.0e}  ({100 * v / t:.0f}% of tol)")


def _ensure_host_libs():
    """Build the generator's host filler if nothing is built yet (gcc, seconds)."""
    lib = os.path.join(ROOT, "synth", "libsynth_host.so")
    if not os.path.exists(lib):
        from synth.build import build_host_only
        build_host_only()


_ensure_host_libs()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")
