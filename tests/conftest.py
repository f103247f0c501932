import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; fails loudly when it is missing or no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    import block_sparse_attention_sparge_amd as sp
    sp.load_library()
    return sp


# Parity records (mask near-tie counts, output errors) that the GPU tests add;
# printed as one section at the end of the run so that they survive a quiet (-q) run.
_PARITY_RECORDS = []


@pytest.fixture(scope="session")
def parity_log():
    """Append (label, {name: value}) records; they are printed in the terminal summary."""
    return _PARITY_RECORDS


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not _PARITY_RECORDS:
        return
    terminalreporter.section("parity records (mask near-ties within 1e-5 of the top-k cut; output error)")
    for label, rec in _PARITY_RECORDS:
        terminalreporter.write_line(label + ": " + " ".join(
            f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}" for k, v in rec.items()))
