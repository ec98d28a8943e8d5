import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


@pytest.fixture(scope="session")
def hip_lib():
    """The HIP library's Python binding; skips when no GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from eagle_tree_verification_amd import api
    api.load()  # raises if the shared library is missing
    return api


def pytest_terminal_summary(terminalreporter):
    """One line per session on the near-tie exclusions of the walk
    comparisons (sequences excluded from bit-exact comparison because the
    oracle confirms a near tie), with the cases that had any."""
    helpers = sys.modules.get("gpu_helpers")
    if helpers is None or not getattr(helpers, "EXCLUSIONS", None):
        return
    rec = helpers.EXCLUSIONS
    compared = sum(c for _, c, _ in rec)
    excluded = sum(len(e) for _, _, e in rec)
    worst = max(len(e) for _, _, e in rec)
    terminalreporter.write_line(
        f"near-tie exclusions: {excluded} of {compared} walks compared over {len(rec)} "
        f"comparisons (at most {worst} in one case)")
    for case, c, e in rec:
        if e:
            terminalreporter.write_line(f"  {case}: excluded {e} of {c}")
