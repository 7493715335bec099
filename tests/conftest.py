import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload parity (minutes on the CPU oracle)")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, on a machine that has a GPU. Fails loudly otherwise."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda.is_available() is False")
    import linear_attention_ssm_amd as gdn
    return gdn


def pytest_terminal_summary(terminalreporter):
    """The measured parity figures (max|result - oracle| / max|oracle|): the
    largest fraction of its bar per test file, and every long-sequence and
    full-size figure (the worst over the scan schedules)."""
    try:
        from tests.helpers import PARITY
    except ImportError:
        return
    if not PARITY:
        return
    import re
    tr = terminalreporter
    tr.section("measured parity: max|result - oracle| / max|oracle|")
    worst = {}
    for r in PARITY:
        mod = r["test"].split("::")[0] or "?"
        frac = r["err"] / r["tol"]
        if mod not in worst or frac > worst[mod][0]:
            worst[mod] = (frac, r)
    for mod, (frac, r) in sorted(worst.items()):
        n = sum(1 for x in PARITY if x["test"].split("::")[0] == mod)
        tr.write_line(f"{mod}: {n} figures, worst {r['err']:.2e} (bar {r['tol']:.0e}) at {r['what']}")
    long_rows = {}
    for r in PARITY:
        if "long_decay" not in r["test"]:
            continue
        key = re.sub(r" (prefill|chain) schedule=\(\d, \d\)", "", r["what"])
        long_rows[key] = max(long_rows.get(key, 0.0), r["err"])
    for key, err in long_rows.items():
        tr.write_line(f"  {key}: {err:.2e} (worst over entries and scan schedules)")
