import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C ABI)")
    config.addinivalue_line("markers", "slow: full-size workloads")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def pytest_sessionfinish(session, exitstatus):
    """Write the measured code-mismatch counts of the GPU parity tests as JSON
    to the path in COAT_PARITY_STATS, when it is set and a GPU run produced
    some."""
    path = os.environ.get("COAT_PARITY_STATS")
    if not path:
        return
    try:
        import parity
    except Exception:
        return
    if not parity.STATS and not parity.BF16_STATS:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    tot_n = sum(r["n"] for r in parity.STATS)
    tot_bad = sum(r["own_mismatches"] for r in parity.STATS)
    rule_n = sum(r["rule_n"] for r in parity.STATS)
    rule_bad = sum(r["rule_mismatches"] for r in parity.STATS)
    with open(path, "w") as f:
        json.dump({"elements_compared": tot_n, "mismatches_vs_oracle_codes": tot_bad,
                   "mismatch_fraction": tot_bad / max(tot_n, 1),
                   "max_grid_steps_vs_oracle_codes": max((r["own_max_steps"] for r in parity.STATS), default=0),
                   "rule_elements": rule_n, "rule_mismatches": rule_bad,
                   "rule_mismatch_fraction": rule_bad / max(rule_n, 1),
                   "rule_max_grid_steps": max((r["rule_max_steps"] for r in parity.STATS), default=0),
                   "amax_max_ulps": max((r["amax_max_ulps"] for r in parity.STATS), default=0),
                   "per_comparison": parity.STATS,
                   "bf16_outputs": [{"what": w, "n": n, "not_identical": b, "not_identical_fraction": b / max(n, 1)}
                                    for w, n, b in parity.BF16_STATS]}, f, indent=1)
