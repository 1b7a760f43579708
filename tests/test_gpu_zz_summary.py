"""Session-wide exception rate of the stochastic parity checks (runs last: the
file name sorts after the other GPU test files)."""
import json
import os

import pytest

from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_zz_exception_rate():
    s = dict(G.STATS)
    if s["evaluated"] == 0:
        pytest.skip("no stochastic parity check ran in this session")
    s["exception_rate"] = s["exceptions"] / s["evaluated"]
    os.makedirs("gpurun_out", exist_ok=True)
    with open(os.path.join("gpurun_out", "parity_summary.json"), "w") as f:
        json.dump(s, f, indent=1)
    G.say(f"parity summary: {s}")
    assert s["exception_rate"] < 1e-4, s
