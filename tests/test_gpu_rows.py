"""GPU parity of the streaming row statistics (max, log-sum-exp at T, argmax)."""
import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
import gen
import oracle
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [gen.DT_F32, gen.DT_BF16, gen.DT_F16])
@pytest.mark.parametrize("V,T", [(128256, 0.7), (129280, 1.0), (32000, 1.0), (12345, 2.0), (5, 0.5)])
def test_row_stats_match_oracle(dtype, V, T):
    rows = 24
    x = gen.normal_pair(gen.key(50, V, dtype), 3.0, 0, 0.0, rows * V, dtype, want_b=False)[0]
    G.say(f"row_stats dtype={dtype} V={V} T={T}")
    r = sv.row_stats(G.to_dev(x.reshape(rows, V), dtype), T)
    o = oracle.row_stats(x, V, dtype, T)
    np.testing.assert_array_equal(r["argmax"].cpu().numpy(), o["argmax"])
    np.testing.assert_array_equal(r["max"].cpu().numpy().astype(np.float64), o["max"])
    lse = r["lse"].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(lse, o["lse"], rtol=1e-5, atol=1e-5)
    assert np.all(r["err_flags"].cpu().numpy() == 0)


def test_row_stats_special_rows():
    V = 9000
    x = np.zeros((4, V), np.float32)
    x[0, :] = -np.inf
    x[1, 4000] = np.nan
    x[2, :] = -np.inf
    x[2, 8999] = 3.0
    x[3, [100, 8192, 8193]] = 5.0
    r = sv.row_stats(G.to_dev(x), 1.0)
    o = oracle.row_stats(x, V, gen.DT_F32, 1.0)
    np.testing.assert_array_equal(r["err_flags"].cpu().numpy(), o["err"])
    np.testing.assert_array_equal(r["argmax"].cpu().numpy(), o["argmax"])
    assert r["argmax"].cpu().numpy()[3] == 100
    assert r["argmax"].cpu().numpy()[2] == 8999
