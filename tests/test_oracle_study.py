"""The quantization-error study (tests/study_quant_error.py) on a short
synthetic trajectory: the qualitative claims of the COAT explainer's
"expansion function" section hold on these states.  The page's own numbers
come from real training states that are not available (parity unpinned for
the 1.63x figure itself)."""
import pytest

import study_quant_error as study


@pytest.fixture(scope="module")
def res(orc):
    return study.study(steps=(1, 10), threads=8)


def test_expansion_lowers_the_first_moments_error(res):
    for t in (1, 10):
        r = res[t]["m-e4m3"]
        assert r["reduction_rel_rmse"] > 1.3 and r["reduction_mean_rel_err"] > 1.3
        assert 1.0 <= r["k_percentiles_5_50_95"][1] <= 3.0  # typical k of m: 1-3


def test_second_moment_k_grows_into_the_typical_range(res):
    r = res[10]["v-e4m3"]
    assert 4.0 <= r["k_percentiles_5_50_95"][1] <= 15.0  # typical k of v: 5-15, reached as v narrows
    assert r["reduction_rel_rmse"] > 2.0


def test_v_formats_equalize_after_expansion(res):
    r4, r5 = res[10]["v-e4m3"], res[10]["v-e5m2"]
    # without expansion E4M3 is clearly better; with it the two are close
    assert r5["k1"]["rel_rmse"] > 1.5 * r4["k1"]["rel_rmse"]
    assert r5["expansion"]["rel_rmse"] < 1.25 * r4["expansion"]["rel_rmse"]


def test_e4m3_is_better_for_the_first_moment(res):
    for t in (1, 10):
        assert res[t]["m-e4m3"]["expansion"]["rel_rmse"] < res[t]["m-e5m2"]["expansion"]["rel_rmse"]
        assert res[t]["m-e4m3"]["k1"]["rel_rmse"] < res[t]["m-e5m2"]["k1"]["rel_rmse"]
