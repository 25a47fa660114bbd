"""Cost model and allocation (Sec. 4.2) against the worked operating points the
paper prints (App. A.4, Table 6 text; blog summary: 70% target -> s1 = 0.7,
s2 = 76.7%)."""
import pytest

from free_sparse_swiglu_amd import costmodel


def test_effective_sparsity_definition():
    assert costmodel.effective_sparsity(0.0, 0.0) == pytest.approx(-2.0 / 9.0)
    assert costmodel.effective_sparsity(1.0, 0.7) == pytest.approx(0.7)
    assert costmodel.prox_cost(1.0, 1.0) == 0.0


def test_allocations_match_pages(golden):
    fx = golden("pages_values.json")["allocations"]
    for pt in fx["points"]:
        s1, s2 = costmodel.allocate(pt["e"], fx["alpha"], fx["s_ref"], tuple(fx["s1_range"]))
        assert costmodel.effective_sparsity(s1, s2, fx["alpha"]) == pytest.approx(pt["e"], abs=1e-12)
        assert fx["s1_range"][0] <= s1 <= fx["s1_range"][1]
        if "s1" in pt:
            assert s1 == pytest.approx(pt["s1"], abs=1e-12)
        # printed to 0.1 percentage point
        assert abs(s2 - pt["s2"]) <= 0.0005 + 1e-12
    # the two interior points: s1 absorbs the budget (50% -> 0.1, 60% -> 0.55)
    assert costmodel.allocate(0.5)[0] == pytest.approx(0.1)
    assert costmodel.allocate(0.6)[0] == pytest.approx(0.55)
