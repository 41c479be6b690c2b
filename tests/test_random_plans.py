"""Planner parity and plan shape on seeded random packs (no GPU): the C planner must match the
oracle's tiles, items, costs and placement bit for bit, and every plan must hold what the
kernels assume of it.  The GPU parity test of the same cases launches only plans that pass
here."""
import pytest

from tests import _random_cases as R
from tests.test_capi import make_plan
from tests.test_capi import test_planner_matches_oracle as planner_matches_oracle

CASES = [R.random_case(s) for s in range(40)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_pack_planner_matches_oracle(case):
    planner_matches_oracle(*CASES[case])


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_pack_plan_shapes(case):
    lens, h_q, h_kv, d, B, W, kw = CASES[case]
    plan, _ = make_plan(lens, h_q, h_kv, d, B, W, **kw)
    R.check_plan_shapes(plan, sum(lens), h_q, h_kv)


def test_random_cases_cover_the_shapes():
    """The generator reaches every head dim, GQA group sizes 1 to 8, all three placement modes,
    empty and one-token samples, and packs shorter than one key block."""
    ds = {c[3] for c in CASES}
    groups = {c[1] // c[2] for c in CASES}
    modes = {c[6].get("assign", 0) for c in CASES}
    assert ds == {64, 128}
    assert {1, 2, 3, 4, 8} <= groups
    assert modes == {0, 1, 2}
    assert any(0 in c[0] for c in CASES) and any(1 in c[0] for c in CASES)
    assert any(sum(c[0]) < 64 for c in CASES) or any(min(x for x in c[0] if x) < 64 for c in CASES)
