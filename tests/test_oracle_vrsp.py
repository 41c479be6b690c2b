"""Pins of the VRSP reference (oracle/vrsp.py) and parity of the library's libra_vrsp with it.

VRSP is Algorithm 1 of the Libra technical review (section 4.2): exact-cardinality
heaviest-first placement of packed sequences into pools, workload F = sum of squared
sample lengths (eq. 1).  Host code only: these tests run without a GPU.
"""
import json
import os

import numpy as np
import pytest

import oracle.vrsp as V

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vrsp_hand.json")


def test_hand_worked_window():
    g = json.load(open(GOLDEN))
    pool_of, order, load = V.vrsp(g["workload"], g["pool_size"])
    assert pool_of == g["pool_of"] and order == g["order"] and load == g["pool_load"]
    assert V.imbalance(load) == pytest.approx(g["r_minus_1"])


def test_workload_proxy_eq1_example():
    # One 40K-token sample costs ten times ten 4K-token samples (review, section 3.1).
    assert V.workload([40000]) == 10 * V.workload([4000] * 10)
    assert V.workload([3, 0, 4]) == 25


def _windows(seed, n=60):
    rng = np.random.default_rng(seed)
    for t in range(n):
        P = int(rng.integers(1, 9))
        K = int(rng.integers(1, 17))
        if t % 3 == 0:
            F = rng.integers(0, 4, P * K).tolist()            # many ties
        else:
            F = (np.exp(rng.normal(13, 2.0, P * K))).astype(np.int64).tolist()
        yield F, P


def test_exact_cardinality_and_permutation():
    for F, P in _windows(1):
        pool_of, order, load = V.vrsp(F, P)
        K = len(F) // P
        assert sorted(order) == list(range(len(F)))
        assert np.bincount(pool_of, minlength=K).tolist() == [P] * K
        for k in range(K):
            members = order[k * P:(k + 1) * P]
            assert all(pool_of[i] == k for i in members)
            assert load[k] == sum(F[i] for i in members)


def test_pool_size_one_is_the_sorted_order():
    F = [3, 7, 7, 0, 5]
    pool_of, order, _ = V.vrsp(F, 1)
    assert order == [1, 2, 4, 0, 3]                   # decreasing F, ties by index
    assert [pool_of[i] for i in order] == list(range(5))


def test_one_pool_takes_everything_in_sorted_order():
    F = [3, 7, 7, 0, 5, 1]
    pool_of, order, load = V.vrsp(F, 6)
    assert pool_of == [0] * 6 and order == [1, 2, 4, 0, 5, 3] and load == [sum(F)]


def test_equal_workloads_fill_round_robin():
    # Every load ties at each round, so sequence t (in index order) lands on pool t mod K.
    K, P = 5, 4
    pool_of, order, load = V.vrsp([7] * (K * P), P)
    assert pool_of == [t % K for t in range(K * P)]
    assert load == [7 * P] * K


def test_relabelling_keeps_the_pool_loads():
    rng = np.random.default_rng(5)
    F = rng.permutation(np.arange(1, 65) ** 2).tolist()   # distinct workloads
    _, _, load = V.vrsp(F, 8)
    perm = rng.permutation(len(F))
    _, _, load2 = V.vrsp([F[i] for i in perm], 8)
    assert sorted(load) == sorted(load2)


def test_cardinality_overrides_plain_lpt():
    # Plain LPT would put the last light sequence on the light pool (loads 10 and 3); with
    # P = 2 that pool is full, so it must go to the heavy one: loads 11 and 2.
    pool_of, order, load = V.vrsp([10, 1, 1, 1], 2)
    assert load == [11, 2] and pool_of == [0, 1, 1, 0]


def test_balances_better_than_index_order_on_long_tailed_windows():
    rng = np.random.default_rng(7)
    for _ in range(10):
        F = (np.exp(rng.normal(13, 2.0, 128))).astype(np.int64).tolist()
        _, _, load = V.vrsp(F, 8)
        index_order = [sum(F[k * 8:(k + 1) * 8]) for k in range(16)]
        assert V.imbalance(load) <= V.imbalance(index_order)


def test_rejects_partial_pools():
    with pytest.raises(ValueError):
        V.vrsp([1, 2, 3], 2)


# ------------------------------------------------------------- the library's VRSP
@pytest.fixture(scope="module")
def lib():
    import packed_varlen_attention_cu_amd as m
    return m


def test_library_vrsp_matches_reference(lib):
    for seed in (11, 12):
        for F, P in _windows(seed, 80):
            pool_of, order, load = lib.libra_vrsp(F, P)
            r = V.vrsp(F, P)
            assert pool_of.tolist() == r[0] and order.tolist() == r[1] and load.tolist() == r[2]


def test_library_vrsp_hand_worked_window(lib):
    g = json.load(open(GOLDEN))
    pool_of, order, load = lib.libra_vrsp(g["workload"], g["pool_size"])
    assert pool_of.tolist() == g["pool_of"] and order.tolist() == g["order"] and load.tolist() == g["pool_load"]


def test_library_pack_workload(lib):
    assert lib.libra_pack_workload([0, 3, 3, 7]) == 9 + 0 + 16
    assert lib.libra_pack_workload([0]) == 0
    with pytest.raises(lib.LibraError):
        lib.libra_pack_workload([0, 5, 4])
    with pytest.raises(lib.LibraError):
        lib.libra_pack_workload([1, 5])


@pytest.mark.parametrize("F,P", [([1, 2, 3], 2), ([1, -2], 1), ([], 1), ([1, 2], 0)])
def test_library_vrsp_rejects_bad_windows(lib, F, P):
    with pytest.raises(lib.LibraError):
        lib.libra_vrsp(F, P)
