"""Pins of the plain-Python planner (eq. 6-8 tiles, work items, Algorithm 2)."""
import json
import os

import numpy as np
import pytest

from oracle import plan as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_2k_tile_pairs.json")


def cu_of(lens):
    return [0] + list(np.cumsum(lens))


def test_eq8_worked_tables():
    """Hand-derived per-head tile pairs for lengths (1024, 512, 256, 256)."""
    g = json.load(open(GOLDEN))
    cu = cu_of(g["lengths"])
    for B, entry in g["blocks"].items():
        tiles = P.sh_tiles(cu, 2048, h_q=1, B=int(B), W=1)
        assert [t["pairs"] for t in tiles] == entry["pairs"]
        assert [[t["sample_first"], t["sample_last"]] for t in tiles] == entry["sample_ranges"]
        assert sum(entry["pairs"]) == g["pairs_per_head_total"]
    assert sum(x * x for x in g["lengths"]) == g["sum_l_sq"]


@pytest.mark.parametrize("seed", range(6))
def test_tile_pairs_sum_to_closed_form(seed):
    """sum_t pairs_t = h_q * sum_j l_j (l_j + 1) / 2 (eq. 1 and eq. 8)."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, 700, size=int(rng.integers(1, 12)))]
    L = sum(lens)
    if L == 0:
        lens, L = [5], 5
    h_q = 8
    closed = h_q * sum(l * (l + 1) // 2 for l in lens)
    for B in (1, 64, 100, 256, L):
        for W in (1, 2, 8):
            tiles = P.sh_tiles(cu_of(lens), L, h_q, B, W)
            assert sum(t["pairs"] for t in tiles) == closed
            assert len(tiles) == ((L + B - 1) // B) * (h_q // W)


def test_eq1_worked_example():
    """One 40000-token sample does about 10x the attention work of ten 4000-token ones."""
    one = sum(t["pairs"] for t in P.sh_tiles([0, 40000], 40000, 1, 4096, 1))
    ten = sum(t["pairs"] for t in P.sh_tiles(cu_of([4000] * 10), 40000, 1, 4096, 1))
    assert one == 40000 * 40001 // 2 and ten == 10 * (4000 * 4001 // 2)
    assert abs(one / ten - 10.0) < 0.05        # sum of squares ratio is exactly 10


def test_tiles_cut_at_global_positions():
    tiles = P.sh_tiles(cu_of([5, 3, 9]), 17, h_q=4, B=6, W=2)
    assert [(t["tile_id"], t["tok_begin"], t["tok_end"], t["head_begin"]) for t in tiles] == [
        (0, 0, 6, 0), (1, 0, 6, 2), (2, 6, 12, 0), (3, 6, 12, 2), (4, 12, 17, 0), (5, 12, 17, 2)]
    # block 0: s0 q0..4 (15) + s1 q0 (1); block 1: s1 q1..2 (5) + s2 q0..3 (10); block 2: s2 q4..8 (35)
    assert [t["pairs"] for t in tiles] == [32, 32, 30, 30, 70, 70]
    assert [(t["sample_first"], t["sample_last"]) for t in tiles[::2]] == [(0, 1), (1, 2), (2, 2)]


@pytest.mark.parametrize("h_q,h_kv,W", [(4, 4, 2), (32, 8, 8), (32, 4, 8), (8, 1, 2), (32, 4, 4), (6, 2, 3), (12, 4, 6)])
def test_items_partition_tiles(h_q, h_kv, W):
    rng = np.random.default_rng(h_q * 100 + W)
    lens = [int(x) for x in rng.integers(1, 900, size=9)]
    L = sum(lens)
    cu = cu_of(lens)
    B = 512
    g = h_q // h_kv
    tiles = {t["tile_id"]: t for t in P.sh_tiles(cu, L, h_q, B, W)}
    items = P.fwd_items(cu, L, h_q, h_kv, B, W, overhead=7)
    cover = np.zeros((L, h_q), dtype=np.int64)
    per_tile = {}
    for it in items:
        t = tiles[it["tile_id"]]
        assert it["nheads"] in (1, 2, 4)
        assert it["nrows"] * it["nheads"] <= P.ITEM_COLUMNS
        assert t["tok_begin"] <= it["row0"] and it["row0"] + it["nrows"] <= t["tok_end"]
        for h in range(it["head0"], it["head0"] + it["nheads"]):
            assert h // g == it["kv_head"]
            assert t["head_begin"] <= h < t["head_begin"] + t["head_count"]
        cover[it["row0"]:it["row0"] + it["nrows"], it["head0"]:it["head0"] + it["nheads"]] += 1
        assert it["cost"] == it["pairs"] + 7
        per_tile[it["tile_id"]] = per_tile.get(it["tile_id"], 0) + it["pairs"]
    assert (cover == 1).all()
    assert all(per_tile[i] == t["pairs"] for i, t in tiles.items())
    assert [it["id"] for it in items] == list(range(len(items)))


def test_kv_items_cover_keys_and_pairs():
    lens = [300, 1, 0, 517, 90]
    L = sum(lens)
    items = P.kv_items(cu_of(lens), L, h_q=8, h_kv=2)
    cover = np.zeros((L, 2), dtype=np.int64)
    for it in items:
        cover[it["row0"]:it["row0"] + it["nrows"], it["kv_head"]] += 1
        assert it["nheads"] == 4 and it["head0"] == it["kv_head"] * 4
    assert (cover == 1).all()
    # every causal pair counted once from the key side: same total as from the query side
    assert sum(it["pairs"] for it in items) == 8 * sum(l * (l + 1) // 2 for l in lens)


def test_algorithm2_hand_case_lpt():
    # C = 1.03 * 20 / 2 = 10.3; order 0,1,2,3,4.  Loads: [5,0] [5,5] [9,5] [9,8];
    # unit 4 (3) fits nowhere (12, 11 > 10.3) -> fallback to the least loaded (worker 1).
    sigma, order = P.place([5, 5, 4, 3, 3], 2, 0.03)
    assert order == [0, 1, 2, 3, 4]
    assert sigma == [0, 1, 0, 1, 1]
    offsets, ids, load = P.queue([5, 5, 4, 3, 3], 2, 0.03)
    assert offsets == [0, 2, 5] and ids == [0, 2, 1, 3, 4] and load == [9, 11]


def test_algorithm2_hand_case_comm_then_fallback():
    # tau = 0, C = 7.  dcomm prefers worker 1.  Unit 0 (6) -> worker 1 (comm first);
    # unit 1 (4): only worker 0 fits -> 0; unit 2 (4): nothing fits -> least loaded (0).
    dcomm = lambda t, r: 0 if r == 1 else 1
    sigma, _ = P.place([6, 4, 4], 2, 0.0, dcomm)
    assert sigma == [1, 0, 0]


def test_algorithm2_ties_by_id_and_worker():
    sigma, order = P.place([3, 3, 3, 3], 3, 0.03)
    assert order == [0, 1, 2, 3]
    assert sigma == [0, 1, 2, 0]


def test_round_robin_ablation():
    offsets, ids, load = P.queue([9, 1, 1, 9], 2, mode="rr")
    assert offsets == [0, 2, 4] and ids == [0, 2, 1, 3] and load == [10, 10]


def test_lpt_balances_better_than_round_robin():
    rng = np.random.default_rng(3)
    costs = [int(x) for x in (rng.lognormal(8, 2, size=600))]
    _, _, lpt = P.queue(costs, 16)
    _, _, rr = P.queue(costs, 16, mode="rr")
    mean = sum(costs) / 16
    assert max(lpt) / mean < max(rr) / mean
    assert max(lpt) <= max(max(costs), 1.03 * mean + max(costs))


def test_kv_zigzag_units_hand_worked():
    """lens (1000, 500), one KV head: chunks of 192 keys end in sample 0 for c = 0..4 and in
    sample 1 for c = 5..7 (chunk 5 straddles).  Pairs: (0, 4), (1, 3), 2 alone; (5, 7), 6 alone."""
    cu = [0, 1000, 1500]
    kv = P.kv_items(cu, 1500, 2, 1)
    assert [it["row0"] for it in kv] == [0, 192, 384, 576, 768, 960, 1152, 1344]
    assert P.zigzag_units(cu, kv, last_key=True) == [(0, 4), (1, 3), (2, None), (5, 7), (6, None)]
    offsets, ids, flags, load = P.zigzag_queue(cu, kv, 1, last_key=True)      # one worker: pairs cannot unbalance
    # every item once; a pair's second chunk follows its first and walks up
    assert sorted(ids) == list(range(8))
    for a, b in [(0, 4), (1, 3), (5, 7)]:
        i = ids.index(a)
        assert ids[i + 1] == b and flags[i] == 0 and flags[i + 1] == P.REVERSE
    assert flags[ids.index(2)] == 0 and flags[ids.index(6)] == 0
    # pairs of one group cost the same: each chunk's query-block walk shortens by 3 blocks per chunk
    c = {it["id"]: it["cost"] for it in kv}
    assert c[0] + c[4] == c[1] + c[3]


def test_kv_zigzag_falls_back_when_pairs_unbalance():
    """One long sample and one KV head over many workers: equal-cost pairs would leave some
    workers a whole pair more than others (more than 0.5 % above the mean), so the single
    chunks are placed, all walking down, exactly as LPT over single chunks places them."""
    cu = [0, 40000, 40100]
    kv = P.kv_items(cu, 40100, 8, 1)
    offsets, ids, flags, load = P.zigzag_queue(cu, kv, 64, last_key=True)
    assert not any(flags)
    s_off, s_ids, s_load = P.queue([it["cost"] for it in kv], 64)
    assert (offsets, ids, load) == (s_off, s_ids, s_load)


def test_fwd_zigzag_pairs_hand_worked():
    """One sample of 1000 tokens, 4 query heads on one KV head, tiles of 500 x 4 heads: forward
    items of 96 rows x 4 heads, cut per tile (rows 0-479 in 5 items, 480-499 alone; the same
    for 500-999).  In row order the 12 items pair first-with-last: (0, 11), (1, 10), ..."""
    cu = [0, 1000]
    items = P.fwd_items(cu, 1000, 4, 1, 500, 4)
    assert [(it["row0"], it["nrows"]) for it in items] == [(0, 96), (96, 96), (192, 96), (288, 96), (384, 96),
                                                          (480, 20), (500, 96), (596, 96), (692, 96),
                                                          (788, 96), (884, 96), (980, 20)]
    assert P.zigzag_units(cu, items) == [(0, 11), (1, 10), (2, 9), (3, 8), (4, 7), (5, 6)]


def test_weighted_placement_hand_worked():
    """Two workers, worker 0 twice as fast: 6 -> worker 0 (finishes at 3 vs 6); 4 -> worker 1
    (4 vs 5); 3 -> worker 0 (4.5 vs 7).  Equal speeds give plain LPT."""
    sigma, order = P.place([6, 4, 3], 2, speed=[2000, 1000, 0, 0, 0, 0, 0, 0])
    assert order == [0, 1, 2] and sigma == [0, 1, 0]
    assert P.place([6, 4, 3], 2, speed=[700] * 8) == P.place([6, 4, 3], 2)
