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
        assert it["cost"] == P.executed_slots(P._ranges(cu), it["row0"], it["nrows"], it["nheads"]) + 7
        assert it["cost"] - 7 >= it["pairs"]
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


# ------------------------------------------------ executed-work costs, worked by hand
HAND_CU = [0, 100, 400, 450]          # samples of 100, 300 and 50 tokens


def test_kv_item_cost_hand_worked():
    """Chunks of 192 keys, g = 2.  Chunk 0 (keys 0-191): its last key lies in sample 1, which ends
    at 400, so the query walk runs from 0 up to 400: ceil(400 / 64) = 7 blocks; executed
    2 x 7 x 64 x 192 = 172032.  Pairs: keys 0-99 see 100 - k queries (5050 in all), keys 100-191
    see 400 - k (209 + ... + 300 = 23414): 2 x 28464 = 56928.  Chunk 1 (192-383): walk 192 -> 400,
    ceil(208 / 64) = 4 blocks, 2 x 4 x 64 x 192 = 98304; pairs 2 x (17 + ... + 208) = 43200.
    Chunk 2 (384-449, 66 keys): its last key is in sample 2 (ends 450): walk 384 -> 450,
    ceil(66 / 64) = 2 blocks, 2 x 2 x 64 x 66 = 16896; pairs 2 x (136 + 1275) = 2822."""
    kv = P.kv_items(HAND_CU, 450, h_q=4, h_kv=2)
    got = [(it["row0"], it["nrows"], it["kv_head"], it["pairs"], it["cost"]) for it in kv]
    assert got == [(0, 192, 0, 56928, 172032), (0, 192, 1, 56928, 172032),
                   (192, 192, 0, 43200, 98304), (192, 192, 1, 43200, 98304),
                   (384, 66, 0, 2822, 16896), (384, 66, 1, 2822, 16896)]
    assert [it["cost"] for it in P.kv_items(HAND_CU, 450, 4, 2, overhead=5)] == [172037] * 2 + [98309] * 2 + [16901] * 2


def test_fwd_item_executed_cost_hand_worked():
    """One tile of 450 tokens x 4 heads on one KV head: items of 96 rows x 4 heads, twelve waves of
    32 rows (three row ranges, four heads each).  An item's walk runs from the block holding the
    start of its first row's sample to the block holding its last row, and every wave counts
    every block of it.  Rows 0-95 (sample 0, start 0): blocks 0-1, 2 x 12 = 24 wave-blocks.
    Rows 96-191 (first row in sample 0): blocks 0-2, 3 x 12 = 36.  Rows 192-287 (sample 1,
    start 100, block 1): blocks 1-4, 48.  Rows 288-383: blocks 1-5, 60.  Rows 384-449 (66 rows,
    first row in sample 1, three row ranges): blocks 1-7, 7 x 12 = 84.  Each wave-block is
    32 x 64 = 2048 slots.  Pairs: rows 0-95 are sample 0's first 96 queries,
    4 x 96 x 97 / 2 = 18624."""
    items = P.fwd_items(HAND_CU, 450, 4, 1, 450, 4)
    assert [(it["row0"], it["nrows"], it["nheads"]) for it in items] == [(0, 96, 4), (96, 96, 4), (192, 96, 4),
                                                                        (288, 96, 4), (384, 66, 4)]
    assert [it["cost"] for it in items] == [2048 * b for b in (24, 36, 48, 60, 84)]
    assert items[0]["pairs"] == 18624
    by_pairs = P.fwd_items(HAND_CU, 450, 4, 1, 450, 4, overhead=3, cost="pairs")
    assert [it["cost"] for it in by_pairs] == [it["pairs"] + 3 for it in items]


def test_dq_item_executed_cost_hand_worked():
    """The same tile cut into dQ items of 64 rows x 4 heads (eight waves: two row ranges of four
    heads).  Rows 0-63: block 0, 1 x 8.  64-127: blocks 0-1, 16.  128-191 (sample 1, start 100,
    block 1): blocks 1-2, 16.  192-255: blocks 1-3, 24.  256-319: 1-4, 32.  320-383: 1-5, 40.
    384-447 (first row in sample 1): 1-6, 48.  448-449 (2 rows, one row range, four waves;
    first row in sample 2, start 400, block 6): blocks 6-7, 2 x 4 = 8."""
    items = P.fwd_items(HAND_CU, 450, 4, 1, 450, 4, columns=P.DQ_ITEM_COLUMNS)
    assert [(it["row0"], it["nrows"]) for it in items] == [(r, 64) for r in range(0, 448, 64)] + [(448, 2)]
    assert [it["cost"] for it in items] == [2048 * b for b in (8, 16, 16, 24, 32, 40, 48, 8)]


def test_executed_cost_pins_catch_block_size_slips(monkeypatch):
    """Planted in the oracle: a wrong key-block size, or query blocks of the dK/dV walk taken at
    the wrong alignment; the hand pins above must fail."""
    monkeypatch.setattr(P, "KEY_BLOCK", 32)
    with pytest.raises(AssertionError):
        test_fwd_item_executed_cost_hand_worked()
    with pytest.raises(AssertionError):
        test_dq_item_executed_cost_hand_worked()
    monkeypatch.undo()
    monkeypatch.setattr(P, "QUERY_TILE", 64)
    with pytest.raises(AssertionError):
        test_dq_item_executed_cost_hand_worked()
    monkeypatch.undo()
    monkeypatch.setattr(P, "KV_QUERY_BLOCK", 128)
    with pytest.raises(AssertionError):
        test_kv_item_cost_hand_worked()


def test_executed_cost_covers_pairs_and_counts_the_whole_walk():
    """Executed slots are at least the pairs (every pair lies in a block of the walk).  An item of
    384 rows of one head at rows 4224-4607 of an 8192-token sample walks blocks 0 .. 4607 / 64 =
    71, and all twelve waves count all 72 of them, though the first wave's rows see keys only up
    to block 4255 / 64 = 66.  An item whose first row lies in an earlier sample walks that
    sample too: rows 96-191 of samples [0, 100) and [100, 400) start at block 0."""
    cu = [0, 8192]
    items = P.fwd_items(cu, 8192, 1, 1, 8192, 1)
    it = next(i for i in items if i["row0"] == 4224)
    assert it["cost"] == 12 * 72 * 2048
    for i in items:
        assert i["cost"] >= i["pairs"]
    assert P.executed_slots(P._ranges(HAND_CU), 96, 96, 1) == 3 * 3 * 2048
    assert P.executed_slots(P._ranges(HAND_CU), 100, 92, 1) == 3 * 2 * 2048


# ------------------------------------------------ Algorithm 2 with the L2 residency term
def test_l2_residency_hand_worked():
    """Ten workers (worker r on XCD r mod 8: workers 0 and 8 share XCD 0, 1 and 9 share XCD 1),
    tau = 1: a worker fits while load + cost <= 2 x 14 / 10 = 2.8 (sum of costs 14).  Units
    (cost, groups): 0 (6, A), 1 (3, B), 2 (3, A), 3 (1, B), 4 (1, B); volumes A = 5, B = 7.
      unit 0: fits nowhere; all loads 0 and all terms 5 -> worker 0; XCD 0 holds A.
      unit 1: fits nowhere; least load 0 on workers 1-9, terms all 7 -> worker 1; XCD 1 holds B.
      unit 2: fits nowhere; least load 0 on workers 2-9, and worker 8 (XCD 0) already holds A
              (term 0 against 5) -> worker 8.
      unit 3: fits on workers 2-7 and 9 (load 0); worker 9 (XCD 1) holds B -> term 0 -> 9.
      unit 4: fits on 2-7 (load 0, term 7) and 9 (load 1, term 0): the term ranks before the
              load within the target -> 9.
    Without the term the same units go to workers 0, 1, 2, 3, 4 (least load, then id)."""
    A_, B_ = 0, 1
    res = P.L2Residency([{A_}, {B_}, {A_}, {B_}, {B_}], {A_: 5, B_: 7})
    sigma, order = P.place([6, 3, 3, 1, 1], 10, 1.0, dcomm=res.dcomm, commit=res.commit)
    assert order == [0, 1, 2, 3, 4] and sigma == [0, 1, 8, 9, 9]
    assert res.held[0] == {A_} and res.held[1] == {B_}
    assert P.place([6, 3, 3, 1, 1], 10, 1.0)[0] == [0, 1, 2, 3, 4]


def test_item_kv_groups_are_the_samples_its_rows_meet():
    """eq. 7 for items: rows 96-191 of HAND_CU meet samples 0 and 1; with h_kv = 2 and KV head 1
    the group ids are 0 * 2 + 1 and 1 * 2 + 1.  Empty samples hold no group."""
    it = dict(row0=96, nrows=96, kv_head=1)
    assert P.kv_groups(HAND_CU, it, 2) == {1, 3}
    assert P.kv_groups([0, 100, 100, 400], dict(row0=99, nrows=2, kv_head=0), 1) == {0, 2}
    assert P.group_volumes(HAND_CU, 2) == {0: 100, 1: 100, 2: 300, 3: 300, 4: 50, 5: 50}


def test_l2_mode_places_every_item_once_and_keeps_loads():
    """On a random pack the L2 mode places the same items (each once) with the same total load,
    and no worker ends beyond the soft target by more than one unit's cost."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 700, size=12)]
    cu = cu_of(lens)
    L = sum(lens)
    items = P.fwd_items(cu, L, 8, 2, 512, 4)
    o1, ids1, f1, load1 = P.zigzag_queue(cu, items, 16, 0.03, "lpt", h_kv=2)
    o2, ids2, f2, load2 = P.zigzag_queue(cu, items, 16, 0.03, "l2", h_kv=2)
    assert sorted(ids2) == sorted(ids1) == list(range(len(items)))
    assert sum(load2) == sum(load1)
    unit_max = max(it["cost"] for it in items) * 2
    assert max(load2) <= 1.03 * sum(load2) / 16 + unit_max
