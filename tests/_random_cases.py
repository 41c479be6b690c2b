"""Seeded random packs and planner settings, shared by the CPU plan checks and the GPU parity
tests.  Shapes and settings only: no attention arithmetic lives here.

Each case draws a GQA shape (h_kv in {1, 2, 4}, group sizes 1-8, h_q <= 32, d in {64, 128}), a
pack of up to about 2600 tokens mixing empty, one-token, block-edge (64 k - 1 .. 64 k + 1) and
lognormal samples, an SH-Tile shape (any B >= 16, any W dividing h_q) and planner settings
(placement mode, worker count, cost model, item overhead, tau, per-class speeds)."""
from __future__ import annotations

import numpy as np

ITEM_COLUMNS = {"fwd": 384, "dq": 256}   # query columns per forward / dQ work item
KV_ITEM_KEYS = 192                       # keys per dK/dV work item


def random_case(seed: int):
    """(lengths, h_q, h_kv, d, B, W, planner keywords) of case `seed`."""
    rng = np.random.default_rng(7919 + seed)
    h_kv = int(rng.choice([1, 2, 4]))
    groups = [g for g in (1, 2, 3, 4, 6, 8) if h_kv * g <= 32]
    h_q = h_kv * int(rng.choice(groups))
    d = int(rng.choice([64, 128]))
    total = int(rng.integers(1, 2600))
    lens, left = [], total
    while left > 0 and len(lens) < 400:
        kind = int(rng.integers(0, 6))
        if kind == 0:
            x = 0
        elif kind == 1:
            x = 1
        elif kind == 2:
            x = 64 * int(rng.integers(1, 8)) + int(rng.integers(-1, 2))
        else:
            x = int(rng.lognormal(5.0, 1.3)) + 1
        x = min(x, left)
        lens.append(x)
        left -= x
    if left > 0:
        lens.append(left)
    if rng.random() < 0.3:
        lens = [0] + lens
    if rng.random() < 0.3:
        lens = lens + [0]
    L = sum(lens)
    B = int(rng.integers(16, L + 200))
    W = int(rng.choice([w for w in range(1, h_q + 1) if h_q % w == 0]))
    kw = {"assign": int(rng.choice([0, 0, 1, 2]))}
    if rng.random() < 0.5:
        kw["num_cus"] = int(rng.integers(1, 97))
    if rng.random() < 0.3:
        kw["cost"] = 1
    if rng.random() < 0.3:
        kw["item_overhead"] = int(rng.integers(0, 50000))
    if rng.random() < 0.3:
        kw["tau"] = float(rng.choice([0.0, 0.01, 0.1]))
    if rng.random() < 0.3:
        kw["worker_speed"] = [int(x) for x in rng.integers(500, 2001, 8)]
    return lens, h_q, h_kv, d, B, W, kw


def check_plan_shapes(plan, L: int, h_q: int, h_kv: int) -> None:
    """What the kernels assume of a plan before they index with it: every item inside the pack
    and the heads of its KV head, at most one item's columns (forward, dQ) or keys (dK/dV),
    and every queue a permutation of its items split by non-decreasing offsets."""
    g = h_q // h_kv
    ncu = plan.info.num_cus
    for name, items, off in (("fwd", plan.items, plan.cu_off), ("dq", plan.dq_items, plan.dq_cu_off),
                             ("kv", plan.kv_items, plan.kv_cu_off)):
        off = np.asarray(off, dtype=np.int64)
        assert len(off) == ncu + 1 and off[0] == 0 and off[-1] == len(items), name
        assert (np.diff(off) >= 0).all(), name
        assert sorted(int(x) for x in items["id"]) == list(range(len(items))), name
        row0 = items["row0"].astype(np.int64)
        nrows = items["nrows"].astype(np.int64)
        nh = items["nheads"].astype(np.int64)
        h0 = items["head0"].astype(np.int64)
        kv = items["kv_head"].astype(np.int64)
        assert (nrows >= 1).all() and (row0 >= 0).all() and (row0 + nrows <= L).all(), name
        assert (kv >= 0).all() and (kv < h_kv).all(), name
        assert (h0 >= kv * g).all() and (h0 + nh <= (kv + 1) * g).all(), name
        if name == "kv":
            assert (nh == g).all() and (nrows <= KV_ITEM_KEYS).all(), name
        else:
            assert np.isin(nh, (1, 2, 4)).all(), name
            assert (nrows * nh <= ITEM_COLUMNS[name]).all(), name
