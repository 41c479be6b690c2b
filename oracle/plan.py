"""Reference SH-Tile planner and FLOPs-aware placement, in plain Python.

TEST INFRASTRUCTURE ONLY.  Used by the tests to check the library's planner
bit for bit; it shares no code with it.

SH-Tiles (Libra technical review, section 5.1, eq. 6).  The packed sequence
is cut at global token positions into blocks of at most B tokens (a block may
straddle samples, the last one may be short) and the h_q query heads into
equal contiguous shards of W heads.  Tile t = (block b, shard s) with
tile_id = b * S + s, S = h_q / W (block-major: the pages break placement ties
"by tile ID" and leave the numbering open, so this is a reading).

KV groups (section 5.2, eq. 7).  K(t) is the set of samples the block
intersects; it is contiguous, so it is reported as [sample_first, sample_last].

Tile FLOPs (section 5.3, eq. 8).  For every sample j that block b intersects,
with sample-local query positions a..e-1 inside the block, query position q
pairs with q + 1 keys; pairs_t = W * sum_j sum_{q=a}^{e-1} (q + 1).  Forward
FLOPs are 4 * d per pair (two matrix products of 2 * d each).

Work items (a reading: on one GPU the workers are CUs and a whole SH-Tile is
too coarse for 256 of them).  Every tile is split into items that one
workgroup runs, of at most c query columns (positions x heads): c = 384 for
the forward kernel, c = 256 for the dQ kernel, which cuts the same tiles into
its own items and places them the same way:
  * for each KV head kappa whose query heads meet the tile's shard, the heads
    H = shard ∩ group(kappa) are cut into groups of nh heads, nh = 4 if |H| is a
    multiple of 4, else 2 if even, else 1;
  * each head group takes the tile's rows in chunks of c / nh positions.
An item's pairs are eq. 8 restricted to its rows and heads.  Items are
numbered in (tile_id, kappa, head group, row chunk) order.

Item cost (a reading: the pages cost a tile by its causal pairs, eq. 8, which
measures the useful work but not what a kernel that steps through whole
64-key blocks executes).  An item's workgroup holds its rows in waves of 32
query positions of one head (nh * ceil(nrows / 32) waves) and steps through
the 64-key blocks floor(start_j / 64) .. floor((row0 + nrows - 1) / 64), j
being the sample of its first row.  Every step copies a block and
synchronises the workgroup whether or not a wave's rows see a key in it, so a
step costs about the same for every wave.  The executed cost counts 32 x 64
query-key slots for every (wave, block) of that walk, plus a fixed per-item
overhead (a planner parameter).  The "pairs" cost model (eq. 8 pairs plus the
overhead) is kept for comparison.

Key-major items for the dK/dV pass: keys are cut at global positions into
chunks of 192 (the dK/dV kernel's six key groups of 32); item (chunk c, KV
head kappa) has id c * h_kv + kappa and covers all g = h_q / h_kv query heads
of kappa.  Its pairs count, for every key k in the chunk, the queries q >= k
of k's sample: g * sum_k (end(k) - k).  Its cost is the work the dK/dV kernel
executes for it, masked or not: g heads x the query blocks of 64 rows from
the chunk's first key rounded down to a multiple of 64 up to the end of the
sample of its last key x 64 rows x its keys, plus the overhead.

Zigzag units (a reading for one GPU: the pages place tiles, not items, and
say nothing of walk order).  A forward or dQ item walks the key blocks of its
rows up from the start of its first row's sample; a dK/dV item walks the
query blocks of its keys down from the end of its last key's sample.  Items
of one group (the sample of the first row, or of the last key for dK/dV
items; the KV head; the first head) are taken in row order u_0 .. u_{m-1};
u_i is paired with u_{m-1-i} (the middle item of an odd group stands alone).
A pair is placed as one unit of cost f(u_i) + f(u_{m-1-i}), numbered by its
first item's id, and its worker runs u_i in the default order, then u_{m-1-i}
in reverse (flag REVERSE).  Pairs of a group then cost the same, and pairs
that start together read the same block at every step, which lets the
workers of one L2 share the streamed rows.  Pairs are coarser units than
single items: they are kept only if plain least-finish placement of the pairs
leaves the largest worker finish time within 0.5 % of the mean one;
otherwise the single items are placed, none reversed (a pack dominated by
one sample and one KV head, such as the 1M-token share, would otherwise lose
its balance).

Placement (Algorithm 2, section 5.4).  Units go out heaviest first, equal
costs in id order.  A unit goes to a worker that stays within the soft
target of (1 + tau) times the even share if there is one -- among those the
one whose communication term is smallest, then the least loaded, then the
lowest id -- and otherwise to the least loaded worker, then smallest
communication, then lowest id.  Loads are read as finish times load / speed:
worker r belongs to speed class r mod 8 (the XCD that runs workgroup r),
speeds in thousandths with 0 read as 1000 (an extension for workers of
unequal speed; equal speeds give the section's rule exactly).  A worker
runs its units in the order they were placed.

The communication term (eq. 9) on one GPU.  Every tensor is in HBM, so
nothing is sent; what an XCD fetches into its L2 plays the part of what a
worker fetches over the network.  A unit's KV groups are (sample j, KV head
kappa) for each non-empty sample j its rows meet (its key rows for dK/dV
items; for a zigzag pair, the union of both items' groups), each of volume
l_j tokens.  C_x is the set of groups already committed to XCD x, and
dcomm(t, r) is the summed volume of t's groups not in C_{r mod 8}; after t
goes to r, its groups join C_{r mod 8}.  Eq. 9's second term (Q and output
away from a Q-home worker) has no counterpart: there is no Q home on one GPU.
Mode "lpt" takes dcomm = 0, mode "l2" the residency term, mode "rr" is the
no-placement ablation (unit i to worker i mod |W|).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

ITEM_COLUMNS = 384                       # query positions x heads per forward item
DQ_ITEM_COLUMNS = 256                    # query positions x heads per dQ item
KV_CHUNK = 192                           # keys per dK/dV item
KV_QUERY_BLOCK = 64                      # query rows per step of the dK/dV kernel
REVERSE = 1                              # item flag: walk in the reverse of the default order
QUERY_TILE = 32                          # query positions per wave of the forward and dQ kernels
KEY_BLOCK = 64                           # keys per block the forward and dQ kernels compute


def _ranges(cu):
    cu = [int(x) for x in cu]
    if not cu or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    for a, b in zip(cu, cu[1:]):
        if b < a:
            raise ValueError("cu_seqlens must be non-decreasing")
    return [(cu[j], cu[j + 1]) for j in range(len(cu) - 1)]


def _triangle_sum(a: int, e: int) -> int:
    """sum_{q=a}^{e-1} (q + 1), summed term by term."""
    return sum(q + 1 for q in range(a, e))


def _block_pairs(ranges, lo: int, hi: int):
    """Per-head causal pairs of query rows [lo, hi) and the non-empty samples they touch."""
    pairs = 0
    touched = []
    for j, (s, e) in enumerate(ranges):
        a, b = max(lo, s), min(hi, e)
        if a >= b:
            continue
        touched.append(j)
        pairs += _triangle_sum(a - s, b - s)
    return pairs, touched


def sh_tiles(cu, total_tokens: int, h_q: int, B: int, W: int) -> list:
    """Tiles in tile_id order, each with its rows, heads, K(t) and eq. 8 pairs."""
    if B <= 0 or W <= 0 or h_q % W:
        raise ValueError("bad tile shape")
    ranges = _ranges(cu)
    if ranges and ranges[-1][1] != total_tokens:
        raise ValueError("cu_seqlens must end at L")
    S = h_q // W
    nblocks = (total_tokens + B - 1) // B
    out = []
    for b in range(nblocks):
        lo, hi = b * B, min(total_tokens, (b + 1) * B)
        per_head, touched = _block_pairs(ranges, lo, hi)
        for s in range(S):
            out.append(dict(tile_id=b * S + s, block=b, shard=s, tok_begin=lo, tok_end=hi,
                            head_begin=s * W, head_count=W,
                            sample_first=touched[0], sample_last=touched[-1],
                            pairs=W * per_head))
    return out


def _head_group_size(n: int) -> int:
    if n % 4 == 0:
        return 4
    if n % 2 == 0:
        return 2
    return 1


def executed_slots(ranges, row0: int, nrows: int, nheads: int) -> int:
    """Query-key slots of one forward or dQ item's walk: every key block from the one holding
    the start of its first row's sample to the one holding its last row, for every wave (32
    rows of one head), times 32 x 64."""
    start = next(s for s, end in ranges if s <= row0 < end)
    blocks = range(start // KEY_BLOCK, (row0 + nrows - 1) // KEY_BLOCK + 1)
    waves = nheads * -(-nrows // QUERY_TILE)
    return waves * len(blocks) * QUERY_TILE * KEY_BLOCK


def fwd_items(cu, total_tokens, h_q, h_kv, B, W, overhead=0, columns=ITEM_COLUMNS, cost="executed") -> list:
    """Forward work items in id order (dQ items: columns=DQ_ITEM_COLUMNS); cost "executed" or
    "pairs"."""
    g = h_q // h_kv
    ranges = _ranges(cu)
    items = []
    for t in sh_tiles(cu, total_tokens, h_q, B, W):
        h_lo, h_hi = t["head_begin"], t["head_begin"] + t["head_count"]
        for kappa in range(h_lo // g, (h_hi - 1) // g + 1):
            heads = list(range(max(h_lo, kappa * g), min(h_hi, (kappa + 1) * g)))
            nh = _head_group_size(len(heads))
            rows = columns // nh
            for gi in range(len(heads) // nh):
                for r0 in range(t["tok_begin"], t["tok_end"], rows):
                    r1 = min(t["tok_end"], r0 + rows)
                    per_head, _ = _block_pairs(ranges, r0, r1)
                    work = (nh * per_head if cost == "pairs"
                            else executed_slots(ranges, r0, r1 - r0, nh))
                    items.append(dict(id=len(items), tile_id=t["tile_id"], row0=r0, nrows=r1 - r0,
                                      kv_head=kappa, head0=heads[gi * nh], nheads=nh,
                                      pairs=nh * per_head, cost=work + overhead))
    return items


def kv_items(cu, total_tokens, h_q, h_kv, overhead=0) -> list:
    """dK/dV work items in id order (chunk-major, then KV head)."""
    g = h_q // h_kv
    ranges = _ranges(cu)
    items = []
    nchunks = (total_tokens + KV_CHUNK - 1) // KV_CHUNK
    for c in range(nchunks):
        lo, hi = c * KV_CHUNK, min(total_tokens, (c + 1) * KV_CHUNK)
        per_head = 0
        for s, e in ranges:
            a, b = max(lo, s), min(hi, e)
            per_head += sum(e - k for k in range(a, b))
        last_end = next(e for s, e in ranges if s <= hi - 1 < e)   # the last key's sample
        q_first = lo - lo % KV_QUERY_BLOCK
        q_blocks = -(-(last_end - q_first) // KV_QUERY_BLOCK)
        executed = g * q_blocks * KV_QUERY_BLOCK * (hi - lo)
        for kappa in range(h_kv):
            items.append(dict(id=len(items), tile_id=-1, row0=lo, nrows=hi - lo, kv_head=kappa,
                              head0=kappa * g, nheads=g, pairs=g * per_head,
                              cost=executed + overhead))
    return items


def _speeds(speed):
    s = [int(x) if x else 1000 for x in (speed if speed is not None else [0] * 8)]
    return s, all(x == s[0] for x in s)


def _f32(x: float) -> float:
    """The value a float parameter has once stored as a C float (the plan holds tau so)."""
    return float(np.float32(x))


def place(costs, n_workers: int, tau: float = 0.03, dcomm=None, speed=None, commit=None):
    """Algorithm 2: returns (worker of each unit, units in placement order).

    One argmin per unit over a key that ranks every worker within the soft
    target ahead of every worker beyond it: (0, dcomm, finish, r) within,
    (1, finish, dcomm, r) beyond, where finish = (load + cost) / speed.  Within
    the target means finish <= (1 + tau) * sum(cost) / sum(speed), evaluated
    as (load + cost) * sum(speed) <= (1 + tau) * sum(cost) * speed in double
    precision.  dcomm(t, r) is the communication term (0 when None);
    commit(t, r), if given, is told of each placement."""
    s, _ = _speeds(speed)
    n = len(costs)
    speed_sum = float(sum(s[r % 8] for r in range(n_workers)))
    budget = (1.0 + _f32(tau)) * float(sum(costs))
    load = [0] * n_workers
    sigma = [None] * n
    order = sorted(range(n), key=lambda t: (-costs[t], t))
    for t in order:
        f = costs[t]

        def key(r):
            d = dcomm(t, r) if dcomm else 0
            finish = Fraction(load[r] + f, s[r % 8])
            if float(load[r] + f) * speed_sum <= budget * float(s[r % 8]):
                return (0, d, finish, r)
            return (1, finish, d, r)

        r = min(range(n_workers), key=key)
        sigma[t] = r
        load[r] += f
        if commit:
            commit(t, r)
    return sigma, order


def round_robin(n_units: int, n_workers: int):
    return [i % n_workers for i in range(n_units)], list(range(n_units))


class L2Residency:
    """Eq. 9's KV term on one GPU: the groups each XCD (worker r mod 8) has committed to."""

    def __init__(self, unit_groups, volume, n_xcd=8):
        self.groups = unit_groups          # per unit: set of group ids
        self.volume = volume               # group id -> volume (tokens)
        self.n_xcd = n_xcd
        self.held = [set() for _ in range(n_xcd)]

    def dcomm(self, t, r):
        held = self.held[r % self.n_xcd]
        return sum(self.volume[g] for g in self.groups[t] if g not in held)

    def commit(self, t, r):
        self.held[r % self.n_xcd] |= self.groups[t]


def queue(costs, n_workers, tau=0.03, mode="lpt", speed=None, residency=None):
    """Per-worker queues as CSR: (offsets[n_workers + 1], unit ids, per-worker load).  Mode
    "l2" needs ``residency`` (an L2Residency over the same units)."""
    if mode == "lpt":
        sigma, order = place(costs, n_workers, tau, speed=speed)
    elif mode == "l2":
        sigma, order = place(costs, n_workers, tau, dcomm=residency.dcomm, speed=speed,
                             commit=residency.commit)
    else:
        sigma, order = round_robin(len(costs), n_workers)
    per = [[] for _ in range(n_workers)]
    for t in order:
        per[sigma[t]].append(t)
    offsets = [0]
    ids = []
    for r in range(n_workers):
        ids += per[r]
        offsets.append(len(ids))
    load = [sum(costs[t] for t in per[r]) for r in range(n_workers)]
    return offsets, ids, load


def group_key(cu, it, last_key=False):
    """Zigzag group of an item: (sample, KV head, first head), the sample being that of its
    first row (forward, dQ items) or of its last key (dK/dV items)."""
    r = it["row0"] + (it["nrows"] - 1 if last_key else 0)
    j = next(j for j, (s, e) in enumerate(_ranges(cu)) if s <= r < e)
    return (j, it["kv_head"], it["head0"])


def kv_groups(cu, it, h_kv):
    """KV groups of an item (eq. 7): (sample, KV head) of every non-empty sample its rows meet,
    as ids j * h_kv + kappa."""
    lo, hi = it["row0"], it["row0"] + it["nrows"]
    return {j * h_kv + it["kv_head"] for j, (s, e) in enumerate(_ranges(cu)) if s < hi and e > lo and e > s}


def group_volumes(cu, h_kv):
    return {j * h_kv + kappa: e - s for j, (s, e) in enumerate(_ranges(cu)) for kappa in range(h_kv)}


def zigzag_units(cu, items, last_key=False) -> list:
    """Zigzag units of ``items`` (in id order): [(first id, second id or None)], numbered by the
    first item's id."""
    groups = {}
    for it in items:
        groups.setdefault(group_key(cu, it, last_key), []).append(it)
    partner = {}
    for its in groups.values():
        its = sorted(its, key=lambda it: it["row0"])
        n = len(its)
        for i in range((n + 1) // 2):
            a, b = its[i], its[n - 1 - i]
            partner[a["id"]] = None if a is b else b["id"]
    return [(a, partner[a]) for a in sorted(partner)]


def finish_max_over_mean(load, n_workers, speed=None):
    """Largest finish time load / speed over the mean one (float64, summed in worker order)."""
    s, _ = _speeds(speed)
    mx = sm = 0.0
    for r in range(n_workers):
        f = float(load[r]) / float(s[r % 8])
        mx = max(mx, f)
        sm += f
    return mx * n_workers / sm if sm > 0 else 1.0


def zigzag_queue(cu, items, n_workers, tau=0.03, mode="lpt", last_key=False, speed=None, h_kv=None):
    """Per-worker queues as CSR: (offsets, item ids, item flags, per-worker load).  Units are
    placed like any other units; each expands into its first item (default walk), then its
    second (flag REVERSE).  If least-finish placement of the pairs leaves the largest finish time
    more than 0.5 % above the mean one, the single items are placed instead, none reversed.
    Mode "l2" (Algorithm 2 with the L2 residency term) needs h_kv."""
    units = zigzag_units(cu, items, last_key)
    costs = [items[a]["cost"] + (items[b]["cost"] if b is not None else 0) for a, b in units]
    trial = "rr" if mode == "rr" else "lpt"
    _, _, trial_load = queue(costs, n_workers, tau, trial, speed)
    if finish_max_over_mean(trial_load, n_workers, speed) > 1.005:     # pairs too coarse: single items
        units = [(it["id"], None) for it in items]
        costs = [it["cost"] for it in items]
    residency = None
    if mode == "l2":
        groups = [kv_groups(cu, items[a], h_kv) | (kv_groups(cu, items[b], h_kv) if b is not None else set())
                  for a, b in units]
        residency = L2Residency(groups, group_volumes(cu, h_kv))
    u_off, u_ids, load = queue(costs, n_workers, tau, mode, speed, residency)
    offsets, ids, flags = [0], [], []
    for r in range(n_workers):
        for u in u_ids[u_off[r]:u_off[r + 1]]:
            a, b = units[u]
            ids.append(a)
            flags.append(0)
            if b is not None:
                ids.append(b)
                flags.append(REVERSE)
        offsets.append(len(ids))
    return offsets, ids, flags, load
