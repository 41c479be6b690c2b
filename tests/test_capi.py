"""C-ABI tests that need no GPU: exports, planner parity with the oracle, host validation.

The library is loaded on the CPU machine (the HIP runtime loads without a device);
every call here returns before anything would be enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import packed_varlen_attention_cu_amd as lib
from oracle import plan as P
import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "libra.h")
FAKE = 0x100000           # a well-aligned address that is never dereferenced on the host


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:libra_status|const char \*|size_t)\s*\*?\s*(libra_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    handle = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n


def test_counting_build_exports_its_header_and_the_library():
    """liblibra_debug.so: every libra.h entry point plus the libra_debug.h counter functions; the
    regular library has no counter."""
    dbg_header = os.path.join(os.path.dirname(HEADER), "libra_debug.h")
    extra = sorted(set(re.findall(r"^\s*libra_status\s+(libra_\w+)\s*\(", open(dbg_header).read(), re.M)))
    assert extra == ["libra_debug_reset_unmasked_pairs", "libra_debug_unmasked_pairs"]
    handle = ctypes.CDLL(os.path.join(os.path.dirname(lib.LIB_PATH), "liblibra_debug.so"))
    for n in declared_functions() + extra:
        assert hasattr(handle, n), n
    regular = ctypes.CDLL(lib.LIB_PATH)
    assert not any(hasattr(regular, n) for n in extra)


def make_plan(lens, h_q, h_kv, d, B, W, **kw):
    cu = synth.cu_seqlens(lens)
    return lib.Plan(cu, total_tokens=int(sum(lens)), h_q=h_q, h_kv=h_kv, head_dim=d, tile_tokens=B,
                    tile_heads=W, **kw), cu


CASES = [
    ([1024, 512, 256, 256], 4, 4, 64, 256, 2, {}),
    ([1024, 512, 256, 256], 4, 4, 64, 384, 1, {"num_cus": 16}),
    ([5, 0, 3, 9, 0], 4, 2, 128, 6, 2, {"num_cus": 3}),
    (list(synth.make_lengths(synth.WORKLOADS["gqa_32k"].with_tokens(9000), 0)), 32, 8, 128, 4096, 8, {}),
    (list(synth.make_lengths(synth.WORKLOADS["train_256k"].with_tokens(7000), 1)), 32, 4, 128, 1000, 4,
     {"num_cus": 64, "item_overhead": 4096}),
    (list(synth.make_lengths(synth.WORKLOADS["share_1m"].with_tokens(6000, (4000,)), 2)), 8, 1, 128, 512, 2,
     {"num_cus": 32}),
    ([7, 300, 1, 1, 250], 12, 4, 64, 100, 6, {"num_cus": 9}),
    ([400, 600], 8, 2, 128, 128, 8, {"assign": 1, "num_cus": 7}),
    # workers of unequal speed (eight classes, worker mod 8)
    (list(synth.make_lengths(synth.WORKLOADS["train_256k"].with_tokens(7000), 1)), 32, 4, 128, 1000, 4,
     {"num_cus": 24, "worker_speed": [1000, 940, 1010, 950, 1060, 1000, 990, 940]}),
    ([1024, 512, 256, 256], 4, 4, 64, 256, 2, {"num_cus": 13, "worker_speed": [500, 2000, 0, 1000, 1500, 800, 0, 700]}),
    # eq. 8 pairs as the forward / dQ item cost
    (list(synth.make_lengths(synth.WORKLOADS["gqa_32k"].with_tokens(9000), 1)), 32, 8, 128, 4096, 8,
     {"num_cus": 40, "cost": 1}),
    # Algorithm 2 with the L2 residency term (per-XCD committed KV groups)
    (list(synth.make_lengths(synth.WORKLOADS["gqa_32k"].with_tokens(9000), 0)), 32, 8, 128, 4096, 8,
     {"assign": 2}),
    (list(synth.make_lengths(synth.WORKLOADS["train_256k"].with_tokens(7000), 1)), 32, 4, 128, 1000, 4,
     {"assign": 2, "num_cus": 24, "worker_speed": [1000, 940, 1010, 950, 1060, 1000, 990, 940]}),
    ([7, 300, 1, 0, 1, 250, 900], 12, 4, 64, 100, 6, {"assign": 2, "num_cus": 19, "tau": 0.0}),
    (list(synth.make_lengths(synth.WORKLOADS["share_1m"].with_tokens(6000, (4000,)), 2)), 8, 1, 128, 512, 2,
     {"num_cus": 32, "assign": 2}),
]


@pytest.mark.parametrize("lens,h_q,h_kv,d,B,W,kw", CASES)
def test_planner_matches_oracle(lens, h_q, h_kv, d, B, W, kw):
    plan, cu = make_plan(lens, h_q, h_kv, d, B, W, **kw)
    L = int(sum(lens))
    info = plan.info
    ncu = kw.get("num_cus", 0) or 256
    assert info.num_cus == ncu
    # tiles (eq. 6-8)
    ref_tiles = P.sh_tiles(cu, L, h_q, B, W)
    got = plan.tiles
    assert len(got) == len(ref_tiles)
    for g_, r in zip(got, ref_tiles):
        for f in ("tile_id", "block", "shard", "tok_begin", "tok_end", "head_begin", "head_count",
                  "sample_first", "sample_last", "pairs"):
            assert int(g_[f]) == r[f], f
    assert info.total_pairs == sum(t["pairs"] for t in ref_tiles)
    # forward items and their placement
    mode = {0: "lpt", 1: "rr", 2: "l2"}[kw.get("assign", 0)]
    cost = {0: "executed", 1: "pairs"}[kw.get("cost", 0)]
    tau = kw.get("tau", 0.03)
    ov = kw.get("item_overhead", 0)
    items = P.fwd_items(cu, L, h_q, h_kv, B, W, overhead=ov, cost=cost)
    sp = kw.get("worker_speed")
    offsets, ids, flags, load = P.zigzag_queue(cu, items, ncu, tau, mode, speed=sp, h_kv=h_kv)
    assert list(plan.cu_off) == offsets
    got_items = plan.items
    assert [int(x) for x in got_items["id"]] == ids
    assert [int(x) for x in got_items["flags"]] == flags
    for g_, i in zip(got_items, ids):
        r = items[i]
        for f in ("row0", "nrows", "kv_head", "head0", "nheads", "tile_id", "cost", "pairs"):
            assert int(g_[f]) == r[f], f
    assert info.load_max == max(load) and info.load_sum == sum(load)
    assert [int(t["n_items"]) for t in got] == [sum(1 for it in items if it["tile_id"] == t["tile_id"])
                                               for t in ref_tiles]
    # dQ items (the same tiles, cut for the dQ kernel) and their placement
    dq = P.fwd_items(cu, L, h_q, h_kv, B, W, overhead=ov, columns=P.DQ_ITEM_COLUMNS, cost=cost)
    offsets, ids, flags, load = P.zigzag_queue(cu, dq, ncu, tau, mode, speed=sp, h_kv=h_kv)
    assert list(plan.dq_cu_off) == offsets
    got_dq = plan.dq_items
    assert [int(x) for x in got_dq["id"]] == ids
    assert [int(x) for x in got_dq["flags"]] == flags
    for g_, i in zip(got_dq, ids):
        r = dq[i]
        for f in ("row0", "nrows", "kv_head", "head0", "nheads", "tile_id", "cost", "pairs"):
            assert int(g_[f]) == r[f], f
    assert info.dq_load_max == max(load) and info.dq_load_sum == sum(load)
    # key-major dK/dV items and their placement
    kv = P.kv_items(cu, L, h_q, h_kv, overhead=ov)
    offsets, ids, flags, load = P.zigzag_queue(cu, kv, ncu, tau, mode, last_key=True, speed=sp, h_kv=h_kv)
    assert list(plan.kv_cu_off) == offsets
    got_kv = plan.kv_items
    assert [int(x) for x in got_kv["id"]] == ids
    assert [int(x) for x in got_kv["flags"]] == flags
    for g_, i in zip(got_kv, ids):
        r = kv[i]
        for f in ("row0", "nrows", "kv_head", "head0", "nheads", "tile_id", "cost", "pairs"):
            assert int(g_[f]) == r[f], f
    assert info.kv_load_max == max(load) and info.kv_load_sum == sum(load)


def test_plan_is_bitwise_deterministic():
    lens = list(synth.make_lengths(synth.WORKLOADS["train_256k"], 0))
    a, _ = make_plan(lens, 32, 4, 128, 8192, 4)
    b, _ = make_plan(lens, 32, 4, 128, 8192, 4)
    assert np.array_equal(a.host, b.host)


@pytest.mark.parametrize("name", ["gqa_32k", "skew_128k_a", "skew_128k_b", "share_1m", "train_256k"])
def test_full_size_plans_match_closed_form_and_balance(name):
    w = synth.WORKLOADS[name]
    lens = synth.make_lengths(w, 0)
    pairs = w.h_q * int((lens * (lens + 1) // 2).sum())
    by_pairs, cu = make_plan(list(lens), w.h_q, w.h_kv, w.head_dim, w.tile_tokens, w.tile_heads,
                             cost=lib.COST_PAIRS)
    assert by_pairs.info.total_pairs == pairs
    assert by_pairs.info.load_sum == pairs                   # no overhead: cost == pairs
    plan, _ = make_plan(list(lens), w.h_q, w.h_kv, w.head_dim, w.tile_tokens, w.tile_heads)
    assert plan.info.total_pairs == pairs
    assert plan.info.load_sum >= pairs                        # executed slots cover every pair
    # the dK/dV queue of the 32K pack has only 1368 items for 256 workers: 1.011
    for mx, sm, bound in ((plan.info.load_max, plan.info.load_sum, 1.01),
                          (plan.info.dq_load_max, plan.info.dq_load_sum, 1.01),
                          (plan.info.kv_load_max, plan.info.kv_load_sum, 1.02)):
        assert mx / (sm / 256) < bound, name
    l2, _ = make_plan(list(lens), w.h_q, w.h_kv, w.head_dim, w.tile_tokens, w.tile_heads,
                      assign=lib.ASSIGN_PLACER_L2)
    assert l2.info.load_sum == plan.info.load_sum
    assert l2.info.load_max / (l2.info.load_sum / 256) <= 1.03 + 1e-9 or \
        l2.info.load_max <= plan.info.load_max, name         # within the soft target, or no worse


def test_plan_check_rejects_corruption():
    plan, _ = make_plan([100, 200], 4, 2, 128, 64, 2)
    lib.libra_plan_check(plan.host)
    bad = plan.host.copy()
    bad[plan.info.off_items + 5] ^= 0x40
    with pytest.raises(lib.LibraError) as e:
        lib.libra_plan_check(bad)
    assert e.value.status == lib.LIBRA_EINVAL
    with pytest.raises(lib.LibraError):
        lib.libra_plan_check(plan.host[:-8].copy())


def _params(**over):
    p = dict(total_tokens=10, num_samples=2, h_q=4, h_kv=2, head_dim=128, tile_tokens=4, tile_heads=2,
             num_cus=0, tau=0.03, assign=0, item_overhead=0,
             worker_speed=(ctypes.c_uint16 * 8)(*([0] * 8)), cost=0, reserved=0)
    p.update(over)
    return lib.PlanParams(*[p[f] for f, _ in lib.PlanParams._fields_])


def _plan_status(cu, params, capacity=None):
    cu = np.asarray(cu, dtype=np.int32)
    need = ctypes.c_size_t(0)
    st = lib._lib.libra_plan(cu.ctypes.data, ctypes.byref(params), None, ctypes.byref(need))
    if st != 0 or capacity is None:
        return st, need.value
    buf = np.zeros(capacity // 8 + 1, dtype=np.uint64)
    cap = ctypes.c_size_t(capacity)
    st = lib._lib.libra_plan(cu.ctypes.data, ctypes.byref(params), buf.ctypes.data, ctypes.byref(cap))
    return st, cap.value


@pytest.mark.parametrize("cu,over,status", [
    ([1, 4, 10], {}, lib.LIBRA_EINVAL),                       # cu[0] != 0
    ([0, 6, 4], {}, lib.LIBRA_EINVAL),                        # decreasing
    ([0, 4, 9], {}, lib.LIBRA_EINVAL),                        # cu[n] != L
    ([0, 4, 10], {"h_q": 5}, lib.LIBRA_EINVAL),               # h_q % h_kv
    ([0, 4, 10], {"tile_heads": 3}, lib.LIBRA_EINVAL),        # W does not divide h_q
    ([0, 4, 10], {"tile_tokens": 0}, lib.LIBRA_EINVAL),
    ([0, 4, 10], {"num_cus": -1}, lib.LIBRA_EINVAL),
    ([0, 4, 10], {"assign": 7}, lib.LIBRA_EINVAL),
    ([0, 4, 10], {"cost": 2}, lib.LIBRA_EINVAL),
    ([0, 4, 10], {"reserved": 1}, lib.LIBRA_EINVAL),
    ([0, 4, 10], {"assign": 2}, lib.LIBRA_OK),
    ([0, 4, 10], {"tau": float("nan")}, lib.LIBRA_EINVAL),
    ([0, 4, 10], {"item_overhead": -1}, lib.LIBRA_EINVAL),
    ([0, 4, 10], {"head_dim": 96}, lib.LIBRA_EUNSUPPORTED),
    ([0, 4, 10], {}, lib.LIBRA_OK),
])
def test_plan_errors(cu, over, status):
    assert _plan_status(cu, _params(**over))[0] == status


def test_plan_reports_size_when_buffer_too_small():
    st, need = _plan_status([0, 4, 10], _params())
    assert st == 0 and need > 0
    st, got = _plan_status([0, 4, 10], _params(), capacity=need - 8)
    assert st == lib.LIBRA_ESIZE and got == need


def test_empty_pack_plans_and_runs_nothing():
    plan = lib.Plan(np.array([0], dtype=np.int32), total_tokens=0, h_q=4, h_kv=2, head_dim=128,
                    tile_tokens=64, tile_heads=2)
    assert plan.info.n_tiles == 0 and plan.info.n_items == 0 and plan.info.n_dq_items == 0
    assert plan.info.n_kv_items == 0
    # L = 0: every entry point returns OK before touching any pointer or the device
    lib.libra_attn_fwd(plan.host, None, None, None, None, None, None, None, 0.1, None, None)
    lib.libra_attn_bwd(plan.host, None, None, None, None, None, None, None, None, None, None, None, 0.1,
                       None, 0, None, None)


# ------------------------------------------------------------- forward / backward validation
@pytest.fixture(scope="module")
def small_plan():
    plan, cu = make_plan([100, 28], 4, 2, 128, 64, 2)
    return plan


def fwd_args(plan, **over):
    a = dict(plan_host=plan.host, plan_dev=FAKE, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, o=FAKE, lse=FAKE,
             scale=0.1, rec=None, stream=None)
    a.update(over)
    return a


def call_fwd(a):
    return lib._lib.libra_attn_fwd(a["plan_host"].ctypes.data, a["plan_dev"], a["q"], a["k"], a["v"], a["cu"],
                                   a["o"], a["lse"], a["scale"], a["rec"], a["stream"])


@pytest.mark.parametrize("over,status", [
    ({"q": None}, lib.LIBRA_EINVAL), ({"k": None}, lib.LIBRA_EINVAL), ({"v": None}, lib.LIBRA_EINVAL),
    ({"o": None}, lib.LIBRA_EINVAL), ({"lse": None}, lib.LIBRA_EINVAL), ({"cu": None}, lib.LIBRA_EINVAL),
    ({"plan_dev": None}, lib.LIBRA_EINVAL), ({"v": FAKE + 8}, lib.LIBRA_EINVAL),
    ({"q": FAKE + 8}, lib.LIBRA_EINVAL), ({"rec": FAKE + 4}, lib.LIBRA_EINVAL),
    ({"lse": FAKE + 2}, lib.LIBRA_EINVAL),
    ({"scale": 0.0}, lib.LIBRA_EINVAL), ({"scale": float("nan")}, lib.LIBRA_EINVAL),
    ({"scale": -1.0}, lib.LIBRA_EINVAL),
])
def test_fwd_validation(small_plan, over, status):
    assert call_fwd(fwd_args(small_plan, **over)) == status


def test_fwd_rejects_foreign_plan(small_plan):
    bad = small_plan.host.copy()
    bad[0] ^= 1
    assert call_fwd(fwd_args(small_plan, plan_host=bad)) == lib.LIBRA_EINVAL


@pytest.mark.parametrize("where", ["items", "dq", "kv", "cu_off", "header"])
def test_launches_reject_a_plan_whose_checksum_fails(small_plan, where):
    """Every launch entry point verifies the host plan's checksum before enqueuing anything."""
    info = small_plan.info
    off = {"items": info.off_items + 3, "dq": info.off_dq_items + 17, "kv": info.off_kv_items + 40,
           "cu_off": info.off_cu_off + 4, "header": 40}[where]        # 40: inside params (h_kv)
    bad = small_plan.host.copy()
    bad[off] ^= 0x10
    assert call_fwd(fwd_args(small_plan, plan_host=bad)) == lib.LIBRA_EINVAL
    h = bad.ctypes.data
    bws = 1 << 20
    assert lib._lib.libra_attn_bwd_dkdv(h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        ctypes.c_float(0.1), FAKE, bws, None, None) == lib.LIBRA_EINVAL
    assert lib._lib.libra_attn_bwd_dq(h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1),
                                      FAKE, bws, None, None) == lib.LIBRA_EINVAL
    assert lib._lib.libra_attn_bwd_prepare(h, FAKE, FAKE, FAKE, FAKE, bws, None) == lib.LIBRA_EINVAL
    assert lib._lib.libra_attn_bwd(h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   ctypes.c_float(0.1), FAKE, bws, None, None) == lib.LIBRA_EINVAL


def test_binding_constants_match_the_header():
    text = open(HEADER).read()

    def define(name):
        return int(re.search(rf"#define {name} (0x[0-9A-Fa-f]+|\d+)u?", text).group(1), 0)

    def enum(name):
        return int(re.search(rf"\b{name} = (-?\d+)", text).group(1))
    assert lib.PLAN_VERSION == define("LIBRA_PLAN_VERSION")
    assert lib.PLAN_MAGIC == define("LIBRA_PLAN_MAGIC")
    assert lib.RECORD_PLAN_MISMATCH == define("LIBRA_RECORD_PLAN_MISMATCH")
    assert lib.RECORD_WAIT_EXPIRED == define("LIBRA_RECORD_WAIT_EXPIRED")
    for name in ("LIBRA_EINVAL", "LIBRA_ESIZE", "LIBRA_EUNSUPPORTED", "LIBRA_EHIP", "LIBRA_EHOST"):
        assert getattr(lib, name) == enum(name), name
    for py, c in (("ASSIGN_PLACER", "LIBRA_ASSIGN_PLACER"), ("ASSIGN_ROUND_ROBIN", "LIBRA_ASSIGN_ROUND_ROBIN"),
                  ("ASSIGN_PLACER_L2", "LIBRA_ASSIGN_PLACER_L2"), ("COST_EXECUTED", "LIBRA_COST_EXECUTED"),
                  ("COST_PAIRS", "LIBRA_COST_PAIRS"), ("QUEUE_KV", "LIBRA_QUEUE_KV")):
        assert getattr(lib, py) == enum(c), c


def test_wrappers_check_tensors_against_the_plan(small_plan):
    """The torch wrappers refuse tensors that do not match the plan before any library call
    (shapes first, then dtype, contiguity and device: CPU tensors of the right shape fail last)."""
    import torch
    L, h_q, h_kv, d = 128, 4, 2, 128
    bf = torch.bfloat16
    q = torch.zeros(L, h_q, d, dtype=bf)
    k = torch.zeros(L, h_kv, d, dtype=bf)
    v = torch.zeros(L, h_kv, d, dtype=bf)
    with pytest.raises(ValueError, match="q: shape"):
        lib.attn_fwd(small_plan, q[:-1], k, v)
    with pytest.raises(ValueError, match="k: shape"):
        lib.attn_fwd(small_plan, q, torch.zeros(L, h_q, d, dtype=bf), v)
    with pytest.raises(ValueError, match="v: dtype"):
        lib.attn_fwd(small_plan, q, k, v.float())
    with pytest.raises(ValueError, match="contiguous"):
        lib.attn_fwd(small_plan, q, k, torch.zeros(L, d, h_kv, dtype=bf).transpose(1, 2))
    with pytest.raises(ValueError, match="lse: shape"):
        lib.attn_fwd(small_plan, q, k, v, lse=torch.zeros(L, h_q))
    with pytest.raises(ValueError, match="on a GPU"):
        lib.attn_fwd(small_plan, q, k, v)
    lse = torch.zeros(h_q, L)
    with pytest.raises(ValueError, match="dout: shape"):
        lib.attn_bwd(small_plan, q, k, v, q, lse, q[:, :2])
    with pytest.raises(ValueError, match="on a GPU"):
        lib.attn_bwd(small_plan, q, k, v, q, lse, q)


def test_phase_entry_points_validate(small_plan):
    h = small_plan.host.ctypes.data
    bws = lib.libra_attn_bwd_workspace(small_plan.host)
    L_ = lib._lib
    assert L_.libra_attn_bwd_prepare(h, None, FAKE, FAKE, FAKE, bws, None) == lib.LIBRA_EINVAL
    assert L_.libra_attn_bwd_prepare(h, FAKE, None, FAKE, FAKE, bws, None) == lib.LIBRA_EINVAL
    assert L_.libra_attn_bwd_prepare(h, FAKE, FAKE, None, FAKE, bws, None) == lib.LIBRA_EINVAL
    assert L_.libra_attn_bwd_prepare(h, FAKE, FAKE, FAKE + 2, FAKE, bws, None) == lib.LIBRA_EINVAL
    assert L_.libra_attn_bwd_prepare(h, FAKE, FAKE, FAKE, FAKE + 16, bws, None) == lib.LIBRA_EINVAL
    assert L_.libra_attn_bwd_prepare(h, FAKE, FAKE, FAKE, FAKE, bws - 1, None) == lib.LIBRA_ESIZE
    dkdv = [h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, bws, None, None]
    for i in (2, 3, 4, 5, 6, 7, 8, 9):           # q k v dout lse cu dk dv
        args = list(dkdv)
        args[i] = None
        assert L_.libra_attn_bwd_dkdv(*args) == lib.LIBRA_EINVAL, i
    dq = [h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, bws, None, None]
    for i in (2, 3, 4, 5, 6, 7, 8):              # q k v dout lse cu dq: v is read by the dQ kernel
        args = list(dq)
        args[i] = None
        assert L_.libra_attn_bwd_dq(*args) == lib.LIBRA_EINVAL, i
    args = list(dq)
    args[9] = ctypes.c_float(float("inf"))
    assert L_.libra_attn_bwd_dq(*args) == lib.LIBRA_EINVAL


def test_bwd_validation(small_plan):
    h = small_plan.host.ctypes.data
    bws = lib.libra_attn_bwd_workspace(small_plan.host)
    full = [h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, bws,
            None, None]
    for i in range(1, 12):
        args = list(full)
        args[i] = None
        assert lib._lib.libra_attn_bwd(*args) == lib.LIBRA_EINVAL, i
    args = list(full)
    args[14] = bws - 1
    assert lib._lib.libra_attn_bwd(*args) == lib.LIBRA_ESIZE


def test_noalloc_backward_validates_and_caps_its_size(small_plan):
    """The backward without allocation takes libra_attn_bwd's checks, and a plan whose workspace
    exceeds the library's 64 MiB array gets LIBRA_ESIZE; both return before the device is touched."""
    h = small_plan.host.ctypes.data
    full = [h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), None, None]
    for i in range(1, 12):
        args = list(full)
        args[i] = None
        assert lib._lib.libra_attn_bwd_noalloc(*args) == lib.LIBRA_EINVAL, i
    args = list(full)
    args[12] = ctypes.c_float(0.0)
    assert lib._lib.libra_attn_bwd_noalloc(*args) == lib.LIBRA_EINVAL
    text = open(HEADER).read()
    assert lib.NOALLOC_SCRATCH_BYTES == int(re.search(r"#define LIBRA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                                                        text).group(1)) << 20
    # 32 heads x 262144 tokens fit exactly (2 x 4 bytes each); one more sample of 64 tokens does not
    for L, status in ((262144, None), (262144 + 64, lib.LIBRA_ESIZE)):
        big = lib.Plan(np.array([0, L], dtype=np.int32), total_tokens=L, h_q=32, h_kv=4, head_dim=128,
                       tile_tokens=8192, tile_heads=32)
        assert lib.libra_attn_bwd_workspace(big.host) <= lib.NOALLOC_SCRATCH_BYTES or status is not None
        if status is not None:
            args = list(full)
            args[0] = big.host.ctypes.data
            assert lib._lib.libra_attn_bwd_noalloc(*args) == status


def test_workspace_sizes(small_plan):
    # D and LSE * log2(e): fp32 [h_q][L] each, 256-byte aligned (L = 128, h_q = 4)
    assert lib.libra_attn_bwd_workspace(small_plan.host) == 2 * 2048


def test_status_strings():
    assert lib.libra_status_str(0) == "ok"
    assert lib.libra_status_str(-2) == "buffer too small"
    assert lib.libra_status_str(123) == "unknown status"
    # every status the header declares has its own text
    text = open(HEADER).read()
    codes = [int(v) for v in re.findall(r"LIBRA_E\w+\s*=\s*(-\d+)", text)]
    assert len(codes) >= 5
    for c in codes:
        assert lib.libra_status_str(c) not in ("unknown status", "ok"), c


def test_last_hip_error_is_empty_without_a_failed_launch():
    import threading
    got = []
    t = threading.Thread(target=lambda: got.append(lib.libra_last_hip_error()))
    t.start()
    t.join()
    assert got == [""]


def test_library_shares_torchs_hip_runtime():
    """Exactly one HIP runtime is mapped once the package is imported."""
    maps = open(f"/proc/{os.getpid()}/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_worker_speed_recovers_class_rates():
    """Records whose busy ticks are load x 1000 / speed of the worker's class give back those
    speeds, scaled to a mean of 1000 (host function, synthetic records)."""
    lens = list(synth.make_lengths(synth.WORKLOADS["train_256k"].with_tokens(20000), 0))
    plan, cu = make_plan(lens, 32, 4, 128, 4096, 4, num_cus=64)
    speed = np.array([1000, 900, 1100, 950, 1050, 1000, 980, 1020], dtype=np.float64)
    for q, items, off in ((lib.QUEUE_FWD, plan.items, plan.cu_off), (lib.QUEUE_DQ, plan.dq_items, plan.dq_cu_off),
                          (lib.QUEUE_KV, plan.kv_items, plan.kv_cu_off)):
        rec = np.zeros(64, dtype=lib.RECORD_DTYPE)
        for w in range(64):
            load = int(items["cost"][off[w]:off[w + 1]].sum())
            rec["t_start"][w] = 1000
            rec["t_end"][w] = 1000 + int(round(load * 1000 / speed[w % 8] / 1000))
        got = lib.libra_worker_speed(plan.host, q, rec).astype(np.float64)
        expect = 1000 * speed / speed.mean()
        assert np.all(np.abs(got - expect) <= 1.0), (q, got, expect)
    with pytest.raises(lib.LibraError):
        lib.libra_worker_speed(plan.host, 3, np.zeros(64, dtype=lib.RECORD_DTYPE))
