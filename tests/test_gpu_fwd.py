"""Forward parity of the HIP path against the fp64 oracle (needs an MI355X).

Small packs are compared element by element over every output; the full-size
workloads are compared on sampled rows (sample edges, tile boundaries, random
rows) plus whole-tensor properties (every output written and finite).
"""
import numpy as np
import pytest

import synth
from tests import _support as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_attention_cu_amd as m
    return m


def run_fwd(lib, w, cu, t, **plan_kw):
    import torch
    plan = S.make_plan(w, cu, **plan_kw)
    q, k, v = S.to_dev(t["q"]), S.to_dev(t["k"]), S.to_dev(t["v"])
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.h_q, w.total_tokens), float("nan"), dtype=torch.float32, device=q.device)
    lib.attn_fwd(plan, q, k, v, S.scale_of(w), out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse, plan


def full_check(lib, w, cu, t, what, **plan_kw):
    import oracle.attention as A
    S.say(f"[fwd] {what}: L={w.total_tokens} h={w.h_q}/{w.h_kv} d={w.head_dim} samples={len(cu) - 1} {plan_kw}")
    o, lse, _ = run_fwd(lib, w, cu, t, **plan_kw)
    o_ref, lse_ref = A.forward(A.widen_bf16(t["q"]), A.widen_bf16(t["k"]), A.widen_bf16(t["v"]), cu,
                               S.scale_of(w))
    S.check_out(S.from_dev_bf16(o), o_ref, what)
    S.check_lse(lse.cpu().numpy().astype(np.float64), lse_ref, what)
    return o, lse


SMALL = [
    ("tiny_2k", None, None, {}),
    ("gqa_32k", 3001, None, {}),
    ("gqa_32k", 3001, None, {"tile_tokens": 1000, "tile_heads": 2}),
    ("skew_128k_a", 5000, (2500,), {}),
    ("share_1m", 6000, (4000,), {}),
    ("share_1m", 6000, (4000,), {"tile_tokens": 333, "tile_heads": 8}),
    ("train_256k", 4100, None, {}),
    ("train_256k", 4100, None, {"assign": 1, "num_cus": 7}),
]


@pytest.mark.parametrize("name,L,first,kw", SMALL)
def test_fwd_small_full(lib, name, L, first, kw):
    base = synth.WORKLOADS[name]
    w = base if L is None else base.with_tokens(L, first_lengths=first)
    cu = synth.cu_seqlens(synth.make_lengths(w, 0))
    t = synth.make_tensors(w, 0)
    full_check(lib, w, cu, t, name, **kw)


@pytest.mark.parametrize("lens", [
    [1] * 300,                       # every token starts a sample
    [0, 5, 0, 0, 130, 1, 0, 64],     # empty samples between real ones
    [1],                             # one token
    [64],                            # exactly one key block
    [63, 65, 1, 127, 2],             # ragged around block edges
    [0, 0, 33, 1, 0, 0],             # empty samples first and last
])
def test_fwd_edge_packs(lib, lens):
    L = sum(lens)
    w = synth.Workload("edge", L, 4, 2, 128, 100, 2, fixed_lengths=tuple(lens), fill=False)
    cu = synth.cu_seqlens(lens)
    t = synth.make_tensors(w, 3)
    full_check(lib, w, cu, t, f"edge{lens[:6]}")


def test_fwd_first_token_and_identical_v_bit_exact(lib):
    """Row 0 of a sample sees only itself: O = V exactly.  Equal V rows pass through exactly."""
    lens = [1, 7, 300, 2, 900, 33]
    L = sum(lens)
    w = synth.Workload("exact", L, 8, 2, 128, 256, 4, fixed_lengths=tuple(lens), fill=False)
    cu = synth.cu_seqlens(lens)
    t = synth.make_tensors(w, 5)
    v = t["v"].copy()
    for j in range(len(lens)):     # samples 3..5 get one V row repeated
        if j >= 3:
            v[cu[j]:cu[j + 1]] = v[cu[j]]
    t["v"] = v
    o, lse, _ = run_fwd(lib, w, cu, t)
    ob = S.bits_of(o)
    g = w.h_q // w.h_kv
    for j in range(len(lens)):
        s = cu[j]
        for h in range(w.h_q):
            assert np.array_equal(ob[s, h], v[s, h // g]), (j, h)
            if j >= 3:
                assert np.array_equal(ob[cu[j]:cu[j + 1], h], np.broadcast_to(v[s, h // g], (lens[j], 128))), (j, h)


def test_fwd_plan_reuse_and_tilings_agree(lib):
    """One plan serves several calls; different SH-Tile shapes give the same result within tolerance."""
    w = synth.WORKLOADS["gqa_32k"].with_tokens(2500)
    cu = synth.cu_seqlens(synth.make_lengths(w, 1))
    t = synth.make_tensors(w, 1)
    outs = []
    for kw in ({}, {"tile_tokens": 128, "tile_heads": 1}, {"tile_tokens": 2500, "tile_heads": 32}):
        o1, l1, plan = run_fwd(lib, w, cu, t, **kw)
        outs.append(S.from_dev_bf16(o1))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 2 * S.O_MAX


def test_fwd_pool_equals_separate_launches(lib):
    """Two packs pooled into one plan and one launch (the rows of the second follow the first):
    the pool matches the oracle, and each pack's rows match its own launch within tolerance,
    since the block-diagonal mask keeps the packs apart."""
    base = synth.WORKLOADS["skew_128k_a"]
    wa = base.with_tokens(3000, first_lengths=(1500,))
    wb = base.with_tokens(2001, first_lengths=())
    la, lb = synth.make_lengths(wa, 2), synth.make_lengths(wb, 3)
    ta, tb = synth.make_tensors(wa, 2), synth.make_tensors(wb, 3)
    oa, lsa, _ = run_fwd(lib, wa, synth.cu_seqlens(la), ta)
    ob, lsb, _ = run_fwd(lib, wb, synth.cu_seqlens(lb), tb)
    wp = base.with_tokens(wa.total_tokens + wb.total_tokens, first_lengths=(), name="pool")
    cup = synth.cu_seqlens(np.concatenate([la, lb]))
    tp = {n: np.concatenate([ta[n], tb[n]]) for n in ("q", "k", "v")}
    op, lsp = full_check(lib, wp, cup, tp, "pool of two packs")
    op, lsp = S.from_dev_bf16(op), lsp.cpu().numpy()
    sep = np.concatenate([S.from_dev_bf16(oa), S.from_dev_bf16(ob)])
    assert np.max(np.abs(op - sep)) <= 2 * S.O_MAX
    assert np.max(np.abs(lsp - np.concatenate([lsa.cpu().numpy(), lsb.cpu().numpy()], axis=1))) <= 2 * S.LSE_MAX


@pytest.mark.parametrize("kind", ["x4", "x8", "rising", "falling"])
def test_fwd_extreme_logits(lib, kind):
    """Logits far outside the N(0, 1) range: large jumps of the running maximum (x4, x8), a
    rescale at every key block (rising), weights that underflow behind an early maximum
    (falling).  Both head sizes."""
    lens = [700, 1, 500, 64, 235]
    for d in (128, 64):
        w = synth.Workload(f"logits-{kind}", sum(lens), 8, 2, d, 512, 4, fixed_lengths=tuple(lens), fill=False)
        cu = synth.cu_seqlens(lens)
        t = S.extreme_logit_inputs(w, cu, kind, 6)
        full_check(lib, w, cu, t, f"{kind} d={d}")


@pytest.mark.parametrize("h_q,h_kv,d,tile_heads", [(12, 4, 128, 3), (6, 6, 64, 2), (16, 1, 128, 8),
                                                    (32, 16, 64, 32)])
def test_fwd_gqa_group_shapes(lib, h_q, h_kv, d, tile_heads):
    """Group sizes 3, 1, 16 and 2, head counts that are not powers of two, both head sizes."""
    w = synth.Workload(f"g{h_q}x{h_kv}", 2300, h_q, h_kv, d, 700, tile_heads, first_lengths=(900,))
    cu = synth.cu_seqlens(synth.make_lengths(w, 4))
    t = synth.make_tensors(w, 4)
    full_check(lib, w, cu, t, w.name)


FULL = [("gqa_32k", 96, 1), ("skew_128k_a", 64, 2), ("skew_128k_b", 64, 2), ("train_256k", 64, 4),
        ("share_1m", 12, 16)]


@pytest.mark.parametrize("name,n_random,stride", FULL)
def test_fwd_full_size_sampled(lib, name, n_random, stride):
    import torch
    w = synth.WORKLOADS[name]
    cu = synth.cu_seqlens(synth.make_lengths(w, 0))
    S.say(f"[fwd-full] {name}: generating inputs")
    t = synth.make_tensors(w, 0)
    S.say(f"[fwd-full] {name}: GPU run L={w.total_tokens}")
    o, lse, plan = run_fwd(lib, w, cu, t)
    assert not torch.isnan(o).any().item(), "some output element was never written"
    assert torch.isfinite(lse).all().item()
    rows = S.sample_rows(cu, w.tile_tokens, n_random, seed=7, boundary_stride=stride)
    S.say(f"[fwd-full] {name}: oracle on {rows.size} rows")
    rows, o_ref, lse_ref = S.oracle_fwd_rows(t["q"], t["k"], t["v"], cu, S.scale_of(w), rows)
    idx = torch.from_numpy(rows).cuda()
    S.check_out(S.from_dev_bf16(o.index_select(0, idx)), o_ref, name)
    S.check_lse(lse.index_select(1, idx).cpu().numpy().astype(np.float64), lse_ref, name)
