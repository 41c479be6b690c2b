"""The backward phase entry points reproduce the one-call entry point bit for bit,
and the per-CU records account for every work item (needs an MI355X)."""
import math

import numpy as np
import pytest

import synth
from tests import _support as S

pytestmark = pytest.mark.gpu


def test_phases_match_one_call_entry_points():
    import torch
    import packed_varlen_attention_cu_amd as lib
    w = synth.WORKLOADS["train_256k"].with_tokens(5000)
    cu = synth.cu_seqlens(synth.make_lengths(w, 2))
    t = synth.make_tensors(w, 2, names=("q", "k", "v", "dout"))
    q, k, v, do = (S.to_dev(t[n]) for n in ("q", "k", "v", "dout"))
    plan = S.make_plan(w, cu)
    scale = 1.0 / math.sqrt(w.head_dim)
    S.say("[phases] one-call forward/backward")
    o1, l1 = lib.attn_fwd(plan, q, k, v, scale)
    g1 = lib.attn_bwd(plan, q, k, v, o1, l1, do, scale)
    torch.cuda.synchronize()

    S.say("[phases] phase entry points")
    dev = q.device
    plan_dev, cu_dev = plan.device(dev)
    sh = torch.cuda.current_stream(dev).cuda_stream
    ncu = plan.info.num_cus
    bws = lib.libra_attn_bwd_workspace(plan.host)
    wb = torch.empty(bws, dtype=torch.uint8, device=dev)
    rec = torch.zeros(3 * ncu * 32, dtype=torch.uint8, device=dev)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lib.libra_attn_fwd(plan.host, plan_dev, q, k, v, cu_dev, o2, l2, scale, rec[:ncu * 32], sh)
    lib.libra_attn_bwd_prepare(plan.host, o2, do, l2, wb, bws, sh)
    lib.libra_attn_bwd_dkdv(plan.host, plan_dev, q, k, v, do, l2, cu_dev, dk, dv, scale, wb, bws,
                            rec[ncu * 32:2 * ncu * 32], sh)
    lib.libra_attn_bwd_dq(plan.host, plan_dev, q, k, v, do, l2, cu_dev, dq, scale, wb, bws,
                          rec[2 * ncu * 32:], sh)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, (dq, dk, dv)):
        assert torch.equal(a, b)
    r = rec.cpu().numpy().view(lib.RECORD_DTYPE).reshape(3, ncu)
    assert int(r[0]["n_items"].sum()) == plan.info.n_items
    assert int(r[1]["n_items"].sum()) == plan.info.n_kv_items
    assert int(r[2]["n_items"].sum()) == plan.info.n_dq_items
    assert (r["t_end"] >= r["t_start"]).all()
