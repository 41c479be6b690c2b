"""The backward phase entry points reproduce the one-call entry point bit for bit,
and the per-CU records account for every work item (needs an MI355X)."""
import math

import numpy as np
import pytest

import synth
from tests import _support as S


def _has_gpu():
    import torch
    return torch.cuda.is_available()


pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not _has_gpu(), reason="no GPU")]


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
    assert (r["flags"] == 0).all()       # no plan mismatch, no expired wait in the dK/dV pass


def test_device_plan_from_another_plan_runs_nothing():
    """A device plan copied from a different plan (another packing) has another checksum: every
    workgroup of the forward and backward kernels sees the mismatch, runs no item and flags its
    record; the outputs keep what they held.  The kernels read only the checksum field of the
    foreign copy, which any plan buffer holds."""
    import torch
    import packed_varlen_attention_cu_amd as lib
    w = synth.WORKLOADS["train_256k"].with_tokens(3000)
    cu_a = synth.cu_seqlens(synth.make_lengths(w, 0))
    cu_b = synth.cu_seqlens(synth.make_lengths(w, 1))
    plan_a, plan_b = S.make_plan(w, cu_a), S.make_plan(w, cu_b)
    assert plan_a.info.checksum != plan_b.info.checksum
    t = synth.make_tensors(w, 0, names=("q", "k", "v", "dout"))
    q, k, v, do = (S.to_dev(t[n]) for n in ("q", "k", "v", "dout"))
    dev = q.device
    dev_b, cu_dev = plan_b.device(dev)[0], plan_a.device(dev)[1]
    ncu = plan_a.info.num_cus
    rec = torch.zeros(3 * ncu * lib.RECORD_DTYPE.itemsize, dtype=torch.uint8, device=dev)
    o = torch.full_like(q, 7.0)
    lse = torch.full((w.h_q, w.total_tokens), 7.0, dtype=torch.float32, device=dev)
    stream = lib._stream_handle(dev)
    S.say("[guard] forward with a foreign device plan")
    lib.libra_attn_fwd(plan_a.host, dev_b, q, k, v, cu_dev, o, lse, S.scale_of(w), rec[:ncu * 32], stream)
    dq, dk, dv = (torch.full_like(x, 7.0) for x in (q, k, v))
    ws_bytes = lib.libra_attn_bwd_workspace(plan_a.host)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    S.say("[guard] backward with a foreign device plan")
    lib.libra_attn_bwd(plan_a.host, dev_b, q, k, v, o, do, lse, cu_dev, dq, dk, dv, S.scale_of(w), ws, ws_bytes,
                       rec[ncu * 32:], stream)
    torch.cuda.synchronize()
    r = rec.cpu().numpy().view(lib.RECORD_DTYPE)
    assert (r["flags"] == lib.RECORD_PLAN_MISMATCH).all() and (r["n_items"] == 0).all()
    for x in (o, dq, dk, dv):
        assert (x.float() == 7.0).all().item()
    assert (lse == 7.0).all().item()
