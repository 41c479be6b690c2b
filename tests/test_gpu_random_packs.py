"""Forward and backward parity on seeded random packs (needs an MI355X): GQA shapes with group
sizes 1 to 8 and head dims 64 and 128, packs mixing empty, one-token, block-edge and lognormal
samples, any SH-Tile shape, and every placement mode, worker count, cost model and speed
setting the planner takes.  Every output and gradient is compared with the fp64 oracle.  The
same cases pass the CPU plan checks (C planner equal to the oracle, plan shapes) first, and each
plan's shapes are checked again here before its launch."""
import pytest

import synth
from tests import _random_cases as R
from tests import _support as S

pytestmark = pytest.mark.gpu

N_CASES = 40


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_attention_cu_amd as m
    return m


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_pack_fwd_bwd(lib, case):
    import torch
    import oracle.attention as A
    lens, h_q, h_kv, d, B, W, kw = R.random_case(case)
    L = sum(lens)
    w = synth.Workload(f"random{case}", L, h_q, h_kv, d, B, W, fixed_lengths=tuple(lens), fill=False)
    cu = synth.cu_seqlens(lens)
    S.say(f"[random] case {case}: L={L} samples={len(lens)} h={h_q}/{h_kv} d={d} B={B} W={W} {kw}")
    plan = lib.Plan(cu, total_tokens=L, h_q=h_q, h_kv=h_kv, head_dim=d, tile_tokens=B, tile_heads=W, **kw)
    R.check_plan_shapes(plan, L, h_q, h_kv)
    t = synth.make_tensors(w, case, names=("q", "k", "v", "dout"))
    q, k, v, do = (S.to_dev(t[n]) for n in ("q", "k", "v", "dout"))
    o, lse = lib.attn_fwd(plan, q, k, v, S.scale_of(w))
    dq, dk, dv = lib.attn_bwd(plan, q, k, v, o, lse, do, S.scale_of(w))
    torch.cuda.synchronize()
    args = [A.widen_bf16(t[n]) for n in ("q", "k", "v")]
    o_ref, lse_ref = A.forward(*args, cu, S.scale_of(w))
    S.check_out(S.from_dev_bf16(o), o_ref, f"case {case}")
    S.check_lse(lse.cpu().numpy().astype("float64"), lse_ref, f"case {case}")
    ref = A.backward(*args, A.widen_bf16(t["dout"]), cu, S.scale_of(w))
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        S.check_grad(S.from_dev_bf16(g), r, f"case {case} {name}")
