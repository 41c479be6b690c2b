"""The backward entry point that allocates nothing (libra_attn_bwd_noalloc, for callers that
cannot allocate) against the regular backward (libra_attn_bwd with a caller workspace), through
the C ABI on an MI355X: two calls in a row, the second on a smaller pack, must give the regular
entry point's dq, dk and dv bit for bit (the same kernels on the same inputs; only the workspace
differs: a device array inside the library instead of a caller buffer)."""
import ctypes

import numpy as np
import pytest

import synth
from tests import _support as S

pytestmark = pytest.mark.gpu


def _run_both(lib, w, seed):
    import torch
    cu = synth.cu_seqlens(synth.make_lengths(w, seed))
    t = synth.make_tensors(w, seed, names=("q", "k", "v", "dout"))
    plan = S.make_plan(w, cu)
    q, k, v, do = (S.to_dev(t[n]) for n in ("q", "k", "v", "dout"))
    dev = q.device
    plan_dev, cu_dev = plan.device(dev)
    o, lse = lib.attn_fwd(plan, q, k, v, S.scale_of(w))
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    outs = []
    for noalloc in (False, True):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        for x in (dq, dk, dv):
            x.fill_(float("nan"))           # anything left unwritten shows
        if noalloc:
            lib.libra_attn_bwd_noalloc(plan.host, plan_dev, q, k, v, o, do, lse, cu_dev, dq, dk, dv,
                                       S.scale_of(w), None, stream)
        else:
            ws_bytes = lib.libra_attn_bwd_workspace(plan.host)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            lib.libra_attn_bwd(plan.host, plan_dev, q, k, v, o, do, lse, cu_dev, dq, dk, dv, S.scale_of(w),
                               ws, ws_bytes, None, stream)
        torch.cuda.synchronize()
        outs.append([S.bits_of(x) for x in (dq, dk, dv)])
    return outs, t, cu


def test_noalloc_backward_equals_the_regular_one_twice():
    import torch
    import oracle.attention as A
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_attention_cu_amd as lib_
    base = synth.WORKLOADS["train_256k"]
    for L, seed in ((6000, 1), (2100, 2)):          # the second call: a smaller pack
        w = base.with_tokens(L)
        S.say(f"[noalloc] train_256k shape, L={L}, seed {seed}")
        (reg, noa), t, cu = _run_both(lib_, w, seed)
        for name, a, b in zip(("dq", "dk", "dv"), reg, noa):
            assert np.array_equal(a, b), f"{name}: the two entry points differ"
        ref = A.backward(*(A.widen_bf16(t[n]) for n in ("q", "k", "v", "dout")), cu, S.scale_of(w))
        for name, g, r in zip(("dq", "dk", "dv"), noa, ref):
            S.check_grad(synth.bf16_bits_to_f32(g).astype(np.float64), r, f"noalloc {name}")
