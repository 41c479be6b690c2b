"""Element offsets past 2^31 (needs an MI355X; about 45 GB of device memory).

A 1M-token pack with 32 query heads of d = 128 holds 2^32 elements in each of q, o, dout and
dq, so every query-side address in the second half of the pack lies beyond what a 32-bit
element index reaches.  The forward and backward run on the whole pack; rows and complete
(sample, KV head) units in its last half are compared with the fp64 oracle, and every output
must be finite.
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


@pytest.mark.timeout(900)
def test_fwd_bwd_offsets_beyond_int32(lib):
    import torch
    w = synth.WORKLOADS["train_256k"].with_tokens(1 << 20, name="train_1m")
    assert w.total_tokens * w.h_q * w.head_dim == 1 << 32
    cu = synth.cu_seqlens(synth.make_lengths(w, 5))
    lens = np.diff(cu)
    S.say(f"[large] L={w.total_tokens} h={w.h_q}/{w.h_kv} samples={len(lens)} max={int(lens.max())}: inputs")
    t = synth.make_tensors(w, 5, names=("q", "k", "v", "dout"))
    S.say("[large] GPU forward and backward")
    plan = S.make_plan(w, cu)
    q, k, v, do = (S.to_dev(t[n]) for n in ("q", "k", "v", "dout"))
    o, lse = lib.attn_fwd(plan, q, k, v, S.scale_of(w))
    dq, dk, dv = lib.attn_bwd(plan, q, k, v, o, lse, do, S.scale_of(w))
    torch.cuda.synchronize()
    del q, do
    for name, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(x.float() if x.dtype != torch.float32 else x).all().item(), name

    half = w.total_tokens // 2
    rng = np.random.default_rng(3)
    # forward: the pack's last rows, the tails of the last two samples, random rows of the upper half
    rows = set(range(w.total_tokens - 64, w.total_tokens))
    for j in range(len(lens) - 2, len(lens)):
        e = int(cu[j + 1])
        rows.update(range(max(int(cu[j]), e - 96), e))
    rows.update(int(r) for r in rng.integers(half, w.total_tokens, 256))
    rows = np.array(sorted(rows), dtype=np.int64)
    S.say(f"[large] oracle forward on {rows.size} rows")
    rows, o_ref, lse_ref = S.oracle_fwd_rows(t["q"], t["k"], t["v"], cu, S.scale_of(w), rows)
    idx = torch.from_numpy(rows).cuda()
    S.check_out(S.from_dev_bf16(o.index_select(0, idx)), o_ref, "1M x 32 heads")
    S.check_lse(lse.index_select(1, idx).cpu().numpy().astype(np.float64), lse_ref, "1M x 32 heads")

    # backward: complete short samples of the upper half and the last 192 rows of its last long one
    g = w.h_q // w.h_kv
    upper = [j for j in range(len(lens)) if cu[j] >= half and lens[j] > 0]
    short = [j for j in upper if lens[j] <= 1024][-8:]
    longs = [j for j in upper if lens[j] > 1024][-1:]
    units = [(j, int(rng.integers(0, w.h_kv)), 0) for j in short]
    units += [(j, int(rng.integers(0, w.h_kv)), int(lens[j]) - 192) for j in longs]
    S.say(f"[large] oracle backward on {len(units)} units")
    refs = S.oracle_bwd_tails(t["q"], t["k"], t["v"], t["dout"], cu, S.scale_of(w), units)
    got = {n: [] for n in ("dq", "dk", "dv")}
    want = {n: [] for n in ("dq", "dk", "dv")}
    for (j, kv, first), (rq, rk, rv) in zip(units, refs):
        s, e = int(cu[j]) + first, int(cu[j + 1])
        got["dq"].append(S.from_dev_bf16(dq[s:e, kv * g:(kv + 1) * g]).ravel())
        got["dk"].append(S.from_dev_bf16(dk[s:e, kv]).ravel())
        got["dv"].append(S.from_dev_bf16(dv[s:e, kv]).ravel())
        want["dq"].append(rq.ravel())
        want["dk"].append(rk.ravel())
        want["dv"].append(rv.ravel())
    for n in ("dq", "dk", "dv"):
        S.check_grad(np.concatenate(got[n]), np.concatenate(want[n]), f"1M x 32 heads {n}")
