"""Eq. 8's pair count inside the forward kernel (needs an MI355X).

The counting build of the library (liblibra_debug.so, include/libra_debug.h) has the forward
kernel count the (query, key, head) triples it leaves unmasked.  Eq. 8 of the Libra technical
review (section 5.3) counts exactly the causal pairs, and over a whole pack they sum to
h_q * sum_j l_j (l_j + 1) / 2: the skip / full / diagonal classification of every key block,
the element mask on the diagonal blocks and the reversed walks of zigzag partners must add up
to that integer exactly.
"""
import ctypes
import os

import numpy as np
import pytest

import synth
from tests import _support as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_attention_cu_amd as m
    path = os.path.join(os.path.dirname(m.LIB_PATH), "liblibra_debug.so")
    dbg = ctypes.CDLL(path)
    dbg.libra_attn_fwd.argtypes = m._lib.libra_attn_fwd.argtypes
    dbg.libra_attn_fwd.restype = ctypes.c_int
    dbg.libra_debug_unmasked_pairs.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    dbg.libra_debug_unmasked_pairs.restype = ctypes.c_int
    dbg.libra_debug_reset_unmasked_pairs.argtypes = []
    dbg.libra_debug_reset_unmasked_pairs.restype = ctypes.c_int
    return m, dbg


CASES = [
    ("tiny_2k", None, {}),
    ("train_256k", 20000, {}),
    ("train_256k", 20000, {"assign": 2}),
    ("train_256k", 20000, {"cost": 1, "num_cus": 37}),
    ("share_1m", 24000, {}),
]


@pytest.mark.parametrize("name,L,kw", CASES)
def test_forward_counts_exactly_the_causal_pairs(libs, name, L, kw):
    import torch
    m, dbg = libs
    base = synth.WORKLOADS[name]
    w = base if L is None else base.with_tokens(L, first_lengths=(L // 2,) if base.first_lengths else None)
    lens = synth.make_lengths(w, 3)
    cu = synth.cu_seqlens(lens)
    t = synth.make_tensors(w, 3)
    S.say(f"[pairs] {name} L={w.total_tokens} samples={len(lens)} {kw}")
    plan = S.make_plan(w, cu, **kw)
    q, k, v = (S.to_dev(t[n]) for n in ("q", "k", "v"))
    dev = q.device
    plan_dev, cu_dev = plan.device(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.h_q, w.total_tokens), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    assert dbg.libra_debug_reset_unmasked_pairs() == 0
    st = dbg.libra_attn_fwd(plan.host.ctypes.data, plan_dev.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            cu_dev.data_ptr(), o.data_ptr(), lse.data_ptr(), S.scale_of(w), None, stream)
    assert st == 0
    torch.cuda.synchronize()
    got = ctypes.c_uint64(0)
    assert dbg.libra_debug_unmasked_pairs(ctypes.byref(got)) == 0
    lens = np.asarray(lens, dtype=np.int64)
    expect = w.h_q * int((lens * (lens + 1) // 2).sum())
    S.say(f"  counted {got.value}, closed form {expect}")
    assert got.value == expect == plan.info.total_pairs
