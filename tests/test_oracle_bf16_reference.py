"""Pins of the bf16 PyTorch reference that scales the pages' tolerance criterion (Libra paper,
section 6.7: errors within 2x those of a bf16 PyTorch reference).

The reference is a torch graph; run in float64 it must be the fp64 oracle itself (which pins its
mask, scale, GQA mapping and gradient sums).  In bf16 its errors on the seeded inputs of the
extreme-logit tests are stored in tests/golden/bf16_yardstick.json, written by
tests/golden/make_bf16_yardstick.py from oracle/ alone, so that a change in its rounding (an extra
bf16 rounding, a different precision) shows up as a changed yardstick.
"""
import json
import os
import sys

import numpy as np
import pytest

from oracle import attention as A, bf16_reference as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
sys.path.insert(0, GOLDEN)
import make_bf16_yardstick as MK  # noqa: E402


def _random_pack(rng, lens, h_q, h_kv, d):
    L = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((L, h_q, d))
    k = rng.standard_normal((L, h_kv, d))
    v = rng.standard_normal((L, h_kv, d))
    do = rng.standard_normal((L, h_q, d))
    return q, k, v, do, cu


@pytest.mark.parametrize("lens,h_q,h_kv", [([40, 1, 23, 0, 64], 4, 2), ([17, 0, 1, 9], 3, 3),
                                           ([33, 5], 6, 2), ([1], 2, 1)])
def test_float64_graph_is_the_oracle(lens, h_q, h_kv):
    import torch
    rng = np.random.default_rng(sum(lens) + h_q)
    q, k, v, do, cu = _random_pack(rng, lens, h_q, h_kv, 16)
    scale = 0.3
    o, *g = R.attention(q, k, v, do, cu, scale, dtype=torch.float64)
    o_ref, _ = A.forward(q, k, v, cu, scale)
    g_ref = A.backward(q, k, v, do, cu, scale)
    assert np.abs(o - o_ref).max() <= 1e-12
    for a, r in zip(g, g_ref):
        assert np.abs(a - r).max() <= 1e-11 * max(1.0, np.abs(r).max())


def test_float64_pin_catches_a_mask_slip(monkeypatch):
    """Planted in the reference: the diagonal key excluded from the mask."""
    import torch
    monkeypatch.setattr(R, "_causal", lambda n: torch.ones(n, n, dtype=torch.bool).tril(-1) |
                        (torch.eye(n, dtype=torch.bool) & (torch.arange(n) == 0)[:, None]))
    with pytest.raises(AssertionError):
        test_float64_graph_is_the_oracle([40, 1, 23, 0, 64], 4, 2)


def test_bf16_errors_equal_the_stored_yardstick():
    doc = json.load(open(os.path.join(GOLDEN, "bf16_yardstick.json")))
    assert tuple(doc["pack"]["lens"]) == MK.LENS and doc["pack"]["seed"] == MK.SEED
    for kind, want in doc["errors"].items():
        got = MK.errors(kind)
        for key, value in want.items():
            assert got[key] == pytest.approx(value, rel=0.02), (kind, key, got[key], value)


def test_bf16_errors_are_bf16_level_on_normal_inputs():
    """On N(0, 1) inputs the bf16 evaluation errs at the bf16 level: above zero (it does round)
    and within the fixed tolerances the kernels are held to."""
    e = MK.errors("normal")
    assert 0 < e["o_max_abs"] <= 2e-2
    for key in ("dq_max_rel", "dk_max_rel", "dv_max_rel"):
        assert 1e-3 < e[key] <= 5e-2, key
