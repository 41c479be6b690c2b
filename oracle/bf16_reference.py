"""The bf16 PyTorch reference that scales the pages' tolerance criterion.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``); it shares no code
with the HIP path.

The Libra paper (section 6.7, "Numerical Fidelity") states its accuracy
criterion as FlashAttention's test-suite rule: the kernel's error against a
high-precision reference stays within twice the error of a plain PyTorch
evaluation of the same attention in bf16.  This module is that plain
evaluation, written with torch on the CPU: per sample, the scores are a bf16
matrix product scaled in bf16, the causal mask is applied with -inf, the
softmax and the product with V run in bf16, and autograd supplies the
gradients for the output gradient dO.  GQA repeats each KV head over its
query heads (contiguous groups), so autograd sums dK and dV over the group.

``dtype`` selects the precision of every tensor: torch.bfloat16 gives the
yardstick; torch.float64 gives the same graph in double precision, which must
reproduce the fp64 oracle (that is how the graph itself is checked).
"""
from __future__ import annotations

import numpy as np


def _causal(n: int):
    """Mask of the keys each of n sample-local queries may see: key k <= query i."""
    import torch
    return torch.ones(n, n, dtype=torch.bool).tril()


def _ranges(cu_seqlens):
    cu = [int(x) for x in cu_seqlens]
    return [(cu[j], cu[j + 1]) for j in range(len(cu) - 1)]


def attention(q, k, v, dout, cu_seqlens, scale, dtype=None):
    """(o, dq, dk, dv) of the plain PyTorch evaluation, as float64 numpy arrays.

    q, dout: [L, h_q, d]; k, v: [L, h_kv, d] (float64 arrays; for the bf16
    yardstick they hold bf16 values, so the conversion is exact)."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    L, h_q, d = q.shape
    h_kv = k.shape[1]
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    g = h_q // h_kv
    out = [np.zeros(q.shape), np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
    for start, end in _ranges(cu_seqlens):
        n = end - start
        if n == 0:
            continue

        def leaf(x):
            # [n, heads, d] -> [heads, n, d] in the working precision
            return torch.from_numpy(np.ascontiguousarray(x[start:end].transpose(1, 0, 2))).to(dtype) \
                .requires_grad_(True)

        Q, K, V = leaf(q), leaf(k), leaf(v)
        dO = torch.from_numpy(np.ascontiguousarray(dout[start:end].transpose(1, 0, 2))).to(dtype)
        Kr = K.repeat_interleave(g, dim=0)          # query head h reads KV head h // g
        Vr = V.repeat_interleave(g, dim=0)
        S = torch.matmul(Q, Kr.transpose(1, 2).contiguous()) * scale
        P = torch.softmax(S.masked_fill(~_causal(n), float("-inf")), dim=-1)
        O = torch.matmul(P, Vr)
        dQ, dK, dV = torch.autograd.grad(O, (Q, K, V), dO)
        for i, t in enumerate((O, dQ, dK, dV)):
            out[i][start:end] = t.detach().to(torch.float64).numpy().transpose(1, 0, 2)
    return tuple(out)
