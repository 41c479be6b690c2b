"""fp64 CPU oracle: block-diagonal causal softmax attention over one packed sequence.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU
baseline call this module; the library never does, and it shares no code with
the HIP path (no kernels, helpers, tables or pre/post-processing).

What it computes (Libra technical review, section 1 "Sequence packing" and
section 5.3 under eq. 8; Libra paper, section 2.3): samples are concatenated
into one sequence of L tokens; a query at sample-local position q attends to
the keys of its own sample at sample-local positions 0..q (diagonal included)
and to nothing in any other sample.  Attention itself is the usual
softmax(scale * Q K^T) V per query head; query head h reads key/value head
floor(h / g) with g = h_q / h_kv (contiguous GQA groups; the pages name KV head
counts but not the mapping, so this is the plain reading).

Everything runs in float64 on the exact widening of the bf16 inputs.  Each
(sample, head) pair is evaluated on its own, straight from the definition:

    S = scale * Q K^T, with S[i, k] = -inf for k > i
    m_i = max_k S[i, k];  P = exp(S - m);  l_i = sum_k P[i, k]
    O_i = sum_k P[i, k] V_k / l_i;  LSE_i = m_i + ln l_i

Rows are visited in groups only to bound memory: every row still sees its
whole key prefix in one matrix product, so grouping changes no arithmetic of
the definition.

The backward is the analytic gradient of L = sum(O * dO) for that definition
(the pages only say dQ, dK, dV come back along reversed transfers and meet
FlashAttention's test tolerance, Libra paper section 4.3.3 and section 6.7):

    Phat = P / l;  dV_k = sum_i Phat[i, k] dO_i;  dP = dO V^T
    D_i = sum_k Phat[i, k] dP[i, k];  dS = Phat * (dP - D)
    dQ_i = scale * sum_k dS[i, k] K_k;  dK_k = scale * sum_i dS[i, k] Q_i

dK and dV of a KV head sum over its g query heads.
"""
from __future__ import annotations

import numpy as np

MAX_MATRIX_ELEMS = 1 << 24   # bound on one rows x keys fp64 matrix (128 MiB)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (uint16)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns")
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sample_ranges(cu_seqlens, total_tokens: int = None) -> list:
    """[(start, end), ...] of every sample; validates the prefix array."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    if np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    if total_tokens is not None and cu[-1] != total_tokens:
        raise ValueError("cu_seqlens must end at L")
    return [(int(cu[j]), int(cu[j + 1])) for j in range(cu.size - 1)]


def _group(h_q: int, h_kv: int) -> int:
    if h_kv <= 0 or h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    return h_q // h_kv


def kv_head(h: int, h_q: int, h_kv: int) -> int:
    """KV head read by query head h: contiguous groups of g = h_q / h_kv query heads."""
    return h // _group(h_q, h_kv)


def _row_groups(first: int, last: int, keys: int):
    """Split sample-local rows [first, last) into groups whose matrices stay bounded."""
    step = max(1, min(last - first, MAX_MATRIX_ELEMS // max(1, keys)))
    r = first
    while r < last:
        yield r, min(last, r + step)
        r += step


def _scores(Qr, K, rows, scale):
    """scale * Q K^T for the sample-local query rows ``rows``; key k > row is masked."""
    S = scale * (Qr @ K.T)
    S[np.arange(K.shape[0])[None, :] > np.asarray(rows)[:, None]] = -np.inf
    return S


def attend_rows(Qr, K, V, rows, scale):
    """O and LSE of query rows of one sample and one head.

    Qr [n, d] holds the queries at sample-local positions ``rows``; K and V
    [m, d] hold the sample's keys and values 0..m-1 with m > max(rows).
    Row i sees keys 0..i only.
    """
    S = _scores(Qr, K, rows, scale)
    m = S.max(axis=1)
    P = np.exp(S - m[:, None])
    l = P.sum(axis=1)
    return (P @ V) / l[:, None], m + np.log(l)


def head_rows(q, k, v, start, end, h, kv, first, last, scale):
    """O rows and LSE of sample-local rows [first, last) of one sample and one Q head.

    q, k, v are float64 [L, heads, d]; (start, end) is the sample's token range.
    """
    d = q.shape[2]
    O = np.empty((last - first, d))
    lse = np.empty(last - first)
    for r0, r1 in _row_groups(first, last, last):
        o_g, l_g = attend_rows(q[start + r0:start + r1, h], k[start:start + r1, kv],
                               v[start:start + r1, kv], np.arange(r0, r1), scale)
        O[r0 - first:r1 - first] = o_g
        lse[r0 - first:r1 - first] = l_g
    return O, lse


def forward(q, k, v, cu_seqlens, scale):
    """Full forward: O [L, h_q, d] and LSE [h_q, L] (natural log), float64."""
    L, h_q, d = q.shape
    g = _group(h_q, k.shape[1])
    o = np.zeros((L, h_q, d))
    lse = np.zeros((h_q, L))
    for start, end in sample_ranges(cu_seqlens, L):
        n = end - start
        if n == 0:
            continue
        for h in range(h_q):
            O, s = head_rows(q, k, v, start, end, h, kv_head(h, h_q, k.shape[1]), 0, n, scale)
            o[start:end, h] = O
            lse[h, start:end] = s
    return o, lse


def forward_rows(q, k, v, cu_seqlens, scale, rows):
    """O[rows] [n, h_q, d] and LSE[:, rows] [h_q, n] for selected global rows."""
    L, h_q, d = q.shape
    g = _group(h_q, k.shape[1])
    ranges = sample_ranges(cu_seqlens, L)
    starts = np.array([s for s, _ in ranges], dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, h_q, d))
    lse = np.zeros((h_q, rows.size))
    for idx, row in enumerate(rows):
        j = int(np.searchsorted(starts, row, side="right")) - 1
        while ranges[j][1] <= row:      # skip empty samples that share the start
            j += 1
        start, end = ranges[j]
        i = int(row) - start
        for h in range(h_q):
            O, s = head_rows(q, k, v, start, end, h, kv_head(h, h_q, k.shape[1]), i, i + 1, scale)
            o[idx, h] = O[0]
            lse[h, idx] = s[0]
    return o, lse


def backward_tail(q, k, v, dout, start, end, kv, first, scale):
    """Gradients of one (sample, KV head) unit restricted to sample-local rows [first, n).

    Returns dq [n - first, g, d] for the g query heads of KV head ``kv`` and
    dk, dv [n - first, d] for the keys [first, n).  Keys at or after ``first``
    receive contributions only from queries at or after them, so these dk/dv
    rows are complete; dq rows are complete by construction.
    """
    h_q, d = q.shape[1], q.shape[2]
    g = _group(h_q, k.shape[1])
    n = end - start
    dq = np.zeros((n - first, g, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    heads = [h for h in range(h_q) if kv_head(h, h_q, k.shape[1]) == kv]
    for hh, h in enumerate(heads):
        for r0, r1 in _row_groups(first, n, n):
            Qr = q[start + r0:start + r1, h]
            dOr = dout[start + r0:start + r1, h]
            K = k[start:start + r1, kv]
            V = v[start:start + r1, kv]
            S = _scores(Qr, K, np.arange(r0, r1), scale)
            m = S.max(axis=1)
            P = np.exp(S - m[:, None])
            Phat = P / P.sum(axis=1)[:, None]
            dP = dOr @ V.T
            D = (Phat * dP).sum(axis=1)
            dS = Phat * (dP - D[:, None])
            dq[r0 - first:r1 - first, hh] = scale * (dS @ K)
            dk[:r1] += scale * (dS.T @ Qr)
            dv[:r1] += Phat.T @ dOr
    return dq, dk[first:], dv[first:]


def backward(q, k, v, dout, cu_seqlens, scale):
    """Full backward: dq [L, h_q, d], dk and dv [L, h_kv, d], float64."""
    L, h_q, d = q.shape
    h_kv = k.shape[1]
    g = _group(h_q, h_kv)
    dq = np.zeros((L, h_q, d))
    dk = np.zeros((L, h_kv, d))
    dv = np.zeros((L, h_kv, d))
    for start, end in sample_ranges(cu_seqlens, L):
        if end == start:
            continue
        for kv in range(h_kv):
            a, b, c = backward_tail(q, k, v, dout, start, end, kv, 0, scale)
            dq[start:end, kv * g:(kv + 1) * g] = a
            dk[start:end, kv] = b
            dv[start:end, kv] = c
    return dq, dk, dv
