"""Pins of the fp64 attention oracle against facts it does not compute itself.

Each check below is chosen so that a plausible slip in the oracle (a mask off
by one, a dropped normaliser, a wrong GQA head, a transposed operand, a sign
error in the backward) fails at least one of them; the mutant tests at the end
plant such slips in the oracle and confirm the pins catch them.
"""
import numpy as np
import pytest
import scipy.special

from oracle import attention as A

RNG = np.random.default_rng(1234)


def rand_pack(rng, L, max_len=None, allow_empty=True):
    lens = []
    left = L
    while left > 0:
        ell = int(rng.integers(0 if allow_empty else 1, (max_len or L) + 1))
        ell = min(ell, left)
        lens.append(ell)
        left -= ell
    if allow_empty and rng.random() < 0.5:
        lens.insert(int(rng.integers(0, len(lens) + 1)), 0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return lens, cu


def rand_qkv(rng, L, h_q, h_kv, d):
    return (rng.standard_normal((L, h_q, d)), rng.standard_normal((L, h_kv, d)),
            rng.standard_normal((L, h_kv, d)))


def dense_reference(q, k, v, lens, scale):
    """Brute force over the whole L x L matrix with an explicit block-diagonal causal mask."""
    L, h_q, d = q.shape
    g = h_q // k.shape[1]
    seg = np.repeat(np.arange(len(lens)), lens)
    allowed = (seg[:, None] == seg[None, :]) & (np.arange(L)[None, :] <= np.arange(L)[:, None])
    o = np.zeros_like(q)
    lse = np.zeros((h_q, L))
    for h in range(h_q):
        S = scale * np.einsum("id,kd->ik", q[:, h], k[:, h // g])
        S = np.where(allowed, S, -np.inf)
        o[:, h] = scipy.special.softmax(S, axis=1) @ v[:, h // g]
        lse[h] = scipy.special.logsumexp(S, axis=1)
    return o, lse


# ---------------------------------------------------------------- P1 brute force
@pytest.mark.parametrize("case", range(12))
def test_brute_force_dense_mask(case):
    rng = np.random.default_rng(100 + case)
    L = int(rng.integers(1, 65))
    lens, cu = rand_pack(rng, L, max_len=int(rng.integers(1, L + 1)))
    h_kv = int(rng.choice([1, 2]))
    h_q = h_kv * int(rng.choice([1, 2, 3]))
    d = int(rng.choice([4, 8]))
    q, k, v = rand_qkv(rng, L, h_q, h_kv, d)
    scale = 1 / np.sqrt(d)
    o, lse = A.forward(q, k, v, cu, scale)
    o_ref, lse_ref = dense_reference(q, k, v, lens, scale)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


# ---------------------------------------------------- P2 packed == each sample alone
def test_packed_equals_separate():
    rng = np.random.default_rng(7)
    lens, cu = rand_pack(rng, 120, max_len=50)
    q, k, v = rand_qkv(rng, 120, 4, 2, 8)
    o, lse = A.forward(q, k, v, cu, 0.3)
    for j in range(len(lens)):
        s, e = int(cu[j]), int(cu[j + 1])
        if s == e:
            continue
        oj, lj = A.forward(q[s:e], k[s:e], v[s:e], np.array([0, e - s]), 0.3)
        assert np.array_equal(oj, o[s:e])
        assert np.array_equal(lj, lse[:, s:e])


# ---------------------------------------------------- P3 tiled == untiled (eq. 6-7)
@pytest.mark.parametrize("B,W", [(7, 1), (16, 2), (33, 4), (200, 4)])
def test_tiled_equals_untiled(B, W):
    rng = np.random.default_rng(11)
    L, h_q, h_kv, d = 150, 4, 2, 8
    lens, cu = rand_pack(rng, L, max_len=60)
    q, k, v = rand_qkv(rng, L, h_q, h_kv, d)
    o_full, lse_full = A.forward(q, k, v, cu, 0.25)
    o_t = np.full_like(o_full, np.nan)
    lse_t = np.full_like(lse_full, np.nan)
    g = h_q // h_kv
    ranges = A.sample_ranges(cu, L)
    for b in range((L + B - 1) // B):
        lo, hi = b * B, min(L, (b + 1) * B)
        for s in range(h_q // W):
            for (st, en) in ranges:           # the KV groups K(t) of the tile
                a, e = max(lo, st), min(hi, en)
                if a >= e:
                    continue
                for h in range(s * W, (s + 1) * W):
                    O, ls = A.head_rows(q, k, v, st, en, h, h // g, a - st, e - st, 0.25)
                    o_t[a:e, h] = O
                    lse_t[h, a:e] = ls
    assert not np.isnan(o_t).any()
    assert np.max(np.abs(o_t - o_full)) <= 1e-13
    assert np.max(np.abs(lse_t - lse_full)) <= 1e-13


# ---------------------------------------------------- P5 first token = its own V
def test_first_token_outputs_own_v():
    rng = np.random.default_rng(5)
    lens, cu = rand_pack(rng, 90, max_len=30, allow_empty=False)
    q, k, v = rand_qkv(rng, 90, 4, 2, 16)
    o, lse = A.forward(q, k, v, cu, 0.2)
    for j in range(len(lens)):
        s = int(cu[j])
        for h in range(4):
            assert np.array_equal(o[s, h], v[s, h // 2])
            assert abs(lse[h, s] - 0.2 * float(np.dot(q[s, h], k[s, h // 2]))) <= 1e-12


# ---------------------------------------------------- P6 identical V rows pass through
def test_identical_v_passes_through():
    rng = np.random.default_rng(6)
    lens, cu = rand_pack(rng, 100, max_len=40, allow_empty=False)
    q, k, _ = rand_qkv(rng, 100, 2, 1, 8)
    v = np.empty((100, 1, 8))
    for j in range(len(lens)):
        v[cu[j]:cu[j + 1], 0] = rng.standard_normal(8)
    o, _ = A.forward(q, k, v, cu, 0.4)
    for j in range(len(lens)):
        for h in range(2):
            assert np.max(np.abs(o[cu[j]:cu[j + 1], h] - v[cu[j], 0])) <= 1e-14


# ---------------------------------------------------- P7 K = 0: prefix mean / ln(i+1)
def test_zero_keys_closed_form():
    rng = np.random.default_rng(8)
    lens, cu = rand_pack(rng, 80, max_len=35)
    q, _, v = rand_qkv(rng, 80, 2, 1, 8)
    k = np.zeros((80, 1, 8))
    dout = rng.standard_normal((80, 2, 8))
    o, lse = A.forward(q, k, v, cu, 0.3)
    dq, dk, dv = A.backward(q, k, v, dout, cu, 0.3)
    for j in range(len(lens)):
        s, e = int(cu[j]), int(cu[j + 1])
        if s == e:
            continue
        n = e - s
        counts = np.arange(1, n + 1)[:, None]
        prefix_mean = np.cumsum(v[s:e, 0], axis=0) / counts
        for h in range(2):
            assert np.max(np.abs(o[s:e, h] - prefix_mean)) <= 1e-13
            assert np.max(np.abs(lse[h, s:e] - np.log(np.arange(1, n + 1)))) <= 1e-13
        # dV_k = sum over heads and i >= k of dO_i / (i + 1): a reversed cumulative sum.
        w = dout[s:e].sum(axis=1) / counts
        suffix = np.cumsum(w[::-1], axis=0)[::-1]
        assert np.max(np.abs(dv[s:e, 0] - suffix)) <= 1e-12
    assert np.max(np.abs(dq)) == 0.0


# ---------------------------------------------------- P8 finite differences
def test_backward_matches_finite_differences():
    rng = np.random.default_rng(9)
    lens = [3, 0, 5, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    L, h_q, h_kv, d = 9, 4, 2, 3
    q, k, v = rand_qkv(rng, L, h_q, h_kv, d)
    dout = rng.standard_normal((L, h_q, d))
    scale = 0.7
    dq, dk, dv = A.backward(q, k, v, dout, cu, scale)

    def loss(q_, k_, v_):
        return float(np.sum(A.forward(q_, k_, v_, cu, scale)[0] * dout))

    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                       loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        assert np.max(np.abs(fd - grad)) <= 1e-7, name


# ---------------------------------------------------- P9 GQA == MHA with repeated K/V
def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(10)
    lens, cu = rand_pack(rng, 60, max_len=25)
    h_q, h_kv, d = 6, 2, 8
    g = h_q // h_kv
    q, k, v = rand_qkv(rng, 60, h_q, h_kv, d)
    dout = rng.standard_normal((60, h_q, d))
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    o, lse = A.forward(q, k, v, cu, 0.3)
    o2, lse2 = A.forward(q, kr, vr, cu, 0.3)
    assert np.max(np.abs(o - o2)) <= 1e-14 and np.max(np.abs(lse - lse2)) <= 1e-14
    dq, dk, dv = A.backward(q, k, v, dout, cu, 0.3)
    dq2, dk2, dv2 = A.backward(q, kr, vr, dout, cu, 0.3)
    assert np.max(np.abs(dq - dq2)) <= 1e-13
    assert np.max(np.abs(dk - dk2.reshape(60, h_kv, g, d).sum(2))) <= 1e-13
    assert np.max(np.abs(dv - dv2.reshape(60, h_kv, g, d).sum(2))) <= 1e-13


# ---------------------------------------------------- sampled entry points == full
def test_rows_and_tail_match_full():
    rng = np.random.default_rng(12)
    lens, cu = rand_pack(rng, 140, max_len=70)
    q, k, v = rand_qkv(rng, 140, 4, 2, 8)
    dout = rng.standard_normal((140, 4, 8))
    o, lse = A.forward(q, k, v, cu, 0.3)
    rows = rng.choice(140, 25, replace=False)
    o_r, lse_r = A.forward_rows(q, k, v, cu, 0.3, rows)
    assert np.max(np.abs(o_r - o[rows])) <= 1e-13
    assert np.max(np.abs(lse_r - lse[:, rows])) <= 1e-13
    dq, dk, dv = A.backward(q, k, v, dout, cu, 0.3)
    for j in range(len(lens)):
        s, e = int(cu[j]), int(cu[j + 1])
        if e - s < 3:
            continue
        first = (e - s) // 2
        for kv in range(2):
            a, b, c = A.backward_tail(q, k, v, dout, s, e, kv, first, 0.3)
            assert np.max(np.abs(a - dq[s + first:e, kv * 2:kv * 2 + 2])) <= 1e-13
            assert np.max(np.abs(b - dk[s + first:e, kv])) <= 1e-13
            assert np.max(np.abs(c - dv[s + first:e, kv])) <= 1e-13


def test_widen_bf16_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    expect = [1.0, -1.0, 0.0, 3.140625, 3.3895313892515355e38, 9.183549615799121e-41]
    assert A.widen_bf16(bits).tolist() == expect


def test_rejects_bad_cu_seqlens():
    with pytest.raises(ValueError):
        A.sample_ranges([1, 3])
    with pytest.raises(ValueError):
        A.sample_ranges([0, 5, 3])
    with pytest.raises(ValueError):
        A.sample_ranges([0, 3], total_tokens=4)


# ---------------------------------------------------- planted slips are caught
def _mutant_scores(offset):
    def scores(Qr, K, rows, scale):
        S = scale * (Qr @ K.T)
        S[np.arange(K.shape[0])[None, :] > np.asarray(rows)[:, None] + offset] = -np.inf
        return S
    return scores


@pytest.mark.parametrize("offset", [1, -1])
def test_pins_catch_mask_off_by_one(monkeypatch, offset):
    monkeypatch.setattr(A, "_scores", _mutant_scores(offset))
    rng = np.random.default_rng(100)
    with np.errstate(invalid="ignore"):
        with pytest.raises(AssertionError):
            test_zero_keys_closed_form()
        with pytest.raises(AssertionError):
            test_brute_force_dense_mask(3)


def test_pins_catch_wrong_gqa_head(monkeypatch):
    monkeypatch.setattr(A, "kv_head", lambda h, h_q, h_kv: h % h_kv)   # interleaved groups
    with pytest.raises(AssertionError):
        test_gqa_equals_repeated_mha()


def test_pins_catch_backward_sign_slip(monkeypatch):
    orig = A.backward_tail

    def slipped(*a, **kw):
        dq, dk, dv = orig(*a, **kw)
        return dq, -dk, dv
    monkeypatch.setattr(A, "backward_tail", slipped)
    with pytest.raises(AssertionError):
        test_backward_matches_finite_differences()


def test_per_head_unit_assembly_equals_the_full_backward():
    """The GPU tests' complete-unit check runs one oracle problem per query head in threads and
    sums dK and dV over the group: that must equal the oracle's own backward of the unit."""
    from tests import _support as S
    rng = np.random.default_rng(21)
    lens = [70, 130]
    L = sum(lens)
    cu = np.array([0, 70, 200])
    bits = {n: rng.integers(0x3000, 0x4000, size=(L, h, 32), dtype=np.uint16) | (rng.integers(0, 2, size=(L, h, 32), dtype=np.uint16) << 15)
            for n, h in (("q", 6), ("k", 2), ("v", 2), ("dout", 6))}
    full = A.backward(*(A.widen_bf16(bits[n]) for n in ("q", "k", "v", "dout")), cu, 0.2)
    dq, dk, dv = S.oracle_bwd_unit(bits["q"], bits["k"], bits["v"], bits["dout"], 70, 200, 1, 3, 0.2)
    assert np.allclose(dq, full[0][70:200, 3:6], rtol=0, atol=1e-12)
    assert np.allclose(dk, full[1][70:200, 1], rtol=0, atol=1e-12)
    assert np.allclose(dv, full[2][70:200, 1], rtol=0, atol=1e-12)
