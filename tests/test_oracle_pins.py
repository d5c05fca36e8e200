"""Pins of the fp64 oracle against facts fixed by the mathematics, not by the
oracle itself: closed forms, a 50-digit brute force, a torch fp64 CPU
composition of the definition differentiated by autograd (for the backward an
independent derivation of the gradient), central finite differences for the
backward, invariants, and reductions of GQA / packed batches / wide windows to
simpler calls.

Exact attention is defined on the FlashAttention-2 overview page
(lshu.cn/news/55956), section 2.1 (score matrix, row softmax, weighted sum of
V) and claimed exact in its section 1; causal masking is its section 4.2
question 4; the sliding window is named on the install guide page
(yfxerp.com/news/195771), section 1.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def torch_mask(nq, nk, causal, left, right):
    """Boolean visibility mask built from torch.tril/triu offsets (bottom-right
    aligned): an independent formulation of the visible set."""
    m = torch.ones(nq, nk, dtype=torch.bool)
    off = nk - nq
    if causal:
        m &= torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=off)
    if left >= 0:
        m &= torch.ones(nq, nk, dtype=torch.bool).triu(diagonal=off - left)
    if right >= 0:
        m &= torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=off + right)
    return m


def sdpa_reference(q, k, v, do, scale, causal, left, right):
    """torch fp64 CPU attention (math path) + autograd; rows with no visible
    key are excluded from the comparison by the caller."""
    b, nq, h, d = q.shape
    hk = k.shape[2]
    g = h // hk
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    kr = kt.repeat_interleave(g, dim=2).transpose(1, 2)
    vr = vt.repeat_interleave(g, dim=2).transpose(1, 2)
    mask = torch_mask(nq, k.shape[1], causal, left, right)
    scores = (qt.transpose(1, 2) @ kr.transpose(-1, -2)) * scale
    scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    p = torch.softmax(scores, dim=-1)
    out = (p @ vr).transpose(1, 2)
    out.backward(torch.tensor(do))
    return (out.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(),
            kt.grad.numpy(), vt.grad.numpy())


CASES = [
    # b, nq, nk, h, hk, d, causal, left, right
    (2, 37, 37, 4, 4, 16, False, -1, -1),
    (2, 37, 37, 4, 2, 16, True, -1, -1),
    (1, 50, 50, 3, 1, 8, True, 7, 0),
    (1, 41, 41, 2, 2, 8, False, 5, 3),
    (2, 20, 33, 4, 2, 8, True, -1, -1),   # Nq < Nk: bottom-right causal
    (1, 33, 33, 2, 2, 8, False, 0, 0),    # window of one key: self only
]


@pytest.mark.parametrize("case", CASES)
def test_matches_torch_autograd_composition(oracle_mod, case):
    b, nq, nk, h, hk, d, causal, left, right = case
    q = rnd((b, nq, h, d), 1)
    k = rnd((b, nk, hk, d), 2)
    v = rnd((b, nk, hk, d), 3)
    do = rnd((b, nq, h, d), 4)
    scale = 1 / math.sqrt(d)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=scale, causal=causal, window=(left, right))
    dq, dk, dv, o2, lse2 = oracle_mod.attention_bwd(q, k, v, do, scale=scale, causal=causal,
                                                    window=(left, right))
    ro, rl, rdq, rdk, rdv = sdpa_reference(q, k, v, do, scale, causal, left, right)
    assert np.allclose(o, ro, atol=1e-13, rtol=0)
    assert np.allclose(lse, rl, atol=1e-13, rtol=0)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    assert np.allclose(dq, rdq, atol=1e-12, rtol=0)
    assert np.allclose(dk, rdk, atol=1e-12, rtol=0)
    assert np.allclose(dv, rdv, atol=1e-12, rtol=0)


def test_zero_queries_give_mean_of_visible_values(oracle_mod):
    """All scores equal (q = 0): O_i is the mean of the visible V rows and
    LSE_i = ln(#visible).  Causal: prefix means; window (left=L, right=0):
    means of the last min(i, L)+1 rows."""
    n, d, L = 40, 8, 6
    q = np.zeros((1, n, 1, d))
    k = rnd((1, n, 1, d), 5)
    v = rnd((1, n, 1, d), 6)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.3, causal=True)
    prefix = np.cumsum(v[0, :, 0, :], axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(o[0, :, 0, :], prefix, atol=1e-14)
    assert np.allclose(lse[0, 0], np.log(np.arange(1, n + 1)), atol=1e-14)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.3, causal=True, window=(L, 0))
    for i in range(n):
        lo = max(0, i - L)
        assert np.allclose(o[0, i, 0], v[0, lo:i + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(i + 1 - lo)) < 1e-14
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.3, causal=False)
    assert np.allclose(o[0, :, 0], v[0, :, 0].mean(axis=0), atol=1e-14)
    assert np.allclose(lse, math.log(n), atol=1e-14)


def test_equal_keys_give_mean_and_shifted_lse(oracle_mod):
    """All K rows equal to c: every score of row i equals s q_i.c, so O_i is
    the visible mean and LSE_i = s q_i.c + ln n_i."""
    n, d, s = 25, 4, 0.7
    q = rnd((1, n, 2, d), 7)
    c = rnd((d,), 8)
    k = np.broadcast_to(c, (1, n, 2, d)).copy()
    v = rnd((1, n, 2, d), 9)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=s, causal=True)
    for h in range(2):
        prefix = np.cumsum(v[0, :, h], axis=0) / np.arange(1, n + 1)[:, None]
        assert np.allclose(o[0, :, h], prefix, atol=1e-13)
        want = s * q[0, :, h] @ c + np.log(np.arange(1, n + 1))
        assert np.allclose(lse[0, h], want, atol=1e-13)


def test_dominant_key_selects_its_value(oracle_mod):
    """One key aligned with q_i with a large score gap: O_i -> V_{j*} with
    error at most (n-1) e^{-gap} max|V| (the others' total weight)."""
    n, d = 30, 8
    q = rnd((1, n, 1, d), 10)
    k = rnd((1, n, 1, d), 11) * 0.01
    v = rnd((1, n, 1, d), 12)
    i, jstar, alpha = 20, 13, 60.0
    k[0, jstar, 0] = alpha * q[0, i, 0] / np.linalg.norm(q[0, i, 0])
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=1.0, causal=True)
    s = k[0, :i + 1, 0] @ q[0, i, 0]
    gap = s[jstar] - np.max(np.delete(s, jstar))
    bound = i * math.exp(-gap) * np.abs(v).max() * 2
    assert gap > 30
    assert np.abs(o[0, i, 0] - v[0, jstar, 0]).max() <= bound + 1e-15


def test_causal_first_row_is_first_value(oracle_mod):
    q = rnd((2, 9, 3, 8), 13)
    k = rnd((2, 9, 3, 8), 14)
    v = rnd((2, 9, 3, 8), 15)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.4, causal=True)
    assert np.array_equal(o[:, 0], v[:, 0])
    want = 0.4 * np.einsum("bhc,bhc->bh", q[:, 0], k[:, 0])
    assert np.allclose(lse[:, :, 0], want, atol=1e-15)


def test_key_shift_invariance(oracle_mod):
    """k_j -> k_j + c for all j: O unchanged, LSE_i += s q_i.c."""
    q = rnd((1, 21, 2, 8), 16)
    k = rnd((1, 21, 2, 8), 17)
    v = rnd((1, 21, 2, 8), 18)
    c = rnd((8,), 19)
    for causal, win in [(True, (-1, -1)), (False, (4, 2))]:
        o1, l1 = oracle_mod.attention_fwd(q, k, v, scale=0.5, causal=causal, window=win)
        o2, l2 = oracle_mod.attention_fwd(q, k + c, v, scale=0.5, causal=causal, window=win)
        assert np.allclose(o1, o2, atol=1e-13)
        shift = 0.5 * np.einsum("bihc,c->bhi", q, c)
        assert np.allclose(l2 - l1, shift, atol=1e-13)


def test_linear_in_v_and_permutation_invariant(oracle_mod):
    q = rnd((1, 17, 2, 8), 20)
    k = rnd((1, 17, 2, 8), 21)
    v1 = rnd((1, 17, 2, 8), 22)
    v2 = rnd((1, 17, 2, 8), 23)
    a = -1.7
    o1, _ = oracle_mod.attention_fwd(q, k, v1, scale=0.3, causal=True)
    o2, _ = oracle_mod.attention_fwd(q, k, v2, scale=0.3, causal=True)
    o3, _ = oracle_mod.attention_fwd(q, k, v1 + a * v2, scale=0.3, causal=True)
    assert np.allclose(o3, o1 + a * o2, atol=1e-13)
    perm = np.random.default_rng(24).permutation(17)
    o4, l4 = oracle_mod.attention_fwd(q, k, v1, scale=0.3, causal=False)
    o5, l5 = oracle_mod.attention_fwd(q, k[:, perm], v1[:, perm], scale=0.3, causal=False)
    assert np.allclose(o4, o5, atol=1e-13) and np.allclose(l4, l5, atol=1e-13)


def test_zero_scale_is_uniform_attention(oracle_mod):
    q = rnd((1, 12, 1, 4), 25)
    k = rnd((1, 12, 1, 4), 26)
    v = rnd((1, 12, 1, 4), 27)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.0, causal=True)
    prefix = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, 13)[:, None]
    assert np.allclose(o[0, :, 0], prefix, atol=1e-14)


def _decimal_attention(q, k, v, scale, causal):
    """50-digit brute force of one head: q (n, d), k (m, d), v (m, d)."""
    getcontext().prec = 50
    n, m = len(q), len(k)
    D = lambda x: Decimal(float(x))
    out, lses = [], []
    sc = D(scale)
    for i in range(n):
        js = [j for j in range(m) if not causal or j <= i + (m - n)]
        s = [sc * sum(D(q[i][c]) * D(k[j][c]) for c in range(len(q[i]))) for j in js]
        mx = max(s)
        e = [(x - mx).exp() for x in s]
        tot = sum(e)
        out.append([sum(e[t] * D(v[js[t]][c]) for t in range(len(js))) / tot
                    for c in range(len(v[0]))])
        lses.append(mx + tot.ln())
    return out, lses


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_50_digits(oracle_mod, causal):
    q = rnd((1, 6, 1, 3), 30)
    k = rnd((1, 6, 1, 3), 31)
    v = rnd((1, 6, 1, 3), 32)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.8, causal=causal)
    bo, bl = _decimal_attention(q[0, :, 0], k[0, :, 0], v[0, :, 0], 0.8, causal)
    assert np.allclose(o[0, :, 0], np.array(bo, dtype=float), atol=1e-14, rtol=0)
    assert np.allclose(lse[0, 0], np.array(bl, dtype=float), atol=1e-14, rtol=0)


FD_CASES = [
    dict(b=1, n=9, h=2, hk=2, d=4, causal=True, win=(-1, -1), lens=None),
    dict(b=1, n=12, h=4, hk=2, d=4, causal=True, win=(3, 0), lens=None),
    dict(b=2, n=8, h=2, hk=1, d=3, causal=False, win=(-1, -1), lens=None),
    dict(b=3, n=0, h=2, hk=2, d=4, causal=True, win=(2, 0), lens=[5, 1, 7]),
]


@pytest.mark.parametrize("case", FD_CASES)
def test_backward_matches_central_finite_differences(oracle_mod, case):
    """L = sum(dO * O); dL/dx by central differences in fp64 (step 1e-6)."""
    lens = case["lens"]
    h, hk, d = case["h"], case["hk"], case["d"]
    if lens is None:
        qs = (case["b"], case["n"], h, d)
        ks = (case["b"], case["n"], hk, d)
        cu = None
    else:
        qs = (sum(lens), h, d)
        ks = (sum(lens), hk, d)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, do = rnd(qs, 40), rnd(ks, 41), rnd(ks, 42), rnd(qs, 43)
    kw = dict(scale=0.6, causal=case["causal"], window=case["win"], cu_seqlens=cu)
    dq, dk, dv, _, _ = oracle_mod.attention_bwd(q, k, v, do, **kw)

    def loss(qq, kk, vv):
        o, _ = oracle_mod.attention_fwd(qq, kk, vv, **kw)
        return float(np.sum(do * o))

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = list(args); am = list(args)
            pos = "qkv".index(name)
            ap[pos] = xp; am[pos] = xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * eps)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-30)
        assert err < 1e-6, (name, err)


def test_backward_invariants(oracle_mod):
    """sum_j dS_ij = 0 gives sum_j dK_j = 0; softmax rows summing to one give
    sum_j dV_j = sum over the group's rows of dO_i."""
    q, k, v, do = rnd((2, 30, 4, 8), 50), rnd((2, 30, 2, 8), 51), rnd((2, 30, 2, 8), 52), rnd((2, 30, 4, 8), 53)
    for win in [(-1, -1), (5, 0)]:
        dq, dk, dv, _, _ = oracle_mod.attention_bwd(q, k, v, do, scale=0.4, causal=True, window=win)
        assert np.abs(dk.sum(axis=1)).max() < 1e-12
        want = do.reshape(2, 30, 2, 2, 8).sum(axis=(1, 3))
        assert np.allclose(dv.sum(axis=1), want, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv(oracle_mod):
    q, k, v, do = rnd((1, 19, 6, 8), 60), rnd((1, 19, 2, 8), 61), rnd((1, 19, 2, 8), 62), rnd((1, 19, 6, 8), 63)
    kw = dict(scale=0.3, causal=True, window=(6, 0))
    dq, dk, dv, o, lse = oracle_mod.attention_bwd(q, k, v, do, **kw)
    kr, vr = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)
    dq2, dk2, dv2, o2, lse2 = oracle_mod.attention_bwd(q, kr, vr, do, **kw)
    assert np.allclose(o, o2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)
    assert np.allclose(dq, dq2, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(1, 19, 2, 3, 8).sum(axis=3), atol=1e-13)
    assert np.allclose(dv, dv2.reshape(1, 19, 2, 3, 8).sum(axis=3), atol=1e-13)


def test_packed_batch_equals_independent_calls(oracle_mod):
    lens = [7, 1, 13, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = cu[-1]
    q, k, v, do = rnd((T, 4, 8), 70), rnd((T, 2, 8), 71), rnd((T, 2, 8), 72), rnd((T, 4, 8), 73)
    kw = dict(scale=0.35, causal=True, window=(3, 0))
    dq, dk, dv, o, lse = oracle_mod.attention_bwd(q, k, v, do, cu_seqlens=cu, **kw)
    for b, L in enumerate(lens):
        s = slice(cu[b], cu[b + 1])
        r = oracle_mod.attention_bwd(q[None, s], k[None, s], v[None, s], do[None, s], **kw)
        assert np.allclose(dq[s], r[0][0], atol=1e-14)
        assert np.allclose(dk[s], r[1][0], atol=1e-14)
        assert np.allclose(dv[s], r[2][0], atol=1e-14)
        assert np.allclose(o[s], r[3][0], atol=1e-14)
        assert np.allclose(lse[:, s], r[4][0], atol=1e-14)


def test_packed_batch_with_own_key_lengths_equals_independent_calls(oracle_mod):
    """Packed queries and keys with lengths of their own (cu_seqlens_k):
    sequence b is the fixed-layout call on its Lq queries and Lk keys,
    bottom-right aligned, empty sequences included."""
    lq, lk = [5, 0, 9, 3, 1], [11, 4, 9, 2, 0]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, do = rnd((cq[-1], 4, 8), 74), rnd((cq[-1], 4, 8), 77)
    k, v = rnd((ck[-1], 2, 8), 75), rnd((ck[-1], 2, 8), 76)
    kw = dict(scale=0.45, causal=True, window=(4, 0))
    dq, dk, dv, o, lse = oracle_mod.attention_bwd(q, k, v, do, cu_seqlens=cq, cu_seqlens_k=ck, **kw)
    for b in range(len(lq)):
        sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        if lq[b] == 0:
            assert np.all(dk[sk] == 0) and np.all(dv[sk] == 0)
            continue
        r = oracle_mod.attention_bwd(q[None, sq], k[None, sk], v[None, sk], do[None, sq], **kw)
        o1, l1 = oracle_mod.attention_fwd(q[None, sq], k[None, sk], v[None, sk], **kw)
        assert np.allclose(dq[sq], r[0][0], atol=1e-14)
        assert np.allclose(dk[sk], r[1][0], atol=1e-14) and np.allclose(dv[sk], r[2][0], atol=1e-14)
        assert np.allclose(o[sq], o1[0], atol=1e-14, equal_nan=True)
        assert np.allclose(lse[:, sq], l1[0], atol=1e-14, equal_nan=True)


def test_wide_window_equals_plain_causal(oracle_mod):
    q, k, v = rnd((1, 23, 2, 8), 80), rnd((1, 23, 2, 8), 81), rnd((1, 23, 2, 8), 82)
    o1, l1 = oracle_mod.attention_fwd(q, k, v, scale=0.5, causal=True)
    o2, l2 = oracle_mod.attention_fwd(q, k, v, scale=0.5, causal=True, window=(22, 0))
    o3, l3 = oracle_mod.attention_fwd(q, k, v, scale=0.5, causal=False, window=(-1, 0))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_rows_without_visible_keys(oracle_mod):
    """Nq > Nk with bottom-right causal alignment: the first Nq-Nk rows see no
    key and get O = 0, LSE = -inf (zero gradients)."""
    q, k, v, do = rnd((1, 10, 1, 4), 90), rnd((1, 6, 1, 4), 91), rnd((1, 6, 1, 4), 92), rnd((1, 10, 1, 4), 93)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.5, causal=True)
    assert np.all(o[0, :4] == 0) and np.all(np.isneginf(lse[0, 0, :4]))
    assert np.all(np.isfinite(lse[0, 0, 4:]))
    dq, dk, dv, _, _ = oracle_mod.attention_bwd(q, k, v, do, scale=0.5, causal=True)
    assert np.all(dq[0, :4] == 0)
    assert np.allclose(o[0, 4], v[0, 0])


def test_selection_returns_the_same_values(oracle_mod):
    q, k, v, do = rnd((2, 40, 4, 8), 100), rnd((2, 40, 2, 8), 101), rnd((2, 40, 2, 8), 102), rnd((2, 40, 4, 8), 103)
    kw = dict(scale=0.3, causal=True, window=(9, 0))
    full = oracle_mod.attention_bwd(q, k, v, do, **kw)
    fo, fl = oracle_mod.attention_fwd(q, k, v, **kw)
    rows = np.array([0, 3, 39], dtype=np.int32)
    so, sl = oracle_mod.attention_fwd(q, k, v, rows=rows, heads=[1, 3], **kw)
    assert np.array_equal(so[:, rows][:, :, [1, 3]], fo[:, rows][:, :, [1, 3]])
    assert np.isnan(so[:, 1]).all() and np.isnan(so[:, :, 0]).all()
    part = oracle_mod.attention_bwd(q, k, v, do, q_rows=[5, 17], k_rows=[2, 38], kv_heads=[1], **kw)
    assert np.array_equal(part[0][:, [5, 17], 2:], full[0][:, [5, 17], 2:])
    assert np.array_equal(part[1][:, [2, 38], 1], full[1][:, [2, 38], 1])
    assert np.array_equal(part[2][:, [2, 38], 1], full[2][:, [2, 38], 1])
    assert np.isnan(part[1][:, :, 0]).all()


def test_score_matrix_size_quoted_by_the_pages():
    """The standard forward's N x N fp16 score matrix (2 bytes per entry) is
    what the tiled method never writes; the pages quote its size."""
    facts = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
    for n, want in facts["score_matrix_bytes_fp16"].items():
        assert int(n) * int(n) * 2 == want
