"""Pins of the oracle's dropout (the dropout_p argument of the attention call,
FlashAttention-2 overview page lshu.cn/news/55956, section 3.3) against facts
outside the oracle:

* the generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011) reproduces the known-answer vectors
  published with its reference implementation (Random123), and the same round
  construction on 64-bit words reproduces numpy's independent Philox4x64-10;
* the keep threshold's arithmetic and the kept fraction (binomial bound);
* how the mask enters the output: with V the identity, O is the masked,
  rescaled probability matrix, read element by element;
* unbiasedness: the mean of O over many seeds tends to O without dropout;
* the backward: central finite differences of sum(dO * O) with the mask held
  fixed (a fixed seed), and D_i = dO_i . O_i.
"""
import numpy as np
import pytest

# Random123 known-answer vectors for philox4x32 with 10 rounds: (counter, key, output).
PHILOX4X32_10_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("ctr,key,want", PHILOX4X32_10_KAT)
def test_philox4x32_known_answers(oracle_mod, ctr, key, want):
    assert tuple(int(x) for x in oracle_mod.philox4x32_10(ctr, key)) == want


@pytest.mark.parametrize("ctr,key", [((5, 6, 7, 8), (11, 12)), ((2**64 - 2, 0, 3, 2**63), (2**64 - 1, 7)),
                                     ((0, 0, 0, 0), (0, 0))])
def test_round_structure_matches_numpy_philox4x64(oracle_mod, ctr, key):
    """numpy.random.Philox is Philox4x64-10; it increments its 256-bit counter
    before producing each block, so its first block is that of counter + 1."""
    g = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = g.random_raw(4)
    c = list(ctr)
    for w in range(4):  # + 1 with carry across the four 64-bit words
        c[w] = (c[w] + 1) % 2**64
        if c[w] != 0:
            break
    assert [int(x) for x in oracle_mod.philox4x64_10(c, key)] == [int(x) for x in raw]


def test_keep_threshold(oracle_mod):
    t = oracle_mod.dropout_threshold
    assert t(0.0) == 256 and t(0.5) == 128 and t(0.25) == 192
    assert t(0.1) == 230          # 230.4 rounds down
    assert t(0.1 - 0.5 / 256) == 231 and t(0.001) == 256 and t(0.999) == 0


def test_kept_fraction_is_binomial(oracle_mod):
    for p in (0.1, 0.25, 0.5):
        m = oracle_mod.dropout_mask(2, 3, 64, 96, p, seed=123456789)
        n = m.size
        q = oracle_mod.dropout_threshold(p) / 256.0
        assert abs(m.mean() - q) < 5 * np.sqrt(q * (1 - q) / n)


def test_mask_bytes_come_from_the_documented_words(oracle_mod):
    """Element (b, h, i, j): byte j % 4 of word i % 4 of the block at counter
    (j / 4, i / 4, h, b), key = the seed's two 32-bit halves."""
    seed = 0x0123456789ABCDEF
    p = 0.3
    tt = oracle_mod.dropout_threshold(p)
    m = oracle_mod.dropout_mask(2, 2, 9, 13, p, seed)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    for b, h, i, j in [(0, 0, 0, 0), (1, 1, 8, 12), (0, 1, 5, 7), (1, 0, 3, 4)]:
        w = oracle_mod.philox4x32_10((j >> 2, i >> 2, h, b), key)
        u = (int(w[i & 3]) >> (8 * (j & 3))) & 0xFF
        assert m[b, h, i, j] == (u < tt)


def test_identity_values_expose_the_masked_probabilities(oracle_mod):
    """With Nk = d and V = I, O_ij = P_ij M_ij s: the output shows each keep
    decision (O_ij = 0 or P_ij s), and the undropped P from the same call's LSE."""
    n, d, h, p, seed = 16, 16, 2, 0.4, 77
    q, k = rnd((1, n, h, d), 1), rnd((1, n, h, d), 2)
    v = np.broadcast_to(np.eye(d)[None, :, None, :], (1, n, h, d)).copy()
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=0.5, causal=True, dropout_p=p, seed=seed)
    mask = oracle_mod.dropout_mask(1, h, n, n, p, seed)
    s = 256.0 / oracle_mod.dropout_threshold(p)
    for hh in range(h):
        sc = 0.5 * q[0, :, hh] @ k[0, :, hh].T
        vis = np.tril(np.ones((n, n), dtype=bool))
        pm = np.where(vis, np.exp(sc - lse[0, hh][:, None]), 0.0)   # undropped softmax
        assert np.allclose(pm.sum(1), 1.0, atol=1e-13)
        want = pm * mask[0, hh] * s
        assert np.allclose(o[0, :, hh], want, atol=1e-14, rtol=0)


def test_zero_probability_is_plain_attention(oracle_mod):
    q, k, v, do = rnd((2, 20, 4, 8), 3), rnd((2, 20, 2, 8), 4), rnd((2, 20, 2, 8), 5), rnd((2, 20, 4, 8), 6)
    kw = dict(scale=0.4, causal=True, window=(6, 0))
    o0, l0 = oracle_mod.attention_fwd(q, k, v, **kw)
    o1, l1 = oracle_mod.attention_fwd(q, k, v, dropout_p=0.0, seed=99, **kw)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = oracle_mod.attention_bwd(q, k, v, do, **kw)[:3]
    g1 = oracle_mod.attention_bwd(q, k, v, do, dropout_p=0.0, seed=99, **kw)[:3]
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


def test_lse_is_that_of_the_undropped_softmax(oracle_mod):
    q, k, v = rnd((1, 24, 2, 8), 7), rnd((1, 24, 2, 8), 8), rnd((1, 24, 2, 8), 9)
    _, l0 = oracle_mod.attention_fwd(q, k, v, scale=0.7, causal=True)
    _, l1 = oracle_mod.attention_fwd(q, k, v, scale=0.7, causal=True, dropout_p=0.3, seed=5)
    assert np.array_equal(l0, l1)


def test_dropout_is_unbiased_over_seeds(oracle_mod):
    """E[M s] = (T / 256) (256 / T) = 1, so the mean of O over independent seeds
    converges to O without dropout; the bound is 6 standard errors per entry."""
    q, k, v = rnd((1, 12, 1, 4), 10), rnd((1, 12, 1, 4), 11), rnd((1, 12, 1, 4), 12)
    kw = dict(scale=0.9, causal=True)
    o_ref, _ = oracle_mod.attention_fwd(q, k, v, **kw)
    outs = np.stack([oracle_mod.attention_fwd(q, k, v, dropout_p=0.3, seed=1000 + t, **kw)[0]
                     for t in range(600)])
    mean, se = outs.mean(0), outs.std(0) / np.sqrt(len(outs))
    assert np.all(np.abs(mean - o_ref) <= 6 * se + 1e-12)


FD_DROP_CASES = [
    dict(b=1, n=9, h=2, hk=2, d=4, causal=True, win=(-1, -1), p=0.3, seed=11),
    dict(b=2, n=10, h=4, hk=2, d=3, causal=False, win=(-1, -1), p=0.5, seed=2**40 + 3),
    dict(b=1, n=12, h=2, hk=1, d=4, causal=True, win=(4, 0), p=0.2, seed=7),
]


@pytest.mark.parametrize("case", FD_DROP_CASES)
def test_dropout_backward_matches_central_finite_differences(oracle_mod, case):
    """The mask depends only on positions and the seed, so L = sum(dO * O) is a
    smooth function of q, k, v at a fixed seed; dL/dx by central differences."""
    h, hk, d = case["h"], case["hk"], case["d"]
    qs, ks = (case["b"], case["n"], h, d), (case["b"], case["n"], hk, d)
    q, k, v, do = rnd(qs, 40), rnd(ks, 41), rnd(ks, 42), rnd(qs, 43)
    kw = dict(scale=0.6, causal=case["causal"], window=case["win"], dropout_p=case["p"], seed=case["seed"])
    dq, dk, dv, o, _ = oracle_mod.attention_bwd(q, k, v, do, **kw)

    def loss(qq, kk, vv):
        return float(np.sum(do * oracle_mod.attention_fwd(qq, kk, vv, **kw)[0]))

    eps = 1e-6
    for pos, (x, g) in enumerate(((q, dq), (k, dk), (v, dv))):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p, args_m = [q, k, v], [q, k, v]
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p[pos], args_m[pos] = xp, xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-30)
        assert err < 1e-6, ("qkv"[pos], err)


def test_row_term_is_dout_dot_output(oracle_mod):
    """D_i = sum_j P_ij M_ij s dP_ij equals dO_i . O_i with dropout too: the
    dropout backward needs no other row term."""
    q, k, v, do = rnd((1, 16, 2, 8), 20), rnd((1, 16, 2, 8), 21), rnd((1, 16, 2, 8), 22), rnd((1, 16, 2, 8), 23)
    kw = dict(scale=0.5, causal=True, dropout_p=0.4, seed=31)
    o, _ = oracle_mod.attention_fwd(q, k, v, **kw)
    dq, dk, dv, _, _ = oracle_mod.attention_bwd(q, k, v, do, **kw)
    # sum_j dK_j = scale * sum_ij dS_ij q_i and sum_j dS_ij = sum_j P_ij (M s dP_ij) - D_i sum_j P_ij
    # = D_i - D_i = 0 exactly when D_i = dO_i . O_i: so sum_j dK_j vanishes
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
