"""Seeded random configurations on the GPU, forward and backward against the
fp64 oracle element by element (O max-abs 4e-3 fp16 / 2e-2 bf16, LSE 1e-3,
dQ/dK/dV relative L2 2e-2, the tolerances of the fixed cases).

Each configuration draws, from its own seed: the 16-bit type, a head_dim
among the multiples of 8 up to 256, a GQA ratio, query and key lengths
(equal, or not for the fixed layout), causal or not, a window or none, the
layout (fixed, packed variable-length or padded with seqused) and dropout or
none.  The combinations the fixed cases do not list are where a wrong index
or a missed mask shows.  The KV-cache decode gets the same treatment: GQA
ratio, new tokens, cache lengths (empty included), head_dim, masks and the
split count.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from _bounds import cancel_bound

pytestmark = pytest.mark.gpu

O_TOL = {"fp16": 4e-3, "bf16": 2e-2}
LSE_TOL = 1e-3
GRAD_TOL = 2e-2
N_CONFIGS = 64


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_10_amd as m
    m.lib()
    return m


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    d = int(r.choice([8, 16, 40, 64, 72, 96, 128, 136, 192, 248, 256]))
    g = int(r.choice([1, 2, 4, 8]))
    kv = int(r.integers(1, 3))
    layout = str(r.choice(["fixed", "varlen", "padded"]))
    cfg = dict(dtype=str(r.choice(["fp16", "bf16"])), head_dim=d, heads=g * kv, kv_heads=kv,
               causal=bool(r.integers(0, 2)))
    if r.random() < 0.4:
        cfg["window"] = (int(r.integers(0, 200)), int(r.integers(0, 60)) if r.random() < 0.5 else -1)
    if layout == "varlen":
        n = int(r.integers(1, 5))
        cfg.update(batch=0, seqlen=0, seqlens=[int(x) for x in r.integers(0, 300, n)])
        if sum(cfg["seqlens"]) == 0:
            cfg["seqlens"][0] = 5
    else:
        cfg.update(batch=int(r.integers(1, 4)), seqlen=int(r.integers(1, 320)))
        if r.random() < 0.5:
            cfg["seqlen_k"] = int(r.integers(1, 320))
    drop = float(r.choice([0.0, 0.0, 0.25]))
    used = None
    if layout == "padded":
        nq, nk = cfg["seqlen"], cfg.get("seqlen_k", cfg["seqlen"])
        used = ([int(x) for x in r.integers(0, nq + 1, cfg["batch"])], [int(x) for x in r.integers(0, nk + 1, cfg["batch"])])
    return cfg, layout, drop, used


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.parametrize("seed", range(N_CONFIGS))
def test_random_config(fa, oracle_mod, seed):
    cfg, layout, drop, used = draw(seed)
    say(f"[random {seed}] {layout} drop={drop} used={used} {cfg}")
    p = synth.make_problem(seed=50 + seed, **cfg)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    cu = p.cu_seqlens()
    kw = dict(causal=p.causal, window_size=(p.window_left, p.window_right), softmax_scale=p.scale,
              dropout_p=drop, dropout_seed=77 + seed)
    if cu is not None:
        cud = cu.to(dev)
        kw.update(cu_seqlens_q=cud, cu_seqlens_k=cud, max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    if used is not None:
        kw.update(seqused_q=torch.tensor(used[0], dtype=torch.int32, device=dev),
                  seqused_k=torch.tensor(used[1], dtype=torch.int32, device=dev))
    o, lse = fa.forward(q, k, v, **kw)
    dq, dk, dv = fa.backward(do, q, k, v, o, lse, **kw)
    torch.cuda.synchronize()
    g = lambda t: t.float().cpu().double().numpy()
    got = dict(o=g(o), lse=lse.cpu().double().numpy(), dq=g(dq), dk=g(dk), dv=g(dv))
    okw = dict(scale=p.scale, causal=p.causal, window=(p.window_left, p.window_right), dropout_p=drop,
               seed=77 + seed, threads=16)
    if used is None:
        rdq, rdk, rdv, ro, rlse = oracle_mod.attention_bwd(p.q, p.k, p.v, p.do,
                                                           cu_seqlens=None if cu is None else cu.numpy(), **okw)
        ref = dict(o=ro, lse=rlse, dq=rdq, dk=rdk, dv=rdv)
        ins = dict(q=g(p.q), k=g(p.k), v=g(p.v), do=g(p.do))
    else:
        # padded: the oracle on the valid prefixes, packed with their own prefix sums
        uq, uk = used
        cq = np.concatenate([[0], np.cumsum(uq)]).astype(np.int32)
        ck = np.concatenate([[0], np.cumsum(uk)]).astype(np.int32)
        cat = lambda x, u: np.concatenate([x[b, :u[b]].double().numpy() for b in range(p.batch)])
        ins = dict(q=cat(p.q, uq), k=cat(p.k, uk), v=cat(p.v, uk), do=cat(p.do, uq))
        rdq, rdk, rdv, ro, rlse = oracle_mod.attention_bwd(ins["q"], ins["k"], ins["v"], ins["do"],
                                                           cu_seqlens=cq, cu_seqlens_k=ck, **okw)
        for b in range(p.batch):  # padded rows as the definition fixes them
            assert np.all(got["o"][b, uq[b]:] == 0) and np.all(np.isneginf(got["lse"][b, :, uq[b]:]))
            assert np.all(got["dq"][b, uq[b]:] == 0)
            assert np.all(got["dk"][b, uk[b]:] == 0) and np.all(got["dv"][b, uk[b]:] == 0)
        pk = lambda x, u: np.concatenate([x[b, :u[b]] for b in range(p.batch)])
        got = dict(o=pk(got["o"], uq), lse=np.concatenate([got["lse"][b, :, :uq[b]] for b in range(p.batch)], axis=1),
                   dq=pk(got["dq"], uq), dk=pk(got["dk"], uk), dv=pk(got["dv"], uk))
        ref = dict(o=ro, lse=rlse, dq=rdq, dk=rdk, dv=rdv)
    eo = float(np.abs(got["o"] - ref["o"]).max()) if ref["o"].size else 0.0
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isneginf(got["lse"]), np.isneginf(ref["lse"]))
    el = float(np.abs(got["lse"][fin] - ref["lse"][fin]).max()) if fin.any() else 0.0
    errs = {n: rel_l2(got[n], ref[n]) for n in ("dq", "dk", "dv") if np.linalg.norm(ref[n]) > 0}
    say(f"  O {eo:.2e} LSE {el:.2e} " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    assert eo <= O_TOL[p.dtype] and el <= LSE_TOL
    for n, e in errs.items():
        assert e <= GRAD_TOL, n
    for n in ("dq", "dk", "dv"):
        if np.linalg.norm(ref[n]) > 0:
            continue
        if n == "dv" or not fin.any():
            # no kept probability / no visible pair: the kernels write exact zeros
            assert np.all(got[n] == 0), n
        else:
            # visible pairs whose terms cancel exactly (every visible row sees one
            # key, so dS = P (dP - D) = 0): rounding only, within the bound below
            assert np.linalg.norm(got[n]) <= cancel_bound(ins, ref["o"], p.scale, drop, oracle_mod)[n], n


def draw_decode(seed):
    r = np.random.default_rng(5000 + seed)
    kv = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 4, 8, 16]))
    cap = int(r.integers(1, 2000))
    batch = int(r.integers(1, 5))
    cfg = dict(dtype=str(r.choice(["fp16", "bf16"])), batch=batch, heads=g * kv, kv_heads=kv,
               seqlen_q=int(r.choice([1, 2, 5, 8, 16, 33])), capacity=cap,
               head_dim=int(r.choice([8, 64, 80, 128, 200, 256])), causal=bool(r.integers(0, 2)),
               cache_lens=[int(x) for x in r.integers(0, cap + 1, batch)])
    if r.random() < 0.3:
        cfg["window"] = (int(r.integers(0, 300)), int(r.integers(0, 10)) if r.random() < 0.5 else -1)
    return cfg, int(r.choice([0, 0, 1, 3]))


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(fa, oracle_mod, seed):
    cfg, splits = draw_decode(seed)
    say(f"[random decode {seed}] splits={splits} {cfg}")
    p = synth.make_decode(seed=60 + seed, **cfg)
    dev = torch.device("cuda:0")
    o, lse = fa.forward_kvcache(p.q.to(dev), p.k_cache.to(dev), p.v_cache.to(dev), p.cache_seqlens().to(dev),
                                causal=p.causal, window_size=(p.window_left, p.window_right),
                                softmax_scale=p.scale, num_splits=splits)
    torch.cuda.synchronize()
    go, gl = o.float().cpu().double().numpy(), lse.cpu().double().numpy()
    eo = el = 0.0
    for b in range(p.batch):  # the new tokens against each sequence's valid prefix, bottom-right aligned
        n = p.cache_lens[b]
        ro, rl = oracle_mod.attention_fwd(p.q[b:b + 1], p.k_cache[b:b + 1, :n], p.v_cache[b:b + 1, :n],
                                          scale=p.scale, causal=p.causal, window=(p.window_left, p.window_right))
        assert np.array_equal(np.isneginf(gl[b]), np.isneginf(rl[0]))
        eo = max(eo, float(np.abs(go[b] - ro[0]).max()))
        fin = np.isfinite(rl[0])
        if fin.any():
            el = max(el, float(np.abs(gl[b][fin] - rl[0][fin]).max()))
    say(f"  O {eo:.2e} LSE {el:.2e}")
    assert eo <= O_TOL[p.dtype] and el <= LSE_TOL


@pytest.mark.parametrize("dtype,head_dim,layout", [("bf16", 72, "fixed"), ("fp16", 128, "fixed"),
                                                   ("bf16", 256, "fixed"), ("bf16", 64, "varlen")])
def test_single_visible_key(fa, oracle_mod, dtype, head_dim, layout):
    """Causal with window (0, 7): every query sees only its own key.  P is then
    one-hot, so O = V and dV = dO exactly (P rounds to exactly 1; one head per
    kv head), LSE_i = scale q_i . k_i, and dS = P (dP - D) = 0: dQ and dK
    vanish up to rounding.  With O = V exactly, D_i and dP_ii are the same fp32
    dot product of 16-bit values summed in different orders, so
    |dS_ii| <= E_i = 8 d 2^-24 |dO_i| |V_i| (twice the worst-case summation
    error of each, times 2), |dQ_i| <= scale |K_i| E_i and |dK_i| <= scale |Q_i| E_i."""
    cfg = dict(dtype=dtype, head_dim=head_dim, heads=3, kv_heads=3, causal=True, window=(0, 7))
    if layout == "varlen":
        cfg.update(batch=0, seqlen=0, seqlens=[1, 130, 67])
    else:
        cfg.update(batch=2, seqlen=150)
    p = synth.make_problem(seed=91, **cfg)
    say(f"[single key] {layout} {cfg}")
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    cu = p.cu_seqlens()
    kw = dict(causal=True, window_size=(0, 7), softmax_scale=p.scale)
    if cu is not None:
        cud = cu.to(dev)
        kw.update(cu_seqlens_q=cud, cu_seqlens_k=cud, max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    o, lse = fa.forward(q, k, v, **kw)
    dq, dk, dv = fa.backward(do, q, k, v, o, lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), p.v) and torch.equal(dv.cpu(), p.do)
    g = lambda t: t.float().cpu().double().numpy()
    qd, kd = g(p.q), g(p.k)
    lse_ref = p.scale * np.einsum("...hd,...hd->...h", qd, kd)  # [tokens..., heads]
    got_lse = lse.cpu().double().numpy()
    got_lse = np.moveaxis(got_lse, -2, -1) if cu is None else got_lse.T  # to [..., tokens, heads]
    assert np.abs(got_lse - lse_ref).max() <= LSE_TOL
    rn = lambda x: np.linalg.norm(x, axis=-1)  # per (token, head)
    e = 8 * p.head_dim * 2.0 ** -24 * rn(g(p.do)) * rn(g(p.v))
    bq, bk = p.scale * rn(kd) * e, p.scale * rn(qd) * e
    gq, gk = rn(g(dq)), rn(g(dk))
    say(f"  max |dQ_i| / bound {np.max(gq / bq):.2e}, max |dK_i| / bound {np.max(gk / bk):.2e}")
    assert np.all(gq <= bq) and np.all(gk <= bk)


def test_many_heads_wide_rows(fa, oracle_mod):
    """2048 query heads over 512 kv heads at head_dim 256: a token row is 1 MiB
    of queries, so the direct loads of a tile reach tens of MiB past its base
    (32-bit offsets).  130 tokens span several tiles with a ragged tail; the
    oracle checks the first and the last kv-head group (4 query heads each,
    complete GQA groups, so their dK and dV are fully determined)."""
    p = synth.make_problem(dtype="bf16", batch=1, heads=2048, kv_heads=512, seqlen=130, head_dim=256,
                           causal=True, seed=17)
    say("[many heads] bf16 b1 h2048 kv512 n130 d256 causal")
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    o, lse = fa.forward(q, k, v, causal=True, softmax_scale=p.scale)
    dq, dk, dv = fa.backward(do, q, k, v, o, lse, causal=True, softmax_scale=p.scale)
    torch.cuda.synchronize()
    g = lambda t: t.float().cpu().double().numpy()
    for hs, ks in ((slice(0, 4), slice(0, 1)), (slice(2044, 2048), slice(511, 512))):
        rdq, rdk, rdv, ro, rlse = oracle_mod.attention_bwd(p.q[:, :, hs], p.k[:, :, ks], p.v[:, :, ks],
                                                           p.do[:, :, hs], scale=p.scale, causal=True, threads=16)
        eo = float(np.abs(g(o[:, :, hs]) - ro).max())
        el = float(np.abs(lse[:, hs].cpu().double().numpy() - rlse).max())
        errs = {n: rel_l2(g(x), r) for n, x, r in (("dq", dq[:, :, hs], rdq), ("dk", dk[:, :, ks], rdk),
                                                   ("dv", dv[:, :, ks], rdv))}
        say(f"  heads {hs.start}..{hs.stop - 1}: O {eo:.2e} LSE {el:.2e} " +
            " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
        assert eo <= O_TOL["bf16"] and el <= LSE_TOL and all(e <= GRAD_TOL for e in errs.values())
