"""Parity of the HIP path (through the C-ABI) with the fp64 CPU oracle.

Small problems spanning several tiles with ragged tails are compared in
full; the five named workloads are run at full size in the same launch
configuration the benchmark times, and compared on sampled rows and key rows
that the oracle evaluates one by one.  Tolerances: O max-abs 4e-3 (fp16) /
2e-2 (bf16), LSE max-abs 1e-3, dQ/dK/dV relative L2 2e-2.
"""
import math
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


def gpu_run(fa, p, with_bwd=True, deterministic=True):
    dev = torch.device("cuda:0")
    q, k, v = p.q.to(dev), p.k.to(dev), p.v.to(dev)
    cu = p.cu_seqlens()
    cu = cu.to(dev) if cu is not None else None
    kw = dict(causal=p.causal, window_size=(p.window_left, p.window_right), softmax_scale=p.scale,
              cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    o, lse = fa.forward(q, k, v, **kw)
    res = dict(o=o, lse=lse)
    if with_bwd:
        dq, dk, dv = fa.backward(p.do.to(dev), q, k, v, o, lse, deterministic=deterministic, **kw)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.float().cpu().double().numpy() for n, t in res.items()}


def okw(p):
    cu = p.cu_seqlens()
    return dict(scale=p.scale, causal=p.causal, window=(p.window_left, p.window_right),
                cu_seqlens=None if cu is None else cu.numpy())


def max_abs(a, b):
    m = ~np.isnan(b)
    assert m.any()
    return float(np.abs(a[m] - b[m]).max())


def rel_l2(a, b):
    """Relative L2 error (None where the exact gradient vanishes: the
    reference then holds only fp64 rounding noise, and grad_ok bounds the
    GPU result by its own rounding instead)."""
    m = ~np.isnan(b)
    assert m.any()
    den = np.linalg.norm(b[m])
    num = np.linalg.norm(a[m] - b[m])
    if den < 1e-9 * math.sqrt(m.sum()):
        return None
    return float(num / den)


def grad_errors(p, g, ref, o_ref):
    """Relative L2 of dQ, dK, dV against the oracle.  A gradient that vanishes
    exactly (self-only windows: every visible row sees one key, so
    dS = P (dP - D) = 0 and dQ = dK = 0) must instead stay within the
    propagated rounding bound on its norm (tests/_bounds.py)."""
    import oracle
    ins = {n: getattr(p, n).double().numpy() for n in ("q", "k", "v", "do")}
    errs = {}
    for n, r in (("dq", ref[0]), ("dk", ref[1]), ("dv", ref[2])):
        e = rel_l2(g[n], r)
        if e is None:
            bound = cancel_bound(ins, o_ref, p.scale, 0.0, oracle)[n]
            nrm = float(np.linalg.norm(g[n]))
            assert nrm <= bound, (n, nrm, bound)
            e = 0.0
        errs[n] = e
    return errs


def check_lse(g, r):
    m = ~np.isnan(r)
    fin = m & np.isfinite(r)
    ninf = m & np.isneginf(r)
    assert np.all(np.isneginf(g[ninf])), "rows without keys must give LSE = -inf"
    if fin.any():
        err = float(np.abs(g[fin] - r[fin]).max())
        assert err <= LSE_TOL, f"LSE max-abs {err}"
        return err
    return 0.0


def compare_full(fa, p, with_bwd=True, deterministic=True):
    g = gpu_run(fa, p, with_bwd, deterministic)
    import oracle
    if with_bwd:
        dq, dk, dv, o, lse = oracle.attention_bwd(p.q, p.k, p.v, p.do, **okw(p))
    else:
        o, lse = oracle.attention_fwd(p.q, p.k, p.v, **okw(p))
    eo = max_abs(g["o"], o)
    el = check_lse(g["lse"], lse)
    msg = f"O {eo:.2e} LSE {el:.2e}"
    assert eo <= O_TOL[p.dtype], msg
    if with_bwd:
        errs = grad_errors(p, g, (dq, dk, dv), o)
        msg += " " + " ".join(f"{n} {e:.2e}" for n, e in errs.items())
        for n, e in errs.items():
            assert e <= GRAD_TOL, msg
    say(msg)
    return g


SMALL = {
    # id: make_problem kwargs
    "noncausal_fp16_d64_ragged": dict(dtype="fp16", batch=2, heads=3, kv_heads=3, seqlen=300, head_dim=64, causal=False),
    "causal_bf16_d64_gqa": dict(dtype="bf16", batch=2, heads=4, kv_heads=2, seqlen=300, head_dim=64, causal=True),
    "causal_bf16_d128": dict(dtype="bf16", batch=1, heads=4, kv_heads=4, seqlen=530, head_dim=128, causal=True, factor=0.5),
    "noncausal_fp16_d128_gqa4": dict(dtype="fp16", batch=2, heads=8, kv_heads=2, seqlen=200, head_dim=128, causal=False),
    "window_fp16_d128": dict(dtype="fp16", batch=1, heads=2, kv_heads=2, seqlen=700, head_dim=128, causal=True, window=(100, 0)),
    "window_two_sided_bf16_d64": dict(dtype="bf16", batch=1, heads=2, kv_heads=1, seqlen=400, head_dim=64, causal=False, window=(37, 53)),
    "self_only_window_fp16_d64": dict(dtype="fp16", batch=1, heads=2, kv_heads=2, seqlen=130, head_dim=64, causal=False, window=(0, 0)),
    "causal_q_shorter_than_k_bf16_d128": dict(dtype="bf16", batch=2, heads=2, kv_heads=2, seqlen=150, seqlen_k=333, head_dim=128, causal=True),
    "causal_q_longer_than_k_fp16_d64": dict(dtype="fp16", batch=1, heads=2, kv_heads=2, seqlen=333, seqlen_k=150, head_dim=64, causal=True),
    "noncausal_q_longer_than_k_bf16_d64": dict(dtype="bf16", batch=1, heads=2, kv_heads=1, seqlen=300, seqlen_k=70, head_dim=64, causal=False),
    "varlen_causal_window_fp16_d128": dict(dtype="fp16", batch=0, heads=4, kv_heads=2, seqlen=0, head_dim=128, causal=True,
                                           window=(200, 0), seqlens=[1, 63, 64, 65, 255, 256, 257, 0, 500]),
    "varlen_noncausal_bf16_d64": dict(dtype="bf16", batch=0, heads=2, kv_heads=2, seqlen=0, head_dim=64, causal=False,
                                      seqlens=[17, 300, 129]),
    "single_token_bf16_d128": dict(dtype="bf16", batch=3, heads=2, kv_heads=1, seqlen=1, head_dim=128, causal=True),
    "zero_scale_causal_fp16_d64": dict(dtype="fp16", batch=1, heads=2, kv_heads=2, seqlen=200, head_dim=64, causal=True, scale=0.0),
    "large_scores_bf16_d128": dict(dtype="bf16", batch=1, heads=2, kv_heads=2, seqlen=260, head_dim=128, causal=True, scale=0.8),
    # batch * kv_heads a multiple of 8: the grids place each GQA group's query heads on one XCD
    "gqa_groups_on_one_xcd_bf16_d128": dict(dtype="bf16", batch=2, heads=16, kv_heads=4, seqlen=270, head_dim=128,
                                            causal=True),
    "gqa_groups_on_one_xcd_varlen_fp16_d64": dict(dtype="fp16", batch=0, heads=6, kv_heads=2, seqlen=0, head_dim=64,
                                                  causal=False, seqlens=[40, 1, 130, 0]),
}


@pytest.mark.parametrize("det", [False, True], ids=["atomic_dq", "dq_pass"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(fa, name, det):
    say(f"[parity] {name} deterministic={det}")
    p = synth.make_problem(seed=7, **SMALL[name])
    compare_full(fa, p, deterministic=det)


@pytest.mark.parametrize("det", [False, True], ids=["atomic_dq", "dq_pass"])
def test_masked_key_far_above_visible(fa, det):
    """A key hidden by the causal mask from most rows, whose score lies far
    above everything those rows can see: every query is 2.0 in every
    component and key 150 is 40.0 in every component (exact in bf16), so at
    d = 64 and scale 1/8 its score is 640 against visible scores of a few
    units.  Rows before 150 share edge tiles with it in the backward, where
    its probability is recomputed from their LSE: exp2 of about 900 overflows
    fp32 unless the recomputed probability is clamped, and inf * 0 would
    follow before the mask removes it.  Rows from 150 on see the key and put
    almost all their weight on it."""
    say(f"[parity] masked key far above visible deterministic={det}")
    p = synth.make_problem(seed=11, dtype="bf16", batch=1, heads=2, kv_heads=1, seqlen=200, head_dim=64, causal=True)
    p.q.fill_(2.0)
    p.k[:, 150] = 40.0
    g = compare_full(fa, p, deterministic=det)
    for n, t in g.items():
        assert np.isfinite(t[~np.isneginf(t)]).all(), n


@pytest.mark.parametrize("name", ["causal_bf16_d64_gqa", "causal_bf16_d128", "varlen_causal_window_fp16_d128"])
def test_repeatable_bytes(fa, name):
    """The deterministic path (separate dQ pass, no atomics): two runs on the
    same inputs give identical bytes.  The atomic path: dK, dV identical
    (they never use atomics), dQ equal up to the order of its float32
    additions."""
    p = synth.make_problem(seed=3, **SMALL[name])
    a = gpu_run(fa, p, deterministic=True)
    b = gpu_run(fa, p, deterministic=True)
    for n in a:
        assert np.array_equal(a[n], b[n], equal_nan=True), n
    c = gpu_run(fa, p, deterministic=False)
    for n in ("o", "lse", "dk", "dv"):
        assert np.array_equal(a[n], c[n], equal_nan=True), n
    den = np.linalg.norm(a["dq"])
    assert np.linalg.norm(c["dq"] - a["dq"]) <= 1e-2 * den, "atomic dQ against the dQ pass"


def test_outputs_stay_inside_their_buffers(fa):
    """Guard bands around every output of a packed call stay untouched."""
    p = synth.make_problem(seed=5, **SMALL["varlen_causal_window_fp16_d128"])
    dev = torch.device("cuda:0")
    pad = 4096
    def padded(like, dtype=None):
        dtype = dtype or like.dtype
        buf = torch.full((like.numel() + 2 * pad,), 7.0, dtype=dtype, device=dev)
        return buf, buf[pad:pad + like.numel()].view(like.shape)
    q, k, v, do = p.q.to(dev), p.k.to(dev), p.v.to(dev), p.do.to(dev)
    cu = p.cu_seqlens().to(dev)
    ob, o = padded(q)
    lb, lse = padded(torch.empty(p.heads, q.shape[0]), torch.float32)
    kw = dict(causal=True, window_size=(200, 0), softmax_scale=p.scale, cu_seqlens_q=cu, cu_seqlens_k=cu,
              max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    fa.forward(q, k, v, out=o, lse=lse, **kw)
    dqb, dq = padded(q)
    dkb, dk = padded(k)
    dvb, dv = padded(v)
    fa.backward(do, q, k, v, o, lse, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    for buf in (ob, lb, dqb, dkb, dvb):
        assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0)


def test_empty_inputs(fa):
    dev = torch.device("cuda:0")
    # no keys at all: O = 0, LSE = -inf, dQ = 0
    q = torch.randn(1, 40, 2, 64, device=dev, dtype=torch.float16)
    k = torch.empty(1, 0, 2, 64, device=dev, dtype=torch.float16)
    o, lse = fa.forward(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    dq, dk, dv = fa.backward(torch.randn_like(q), q, k, k, o, lse)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
    # no queries: dK = dV = 0
    q0 = torch.empty(1, 0, 2, 64, device=dev, dtype=torch.bfloat16)
    k1 = torch.randn(1, 33, 2, 64, device=dev, dtype=torch.bfloat16)
    o0, l0 = fa.forward(q0, k1, k1, causal=True)
    dq0, dk1, dv1 = fa.backward(o0, q0, k1, k1, o0, l0, causal=True)
    torch.cuda.synchronize()
    assert torch.all(dk1 == 0) and torch.all(dv1 == 0)
    # empty batch
    qb = torch.empty(0, 16, 2, 128, device=dev, dtype=torch.bfloat16)
    ob, lb = fa.forward(qb, qb, qb)
    torch.cuda.synchronize()
    assert ob.numel() == 0


def test_autograd_entry(fa):
    p = synth.make_problem(seed=11, dtype="bf16", batch=1, heads=2, kv_heads=2, seqlen=96, head_dim=64, causal=True)
    dev = torch.device("cuda:0")
    q = p.q.to(dev).requires_grad_()
    k = p.k.to(dev).requires_grad_()
    v = p.v.to(dev).requires_grad_()
    out = fa.flash_attn_func(q, k, v, causal=True)
    out.backward(p.do.to(dev))
    torch.cuda.synchronize()
    import oracle
    dq, dk, dv, o, _ = oracle.attention_bwd(p.q, p.k, p.v, p.do, **okw(p))
    assert max_abs(out.detach().double().cpu().numpy(), o) <= O_TOL["bf16"]
    for g, r in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert rel_l2(g.double().cpu().numpy(), r) <= GRAD_TOL


# ---------------------------------------------------------------------------
# Full-size workloads, sampled.
# ---------------------------------------------------------------------------
def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, n // 2, n - 2, n - 1]
    rest = rng.choice(n, size=min(n, count), replace=False)
    return np.unique(np.clip(np.concatenate([fixed, rest]), 0, n - 1)).astype(np.int32)


FULL = {
    # workload: (query heads to check, kv heads for dK/dV, dK/dV key rows)
    "fp16_noncausal_b1_h2_n128_d64": None,  # small enough to compare in full
    "bf16_causal_b4_h16_n2048_d64": dict(heads=[0, 9], kv_heads=[3], krows="all"),
    "bf16_causal_b1_h32_n8192_d128": dict(heads=[0, 17, 31], kv_heads=[5], krows="spread"),
    "bf16_causal_gqa_b1_h32kv8_n32768_d128": dict(heads=[0, 13, 30], kv_heads=[6], krows="tail"),
    "fp16_causal_window4096_varlen_b2_h16_d128": dict(heads=[2, 15], kv_heads=[8], krows="window"),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_workload(fa, name):
    say(f"[parity-full] {name}: generating inputs")
    p = synth.workload(name)
    spec = FULL[name]
    if spec is None:
        compare_full(fa, p, with_bwd=True)
        return
    say(f"[parity-full] {name}: GPU forward+backward")
    g = gpu_run(fa, p)
    import oracle
    n = p.seqlen_q
    rows = sample_rows(n, 48, 1)
    say(f"[parity-full] {name}: oracle forward on {len(rows)} rows x {len(spec['heads'])} heads")
    o, lse = oracle.attention_fwd(p.q, p.k, p.v, rows=rows, heads=spec["heads"], **okw(p))
    eo = max_abs(g["o"], o)
    el = check_lse(g["lse"], lse)
    assert eo <= O_TOL[p.dtype], f"O max-abs {eo}"
    # backward: dQ on sampled rows of the checked kv heads' groups, dK/dV on key rows
    if spec["krows"] == "all":
        krows = None
    elif spec["krows"] == "spread":
        krows = np.concatenate([np.arange(0, 32), np.arange(n // 2, n // 2 + 32), np.arange(n - 64, n)])
    elif spec["krows"] == "tail":
        # the first keys (the longest accumulations: every row of all the group's
        # heads), a block mid-sequence and the tail
        krows = np.concatenate([np.arange(0, 64), np.arange(n // 2, n // 2 + 64), np.arange(n - 600, n - 536),
                                np.arange(n - 64, n)])
    else:  # sliding window: a block of keys mid-sequence and the tail of the shortest sequence
        m = min(p.seqlens)
        krows = np.concatenate([np.arange(m // 2, m // 2 + 64), np.arange(m - 64, m)])
    qrows = sample_rows(n, 24, 2)
    say(f"[parity-full] {name}: oracle backward")
    dq, dk, dv, _, _ = oracle.attention_bwd(p.q, p.k, p.v, p.do, q_rows=qrows,
                                            k_rows=None if krows is None else krows.astype(np.int32),
                                            kv_heads=spec["kv_heads"], **okw(p))
    errs = {nm: rel_l2(g[nm], r) for nm, r in (("dq", dq), ("dk", dk), ("dv", dv))}
    assert all(e is not None for e in errs.values()), errs
    say(f"[parity-full] {name}: O {eo:.2e} LSE {el:.2e} " + " ".join(f"{a} {b:.2e}" for a, b in errs.items()))
    for nm, e in errs.items():
        assert e <= GRAD_TOL, (nm, e)
    # properties that hold at any size: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per kv head
    dkg = torch.from_numpy(g["dk"])
    dvg = torch.from_numpy(g["dv"])
    do = p.do.double()
    grp = p.heads // p.kv_heads
    if p.varlen:
        cu = p.cu_seqlens().tolist()
        for b in range(p.batch):
            sl = slice(cu[b], cu[b + 1])
            sdk = dkg[sl].sum(0)
            sdv = dvg[sl].sum(0)
            want = do[sl].reshape(-1, p.kv_heads, grp, p.head_dim).sum((0, 2))
            assert float((sdv - want).norm() / want.norm()) <= GRAD_TOL
            assert float(sdk.abs().max()) <= 1e-2 * float(dkg[sl].abs().max()) * math.sqrt(sl.stop - sl.start)
    else:
        sdv = dvg.sum(1)
        want = do.reshape(p.batch, p.seqlen_q, p.kv_heads, grp, p.head_dim).sum((1, 3))
        assert float((sdv - want).norm() / want.norm()) <= GRAD_TOL
        # sum_j dS_ij = 0 for every row, so sum_j dK_j = 0 per (batch, kv head, column)
        sdk = dkg.sum(1)
        assert float(sdk.abs().max()) <= 1e-2 * float(dkg.abs().max()) * math.sqrt(p.seqlen_k)


def test_long_sequence_131072(fa):
    """One 131072-token sequence (bf16, causal, 4 query heads over 2 kv heads,
    d = 64): tile counts, row offsets and LSE indices four times past the
    largest named workload.  The oracle checks the forward and dQ on sampled
    rows and dK/dV on the last 64 keys (the only rows that see them are the
    last ones, so the oracle's work stays small); every key's dK and dV enter
    the invariants sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per kv head."""
    say("[parity-long] 131072 tokens: generating inputs")
    p = synth.make_problem(seed=21, dtype="bf16", batch=1, heads=4, kv_heads=2, seqlen=131072, head_dim=64,
                           causal=True)
    say("[parity-long] GPU forward+backward")
    g = gpu_run(fa, p)
    import oracle
    n = p.seqlen_q
    rows = sample_rows(n, 24, 3)
    say("[parity-long] oracle forward on sampled rows")
    o, lse = oracle.attention_fwd(p.q, p.k, p.v, rows=rows, heads=[0, 3], **okw(p))
    eo = max_abs(g["o"], o)
    el = check_lse(g["lse"], lse)
    assert eo <= O_TOL[p.dtype], f"O max-abs {eo}"
    qrows = sample_rows(n, 16, 4)
    krows = np.arange(n - 64, n).astype(np.int32)
    say("[parity-long] oracle backward on sampled rows and the last 64 keys")
    dq, dk, dv, _, _ = oracle.attention_bwd(p.q, p.k, p.v, p.do, q_rows=qrows, k_rows=krows, kv_heads=[1], **okw(p))
    errs = {nm: rel_l2(g[nm], r) for nm, r in (("dq", dq), ("dk", dk), ("dv", dv))}
    assert all(e is not None for e in errs.values()), errs
    say(f"[parity-long] O {eo:.2e} LSE {el:.2e} " + " ".join(f"{a} {b:.2e}" for a, b in errs.items()))
    for nm, e in errs.items():
        assert e <= GRAD_TOL, (nm, e)
    dkg = torch.from_numpy(g["dk"])
    dvg = torch.from_numpy(g["dv"])
    sdv = dvg.sum(1)
    want = p.do.double().reshape(1, n, 2, 2, 64).sum((1, 3))
    assert float((sdv - want).norm() / want.norm()) <= GRAD_TOL
    assert float(dkg.sum(1).abs().max()) <= 1e-2 * float(dkg.abs().max()) * math.sqrt(n)

