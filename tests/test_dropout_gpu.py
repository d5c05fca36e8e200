"""Dropout on the GPU (fa_fwd / fa_bwd with dropout_p > 0) against the fp64
oracle's dropout, which draws the same Philox4x32-10 keep decisions from its
own implementation.

* The keep mask itself is compared bit for bit: with V the identity (Nk = d),
  O_ij = P_ij M_ij s, so the zero pattern of O is the mask.
* Forward and backward are compared element by element on small cases
  (tolerances as without dropout: O max-abs 4e-3 fp16 / 2e-2 bf16, LSE
  max-abs 1e-3, dQ/dK/dV relative L2 2e-2), and on sampled rows of the 8K
  workload at full size.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synth

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


def kw_of(p, drop, seed):
    cu = p.cu_seqlens()
    return dict(scale=p.scale, causal=p.causal, window=(p.window_left, p.window_right),
                cu_seqlens=None if cu is None else cu.numpy(), dropout_p=drop, seed=seed)


def gpu_run(fa, p, drop, seed, with_bwd=True):
    dev = torch.device("cuda:0")
    q, k, v = p.q.to(dev), p.k.to(dev), p.v.to(dev)
    cu = p.cu_seqlens()
    cu = cu.to(dev) if cu is not None else None
    kw = dict(causal=p.causal, window_size=(p.window_left, p.window_right), softmax_scale=p.scale,
              cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k,
              dropout_p=drop, dropout_seed=seed)
    o, lse = fa.forward(q, k, v, **kw)
    res = dict(o=o, lse=lse)
    if with_bwd:
        res.update(zip(("dq", "dk", "dv"), fa.backward(p.do.to(dev), q, k, v, o, lse, **kw)))
    torch.cuda.synchronize()
    return {n: t.float().cpu().double().numpy() for n, t in res.items()}


def rel_l2(a, b):
    m = ~np.isnan(b)
    return float(np.linalg.norm(a[m] - b[m]) / max(np.linalg.norm(b[m]), 1e-30))


def max_abs(a, b):
    m = ~np.isnan(b)
    return float(np.abs(a[m] - b[m]).max())


@pytest.mark.parametrize("d,dtype,p,seed", [(64, "fp16", 0.3, 1), (128, "bf16", 0.5, 2**63 + 12345),
                                            (64, "bf16", 0.1, 7), (128, "fp16", 0.85, 99)])
def test_mask_matches_oracle_bit_for_bit(fa, oracle_mod, d, dtype, p, seed):
    """Nk = d keys, V = I: O_ij is P_ij * 256/T where kept and exactly 0 where
    dropped (causal: also 0 above the diagonal)."""
    say(f"[dropout mask] d={d} {dtype} p={p}")
    h, n = 3, d
    prob = synth.make_problem(dtype=dtype, batch=2, heads=h, kv_heads=h, seqlen=n, head_dim=d,
                              causal=True, seed=4, with_do=False)
    eye = torch.eye(d, dtype=prob.q.dtype)
    prob.v = eye[None, :, None, :].expand(2, n, h, d).contiguous()
    g = gpu_run(fa, prob, p, seed, with_bwd=False)
    mask = oracle_mod.dropout_mask(2, h, n, n, p, seed)
    vis = np.tril(np.ones((n, n), dtype=bool))
    want = mask.astype(bool) & vis[None, None]
    got = np.transpose(g["o"], (0, 2, 1, 3)) != 0  # (b, h, i, j)
    bad = int((got != want).sum())
    say(f"  {bad} of {want.size} keep decisions differ; kept {want.mean():.3f}")
    assert bad == 0


SMALL = {
    "causal_bf16_d64_gqa": (dict(dtype="bf16", batch=2, heads=4, kv_heads=2, seqlen=300, head_dim=64, causal=True), 0.2),
    "causal_bf16_d128": (dict(dtype="bf16", batch=1, heads=4, kv_heads=4, seqlen=530, head_dim=128, causal=True,
                              factor=0.5), 0.1),
    "noncausal_fp16_d128_gqa4": (dict(dtype="fp16", batch=2, heads=8, kv_heads=2, seqlen=200, head_dim=128,
                                      causal=False), 0.5),
    "window_fp16_d64": (dict(dtype="fp16", batch=1, heads=2, kv_heads=2, seqlen=400, head_dim=64, causal=True,
                             window=(100, 0)), 0.3),
    "varlen_causal_fp16_d128": (dict(dtype="fp16", batch=0, heads=4, kv_heads=2, seqlen=0, head_dim=128, causal=True,
                                     seqlens=[1, 63, 65, 257, 0, 300]), 0.25),
    "q_shorter_than_k_bf16_d64": (dict(dtype="bf16", batch=2, heads=2, kv_heads=1, seqlen=150, seqlen_k=333,
                                       head_dim=64, causal=True), 0.4),
    "gqa_groups_on_one_xcd_bf16_d128": (dict(dtype="bf16", batch=2, heads=12, kv_heads=4, seqlen=160, head_dim=128,
                                             causal=True), 0.3),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_dropout_parity(fa, oracle_mod, name):
    kwargs, drop = SMALL[name]
    say(f"[dropout parity] {name} p={drop}")
    p = synth.make_problem(seed=9, **kwargs)
    seed = 0xC0FFEE + len(name)
    g = gpu_run(fa, p, drop, seed)
    dq, dk, dv, o, lse = oracle_mod.attention_bwd(p.q, p.k, p.v, p.do, **kw_of(p, drop, seed))
    eo = max_abs(g["o"], o)
    fin = np.isfinite(lse)
    el = float(np.abs(g["lse"][fin] - lse[fin]).max()) if fin.any() else 0.0
    assert np.all(np.isneginf(g["lse"][~fin]))
    errs = {n: rel_l2(g[n], r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv))}
    say(f"  O {eo:.2e} LSE {el:.2e} " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    assert eo <= O_TOL[p.dtype] and el <= LSE_TOL
    for e in errs.values():
        assert e <= GRAD_TOL


def test_zero_probability_runs_the_plain_kernels(fa):
    p = synth.make_problem(seed=2, **SMALL["causal_bf16_d64_gqa"][0])
    a = gpu_run(fa, p, 0.0, 0)
    b = gpu_run(fa, p, 0.0, 12345)
    for n in a:
        assert np.array_equal(a[n], b[n], equal_nan=True), n


def test_seed_decides_the_mask(fa):
    p = synth.make_problem(seed=2, **SMALL["causal_bf16_d128"][0])
    a = gpu_run(fa, p, 0.3, 5, with_bwd=False)
    b = gpu_run(fa, p, 0.3, 5, with_bwd=False)
    c = gpu_run(fa, p, 0.3, 6, with_bwd=False)
    assert np.array_equal(a["o"], b["o"])
    assert not np.array_equal(a["o"], c["o"])
    assert np.array_equal(a["lse"], c["lse"])  # LSE is that of the undropped softmax


def test_autograd_backward_reuses_the_forward_seed(fa):
    dev = torch.device("cuda:0")
    p = synth.make_problem(seed=3, **SMALL["causal_bf16_d64_gqa"][0])
    q, k, v = (t.to(dev).requires_grad_() for t in (p.q, p.k, p.v))
    do = p.do.to(dev)
    out = fa.flash_attn_func(q, k, v, dropout_p=0.2, causal=True, dropout_seed=77)
    out.backward(do)
    torch.cuda.synchronize()
    o2, lse2 = fa.forward(q.detach(), k.detach(), v.detach(), causal=True, dropout_p=0.2, dropout_seed=77)
    dq2, dk2, dv2 = fa.backward(do, q.detach(), k.detach(), v.detach(), o2, lse2, causal=True,
                                dropout_p=0.2, dropout_seed=77)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o2)
    assert torch.equal(q.grad, dq2) and torch.equal(k.grad, dk2) and torch.equal(v.grad, dv2)


def test_full_size_workload_sampled(fa, oracle_mod):
    """The 8K workload with dropout 0.1, in the benchmark's launch shapes;
    sampled query rows (O, LSE, dQ) and key rows of two kv heads (dK, dV)."""
    name = "bf16_causal_b1_h32_n8192_d128"
    say(f"[dropout full size] {name}")
    p = synth.workload(name)
    drop, seed = 0.1, 2024
    g = gpu_run(fa, p, drop, seed)
    rows = np.array([0, 1, 777, 4095, 4096, 8000, 8191])
    kv_heads = np.array([3, 30])
    dq, dk, dv, o, lse = oracle_mod.attention_bwd(p.q, p.k, p.v, p.do, q_rows=rows, k_rows=rows,
                                                  kv_heads=kv_heads, threads=16, **kw_of(p, drop, seed))
    heads = kv_heads  # MHA: query head = kv head
    go, ro = g["o"][:, rows][:, :, heads], o[:, rows][:, :, heads]
    eo = max_abs(go, ro)
    el = float(np.abs(g["lse"][:, heads][:, :, rows] - lse[:, heads][:, :, rows]).max())
    e = {n: rel_l2(g[n][:, rows][:, :, heads], r[:, rows][:, :, heads]) for n, r in (("dq", dq), ("dk", dk), ("dv", dv))}
    say(f"  O {eo:.2e} LSE {el:.2e} " + " ".join(f"{n} {x:.2e}" for n, x in e.items()))
    assert eo <= O_TOL["bf16"] and el <= LSE_TOL
    for x in e.values():
        assert x <= GRAD_TOL
