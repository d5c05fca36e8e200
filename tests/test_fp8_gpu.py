"""FP8 forward on the GPU (fa_fwd_fp8) against the fp64 oracle's attention of
the dequantised inputs (FlashAttention-2 overview page, lshu.cn/news/55956,
section 5.2: FP8 inputs in float8_e4m3fn).

The kernel rounds the probabilities to E4M3 before P.V, so its O is not the
exact attention: the tolerance is derived per element from that arithmetic
(the pages state none for FP8).  With P relative to the row's largest
probability (the kernel keeps p' = 2^4 P <= 256, inside E4M3's range),
round-to-nearest-even on 3 mantissa bits moves each P_ij by at most
2^-4 P_ij (normal range) or 2^-10 / 2^4 = 2^-14 (subnormal spacing 2^-9,
halved, over the 2^4 offset).  Summed against V and normalised by the
unrounded row sum:

    |O_ic - O*_ic| <= (2^-4 + 2^-12) A_ic + 2^-14 S_ic / L_i
                      + (e^(2 E_i) - 1) (A_ic + |O*_ic|) + u |O*_ic| + slack

    A_ic = sum_j P_ij |v_jc|          (the oracle on |V|)
    S_ic = sum over visible j of |v_jc|  (the oracle on |V| at scale 0, times
                                       the visible count e^LSE0)
    L_i  = sum_j exp(s_ij - max_j s_ij) = e^(LSE_i - max_j s_ij), max_j s_ij
           from above by the oracle's LSE at 10^4 times the scale, / 10^4
    E_i  = 2^-12 scale max_j sum_d |q_id k_jd|, the bound on the score error of
           the FP8 dot products (observed within 2^-14.7 of the sum of the
           products' magnitudes on gfx950), bounded the same way
    u    = 2^-8 (bf16 out) or 2^-11 (fp16 out), the output rounding
    2^-12 A: the P.V products' own accumulation error.

LSE uses the unrounded probabilities: |LSE - LSE*| <= 1e-3 + E_i.  A case
with V = I (as many keys as head_dim) makes each output column one key's
rounded probability, so any key placed in the wrong byte of an operand
shows at once.
"""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

TEMP = 1.0e4
U_OUT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


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


def dequant(oracle_mod, p):
    return (oracle_mod.fp8_e4m3_decode(p.q) * p.descale_q, oracle_mod.fp8_e4m3_decode(p.k) * p.descale_k,
            oracle_mod.fp8_e4m3_decode(p.v) * p.descale_v)


def reference_and_bound(oracle_mod, p, out_dtype, **sel):
    """Oracle O*, LSE* and the per-element bounds of the O and LSE errors."""
    q, k, v = dequant(oracle_mod, p)
    cu = p.cu_seqlens()
    kw = dict(causal=p.causal, window=(p.window_left, p.window_right),
              cu_seqlens=None if cu is None else cu.numpy(), threads=16, **sel)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale=p.scale, **kw)
    av = np.abs(v)
    a_, _ = oracle_mod.attention_fwd(q, k, av, scale=p.scale, **kw)
    mean0, lse0 = oracle_mod.attention_fwd(q, k, av, scale=0.0, **kw)
    _, lse_t = oracle_mod.attention_fwd(q, k, v, scale=p.scale * TEMP, **kw)
    _, lse_m = oracle_mod.attention_fwd(np.abs(q), np.abs(k), v, scale=p.scale * TEMP, **kw)
    smax = lse_t / TEMP                 # >= the row's largest score
    e = 2.0 ** -12 * (lse_m / TEMP)     # >= 2^-12 scale max_j sum_d |q_d k_d|
    with np.errstate(invalid="ignore"):
        L = np.exp(lse - smax)          # <= the true L (safe)
    # rows without a visible key (O = 0 exactly): no score error, L = 1
    e = np.where(np.isfinite(e), e, 0.0)
    L = np.where(np.isfinite(L) & (L > 0), L, 1.0)

    def per_row(x):  # (B, H, N) or packed (H, T) row quantities -> broadcast over O's layout
        if cu is None:
            return np.transpose(x, (0, 2, 1))[..., None]
        return np.transpose(x, (1, 0))[..., None]

    s_abs = mean0 * per_row(np.exp(lse0))
    Lr, er = per_row(L), per_row(e)
    fo = np.expm1(2.0 * er)
    bound = (2.0 ** -4 + 2.0 ** -12) * a_ + 2.0 ** -14 * s_abs / Lr + fo * (a_ + np.abs(o)) \
        + U_OUT[out_dtype] * np.abs(o)
    bound = bound * 1.01 + 1e-6 * np.nanmax(np.abs(o))
    lse_bound = 1e-3 + e
    return o, lse, bound, lse_bound


def run_gpu(fa, p, out_dtype=torch.bfloat16, used=None):
    dev = torch.device("cuda:0")
    q, k, v = p.q.to(dev), p.k.to(dev), p.v.to(dev)
    cu = p.cu_seqlens()
    cu = cu.to(dev) if cu is not None else None
    kw = dict(causal=p.causal, window_size=(p.window_left, p.window_right), softmax_scale=p.scale,
              cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=p.seqlen_q if cu is not None else None,
              max_seqlen_k=p.seqlen_k if cu is not None else None, out_dtype=out_dtype)
    if used is not None:
        kw.update(seqused_q=used[0], seqused_k=used[1])
    o, lse = fa.forward_fp8(q, k, v, p.descale_q, p.descale_k, p.descale_v, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def check(name, got_o, got_lse, o, lse, bound, lse_bound):
    m = ~np.isnan(o)
    err = np.abs(got_o - o)
    ratio = float(np.nanmax(np.where(m, err / bound, 0.0)))
    fin = np.isfinite(lse)
    assert np.array_equal(np.isneginf(got_lse[~np.isnan(lse)]), np.isneginf(lse[~np.isnan(lse)]))
    el = float(np.abs(got_lse[fin] - lse[fin]).max()) if fin.any() else 0.0
    lse_ok = bool(np.all(np.abs(got_lse[fin] - lse[fin]) <= lse_bound[fin])) if fin.any() else True
    rel = float(np.linalg.norm(err[m]) / max(np.linalg.norm(o[m]), 1e-30))
    say(f"  {name}: O err / bound max {ratio:.3f}, rel-L2 {rel:.3e}; LSE max err {el:.2e}")
    assert ratio <= 1.0, "O outside the derived bound"
    assert lse_ok, "LSE outside its bound"
    assert rel <= 0.06


@pytest.mark.parametrize("d,causal,heads,kv_heads", [(128, True, 4, 2), (128, False, 2, 2), (64, True, 2, 1),
                                                     (64, False, 3, 3), (80, True, 2, 2), (32, False, 2, 1)])
def test_identity_values_show_each_rounded_probability(fa, oracle_mod, d, causal, heads, kv_heads):
    """Nk = d keys and V = I: O_ic is key c's probability for query i."""
    say(f"[fp8 identity] d={d} causal={causal} heads={heads}/{kv_heads}")
    p = synth.make_problem(dtype="fp8", batch=2, heads=heads, kv_heads=kv_heads, seqlen=d, head_dim=d,
                           causal=causal, seed=41, scale=0.5 / np.sqrt(d))
    eye = torch.zeros(d, d, dtype=torch.uint8)
    eye[torch.arange(d), torch.arange(d)] = 0x38  # 1.0
    p.v = eye[None, :, None, :].expand(2, d, kv_heads, d).contiguous().view(torch.float8_e4m3fn)
    p.descale_v = 1.0
    got_o, got_lse = run_gpu(fa, p)
    o, lse, bound, lb = reference_and_bound(oracle_mod, p, torch.bfloat16)
    check("identity", got_o, got_lse, o, lse, bound, lb)


CASES = {
    "causal_d128_gqa_bf16": (dict(batch=2, heads=8, kv_heads=2, seqlen=530, head_dim=128, causal=True), torch.bfloat16),
    "noncausal_d64_fp16": (dict(batch=2, heads=4, kv_heads=4, seqlen=300, head_dim=64, causal=False), torch.float16),
    "window_d128": (dict(batch=1, heads=4, kv_heads=1, seqlen=700, head_dim=128, causal=True, window=(150, 0)),
                    torch.bfloat16),
    "two_sided_window_d64": (dict(batch=1, heads=2, kv_heads=2, seqlen=400, head_dim=64, causal=False,
                                  window=(64, 33)), torch.bfloat16),
    "q_shorter_than_k_d128": (dict(batch=2, heads=4, kv_heads=2, seqlen=150, seqlen_k=431, head_dim=128,
                                   causal=True), torch.bfloat16),
    "q_longer_than_k_d64": (dict(batch=1, heads=2, kv_heads=1, seqlen=333, seqlen_k=120, head_dim=64, causal=True),
                            torch.float16),
    "varlen_causal_d128": (dict(batch=0, heads=4, kv_heads=2, seqlen=0, head_dim=128, causal=True,
                                seqlens=[1, 255, 0, 257, 600]), torch.bfloat16),
    "large_scores_d128": (dict(batch=1, heads=2, kv_heads=2, seqlen=300, head_dim=128, causal=True, scale=0.5,
                               factor=3.0), torch.bfloat16),
    "gqa_groups_on_one_xcd_d128": (dict(batch=4, heads=8, kv_heads=2, seqlen=200, head_dim=128, causal=True),
                                   torch.bfloat16),
    # head dims between the tile widths: zero Q^T past head_dim, clamped tile loads, no stores past it
    "d16_noncausal": (dict(batch=2, heads=2, kv_heads=1, seqlen=150, head_dim=16, causal=False), torch.bfloat16),
    "d48_causal_gqa": (dict(batch=1, heads=4, kv_heads=2, seqlen=333, head_dim=48, causal=True), torch.float16),
    "d96_window": (dict(batch=2, heads=2, kv_heads=2, seqlen=300, head_dim=96, causal=True, window=(90, 0)),
                   torch.bfloat16),
    "d112_q_shorter_than_k": (dict(batch=1, heads=3, kv_heads=1, seqlen=120, seqlen_k=290, head_dim=112,
                                   causal=True), torch.bfloat16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_parity(fa, oracle_mod, name):
    kwargs, out_dtype = CASES[name]
    say(f"[fp8 parity] {name}")
    p = synth.make_problem(dtype="fp8", seed=42, **kwargs)
    got_o, got_lse = run_gpu(fa, p, out_dtype)
    o, lse, bound, lb = reference_and_bound(oracle_mod, p, out_dtype)
    check(name, got_o, got_lse, o, lse, bound, lb)


def test_padded_batch(fa, oracle_mod):
    """seqused: rows past a sequence's valid length are O = 0, LSE = -inf."""
    p = synth.make_problem(dtype="fp8", batch=3, heads=4, kv_heads=2, seqlen=260, head_dim=128, causal=True, seed=43)
    used = [260, 100, 0]
    dev = torch.device("cuda:0")
    ut = torch.tensor(used, dtype=torch.int32, device=dev)
    got_o, got_lse = run_gpu(fa, p, used=(ut, ut))
    for b, u in enumerate(used):
        assert np.all(got_o[b, u:] == 0) and np.all(np.isneginf(got_lse[b, :, u:]))
        if u == 0:
            continue
        sub = synth.make_problem(dtype="fp8", batch=1, heads=4, kv_heads=2, seqlen=u, head_dim=128, causal=True,
                                 seed=43)
        sub.q, sub.k, sub.v = p.q[b:b + 1, :u], p.k[b:b + 1, :u], p.v[b:b + 1, :u]
        sub.descale_q, sub.descale_k, sub.descale_v = p.descale_q, p.descale_k, p.descale_v
        o, lse, bound, lb = reference_and_bound(oracle_mod, sub, torch.bfloat16)
        check(f"padded seq {b}", got_o[b:b + 1, :u], got_lse[b:b + 1, :, :u], o, lse, bound, lb)


def test_descales(fa):
    """Powers of two: (dq, dk) = (2, 0.5) and (0.5, 2) give the same bytes;
    doubling dv doubles O exactly and leaves LSE alone."""
    p = synth.make_problem(dtype="fp8", batch=1, heads=2, kv_heads=2, seqlen=200, head_dim=128, causal=True, seed=44)
    dev = torch.device("cuda:0")
    q, k, v = p.q.to(dev), p.k.to(dev), p.v.to(dev)
    o1, l1 = fa.forward_fp8(q, k, v, 2.0, 0.5, 0.01, causal=True)
    o2, l2 = fa.forward_fp8(q, k, v, 0.5, 2.0, 0.01, causal=True)
    o3, l3 = fa.forward_fp8(q, k, v, 2.0, 0.5, 0.02, causal=True)
    u8 = q.view(torch.uint8)
    o4, l4 = fa.forward_fp8(u8, k.view(torch.uint8), v.view(torch.uint8), 2.0, 0.5, 0.01, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, 2 * o1) and torch.equal(l3, l1)
    assert torch.equal(o4, o1) and torch.equal(l4, l1)


@pytest.mark.parametrize("d", [64, 48])
def test_empty_and_guard_bands(fa, d):
    dev = torch.device("cuda:0")
    e = torch.empty(1, 0, 2, d, dtype=torch.float8_e4m3fn, device=dev)
    o, lse = fa.forward_fp8(e, e, e, 1.0, 1.0, 1.0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and lse.numel() == 0
    p = synth.make_problem(dtype="fp8", batch=1, heads=3, kv_heads=1, seqlen=257, head_dim=d, causal=True, seed=45)
    q, k, v = p.q.to(dev), p.k.to(dev), p.v.to(dev)
    pad = 4096
    buf = torch.full((q.numel() + 2 * pad,), 5.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + q.numel()].view(q.shape)
    fa.forward_fp8(q, k, v, p.descale_q, p.descale_k, p.descale_v, causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 5.0) and torch.all(buf[-pad:] == 5.0)
    assert torch.isfinite(out.float()).all()


def test_full_size_workload_sampled(fa, oracle_mod):
    """The 8K FP8 workload in the launch shape the benchmark times; sampled
    query rows of three heads."""
    name = "fp8_causal_b1_h32_n8192_d128"
    say(f"[fp8 full size] {name}")
    p = synth.workload(name)
    got_o, got_lse = run_gpu(fa, p)
    rows = np.array([0, 1, 255, 256, 3001, 4095, 8000, 8191])
    heads = np.array([0, 17, 31])
    o, lse, bound, lb = reference_and_bound(oracle_mod, p, torch.bfloat16, rows=rows, heads=heads)
    sel = lambda x: x[:, rows][:, :, heads]
    sl = lambda x: x[:, heads][:, :, rows]
    check(name, sel(got_o), sl(got_lse), sel(o), sl(lse), sel(bound), sl(lb))


def draw_fp8(seed):
    r = np.random.default_rng(7000 + seed)
    kv = int(r.integers(1, 3))
    cfg = dict(head_dim=int(16 * r.integers(1, 9)), heads=kv * int(r.choice([1, 2, 4])), kv_heads=kv,
               causal=bool(r.integers(0, 2)))
    if r.random() < 0.3:
        cfg["window"] = (int(r.integers(0, 150)), int(r.integers(0, 40)) if r.random() < 0.5 else -1)
    if r.random() < 0.3:
        cfg.update(batch=0, seqlen=0, seqlens=[int(x) for x in r.integers(1, 260, int(r.integers(1, 4)))])
    else:
        cfg.update(batch=int(r.integers(1, 3)), seqlen=int(r.integers(1, 300)))
        if r.random() < 0.4:
            cfg["seqlen_k"] = int(r.integers(1, 300))
    return cfg, (torch.bfloat16 if r.random() < 0.5 else torch.float16)


@pytest.mark.parametrize("seed", range(16))
def test_random_fp8(fa, oracle_mod, seed):
    """Seeded random shapes, masks and layouts, against the derived bound."""
    cfg, out_dtype = draw_fp8(seed)
    say(f"[fp8 random {seed}] {cfg}")
    p = synth.make_problem(dtype="fp8", seed=80 + seed, **cfg)
    got_o, got_lse = run_gpu(fa, p, out_dtype)
    o, lse, bound, lb = reference_and_bound(oracle_mod, p, out_dtype)
    check(f"random {seed}", got_o, got_lse, o, lse, bound, lb)
