"""The allocation-free backward (fa_bwd_noalloc, through the C-ABI) against
fa_bwd on the deterministic path: the same kernels on the same inputs, so the
outputs must be byte-identical (stricter than the oracle tolerances).  Two
calls in a row, the second on a smaller problem, since every call on a GPU
shares the library's scratch array; plus the size limit and argument checks."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


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


CASES = [
    dict(dtype="bf16", batch=2, heads=8, kv_heads=2, seqlen=700, head_dim=128, causal=True, factor=0.5),
    dict(dtype="fp16", batch=1, heads=4, kv_heads=4, seqlen=150, head_dim=64, causal=False, window=(40, 7)),
]


def run_both(fa, p):
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    kw = dict(causal=p.causal, window_size=(p.window_left, p.window_right), softmax_scale=p.scale)
    o, lse = fa.forward(q, k, v, **kw)
    ref = fa.backward(do, q, k, v, o, lse, deterministic=True, **kw)
    got = tuple(torch.full_like(t, float("nan")) for t in ref)
    fa.backward_noalloc(do, q, k, v, o, lse, *got, **kw)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_fa_bwd_twice_second_smaller(fa):
    for i, cfg in enumerate(CASES):
        say(f"[noalloc] call {i}: {cfg}")
        p = synth.make_problem(seed=21 + i, **cfg)
        ref, got = run_both(fa, p)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_noalloc_packed_batch(fa):
    p = synth.make_problem(seed=5, dtype="fp16", batch=0, heads=4, kv_heads=2, seqlen=0, head_dim=128, causal=True,
                           window=(200, 0), seqlens=[1, 63, 300, 0, 129])
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    cu = p.cu_seqlens().to(dev)
    kw = dict(causal=True, window_size=(200, 0), softmax_scale=p.scale, cu_seqlens_q=cu, cu_seqlens_k=cu,
              max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    o, lse = fa.forward(q, k, v, **kw)
    ref = fa.backward(do, q, k, v, o, lse, deterministic=True, **kw)
    got = tuple(torch.full_like(t, float("nan")) for t in ref)
    fa.backward_noalloc(do, q, k, v, o, lse, *got, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_noalloc_limit_and_arguments(fa):
    import ctypes
    L = fa.lib()
    P = ctypes.c_void_p(0x10000)
    common = [None, None, None, None]
    # 2^21 + 1 (row, head) pairs: beyond the scratch array (rejected before any launch)
    rc = L.fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, *common, 1, 1, 1, (1 << 21) + 1, 16, 64, 1, -1, -1, 0.125,
                          0.0, 0, 1, None)
    assert rc == 4  # FA_ERR_WORKSPACE
    rc = L.fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, *common, 1, 3, 2, 16, 16, 64, 1, -1, -1, 0.125, 0.0, 0, 1, None)
    assert rc == 1  # heads % kv_heads: FA_ERR_INVALID_ARG
    rc = L.fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, *common, 1, 4, 2, 16, 16, 36, 1, -1, -1, 0.125, 0.0, 0, 1, None)
    assert rc == 2  # head_dim 36: FA_ERR_UNSUPPORTED
