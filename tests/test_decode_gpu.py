"""Parity of the KV-cache decode path (fa_fwd_kvcache, through the C-ABI)
with the fp64 CPU oracle.

The oracle takes each sequence on its own: the new tokens against the valid
prefix of that sequence's cache, bottom-right aligned (token t of Nq sits at
position len - Nq + t), which is the same definition fa_fwd follows with
Nq != Nk.  Small cases are compared in full; the full-size decode workloads
on every row (one token) or on sampled heads (eight tokens).  Tolerances are
the forward's: O max-abs 4e-3 (fp16) / 2e-2 (bf16), LSE max-abs 1e-3.
"""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

O_TOL = {"fp16": 4e-3, "bf16": 2e-2}
LSE_TOL = 1e-3


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


def gpu_decode(fa, p, num_splits=0, lens=True):
    dev = torch.device("cuda:0")
    q, kc, vc = p.q.to(dev), p.k_cache.to(dev), p.v_cache.to(dev)
    cs = p.cache_seqlens().to(dev) if lens else None
    o, lse = fa.forward_kvcache(q, kc, vc, cs, causal=p.causal,
                                window_size=(p.window_left, p.window_right),
                                softmax_scale=p.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def oracle_decode(oracle, p, heads=None):
    B, Nq, H, D = p.q.shape
    o = np.full((B, Nq, H, D), np.nan)
    lse = np.full((B, H, Nq), np.nan)
    for b in range(B):
        n = p.cache_lens[b]
        ob, lb = oracle.attention_fwd(p.q[b:b + 1], p.k_cache[b:b + 1, :n], p.v_cache[b:b + 1, :n],
                                      scale=p.scale, causal=p.causal,
                                      window=(p.window_left, p.window_right), heads=heads)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def compare(p, got, want, heads=None):
    go, gl = got
    wo, wl = want
    if heads is not None:
        go, wo = go[:, :, heads], wo[:, :, heads]
        gl, wl = gl[:, heads], wl[:, heads]
    assert not np.isnan(wo).any() and not np.isnan(wl).any()
    assert np.isfinite(go).all(), "non-finite O"
    err_o = float(np.max(np.abs(go - wo))) if go.size else 0.0
    fin = np.isfinite(wl)
    assert np.array_equal(np.isfinite(gl), fin), "LSE -inf pattern differs"
    assert (gl[~fin] == -np.inf).all()
    err_l = float(np.max(np.abs(gl[fin] - wl[fin]))) if fin.any() else 0.0
    # rows without visible keys are exactly zero
    empty = ~fin  # (B, H, Nq)
    if empty.any():
        z = np.transpose(go, (0, 2, 1, 3))[empty]
        assert (z == 0).all(), "empty rows must be zero"
    say(f"  O max-abs {err_o:.3e} (tol {O_TOL[p.dtype]}), LSE max-abs {err_l:.3e}")
    assert err_o <= O_TOL[p.dtype]
    assert err_l <= LSE_TOL


SMALL = {
    # GQA group of 4, one token, ragged lengths incl. an empty and a 1-key cache
    "bf16_g4_q1_d128": dict(dtype="bf16", batch=4, heads=8, kv_heads=2, seqlen_q=1, capacity=700,
                            head_dim=128, causal=True, cache_lens=[0, 1, 333, 700]),
    # MHA, 16 tokens, d64, lengths on and off the 32-key step
    "fp16_g1_q16_d64": dict(dtype="fp16", batch=2, heads=4, kv_heads=4, seqlen_q=16, capacity=517,
                            head_dim=64, causal=True, cache_lens=[16, 517]),
    # 8 heads x 8 tokens = 64 rows per kv head: two row blocks
    "bf16_g8_q8_d128_two_row_blocks": dict(dtype="bf16", batch=2, heads=16, kv_heads=2, seqlen_q=8,
                                           capacity=1000, head_dim=128, causal=True,
                                           cache_lens=[999, 500]),
    # sliding window (64 back, none ahead), MQA
    "fp16_window64_mqa_q4_d128": dict(dtype="fp16", batch=2, heads=4, kv_heads=1, seqlen_q=4,
                                      capacity=900, head_dim=128, causal=True, window=(64, 0),
                                      cache_lens=[900, 450]),
    # fewer keys than tokens: the first token of sequence 0 sees nothing
    "bf16_short_cache_q3_d64": dict(dtype="bf16", batch=2, heads=2, kv_heads=1, seqlen_q=3,
                                    capacity=40, head_dim=64, causal=True, cache_lens=[2, 40]),
    # non-causal: every new token sees the whole valid cache
    "fp16_noncausal_g2_q5_d64": dict(dtype="fp16", batch=3, heads=4, kv_heads=2, seqlen_q=5,
                                     capacity=300, head_dim=64, causal=False, cache_lens=[7, 64, 300]),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_small(fa, oracle_mod, name):
    say(f"decode small {name}")
    p = synth.make_decode(seed=3, **SMALL[name])
    compare(p, gpu_decode(fa, p), oracle_decode(oracle_mod, p))


@pytest.mark.parametrize("num_splits", [1, 3, 7, 1000])
def test_decode_split_counts(fa, oracle_mod, num_splits):
    say(f"decode split count {num_splits}")
    p = synth.make_decode(seed=5, dtype="bf16", batch=2, heads=8, kv_heads=2, seqlen_q=2, capacity=1500,
                          head_dim=128, causal=True, cache_lens=[1500, 777])
    compare(p, gpu_decode(fa, p, num_splits=num_splits), oracle_decode(oracle_mod, p))


def test_decode_full_cache_without_lengths(fa, oracle_mod):
    say("decode cache_seqlens=NULL")
    p = synth.make_decode(seed=7, dtype="fp16", batch=2, heads=4, kv_heads=2, seqlen_q=1, capacity=613,
                          head_dim=64, causal=True)
    compare(p, gpu_decode(fa, p, lens=False), oracle_decode(oracle_mod, p))


def test_decode_matches_forward(fa):
    """Same inputs through fa_fwd (caches trimmed to equal lengths): the two
    paths agree to the forward's tolerance."""
    say("decode vs fa_fwd")
    p = synth.make_decode(seed=11, dtype="bf16", batch=2, heads=8, kv_heads=2, seqlen_q=4, capacity=2000,
                          head_dim=128, causal=True)
    o, lse = gpu_decode(fa, p)
    dev = torch.device("cuda:0")
    of, lf = fa.forward(p.q.to(dev), p.k_cache.to(dev), p.v_cache.to(dev), causal=True, softmax_scale=p.scale)
    torch.cuda.synchronize()
    assert np.max(np.abs(o - of.float().cpu().double().numpy())) <= O_TOL["bf16"]
    assert np.max(np.abs(lse - lf.cpu().double().numpy())) <= LSE_TOL


def test_decode_empty_batch(fa):
    dev = torch.device("cuda:0")
    q = torch.empty(0, 1, 4, 64, dtype=torch.float16, device=dev)
    kc = torch.empty(0, 100, 2, 64, dtype=torch.float16, device=dev)
    o, lse = fa.forward_kvcache(q, kc, kc, None)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (0, 4, 1)


@pytest.mark.parametrize("name", list(synth.DECODE_WORKLOADS))
def test_decode_workload_full_size(fa, oracle_mod, name):
    say(f"decode workload {name}")
    p = synth.decode_workload(name)
    heads = None if p.seqlen_q == 1 else np.array([0, 13, 31])
    compare(p, gpu_decode(fa, p), oracle_decode(oracle_mod, p, heads=heads), heads=heads)
