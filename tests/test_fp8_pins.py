"""Pins of the oracle's FP8 side (the FP8 forward: inputs in the 8-bit E4M3
format with per-tensor scales, the hardware path the FlashAttention-2
overview page, lshu.cn/news/55956, section 5.2, describes for H100 with
float8_e4m3fn) against facts outside the oracle:

* the decoder: every one of the 256 codes against torch's float8_e4m3fn
  conversion (an independent implementation of the same format), and the
  format's closed forms (largest value 448, smallest normal 2^-6, smallest
  subnormal 2^-9, the two NaN codes, sign symmetry, monotone order);
* the dequantising attention: against attention on tensors decoded by torch
  instead, and invariants of the per-tensor descales that a misplaced scale
  would break (descale_q and descale_k only act through their product, which
  is interchangeable with softmax_scale; descale_v scales O linearly and leaves
  LSE alone);
* the seeded FP8 inputs: codes are the round-to-nearest E4M3 of x / descale,
  with the tensor's largest magnitude at exactly 448.
"""
import numpy as np
import pytest
import torch

import synth


def torch_decode(codes_u8):
    return torch.from_numpy(np.ascontiguousarray(codes_u8, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_all_codes_match_torch(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    mine, ref = oracle_mod.fp8_e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # signed zeros too
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_format_closed_forms(oracle_mod):
    d = oracle_mod.fp8_e4m3_decode
    assert d(np.array([0x7E], dtype=np.uint8))[0] == 448.0
    assert d(np.array([0x08], dtype=np.uint8))[0] == 2.0 ** -6
    assert d(np.array([0x01], dtype=np.uint8))[0] == 2.0 ** -9
    assert d(np.array([0x07], dtype=np.uint8))[0] == 7 * 2.0 ** -9
    assert d(np.array([0x38], dtype=np.uint8))[0] == 1.0
    assert d(np.array([0x39], dtype=np.uint8))[0] == 1.125
    nan = d(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.all(np.isnan(nan))
    pos = d(np.arange(0x00, 0x7F, dtype=np.uint8))
    neg = d(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(neg, -pos)
    # 8 mantissa steps per binade: code c of exponent e is 2^(e-3) below code c + 1;
    # the subnormals (and zero) are spaced 2^-9, the spacing of the first binade
    for c in range(0x08, 0x7E):
        e = (c >> 3) - 7
        assert pos[c + 1] - pos[c] == 2.0 ** (e - 3)
    assert np.array_equal(np.diff(pos[:0x09]), np.full(8, 2.0 ** -9))


def _rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _codes(x):
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn)


def test_dequantised_attention_matches_torch_decoded_inputs(oracle_mod):
    q8, k8, v8 = _codes(_rnd((2, 19, 4, 16), 1, 60)), _codes(_rnd((2, 23, 2, 16), 2, 60)), \
        _codes(_rnd((2, 23, 2, 16), 3, 60))
    dq, dk, dv = 0.011, 0.0093, 0.02
    kw = dict(scale=0.25, causal=True, window=(9, 0))
    o, lse = oracle_mod.attention_fwd_fp8(q8, k8, v8, dq, dk, dv, **kw)
    q = q8.double().numpy() * dq
    k = k8.double().numpy() * dk
    v = v8.double().numpy() * dv
    o2, lse2 = oracle_mod.attention_fwd(q, k, v, **kw)
    assert np.array_equal(o, o2, equal_nan=True) and np.array_equal(lse, lse2, equal_nan=True)


def test_descale_invariants(oracle_mod):
    q8, k8, v8 = _codes(_rnd((1, 17, 2, 32), 4, 40)), _codes(_rnd((1, 17, 2, 32), 5, 40)), \
        _codes(_rnd((1, 17, 2, 32), 6, 40))
    kw = dict(causal=True)
    o, lse = oracle_mod.attention_fwd_fp8(q8, k8, v8, 0.01, 0.02, 0.5, scale=0.3, **kw)
    # only the product descale_q * descale_k acts (powers of two: exact)
    o2, lse2 = oracle_mod.attention_fwd_fp8(q8, k8, v8, 0.02, 0.01, 0.5, scale=0.3, **kw)
    o3, lse3 = oracle_mod.attention_fwd_fp8(q8, k8, v8, 0.04, 0.005, 0.5, scale=0.3, **kw)
    assert np.allclose(o, o2, rtol=0, atol=1e-15) and np.allclose(lse, lse2, rtol=0, atol=1e-13)
    assert np.allclose(o, o3, rtol=0, atol=1e-15) and np.allclose(lse, lse3, rtol=0, atol=1e-13)
    # and it is interchangeable with softmax_scale
    o4, lse4 = oracle_mod.attention_fwd_fp8(q8, k8, v8, 0.02, 0.02, 0.5, scale=0.15, **kw)
    assert np.allclose(o, o4, rtol=0, atol=1e-15) and np.allclose(lse, lse4, rtol=0, atol=1e-13)
    # descale_v: O linear, LSE untouched
    o5, lse5 = oracle_mod.attention_fwd_fp8(q8, k8, v8, 0.01, 0.02, 1.5, scale=0.3, **kw)
    assert np.allclose(o5, 3.0 * o, rtol=1e-13, atol=1e-13 * np.abs(o5).max()) and np.array_equal(lse5, lse)


def test_seeded_fp8_inputs_are_rounded_scaled_normals(oracle_mod):
    p = synth.make_problem(dtype="fp8", batch=1, heads=2, kv_heads=1, seqlen=40, head_dim=32, causal=True,
                           seed=7, factor=0.5)
    for t, desc, stream, shape in ((p.q, p.descale_q, synth.STREAM_Q, (1, 40, 2, 32)),
                                   (p.k, p.descale_k, synth.STREAM_K, (1, 40, 1, 32))):
        assert t.dtype == torch.float8_e4m3fn and tuple(t.shape) == shape
        x = synth.normals_f64(16 * 7 + stream, int(np.prod(shape))) * 0.5
        assert desc == np.abs(x).max() / 448.0
        vals = oracle_mod.fp8_e4m3_decode(t).ravel()
        assert np.abs(vals).max() == 448.0
        # nearest representable value of x / descale (ties never occur for these draws)
        grid = oracle_mod.fp8_e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
        y = np.abs(x / desc)
        idx = np.clip(np.searchsorted(grid, y), 1, len(grid) - 1)
        near = np.where(y - grid[idx - 1] <= grid[idx] - y, grid[idx - 1], grid[idx])
        assert np.array_equal(np.abs(vals), near)
