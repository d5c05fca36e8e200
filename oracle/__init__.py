"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product path never imports it.

``attention_oracle.cpp`` holds the definition (standard attention written
out in double precision, see its header for the readings taken); this module
builds it with g++ and calls it through ctypes on float64 numpy arrays.
Entries the caller did not select are returned as NaN.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle (g++, no fast-math: IEEE double throughout)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-fPIC", "-shared",
                               "-pthread", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D, U64 = ctypes.c_double, ctypes.c_uint64
        lib.oracle_attention_fwd.argtypes = [P] * 7 + [I] * 9 + \
            [D, P, I, P, I, I, D, U64]
        lib.oracle_attention_fwd.restype = I
        lib.oracle_attention_bwd.argtypes = [P] * 11 + [I] * 9 + \
            [D, P, I, P, I, P, I, I, D, U64]
        lib.oracle_attention_bwd.restype = I
        lib.oracle_philox4x32_10.argtypes = [P, P, P]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_philox4x64_10.argtypes = [P, P, P]
        lib.oracle_philox4x64_10.restype = None
        lib.oracle_dropout_threshold.argtypes = [D]
        lib.oracle_dropout_threshold.restype = I
        lib.oracle_dropout_mask.argtypes = [I, I, I, I, D, U64, P]
        lib.oracle_dropout_mask.restype = None
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> exact float64
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _geometry(q, k, heads_hint, cu, cu_k=None):
    if cu is None:
        b, nq, h, d = q.shape
        _, nk, hk, _ = k.shape
        return b, h, hk, nq, nk, d
    cu_k = cu if cu_k is None else cu_k
    if len(cu_k) != len(cu):
        raise ValueError("cu_seqlens and cu_seqlens_k must describe the same number of sequences")
    _, h, d = q.shape
    _, hk, _ = k.shape
    lq, lk = np.diff(cu), np.diff(cu_k)
    mq = int(lq.max()) if len(lq) else 0
    mk = int(lk.max()) if len(lk) else 0
    return len(cu) - 1, h, hk, mq, mk, d


def attention_fwd(q, k, v, *, scale, causal=False, window=(-1, -1),
                  cu_seqlens=None, rows=None, heads=None, threads=0,
                  dropout_p=0.0, seed=0, cu_seqlens_k=None):
    """O and LSE of exact attention.  q: (B, Nq, H, d) or packed (T, H, d);
    k, v: (B, Nk, Hkv, d) or (T, Hkv, d).  ``cu_seqlens`` (B+1 prefix sums)
    marks a packed batch, used for both queries and keys unless
    ``cu_seqlens_k`` gives the keys' own.  ``rows`` /
    ``heads`` restrict the computed query rows (positions within each
    sequence) / query heads; the rest stays NaN.  ``dropout_p`` / ``seed``:
    dropout with the Philox4x32-10 keep decisions (see the C++ header)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = _i32(cu_seqlens)
    cuk = cu if cu_seqlens_k is None or cu is None else _i32(cu_seqlens_k)
    B, H, HK, NQ, NK, D = _geometry(q, k, None, cu, cuk)
    o = np.full(q.shape, np.nan)
    lse = np.full((B, H, NQ) if cu is None else (H, q.shape[0]), np.nan)
    rs, hs = _i32(rows), _i32(heads)
    rc = _load().oracle_attention_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu), _ptr(cuk),
        B, H, HK, NQ, NK, D, int(bool(causal)), int(window[0]), int(window[1]),
        float(scale), _ptr(rs), 0 if rs is None else len(rs),
        _ptr(hs), 0 if hs is None else len(hs), int(threads),
        float(dropout_p), int(seed) & (2**64 - 1))
    if rc:
        raise ValueError("oracle_attention_fwd: bad arguments")
    return o, lse


def attention_bwd(q, k, v, dout, *, scale, causal=False, window=(-1, -1),
                  cu_seqlens=None, q_rows=None, k_rows=None, kv_heads=None,
                  threads=0, dropout_p=0.0, seed=0, cu_seqlens_k=None):
    """dQ, dK, dV (and the oracle's own O, LSE on the rows it needed) of exact
    attention for upstream gradient ``dout``.  ``cu_seqlens_k`` as in
    attention_fwd.  ``q_rows`` restricts dQ rows,
    ``k_rows`` the dK/dV rows, ``kv_heads`` the kv heads (with all query
    heads of their groups); unselected entries stay NaN."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = _i32(cu_seqlens)
    cuk = cu if cu_seqlens_k is None or cu is None else _i32(cu_seqlens_k)
    B, H, HK, NQ, NK, D = _geometry(q, k, None, cu, cuk)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(k.shape, np.nan)
    o = np.full(q.shape, np.nan)
    lse = np.full((B, H, NQ) if cu is None else (H, q.shape[0]), np.nan)
    qr, kr, kh = _i32(q_rows), _i32(k_rows), _i32(kv_heads)
    rc = _load().oracle_attention_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(o), _ptr(lse), _ptr(cu), _ptr(cuk),
        B, H, HK, NQ, NK, D, int(bool(causal)), int(window[0]), int(window[1]),
        float(scale), _ptr(qr), 0 if qr is None else len(qr),
        _ptr(kr), 0 if kr is None else len(kr),
        _ptr(kh), 0 if kh is None else len(kh), int(threads),
        float(dropout_p), int(seed) & (2**64 - 1))
    if rc:
        raise ValueError("oracle_attention_bwd: bad arguments")
    return dq, dk, dv, o, lse


def philox4x32_10(counter, key):
    """Philox4x32-10 output block for a 4-word counter and 2-word key."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox4x64_10(counter, key):
    """Philox4x64-10 output block (checks the shared round structure)."""
    c = np.ascontiguousarray(counter, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    _load().oracle_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def dropout_threshold(p: float) -> int:
    """Keep threshold T: an element is kept iff its 8-bit draw is below T."""
    return int(_load().oracle_dropout_threshold(float(p)))


def dropout_mask(batch, heads, lq, lk, p, seed):
    """Keep decisions (uint8, 1 = kept) of elements (b, h, i, j)."""
    out = np.zeros((batch, heads, lq, lk), dtype=np.uint8)
    _load().oracle_dropout_mask(int(batch), int(heads), int(lq), int(lk), float(p),
                                int(seed) & (2**64 - 1), _ptr(out))
    return out


def _u8(x):
    """FP8 codes as a uint8 numpy array (accepts torch float8 / uint8 tensors)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu()
        if x.dtype != torch.uint8:
            x = x.view(torch.uint8)
        x = x.numpy()
    return np.ascontiguousarray(x, dtype=np.uint8)


def fp8_e4m3_decode(codes):
    """Values of FP8 E4M3 codes as float64, from the format's definition (OCP
    8-bit floating point specification, E4M3 without infinities): sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9; S.1111.111 is NaN, so the largest value is
    1.75 * 2^8 = 448."""
    c = _u8(codes)
    e = ((c >> 3) & 0xF).astype(np.int64)
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def attention_fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, **kw):
    """Exact attention (attention_fwd) of dequantised FP8 inputs: each tensor
    is descale * E4M3(code), per tensor.  The scores are those of the
    dequantised Q and K, so softmax_scale applies on top of the descales."""
    q = fp8_e4m3_decode(q8) * float(descale_q)
    k = fp8_e4m3_decode(k8) * float(descale_k)
    v = fp8_e4m3_decode(v8) * float(descale_v)
    return attention_fwd(q, k, v, **kw)
