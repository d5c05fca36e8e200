"""Seeded synthetic inputs for exact attention: the one module that both the
oracle side and the HIP side consume.

It holds no attention arithmetic: it only draws numbers.  Every tensor is a
pure function of (seed, stream id, element index), so the bytes do not depend
on numpy/torch versions or on the chunking used to produce them:

* counter-based generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014).  Element n of stream s is the
  SplitMix64 finaliser applied to ``key(s) + (n + 1) * 0x9E3779B97F4A7C15``,
  where ``key(s)`` is the finaliser applied to ``s``;
* normals: Box-Muller on consecutive output pairs (2m, 2m+1), giving the
  cosine branch at even and the sine branch at odd element indices, in float64;
* rounding: float64 -> float32 (round to nearest even) -> the 16-bit input
  dtype (round to nearest even);
* FP8 inputs ("fp8"): per-tensor scale amax / 448, then float64 / scale ->
  float32 -> FP8 E4M3 (torch.float8_e4m3fn, round to nearest even); the
  problem carries the descales (the scales themselves).

Streams for one seed: Q = 16*seed + 0, K = +1, V = +2, dO = +3, lengths = +4.
Tensors are laid out (batch, seqlen, heads, head_dim) with the last dimension
contiguous; variable-length batches are packed to (total, heads, head_dim).

The named workloads stand in for the pages' own (model-level runs that need
trained weights): a small non-causal fp16 case, a causal d=64 batch, a
7B-layer attention shape at 8K, a long-context GQA shape at 32K and a packed
sliding-window batch.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22  # elements drawn per numpy pass (bounds temporary memory)

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_LEN = 0, 1, 2, 3, 4


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _key(stream: int) -> np.uint64:
    return _mix(np.array([stream], dtype=np.uint64))[0]


def raw_u64(stream: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of one SplitMix64 stream."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(_key(stream) + idx * _GAMMA)


def normals_f64(stream: int, count: int) -> np.ndarray:
    """``count`` standard normals of one stream, float64, element n of the
    stream being the cosine (n even) or sine (n odd) branch of Box-Muller on
    the raw pair (2*(n//2), 2*(n//2)+1)."""
    out = np.empty(count, dtype=np.float64)
    two53 = float(1 << 53)

    def fill(c0):
        c1 = min(count, c0 + _CHUNK)
        p0 = c0 // 2
        p1 = (c1 + 1) // 2
        raw = raw_u64(stream, 2 * p0, 2 * (p1 - p0))
        a = raw[0::2]
        b = raw[1::2]
        u1 = ((a >> np.uint64(11)).astype(np.float64) + 1.0) / two53  # (0, 1]
        u2 = (b >> np.uint64(11)).astype(np.float64) / two53          # [0, 1)
        r = np.sqrt(-2.0 * np.log(u1))
        t = 2.0 * math.pi * u2
        pair = np.empty(2 * (p1 - p0), dtype=np.float64)
        pair[0::2] = r * np.cos(t)
        pair[1::2] = r * np.sin(t)
        off = c0 - 2 * p0
        out[c0:c1] = pair[off:off + (c1 - c0)]

    starts = range(0, count, _CHUNK)
    if count > _CHUNK:
        # chunks are independent (counter-based), so threads change nothing
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, starts))
    else:
        for c0 in starts:
            fill(c0)
    return out


def uniform_ints(stream: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` integers uniform on [lo, hi], both ends included."""
    raw = raw_u64(stream, 0, count)
    u = (raw >> np.uint64(11)).astype(np.float64) / float(1 << 53)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)


def _to_dtype(x64: np.ndarray, dtype: str):
    """Round float64 -> float32 -> 16-bit, both steps to nearest even.
    Returns a torch CPU tensor of the 16-bit dtype."""
    import torch
    x32 = torch.from_numpy(x64.astype(np.float32))
    if dtype == "fp16":
        return x32.to(torch.float16)
    if dtype == "bf16":
        return x32.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def tensor(seed: int, stream: int, shape, dtype: str, factor: float = 1.0):
    """One seeded 16-bit tensor of ``shape`` (torch, CPU)."""
    n = int(np.prod(shape))
    x = normals_f64(16 * seed + stream, n)
    if factor != 1.0:
        x *= factor
    return _to_dtype(x, dtype).reshape(tuple(shape))


FP8_MAX = 448.0  # largest finite FP8 E4M3 value


def tensor_fp8(seed: int, stream: int, shape, factor: float = 1.0):
    """One seeded FP8 E4M3 tensor (torch.float8_e4m3fn, CPU) and its descale:
    the normals of the stream, divided by amax / 448 and rounded to E4M3."""
    import torch
    n = int(np.prod(shape))
    x = normals_f64(16 * seed + stream, n)
    if factor != 1.0:
        x *= factor
    amax = float(np.abs(x).max()) if n else 0.0
    descale = amax / FP8_MAX if amax > 0 else 1.0
    t = torch.from_numpy((x / descale).astype(np.float32)).to(torch.float8_e4m3fn)
    return t.reshape(tuple(shape)), descale


@dataclass
class Problem:
    """One attention problem: shapes, mask and the seeded tensors (CPU)."""
    dtype: str
    batch: int
    heads: int
    kv_heads: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    causal: bool
    window_left: int = -1
    window_right: int = -1
    scale: float = 0.0
    seqlens: list | None = None  # per-sequence lengths when packed
    q: object = None
    k: object = None
    v: object = None
    do: object = None
    meta: dict = field(default_factory=dict)
    descale_q: float = 1.0  # FP8 problems: value = descale * E4M3(code)
    descale_k: float = 1.0
    descale_v: float = 1.0

    @property
    def varlen(self) -> bool:
        return self.seqlens is not None

    def cu_seqlens(self):
        import torch
        if self.seqlens is None:
            return None
        cu = np.zeros(len(self.seqlens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.seqlens)
        return torch.from_numpy(cu)


def make_problem(*, dtype: str, batch: int, heads: int, kv_heads: int,
                 seqlen: int, head_dim: int, causal: bool,
                 window=(-1, -1), scale: float | None = None,
                 factor: float = 1.0, seed: int = 0, with_do: bool = True,
                 varlen_range=None, seqlen_k: int | None = None,
                 seqlens=None) -> Problem:
    """Draw one problem.  ``varlen_range=(lo, hi)`` draws one length per
    sequence uniformly on [lo, hi] (stream 4) and packs the batch; ``seqlens``
    gives the lengths explicitly instead."""
    seqlen_k = seqlen if seqlen_k is None else seqlen_k
    if seqlens is not None:
        batch = len(seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    lens = None
    if varlen_range is not None:
        lens = [int(x) for x in uniform_ints(16 * seed + STREAM_LEN, batch,
                                             varlen_range[0], varlen_range[1])]
    elif seqlens is not None:
        lens = [int(x) for x in seqlens]
    if lens is not None:
        if seqlen_k != seqlen:
            raise ValueError("packed batches are self-attention here")
        total = sum(lens)
        qshape = (total, heads, head_dim)
        kshape = (total, kv_heads, head_dim)
        seqlen = seqlen_k = max(lens) if lens else 0
    else:
        qshape = (batch, seqlen, heads, head_dim)
        kshape = (batch, seqlen_k, kv_heads, head_dim)
    p = Problem(dtype=dtype, batch=batch, heads=heads, kv_heads=kv_heads,
                seqlen_q=seqlen, seqlen_k=seqlen_k, head_dim=head_dim,
                causal=causal, window_left=window[0], window_right=window[1],
                scale=scale, seqlens=lens)
    if dtype == "fp8":
        p.q, p.descale_q = tensor_fp8(seed, STREAM_Q, qshape, factor)
        p.k, p.descale_k = tensor_fp8(seed, STREAM_K, kshape, factor)
        p.v, p.descale_v = tensor_fp8(seed, STREAM_V, kshape, factor)
        p.meta = dict(seed=seed, factor=factor)
        return p  # forward only: no dO
    p.q = tensor(seed, STREAM_Q, qshape, dtype, factor)
    p.k = tensor(seed, STREAM_K, kshape, dtype, factor)
    p.v = tensor(seed, STREAM_V, kshape, dtype, factor)
    if with_do:
        p.do = tensor(seed, STREAM_DO, qshape, dtype, 1.0)
    p.meta = dict(seed=seed, factor=factor)
    return p


# The five workloads, stated by what they are.
WORKLOADS = {
    "fp16_noncausal_b1_h2_n128_d64": dict(
        dtype="fp16", batch=1, heads=2, kv_heads=2, seqlen=128, head_dim=64,
        causal=False, scale=1.0 / 8.0, factor=1.0),
    "bf16_causal_b4_h16_n2048_d64": dict(
        dtype="bf16", batch=4, heads=16, kv_heads=16, seqlen=2048, head_dim=64,
        causal=True, scale=1.0 / 8.0, factor=1.0),
    "bf16_causal_b1_h32_n8192_d128": dict(
        dtype="bf16", batch=1, heads=32, kv_heads=32, seqlen=8192, head_dim=128,
        causal=True, scale=1.0 / math.sqrt(128.0), factor=0.5),
    "bf16_causal_gqa_b1_h32kv8_n32768_d128": dict(
        dtype="bf16", batch=1, heads=32, kv_heads=8, seqlen=32768, head_dim=128,
        causal=True, scale=1.0 / math.sqrt(128.0), factor=0.5),
    # FP8 forward on the 8K shape: E4M3 inputs with per-tensor scales
    "fp8_causal_b1_h32_n8192_d128": dict(
        dtype="fp8", batch=1, heads=32, kv_heads=32, seqlen=8192, head_dim=128,
        causal=True, scale=1.0 / math.sqrt(128.0), factor=0.5),
    "fp16_causal_window4096_varlen_b2_h16_d128": dict(
        dtype="fp16", batch=2, heads=16, kv_heads=16, seqlen=16384, head_dim=128,
        causal=True, window=(4096, 0), scale=1.0 / math.sqrt(128.0), factor=1.0,
        varlen_range=(8192, 16384)),
}


def workload(name: str, seed: int = 0, with_do: bool = True) -> Problem:
    return make_problem(seed=seed, with_do=with_do, **WORKLOADS[name])


@dataclass
class DecodeProblem:
    """New query tokens against a key/value cache (CPU tensors).  The caches
    hold ``capacity`` rows per sequence, of which the first ``cache_lens[b]``
    are valid and already include the new tokens' own keys and values."""
    dtype: str
    batch: int
    heads: int
    kv_heads: int
    seqlen_q: int
    capacity: int
    head_dim: int
    causal: bool
    window_left: int = -1
    window_right: int = -1
    scale: float = 0.0
    cache_lens: list | None = None
    q: object = None
    k_cache: object = None
    v_cache: object = None

    def cache_seqlens(self):
        import torch
        return torch.tensor(self.cache_lens, dtype=torch.int32)


def make_decode(*, dtype: str, batch: int, heads: int, kv_heads: int, seqlen_q: int,
                capacity: int, head_dim: int, causal: bool, window=(-1, -1),
                scale: float | None = None, factor: float = 1.0, seed: int = 0,
                len_range=None, cache_lens=None) -> DecodeProblem:
    """Draw one decode problem.  ``len_range=(lo, hi)`` draws each sequence's
    cache length uniformly on [lo, hi] (stream 4); ``cache_lens`` gives them
    explicitly; by default every sequence fills the capacity."""
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    if cache_lens is not None:
        lens = [int(x) for x in cache_lens]
    elif len_range is not None:
        lens = [int(x) for x in uniform_ints(16 * seed + STREAM_LEN, batch, len_range[0], len_range[1])]
    else:
        lens = [capacity] * batch
    if len(lens) != batch or any(x < 0 or x > capacity for x in lens):
        raise ValueError("cache lengths must be one per sequence, within the capacity")
    p = DecodeProblem(dtype=dtype, batch=batch, heads=heads, kv_heads=kv_heads, seqlen_q=seqlen_q,
                      capacity=capacity, head_dim=head_dim, causal=causal, window_left=window[0],
                      window_right=window[1], scale=scale, cache_lens=lens)
    p.q = tensor(seed, STREAM_Q, (batch, seqlen_q, heads, head_dim), dtype, factor)
    p.k_cache = tensor(seed, STREAM_K, (batch, capacity, kv_heads, head_dim), dtype, factor)
    p.v_cache = tensor(seed, STREAM_V, (batch, capacity, kv_heads, head_dim), dtype, factor)
    return p


# Decode workloads: one new token per sequence of a GQA model with a long,
# ragged cache (the inference half of the long-context shape above), and a
# block of 8 new tokens per sequence on the same caches.
DECODE_WORKLOADS = {
    "bf16_decode_gqa_b8_h32kv8_q1_cache32768_d128": dict(
        dtype="bf16", batch=8, heads=32, kv_heads=8, seqlen_q=1, capacity=32768, head_dim=128,
        causal=True, factor=0.5, len_range=(16384, 32768)),
    "bf16_decode_gqa_b8_h32kv8_q8_cache32768_d128": dict(
        dtype="bf16", batch=8, heads=32, kv_heads=8, seqlen_q=8, capacity=32768, head_dim=128,
        causal=True, factor=0.5, len_range=(16384, 32768)),
}


def decode_workload(name: str, seed: int = 0) -> DecodeProblem:
    return make_decode(seed=seed, **DECODE_WORKLOADS[name])
