"""Exact tiled attention for AMD MI355X (gfx950): a thin Python binding over
the C-ABI library ``libfa.so`` (declared in ``include/fa.h``).

Every step of the computation runs in the library's HIP kernels; this module
only checks tensor metadata, passes ``data_ptr()`` values and the current
HIP stream, and maps status codes to exceptions.  PyTorch supplies device
memory and streams.  There is no fallback: if ``libfa.so`` is missing or the
device is not a gfx950, calls raise.

The call shapes follow flash_attn_func(q, k, v, dropout_p, softmax_scale,
causal) on (batch, seqlen, nheads, headdim) tensors from the FlashAttention-2
overview page (lshu.cn/news/55956, section 3.3), with window_size and packed
variable-length batches as named on the pages.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # first: libfa.so then binds to the HIP runtime torch already loaded

__all__ = [
    "FaError", "lib", "forward", "backward", "Plan", "flash_attn_func",
    "flash_attn_varlen_func", "workspace_size", "FA_DTYPE_F16", "FA_DTYPE_BF16",
    "forward_kvcache", "kvcache_workspace_size", "kvcache_splits", "DecodePlan",
    "flash_attn_with_kvcache", "new_dropout_seed", "forward_fp8", "Fp8Plan", "backward_noalloc",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1
_STATUS = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED",
           3: "FA_ERR_ARCH", 4: "FA_ERR_WORKSPACE", 5: "FA_ERR_LAUNCH"}
_lib = None


class FaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.fa_strerror(code).decode() if _lib is not None else ""
        super().__init__(f"{where}: {_STATUS.get(code, code)} ({msg})")


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library with argument types set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_tiled_attention_10_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    U64 = ctypes.c_uint64
    L.fa_fwd.argtypes = [P] * 9 + [I] * 9 + [F, F, U64, I, P]
    L.fa_fwd.restype = I
    L.fa_bwd_workspace_size.argtypes = [I] * 6
    L.fa_bwd_workspace_size.restype = S
    L.fa_bwd.argtypes = [P] * 10 + [S] + [P] * 4 + [I] * 9 + [F, F, U64, I, I, P]
    L.fa_bwd.restype = I
    L.fa_bwd_stage.argtypes = [I] + [P] * 10 + [S] + [P] * 4 + [I] * 9 + [F, F, U64, I, I, P]
    L.fa_bwd_stage.restype = I
    L.fa_bwd_noalloc.argtypes = [P] * 13 + [I] * 9 + [F, F, U64, I, P]
    L.fa_bwd_noalloc.restype = I
    L.fa_fwd_fp8.argtypes = [P] * 9 + [I] * 9 + [F, F, F, F, I, P]
    L.fa_fwd_fp8.restype = I
    L.fa_fwd_kvcache_workspace_size.argtypes = [I] * 7
    L.fa_fwd_kvcache_workspace_size.restype = S
    L.fa_fwd_kvcache.argtypes = [P] * 7 + [S] + [I] * 9 + [F, I, I, P]
    L.fa_fwd_kvcache.restype = I
    L.fa_fwd_kvcache_splits.argtypes = [I] * 7
    L.fa_fwd_kvcache_splits.restype = I
    L.fa_strerror.argtypes = [I]
    L.fa_strerror.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = I
    _lib = L
    return L


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    raise TypeError(f"attention inputs must be float16 or bfloat16, got {t.dtype}")


def _check(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (call .contiguous())")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class _Geom:
    """Sizes of one call, from the tensors (fixed length or packed)."""

    def __init__(self, q, k, cu_q, cu_k, max_q, max_k):
        self.varlen = cu_q is not None
        if self.varlen:
            if q.dim() != 3 or k.dim() != 3:
                raise ValueError("packed batches take q as (total_q, heads, d) and k/v as (total_k, kv_heads, d)")
            if cu_k is None:
                raise ValueError("cu_seqlens_q and cu_seqlens_k go together")
            if cu_q.dtype != torch.int32 or cu_k.dtype != torch.int32:
                raise TypeError("cu_seqlens must be int32")
            if cu_q.numel() != cu_k.numel() or cu_q.numel() < 1:
                raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold batch+1 entries")
            self.batch = cu_q.numel() - 1
            _, self.heads, self.d = q.shape
            _, self.kv_heads, dk = k.shape
            # the kernels index rows (and LSE) by the prefix sums: the query-side
            # tensors must hold exactly cu_seqlens_q[-1] rows, k / v at least cu_seqlens_k[-1]
            ends = torch.stack([cu_q[-1], cu_k[-1]]).cpu().tolist()
            if ends[0] != q.shape[0]:
                raise ValueError(f"q holds {q.shape[0]} rows but cu_seqlens_q[-1] = {ends[0]}")
            if ends[1] > k.shape[0]:
                raise ValueError(f"k holds {k.shape[0]} rows but cu_seqlens_k[-1] = {ends[1]}")
            if max_q is None:
                max_q = int((cu_q[1:] - cu_q[:-1]).max().item()) if self.batch else 0
            if max_k is None:
                max_k = int((cu_k[1:] - cu_k[:-1]).max().item()) if self.batch else 0
            self.seqlen_q, self.seqlen_k = int(max_q), int(max_k)
            self.lse_shape = (self.heads, q.shape[0])
        else:
            if q.dim() != 4 or k.dim() != 4:
                raise ValueError("q, k, v must be (batch, seqlen, heads, head_dim)")
            self.batch, self.seqlen_q, self.heads, self.d = q.shape
            bk, self.seqlen_k, self.kv_heads, dk = k.shape
            if bk != self.batch:
                raise ValueError("q and k batch sizes differ")
            self.lse_shape = (self.batch, self.heads, self.seqlen_q)
        if dk != self.d:
            raise ValueError("q and k head_dim differ")


def _default_scale(d: int, softmax_scale):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def _seed(seed) -> int:
    return int(seed) & (2**64 - 1)


def new_dropout_seed() -> int:
    """A 64-bit dropout seed drawn from torch's default CPU generator."""
    return int(torch.randint(0, 2**62, (1,), dtype=torch.int64).item())


def _check_used(used, name, batch, device):
    if used is None:
        return
    _check(used, name, torch.int32, device)
    if used.shape != (batch,):
        raise ValueError(f"{name} must hold one int32 per sequence")


def forward(q, k, v, *, causal=False, window_size=(-1, -1), softmax_scale=None,
            cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
            out=None, lse=None, dropout_p=0.0, dropout_seed=0, seqused_q=None, seqused_k=None):
    """O and LSE of exact attention (see include/fa.h for the definition,
    dropout included).  Returns (out, lse); lse is float32 (batch, heads,
    seqlen_q) or (heads, total_q) for packed batches."""
    L = lib()
    dt = q.dtype
    _check(q, "q"); _check(k, "k", dt, q.device); _check(v, "v", dt, q.device)
    if k.shape != v.shape:
        raise ValueError("k and v shapes differ")
    if cu_seqlens_q is not None:
        _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, q.device)
        _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, q.device)
    g = _Geom(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    _check_used(seqused_q, "seqused_q", g.batch, q.device)
    _check_used(seqused_k, "seqused_k", g.batch, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dt, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None:
        lse = torch.empty(g.lse_shape, dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, q.device)
        if tuple(lse.shape) != g.lse_shape:
            raise ValueError(f"lse must have shape {g.lse_shape}")
    rc = L.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                  _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_q), _ptr(seqused_k),
                  g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k, g.d,
                  int(bool(causal)), int(window_size[0]), int(window_size[1]),
                  _default_scale(g.d, softmax_scale), float(dropout_p), _seed(dropout_seed),
                  _dtype_code(q), _stream(q.device))
    if rc != 0:
        raise FaError(rc, "fa_fwd")
    return out, lse


_FP8_TYPES = (torch.float8_e4m3fn, torch.uint8)


def _fp8_args(q, k, v, descale_q, descale_k, descale_v, causal, window_size, softmax_scale,
              cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, out, lse, out_dtype,
              seqused_q, seqused_k):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, None, q.device)
        if t.dtype not in _FP8_TYPES:
            raise TypeError(f"{name} must hold E4M3 codes (torch.float8_e4m3fn or uint8), got {t.dtype}")
    if k.shape != v.shape:
        raise ValueError("k and v shapes differ")
    if cu_seqlens_q is not None:
        _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, q.device)
        _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, q.device)
    g = _Geom(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    _check_used(seqused_q, "seqused_q", g.batch, q.device)
    _check_used(seqused_k, "seqused_k", g.batch, q.device)
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float16")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    else:
        _check(out, "out", out_dtype, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None:
        lse = torch.empty(g.lse_shape, dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, q.device)
        if tuple(lse.shape) != g.lse_shape:
            raise ValueError(f"lse must have shape {g.lse_shape}")
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
            _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_q), _ptr(seqused_k),
            g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k, g.d,
            int(bool(causal)), int(window_size[0]), int(window_size[1]),
            _default_scale(g.d, softmax_scale), float(descale_q), float(descale_k), float(descale_v),
            FA_DTYPE_BF16 if out_dtype == torch.bfloat16 else FA_DTYPE_F16]
    return args, out, lse


def forward_fp8(q, k, v, descale_q=1.0, descale_k=1.0, descale_v=1.0, *, causal=False, window_size=(-1, -1),
                softmax_scale=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                max_seqlen_k=None, out=None, lse=None, out_dtype=torch.bfloat16, seqused_q=None,
                seqused_k=None):
    """FP8 forward: q, k, v hold E4M3 codes (torch.float8_e4m3fn, or their
    bytes as uint8), each tensor's values being its descale times the code's
    value.  Returns (out, lse): O in ``out_dtype`` (bf16 or fp16), LSE float32,
    of the attention of the dequantised inputs with P rounded to E4M3 before
    P.V (include/fa.h).  head_dim a multiple of 16 up to 128."""
    L = lib()
    args, out, lse = _fp8_args(q, k, v, descale_q, descale_k, descale_v, causal, window_size, softmax_scale,
                               cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, out, lse, out_dtype,
                               seqused_q, seqused_k)
    rc = L.fa_fwd_fp8(*args, _stream(q.device))
    if rc != 0:
        raise FaError(rc, "fa_fwd_fp8")
    return out, lse


class Fp8Plan:
    """Pre-resolved arguments of fa_fwd_fp8 on fixed buffers (benchmark
    loop); ``run()`` enqueues one call on ``stream`` (default: q's current
    torch stream)."""

    def __init__(self, q, k, v, descale_q=1.0, descale_k=1.0, descale_v=1.0, *, causal=False,
                 window_size=(-1, -1), softmax_scale=None, out_dtype=torch.bfloat16, stream=None):
        self._L = lib()
        self.q, self.k, self.v = q, k, v
        args, self.out, self.lse = _fp8_args(q, k, v, descale_q, descale_k, descale_v, causal, window_size,
                                             softmax_scale, None, None, None, None, None, None, out_dtype,
                                             None, None)
        self.stream = stream if stream is not None else torch.cuda.current_stream(q.device)
        self._args = args + [ctypes.c_void_p(self.stream.cuda_stream)]

    def run(self):
        rc = self._L.fa_fwd_fp8(*self._args)
        if rc != 0:
            raise FaError(rc, "fa_fwd_fp8")


def workspace_size(batch, heads, seqlen_q, head_dim, dtype, deterministic=True) -> int:
    code = dtype if isinstance(dtype, int) else (FA_DTYPE_BF16 if dtype == torch.bfloat16 else FA_DTYPE_F16)
    return int(lib().fa_bwd_workspace_size(batch, heads, seqlen_q, head_dim, code, int(bool(deterministic))))


def backward(dout, q, k, v, out, lse, *, causal=False, window_size=(-1, -1),
             softmax_scale=None, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, max_seqlen_k=None, dq=None, dk=None, dv=None,
             workspace=None, dropout_p=0.0, dropout_seed=0, seqused_q=None, seqused_k=None,
             deterministic=True):
    """dQ, dK, dV of exact attention for upstream gradient ``dout``, from the
    forward's ``out`` and ``lse`` (recomputing the scores).  By default
    (``deterministic=True``) dQ comes from the separate dQ pass and every call
    gives the same bytes; ``deterministic=False`` lets head dims up to 128
    accumulate dQ with float32 atomics inside the key-tile pass instead (its
    last bits then vary from call to call; slower on MI355X, whose L2 float
    atomics are the bottleneck there).  See include/fa.h."""
    L = lib()
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check(t, name, dt, q.device)
    _check(lse, "lse", torch.float32, q.device)
    if cu_seqlens_q is not None:
        _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, q.device)
        _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, q.device)
    g = _Geom(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if k.shape != v.shape:
        raise ValueError("k and v shapes differ")
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    if tuple(lse.shape) != g.lse_shape:
        raise ValueError(f"lse must have shape {g.lse_shape}")
    det = int(bool(deterministic))
    _check_used(seqused_q, "seqused_q", g.batch, q.device)
    _check_used(seqused_k, "seqused_k", g.batch, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check(t, name, dt, q.device)
        if t.shape != like.shape:
            raise ValueError(f"{name} must have the shape of its input")
    need = int(L.fa_bwd_workspace_size(g.batch, g.heads, g.seqlen_q, g.d, _dtype_code(q), det))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    rc = L.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                  _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_q), _ptr(seqused_k),
                  g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k, g.d,
                  int(bool(causal)), int(window_size[0]), int(window_size[1]),
                  _default_scale(g.d, softmax_scale), float(dropout_p), _seed(dropout_seed),
                  _dtype_code(q), det, _stream(q.device))
    if rc != 0:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv


def backward_noalloc(dout, q, k, v, out, lse, dq, dk, dv, *, causal=False, window_size=(-1, -1),
                     softmax_scale=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                     max_seqlen_k=None, dropout_p=0.0, dropout_seed=0, seqused_q=None, seqused_k=None):
    """fa_bwd_noalloc: the deterministic backward into caller-given dq, dk, dv
    with the library's own per-device workspace (no allocation by the library
    or here; batch * heads * seqlen_q at most 2^21; overlapping calls on one
    GPU race, see include/fa.h)."""
    L = lib()
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, dt, q.device)
    _check(lse, "lse", torch.float32, q.device)
    g = _Geom(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    for name, t, like in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != like.shape:
            raise ValueError(f"{name} must have the shape of {'q' if like is q else 'k'}")
    if tuple(lse.shape) != g.lse_shape:
        raise ValueError(f"lse must have shape {g.lse_shape}")
    rc = L.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                          _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_q), _ptr(seqused_k),
                          g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k, g.d,
                          int(bool(causal)), int(window_size[0]), int(window_size[1]),
                          _default_scale(g.d, softmax_scale), float(dropout_p), _seed(dropout_seed),
                          _dtype_code(q), _stream(q.device))
    if rc != 0:
        raise FaError(rc, "fa_bwd_noalloc")
    return dq, dk, dv


class Plan:
    """Pre-resolved C-ABI arguments for repeated calls on fixed buffers (the
    benchmark loop): ``fwd()`` runs fa_fwd, ``bwd_stage(s)`` one backward
    kernel, ``bwd()`` all three, each enqueued on ``stream`` (default: the
    current torch stream of q's device).  Buffers are allocated once here.
    ``deterministic`` selects the backward's dQ path as in ``backward``."""

    def __init__(self, q, k, v, dout=None, *, causal=False, window_size=(-1, -1), softmax_scale=None,
                 cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, stream=None,
                 dropout_p=0.0, dropout_seed=0, seqused_q=None, seqused_k=None, deterministic=True):
        L = lib()
        dt = q.dtype
        _check(q, "q"); _check(k, "k", dt, q.device); _check(v, "v", dt, q.device)
        g = _Geom(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
        _check_used(seqused_q, "seqused_q", g.batch, q.device)
        _check_used(seqused_k, "seqused_k", g.batch, q.device)
        self.geom = g
        self.q, self.k, self.v, self.dout = q, k, v, dout
        self.out = torch.empty_like(q)
        self.lse = torch.empty(g.lse_shape, dtype=torch.float32, device=q.device)
        self.cu_q, self.cu_k = cu_seqlens_q, cu_seqlens_k
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        self.stream = st
        sp = ctypes.c_void_p(st.cuda_stream)
        common = [g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k, g.d,
                  int(bool(causal)), int(window_size[0]), int(window_size[1]),
                  _default_scale(g.d, softmax_scale), float(dropout_p), _seed(dropout_seed),
                  _dtype_code(q)]
        self.deterministic = bool(deterministic)
        self._used = (seqused_q, seqused_k)
        self._fwd = [_ptr(q), _ptr(k), _ptr(v), _ptr(self.out), _ptr(self.lse),
                     _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(seqused_q), _ptr(seqused_k)] + common + [sp]
        if dout is not None:
            _check(dout, "dout", dt, q.device)
            self.dq, self.dk, self.dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            det = int(self.deterministic)
            need = int(L.fa_bwd_workspace_size(g.batch, g.heads, g.seqlen_q, g.d, _dtype_code(q), det))
            self.workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
            self._bwd = [_ptr(q), _ptr(k), _ptr(v), _ptr(self.out), _ptr(self.lse), _ptr(dout),
                         _ptr(self.dq), _ptr(self.dk), _ptr(self.dv), _ptr(self.workspace),
                         self.workspace.numel(), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                         _ptr(seqused_q), _ptr(seqused_k)] + common + [det, sp]
        self._L = L

    def fwd(self):
        rc = self._L.fa_fwd(*self._fwd)
        if rc != 0:
            raise FaError(rc, "fa_fwd")

    def bwd_stage(self, stage: int):
        rc = self._L.fa_bwd_stage(stage, *self._bwd)
        if rc != 0:
            raise FaError(rc, f"fa_bwd_stage({stage})")

    def bwd(self):
        rc = self._L.fa_bwd(*self._bwd)
        if rc != 0:
            raise FaError(rc, "fa_bwd")


class _FlashAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, softmax_scale, causal, window_size, cu_q, cu_k, max_q, max_k,
                dropout_p, dropout_seed, used_q, used_k, deterministic):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, lse = forward(q, k, v, causal=causal, window_size=window_size,
                           softmax_scale=softmax_scale, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                           max_seqlen_q=max_q, max_seqlen_k=max_k,
                           dropout_p=dropout_p, dropout_seed=dropout_seed, seqused_q=used_q, seqused_k=used_k)
        ctx.save_for_backward(q, k, v, out, lse, cu_q, cu_k, used_q, used_k)
        ctx.args = (softmax_scale, causal, window_size, max_q, max_k, dropout_p, dropout_seed, deterministic)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, cu_q, cu_k, used_q, used_k = ctx.saved_tensors
        softmax_scale, causal, window_size, max_q, max_k, dropout_p, dropout_seed, deterministic = ctx.args
        dq, dk, dv = backward(dout.contiguous(), q, k, v, out, lse, causal=causal,
                              window_size=window_size, softmax_scale=softmax_scale,
                              cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                              max_seqlen_q=max_q, max_seqlen_k=max_k,
                              dropout_p=dropout_p, dropout_seed=dropout_seed, seqused_q=used_q, seqused_k=used_k,
                              deterministic=deterministic)
        return dq, dk, dv, None, None, None, None, None, None, None, None, None, None, None, None


def flash_attn_func(q, k, v, dropout_p=0.0, softmax_scale=None, causal=False,
                    window_size=(-1, -1), dropout_seed=None, seqused_q=None, seqused_k=None,
                    deterministic=True):
    """Autograd entry with the call shape the pages use.  With dropout_p > 0
    and no dropout_seed, a seed is drawn from torch's default generator; the
    backward reuses the forward's seed.  seqused_q / seqused_k (int32 per
    sequence) make a padded batch: only the first rows of each sequence
    count, the rest of the output and gradients is zero."""
    if dropout_p > 0.0 and dropout_seed is None:
        dropout_seed = new_dropout_seed()
    return _FlashAttn.apply(q, k, v, softmax_scale, causal, tuple(window_size), None, None, None, None,
                            float(dropout_p), 0 if dropout_seed is None else dropout_seed, seqused_q, seqused_k,
                            bool(deterministic))


def flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                           dropout_p=0.0, softmax_scale=None, causal=False, window_size=(-1, -1),
                           dropout_seed=None, deterministic=True):
    """Packed variable-length batches: q (total_q, heads, d), k/v (total_k,
    kv_heads, d), int32 prefix sums cu_seqlens_*; dropout as flash_attn_func."""
    if dropout_p > 0.0 and dropout_seed is None:
        dropout_seed = new_dropout_seed()
    return _FlashAttn.apply(q, k, v, softmax_scale, causal, tuple(window_size),
                            cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                            float(dropout_p), 0 if dropout_seed is None else dropout_seed, None, None,
                            bool(deterministic))


# ---------------------------------------------------------------------------
# Decode over a key/value cache
# ---------------------------------------------------------------------------

def kvcache_workspace_size(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, num_splits=0) -> int:
    """Bytes of workspace fa_fwd_kvcache needs (partial O and LSE per split)."""
    return int(lib().fa_fwd_kvcache_workspace_size(batch, heads, kv_heads, seqlen_q, seqlen_k,
                                                   head_dim, num_splits))


def kvcache_splits(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, num_splits=0) -> int:
    """The number of waves fa_fwd_kvcache's split pass uses for these sizes."""
    return int(lib().fa_fwd_kvcache_splits(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, num_splits))


class _DecGeom:
    def __init__(self, q, k_cache, v_cache, cache_seqlens):
        if q.dim() != 4 or k_cache.dim() != 4:
            raise ValueError("q is (batch, seqlen_q, heads, d); caches are (batch, capacity, kv_heads, d)")
        if k_cache.shape != v_cache.shape:
            raise ValueError("k_cache and v_cache shapes differ")
        self.batch, self.seqlen_q, self.heads, self.d = q.shape
        bk, self.seqlen_k, self.kv_heads, dk = k_cache.shape
        if bk != self.batch:
            raise ValueError("q and cache batch sizes differ")
        if dk != self.d:
            raise ValueError("q and cache head_dim differ")
        if cache_seqlens is not None:
            _check(cache_seqlens, "cache_seqlens", torch.int32, q.device)
            if cache_seqlens.shape != (self.batch,):
                raise ValueError("cache_seqlens must hold one int32 per sequence")
        self.lse_shape = (self.batch, self.heads, self.seqlen_q)


def forward_kvcache(q, k_cache, v_cache, cache_seqlens=None, *, causal=False, window_size=(-1, -1),
                    softmax_scale=None, num_splits=0, out=None, lse=None, workspace=None):
    """Attention of the new tokens ``q`` over the first ``cache_seqlens[b]``
    rows of the caches (which already hold the new tokens' keys and values);
    see include/fa.h.  Returns (out, lse)."""
    L = lib()
    dt = q.dtype
    _check(q, "q"); _check(k_cache, "k_cache", dt, q.device); _check(v_cache, "v_cache", dt, q.device)
    g = _DecGeom(q, k_cache, v_cache, cache_seqlens)
    out = torch.empty_like(q) if out is None else out
    _check(out, "out", dt, q.device)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    lse = torch.empty(g.lse_shape, dtype=torch.float32, device=q.device) if lse is None else lse
    _check(lse, "lse", torch.float32, q.device)
    need = int(L.fa_fwd_kvcache_workspace_size(g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k,
                                               g.d, int(num_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    rc = L.fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _ptr(cache_seqlens),
                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                          g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k, g.d,
                          int(bool(causal)), int(window_size[0]), int(window_size[1]),
                          _default_scale(g.d, softmax_scale), _dtype_code(q), int(num_splits),
                          _stream(q.device))
    if rc != 0:
        raise FaError(rc, "fa_fwd_kvcache")
    return out, lse


def flash_attn_with_kvcache(q, k_cache, v_cache, cache_seqlens=None, softmax_scale=None, causal=False,
                            window_size=(-1, -1), num_splits=0):
    """Inference entry with the KV-cache call shape: returns the output only.
    The new tokens' keys and values must already be in the caches."""
    return forward_kvcache(q, k_cache, v_cache, cache_seqlens, causal=causal, window_size=window_size,
                           softmax_scale=softmax_scale, num_splits=num_splits)[0]


class DecodePlan:
    """Pre-resolved fa_fwd_kvcache arguments on fixed buffers (the benchmark
    loop): ``run()`` enqueues one decode call on ``stream``."""

    def __init__(self, q, k_cache, v_cache, cache_seqlens=None, *, causal=False, window_size=(-1, -1),
                 softmax_scale=None, num_splits=0, stream=None):
        L = lib()
        dt = q.dtype
        _check(q, "q"); _check(k_cache, "k_cache", dt, q.device); _check(v_cache, "v_cache", dt, q.device)
        g = _DecGeom(q, k_cache, v_cache, cache_seqlens)
        self.geom = g
        self.out = torch.empty_like(q)
        self.lse = torch.empty(g.lse_shape, dtype=torch.float32, device=q.device)
        self.nsplit = int(L.fa_fwd_kvcache_splits(g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k,
                                                  g.d, int(num_splits)))
        need = int(L.fa_fwd_kvcache_workspace_size(g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k,
                                                   g.d, int(num_splits)))
        self.workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        self.stream = st
        self._keep = (q, k_cache, v_cache, cache_seqlens)
        self._args = [_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(self.out), _ptr(self.lse),
                      _ptr(cache_seqlens), _ptr(self.workspace), self.workspace.numel(),
                      g.batch, g.heads, g.kv_heads, g.seqlen_q, g.seqlen_k, g.d,
                      int(bool(causal)), int(window_size[0]), int(window_size[1]),
                      _default_scale(g.d, softmax_scale), _dtype_code(q), int(num_splits),
                      ctypes.c_void_p(st.cuda_stream)]
        self._L = L

    def run(self):
        rc = self._L.fa_fwd_kvcache(*self._args)
        if rc != 0:
            raise FaError(rc, "fa_fwd_kvcache")
