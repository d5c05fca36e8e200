"""The C-ABI boundary on a CPU host: the library loads, exports every entry
point include/fa.h declares, and rejects bad arguments with the documented
codes before any HIP call.  No kernel runs here."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, INVALID, UNSUPPORTED, ARCH, WORKSPACE, LAUNCH = range(6)


@pytest.fixture(scope="module")
def L():
    import exact_tiled_attention_10_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        from exact_tiled_attention_10_amd import build
        build.build()
    return fa.lib()


# Fake, 256-byte aligned addresses: only ever passed where validation must
# reject the call before anything touches them, or on a host with no GPU.
FAKE = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(12)]
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="passes fake pointers; only safe where no GPU exists")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_noalloc", "fa_bwd_stage", "fa_bwd_workspace_size", "fa_fwd",
                                    "fa_fwd_fp8", "fa_fwd_kvcache", "fa_fwd_kvcache_splits",
                                    "fa_fwd_kvcache_workspace_size", "fa_strerror", "fa_version"]


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_strerror_and_version(L):
    assert L.fa_strerror(0) == b"ok"
    for code in range(1, 6):
        assert L.fa_strerror(code) not in (b"", b"unknown status")
    assert L.fa_strerror(99) == b"unknown status"
    assert L.fa_version() >= 10000


def fwd(L, **over):
    args = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], o=FAKE[3], lse=FAKE[4], cu_q=None, cu_k=None,
                used_q=None, used_k=None, batch=1, heads=4, kv_heads=2, seqlen_q=128, seqlen_k=128, head_dim=128,
                causal=1, left=-1, right=-1, scale=0.125, drop=0.0, seed=0, dtype=1, stream=None)
    args.update(over)
    return L.fa_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["cu_q"], args["cu_k"],
                    args["used_q"], args["used_k"], args["batch"], args["heads"], args["kv_heads"], args["seqlen_q"], args["seqlen_k"],
                    args["head_dim"], args["causal"], args["left"], args["right"], args["scale"],
                    args["drop"], args["seed"], args["dtype"], args["stream"])


def bwd(L, **over):
    args = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], o=FAKE[3], lse=FAKE[4], do=FAKE[5], dq=FAKE[6],
                dk=FAKE[7], dv=FAKE[8], ws=FAKE[9], wsb=1 << 20, cu_q=None, cu_k=None,
                used_q=None, used_k=None, batch=1, heads=4, kv_heads=2, seqlen_q=128, seqlen_k=128, head_dim=128,
                causal=1, left=-1, right=-1, scale=0.125, drop=0.0, seed=0, dtype=1, det=1, stream=None)
    args.update(over)
    return L.fa_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"], args["dq"],
                    args["dk"], args["dv"], args["ws"], args["wsb"], args["cu_q"], args["cu_k"],
                    args["used_q"], args["used_k"], args["batch"], args["heads"], args["kv_heads"], args["seqlen_q"], args["seqlen_k"],
                    args["head_dim"], args["causal"], args["left"], args["right"], args["scale"],
                    args["drop"], args["seed"], args["dtype"], args["det"], args["stream"])


BAD_FWD = [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(lse=None), INVALID),
    (dict(q=ctypes.c_void_p(0x10008)), INVALID),        # misaligned
    (dict(batch=-1), INVALID), (dict(heads=0), INVALID), (dict(kv_heads=0), INVALID),
    (dict(heads=6, kv_heads=4), INVALID), (dict(seqlen_q=-1), INVALID), (dict(seqlen_k=-5), INVALID),
    (dict(causal=2), INVALID), (dict(left=-2), INVALID), (dict(right=-3), INVALID),
    (dict(scale=-0.5), INVALID), (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(cu_q=FAKE[10]), INVALID),                      # only one of the pair
    (dict(drop=-0.1), INVALID), (dict(drop=1.0), INVALID), (dict(drop=float("nan")), INVALID),
    (dict(used_q=FAKE[11], cu_q=FAKE[10], cu_k=FAKE[9]), INVALID),   # padded lengths with a packed batch
    (dict(used_k=ctypes.c_void_p(0x10002)), INVALID),                # misaligned
    (dict(heads=1 << 16, kv_heads=2), INVALID),  # heads x head_dim = 2^23: tile offsets past 32 bits
    (dict(head_dim=100), UNSUPPORTED), (dict(head_dim=264), UNSUPPORTED), (dict(head_dim=0), UNSUPPORTED),
    (dict(head_dim=252), UNSUPPORTED), (dict(head_dim=4), UNSUPPORTED), (dict(head_dim=-8), UNSUPPORTED),
    (dict(head_dim=512), UNSUPPORTED),
    (dict(dtype=2), UNSUPPORTED), (dict(dtype=-1), UNSUPPORTED),
]


@pytest.mark.parametrize("over,code", BAD_FWD)
def test_fwd_rejects_bad_arguments(L, over, code):
    assert fwd(L, **over) == code


def fwd8(L, **over):
    args = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], o=FAKE[3], lse=FAKE[4], cu_q=None, cu_k=None,
                used_q=None, used_k=None, batch=1, heads=4, kv_heads=2, seqlen_q=128, seqlen_k=128, head_dim=128,
                causal=1, left=-1, right=-1, scale=0.125, dq=0.01, dk=0.02, dv=0.5, dtype=1, stream=None)
    args.update(over)
    return L.fa_fwd_fp8(args["q"], args["k"], args["v"], args["o"], args["lse"], args["cu_q"], args["cu_k"],
                        args["used_q"], args["used_k"], args["batch"], args["heads"], args["kv_heads"],
                        args["seqlen_q"], args["seqlen_k"], args["head_dim"], args["causal"], args["left"],
                        args["right"], args["scale"], args["dq"], args["dk"], args["dv"], args["dtype"],
                        args["stream"])


BAD_FWD8 = [
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(o=ctypes.c_void_p(0x10008)), INVALID),
    (dict(dq=-1.0), INVALID), (dict(dk=float("nan")), INVALID), (dict(dv=float("inf")), INVALID),
    (dict(scale=-1.0), INVALID), (dict(scale=1e30, dq=1e30, dk=1e30), INVALID),   # product overflows
    (dict(heads=6, kv_heads=4), INVALID), (dict(causal=3), INVALID), (dict(cu_k=FAKE[10]), INVALID),
    (dict(used_q=FAKE[11], cu_q=FAKE[10], cu_k=FAKE[9]), INVALID),
    (dict(heads=1 << 16, kv_heads=2), INVALID),
    (dict(head_dim=40), UNSUPPORTED), (dict(head_dim=8), UNSUPPORTED), (dict(head_dim=256), UNSUPPORTED),
    (dict(head_dim=144), UNSUPPORTED),
    (dict(dtype=2), UNSUPPORTED),
]


@pytest.mark.parametrize("over,code", BAD_FWD8)
def test_fwd_fp8_rejects_bad_arguments(L, over, code):
    assert fwd8(L, **over) == code


BAD_BWD = [
    (dict(do=None), INVALID), (dict(dq=None), INVALID), (dict(dk=None), INVALID),
    (dict(dv=None), INVALID), (dict(ws=None), INVALID),
    (dict(dv=ctypes.c_void_p(0x10004)), INVALID),
    (dict(heads=3, kv_heads=2), INVALID), (dict(head_dim=36), UNSUPPORTED),
    (dict(heads=1 << 16, kv_heads=2), INVALID),
    (dict(wsb=2 * 4 * 4 * 128 - 4), WORKSPACE), (dict(wsb=0), WORKSPACE),
    (dict(drop=1.5), INVALID), (dict(drop=float("inf")), INVALID),
    (dict(det=2), INVALID), (dict(det=-1), INVALID),
    (dict(ws=ctypes.c_void_p(0x10008)), INVALID),       # workspace must be 16-byte aligned
    # the atomic path needs the dQ accumulator too: the deterministic size is short
    (dict(det=0, wsb=2 * 4 * 4 * 128), WORKSPACE),
]


@pytest.mark.parametrize("over,code", BAD_BWD)
def test_bwd_rejects_bad_arguments(L, over, code):
    assert bwd(L, **over) == code


@pytest.mark.parametrize("stage", [-1, 3, 100])
def test_bwd_stage_rejects_unknown_stage(L, stage):
    args = [FAKE[i] for i in range(10)] + [1 << 20, None, None, None, None, 1, 4, 2, 128, 128, 128, 1, -1, -1,
                                           0.125, 0.0, 0, 1, 1, None]
    assert L.fa_bwd_stage(stage, *args) == INVALID


def test_bwd_stage_validates_like_fa_bwd(L):
    for det in (0, 1):
        args = [FAKE[i] for i in range(10)] + [16, None, None, None, None, 1, 4, 2, 128, 128, 128, 1, -1, -1,
                                               0.125, 0.1, 7, 1, det, None]
        for stage in range(3):
            assert L.fa_bwd_stage(stage, *args) == WORKSPACE


def test_workspace_size(L):
    f = L.fa_bwd_workspace_size
    # deterministic: D and lse2, one float per (row, head) each
    assert f(2, 8, 1000, 128, 1, 1) == 2 * (2 * 8 * 1000 * 4)
    assert f(1, 4, 128, 64, 0, 1) == 2 * (4 * 128 * 4)
    assert f(0, 4, 128, 64, 0, 1) == 4 and f(0, 4, 128, 64, 0, 0) == 4  # never zero for valid sizes
    assert f(1, 4, 128, 96, 0, 1) == 2 * (4 * 128 * 4) and f(1, 4, 128, 8, 1, 1) == 2 * (4 * 128 * 4)
    assert f(1, 4, 128, 100, 0, 1) == 0 and f(1, 0, 128, 64, 0, 1) == 0 and f(1, 4, 128, 64, 7, 1) == 0
    assert f(1, 4, 128, 64, 0, 2) == 0 and f(1, 4, 128, 64, 0, -1) == 0
    # atomic dQ: first a float32 accumulator of the tile width (64 or 128), padded to 256 bytes
    acc = lambda rows, w: -(-rows * w * 4 // 256) * 256
    assert f(2, 8, 1000, 128, 1, 0) == acc(2 * 8 * 1000, 128) + 2 * (2 * 8 * 1000 * 4)
    assert f(1, 4, 128, 96, 0, 0) == acc(4 * 128, 128) + 2 * (4 * 128 * 4)
    assert f(1, 3, 5, 8, 0, 0) == acc(15, 64) + 2 * (15 * 4)
    # head_dim above 128 always runs the separate dQ pass: no accumulator
    assert f(1, 4, 128, 256, 1, 0) == f(1, 4, 128, 256, 1, 1) == 2 * (4 * 128 * 4)


@no_gpu
def test_valid_call_without_gfx950_reports_arch(L):
    assert fwd(L) == ARCH
    assert bwd(L) == ARCH
    assert fwd(L, drop=0.1, seed=2**64 - 1) == ARCH and bwd(L, drop=0.999, seed=3) == ARCH
    assert fwd(L, used_q=FAKE[10], used_k=FAKE[11]) == ARCH and bwd(L, used_k=FAKE[11]) == ARCH
    assert fwd8(L) == ARCH and fwd8(L, head_dim=64, dtype=0, dq=0.0) == ARCH
    assert fwd8(L, head_dim=16) == ARCH and fwd8(L, head_dim=96) == ARCH and fwd8(L, head_dim=112) == ARCH
    # empty tensors may be NULL: no keys, no queries, empty batch
    assert fwd(L, k=None, v=None, seqlen_k=0) == ARCH
    assert fwd(L, q=None, o=None, lse=None, seqlen_q=0) == ARCH
    assert bwd(L, k=None, v=None, dk=None, dv=None, seqlen_k=0) == ARCH
    # just below the tile-offset bound on heads x head_dim (2^23)
    assert fwd(L, heads=(1 << 16) - 2, kv_heads=2) == ARCH
    assert bwd(L, heads=(1 << 16) - 2, kv_heads=2, wsb=1 << 40) == ARCH


def test_null_pointers_only_for_empty_tensors(L):
    assert fwd(L, k=None, seqlen_k=1) == INVALID
    assert fwd(L, q=None, seqlen_k=0) == INVALID
    assert bwd(L, dq=None, seqlen_k=0) == INVALID
    assert bwd(L, dk=None, seqlen_q=0) == INVALID


def test_python_binding_fails_loudly_without_gpu_tensors():
    import exact_tiled_attention_10_amd as fa
    q = torch.zeros(1, 8, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, q, q)


# ---------------------------------------------------------------------------
# Decode over a key/value cache
# ---------------------------------------------------------------------------

def dec(L, **over):
    args = dict(q=FAKE[0], kc=FAKE[1], vc=FAKE[2], o=FAKE[3], lse=FAKE[4], lens=FAKE[5], ws=FAKE[6],
                wsb=1 << 24, batch=2, heads=8, kv_heads=2, seqlen_q=1, seqlen_k=4096, head_dim=128,
                causal=1, left=-1, right=-1, scale=0.125, dtype=1, splits=0, stream=None)
    args.update(over)
    return L.fa_fwd_kvcache(args["q"], args["kc"], args["vc"], args["o"], args["lse"], args["lens"],
                            args["ws"], args["wsb"], args["batch"], args["heads"], args["kv_heads"],
                            args["seqlen_q"], args["seqlen_k"], args["head_dim"], args["causal"],
                            args["left"], args["right"], args["scale"], args["dtype"], args["splits"],
                            args["stream"])


BAD_DEC = [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(vc=None), INVALID), (dict(o=None), INVALID),
    (dict(lse=None), INVALID), (dict(ws=None), INVALID),
    (dict(ws=ctypes.c_void_p(0x10008)), INVALID),        # workspace must be 16-byte aligned
    (dict(lens=ctypes.c_void_p(0x10002)), INVALID),
    (dict(kc=ctypes.c_void_p(0x10008)), INVALID),
    (dict(heads=6, kv_heads=4), INVALID), (dict(seqlen_q=-1), INVALID), (dict(causal=3), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(left=-7), INVALID),
    (dict(head_dim=84), UNSUPPORTED), (dict(head_dim=264), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED),
    (dict(batch=1 << 16, seqlen_k=1 << 20), INVALID),      # 2^16 x 2^15 steps: beyond 32 bits
    (dict(batch=1 << 20, heads=2048, kv_heads=2048), INVALID),  # 2^31 output rows
    (dict(wsb=16), WORKSPACE),
    (dict(wsb=(512 + 2 * 2) * 32 * 129 * 4 + 3 * 8 - 1), WORKSPACE),  # one byte short (512 waves)
]


@pytest.mark.parametrize("over,code", BAD_DEC)
def test_kvcache_rejects_bad_arguments(L, over, code):
    assert dec(L, **over) == code


def test_kvcache_split_plan(L):
    splits, size = L.fa_fwd_kvcache_splits, L.fa_fwd_kvcache_workspace_size
    # auto: about 512 waves (two per CU), a multiple of kv_heads ...
    assert splits(8, 32, 8, 1, 32768, 128, 0) == 512
    assert splits(8, 32, 8, 1, 32768, 64, 0) == 512
    assert splits(8, 36, 12, 1, 32768, 64, 0) == 504
    # ... capped at one group (kv_heads waves) per 32-key step of every (sequence, row block)
    assert splits(1, 2, 2, 1, 100, 128, 0) == 2 * 4   # 2 segments x 4 steps
    assert splits(1, 32, 8, 1, 0, 128, 0) == 8         # empty cache: one group of kv_heads waves
    # num_splits > 0: waves per (sequence, kv head, row block); row blocks = ceil(g * seqlen_q / 32)
    assert splits(2, 8, 2, 1, 4096, 128, 5) == 5 * 2 * 2
    assert splits(2, 16, 2, 8, 4096, 128, 3) == 3 * 2 * 2 * 2  # 64 rows per kv head: 2 row blocks
    assert splits(2, 8, 2, 1, 4096, 128, 5000) == 2 * 2 * 128  # one step per wave at most
    assert splits(64, 8, 8, 1, 1 << 20, 128, 5000) == 65536
    assert splits(1, 3, 2, 1, 64, 128, 0) == 0 and splits(1, 4, 2, 1, 64, 100, 0) == 0  # invalid
    # workspace: (groups + sequences x row blocks) x kv_heads slots of 32 rows x (tile width + 1)
    # floats, then batch + 1 int64; the tile width is 64 or 128, the smallest holding head_dim
    for b, h, hk, nq, nk, d, ns in [(8, 32, 8, 1, 32768, 128, 0), (2, 16, 2, 8, 1000, 64, 3),
                                    (1, 4, 1, 16, 33, 128, 0), (3, 4, 2, 2, 64, 64, 7),
                                    (2, 8, 2, 1, 500, 96, 0), (2, 8, 2, 1, 500, 40, 2)]:
        w = splits(b, h, hk, nq, nk, d, ns)
        seg = b * hk * ((h // hk * nq + 31) // 32)
        tw = 64 if d <= 64 else 128
        assert size(b, h, hk, nq, nk, d, ns) == (w + seg) * 32 * (tw + 1) * 4 + (b + 1) * 8
    assert size(1, 4, 2, 1, 100, 100, 0) == 0 and size(1, 4, 3, 1, 100, 64, 0) == 0


@no_gpu
def test_kvcache_valid_call_without_gfx950_reports_arch(L):
    assert dec(L) == ARCH
    assert dec(L, lens=None) == ARCH                    # every sequence fills the capacity
    assert dec(L, kc=None, vc=None, seqlen_k=0) == ARCH  # empty caches may be NULL
    assert dec(L, q=None, o=None, lse=None, ws=None, seqlen_q=0) == ARCH


def test_kvcache_binding_fails_loudly_without_gpu_tensors():
    import exact_tiled_attention_10_amd as fa
    q = torch.zeros(1, 1, 2, 64, dtype=torch.float16)
    kc = torch.zeros(1, 16, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_kvcache(q, kc, kc)


@no_gpu
def test_header_compiles_as_c_and_a_c_client_runs(tmp_path, L):
    """include/fa.h is plain C: a C11 program (gcc, -Wall -Werror) includes it,
    links libfa.so and gets the documented codes from the argument checks."""
    import subprocess
    import exact_tiled_attention_10_amd as fa
    src = os.path.join(ROOT, "tests", "c_abi", "check_abi.c")
    exe = str(tmp_path / "check_abi")
    libdir = os.path.dirname(fa.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                    "-L", libdir, "-l:libfa.so", "-Wl,-rpath," + libdir, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
