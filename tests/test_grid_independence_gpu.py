"""Grid-independence of the kernels' results (an LDS-hazard smoke).

Every workgroup of the forward and backward kernels computes its outputs
from its own inputs and its own LDS, synchronised only inside itself, so the
bytes of one sequence must not depend on what else is in the launch: the
same sequence alone (batch 1), at another batch position of a larger batch
(different grid, workgroup order, XCD placement and co-resident
workgroups), inside a packed batch between other sequences, and while an
unrelated large call runs on a second stream, has to give identical O, LSE,
dQ, dK and dV bytes.  A missing barrier or a stage reused too early shows up
as a difference that depends on scheduling.  The atomic-dQ backward adds dQ
in scheduling order, so on that path dQ is left out (its dK, dV are fixed).
"""
import sys

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
        pytest.skip("needs a GPU")
    import exact_tiled_attention_10_amd as m
    return m


def run(fa, q, k, v, do, cu=None, max_len=None, deterministic=True, **mask):
    kw = dict(mask)
    if cu is not None:
        kw.update(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=max_len, max_seqlen_k=max_len)
    o, lse = fa.forward(q, k, v, **kw)
    dq, dk, dv = fa.backward(do, q, k, v, o, lse, deterministic=deterministic, **kw)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def same_bytes(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


def dev_problem(seed, **cfg):
    p = synth.make_problem(seed=seed, **cfg)
    d = torch.device("cuda:0")
    return p, p.q.to(d), p.k.to(d), p.v.to(d), p.do.to(d)


FIXED = {
    "bf16_d128_causal_gqa": dict(dtype="bf16", heads=8, kv_heads=2, seqlen=1024, head_dim=128, causal=True),
    "fp16_d64_noncausal": dict(dtype="fp16", heads=4, kv_heads=4, seqlen=777, head_dim=64, causal=False),
    "bf16_d128_window": dict(dtype="bf16", heads=4, kv_heads=1, seqlen=1500, head_dim=128, causal=True,
                             window=(200, 0)),
}


@pytest.mark.parametrize("det", [True, False], ids=["dq_pass", "atomic_dq"])
@pytest.mark.parametrize("name", list(FIXED))
def test_batch_position(fa, name, det):
    """Sequence s alone equals the same sequence at position 1 of a batch of 3."""
    say(f"[grid] {name} deterministic={det}")
    cfg = FIXED[name]
    mask = dict(causal=cfg["causal"], window_size=cfg.get("window", (-1, -1)))
    p1, q1, k1, v1, do1 = dev_problem(5, batch=1, **cfg)
    p3, q3, k3, v3, do3 = dev_problem(6, batch=3, **cfg)
    for t3, t1 in ((q3, q1), (k3, k1), (v3, v1), (do3, do1)):
        t3[1].copy_(t1[0])
    mask["softmax_scale"] = p1.scale
    a = run(fa, q1, k1, v1, do1, deterministic=det, **mask)
    b = run(fa, q3, k3, v3, do3, deterministic=det, **mask)
    torch.cuda.synchronize()
    for n in ("o", "dq", "dk", "dv"):
        if n == "dq" and not det:
            continue
        same_bytes(b[n][1], a[n][0], f"{name} {n}")
    same_bytes(b["lse"][1], a["lse"][0], f"{name} lse")


def test_packed_position(fa):
    """A sequence alone equals the same sequence between two others in a packed batch."""
    say("[grid] packed fp16 d128 window")
    cfg = dict(dtype="fp16", heads=4, kv_heads=2, head_dim=128, causal=True, window=(128, 0))
    mask = dict(causal=True, window_size=(128, 0))
    pa, qa, ka, va, doa = dev_problem(7, seqlens=[1000], seqlen=1000, batch=1, **cfg)
    pb, qb, kb, vb, dob = dev_problem(8, seqlens=[300, 1000, 517], seqlen=1000, batch=3, **cfg)
    lo, hi = 300, 1300
    for tb, ta in ((qb, qa), (kb, ka), (vb, va), (dob, doa)):
        tb[lo:hi].copy_(ta)
    mask["softmax_scale"] = pa.scale
    cua = pa.cu_seqlens().to(qa.device)
    cub = pb.cu_seqlens().to(qa.device)
    a = run(fa, qa, ka, va, doa, cu=cua, max_len=1000, **mask)
    b = run(fa, qb, kb, vb, dob, cu=cub, max_len=1000, **mask)
    torch.cuda.synchronize()
    for n in ("o", "dq", "dk", "dv"):
        same_bytes(b[n][lo:hi], a[n], f"packed {n}")
    same_bytes(b["lse"][:, lo:hi], a["lse"], "packed lse")


def test_concurrent_stream(fa):
    """The same call, alone and while a large unrelated call runs on a second
    stream (both at the default priority), gives the same bytes."""
    say("[grid] concurrent stream")
    cfg = FIXED["bf16_d128_causal_gqa"]
    mask = dict(causal=True, window_size=(-1, -1))
    p, q, k, v, do = dev_problem(9, batch=2, **cfg)
    mask["softmax_scale"] = p.scale
    ref = run(fa, q, k, v, do, **mask)
    torch.cuda.synchronize()
    pb, qb, kb, vb, dob = dev_problem(10, batch=2, dtype="bf16", heads=16, kv_heads=16, seqlen=4096,
                                      head_dim=128, causal=True)
    s_big, s_small = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(2):
        with torch.cuda.stream(s_big):
            run(fa, qb, kb, vb, dob, causal=True, softmax_scale=pb.scale)
        with torch.cuda.stream(s_small):
            got = run(fa, q, k, v, do, **mask)
        torch.cuda.synchronize()
        for n in ("o", "lse", "dq", "dk", "dv"):
            same_bytes(got[n], ref[n], f"concurrent {n}")


def test_forward_launch_shape(fa):
    """At head_dim 128 the forward runs 4-wave workgroups on grids of fewer than
    four 8-wave workgroups per CU and 8-wave ones otherwise: a sequence alone
    (32 heads x 4 query tiles of 256 rows: 128 workgroups) and the same
    sequence inside a batch of 8 (1024 workgroups) take the two shapes, and
    their bytes must agree."""
    say("[grid] forward launch shape")
    cfg = dict(dtype="bf16", heads=32, kv_heads=8, seqlen=1024, head_dim=128, causal=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 32 * 4 < 4 * cus <= 8 * 32 * 4, "the two grids must fall on both sides of the switch"
    mask = dict(causal=True, window_size=(-1, -1))
    p1, q1, k1, v1, do1 = dev_problem(11, batch=1, **cfg)
    p8, q8, k8, v8, do8 = dev_problem(12, batch=8, **cfg)
    for t8, t1 in ((q8, q1), (k8, k1), (v8, v1), (do8, do1)):
        t8[5].copy_(t1[0])
    mask["softmax_scale"] = p1.scale
    a = run(fa, q1, k1, v1, do1, **mask)
    b = run(fa, q8, k8, v8, do8, **mask)
    torch.cuda.synchronize()
    for n in ("o", "dq", "dk", "dv"):
        same_bytes(b[n][5], a[n][0], f"launch shape {n}")
    same_bytes(b["lse"][5], a["lse"][0], "launch shape lse")
