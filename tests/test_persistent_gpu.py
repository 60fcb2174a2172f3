"""GPU tests of the persistent causal launches.

For causal self-attention (Nq = Nk, no key padding) with more query (or key)
blocks than the device holds at once, the forward kernel and the two backward
kernels run one workgroup per resident slot, each working through a fixed
list of blocks: the blocks of a head are paired heavy with light (block r with
block n - 1 - r), each XCD owns a contiguous range of pairs and its
workgroups take them in turn. A single head has too few blocks for that, so
running the same inputs head by head takes the one-block-per-workgroup
launch. The two must agree bit for bit (every block is the same computation
whichever workgroup runs it), and sampled heads are also checked against the
oracle. The shapes are chosen so that the pairs share out evenly over the
256 CUs (forward, one workgroup per CU) and over 512 slots (backward with
D = 128, two per CU; 768 with D = 64, three per CU), including an odd block count, where the middle block
has no partner.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as orc
from test_backward_gpu import check_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    import flashattention_online_softmax_forward_amd as m
    from flashattention_online_softmax_forward_amd import _lib

    _lib.load()
    return m


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def pairs_fill(n_bh, blocks, slots):
    """The launch rule: more blocks than slots, at least one pair per slot,
    and at most 5% lost to the last round of pairs."""
    pairs = n_bh * ((blocks + 1) // 2)
    rounds = -(-pairs // slots)
    return n_bh * blocks > slots and pairs >= slots and (rounds * slots - pairs) * 20 <= pairs


FWD_CASES = [
    # (B, H, N, D, causal): query blocks of 256 rows
    (4, 32, 1024, 128, 1),   # 4 blocks per head: pairs (3, 0) and (2, 1)
    (4, 32, 768, 64, 2),     # 3 blocks: pair (2, 0) and block 1 alone; bottom-right alignment
    (4, 32, 1000, 128, 1),   # 4 blocks, the last one ragged (232 rows)
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_persistent_forward_matches_per_head(fa, case):
    B, H, N, D, causal = case
    print(f"[case] persistent fwd {case}", flush=True)
    assert pairs_fill(B * H, -(-N // 256), 256)
    q, k, v = synth.make_qkv(B, H, N, N, D, torch.bfloat16, seed=41, qk_mul=3.0 if D == 128 else 1.0)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = fa.fa_forward(qd, kd, vd, causal=causal)
    for b in range(B):
        for h in range(H):
            o1, l1 = fa.fa_forward(qd[b:b + 1, h:h + 1].contiguous(), kd[b:b + 1, h:h + 1].contiguous(),
                                   vd[b:b + 1, h:h + 1].contiguous(), causal=causal)
            assert torch.equal(o[b, h], o1[0, 0]) and torch.equal(lse[b, h], l1[0, 0]), f"head ({b},{h})"
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    for b, h in ((0, 0), (B - 1, H - 1), (1, 7)):
        ro, rl = orc.attention(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]), f64(v[b:b + 1, h:h + 1]),
                               scale, causal)
        err = np.abs(f64(o[b, h]) - ro[0, 0])
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, f"O vs oracle ({b},{h}): {err.max():.3e}"
        assert np.abs(f64(lse[b, h]) - rl[0, 0]).max() <= 1e-3, f"LSE vs oracle ({b},{h})"


BWD_CASES = [
    # (B, H, N, D, causal): query and key blocks of 128 rows
    (4, 32, 1024, 128, 1),   # 8 blocks per head: four pairs
    (4, 64, 384, 128, 1),    # 3 blocks: pair (2, 0) and block 1 alone
    (4, 48, 1024, 64, 1),    # D = 64: three workgroups per CU, 768 slots
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_persistent_backward_matches_per_head(fa, case):
    B, H, N, D, causal = case
    print(f"[case] persistent bwd {case}", flush=True)
    assert pairs_fill(B * H, -(-N // 128), 512 if D == 128 else 768)
    q, k, v = synth.make_qkv(B, H, N, N, D, torch.bfloat16, seed=42)
    do = synth.make_do(B, H, N, D, torch.bfloat16, seed=42)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_forward(qd, kd, vd, causal=causal)
    dq, dk, dv = fa.fa_backward(qd, kd, vd, o, dod, lse, causal=causal)
    for b in range(B):
        for h in range(H):
            sl = lambda t: t[b:b + 1, h:h + 1].contiguous()
            g1 = fa.fa_backward(sl(qd), sl(kd), sl(vd), sl(o), sl(dod), sl(lse), causal=causal)
            for name, full, one in zip(("dq", "dk", "dv"), (dq, dk, dv), g1):
                assert torch.equal(full[b, h], one[0, 0]), f"{name} head ({b},{h})"
    torch.cuda.synchronize()
    got = (f64(o), f64(lse), f64(dq), f64(dk), f64(dv))
    check_case(f"persistent bwd {case}", q, k, v, do, causal, got, heads=[(0, 0), (B - 1, H - 1), (2, 5)])


@pytest.mark.parametrize("kind", ["f16", "rope"])
def test_persistent_forward_f16_and_rope(fa, kind):
    """The fp16 forward and the fused-RoPE forward run the same persistent
    kernel template: batched against head by head, bit for bit."""
    B, H, N, D = 4, 32, 1024, 128
    print(f"[case] persistent fwd {kind}", flush=True)
    dtype = torch.float16 if kind == "f16" else torch.bfloat16
    q, k, v = synth.make_qkv(B, H, N, N, D, dtype, seed=43)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    if kind == "f16":
        run = lambda a, b, c: fa.fa_forward_f16(a, b, c, causal=True)  # noqa: E731
    else:
        cos, sin = (t.to(DEV) for t in synth.rope_tables(N, D))
        run = lambda a, b, c: fa.fa_forward_rope(a, b, c, cos, sin, causal=True)  # noqa: E731
    o, lse = run(qd, kd, vd)
    for b in range(B):
        for h in range(H):
            sl = lambda t: t[b:b + 1, h:h + 1].contiguous()  # noqa: E731
            o1, l1 = run(sl(qd), sl(kd), sl(vd))
            assert torch.equal(o[b, h], o1[0, 0]) and torch.equal(lse[b, h], l1[0, 0]), f"head ({b},{h})"
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
