"""GPU parity of the fp16 forward pass, the RoPE kernel and the forward pass
with the fused RoPE prologue, against the fp64 oracle.

fp16 tolerance: the workload definition states bf16 O tolerances (max-abs
2e-2, mean-abs 2e-3); they come from bf16 rounding of P and O (unit roundoff
2^-8). The same error model with fp16's unit roundoff 2^-11 scales them by
1/8: max-abs 2.5e-3, mean-abs 2.5e-4. LSE keeps the fp32-accumulation bound
1e-3 of the bf16 tests.

RoPE kernel bound, per element: the rotation is two fp32 products and one
fused multiply-add (error <= 2^-23 (|a c| + |b s|)) and a final rounding to
the element type (<= u |y|, u = 2^-8 bf16, 2^-11 fp16; below fp16's smallest
normal, 2^-14, the spacing is a fixed 2^-24, so the rounding error there is
up to 2^-25 absolute), times 1.01.

Forward with RoPE: rope(Q) and rope(K) are rounded to the element type before
the score product, so each score s_ij moves by at most
scale (2u + u^2) sum_d |q~_id| |k~_jd| (q~, k~ the exact rotated rows), and
LSE_i, a P-weighted mean of those moves, by at most
scale (2u + u^2) sum_j P_ij |q~_i| . |k~_j|; the LSE bound is that plus 1e-4
(the fp32 accumulation error of the unrotated path, ~1e-5). The O tolerances
above hold unchanged (the measured O errors stay far inside them).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
from grad_bounds import bounds_head
from oracle import attention as orc

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.bfloat16: (2e-2, 2e-3, 1e-3), torch.float16: (2.5e-3, 2.5e-4, 1e-3)}
UNIT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
SUBNORMAL_HALF_ULP = {torch.bfloat16: 2.0 ** -134, torch.float16: 2.0 ** -25}


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


def check(tag, o, lse, ro, rl, dtype, lse_bound=None):
    mx, mean, ltol = TOL[dtype]
    empty = np.isneginf(rl)
    assert np.isfinite(o).all(), tag
    assert np.array_equal(np.isneginf(lse), empty), tag
    assert not o[empty].any(), tag
    err_o = np.abs(o[~empty] - ro[~empty])
    err_l = np.abs(lse[~empty] - rl[~empty])
    print(f"[f16/rope] {tag}: O max {err_o.max():.3e} mean {err_o.mean():.3e}  LSE max {err_l.max():.3e}",
          flush=True)
    assert err_o.max() <= mx and err_o.mean() <= mean, tag
    if lse_bound is None:
        assert err_l.max() <= ltol, tag
    else:
        ratio = err_l / lse_bound[~empty]
        print(f"[f16/rope] {tag}: LSE err/bound {ratio.max():.3f}", flush=True)
        assert ratio.max() <= 1.0, tag


F16_CASES = [
    # (B, H, Nq, Nk, D, causal, kv_lens, qk_mul)
    (1, 2, 256, 256, 128, 0, None, 1.0),
    (1, 2, 256, 256, 128, 1, None, 1.0),
    (2, 3, 300, 300, 64, 1, None, 1.0),
    (1, 2, 77, 300, 128, 2, None, 1.0),
    (1, 4, 513, 513, 128, 1, None, 3.0),
    (2, 2, 129, 1025, 64, 0, [1025, 200], 3.0),
    (2, 2, 300, 77, 128, 2, [77, 30], 1.0),
]


@pytest.mark.parametrize("case", F16_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[6]}-{c[7]}")
def test_fp16_forward(fa, case):
    B, H, Nq, Nk, D, causal, kv_lens, mul = case
    print(f"[case] fp16 {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.float16, seed=51, qk_mul=mul)
    lens = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    o, lse = fa.fa_forward_f16(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, kv_lens=lens)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), causal, kv_lens=kv_lens)
    check(f"fp16 {case}", f64(o), f64(lse), ro, rl, torch.float16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("style", [0, 1], ids=["half", "pairs"])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_kernel(fa, dtype, style, D):
    print(f"[case] rope kernel {dtype} style={style} D={D}", flush=True)
    B, H, N = 2, 3, 301
    x = synth.normal((B, H, N, D), dtype, 52, 0) * 1
    cos, sin = synth.rope_tables(N + 7, D)
    y = fa.fa_rope(x.to(DEV), cos.to(DEV), sin.to(DEV), style=style)
    torch.cuda.synchronize()
    xn, cn, sn = f64(x), cos.double().numpy(), sin.double().numpy()
    rot = orc.rope if style == 0 else orc.rope_pairs
    ref = np.stack([np.stack([rot(xn[b, h], cn[:N], sn[:N]) for h in range(H)]) for b in range(B)])
    # |a c| + |b s| of every output element (the pair partner is the other half / the other pair element)
    if style == 0:
        a, bb = xn[..., : D // 2], xn[..., D // 2:]
        mag = np.concatenate([np.abs(a * cn[:N]) + np.abs(bb * sn[:N]), np.abs(bb * cn[:N]) + np.abs(a * sn[:N])],
                             axis=-1)
    else:
        x0, x1 = xn[..., 0::2], xn[..., 1::2]
        mag = np.empty_like(xn)
        mag[..., 0::2] = np.abs(x0 * cn[:N]) + np.abs(x1 * sn[:N])
        mag[..., 1::2] = np.abs(x1 * cn[:N]) + np.abs(x0 * sn[:N])
    bound = 1.01 * (UNIT[dtype] * np.abs(ref) + 2.0 ** -23 * mag + SUBNORMAL_HALF_ULP[dtype])
    err = np.abs(f64(y) - ref)
    print(f"[f16/rope] rope kernel {dtype} style={style} D={D}: err/bound {np.max(err / bound):.3f}", flush=True)
    assert (err <= bound).all()
    # in place gives the same bits
    xi = x.to(DEV).clone()
    fa.fa_rope(xi, cos.to(DEV), sin.to(DEV), style=style, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi.cpu(), y.cpu())


ROPE_CASES = [
    # (B, H, Nq, Nk, D, causal, kv_lens, style, dtype)
    (1, 2, 256, 256, 128, 1, None, 0, torch.bfloat16),
    (1, 2, 256, 256, 64, 0, None, 1, torch.bfloat16),
    (1, 2, 300, 300, 128, 1, None, 1, torch.float16),
    (2, 2, 77, 300, 128, 2, [300, 120], 0, torch.bfloat16),
    (2, 2, 300, 77, 64, 2, None, 0, torch.float16),
    (1, 4, 1000, 1000, 128, 1, None, 0, torch.float16),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[6]}-{c[7]}-{c[8]}")
def test_forward_rope(fa, case):
    B, H, Nq, Nk, D, causal, kv_lens, style, dtype = case
    print(f"[case] forward rope {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, dtype, seed=53)
    cos, sin = synth.rope_tables(max(Nq, Nk) + 3, D)
    lens = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    o, lse = fa.fa_forward_rope(q.to(DEV), k.to(DEV), v.to(DEV), cos.to(DEV), sin.to(DEV), style=style,
                                causal=causal, kv_lens=lens)
    torch.cuda.synchronize()
    cn, sn = cos.double().numpy(), sin.double().numpy()
    scale = 1.0 / math.sqrt(D)
    ro, rl = orc.attention_rope(f64(q), f64(k), f64(v), cn, sn, scale, causal, kv_lens=kv_lens, style=style)
    qr, kr = orc.rope_qk(f64(q), f64(k), cn, sn, causal, kv_lens, style)
    u = UNIT[dtype]
    lse_bound = np.empty(rl.shape)
    for b in range(B):
        L = None if kv_lens is None else kv_lens[b]
        for h in range(H):
            p = orc.softmax_weights(qr[b, h], kr[b, h], scale, causal, L)
            lse_bound[b, h] = scale * (2 * u + u * u) * (p * (np.abs(qr[b, h]) @ np.abs(kr[b, h]).T)).sum(axis=1)
    check(f"rope {case}", f64(o), f64(lse), ro, rl, dtype, lse_bound=lse_bound + 1e-4)
    # the rotation matters: attention of the unrotated inputs differs
    o0, _ = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), causal, kv_lens=kv_lens)
    assert np.abs(o0 - ro).max() > 0.05


def test_forward_rope_equals_rope_then_forward(fa):
    """The fused prologue gives the same bits as fa_rope on Q and K followed
    by the plain forward (both round the rotated values the same way)."""
    q, k, v = synth.make_qkv(1, 4, 333, 333, 128, torch.bfloat16, seed=54, device=DEV)
    cos, sin = synth.rope_tables(333, 128, device=DEV)
    a = fa.fa_forward_rope(q, k, v, cos, sin, style="half", causal=1)
    b = fa.fa_forward(fa.fa_rope(q, cos, sin), fa.fa_rope(k, cos, sin), v, causal=1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


DEC16_CASES = [
    # (B, H, Nk, D, splits, kv_lens)
    (4, 8, 5000, 128, 16, None),
    (3, 4, 777, 64, 64, [700, 0, 64]),
]


@pytest.mark.parametrize("case", DEC16_CASES, ids=lambda c: "x".join(map(str, c[:5])) + f"-{c[5]}")
def test_fp16_decode(fa, case):
    B, H, Nk, D, S, kv_lens = case
    print(f"[case] fp16 decode {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, 1, Nk, D, torch.float16, seed=55)
    lens = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    o, lse = fa.fa_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), S, kv_lens=lens)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    ro, rl = orc.decode(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), kv_lens=kv_lens)
    check(f"fp16 decode {case}", f64(o)[:, :, 0], f64(lse), ro[:, :, 0], rl[:, :, 0], torch.float16)


BWD16_CASES = [
    # (B, H, Nq, Nk, D, causal, kv_lens, qk_mul)
    (1, 2, 256, 256, 128, 0, None, 1.0),
    (1, 2, 300, 300, 64, 1, None, 1.0),
    (2, 2, 129, 400, 128, 2, [400, 100], 1.0),
    (1, 2, 513, 513, 128, 1, None, 3.0),
    (2, 2, 150, 333, 128, 0, [333, 90], 1.0),   # non-causal D = 128: ragged rows, padded keys
]


@pytest.mark.parametrize("case", BWD16_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[6]}-{c[7]}")
def test_fp16_backward(fa, case):
    """fp16 gradients within the bounds of tests/grad_bounds.py with fp16's
    unit roundoff 2^-11 and subnormal half-spacing 2^-25."""
    B, H, Nq, Nk, D, causal, kv_lens, mul = case
    print(f"[case] fp16 bwd {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.float16, seed=56, qk_mul=mul)
    do = synth.make_do(B, H, Nq, D, torch.float16, seed=56)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    lens = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    o, lse = fa.fa_forward_f16(qd, kd, vd, causal=causal, kv_lens=lens)
    dq, dk, dv = fa.fa_backward(qd, kd, vd, o, dod, lse, causal=causal, kv_lens=lens)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float16
    qn, kn, vn, don = f64(q), f64(k), f64(v), f64(do)
    on, ln, got = f64(o), f64(lse), (f64(dq), f64(dk), f64(dv))
    scale = 1.0 / math.sqrt(D)
    rl = orc.attention(qn, kn, vn, scale, causal, kv_lens=kv_lens)[1]
    worst = 0.0
    for b in range(B):
        L = Nk if kv_lens is None else kv_lens[b]
        ref = orc.attention_backward(qn[b:b + 1], kn[b:b + 1], vn[b:b + 1], don[b:b + 1], scale, causal,
                                     kv_lens=[L])
        for h in range(H):
            empty = np.isneginf(rl[b, h])
            lse_err = np.where(empty, 0.0, np.abs(np.where(empty, 0.0, ln[b, h]) - np.where(empty, 0.0, rl[b, h])))
            bounds = bounds_head(qn[b, h], kn[b, h], vn[b, h], don[b, h], on[b, h], lse_err, scale, causal, L,
                                 u=2.0 ** -11, tiny=2.0 ** -25)
            for name, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bounds):
                ratio = np.abs(g[b, h] - r[0, h]) / bd
                worst = max(worst, float(ratio.max()))
                assert np.isfinite(g[b, h]).all() and ratio.max() <= 1.0, f"{case} {name} ({b},{h}) {ratio.max():.3f}"
    print(f"[f16/rope] fp16 bwd {case}: worst err/bound {worst:.3f}", flush=True)
