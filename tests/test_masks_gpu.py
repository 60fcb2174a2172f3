"""GPU parity of key padding (kv_lens), bottom-right causal alignment and
fully masked rows, for the bf16 and fp32 forward passes, the split-KV decode
and the backward pass, against the fp64 oracle.

Rows that may attend no key must come back as exactly O = 0 and LSE = -inf
(never NaN); every other row is held to the same tolerances as the unmasked
tests (bf16 O max-abs 2e-2, mean-abs 2e-3, LSE 1e-3; fp32 O and LSE 1e-5;
gradients within the bounds of tests/grad_bounds.py).
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
BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 1e-3
F32_MAX, F32_LSE = 1e-5, 1e-5


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


def lens_tensor(kv_lens):
    return None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)


def check_forward(tag, o, lse, ro, rl, max_tol, mean_tol, lse_tol):
    empty = np.isneginf(rl)
    assert np.isfinite(o).all(), f"{tag}: non-finite O"
    assert not np.isnan(lse).any(), f"{tag}: NaN LSE"
    assert np.array_equal(np.isneginf(lse), empty), f"{tag}: rows with LSE = -inf differ"
    assert not o[empty].any(), f"{tag}: a fully masked row is not zero"
    full = ~empty
    err_o = np.abs(o[full] - ro[full])
    err_l = np.abs(lse[full] - rl[full])
    print(f"[mask] {tag}: {int(empty.sum())} empty rows; O max {err_o.max() if err_o.size else 0:.3e} "
          f"mean {err_o.mean() if err_o.size else 0:.3e}  LSE max {err_l.max() if err_l.size else 0:.3e}",
          flush=True)
    if err_o.size:
        assert err_o.max() <= max_tol and err_o.mean() <= mean_tol and err_l.max() <= lse_tol, tag


FWD_CASES = [
    # (B, H, Nq, Nk, D, causal, kv_lens, qk_mul)
    (1, 2, 77, 300, 128, 2, None, 1.0),            # bottom-right, Nq < Nk
    (1, 2, 300, 77, 128, 2, None, 1.0),            # bottom-right, Nq > Nk: 223 empty rows
    (1, 2, 300, 77, 64, 2, None, 1.0),
    (2, 2, 256, 256, 64, 2, None, 1.0),            # bottom-right = top-left when Nq == Nk
    (3, 2, 130, 300, 128, 0, [300, 1, 0], 1.0),    # padding; a batch entry with no key
    (2, 2, 256, 256, 64, 1, [256, 70], 1.0),       # padding + top-left
    (2, 1, 64, 1000, 128, 2, [1000, 33], 1.0),     # padding + bottom-right
    (2, 2, 700, 129, 64, 2, [129, 64], 1.0),       # bottom-right with many empty rows
    (1, 4, 513, 1025, 128, 2, [777], 3.0),         # rescale stress under masks
    (2, 2, 300, 300, 128, 1, [0, 299], 1.0),       # top-left with an empty batch entry
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[6]}")
def test_masked_bf16_forward(fa, case):
    B, H, Nq, Nk, D, causal, kv_lens, mul = case
    print(f"[case] masked bf16 {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.bfloat16, seed=41, qk_mul=mul)
    o, lse = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, kv_lens=lens_tensor(kv_lens))
    torch.cuda.synchronize()
    ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), causal, kv_lens=kv_lens)
    check_forward(f"bf16 {case}", f64(o), f64(lse), ro, rl, BF16_MAX, BF16_MEAN, BF16_LSE)


F32_CASES = [
    (1, 1, 256, 256, 64, 2, [200], 1.0),
    (2, 1, 100, 40, 128, 2, None, 1.0),
    (3, 1, 64, 130, 64, 0, [130, 0, 7], 1.0),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[6]}")
def test_masked_fp32_forward(fa, case):
    B, H, Nq, Nk, D, causal, kv_lens, _ = case
    print(f"[case] masked fp32 {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.float32, seed=42)
    o, lse = fa.fa_forward_f32(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, kv_lens=lens_tensor(kv_lens))
    torch.cuda.synchronize()
    ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), causal, kv_lens=kv_lens)
    check_forward(f"fp32 {case}", f64(o), f64(lse), ro, rl, F32_MAX, F32_MAX, F32_LSE)


def test_bottom_right_square_equals_top_left_bitwise(fa):
    q, k, v = synth.make_qkv(2, 2, 333, 333, 128, torch.bfloat16, seed=43, device=DEV)
    a = fa.fa_forward(q, k, v, causal=1)
    b = fa.fa_forward(q, k, v, causal="bottom_right")
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_padding_ignores_padded_values(fa):
    """Whatever the padded keys hold (here huge values) cannot reach O."""
    q, k, v = synth.make_qkv(2, 2, 100, 200, 64, torch.bfloat16, seed=44, device=DEV)
    lens = lens_tensor([150, 61])
    a = fa.fa_forward(q, k, v, causal=0, kv_lens=lens)
    k2, v2 = k.clone(), v.clone()
    k2[0, :, 150:] = 1e4
    v2[0, :, 150:] = -1e4
    k2[1, :, 61:] = 3e3
    v2[1, :, 61:] = float("inf")
    b = fa.fa_forward(q, k2, v2, causal=0, kv_lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _garbage_padding(k, v, lens):
    """K/V copies whose padded keys hold NaN, +inf and huge values."""
    k2, v2 = k.clone(), v.clone()
    for b, L in enumerate(lens):
        k2[b, :, L:] = float("nan")
        v2[b, :, L::2] = float("inf")
        v2[b, :, L + 1::2] = float("nan")
    return k2, v2


def test_padding_ignores_nan_keys_forward_backward_decode(fa):
    """Padded keys holding NaN or inf leave every output bitwise unchanged:
    forward (both causal alignments), backward (dK, dV of padded keys are 0)
    and split-KV decode. Lengths end inside a tile, on a tile edge and at 0."""
    lens_list = [150, 64, 0]
    lens = lens_tensor(lens_list)
    q, k, v = synth.make_qkv(3, 2, 100, 200, 128, torch.bfloat16, seed=45, device=DEV)
    k2, v2 = _garbage_padding(k, v, lens_list)
    do = synth.make_do(3, 2, 100, 128, torch.bfloat16, seed=45).to(DEV)
    for causal in (0, 2):
        o_a, l_a = fa.fa_forward(q, k, v, causal=causal, kv_lens=lens)
        o_b, l_b = fa.fa_forward(q, k2, v2, causal=causal, kv_lens=lens)
        ga = fa.fa_backward(q, k, v, o_a, do, l_a, causal=causal, kv_lens=lens)
        gb = fa.fa_backward(q, k2, v2, o_b, do, l_b, causal=causal, kv_lens=lens)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b), f"forward causal={causal}"
        for name, x, y in zip(("dq", "dk", "dv"), ga, gb):
            assert torch.equal(x, y), f"backward {name} causal={causal}"
        for b, L in enumerate(lens_list):
            assert not gb[1][b, :, L:].any() and not gb[2][b, :, L:].any(), f"padded dK/dV b={b}"
    qd, kd, vd = synth.make_qkv(3, 2, 1, 333, 64, torch.bfloat16, seed=46, device=DEV)
    dlens = [333, 65, 0]
    kd2, vd2 = _garbage_padding(kd, vd, dlens)
    la = lens_tensor(dlens)
    oa, sa = fa.fa_decode_splitkv(qd, kd, vd, 8, kv_lens=la)
    ob, sb = fa.fa_decode_splitkv(qd, kd2, vd2, 8, kv_lens=la)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(sa, sb)


DEC_CASES = [
    # (B, H, Nk, D, splits, kv_lens)
    (4, 8, 5000, 128, 16, [5000, 1, 0, 2049]),
    (3, 4, 777, 64, 64, [700, 63, 64]),
    (2, 2, 40, 128, 64, [40, 5]),           # more splits than keys
]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: "x".join(map(str, c[:5])))
def test_masked_decode(fa, case):
    B, H, Nk, D, S, kv_lens = case
    print(f"[case] masked decode {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, 1, Nk, D, torch.bfloat16, seed=45)
    o, lse = fa.fa_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), S, kv_lens=lens_tensor(kv_lens))
    torch.cuda.synchronize()
    ro, rl = orc.decode(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), kv_lens=kv_lens)
    check_forward(f"decode {case}", f64(o)[:, :, 0], f64(lse), ro[:, :, 0], rl[:, :, 0], BF16_MAX, BF16_MEAN,
                  BF16_LSE)


BWD_CASES = [
    # (B, H, Nq, Nk, D, causal, kv_lens)
    (1, 2, 77, 300, 128, 2, None),
    (1, 2, 300, 77, 64, 2, None),
    (3, 2, 130, 300, 128, 0, [300, 1, 0]),
    (2, 2, 256, 256, 64, 1, [256, 70]),
    (2, 1, 200, 520, 128, 2, [520, 150]),
    (2, 2, 129, 200, 64, 2, [200, 100]),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[6]}")
def test_masked_backward(fa, case):
    B, H, Nq, Nk, D, causal, kv_lens = case
    print(f"[case] masked bwd {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.bfloat16, seed=46)
    do = synth.make_do(B, H, Nq, D, torch.bfloat16, seed=46)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    lens = lens_tensor(kv_lens)
    o, lse = fa.fa_forward(qd, kd, vd, causal=causal, kv_lens=lens)
    dq, dk, dv = fa.fa_backward(qd, kd, vd, o, dod, lse, causal=causal, kv_lens=lens)
    torch.cuda.synchronize()
    qn, kn, vn, don = f64(q), f64(k), f64(v), f64(do)
    on, ln, dqn, dkn, dvn = f64(o), f64(lse), f64(dq), f64(dk), f64(dv)
    scale = 1.0 / math.sqrt(D)
    ro, rl = orc.attention(qn, kn, vn, scale, causal, kv_lens=kv_lens)
    worst = 0.0
    for b in range(B):
        L = Nk if kv_lens is None else kv_lens[b]
        rq, rk, rv = orc.attention_backward(qn[b:b + 1], kn[b:b + 1], vn[b:b + 1], don[b:b + 1], scale, causal,
                                            kv_lens=[L])
        for h in range(H):
            empty = np.isneginf(rl[b, h])
            assert np.array_equal(np.isneginf(ln[b, h]), empty)
            lse_err = np.where(empty, 0.0, np.abs(np.where(empty, 0.0, ln[b, h]) - np.where(empty, 0.0, rl[b, h])))
            bq, bk, bv = bounds_head(qn[b, h], kn[b, h], vn[b, h], don[b, h], on[b, h], lse_err, scale, causal, L)
            for name, g, r, bd in (("dq", dqn[b, h], rq[0, h], bq), ("dk", dkn[b, h], rk[0, h], bk),
                                   ("dv", dvn[b, h], rv[0, h], bv)):
                assert np.isfinite(g).all(), f"{case} {name} not finite"
                ratio = np.abs(g - r) / bd
                worst = max(worst, float(ratio.max()))
                assert ratio.max() <= 1.0, f"{case} {name} ({b},{h}) err/bound {ratio.max():.3f}"
            assert not dqn[b, h][empty].any(), f"{case}: empty rows must get dQ = 0"
            assert not dkn[b, h][L:].any() and not dvn[b, h][L:].any(), f"{case}: padded keys must get 0"
    print(f"[mask] bwd {case}: worst err/bound {worst:.3f}", flush=True)
