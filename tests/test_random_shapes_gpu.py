"""Seeded random sweep of shapes and options through every entry point,
against the fp64 oracle.

Each case draws B, H, Nq, Nk, D, the causal mode, key padding and the input
scale from a fixed seed, so the sweep is the same on every run; sizes stay
small enough for the oracle to finish in well under a second per case but
cross the tile boundaries of every kernel (32, 64, 128 and 256 rows) at
random offsets. Tolerances are those of the dedicated tests: bf16 O max-abs
2e-2 / mean-abs 2e-3 and LSE 1e-3; fp16 one eighth of the bf16 O bounds;
gradients within tests/grad_bounds.py; fp32 1e-5, the stated bound for
unit-variance inputs, times mul^2 when Q and K are scaled by mul: the fp32
error of a score is proportional to sum |q| |k|, which grows by mul^2, and
O and LSE inherit it.
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
TOL = {torch.bfloat16: (2e-2, 2e-3, 1e-3), torch.float16: (2.5e-3, 2.5e-4, 1e-3), torch.float32: (1e-5, 1e-5, 1e-5)}


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


def draw(seed):
    r = np.random.default_rng(seed)
    B = int(r.integers(1, 4))
    H = int(r.integers(1, 4))
    Nq = int(r.choice([1, 2, 31, 33, 64, 65, 127, 129, 200, 255, 257, 300, 511]))
    Nk = int(r.choice([1, 3, 32, 63, 64, 96, 128, 130, 250, 256, 333, 512, 600]))
    D = int(r.choice([64, 128]))
    causal = int(r.integers(0, 3))
    kv_lens = None
    if r.random() < 0.5:
        kv_lens = [int(x) for x in r.integers(0, Nk + 1, size=B)]
    mul = float(r.choice([1.0, 3.0]))
    return B, H, Nq, Nk, D, causal, kv_lens, mul


def check(tag, o, lse, ro, rl, dtype, mul=1.0):
    mx, mean, ltol = TOL[dtype]
    if dtype == torch.float32:
        mx, mean, ltol = mx * mul * mul, mean * mul * mul, ltol * mul * mul
    empty = np.isneginf(rl)
    assert np.isfinite(o).all(), tag
    assert np.array_equal(np.isneginf(lse), empty), tag
    assert not o[empty].any(), tag
    if (~empty).any():
        err_o = np.abs(o[~empty] - ro[~empty])
        err_l = np.abs(lse[~empty] - rl[~empty])
        assert err_o.max() <= mx and err_o.mean() <= mean and err_l.max() <= ltol, \
            f"{tag}: O max {err_o.max():.3e} mean {err_o.mean():.3e} LSE {err_l.max():.3e}"


SEEDS = list(range(1000, 1048))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_forward_and_backward(fa, seed):
    B, H, Nq, Nk, D, causal, kv_lens, mul = draw(seed)
    case = (B, H, Nq, Nk, D, causal, kv_lens, mul)
    print(f"[case] random seed {seed}: {case}", flush=True)
    scale = 1.0 / math.sqrt(D)
    lens = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    for dtype, fwd in ((torch.bfloat16, fa.fa_forward), (torch.float16, fa.fa_forward_f16),
                       (torch.float32, fa.fa_forward_f32)):
        q, k, v = synth.make_qkv(B, H, Nq, Nk, D, dtype, seed=seed, qk_mul=mul)
        o, lse = fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, kv_lens=lens)
        torch.cuda.synchronize()
        ro, rl = orc.attention(f64(q), f64(k), f64(v), scale, causal, kv_lens=kv_lens)
        check(f"seed {seed} {dtype} forward {case}", f64(o), f64(lse), ro, rl, dtype, mul)
        if dtype == torch.float32:
            continue
        # Backward through the same entry point family, from this forward's O and LSE.
        do = synth.make_do(B, H, Nq, D, dtype, seed=seed)
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
        dq, dk, dv = fa.fa_backward(qd, kd, vd, o, dod, lse, causal=causal, kv_lens=lens)
        torch.cuda.synchronize()
        u, tiny = (2.0 ** -8, 2.0 ** -134) if dtype == torch.bfloat16 else (2.0 ** -11, 2.0 ** -25)
        qn, kn, vn, don, on, ln = f64(q), f64(k), f64(v), f64(do), f64(o), f64(lse)
        got = (f64(dq), f64(dk), f64(dv))
        for b in range(B):
            L = Nk if kv_lens is None else kv_lens[b]
            ref = orc.attention_backward(qn[b:b + 1], kn[b:b + 1], vn[b:b + 1], don[b:b + 1], scale, causal,
                                         kv_lens=[L])
            for h in range(H):
                emp = np.isneginf(rl[b, h])
                lerr = np.where(emp, 0.0, np.abs(np.where(emp, 0.0, ln[b, h]) - np.where(emp, 0.0, rl[b, h])))
                bounds = bounds_head(qn[b, h], kn[b, h], vn[b, h], don[b, h], on[b, h], lerr, scale, causal, L,
                                     u=u, tiny=tiny)
                for name, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bounds):
                    ratio = np.abs(g[b, h] - r[0, h]) / bd
                    assert np.isfinite(g[b, h]).all() and ratio.max() <= 1.0, \
                        f"seed {seed} {dtype} {name} ({b},{h}) err/bound {ratio.max():.3f} {case}"


@pytest.mark.parametrize("seed", list(range(2000, 2016)))
def test_random_decode(fa, seed):
    r = np.random.default_rng(seed)
    B, H = int(r.integers(1, 5)), int(r.integers(1, 5))
    Nk = int(r.choice([1, 5, 64, 333, 1000, 4097]))
    D = int(r.choice([64, 128]))
    S = int(r.choice([1, 3, 16, 64, 100]))
    kv_lens = [int(x) for x in r.integers(0, Nk + 1, size=B)] if r.random() < 0.5 else None
    print(f"[case] random decode seed {seed}: B={B} H={H} Nk={Nk} D={D} S={S} lens={kv_lens}", flush=True)
    lens = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    for dtype in (torch.bfloat16, torch.float16):
        q, k, v = synth.make_qkv(B, H, 1, Nk, D, dtype, seed=seed)
        o, lse = fa.fa_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), S, kv_lens=lens)
        torch.cuda.synchronize()
        ro, rl = orc.decode(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), kv_lens=kv_lens)
        check(f"seed {seed} {dtype} decode", f64(o)[:, :, 0], f64(lse), ro[:, :, 0], rl[:, :, 0], dtype)
