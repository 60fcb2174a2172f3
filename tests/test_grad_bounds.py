"""The gradient bounds of tests/grad_bounds.py are not vacuous: gradients
that carry only the rounding of their bf16 outputs pass them, and each
plausible kernel mistake below (a mask off by one, a dropped ragged tile, a
missing scale, D or the LSE taken from the wrong row, swapped keys, a flipped
sign, the other causal alignment) fails them on small seeded inputs."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
from grad_bounds import bounds_head
from oracle import attention as orc


def bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def inputs(nq, nk, D, seed, mul=1.0):
    q, k, v = synth.make_qkv(1, 1, nq, nk, D, torch.bfloat16, seed=seed, qk_mul=mul)
    do = synth.make_do(1, 1, nq, D, torch.bfloat16, seed=seed)
    return [t[0, 0].double().numpy() for t in (q, k, v, do)]


def grads_from_p(p, q, k, v, do, scale, d=None):
    """Chain rule on a given probability matrix (the mutants' P); D defaults
    to rowsum(P * dP)."""
    dp = do @ v.T
    if d is None:
        d = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - d)
    return scale * (ds @ k), scale * (ds.T @ q), p.T @ do


def violates(bounds, got, ref):
    return any((np.abs(g - r) > b).any() for g, r, b in zip(got, ref, bounds))


CASES = [
    # (Nq, Nk, D, causal, qk_mul)
    (40, 40, 64, False, 1.0),
    (77, 77, 128, True, 1.0),
    (65, 65, 64, True, 3.0),
    (77, 100, 64, True, 1.0),
]


def setup(case, seed=31):
    nq, nk, D, causal, mul = case
    q, k, v, do = inputs(nq, nk, D, seed, mul)
    scale = 1.0 / math.sqrt(D)
    o = orc.attention(q[None, None], k[None, None], v[None, None], scale, causal)[0][0, 0]
    bounds = bounds_head(q, k, v, do, bf16_round(o), np.zeros(nq), scale, causal)
    ref = orc.attention_backward_head(q, k, v, do, scale, causal)
    return q, k, v, do, scale, bounds, ref


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_rounded_exact_gradients_pass(case):
    *_, bounds, ref = setup(case)
    got = [bf16_round(r) for r in ref]
    assert not violates(bounds, got, ref)


def masked_softmax(s, mask):
    s = np.where(mask, s, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def mutants(case, q, k, v, do, scale, ref):
    nq, nk, D, causal, _ = case
    s = scale * (q @ k.T)
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    mask = (j <= i) if causal else np.ones((nq, nk), bool)
    p = masked_softmax(s, mask)
    dq, dk, dv = ref
    out = {}
    if causal:
        strict = (j < i) | ((i == 0) & (j == 0))
        out["diagonal key masked"] = grads_from_p(masked_softmax(s, strict), q, k, v, do, scale)
        wide = j <= i + 1
        out["one key too many"] = grads_from_p(masked_softmax(s, wide), q, k, v, do, scale)
        if nk != nq:
            br = j <= i + (nk - nq)
            out["bottom-right alignment"] = grads_from_p(masked_softmax(s, br), q, k, v, do, scale)
    dp = do @ v.T
    d = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - d)
    if nk > 32:
        last = (nk - 1) // 32 * 32
        if not causal:   # causal: few (or no) rows see the last tile's keys
            out["ragged last key tile dropped from dQ"] = (dq - scale * ds[:, last:] @ k[last:], dk, dv)
        out["second key tile dropped from dQ"] = (dq - scale * ds[:, 32:64] @ k[32:64], dk, dv)
        flip = ds.copy()
        flip[:, 32:64] *= -1
        out["dS sign flipped on a tile (dK)"] = (dq, scale * flip.T @ q, dv)
    out["dK without scale"] = (dq, dk / scale, dv)
    out["dQ without scale"] = (dq / scale, dk, dv)
    out["D from the next row"] = grads_from_p(p, q, k, v, do, scale, d=np.roll(d, -1, axis=0))
    lse = np.log(np.where(mask, np.exp(s - s.max(axis=1, keepdims=True)), 0).sum(axis=1, keepdims=True)) \
        + s.max(axis=1, keepdims=True)
    p_shift = np.where(mask, np.exp(s - np.roll(lse, -1, axis=0)), 0.0)
    out["LSE from the next row"] = grads_from_p(p_shift, q, k, v, do, scale)
    perm = np.arange(nk)
    perm[[0, 1]] = perm[[1, 0]]
    out["two keys swapped in dV"] = (dq, dk, dv[perm])
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_planted_mistakes_fail(case):
    q, k, v, do, scale, bounds, ref = setup(case)
    for name, got in mutants(case, q, k, v, do, scale, ref).items():
        assert violates(bounds, [bf16_round(x) for x in got], ref), f"{case}: '{name}' passes the bounds"
