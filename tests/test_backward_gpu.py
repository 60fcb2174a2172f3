"""GPU parity of the backward pass (recompute from the saved log-sum-exp)
against the fp64 oracle's chain-rule gradients, element by element within the
worst-case bounds that tests/grad_bounds.py derives from the kernels'
arithmetic (bf16 roundings of P, dS and the outputs, fp32 sums, the forward's
LSE and O errors carried into the backward).
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
LSE_TOL = 1e-3          # the forward's own LSE bound (bf16 inputs)


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


def run_gpu(fa, q, k, v, do, causal):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fa_forward(qd, kd, vd, causal=causal)
    dq, dk, dv = fa.fa_backward(qd, kd, vd, o, dod, lse, causal=causal)
    torch.cuda.synchronize()
    return f64(o), f64(lse), f64(dq), f64(dk), f64(dv)


def check_case(tag, q, k, v, do, causal, got, heads=None):
    """Compare the GPU gradients with the oracle on every (b, h) in `heads`
    (all when None), element by element against the derived bounds."""
    o_gpu, lse_gpu, dq, dk, dv = got
    qn, kn, vn, don = f64(q), f64(k), f64(v), f64(do)
    B, H, _, D = qn.shape
    scale = 1.0 / math.sqrt(D)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    maxerr = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, h in heads:
        rl = orc.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], scale, causal)[1]
        lse_err = np.abs(lse_gpu[b, h] - rl[0, 0])
        assert lse_err.max() <= LSE_TOL, f"{tag}: forward LSE error {lse_err.max():.3e}"
        rq, rk, rv = orc.attention_backward_head(qn[b, h], kn[b, h], vn[b, h], don[b, h], scale, causal)
        bq, bk, bv = bounds_head(qn[b, h], kn[b, h], vn[b, h], don[b, h], o_gpu[b, h], lse_err, scale, causal)
        for name, g, r, bd in (("dq", dq[b, h], rq, bq), ("dk", dk[b, h], rk, bk), ("dv", dv[b, h], rv, bv)):
            assert np.isfinite(g).all(), f"{tag} {name} ({b},{h}) not finite"
            err = np.abs(g - r)
            ratio = err / bd
            worst[name] = max(worst[name], float(ratio.max()))
            maxerr[name] = max(maxerr[name], float(err.max()))
            if ratio.max() > 1.0:
                i = np.unravel_index(np.argmax(ratio), ratio.shape)
                raise AssertionError(f"{tag} {name} ({b},{h}) row {i[0]} col {i[1]}: got {g[i]:.6g} "
                                     f"want {r[i]:.6g} err {err[i]:.3e} > bound {bd[i]:.3e}")
    print(f"[bwd] {tag}: max err dq {maxerr['dq']:.2e} dk {maxerr['dk']:.2e} dv {maxerr['dv']:.2e}; "
          f"err/bound dq {worst['dq']:.3f} dk {worst['dk']:.3f} dv {worst['dv']:.3f}", flush=True)


CASES = [
    # (B, H, Nq, Nk, D, causal, qk_mul)
    (1, 2, 256, 256, 128, False, 1.0),
    (1, 2, 256, 256, 128, True, 1.0),
    (1, 2, 256, 256, 64, False, 1.0),
    (1, 2, 256, 256, 64, True, 1.0),
    (2, 3, 300, 300, 64, True, 1.0),       # ragged: 300 = 2*128 + 44 = 9*32 + 12
    (1, 2, 300, 300, 128, False, 1.0),
    (1, 1, 1, 1, 128, False, 1.0),
    (1, 1, 1, 1, 64, True, 1.0),
    (1, 1, 17, 17, 128, True, 1.0),
    (1, 1, 40, 40, 64, False, 1.0),        # few keys: one dropped term exceeds the bound
    (1, 1, 77, 300, 128, False, 1.0),      # Nq < Nk
    (1, 1, 77, 300, 128, True, 1.0),       # top-left causal: keys past row 76 get no gradient
    (1, 1, 300, 77, 64, True, 1.0),        # Nq > Nk
    (1, 4, 513, 513, 128, True, 3.0),      # scores std ~ 9 (the rescale-stress inputs)
    (1, 2, 1000, 1000, 64, True, 1.0),
    (2, 2, 129, 1025, 128, False, 3.0),
    # Non-causal D = 128 with few 32-row tiles: an odd tile count with a
    # ragged second key block, two tiles the second of one row, two whole
    # tiles.
    (1, 2, 96, 160, 128, False, 1.0),
    (1, 1, 33, 64, 128, False, 1.0),
    (1, 1, 64, 64, 128, False, 3.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_backward_matches_oracle(fa, case):
    B, H, Nq, Nk, D, causal, mul = case
    print(f"[case] bwd {case}", flush=True)
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.bfloat16, seed=21, qk_mul=mul)
    do = synth.make_do(B, H, Nq, D, torch.bfloat16, seed=21)
    got = run_gpu(fa, q, k, v, do, causal)
    check_case(f"bwd {case}", q, k, v, do, causal, got)


@pytest.mark.parametrize("name,heads", [
    ("prefill_b1_h32_n2048_d128", [(0, 0), (0, 13), (0, 31)]),
    ("causal_b4_h32_n4096_d128_qkx3", [(0, 0), (3, 31)]),
    ("causal_b1_h16_n16000_d64", [(0, 15)]),
])
def test_backward_workload_sizes(fa, name, heads):
    """The measured prefill shapes, every element of a few sampled heads (one
    head at 16000, whose oracle and bounds take about a minute on the host)."""
    w = synth.WORKLOADS[name]
    print(f"[case] bwd workload {name} heads {heads}", flush=True)
    q, k, v = synth.make_workload(w, seed=22)
    do = synth.make_do(w.B, w.H, w.Nq, w.D, w.dtype, seed=22)
    got = run_gpu(fa, q, k, v, do, w.causal)
    check_case(f"bwd {name}", q, k, v, do, w.causal, got, heads=heads)


def test_backward_zero_output_gradient(fa):
    """dO = 0 gives exactly zero gradients."""
    q, k, v = synth.make_qkv(1, 2, 200, 200, 128, torch.bfloat16, seed=23)
    do = torch.zeros_like(q)
    _, _, dq, dk, dv = run_gpu(fa, q, k, v, do, True)
    assert not dq.any() and not dk.any() and not dv.any()


def test_backward_unseen_keys_are_zero(fa):
    """Top-left causal with Nk > Nq: no query sees keys Nq.., so their dK and
    dV rows are exactly zero (the rest is checked against the oracle)."""
    Nq, Nk = 100, 333
    q, k, v = synth.make_qkv(1, 2, Nq, Nk, 64, torch.bfloat16, seed=24)
    do = synth.make_do(1, 2, Nq, 64, torch.bfloat16, seed=24)
    got = run_gpu(fa, q, k, v, do, True)
    assert not got[3][:, :, Nq:].any() and not got[4][:, :, Nq:].any()
    check_case("bwd unseen keys", q, k, v, do, True, got)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_run_to_run_bitwise(fa, causal):
    """No atomics: two calls give identical bits."""
    q, k, v = synth.make_qkv(1, 4, 700, 700, 128, torch.bfloat16, seed=25, device=DEV)
    do = synth.make_do(1, 4, 700, 128, torch.bfloat16, seed=25, device=DEV)
    o, lse = fa.fa_forward(q, k, v, causal=causal)
    a = fa.fa_backward(q, k, v, o, do, lse, causal=causal)
    b = fa.fa_backward(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_rejects_bad_arguments(fa):
    q, k, v = synth.make_qkv(1, 1, 64, 64, 128, torch.bfloat16, seed=26, device=DEV)
    o, lse = fa.fa_forward(q, k, v)
    with pytest.raises(fa.FAError):
        fa.fa_backward(q, k, v, o, q, lse, workspace=torch.empty(8, dtype=torch.uint8, device=DEV))
    q3, k3, v3 = synth.make_qkv(1, 1, 64, 64, 96, torch.bfloat16, seed=26, device=DEV)
    o3 = torch.empty_like(q3)
    with pytest.raises(fa.FAError):
        fa.fa_backward(q3, k3, v3, o3, q3, lse)
    with pytest.raises(fa.FAError):      # dQ aliasing K
        fa.fa_backward(q, k, v, o, q, lse, dq=k)


@pytest.mark.parametrize("D,causal", [(64, True), (128, False)])
def test_backward_no_queries_zeroes_dk_dv(fa, D, causal):
    """Nq = 0 < Nk: no query reads a key, so dK = dV = 0 (overwriting
    whatever the output buffers held)."""
    k = synth.normal((1, 2, 70, D), torch.bfloat16, 27, synth.K_ID, DEV)
    v = synth.normal((1, 2, 70, D), torch.bfloat16, 27, synth.V_ID, DEV)
    q = torch.empty((1, 2, 0, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dk = torch.ones_like(k)
    dv = torch.ones_like(v)
    fa.fa_backward(q, k, v, q, q, lse, causal=causal, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert not dk.any() and not dv.any()
