"""The allocation-free decode entry point, fa_decode_splitkv_noalloc, against
fa_decode_splitkv (the same kernels with a caller-provided workspace) through
the C ABI: two calls in a row, the second smaller, so the second reuses the
scratch the first left behind. Both must give the same bits, and the oracle
bound of the decode path besides. Collected last: a failure here hides no
other test."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import attention as orc

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 1e-3


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


def run_pair(fa, B, H, Nk, D, S, seed):
    print(f"[noalloc] B={B} H={H} Nk={Nk} D={D} S={S} seed={seed}", flush=True)
    q, k, v = synth.make_qkv(B, H, 1, Nk, D, torch.bfloat16, seed=seed, device=DEV)
    ref_o, ref_l = fa.fa_decode_splitkv(q, k, v, S)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_decode_splitkv_noalloc(q, k, v, S, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))
    ro, rl = orc.decode(f64(q), f64(k), f64(v), 1.0 / np.sqrt(D))
    err = np.abs(f64(out) - ro)
    lerr = np.abs(f64(lse) - rl[..., 0])
    print(f"[noalloc]   O max {err.max():.3e} mean {err.mean():.3e}  LSE max {lerr.max():.3e}", flush=True)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN and lerr.max() <= BF16_LSE


def test_noalloc_matches_workspace_entry_point_twice(fa):
    # first call: 8 x 8 heads x 64 splits x (128 + 2) floats = 2.1 MB of partials
    run_pair(fa, 8, 8, 3000, 128, 64, seed=11)
    # second call, smaller: fewer heads, splits and keys, D = 64
    run_pair(fa, 2, 3, 700, 64, 5, seed=12)


def test_noalloc_decode_workload_size(fa):
    # the decode workload's partial states (17.0 MB) fit the 32 MiB scratch;
    # a smaller cache keeps the oracle quick
    run_pair(fa, 16, 32, 2048, 128, 64, seed=13)


def test_noalloc_rejects_more_than_the_scratch_holds(fa):
    B, H, D = 64, 64, 128
    S = fa.DECODE_NOALLOC_SCRATCH_BYTES // (B * H * (D + 2) * 4) + 1
    assert fa.fa_decode_workspace_bytes(B, H, D, S) > fa.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, H, 1, D, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, H, 4, D, dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(fa.FAError, match="UNSUPPORTED"):
        fa.fa_decode_splitkv_noalloc(q, k, k, S, out=out)
