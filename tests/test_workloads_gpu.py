"""GPU parity at the full workload sizes, in the launch configuration the bench
times (the same library call on the same seeded device-resident inputs).
The oracle checks a sample of rows of every (batch, head) — the first 64, the
last 64 (which hold any ragged tail) and 64 seeded random rows — and, for the
decode workload, 64 of its (batch, head) pairs; each sampled row is computed
by the oracle in full against all keys of its head."""

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

    return m


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def sample_rows(n, seed):
    rng = np.random.default_rng(seed)
    rows = set(range(min(64, n))) | set(range(max(0, n - 64), n)) | set(rng.integers(0, n, 64).tolist())
    return np.array(sorted(rows))


def check_prefill(fa, w, seed=0):
    q, k, v = synth.make_workload(w, seed=seed, device=DEV)
    print(f"[case] {w.name}", flush=True)
    fwd = fa.fa_forward_f32 if w.dtype == torch.float32 else fa.fa_forward
    o, lse = fwd(q, k, v, causal=w.causal, scale=w.scale)
    # A second run at full size gives the same bits (fixed reduction order).
    o2, lse2 = fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    del o2, lse2
    if w.causal and w.dtype != torch.float32:
        # the first row sees key 0 only: O = V[0] bit for bit (see test_parity_gpu)
        assert torch.equal(o[:, :, 0], v[:, :, 0])
    rows = sample_rows(w.Nq, seed + 1)
    rows_t = torch.as_tensor(rows, device=DEV)
    worst_o, worst_l, sum_o, count = 0.0, 0.0, 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            ro, rl = orc.attention_rows(f64(q[b, h].index_select(0, rows_t)), rows, f64(k[b, h]), f64(v[b, h]),
                                        w.scale, w.causal)
            eo = np.abs(f64(o[b, h].index_select(0, rows_t)) - ro)
            el = np.abs(f64(lse[b, h].index_select(0, rows_t)) - rl)
            assert np.isfinite(eo).all() and np.isfinite(el).all()
            worst_o, worst_l = max(worst_o, eo.max()), max(worst_l, el.max())
            sum_o += eo.sum()
            count += eo.size
    mean_o = sum_o / count
    print(f"[parity] {w.name}: O max {worst_o:.3e} mean {mean_o:.3e} LSE max {worst_l:.3e}", flush=True)
    if w.dtype == torch.float32:
        assert worst_o <= 1e-5 and worst_l <= 1e-5
    else:
        assert worst_o <= BF16_MAX and mean_o <= BF16_MEAN and worst_l <= BF16_LSE


@pytest.mark.parametrize("name", [n for n, w in synth.WORKLOADS.items() if not w.is_decode])
def test_prefill_workload(fa, name):
    check_prefill(fa, synth.WORKLOADS[name])


def test_ragged_16001(fa):
    """16000 is a multiple of 128; one more row makes every tile size ragged."""
    w = synth.WORKLOADS["causal_b1_h16_n16000_d64"]
    check_prefill(fa, synth.Workload("causal_b1_h16_n16001_d64", 1, 16, 16001, 16001, 64, torch.bfloat16, causal=True))
    assert w.Nq == 16000


def test_decode_workload(fa):
    w = synth.WORKLOADS["decode_b16_h32_kv32768_d128_s64"]
    q, k, v = synth.make_workload(w, seed=0, device=DEV)
    print(f"[case] {w.name}", flush=True)
    o, lse = fa.fa_decode_splitkv(q, k, v, num_splits=w.num_splits, scale=w.scale)
    o2, lse2 = fa.fa_decode_splitkv(q, k, v, num_splits=w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    rng = np.random.default_rng(5)
    pairs = {(0, 0), (w.B - 1, w.H - 1)} | {(int(b), int(h)) for b, h in zip(rng.integers(0, w.B, 62), rng.integers(0, w.H, 62))}
    worst_o, worst_l, sum_o, count = 0.0, 0.0, 0.0, 0
    for b, h in sorted(pairs):
        ro, rl = orc.attention_rows(f64(q[b, h]), [0], f64(k[b, h]), f64(v[b, h]), w.scale, False)
        eo = np.abs(f64(o[b, h]) - ro)
        el = abs(float(lse[b, h]) - rl[0])
        worst_o, worst_l = max(worst_o, eo.max()), max(worst_l, el)
        sum_o += eo.sum()
        count += eo.size
    mean_o = sum_o / count
    print(f"[parity] {w.name}: {len(pairs)} heads, O max {worst_o:.3e} mean {mean_o:.3e} LSE max {worst_l:.3e}",
          flush=True)
    assert worst_o <= BF16_MAX and mean_o <= BF16_MEAN and worst_l <= BF16_LSE


@pytest.mark.parametrize("B,H,N,D,causal", [
    (1, 1, 131072, 128, False),   # 2048 key tiles per workgroup, 512 query blocks
    (64, 64, 256, 64, True),      # 4096 (batch, head) pairs of one query block each
])
def test_long_and_wide_shapes(fa, B, H, N, D, causal):
    """Sizes past the workloads': a 131072-long sequence (a long key loop per
    workgroup and row indices past 2^16) and a grid of 4096 heads. Sampled
    rows (first, last, random) of a few (batch, head) pairs against the
    oracle, each row over all of its keys."""
    print(f"[case] long/wide {B}x{H}x{N}x{D} causal={causal}", flush=True)
    q, k, v = synth.make_qkv(B, H, N, N, D, torch.bfloat16, seed=9, device=DEV)
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.fa_forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    pairs = {(0, 0), (B - 1, H - 1)} | {(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(3)}
    rows = np.array(sorted(set(range(8)) | set(range(N - 8, N)) | set(rng.integers(0, N, 16).tolist())))
    rows_t = torch.as_tensor(rows, device=DEV)
    worst_o, worst_l = 0.0, 0.0
    for b, h in sorted(pairs):
        ro, rl = orc.attention_rows(f64(q[b, h].index_select(0, rows_t)), rows, f64(k[b, h]), f64(v[b, h]),
                                    scale, causal)
        eo = np.abs(f64(o[b, h].index_select(0, rows_t)) - ro)
        el = np.abs(f64(lse[b, h].index_select(0, rows_t)) - rl)
        assert np.isfinite(eo).all() and np.isfinite(el).all()
        worst_o, worst_l = max(worst_o, eo.max()), max(worst_l, el.max())
    print(f"[parity] long/wide {B}x{H}x{N}x{D}: O max {worst_o:.3e} LSE max {worst_l:.3e}", flush=True)
    assert worst_o <= BF16_MAX and worst_l <= BF16_LSE


@pytest.mark.parametrize("Nk,S", [(1 << 20, 256), (100003, 1000)])
def test_decode_long_cache_and_many_splits(fa, Nk, S):
    """Decode past the workload's sizes: a cache of 2^20 keys in 256 splits of
    4096, and a prime length in 1000 splits (chunks of 101 keys, the last ones
    short or empty), against the oracle over every key of each head."""
    B, H, D = 1, 2, 128
    print(f"[case] decode Nk={Nk} splits={S}", flush=True)
    q, k, v = synth.make_qkv(B, H, 1, Nk, D, torch.bfloat16, seed=11, device=DEV)
    o, lse = fa.fa_decode_splitkv(q, k, v, num_splits=S)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(D)
    worst_o, worst_l = 0.0, 0.0
    for h in range(H):
        ro, rl = orc.attention_rows(f64(q[0, h]), [0], f64(k[0, h]), f64(v[0, h]), scale, False)
        worst_o = max(worst_o, float(np.abs(f64(o[0, h]) - ro).max()))
        worst_l = max(worst_l, abs(float(lse[0, h]) - float(rl[0])))
    print(f"[parity] decode Nk={Nk} splits={S}: O max {worst_o:.3e} LSE max {worst_l:.3e}", flush=True)
    assert worst_o <= BF16_MAX and worst_l <= BF16_LSE
