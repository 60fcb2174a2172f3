"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances (stated by the workload definition): bf16 O max-abs <= 2e-2 and
mean-abs <= 2e-3; fp32 O max-abs <= 1e-5. LSE is not given a bound there; the
one used here follows from the arithmetic: fp32 accumulation of bf16 products
(exact) over D <= 128 terms and an fp32 row sum give an LSE error of order
1e-5 at these sizes, so 1e-3 (bf16 inputs) and 1e-5 (fp32) leave margin
without hiding a wrong row.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as orc

pytestmark = pytest.mark.gpu

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


DEV = "cuda:0"


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def report(tag, err_o, err_l):
    print(f"[parity] {tag}: O max {err_o.max():.3e} mean {err_o.mean():.3e}  LSE max {err_l.max():.3e}", flush=True)


def check_bf16(tag, o, lse, ro, rl):
    err_o = np.abs(f64(o) - ro) if isinstance(o, torch.Tensor) else np.abs(o - ro)
    err_l = np.abs((f64(lse) if isinstance(lse, torch.Tensor) else lse) - rl)
    report(tag, err_o, err_l)
    assert np.isfinite(err_o).all() and np.isfinite(err_l).all(), tag
    assert err_o.max() <= BF16_MAX, tag
    assert err_o.mean() <= BF16_MEAN, tag
    assert err_l.max() <= BF16_LSE, tag


# ---------------------------------------------------------------- fp32 path

F32_CASES = [
    # (B, H, Nq, Nk, D, causal)
    (1, 1, 256, 256, 64, False),      # the single-head fp32 workload
    (1, 1, 256, 256, 64, True),
    (2, 2, 200, 200, 128, False),
    (1, 3, 131, 131, 128, True),
    (1, 1, 77, 300, 64, False),
    (1, 1, 77, 300, 64, True),
    (1, 1, 1, 1, 64, False),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp32_matches_oracle(fa, case):
    B, H, Nq, Nk, D, causal = case
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.float32, seed=11)
    print(f"[case] fp32 {case}", flush=True)
    o, lse = fa.fa_forward_f32(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), causal)
    err_o, err_l = np.abs(f64(o) - ro), np.abs(f64(lse) - rl)
    report(f"fp32 {case}", err_o, err_l)
    assert err_o.max() <= F32_MAX and err_l.max() <= F32_LSE


# ---------------------------------------------------------------- bf16, small sizes, every row

BF16_CASES = [
    # (B, H, Nq, Nk, D, causal, qk_mul)
    (1, 2, 256, 256, 128, False, 1.0),
    (1, 2, 256, 256, 128, True, 1.0),
    (1, 2, 256, 256, 64, False, 1.0),
    (1, 2, 256, 256, 64, True, 1.0),
    (2, 3, 300, 300, 64, True, 1.0),       # ragged: 300 = 2*128 + 44
    (1, 2, 300, 300, 128, False, 1.0),
    (1, 1, 1, 1, 128, False, 1.0),
    (1, 1, 1, 1, 64, True, 1.0),
    (1, 1, 17, 17, 128, True, 1.0),
    (1, 1, 77, 300, 128, False, 1.0),      # Nq < Nk
    (1, 1, 77, 300, 128, True, 1.0),       # top-left causal with Nq < Nk
    (1, 1, 300, 77, 64, True, 1.0),        # Nq > Nk: late rows see every key
    (1, 4, 513, 513, 128, True, 3.0),      # rescale stress (scores std ~ 9)
    (1, 2, 1000, 1000, 64, True, 1.0),
    (2, 2, 129, 1025, 128, False, 3.0),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bf16_matches_oracle(fa, case):
    B, H, Nq, Nk, D, causal, mul = case
    q, k, v = synth.make_qkv(B, H, Nq, Nk, D, torch.bfloat16, seed=12, qk_mul=mul)
    print(f"[case] bf16 {case}", flush=True)
    o, lse = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), causal)
    check_bf16(f"bf16 {case}", o, lse, ro, rl)


def test_bf16_late_max_in_last_tile(fa):
    """A row whose largest score sits in its last key tile (the case the
    'forgot to rescale o' bug fails): keys grow with their index."""
    D, N = 128, 640
    q = torch.ones(1, 1, N, D, dtype=torch.bfloat16)
    ramp = torch.linspace(-2.0, 2.0, N).view(1, 1, N, 1)
    k = (ramp * torch.ones(1, 1, N, D)).to(torch.bfloat16)
    v = synth.normal((1, 1, N, D), torch.bfloat16, 13, synth.V_ID)
    for causal in (False, True):
        o, lse = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
        torch.cuda.synchronize()
        ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), causal)
        check_bf16(f"late max causal={causal}", o, lse, ro, rl)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("peaky_first", [False, True])
def test_rescale_threshold_paths(fa, dtype, D, causal, peaky_first):
    """Row maxima that grow, tile after tile, by amounts under, just over and
    far over the bound b = 15 on P (2^15, base 2), then stop growing. With
    64-key tiles (D = 128) the maxima, in log2 units over the first tile's 0,
    are b - 6.5 (kept: a lane's 32 P sum to at most 2^(b-1.5)), b + 0.7
    (moved: one P alone is past 2^b), 2b - 6 (kept), 2b + 1.5 and 4b (moved),
    4b + 1 (kept), 4b + 140 (moved; P against the kept maximum would
    overflow fp32), then 4b + 139.5 (kept). With 128-key tiles (D = 64) the
    same keys give maxima b - 6.5, 2b - 6 (moved, b + 0.5 up), 4b and
    4b + 140 (moved), then only kept ones. The keys of a tile other than its
    top lie 0.5 to 12 below it, except in the first tile when peaky_first:
    20 to 30 below, so the first tile's row sums are ~1 and D = 128 waves
    take the tile maximum before the exponentials on every later tile
    (otherwise they exponentiate first and check the row sums). Every query
    row is (1, 1, 0, ...) and key j holds a_j as the sum of its first two
    coordinates (the input-type rounding of a_j and that of the remainder),
    so the base-2 score of key j is a_j * scale * log2(e) to about 16 bits;
    the margins above are checked on the scores the kernel sees (up to its
    fp32 rounding)."""
    N = 1024
    b = 15.0
    scale = 1.0 / math.sqrt(D)
    c2 = scale / math.log(2.0)                    # base-2 score per unit of a_j
    rng = np.random.default_rng(30)
    tops = [0.0, b - 6.5, b + 0.7, 2 * b - 6, 2 * b + 1.5, 4 * b, 4 * b + 1, 4 * b + 140, 4 * b + 139.5]
    tile = 64
    a = np.empty(N)
    top_idx = []
    for t0 in range(0, N, tile):
        top = tops[min(t0 // tile, len(tops) - 1)]
        lo, hi = (20.0, 30.0) if (peaky_first and t0 == 0) else (0.5, 12.0)
        a[t0:t0 + tile] = (top - rng.uniform(lo, hi, tile)) / c2
        top_idx.append(t0 + int(rng.integers(0, tile)))
        a[top_idx[-1]] = top / c2
    a_hi = torch.from_numpy(a).to(dtype)
    a_lo = (torch.from_numpy(a) - a_hi.double()).to(dtype)
    a = a_hi.double().numpy() + a_lo.double().numpy()        # the scores the kernel sees
    got = [a[t0:t0 + tile].max() * c2 for t0 in range(0, N, tile)]
    for t, top in enumerate(got):
        want = tops[min(t, len(tops) - 1)]
        assert abs(top - want) < 0.05 and a[top_idx[t]] * c2 == top, (t, top, want)
    q = torch.zeros(1, 2, N, D, dtype=dtype)
    q[..., :2] = 1.0
    k = torch.zeros(1, 2, N, D, dtype=dtype)
    k[..., 0] = a_hi
    k[..., 1] = a_lo
    v = synth.normal((1, 2, N, D), dtype, 31, synth.V_ID)
    fwd = fa.fa_forward if dtype == torch.bfloat16 else fa.fa_forward_f16
    o, lse = fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    ro, rl = orc.attention(f64(q), f64(k), f64(v), scale, causal)
    check_bf16(f"rescale paths {dtype} D={D} causal={causal}", o, lse, ro, rl)


def test_huge_score_magnitudes(fa):
    """Q and K of magnitude ~20: scores of order 10^3..10^4, the softmax is
    one-hot and the stale-maximum path must never overflow."""
    q, k, v = synth.make_qkv(1, 2, 700, 700, 128, torch.bfloat16, seed=32, qk_mul=20.0)
    for causal in (False, True):
        o, lse = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
        torch.cuda.synchronize()
        ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(128), causal)
        err_l = np.abs(f64(lse) - rl) / np.maximum(1.0, np.abs(rl))
        print(f"[parity] huge scores causal={causal}: LSE rel max {err_l.max():.3e}", flush=True)
        assert np.isfinite(f64(o)).all() and err_l.max() <= 1e-5
        check_bf16(f"huge scores causal={causal}", o, lse, ro, f64(lse))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.float32, 64)])
def test_nan_reaches_exactly_the_rows_that_see_it(fa, dtype, D):
    """Causal, 700 keys. Head 1 has a NaN in key 300: every row that sees it
    (300 and later) comes back with NaN in all of O and in its LSE, as the
    softmax of a NaN score is NaN. Head 0 has a NaN in query row 50: that row
    alone is NaN. Every other row, including rows that share a wave (and its
    rescale vote) with rows that met a NaN, keeps the oracle's values."""
    N, bad_k, bad_q = 700, 300, 50
    q, k, v = synth.make_qkv(1, 2, N, N, D, dtype, seed=33)
    k[0, 1, bad_k, 5] = float("nan")
    q[0, 0, bad_q, 7] = float("nan")
    fwd = fa.fa_forward if dtype == torch.bfloat16 else fa.fa_forward_f32
    o, lse = fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    o, lse = f64(o), f64(lse)
    nan_rows = np.zeros((2, N), dtype=bool)
    nan_rows[1, bad_k:] = True
    nan_rows[0, bad_q] = True
    ro, rl = orc.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), True)
    assert np.array_equal(np.isnan(rl[0]), nan_rows) and np.isnan(ro[0][nan_rows]).all()
    assert np.isnan(o[0][nan_rows]).all() and np.isnan(lse[0][nan_rows]).all()
    keep = ~nan_rows
    assert not np.isnan(o[0][keep]).any() and not np.isnan(lse[0][keep]).any()
    if dtype == torch.float32:
        assert np.abs(o[0][keep] - ro[0][keep]).max() <= 1e-5 and np.abs(lse[0][keep] - rl[0][keep]).max() <= 1e-5
    else:
        check_bf16(f"NaN rows D={D} (the other rows)", o[0][keep], lse[0][keep], ro[0][keep], rl[0][keep])


def test_nan_reaches_exactly_the_heads_that_see_it_decode(fa):
    """Split-KV decode, 5000 keys in 8 splits: head 1 has a NaN in key 1234,
    head 2 a NaN in its query (every score of that head is NaN, so whole
    splits hold nothing but NaN scores): both heads come back NaN in O and
    LSE; head 0 keeps the oracle's values."""
    q, k, v = synth.make_qkv(1, 3, 1, 5000, 128, torch.bfloat16, seed=34)
    k[0, 1, 1234, 3] = float("nan")
    q[0, 2, 0, 9] = float("nan")
    o, lse = fa.fa_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), num_splits=8)
    torch.cuda.synchronize()
    o, lse = f64(o), f64(lse)
    assert np.isnan(o[0, 1:]).all() and np.isnan(lse[0, 1:]).all()
    ro, rl = orc.attention(f64(q[:, :1]), f64(k[:, :1]), f64(v[:, :1]), 1.0 / math.sqrt(128), False)
    check_bf16("decode NaN heads (the clean head)", o[:, :1], lse[:, :1], ro, rl)


# ---------------------------------------------------------------- closed forms and invariants on the GPU

@pytest.mark.parametrize("D", [64, 128])
def test_zero_keys_give_prefix_means(fa, D):
    """K = 0: causal row i is the mean of V[0..i] and LSE = ln(i+1); non-causal
    rows are the column mean with LSE = ln(Nk). Independent of the oracle."""
    N = 333
    q = synth.normal((1, 2, N, D), torch.bfloat16, 14, synth.Q_ID)
    k = torch.zeros(1, 2, N, D, dtype=torch.bfloat16)
    v = synth.normal((1, 2, N, D), torch.bfloat16, 14, synth.V_ID)
    vd = f64(v)
    o, lse = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    prefix = np.cumsum(vd, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    check_bf16(f"K=0 causal D={D}", o, lse, prefix, np.broadcast_to(np.log(np.arange(1, N + 1)), (1, 2, N)))
    o, lse = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=False)
    torch.cuda.synchronize()
    check_bf16(f"K=0 full D={D}", o, lse, np.broadcast_to(vd.mean(axis=2, keepdims=True), vd.shape),
               np.full((1, 2, N), math.log(N)))


def test_ones_values_and_causal_first_row(fa):
    B, H, N, D = 1, 3, 400, 128
    q, k, v = synth.make_qkv(B, H, N, N, D, torch.bfloat16, seed=15, qk_mul=3.0)
    ones = torch.ones_like(v)
    for causal in (False, True):
        o, _ = fa.fa_forward(q.to(DEV), k.to(DEV), ones.to(DEV), causal=causal)
        torch.cuda.synchronize()
        assert np.abs(f64(o) - 1.0).max() <= 2.0 ** -8, "V = 1 must give O = 1"
    o, _ = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    # Row 0 attends key 0 only. Its running maximum becomes its own scaled
    # score, so its one weight is exp2 of that score's fp32 rounding error: a
    # few fp32 ulps from 1, which bf16 rounds to exactly 1. Then O = V[0] / l
    # with l that close to 1, and rounding to bf16 gives V[0] back, bit for bit.
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    ofull, _ = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=False)
    torch.cuda.synchronize()
    # the last row sees every key: causal and full agree bit for bit
    assert torch.equal(o[:, :, -1].cpu(), ofull[:, :, -1].cpu())


def test_permuting_keys_and_values(fa):
    B, H, N, D = 1, 2, 320, 128
    q, k, v = synth.make_qkv(B, H, N, N, D, torch.bfloat16, seed=16)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(17))
    o1, l1 = fa.fa_forward(q.to(DEV), k.to(DEV), v.to(DEV))
    o2, l2 = fa.fa_forward(q.to(DEV), k[:, :, perm].contiguous().to(DEV), v[:, :, perm].contiguous().to(DEV))
    torch.cuda.synchronize()
    assert np.abs(f64(o1) - f64(o2)).max() <= 2e-2
    assert np.abs(f64(l1) - f64(l2)).max() <= 1e-3


def test_run_to_run_bitwise(fa):
    """No atomics and a fixed reduction order: two runs agree bit for bit
    (a missing LDS barrier would show up here as a difference)."""
    for (B, H, N, D, causal) in [(1, 8, 1100, 128, True), (1, 8, 1100, 64, False)]:
        q, k, v = synth.make_qkv(B, H, N, N, D, torch.bfloat16, seed=18, device=DEV)
        a = fa.fa_forward(q, k, v, causal=causal)
        b = fa.fa_forward(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    q, k, v = synth.make_qkv(4, 8, 1, 5000, 128, torch.bfloat16, seed=19, device=DEV)
    a = fa.fa_decode_splitkv(q, k, v, num_splits=16)
    b = fa.fa_decode_splitkv(q, k, v, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_lse_optional(fa):
    q, k, v = synth.make_qkv(1, 2, 200, 200, 128, torch.bfloat16, seed=20, device=DEV)
    o1, _ = fa.fa_forward(q, k, v, causal=True)
    o2, l2 = fa.fa_forward(q, k, v, causal=True, want_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)


# ---------------------------------------------------------------- split-KV decode

DECODE_CASES = [
    # (B, H, Nk, D, num_splits)
    (2, 3, 1000, 128, 1),
    (2, 3, 1000, 128, 2),
    (2, 3, 1000, 128, 7),
    (2, 3, 1000, 64, 64),
    (1, 2, 37, 128, 64),       # more splits than keys: empty chunks
    (1, 2, 37, 64, 37),
    (1, 1, 1, 128, 3),
    (3, 5, 4097, 128, 16),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_matches_oracle(fa, case):
    B, H, Nk, D, S = case
    q, k, v = synth.make_qkv(B, H, 1, Nk, D, torch.bfloat16, seed=21)
    print(f"[case] decode {case}", flush=True)
    o, lse = fa.fa_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), num_splits=S)
    torch.cuda.synchronize()
    ro, rl = orc.decode(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D))
    check_bf16(f"decode {case}", o, lse, ro, rl[:, :, 0])


def test_decode_agrees_with_forward(fa):
    q, k, v = synth.make_qkv(2, 4, 1, 3000, 128, torch.bfloat16, seed=22, device=DEV)
    of, lf = fa.fa_forward(q, k, v)
    for S in (1, 2, 64, 3000):
        od, ld = fa.fa_decode_splitkv(q, k, v, num_splits=S)
        torch.cuda.synchronize()
        assert np.abs(f64(od) - f64(of)).max() <= 2e-2
        assert np.abs(f64(ld) - f64(lf)[:, :, 0]).max() <= 1e-3
