"""Pins that tie the fp64 oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` takes the oracle module as its argument so the same checks can be
run on deliberately broken copies of the oracle (tests/test_oracle_mutations.py)
to show that a plausible mistake is caught. None of these re-types the oracle's
own formula: they use printed numbers, closed forms, invariants, an independent
library routine (torch's float64 CPU attention) or a different algorithm
(online recurrences against the two-pass definition).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---- printed worked examples -------------------------------------------------

def pin_worked_example_trace(orc):
    """Online softmax state after every key equals the printed trace (section 11.6)."""
    g = _golden("worked_example.json")
    (m, l, o), states = orc.online_per_key(g["scores"], g["values"], trace=True)
    half_ulp = 0.5 * 10.0 ** (-g["printed_decimals"]) + 1e-12
    assert len(states) == len(g["states"])
    for got, want in zip(states, g["states"]):
        for idx, key in enumerate(["m", "corr", "p", "l", "o"]):
            _close(got[idx], want[key], half_ulp, f"key {want['key']} {key}")
    _close(o / l, g["o_over_l"], 0.5 * 10.0 ** (-g["o_over_l_decimals"]) + 1e-12, "online o/l")


def pin_worked_example_two_pass(orc):
    """The two-pass definition gives the printed 21.546979 and LSE = 3 + ln(1 + e^-1 + e^-2)."""
    g = _golden("worked_example.json")
    q = np.ones((1, 1, 1, 1))
    k = np.array(g["scores"]).reshape(1, 1, 3, 1)
    v = np.array(g["values"]).reshape(1, 1, 3, 1)
    o, lse = orc.attention(q, k, v, 1.0, causal=False)
    _close(o[0, 0, 0, 0], g["o_over_l"], 0.5e-6 + 1e-12, "two-pass o")
    _close(lse[0, 0, 0], 3.0 + math.log(1.0 + math.exp(-1.0) + math.exp(-2.0)), 1e-14, "two-pass lse")


def pin_merge_example(orc):
    """Solution 3: states of {0} and {1, 2} and their merge, as printed."""
    g = _golden("merge_example.json")
    s, v = g["scores"], g["values"]
    tol = 0.5 * 10.0 ** (-g["printed_decimals"]) + 1e-12
    a = orc.online_per_key(s[:1], v[:1])
    b = orc.online_per_key(s[1:], v[1:])
    for state, want, what in [(a, g["part_a"], "{0}"), (b, g["part_b"], "{1,2}")]:
        _close(state[0], want["m"], tol, what + " m")
        _close(state[1], want["l"], tol, what + " l")
        _close(state[2], want["o"], tol, what + " o")
    mm, ml, mo = orc.merge(a, b)
    _close(mm, g["merged"]["m"], tol, "merged m")
    _close(ml, g["merged"]["l"], tol, "merged l")
    _close(mo, g["merged"]["o"], tol, "merged o")
    o, _ = orc.combine([a, b])
    _close(o, g["o_over_l"], 0.5 * 10.0 ** (-g["o_over_l_decimals"]) + 1e-12, "merged o/l")


# ---- closed forms ------------------------------------------------------------

def pin_single_key(orc):
    """Nk = 1: O = V[0] and LSE = scale * q . k_0 for every row, causal or not."""
    q = _rand((2, 3, 5, 8), 1)
    k = _rand((2, 3, 1, 8), 2)
    v = _rand((2, 3, 1, 8), 3)
    scale = 0.37
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, scale, causal)
        _close(o, np.broadcast_to(v, o.shape), 1e-14, "Nk=1 O")
        _close(lse, scale * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0]), 1e-13, "Nk=1 LSE")


def pin_zero_keys_means(orc):
    """K = 0: every allowed key has weight 1/count, so O is a mean of V rows and
    LSE = ln(count). Causal row i averages V[0..i] (prefix means)."""
    nq = nk = 9
    q = _rand((1, 2, nq, 4), 4)
    k = np.zeros((1, 2, nk, 4))
    v = _rand((1, 2, nk, 4), 5)
    o, lse = orc.attention(q, k, v, 0.5, causal=False)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-14, "K=0 full O")
    _close(lse, np.full(lse.shape, math.log(nk)), 1e-14, "K=0 full LSE")
    o, lse = orc.attention(q, k, v, 0.5, causal=True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, nk + 1)[None, None, :, None]
    _close(o, prefix, 1e-14, "K=0 causal O")
    _close(lse, np.broadcast_to(np.log(np.arange(1, nq + 1)), lse.shape), 1e-14, "K=0 causal LSE")


def pin_zero_scale_rectangular(orc):
    """scale = 0 with Nq != Nk: non-causal rows are column means; causal row i
    (top-left) averages V[0..min(i, Nk-1)]."""
    nq, nk = 7, 4
    q = _rand((1, 1, nq, 3), 6)
    k = _rand((1, 1, nk, 3), 7)
    v = _rand((1, 1, nk, 3), 8)
    o, _ = orc.attention(q, k, v, 0.0, causal=True)
    for i in range(nq):
        _close(o[0, 0, i], v[0, 0, : min(i, nk - 1) + 1].mean(axis=0), 1e-14, f"scale=0 causal row {i}")
    o, _ = orc.attention(q, k, v, 0.0, causal=False)
    _close(o[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (nq, 3)), 1e-14, "scale=0 full")


# ---- invariants --------------------------------------------------------------

def pin_weights_sum_to_one(orc):
    q = _rand((13, 6), 9)
    k = _rand((11, 6), 10) * 4.0
    for causal in (False, True):
        p = orc.softmax_weights(q, k, 0.41, causal)
        _close(p.sum(axis=1), np.ones(13), 1e-14, "row sums")
        assert np.all(p >= 0.0)
        if causal:
            assert np.all(p[np.triu_indices(11, 1)] == 0.0), "masked weight not zero"


def pin_ones_values(orc):
    q = _rand((1, 2, 10, 5), 11) * 3.0
    k = _rand((1, 2, 10, 5), 12) * 3.0
    v = np.ones((1, 2, 10, 5))
    for causal in (False, True):
        o, _ = orc.attention(q, k, v, 0.3, causal)
        _close(o, np.ones_like(o), 1e-14, "V=1")


def pin_permutation(orc):
    """Permuting K and V rows together leaves non-causal O and LSE unchanged."""
    q = _rand((2, 1, 6, 7), 13)
    k = _rand((2, 1, 12, 7), 14)
    v = _rand((2, 1, 12, 7), 15)
    perm = np.random.default_rng(16).permutation(12)
    o1, l1 = orc.attention(q, k, v, 0.5)
    o2, l2 = orc.attention(q, k[:, :, perm], v[:, :, perm], 0.5)
    _close(o1, o2, 1e-13, "permuted O")
    _close(l1, l2, 1e-13, "permuted LSE")


def pin_causal_edges(orc):
    """Causal row 0 is V[0] exactly; the last row of a square causal problem sees
    every key and equals the non-causal last row exactly."""
    q = _rand((1, 3, 8, 4), 17) * 2.0
    k = _rand((1, 3, 8, 4), 18) * 2.0
    v = _rand((1, 3, 8, 4), 19)
    oc, lc = orc.attention(q, k, v, 0.7, causal=True)
    of, lf = orc.attention(q, k, v, 0.7, causal=False)
    assert np.array_equal(oc[:, :, 0], v[:, :, 0]), "causal row 0 != V[0]"
    _close(lc[:, :, 0], 0.7 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-14, "causal row 0 LSE")
    assert np.array_equal(oc[:, :, -1], of[:, :, -1]), "causal last row != full last row"
    assert np.array_equal(lc[:, :, -1], lf[:, :, -1])
    assert not np.allclose(oc[:, :, 1:-1], of[:, :, 1:-1]), "causal mask had no effect"


def pin_nan_stays_in_its_rows(orc):
    """A NaN score reaches exactly the rows that attend it (the softmax of a
    row holding a NaN score is NaN, O and LSE alike), and masked keys never
    contribute: a NaN in a key that causal rows cannot see, or in a padding
    key past kv_lens, leaves those rows as they were. A NaN in column c of a
    value row makes column c of O NaN in the rows that attend it, and leaves
    the LSE (a function of the scores alone) and the other columns as they
    were. Where it lands in rows that mask it is not part of the promise: a
    masked weight is an exact zero and 0 * NaN is NaN."""
    q = _rand((1, 2, 9, 4), 40)
    k = _rand((1, 2, 9, 4), 41)
    v = _rand((1, 2, 9, 4), 42)
    o0, l0 = orc.attention(q, k, v, 0.5, causal=True)
    kn = k.copy()
    kn[0, 1, 5, 2] = np.nan
    o1, l1 = orc.attention(q, kn, v, 0.5, causal=True)
    assert np.isnan(o1[0, 1, 5:]).all() and np.isnan(l1[0, 1, 5:]).all(), "rows that see the NaN key"
    assert np.array_equal(o1[0, 1, :5], o0[0, 1, :5]) and np.array_equal(l1[0, 1, :5], l0[0, 1, :5]), \
        "rows before the NaN key changed"
    assert np.array_equal(o1[0, 0], o0[0, 0]) and np.array_equal(l1[0, 0], l0[0, 0]), "other head changed"
    vn = v.copy()
    vn[0, 0, 3, 1] = np.nan
    o2, l2 = orc.attention(q, k, vn, 0.5, causal=True)
    assert np.isnan(o2[0, 0, 3:, 1]).all() and np.array_equal(l2, l0), "NaN value row"
    assert np.array_equal(np.delete(o2, 1, axis=-1), np.delete(o0, 1, axis=-1)), "other columns changed"
    assert np.array_equal(o2[0, 1], o0[0, 1]), "other head changed"
    kp = k.copy()
    kp[0, :, 6:] = np.nan                  # padding: kv_lens = 6
    o3, l3 = orc.attention(q, kp, v, 0.5, causal=False, kv_lens=[6])
    o4, l4 = orc.attention(q, k, v, 0.5, causal=False, kv_lens=[6])
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4), "NaN padding keys leaked"


# ---- an independent library routine -----------------------------------------

def pin_torch_sdpa(orc):
    """torch's float64 CPU scaled_dot_product_attention (top-left causal mask)
    and logsumexp agree with the oracle."""
    for (b, h, nq, nk, d, causal, seed) in [(2, 3, 17, 17, 8, False, 20), (1, 2, 19, 19, 16, True, 21),
                                            (1, 1, 5, 23, 4, False, 22), (1, 2, 23, 9, 4, True, 23)]:
        q = _rand((b, h, nq, d), seed) * 2.0
        k = _rand((b, h, nk, d), seed + 100) * 2.0
        v = _rand((b, h, nk, d), seed + 200)
        scale = 1.0 / math.sqrt(d)
        o, lse = orc.attention(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        _close(o, ref.numpy(), 1e-12, f"sdpa O {nq}x{nk} causal={causal}")
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(~torch.ones(nq, nk, dtype=torch.bool).tril(), -math.inf)
        _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, f"logsumexp {nq}x{nk} causal={causal}")


# ---- a different algorithm reaching the same result ---------------------------

def pin_online_blocked_matches(orc):
    """Block-wise online softmax = two-pass, for block sizes that do and do not
    divide Nk, causal and not, and Nq != Nk."""
    for (nq, nk, causal) in [(9, 9, True), (9, 9, False), (5, 13, False), (13, 13, True), (4, 11, True)]:
        q = _rand((nq, 6), nq * 31 + nk) * 3.0
        k = _rand((nk, 6), nq * 37 + nk) * 3.0
        v = _rand((nk, 6), nq * 41 + nk)
        o_ref, l_ref = orc.attention(q[None, None], k[None, None], v[None, None], 0.45, causal)
        for block in (1, 2, 3, 4, 7, 16, nk + 5):
            o, l = orc.online_blocked(q, k, v, 0.45, causal, block)
            _close(o, o_ref[0, 0], 1e-12, f"blocked O block={block} causal={causal}")
            _close(l, l_ref[0, 0], 1e-12, f"blocked LSE block={block} causal={causal}")


def pin_online_per_key_matches(orc):
    """Per-key recurrence = two-pass on a row whose maximum comes last (the case
    of the exercise 'Find the bug')."""
    s = np.array([0.5, -1.0, 2.0, 1.5, 9.0])
    v = _rand((5, 3), 24)
    m, l, o = orc.online_per_key(s, v)
    q = np.ones((1, 1, 1, 1))
    o_ref, l_ref = orc.attention(q, s.reshape(1, 1, 5, 1), v[None, None], 1.0)
    _close(o / l, o_ref[0, 0, 0], 1e-14, "per-key late max")
    _close(m + math.log(l), l_ref[0, 0, 0], 1e-14, "per-key LSE")


def pin_split_combine(orc):
    """Every chunking of the keys (including empty trailing chunks) merges back
    to the two-pass answer (exercise 'Flash-decoding' with the merge rule)."""
    nk = 37
    q = _rand((1, 1, 1, 8), 25) * 2.0
    k = _rand((1, 1, nk, 8), 26) * 2.0
    v = _rand((1, 1, nk, 8), 27)
    o_ref, l_ref = orc.decode(q, k, v, 0.35)
    for splits in (1, 2, 3, 5, 8, nk, nk + 3, 64):
        bounds = orc.chunk_bounds(nk, splits)
        covered = np.concatenate([np.arange(a, b) for a, b in bounds])
        assert np.array_equal(covered, np.arange(nk)), f"chunks do not tile the keys for S={splits}"
        parts = orc.split_states(q[0, 0, 0], k[0, 0], v[0, 0], 0.35, splits)
        o, lse = orc.combine(parts)
        _close(o, o_ref[0, 0, 0], 1e-13, f"split O S={splits}")
        _close(lse, l_ref[0, 0, 0], 1e-13, f"split LSE S={splits}")


# ---- backward pass ------------------------------------------------------------

def pin_backward_finite_differences(orc):
    """Central differences of the forward oracle: for L = sum(O * G), dL/dX from
    (L(X + h E) - L(X - h E)) / 2h for every element of Q, K and V, against the
    backward oracle (tiny shapes; causal and not; Nq != Nk)."""
    h = 1e-6
    for (nq, nk, d, causal, seed) in [(4, 4, 3, False, 40), (5, 5, 2, True, 41), (3, 6, 3, False, 42)]:
        q = _rand((1, 1, nq, d), seed) * 1.5
        k = _rand((1, 1, nk, d), seed + 1) * 1.5
        v = _rand((1, 1, nk, d), seed + 2)
        g = _rand((1, 1, nq, d), seed + 3)
        scale = 0.6
        dq, dk, dv = orc.attention_backward(q, k, v, g, scale, causal)

        def loss(qq, kk, vv):
            return float(np.sum(orc.attention(qq, kk, vv, scale, causal)[0] * g))

        for name, x, grad in (("Q", q, dq), ("K", k, dk), ("V", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                pos = "QKV".index(name)
                args_p[pos], args_m[pos] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(grad, num, 1e-7, f"finite differences d{name} {nq}x{nk} causal={causal}")


def pin_backward_torch_autograd(orc):
    """torch's float64 CPU autograd through scaled_dot_product_attention (an
    independent library routine) agrees with the backward oracle."""
    for (b, hh, nq, nk, d, causal, seed) in [(1, 2, 11, 11, 8, True, 43), (2, 1, 7, 13, 4, False, 44)]:
        q = _rand((b, hh, nq, d), seed) * 2.0
        k = _rand((b, hh, nk, d), seed + 1) * 2.0
        v = _rand((b, hh, nk, d), seed + 2)
        g = _rand((b, hh, nq, d), seed + 3)
        scale = 1.0 / math.sqrt(d)
        dq, dk, dv = orc.attention_backward(q, k, v, g, scale, causal)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        out.backward(torch.from_numpy(g))
        _close(dq, tq.grad.numpy(), 1e-12, f"autograd dQ causal={causal}")
        _close(dk, tk.grad.numpy(), 1e-12, f"autograd dK causal={causal}")
        _close(dv, tv.grad.numpy(), 1e-12, f"autograd dV causal={causal}")


def pin_backward_closed_forms(orc):
    """dO = 0 gives zero gradients; equal V rows make O independent of Q and K
    (dQ = dK = 0); dK sums to zero over the keys (adding one vector to every
    key shifts each row of S by a constant, which softmax ignores); dV sums
    over the keys to the
    column sums of dO (each row of P sums to one); the causal row 0 sees one
    key, so its dQ is zero."""
    q = _rand((1, 1, 9, 4), 45) * 2.0
    k = _rand((1, 1, 9, 4), 46) * 2.0
    v = _rand((1, 1, 9, 4), 47)
    g = _rand((1, 1, 9, 4), 48)
    for causal in (False, True):
        dq, dk, dv = orc.attention_backward(q, k, v, np.zeros_like(g), 0.5, causal)
        _close(np.abs(dq) + np.abs(dk) + np.abs(dv), np.zeros_like(q), 0.0, f"dO = 0 causal={causal}")
        vconst = np.broadcast_to(_rand((1, 1, 1, 4), 49), v.shape).copy()
        dq, dk, dv = orc.attention_backward(q, k, vconst, g, 0.5, causal)
        _close(dq, np.zeros_like(dq), 1e-13, f"equal V rows dQ causal={causal}")
        _close(dk, np.zeros_like(dk), 1e-13, f"equal V rows dK causal={causal}")
        dq, dk, dv = orc.attention_backward(q, k, v, g, 0.5, causal)
        _close(dk.sum(axis=2), np.zeros((1, 1, 4)), 1e-13, f"sum of dK causal={causal}")
        _close(dv.sum(axis=2), g.sum(axis=2), 1e-13, f"sum of dV causal={causal}")
        if causal:
            _close(dq[0, 0, 0], np.zeros(4), 0.0, "causal row 0 dQ")


# ---- padding masks, bottom-right alignment, fully masked rows ------------------

def _allowed_count(i, nq, nk, causal, kv_len):
    """How many keys row i may attend, counted by hand from the rule."""
    L = nk if kv_len is None else kv_len
    if causal == 0:
        return L
    last = i if causal == 1 else i + (L - nq)      # last visible key index
    return max(0, min(L, last + 1))


def pin_mask_closed_forms(orc):
    """K = 0: each allowed key weighs 1/count, so O is the mean of the first
    count V rows and LSE = ln(count); a row with no allowed key has O = 0 and
    LSE = -inf (the empty sums). Padding, top-left and bottom-right, Nq < Nk,
    Nq > Nk, and a batch entry with no real key."""
    for (nq, nk, causal, kv_lens) in [(6, 9, 0, [9, 4]), (6, 9, 1, [7, 0]), (6, 9, 2, [9, 5]),
                                      (9, 5, 2, [5, 3]), (9, 5, 1, [2, 5]), (4, 4, 2, [4, 1])]:
        q = _rand((2, 2, nq, 3), nq * 7 + nk)
        k = np.zeros((2, 2, nk, 3))
        v = _rand((2, 2, nk, 3), nq * 11 + nk)
        o, lse = orc.attention(q, k, v, 0.7, causal, kv_lens=kv_lens)
        for b in range(2):
            for i in range(nq):
                c = _allowed_count(i, nq, nk, causal, kv_lens[b])
                tag = f"K=0 nq={nq} nk={nk} causal={causal} len={kv_lens[b]} row {i}"
                if c == 0:
                    _close(o[b, :, i], np.zeros((2, 3)), 0.0, tag + " O")
                    assert np.all(lse[b, :, i] == -math.inf), tag + " LSE"
                else:
                    _close(o[b, :, i], v[b, :, :c].mean(axis=1), 1e-14, tag + " O")
                    _close(lse[b, :, i], np.full(2, math.log(c)), 1e-14, tag + " LSE")


def pin_padding_is_truncation(orc):
    """Keys past kv_len are invisible: the result equals attention over the
    first kv_len keys alone, whatever the padded keys hold."""
    nq, nk, L = 7, 12, 8
    q = _rand((1, 2, nq, 4), 60) * 2.0
    k = _rand((1, 2, nk, 4), 61) * 2.0
    v = _rand((1, 2, nk, 4), 62)
    for causal in (0, 1, 2):
        o, lse = orc.attention(q, k, v, 0.5, causal, kv_lens=[L])
        o_t, lse_t = orc.attention(q, k[:, :, :L], v[:, :, :L], 0.5, causal)
        _close(o, o_t, 1e-14, f"padding = truncation O causal={causal}")
        _close(lse, lse_t, 1e-14, f"padding = truncation LSE causal={causal}")
        k2, v2 = k.copy(), v.copy()
        k2[:, :, L:] = 1e3
        v2[:, :, L:] = -7.0
        o2, lse2 = orc.attention(q, k2, v2, 0.5, causal, kv_lens=[L])
        _close(o2, o, 0.0, f"padded keys ignored causal={causal}")
        _close(lse2, lse, 0.0, f"padded keys ignored LSE causal={causal}")


def pin_bottom_right_is_suffix(orc):
    """Bottom-right causal on Nq queries equals the last Nq rows of top-left
    causal attention over Nk queries whose last rows are those queries
    (Nq <= Nk); with Nq > Nk the first Nq - Nk rows see no key and the rest
    are square top-left causal attention of the last Nk queries."""
    nk, d = 11, 4
    k = _rand((1, 1, nk, d), 63) * 2.0
    v = _rand((1, 1, nk, d), 64)
    for nq in (1, 4, 11):
        full_q = _rand((1, 1, nk, d), 65 + nq) * 2.0
        q = full_q[:, :, nk - nq:]
        o, lse = orc.attention(q, k, v, 0.5, 2)
        o_f, lse_f = orc.attention(full_q, k, v, 0.5, True)
        _close(o, o_f[:, :, nk - nq:], 1e-14, f"bottom-right nq={nq} O")
        _close(lse, lse_f[:, :, nk - nq:], 1e-14, f"bottom-right nq={nq} LSE")
    nq = 15
    q = _rand((1, 1, nq, d), 66) * 2.0
    o, lse = orc.attention(q, k, v, 0.5, 2)
    o_sq, lse_sq = orc.attention(q[:, :, nq - nk:], k, v, 0.5, True)
    _close(o[:, :, nq - nk:], o_sq, 1e-14, "bottom-right nq>nk tail O")
    _close(lse[:, :, nq - nk:], lse_sq, 1e-14, "bottom-right nq>nk tail LSE")
    _close(o[:, :, : nq - nk], np.zeros((1, 1, nq - nk, d)), 0.0, "bottom-right empty rows O")
    assert np.all(lse[:, :, : nq - nk] == -math.inf), "bottom-right empty rows LSE"


def pin_masks_torch_sdpa(orc):
    """torch's float64 CPU scaled_dot_product_attention with an explicit
    boolean mask (an independent library routine) on every row that has an
    allowed key, for padding and both causal alignments."""
    for (nq, nk, causal, kv_lens, seed) in [(9, 14, 2, [14, 10], 70), (12, 6, 2, [6, 4], 71),
                                            (8, 13, 1, [5, 13], 72), (10, 10, 0, [3, 10], 73)]:
        q = _rand((2, 2, nq, 8), seed) * 2.0
        k = _rand((2, 2, nk, 8), seed + 1) * 2.0
        v = _rand((2, 2, nk, 8), seed + 2)
        o, lse = orc.attention(q, k, v, 0.3, causal, kv_lens=kv_lens)
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        for b in range(2):
            L = kv_lens[b]
            mask = (j < L) & torch.ones(nq, nk, dtype=torch.bool)
            if causal == 1:
                mask = mask & (j <= i)
            elif causal == 2:
                mask = mask & (j <= i + (L - nq))
            rows = mask.any(dim=1)
            tq, tk, tv = (torch.from_numpy(x[b]) for x in (q, k, v))
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3)
            s = (0.3 * (tq @ tk.transpose(-1, -2))).masked_fill(~mask, -math.inf)
            tag = f"sdpa mask nq={nq} nk={nk} causal={causal} len={L}"
            _close(o[b][:, rows.numpy()], ref.numpy()[:, rows.numpy()], 1e-12, tag)
            _close(lse[b][:, rows.numpy()], torch.logsumexp(s, dim=-1).numpy()[:, rows.numpy()], 1e-12, tag)


def pin_online_blocked_masks(orc):
    """The block-wise online recurrence reaches the two-pass result under
    padding and bottom-right masks, empty rows included."""
    for (nq, nk, causal, L) in [(7, 10, 2, 10), (12, 6, 2, 4), (6, 9, 1, 0), (5, 9, 0, 6)]:
        q = _rand((nq, 5), 80 + nq) * 3.0
        k = _rand((nk, 5), 81 + nk) * 3.0
        v = _rand((nk, 5), 82 + nq)
        o_ref, l_ref = orc.attention(q[None, None], k[None, None], v[None, None], 0.45, causal, kv_lens=[L])
        for block in (1, 3, 4, nk + 2):
            o, l = orc.online_blocked(q, k, v, 0.45, causal, block, kv_len=L)
            _close(o, o_ref[0, 0], 1e-12, f"blocked masked O block={block}")
            assert np.array_equal(np.isinf(l), np.isinf(l_ref[0, 0])), "blocked masked empty rows"
            fin = np.isfinite(l)
            _close(l[fin], l_ref[0, 0][fin], 1e-12, f"blocked masked LSE block={block}")


def pin_decode_padding(orc):
    """Decode over a padded cache = the chunked merge over the real keys only;
    a cache with no real key gives (0, -inf)."""
    nk = 40
    q = _rand((2, 1, 1, 6), 90) * 2.0
    k = _rand((2, 1, nk, 6), 91) * 2.0
    v = _rand((2, 1, nk, 6), 92)
    o, lse = orc.decode(q, k, v, 0.4, kv_lens=[23, 0])
    for splits in (1, 4, 64):
        parts = orc.split_states(q[0, 0, 0], k[0, 0, :23], v[0, 0, :23], 0.4, splits)
        o_c, l_c = orc.combine(parts)
        _close(o[0, 0, 0], o_c, 1e-13, f"padded decode S={splits}")
        _close(lse[0, 0, 0], l_c, 1e-13, f"padded decode LSE S={splits}")
    o_e, l_e = orc.combine([(-math.inf, 0.0, np.zeros(6))] * 3)
    _close(o_e, np.zeros(6), 0.0, "all-empty combine O")
    assert l_e == -math.inf
    _close(o[1, 0, 0], np.zeros(6), 0.0, "decode with no real key O")
    assert lse[1, 0, 0] == -math.inf


def pin_backward_masks(orc):
    """Backward under padding and bottom-right masks: central differences of
    the forward oracle, torch fp64 autograd with an explicit mask (rows with
    keys only: torch's gradient through an empty row is NaN), padded keys
    get dK = dV = 0 and empty rows dQ = 0."""
    h = 1e-6
    for (nq, nk, causal, L, seed) in [(5, 4, 2, 4, 93), (3, 6, 2, 5, 94), (4, 5, 1, 3, 95)]:
        q = _rand((1, 1, nq, 2), seed) * 1.5
        k = _rand((1, 1, nk, 2), seed + 1) * 1.5
        v = _rand((1, 1, nk, 2), seed + 2)
        g = _rand((1, 1, nq, 2), seed + 3)
        dq, dk, dv = orc.attention_backward(q, k, v, g, 0.6, causal, kv_lens=[L])

        def loss(qq, kk, vv):
            return float(np.sum(orc.attention(qq, kk, vv, 0.6, causal, kv_lens=[L])[0] * g))

        for pos, (name, grad) in enumerate((("Q", dq), ("K", dk), ("V", dv))):
            x = (q, k, v)[pos]
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                args_p, args_m = [q, k, v], [q, k, v]
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p[pos], args_m[pos] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(grad, num, 1e-7, f"masked finite differences d{name} nq={nq} nk={nk} causal={causal}")
        _close(dk[:, :, L:], np.zeros_like(dk[:, :, L:]), 0.0, "padded keys dK")
        _close(dv[:, :, L:], np.zeros_like(dv[:, :, L:]), 0.0, "padded keys dV")
    nq, nk, L = 9, 7, 5
    q = _rand((1, 2, nq, 4), 96) * 2.0
    k = _rand((1, 2, nk, 4), 97) * 2.0
    v = _rand((1, 2, nk, 4), 98)
    g = _rand((1, 2, nq, 4), 99)
    dq, dk, dv = orc.attention_backward(q, k, v, g, 0.5, 2, kv_lens=[L])
    i = torch.arange(nq)[:, None]
    j = torch.arange(nk)[None, :]
    mask = (j < L) & (j <= i + (L - nq))
    rows = mask.any(dim=1)
    assert not rows[: nq - L].any() and rows[nq - L:].all()
    _close(dq[0, :, : nq - L], np.zeros((2, nq - L, 4)), 0.0, "empty rows dQ")
    tq, tk, tv = (torch.from_numpy(x[0]).requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[:, rows], tk, tv, attn_mask=mask[rows], scale=0.5)
    out.backward(torch.from_numpy(g[0][:, rows.numpy()]))
    _close(dq[0][:, rows.numpy()], tq.grad.numpy()[:, rows.numpy()], 1e-12, "masked autograd dQ")
    _close(dk[0], tk.grad.numpy(), 1e-12, "masked autograd dK")
    _close(dv[0], tv.grad.numpy(), 1e-12, "masked autograd dV")


# ---- rotary position embeddings ----------------------------------------------

def _angles(pos, half, base=100.0):
    return np.outer(pos, base ** (-np.arange(half) / half))


def pin_rope_closed_forms(orc):
    """Zero angle is the identity; a quarter turn maps the halves (a, b) to
    (-b, a) (pairs: (x0, x1) to (-x1, x0)); every rotated pair keeps its
    length; rotating by alpha then beta is rotating by alpha + beta; the pairs
    form is the half form under the interleaving permutation."""
    x = _rand((5, 8), 100)
    one, zero = np.ones((5, 4)), np.zeros((5, 4))
    _close(orc.rope(x, one, zero), x, 0.0, "rope identity")
    _close(orc.rope_pairs(x, one, zero), x, 0.0, "rope_pairs identity")
    _close(orc.rope(x, zero, one), np.concatenate([-x[:, 4:], x[:, :4]], axis=1), 0.0, "rope quarter turn")
    quarter = np.empty_like(x)
    quarter[:, 0::2], quarter[:, 1::2] = -x[:, 1::2], x[:, 0::2]
    _close(orc.rope_pairs(x, zero, one), quarter, 0.0, "rope_pairs quarter turn")
    th1, th2 = _rand((5, 4), 101), _rand((5, 4), 102)
    y = orc.rope(x, np.cos(th1), np.sin(th1))
    _close(np.hypot(y[:, :4], y[:, 4:]), np.hypot(x[:, :4], x[:, 4:]), 1e-14, "rope keeps pair lengths")
    _close(orc.rope(y, np.cos(th2), np.sin(th2)), orc.rope(x, np.cos(th1 + th2), np.sin(th1 + th2)), 1e-14,
           "rope angles add")
    perm = np.concatenate([np.arange(0, 8, 2), np.arange(1, 8, 2)])   # pairs layout -> halves layout
    z = orc.rope_pairs(x, np.cos(th1), np.sin(th1))
    _close(z[:, perm], orc.rope(x[:, perm], np.cos(th1), np.sin(th1)), 1e-15, "pairs = half under interleaving")


def pin_rope_relative_position(orc):
    """With angles proportional to position, the score of a rotated query at
    position m and key at n depends only on m - n: shifting every position by
    the same amount leaves attention_rope unchanged (non-causal and top-left;
    both styles)."""
    nq, nk, d = 6, 9, 8
    q = _rand((1, 2, nq, d), 103)
    k = _rand((1, 2, nk, d), 104)
    v = _rand((1, 2, nk, d), 105)
    n_pos = 40
    ang = _angles(np.arange(n_pos), d // 2)
    cos, sin = np.cos(ang), np.sin(ang)
    shift = 17
    for style in (orc.ROPE_HALF, orc.ROPE_PAIRS):
        for causal in (0, 1):
            o, lse = orc.attention_rope(q, k, v, cos, sin, 0.4, causal, style=style)
            o2, lse2 = orc.attention_rope(q, k, v, cos[shift:], sin[shift:], 0.4, causal, style=style)
            _close(o, o2, 1e-12, f"rope shift invariance O style={style} causal={causal}")
            _close(lse, lse2, 1e-12, f"rope shift invariance LSE style={style} causal={causal}")
            o0, _ = orc.attention(q, k, v, 0.4, causal)
            assert np.abs(o - o0).max() > 1e-3, "rotation must change the result"
    # bottom-right: the queries are the newest tokens, so they take positions Nk - Nq + i
    o_br, _ = orc.attention_rope(q, k, v, cos, sin, 0.4, 2)
    qr = np.stack([orc.rope(q[0, hh], cos[nk - nq: nk], sin[nk - nq: nk]) for hh in range(2)])[None]
    kr = np.stack([orc.rope(k[0, hh], cos[:nk], sin[:nk]) for hh in range(2)])[None]
    o_ref, _ = orc.attention(qr, kr, v, 0.4, 2)
    _close(o_br, o_ref, 1e-13, "rope bottom-right positions")


ALL_PINS = [
    pin_worked_example_trace,
    pin_worked_example_two_pass,
    pin_merge_example,
    pin_single_key,
    pin_zero_keys_means,
    pin_zero_scale_rectangular,
    pin_weights_sum_to_one,
    pin_ones_values,
    pin_permutation,
    pin_causal_edges,
    pin_torch_sdpa,
    pin_online_blocked_matches,
    pin_online_per_key_matches,
    pin_split_combine,
    pin_backward_finite_differences,
    pin_backward_torch_autograd,
    pin_backward_closed_forms,
    pin_mask_closed_forms,
    pin_padding_is_truncation,
    pin_bottom_right_is_suffix,
    pin_masks_torch_sdpa,
    pin_online_blocked_masks,
    pin_decode_padding,
    pin_backward_masks,
    pin_rope_closed_forms,
    pin_rope_relative_position,
    pin_nan_stays_in_its_rows,
]
