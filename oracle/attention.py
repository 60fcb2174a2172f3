"""fp64 CPU oracle for the FlashAttention forward pass and its split-KV decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests under ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library and imports nothing from it.

Every function here is plain numpy in float64. Inputs are widened exactly from
whatever the GPU consumed (bf16 or fp32 values are representable in fp64).

Sources (the web pages the method is defined on):

* "11. Fusion, recompute, and flash attention" (ML compiler from scratch),
  section 11.2 (S = QK^T/sqrt(D), P = softmax(S) row-wise, O = PV), section 11.6
  (online softmax per key and the merge of two partial states), section 11.9
  (log-sum-exp m + log l saved per row), Pitfalls (fully masked rows),
  Exercise "Causal mask" (query i attends keys j <= i), Exercise
  "Flash-decoding" (split keys into chunks, merge partials in a second step),
  Solutions to exercise 3 (the merge worked with numbers).
* iThome article on FlashAttention (ithelp.ithome.com.tw/articles/10405336),
  sections on standard attention, stable softmax and "the three states"
  (m, l, O with alpha = exp(m - m_new), final O / l).
* "Kernel visualization: Flash Attention 2", section "Write the data back to
  HBM" (L = m + log l written beside O).
* phobos attention stdlib page, "Rotary position embeddings": ``rope``
  (rotate-half form: halves a, b of a row become a cos - b sin, b cos + a sin)
  and ``rope_pairs`` (adjacent pairs 2i, 2i + 1 rotated the same way); cos and
  sin are [R, D / 2], the angles of each row's position.
* phobos attention stdlib page, ``attention`` (mask of the ragged last key
  block) and ``Causal attention``.

What pins each function (tests/test_oracle.py):

* ``attention``: closed forms (Nk = 1; K = 0 gives prefix means with
  LSE = ln(count)), invariants (weights sum to one, V = 1 gives O = 1, joint
  K/V row permutation, causal row 0 = V[0], causal last row = full last row),
  torch's float64 CPU ``scaled_dot_product_attention`` and ``logsumexp`` as an
  independent library routine, and agreement with ``online_blocked``.
* ``online_per_key``: the worked example of section 11.6 (state after every key
  and o/l = 21.546979), checked against tests/golden/worked_example.json.
* ``online_blocked``: agreement with ``attention`` on tiny inputs for block
  sizes that do and do not divide Nk; the late-maximum case of the exercise
  "Find the bug".
* ``merge`` / ``split_states`` / ``combine``: the numbers of the solution to
  exercise 3 (tests/golden/merge_example.json); every chunking of a row gives
  the two-pass answer.
* ``rope`` / ``rope_pairs`` / ``attention_rope``: closed forms (zero angle is
  the identity, a quarter turn maps (a, b) to (-b, a)), every pair keeps its
  length, two rotations add their angles, the pairs form is the half form
  under the interleaving permutation, and the score of a rotated query and
  key depends only on the difference of their positions (shifting every
  position leaves ``attention_rope`` unchanged).
* ``attention_backward``: central finite differences of ``attention`` on tiny
  inputs; torch's float64 CPU autograd through ``scaled_dot_product_attention``
  as an independent library routine; closed forms (dO = 0 gives zero
  gradients; equal V rows make O independent of Q and K, so dQ = dK = 0; the
  rows of dK sum to zero and those of dV to the column sums of dO; the causal
  row 0 sees one key, so its dQ is zero).
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


CAUSAL_NONE, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT = 0, 1, 2


def allowed_keys(i: int, nk: int, causal, nq: int | None = None, kv_len: int | None = None) -> np.ndarray:
    """Boolean mask of the keys query row ``i`` may attend.

    Keys are 0..nk-1, of which the first ``kv_len`` (default all) are real and
    the rest padding, never attended (the padding masks of the Pitfalls
    passage). ``causal``:

    * False / 0: every real key;
    * True / 1, top-left: keys j <= i, counted from the first key (the
      exercise "Causal mask" defines it on square inputs; the same absolute
      rule is kept when Nq != Nk);
    * 2, bottom-right: the last of the ``nq`` query rows is aligned with the
      last real key, j <= i + (kv_len - nq). This is the reading for Nq != Nk
      in which the queries are the newest tokens of the sequence; it equals
      top-left when kv_len == nq, and rows i < nq - kv_len see no key at all.

    A row may end up with no allowed key (padding, bottom-right): see
    ``attention_rows`` for its value.
    """
    j = np.arange(nk)
    real = j < (nk if kv_len is None else kv_len)
    mode = int(causal)
    if mode == CAUSAL_TOP_LEFT:
        return real & causal_top_left(i, j)
    if mode == CAUSAL_BOTTOM_RIGHT:
        off = (nk if kv_len is None else kv_len) - nq
        return real & (j <= i + off)
    return real


def causal_top_left(i, j):
    return j <= i


def attention_rows(q_rows, row_index, k, v, scale: float, causal, nq: int | None = None,
                   kv_len: int | None = None):
    """Two-pass attention for selected query rows of one (batch, head).

    q_rows: [R, D] queries; row_index: [R] their absolute row numbers (used by
    the causal mask); k, v: [Nk, D]; nq: the number of query rows of the head
    (bottom-right alignment); kv_len: real keys (default Nk). Returns
    (O [R, D], LSE [R]).

    Follows section 11.2 and the stable softmax of the iThome article: the
    score row s = scale * q . k_j is materialised, m = max over the allowed
    keys, p = exp(s - m), l = sum p, O = (sum_j p_j v_j) / l. LSE = m + ln l
    on the scaled scores, as the write-back step of the FA2 visualization
    stores it.

    A row with no allowed key (the fully masked row of the Pitfalls passage)
    has no softmax; it gets the values of the empty sums the definition
    reduces to: O = 0 (no value vector is weighted) and LSE = ln 0 = -inf.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    nk = k.shape[0]
    s = scale * (q_rows @ k.T)                       # [R, Nk]
    mask = np.stack([allowed_keys(int(i), nk, causal, nq, kv_len) for i in row_index]).reshape(s.shape)
    empty = ~mask.any(axis=1)
    s = np.where(mask, s, NEG_INF)
    m = s.max(axis=1, keepdims=True)
    m[empty] = 0.0                                    # no key: keep exp(-inf - 0) = 0
    p = np.exp(s - m)                                 # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1, keepdims=True)
    l_div = np.where(empty[:, None], 1.0, l)
    o = (p @ v) / l_div
    with np.errstate(divide="ignore"):
        lse = m[:, 0] + np.log(l[:, 0])               # ln 0 = -inf on empty rows
    return o, lse


def attention(q, k, v, scale: float, causal=False, kv_lens=None):
    """softmax(Q K^T * scale) V over tensors laid out [B, H, N, D].

    q: [B, H, Nq, D]; k, v: [B, H, Nk, D]; kv_lens: optional [B] real key
    counts (keys past them are padding). Returns O [B, H, Nq, D] and
    LSE [B, H, Nq] in float64. This is the definition the method reaches
    exactly (the iThome article calls FlashAttention exact attention): every
    row is computed in two passes by ``attention_rows``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, h, nq, d = q.shape
    o = np.empty((b, h, nq, v.shape[-1]))
    lse = np.empty((b, h, nq))
    rows = np.arange(nq)
    for bi in range(b):
        kv_len = None if kv_lens is None else int(kv_lens[bi])
        for hi in range(h):
            o[bi, hi], lse[bi, hi] = attention_rows(q[bi, hi], rows, k[bi, hi], v[bi, hi], scale, causal,
                                                    nq, kv_len)
    return o, lse


def softmax_weights(q, k, scale: float, causal=False, kv_len: int | None = None):
    """The probability matrix P = softmax(scale * Q K^T) of one (batch, head).

    q: [Nq, D], k: [Nk, D] -> P [Nq, Nk]; masked entries are exactly 0, and
    so is every entry of a row with no allowed key. Exposed so tests can check
    that every (non-empty) row sums to one.
    """
    q, k = _f64(q), _f64(k)
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    mask = np.stack([allowed_keys(i, nk, causal, nq, kv_len) for i in range(nq)]).reshape(s.shape)
    empty = ~mask.any(axis=1)
    s = np.where(mask, s, NEG_INF)
    m = s.max(axis=1, keepdims=True)
    m[empty] = 0.0
    p = np.exp(s - m)
    return p / np.where(empty[:, None], 1.0, p.sum(axis=1, keepdims=True))


# --------------------------------------------------------------------------
# Online softmax: the recurrence the kernels implement, kept here only so the
# tests can check it against the two-pass definition above.
# --------------------------------------------------------------------------

def online_per_key(s, v, trace: bool = False):
    """Online softmax over one score row, one key at a time (section 11.6).

    s: [N] scaled scores; v: [N, Dv] (or [N] for a scalar value). Key j on its
    own is the partial state (s_j, 1, v_j): its maximum is its score, its sum
    e^0 = 1 and its output v_j (a masked score, -inf, is the empty state
    (-inf, 0, 0)). The row's state is these single-key states folded left to
    right with ``merge``, starting from the empty state. Each fold rescales
    the running (l, o) by corr = e^{m - m'} and weighs the new key by
    p = e^{s_j - m'}, m' = max(m, s_j): the per-key recurrence of the section.
    Returns (m, l, o) and, with ``trace``, the list of per-key states
    (m, corr, p, l, o). The answer is o / l.
    """
    s = _f64(s)
    v = _f64(v)
    empty = (NEG_INF, 0.0, np.zeros(v.shape[1:]))
    state = empty
    states = []
    for j in range(s.shape[0]):
        key_state = empty if s[j] == NEG_INF else (float(s[j]), 1.0, v[j])
        _, corr, p = _rescale_weights(state[0], key_state[0])
        state = merge(state, key_state)
        if trace:
            states.append((state[0], corr, p, state[1], np.array(state[2])))
    if trace:
        return state, states
    return state


def online_blocked(q, k, v, scale: float, causal, block: int, kv_len: int | None = None):
    """Block-wise online softmax over keys (the FA2 form of the iThome article).

    For each query row of one (batch, head) and each block of ``block`` keys:
    S_blk = scale * q K_blk^T with masked keys at -inf, m_new = max(m, max S_blk),
    alpha = exp(m - m_new), P = exp(S_blk - m_new), l = alpha l + sum P,
    O = alpha O + P V_blk, m = m_new; after the last block O / l and
    LSE = m + ln l. A block may hold fewer than ``block`` keys at the end
    (the masked last block of the phobos ``attention``). A row that never sees
    an allowed key ends with l = 0 and gets O = 0, LSE = -inf. Plain loops:
    tiny inputs only.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, nk = q.shape[0], k.shape[0]
    out = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        ok = allowed_keys(i, nk, causal, nq, kv_len)
        m, l = NEG_INF, 0.0
        acc = np.zeros(v.shape[1])
        for j0 in range(0, nk, block):
            j1 = min(nk, j0 + block)
            s = scale * (k[j0:j1] @ q[i])
            s = np.where(ok[j0:j1], s, NEG_INF)
            m_new = max(m, float(s.max()))
            if m_new == NEG_INF:          # nothing allowed yet: state stays empty
                continue
            alpha = math.exp(m - m_new)
            p = np.exp(s - m_new)
            l = alpha * l + p.sum()
            acc = alpha * acc + p @ v[j0:j1]
            m = m_new
        if l == 0.0:                      # no allowed key (see attention_rows)
            out[i], lse[i] = 0.0, NEG_INF
            continue
        out[i] = acc / l
        lse[i] = m + math.log(l)
    return out, lse


def _rescale_weights(m1: float, m2: float):
    """The common base m = max(m1, m2) of two partial states and the factors
    e^{m1 - m}, e^{m2 - m} that bring each state onto it. An empty side
    (m_i = -inf) gets factor 0; when both sides are empty the base stays -inf
    and the factors are 1 and 0 (nothing to rescale, nothing to add)."""
    m = max(m1, m2)
    if m == NEG_INF:
        return m, 1.0, 0.0
    return m, math.exp(m1 - m), math.exp(m2 - m)


def merge(a, b):
    """Merge two partial states (m, l, o) into the state of the union of their keys.

    With m = max(m1, m2): l = l1 e^{m1-m} + l2 e^{m2-m}, o = o1 e^{m1-m} + o2 e^{m2-m}
    (section 11.6, proved in the solution to exercise 3). An empty state
    (-inf, 0, 0) is the identity.
    """
    m1, l1, o1 = a
    m2, l2, o2 = b
    m, w1, w2 = _rescale_weights(m1, m2)
    if m == NEG_INF:
        return (NEG_INF, 0.0, np.zeros_like(_f64(o1)))
    return (m, l1 * w1 + l2 * w2, _f64(o1) * w1 + _f64(o2) * w2)


def chunk_bounds(nk: int, num_splits: int):
    """Key ranges of the split-KV decode: chunk c = ceil(nk / num_splits) keys,
    chunk s covers [s*c, min(nk, (s+1)*c)); trailing chunks may be empty."""
    c = -(-nk // num_splits)
    return [(min(nk, s * c), min(nk, (s + 1) * c)) for s in range(num_splits)]


def split_states(q_row, k, v, scale: float, num_splits: int):
    """Partial (m, l, o) of one query row over each key chunk (exercise
    "Flash-decoding"): each chunk is reduced in two passes on its own keys.
    Empty chunks give (-inf, 0, 0)."""
    q_row, k, v = _f64(q_row), _f64(k), _f64(v)
    parts = []
    for j0, j1 in chunk_bounds(k.shape[0], num_splits):
        if j1 <= j0:
            parts.append((NEG_INF, 0.0, np.zeros(v.shape[1])))
            continue
        s = scale * (k[j0:j1] @ q_row)
        m = float(s.max())
        p = np.exp(s - m)
        parts.append((m, float(p.sum()), p @ v[j0:j1]))
    return parts


def combine(parts):
    """Fold a list of partial states with ``merge`` and finish: (o / l, m + ln l),
    or (0, -inf) when no chunk held a key."""
    state = (NEG_INF, 0.0, np.zeros_like(_f64(parts[0][2])))
    for p in parts:
        state = merge(state, p)
    m, l, o = state
    if l == 0.0:                          # every chunk empty: no key at all
        return np.zeros_like(o), NEG_INF
    return o / l, m + math.log(l)


def decode(q, k, v, scale: float, kv_lens=None):
    """Single-token decode: q [B, H, 1, D] over the cache k, v [B, H, Nk, D],
    of which the first kv_lens[b] keys (default all) are real. No causal mask.
    The same definition as ``attention`` with Nq = 1; returns O [B, H, 1, D]
    and LSE [B, H, 1]."""
    return attention(q, k, v, scale, causal=False, kv_lens=kv_lens)


# --------------------------------------------------------------------------
# Rotary position embeddings (phobos page, "Rotary position embeddings").
# --------------------------------------------------------------------------

def rope(x, cos, sin):
    """Rotate-half RoPE of the rows of x [R, D]: with a = x[:, :D/2] and
    b = x[:, D/2:], the row becomes [a cos - b sin, b cos + a sin]; cos and
    sin are [R, D/2]. Both halves are read before either is written."""
    x, cos, sin = _f64(x), _f64(cos), _f64(sin)
    half = x.shape[1] // 2
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=1)


def rope_pairs(x, cos, sin):
    """Adjacent-pair RoPE (GPT-J form): elements x0 = x[:, 2i] and
    x1 = x[:, 2i + 1] become x0 cos - x1 sin and x1 cos + x0 sin; cos and sin
    are [R, D/2]."""
    x, cos, sin = _f64(x), _f64(cos), _f64(sin)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = x0 * cos - x1 * sin
    out[:, 1::2] = x1 * cos + x0 * sin
    return out


ROPE_HALF, ROPE_PAIRS = 0, 1


def rope_qk(q, k, cos, sin, causal=False, kv_lens=None, style: int = ROPE_HALF):
    """rope(Q) and rope(K) of [B, H, N, D] tensors with the positions of
    ``attention_rope``: key j at position j; query row i at position i, or
    i + (Lk - Nq) under bottom-right causal alignment (the queries are then the
    newest tokens), clamped at 0 (such rows see no key)."""
    q, k = _f64(q), _f64(k)
    cos, sin = _f64(cos), _f64(sin)
    b, h, nq, d = q.shape
    nk = k.shape[2]
    rot = rope if style == ROPE_HALF else rope_pairs
    qr = np.empty_like(q)
    kr = np.empty_like(k)
    for bi in range(b):
        L = nk if kv_lens is None else int(kv_lens[bi])
        qpos = np.arange(nq) + (L - nq if int(causal) == CAUSAL_BOTTOM_RIGHT else 0)
        qpos = np.maximum(qpos, 0)
        kpos = np.arange(nk)
        for hi in range(h):
            qr[bi, hi] = rot(q[bi, hi], cos[qpos], sin[qpos])
            kr[bi, hi] = rot(k[bi, hi], cos[kpos], sin[kpos])
    return qr, kr


def attention_rope(q, k, v, cos, sin, scale: float, causal=False, kv_lens=None, style: int = ROPE_HALF):
    """Attention of rotated queries and keys: softmax(rope(Q) rope(K)^T scale) V.

    cos, sin: [P, D/2] tables indexed by position; positions as ``rope_qk``.
    Returns (O, LSE) as ``attention``.
    """
    qr, kr = rope_qk(q, k, cos, sin, causal, kv_lens, style)
    return attention(qr, kr, v, scale, causal, kv_lens)


# --------------------------------------------------------------------------
# Backward pass (the exercise "Backward with recompute" of section 11: dQ, dK,
# dV from O, dO and the saved log-sum-exp).
# --------------------------------------------------------------------------

def attention_backward_head(q, k, v, do, scale: float, causal=False, kv_len: int | None = None):
    """Gradients of O = softmax(scale * Q K^T) V for one (batch, head).

    q: [Nq, D], k, v: [Nk, D], do: [Nq, D] (the gradient of the loss with
    respect to O). Returns (dQ, dK, dV) in float64.

    The chain rule written out on the definition, the way the exercise asks
    for it to be checked (against the gradient of the unfused graph):
        P  = softmax(S),  S = scale * Q K^T (masked keys get P = 0)
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))      (softmax Jacobian, row by row)
        dQ = scale * dS K,   dK = scale * dS^T Q
    rowsum(P * dP) equals rowsum(dO * O) because O = P V; the kernels use the
    second form, this definition the first. A row with no allowed key has
    P = 0 (its O = 0 does not depend on Q, K or V), so it adds nothing.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p = softmax_weights(q, k, scale, causal, kv_len)  # [Nq, Nk]
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, scale: float, causal=False, kv_lens=None):
    """``attention_backward_head`` over [B, H, N, D] tensors; returns
    (dQ, dK, dV) in float64 with the shapes of q, k, v."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for bi in range(q.shape[0]):
        kv_len = None if kv_lens is None else int(kv_lens[bi])
        for hi in range(q.shape[1]):
            dq[bi, hi], dk[bi, hi], dv[bi, hi] = attention_backward_head(
                q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], scale, causal, kv_len)
    return dq, dk, dv
