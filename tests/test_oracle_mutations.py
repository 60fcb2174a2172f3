"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them."""

import os
import types

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTATIONS = {
    "causal_off_by_one": ("return j <= i", "return j < i"),
    "dropped_scale": ("s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T)"),
    "lse_without_max": ("lse = m[:, 0] + np.log(l[:, 0])", "lse = np.log(l[:, 0])"),
    "lse_base_two": ("lse = m[:, 0] + np.log(l[:, 0])", "lse = m[:, 0] + np.log2(l[:, 0])"),
    "no_final_divide": ("o = (p @ v) / l_div", "o = (p @ v)"),
    "wrong_operand": ("o = (p @ v) / l_div", "o = (p @ k) / l_div"),
    "bottom_right_off_by_one": ("return real & (j <= i + off)", "return real & (j < i + off)"),
    "bottom_right_wrong_length": ("off = (nk if kv_len is None else kv_len) - nq", "off = nk - nq"),
    "padding_includes_boundary": ("real = j < (nk if kv_len is None else kv_len)",
                                  "real = j <= (nk if kv_len is None else kv_len)"),
    "padding_ignored_in_backward": ("p = softmax_weights(q, k, scale, causal, kv_len)",
                                    "p = softmax_weights(q, k, scale, causal)"),
    "empty_row_lse_zero": ("lse = m[:, 0] + np.log(l[:, 0])               # ln 0",
                           "lse = m[:, 0] + np.log(np.maximum(l[:, 0], 1.0))  # ln 0"),
    "empty_combine_nan": ("    if l == 0.0:                          # every chunk empty: no key at all",
                          "    if False:"),
    "unshifted_exp": ("p = np.exp(s - m)                                 #", "p = np.exp(s)                                     #"),
    "per_key_state_sum_zero": ("(float(s[j]), 1.0, v[j])", "(float(s[j]), 0.0, v[j])"),
    "per_key_state_wrong_value": ("(float(s[j]), 1.0, v[j])", "(float(s[j]), 1.0, v[0])"),
    "rescale_keeps_old_base": ("return m, math.exp(m1 - m), math.exp(m2 - m)", "return m, 1.0, math.exp(m2 - m)"),
    "blocked_forgot_rescale": ("acc = alpha * acc + p @ v[j0:j1]", "acc = acc + p @ v[j0:j1]"),
    "blocked_alpha_sign": ("alpha = math.exp(m - m_new)", "alpha = math.exp(m_new - m)"),
    "merge_weight_sign": ("return m, math.exp(m1 - m), math.exp(m2 - m)",
                          "return m, math.exp(m - m1), math.exp(m2 - m)"),
    "merge_drops_second_o": ("o1) * w1 + _f64(o2) * w2)", "o1) * w1)"),
    "chunk_floor": ("c = -(-nk // num_splits)", "c = max(1, nk // num_splits)"),
    "bwd_dv_untransposed": ("dv = p.T @ do", "dv = p @ do"),
    "bwd_dp_wrong_operand": ("dp = do @ v.T", "dp = do @ k.T"),
    "bwd_softmax_jacobian_sign": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                                  "ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))"),
    "bwd_softmax_jacobian_dropped": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "rope_sign": ("return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=1)",
                  "return np.concatenate([a * cos + b * sin, b * cos - a * sin], axis=1)"),
    "rope_halves_swapped": ("a, b = x[:, :half], x[:, half:]", "b, a = x[:, :half], x[:, half:]"),
    "rope_pairs_wrong_partner": ("out[:, 1::2] = x1 * cos + x0 * sin", "out[:, 1::2] = x1 * cos + x1 * sin"),
    "rope_query_positions_top_left": ("qpos = np.arange(nq) + (L - nq if int(causal) == CAUSAL_BOTTOM_RIGHT else 0)",
                                      "qpos = np.arange(nq)"),
    "bwd_dq_no_scale": ("dq = scale * (ds @ k)", "dq = ds @ k"),
    "bwd_dk_wrong_operand": ("dk = scale * (ds.T @ q)", "dk = scale * (ds.T @ k)"),
}


def _mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
