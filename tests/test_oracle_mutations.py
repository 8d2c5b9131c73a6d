"""Planted mistakes in the oracle must fail at least one pin.

Each case rewrites one expression of ``oracle/paged_attention.py`` (a dropped
term, a wrong index or sign, a swapped operand), loads the result as a fresh
module on the CPU and runs every pin against it. A mutation that no pin
catches would mean the pins leave that part of the oracle unchecked.
"""

import os
import types

import pytest

from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "paged_attention.py")

MUTATIONS = {
    "gqa_modulo": ("K[:, h // g]", "K[:, h % Hkv]"),
    "gqa_modulo_prefill": ("K[:vis, h // g]", "K[:vis, h % Hkv]"),
    "drop_scale": ("x = scale * (Kh @ qh)", "x = (Kh @ qh)"),
    "drop_normaliser": ("return (p @ Vh) / p.sum()", "return (p @ Vh)"),
    "v_is_k": ("return (p @ Vh) / p.sum()", "return (p @ Kh) / p.sum()"),
    "causal_off_by_one": ("vis = P + i + 1 if causal else L", "vis = P + i if causal else L"),
    "causal_top_left": ("vis = P + i + 1 if causal else L", "vis = i + 1 if causal else L"),
    "indptr_inclusive": ("out[1:] = np.cumsum(s)", "out[:-1] = np.cumsum(s)"),
    "decode_loc_off_by_one": ("req_to_token[req_pool_indices[b], L - 1] if L > 0",
                              "req_to_token[req_pool_indices[b], L - 2] if L > 0"),
    "prefill_loc_no_prefix": ("req_to_token[req_pool_indices[b], P + i]",
                              "req_to_token[req_pool_indices[b], i]"),
    "merge_unweighted": ("num = (w[..., None] * o_parts).sum(axis=-2)",
                         "num = (o_parts).sum(axis=-2)"),
    "split_unaligned": ("chunk = _ceil_div(_ceil_div(L, req), SPLIT_ALIGN) * SPLIT_ALIGN",
                        "chunk = _ceil_div(L, req)"),
    "split_ignores_fixed": ("req = fixed_splits if fixed_splits > 0 else _ceil_div(L, split_tokens)",
                            "req = _ceil_div(L, split_tokens)"),
    "store_ignores_layer": ("k_out[layer, loc[t]] = k_new[t]", "k_out[:, loc[t]] = k_new[t]"),
    "store_negative_loc": ("if loc[t] >= 0:", "if True:"),
    "lse_drops_max": ("lse[h, s] = m + np.log(p.sum())", "lse[h, s] = np.log(p.sum())"),
    "padded_row_nonzero_loc": ("if L > 0 else -1", "if L > 0 else 0"),
    "rope_sin_sign": ("out[t, :, a] = x[t, :, a] * c - x[t, :, b] * s",
                      "out[t, :, a] = x[t, :, a] * c + x[t, :, b] * s"),
    "rope_reads_rotated_a": ("out[t, :, b] = x[t, :, b] * c + x[t, :, a] * s",
                             "out[t, :, b] = x[t, :, b] * c + out[t, :, a] * s"),
    "rope_pairs_swapped": ("return [(2 * i, 2 * i + 1) for i in range(half)]",
                           "return [(2 * i + 1, 2 * i) for i in range(half)]"),
    "rope_half_split_adjacent": ("return [(i, i + half) for i in range(half)]",
                                 "return [(2 * i, 2 * i + 1) for i in range(half)]"),
    "rope_cos_for_sin": ("s = float(freqs_cis[p, i, 1])", "s = float(freqs_cis[p, i, 0])"),
    "rope_position_ignored": ("p = int(positions[t])", "p = 0"),
    "rope_store_unrotated_k": ("layer,\n                      k_rot, np.asarray(v_new",
                               "layer,\n                      np.asarray(k_new, np.float64), np.asarray(v_new"),
    "rope_q_unrotated": ("q_rot = apply_rope(q, positions, freqs_cis, interleaved)",
                         "q_rot = np.asarray(q, np.float64)"),
}


def mutated_oracle(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    mutant = mutated_oracle(old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # AssertionError, or the mutant crashing
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutation {name}"
