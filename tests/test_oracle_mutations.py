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

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle")
SRC = os.path.join(ORACLE_DIR, "paged_attention.py")
SRC_FP8 = os.path.join(ORACLE_DIR, "fp8_kv.py")

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


# planted mistakes in the FP8 module (oracle/fp8_kv.py)
FP8_MUTATIONS = {
    "e4m3_bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "e4m3_subnormal_scale": ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    "e4m3_no_nan_code": ("mag = np.where((e == 15) & (m == 7), np.nan, mag)", "pass"),
    "e4m3_ties_up": ("np.where(lo % 2 == 0, lo, hi)", "hi"),
    "e4m3_ties_down": ("np.where(lo % 2 == 0, lo, hi)", "lo"),
    "e4m3_sign_dropped": ("code = code | np.where(np.signbit(x), 0x80, 0)", "code = code"),
    "e4m3_nan_to_zero": ("code = np.where(np.isnan(x), 0x7F, code)", "code = code"),
    "quantize_multiplies": ("x32 / np.float32(scale)", "x32 * np.float32(scale)"),
    "quantize_fp64_quotient": ("x32 / np.float32(scale)",
                               "np.asarray(x, np.float64) / float(scale)"),
    "store_scales_swapped": ("ks, vs = (np.float32(s) for s in", "vs, ks = (np.float32(s) for s in"),
    "store_layer0_scales": ("np.asarray(kv_scales, np.float32)[layer])",
                            "np.asarray(kv_scales, np.float32)[0])"),
    "store_negative_loc_fp8": ("        if loc[t] >= 0:\n            k_out[layer, loc[t]] = quantize",
                               "        if True:\n            k_out[layer, loc[t]] = quantize"),
    "decode_fp8_ignores_v_scale": ("vp = dequantize(np.asarray(v_codes)[layer:layer + 1], vs)",
                                   "vp = dequantize(np.asarray(v_codes)[layer:layer + 1], 1.0)"),
    "decode_fp8_k_scale_for_v": ("kp = dequantize(np.asarray(k_codes)[layer:layer + 1], ks)",
                                 "kp = dequantize(np.asarray(k_codes)[layer:layer + 1], vs)"),
    "prefill_fp8_ignores_v_scale": ("vp = dequantize(np.asarray(v_codes)[layer:layer + 1], vs)\n    return prefill_attention",
                                    "vp = dequantize(np.asarray(v_codes)[layer:layer + 1], 1.0)\n    return prefill_attention"),
    "prefill_fp8_not_causal": ("scale, causal=causal)", "scale, causal=False)"),
    "rope_fp32_sin_sign": ("out[t, :, a] = ac - bs", "out[t, :, a] = ac + bs"),
    "rope_fp32_reads_rotated": ("out[t, :, b] = bc + as_", "out[t, :, b] = bc + out[t, :, a] * s"),
    "rope_fp8_store_unrotated": ("kc, vc = kv_store_fp8(k_codes, v_codes, layer, k_rot,",
                                 "kc, vc = kv_store_fp8(k_codes, v_codes, layer, k_new,"),
    "decode_fp8_layer0": ("kp = dequantize(np.asarray(k_codes)[layer:layer + 1], ks)",
                          "kp = dequantize(np.asarray(k_codes)[0:1], ks)"),
}


def mutated_oracle(old, new, target=None):
    """The oracle's two modules executed into one namespace, with `old`
    replaced by `new` in the target module's source."""
    target = target or SRC
    texts = {}
    for path in (SRC, SRC_FP8):
        with open(path) as f:
            texts[path] = f.read()
    assert texts[target].count(old) >= 1, f"mutation anchor not found: {old!r}"
    texts[target] = texts[target].replace(old, new)
    # the FP8 module's relative import resolves to the (possibly mutated) namespace
    texts[SRC_FP8] = "\n".join(l for l in texts[SRC_FP8].split("\n")
                               if not l.startswith("from .paged_attention import"))
    mod = types.ModuleType("oracle_mutant")
    exec(compile(texts[SRC], "oracle_mutant", "exec"), mod.__dict__)
    exec(compile(texts[SRC_FP8], "oracle_mutant_fp8", "exec"), mod.__dict__)
    return mod


CASES = {**{k: (o, n, SRC) for k, (o, n) in MUTATIONS.items()},
         **{k: (o, n, SRC_FP8) for k, (o, n) in FP8_MUTATIONS.items()}}


def test_unmutated_namespace_passes_every_pin():
    mod = mutated_oracle("", "")
    for pin in P.ALL_PINS:
        pin(mod)


@pytest.mark.parametrize("name", sorted(CASES))
def test_mutation_is_caught(name):
    old, new, target = CASES[name]
    mutant = mutated_oracle(old, new, target)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # AssertionError, or the mutant crashing
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutation {name}"
