"""fp64 oracle for the FP8 (E4M3) KV-cache variant.

TEST INFRASTRUCTURE ONLY (same rules as the package: the product path never
imports this module, and it shares nothing with the HIP library).

What the pages fix: only that the attention kernels come with an fp8 test
kernel (P4, bullet on renaming the fp8 MMA test file). The format and its use
below are readings, each listed in the design notes:
  R17 the K and V pools may hold one-byte E4M3 codes, the "E4M3" encoding of
      the OCP 8-bit floating point specification (OFP8): bit 7 sign, bits 6..3
      exponent with bias 7, bits 2..0 mantissa; exponent 0 holds the
      subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities; the
      largest finite magnitude is 1.75 * 2^8 = 448.
  R18 each layer has one fp32 scale for K and one for V (kv_scales[layer] =
      (k_scale, v_scale)); a code c in the K pool stands for e4m3(c) * k_scale.
  R19 storing an element x (the new token's K or V element, a bf16 value
      taken as fp32) writes the code of the fp32 quotient fl32(x / scale)
      rounded to the nearest E4M3 value, ties to the even code, with
      magnitudes beyond 448 saturated to 448; NaN gives a NaN code.
  R20 attention over an FP8 pool is the attention over the values the codes
      stand for: the decode definition applied to the dequantised pools.
  R21 the fused RoPE store into an FP8 pool decides each k code on the fp32
      rotation with every product and sum rounded once, in the order
      a' = fl(fl(a c) - fl(b s)), b' = fl(fl(b c) + fl(a s)); v is quantised
      unrotated; q is rotated as for the other pools.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import apply_rope, decode_attention, prefill_attention, rope_pairs

E4M3_MAX = 448.0  # R17: 0x7E = 2^8 * (1 + 6/8)


def e4m3_decode(codes):
    """Value of each E4M3 code, as float64 (R17, the OFP8 E4M3 definition)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """E4M3 code nearest to each value of x, ties to the even code, magnitudes
    beyond 448 saturated, NaN -> 0x7F; the sign (of zero too) goes to bit 7 (R19)."""
    x = np.asarray(x, dtype=np.float64)
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0..126: 0 .. 448, increasing
    a = np.minimum(np.abs(x), E4M3_MAX)
    a = np.where(np.isnan(a), 0.0, a)
    j = np.clip(np.searchsorted(pos, a, side="left"), 1, 0x7E)  # pos[j-1] < a <= pos[j]
    lo, hi = j - 1, j
    dlo = a - pos[lo]
    dhi = pos[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quantize(x, scale):
    """Codes stored for elements x under one scale: the fp32 quotient
    fl32(x / scale), then the nearest E4M3 code (R19)."""
    x32 = np.asarray(x, dtype=np.float32)
    return e4m3_encode(x32 / np.float32(scale))


def dequantize(codes, scale):
    """Values the codes stand for under one scale (R18), float64."""
    return e4m3_decode(codes) * float(np.float32(scale))


def kv_store_fp8(k_codes, v_codes, layer, k_new, v_new, loc, kv_scales):
    """Copies of the uint8 code pools [n_layers, n_slots, Hkv, D] with the new
    tokens' rows quantised into pool[layer, loc[t]] (loc[t] >= 0 only); every
    other byte is unchanged. P1, bullets on single advanced indexing
    buffer[layer_id, loc] and on the 4D layout; R18, R19."""
    k_out = np.array(k_codes, dtype=np.uint8, copy=True)
    v_out = np.array(v_codes, dtype=np.uint8, copy=True)
    ks, vs = (np.float32(s) for s in np.asarray(kv_scales, np.float32)[layer])
    loc = np.asarray(loc)
    for t in range(loc.shape[0]):
        if loc[t] >= 0:
            k_out[layer, loc[t]] = quantize(k_new[t], ks)
            v_out[layer, loc[t]] = quantize(v_new[t], vs)
    return k_out, v_out


def decode_attention_fp8(q, k_codes, v_codes, kv_scales, layer, req_to_token, req_pool_indices,
                         seq_lens, scale):
    """Decode attention over code pools: the decode definition on the
    represented values e4m3(c) * scale of the layer (R20)."""
    ks, vs = np.asarray(kv_scales, np.float32)[layer]
    kp = dequantize(np.asarray(k_codes)[layer:layer + 1], ks)
    vp = dequantize(np.asarray(v_codes)[layer:layer + 1], vs)
    return decode_attention(q, kp, vp, 0, req_to_token, req_pool_indices, seq_lens, scale)


def prefill_attention_fp8(q, k_codes, v_codes, kv_scales, layer, req_to_token, req_pool_indices,
                          seq_lens, qo_indptr, scale, causal=True):
    """Packed prefill over code pools: the prefill definition on the
    represented values e4m3(c) * scale of the layer (R20)."""
    ks, vs = np.asarray(kv_scales, np.float32)[layer]
    kp = dequantize(np.asarray(k_codes)[layer:layer + 1], ks)
    vp = dequantize(np.asarray(v_codes)[layer:layer + 1], vs)
    return prefill_attention(q, kp, vp, 0, req_to_token, req_pool_indices, seq_lens, qo_indptr,
                             scale, causal=causal)


def rope_fp32(x, positions, freqs_cis, interleaved=True):
    """The rotation of R21 in fp32: each product and each sum rounded once to
    fp32 (numpy float32 arithmetic), returned as float32 [T, H, D]."""
    x = np.asarray(x, np.float32)
    T, H, D = x.shape
    tab = np.asarray(freqs_cis, np.float32)
    out = x.copy()
    for t in range(T):
        p = int(positions[t])
        for i, (a, b) in enumerate(rope_pairs(D, interleaved)):
            c, s = tab[p, i, 0], tab[p, i, 1]
            ac, bs = x[t, :, a] * c, x[t, :, b] * s
            bc, as_ = x[t, :, b] * c, x[t, :, a] * s
            out[t, :, a] = ac - bs
            out[t, :, b] = bc + as_
    return out


def rope_kv_store_fp8(q, k_new, v_new, positions, freqs_cis, k_codes, v_codes, layer, loc,
                      kv_scales, interleaved=True):
    """RoPE on the new tokens' q and k, then the quantising store of (rotated
    k, v) into the code pools (R15, R19, R21): returns (q_rot fp64, k_codes',
    v_codes')."""
    q_rot = apply_rope(q, positions, freqs_cis, interleaved)
    k_rot = rope_fp32(k_new, positions, freqs_cis, interleaved)
    kc, vc = kv_store_fp8(k_codes, v_codes, layer, k_rot, np.asarray(v_new, np.float32), loc,
                          kv_scales)
    return q_rot, kc, vc
