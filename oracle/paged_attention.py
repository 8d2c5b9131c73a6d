"""fp64 gather-then-softmax oracle for attention over a paged, slot-indexed KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring for the citation key and
the rule that the product path never imports this module).

What the pages fix, restated:
  * K and V live in separate 4D pools ``[n_layers, n_slots, n_kv_heads,
    head_dim]``, addressed as one advanced index ``pool[layer, loc]``
    (P1, bullets on single advanced indexing and on reverting KVStorage to 4D).
  * Page-table, request-row and cache-location indices are int32 (P1, bullet
    on int32 indices).
  * ``req_to_token`` maps (request row, position) -> slot; attention reads K/V
    through it rather than through a materialised gather (P1, bullet on
    removing Storage.gather; P4, bullet on the FlashAttention backend looking
    K/V up via req_to_token).
  * Decode writes split partials ``o_part`` and an "ml" partial that are later
    combined (P1, bullets on workspace-owned decode_o_part / decode_ml_part).
  * Prefill packs several prompts into one forward; each request's query rows
    are delimited by cumulative query lengths ``qo_indptr`` (P4, bullets on
    packing prompts with a shared prefix start and on per-request final
    logits from cumulative query lengths); cached prefix pages are reused
    (P1, bullet on rebuilding request mappings for cached prefix pages).

Readings where the pages are silent (each is listed in the design notes):
  R1 GQA: query head h reads KV head h // (Hq // Hkv).
  R2 kv_indptr is the exclusive prefix sum of seq_lens.
  R3 seq_lens[b] counts every key visible to request b's last query,
     including the new token(s) already stored.
  R4 prefill causality is bottom-right aligned: new token i of request b sees
     positions 0 .. P_b + i, with P_b = seq_lens[b] - n_b.
  R5 the softmax scale is a caller parameter.
  R6 split boundaries: chunk c_b = round_up(ceil(L_b / S_req), 16); the split
     count is S_b = ceil(L_b / c_b); split s covers [s c_b, min(L_b, (s+1) c_b)).
     S_req = fixed_splits if given, else ceil(L_b / split_tokens); both are
     clamped to [1, max_splits]. S_b = 0 when L_b = 0.
  R7 partials: o_s is normalised (divided by its own l_s); only
     lse_s = m_s + ln(l_s) is uniquely defined, m_s being a stabiliser.
  R8 decode rows with seq_len 0 are padding: their output is zero and their
     new-token location is -1 (a store skips negative locations).
  R13 rotary pairs: interleaved (2i, 2i+1) by default, the pairing of a
     complex-valued freqs_cis table read as consecutive real pairs; the
     half-split pairing (i, i + D/2) is the alternative.
  R14 the rotary table is freqs_cis[max_pos, D/2, 2] = (cos, sin) of the angle
     of pair i at position p, given by the caller (P4, bullet on describing the
     rotary table as cos/sin rather than a complex buffer).
  R15 RoPE is applied to the new tokens' q and k before k is stored; v is
     stored unrotated.
"""

from __future__ import annotations

import numpy as np

SPLIT_ALIGN = 16  # R6 granularity of split boundaries, in tokens


# ---------------------------------------------------------------- kv_store

def kv_store(k_pool, v_pool, layer, k_new, v_new, loc):
    """Return copies of the pools with ``pool[layer, loc[t]] = new[t]`` for every
    t with ``loc[t] >= 0``; every other byte is unchanged.

    P1, bullets on single advanced indexing ``buffer[layer_id, loc]`` and on the
    4D KVStorage layout. Negative locations are padded rows (R8).
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    loc = np.asarray(loc)
    for t in range(loc.shape[0]):
        if loc[t] >= 0:
            k_out[layer, loc[t]] = k_new[t]
            v_out[layer, loc[t]] = v_new[t]
    return k_out, v_out


# ---------------------------------------------------------- index step

def kv_indptr(seq_lens):
    """Exclusive prefix sum of seq_lens as int32 (R2; P1 bullet on updating
    position_ids / seq_lens / kv_indptr in place every step)."""
    s = np.asarray(seq_lens, dtype=np.int64)
    out = np.zeros(s.shape[0] + 1, dtype=np.int64)
    out[1:] = np.cumsum(s)
    if out[-1] >= 2**31:
        raise OverflowError("total KV length does not fit int32")
    return out.astype(np.int32)


def decode_locations(req_to_token, req_pool_indices, seq_lens):
    """Cache location of each request's newest token: ``req_to_token[r_b, L_b - 1]``,
    or -1 for a padded row with L_b = 0 (R3, R8)."""
    B = len(seq_lens)
    loc = np.empty(B, dtype=np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        loc[b] = req_to_token[req_pool_indices[b], L - 1] if L > 0 else -1
    return loc


def prefill_locations(req_to_token, req_pool_indices, seq_lens, qo_indptr):
    """Cache locations of the packed new tokens: row ``qo_indptr[b] + i`` gets
    ``req_to_token[r_b, P_b + i]`` with ``P_b = L_b - n_b`` (R3, R4; P4 bullet on
    cumulative query lengths)."""
    B = len(seq_lens)
    loc = np.empty(int(qo_indptr[B]), dtype=np.int32)
    for b in range(B):
        n = int(qo_indptr[b + 1] - qo_indptr[b])
        P = int(seq_lens[b]) - n
        for i in range(n):
            loc[qo_indptr[b] + i] = req_to_token[req_pool_indices[b], P + i]
    return loc


def _ceil_div(a, b):
    return -(-a // b)


def split_plan(seq_lens, max_splits, fixed_splits=0, split_tokens=256):
    """Per-request split count S_b and chunk length c_b under reading R6."""
    B = len(seq_lens)
    S = np.zeros(B, dtype=np.int32)
    C = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        req = fixed_splits if fixed_splits > 0 else _ceil_div(L, split_tokens)
        req = min(max(req, 1), max_splits)
        chunk = _ceil_div(_ceil_div(L, req), SPLIT_ALIGN) * SPLIT_ALIGN
        S[b] = _ceil_div(L, chunk)
        C[b] = chunk
    return S, C


def split_ranges(L, S, chunk):
    """Token ranges [lo, hi) of the S splits of a request of length L."""
    return [(s * chunk, min(L, (s + 1) * chunk)) for s in range(S)]


# ------------------------------------------------------------- attention

def gathered_kv(k_pool, v_pool, layer, req_to_token, row, n_keys):
    """K and V of one request's first ``n_keys`` positions, gathered through
    ``req_to_token`` and up-cast to fp64: two arrays ``[n_keys, Hkv, D]``."""
    slots = np.asarray(req_to_token[row, :n_keys], dtype=np.int64)
    K = np.asarray(k_pool[layer][slots], dtype=np.float64)
    V = np.asarray(v_pool[layer][slots], dtype=np.float64)
    return K, V


def _softmax_attend(qh, Kh, Vh, scale):
    """softmax(scale * Kh qh) applied to Vh, for one query vector (fp64)."""
    x = scale * (Kh @ qh)
    p = np.exp(x - x.max())
    return (p @ Vh) / p.sum()


def decode_attention(q, k_pool, v_pool, layer, req_to_token, req_pool_indices, seq_lens,
                     scale):
    """One query token per request: ``out[b, h] = softmax(scale q_bh K_b^T) V_b`` over
    the L_b keys of request b, with KV head h // g (R1). Rows with L_b = 0 are 0 (R8).

    q: [B, Hq, D]; pools: [n_layers, n_slots, Hkv, D]. Returns fp64 [B, Hq, D].
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K, V = gathered_kv(k_pool, v_pool, layer, req_to_token, req_pool_indices[b], L)
        for h in range(Hq):
            out[b, h] = _softmax_attend(np.asarray(q[b, h], np.float64), K[:, h // g],
                                        V[:, h // g], scale)
    return out


def decode_split_partials(q, k_pool, v_pool, layer, req_to_token, req_pool_indices,
                          seq_lens, scale, S, chunk):
    """Split-KV partials (R6, R7; P1 bullets on decode_o_part / decode_ml_part).

    Returns, per request b, arrays ``o [Hq, S_b, D]`` (normalised per split) and
    ``lse [Hq, S_b]`` with ``lse_s = log sum_{j in split s} exp(scale q k_j)``.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    g = Hq // Hkv
    result = []
    for b in range(B):
        L, Sb, c = int(seq_lens[b]), int(S[b]), int(chunk[b])
        o = np.zeros((Hq, Sb, D))
        lse = np.full((Hq, Sb), -np.inf)
        if L > 0:
            K, V = gathered_kv(k_pool, v_pool, layer, req_to_token, req_pool_indices[b], L)
            for s, (lo, hi) in enumerate(split_ranges(L, Sb, c)):
                for h in range(Hq):
                    x = scale * (K[lo:hi, h // g] @ np.asarray(q[b, h], np.float64))
                    m = x.max()
                    p = np.exp(x - m)
                    o[h, s] = (p @ V[lo:hi, h // g]) / p.sum()
                    lse[h, s] = m + np.log(p.sum())
        result.append((o, lse))
    return result


def lse_merge(o_parts, lse_parts):
    """Combine split partials: with M = max_s lse_s and w_s = exp(lse_s - M),
    ``o = sum_s w_s o_s / sum_s w_s``. Splits with lse = -inf weigh nothing; if
    every split is empty the result is 0.

    o_parts: [..., S, D]; lse_parts: [..., S]. Returns [..., D].
    """
    o_parts = np.asarray(o_parts, np.float64)
    lse = np.asarray(lse_parts, np.float64)
    if lse.shape[-1] == 0:
        return np.zeros(o_parts.shape[:-2] + (o_parts.shape[-1],))
    M = lse.max(axis=-1, keepdims=True)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lse), np.exp(lse - Msafe), 0.0)
    num = (w[..., None] * o_parts).sum(axis=-2)
    den = w.sum(axis=-1)[..., None]
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def prefill_attention(q, k_pool, v_pool, layer, req_to_token, req_pool_indices, seq_lens,
                      qo_indptr, scale, causal=True, rows=None):
    """Ragged packed paged prefill (P4 bullets on packed prompts and qo_indptr;
    P1 bullet on cached prefix pages).

    New token i of request b is output row ``qo_indptr[b] + i``. With ``causal``
    it sees positions 0 .. P_b + i (R4); without, all L_b positions. q: [T_q, Hq, D].
    ``rows``, if given, restricts the work to those output rows (others are NaN).
    Returns fp64 [T_q, Hq, D].
    """
    T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    g = Hq // Hkv
    B = len(seq_lens)
    out = np.full((T, Hq, D), np.nan) if rows is not None else np.zeros((T, Hq, D))
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(B):
        lo_q, hi_q = int(qo_indptr[b]), int(qo_indptr[b + 1])
        n = hi_q - lo_q
        if n == 0:
            continue
        L = int(seq_lens[b])
        P = L - n
        K, V = gathered_kv(k_pool, v_pool, layer, req_to_token, req_pool_indices[b], L)
        for i in range(n):
            t = lo_q + i
            if wanted is not None and t not in wanted:
                continue
            vis = P + i + 1 if causal else L
            for h in range(Hq):
                out[t, h] = _softmax_attend(np.asarray(q[t, h], np.float64), K[:vis, h // g],
                                            V[:vis, h // g], scale)
    return out


# ------------------------------------------------------- rotary + store

def rope_pairs(D, interleaved):
    """Index pairs (a_i, b_i), i < D/2, that one rotation angle acts on (R13):
    interleaved (2i, 2i+1), the layout of a complex-valued frequency table
    viewed as consecutive real pairs; otherwise half-split (i, i + D/2)."""
    half = D // 2
    if interleaved:
        return [(2 * i, 2 * i + 1) for i in range(half)]
    return [(i, i + half) for i in range(half)]


def apply_rope(x, positions, freqs_cis, interleaved=True):
    """Rotary position embedding of packed 3D rows (P1, bullet on extending the
    rotary embedding to packed 3D inputs; P4, bullet on the cos/sin freqs_cis
    table).

    x: [T, H, D]; positions: [T] int; freqs_cis: [max_pos, D/2, 2] holding
    (cos, sin) of the angle of pair i at each position (R14). Pair i of row t
    is rotated by the angle of (positions[t], i):
        a' = a cos - b sin,   b' = b cos + a sin.
    Returns fp64 [T, H, D].
    """
    x = np.asarray(x, np.float64)
    T, H, D = x.shape
    out = x.copy()
    for t in range(T):
        p = int(positions[t])
        for i, (a, b) in enumerate(rope_pairs(D, interleaved)):
            c = float(freqs_cis[p, i, 0])
            s = float(freqs_cis[p, i, 1])
            out[t, :, a] = x[t, :, a] * c - x[t, :, b] * s
            out[t, :, b] = x[t, :, b] * c + x[t, :, a] * s
    return out


def rope_kv_store(q, k_new, v_new, positions, freqs_cis, k_pool, v_pool, layer, loc,
                  interleaved=True):
    """RoPE on the new tokens' q and k, then the store of (rotated k, v) at the
    cache locations (R15): returns (q_rot fp64 [T, Hq, D], k_pool', v_pool'),
    where the pools are float64 copies with ``pool[layer, loc[t]]`` replaced for
    every t with loc[t] >= 0 (R8) and every other entry unchanged."""
    q_rot = apply_rope(q, positions, freqs_cis, interleaved)
    k_rot = apply_rope(k_new, positions, freqs_cis, interleaved)
    kp, vp = kv_store(np.asarray(k_pool, np.float64), np.asarray(v_pool, np.float64), layer,
                      k_rot, np.asarray(v_new, np.float64), loc)
    return q_rot, kp, vp
