"""Seeded synthetic inputs for paged KV-cache attention.

This module only draws inputs: lengths, slot tables and N(0, 1) values. It
holds none of the attention arithmetic and imports neither the oracle nor the
native library, so the CPU oracle and the HIP path can both be fed from it.

Shapes follow the pages' data model:
  * K and V pools are 4D ``[n_layers, n_slots, n_kv_heads, head_dim]``
    (AstrAI commit 398e8a3e page, bullet on reverting KVStorage to 4D).
  * ``req_to_token`` maps (request row, position) -> slot, int32
    (same page, bullet on int32 page-table / request-row / location indices).
  * Packed prompts are delimited by ``qo_indptr`` (AstrAI commit e58a728b page,
    bullets on packing prompts and on cumulative query lengths).

Slot-assignment structures:
  * ``pages16``: a seeded permutation of 16-slot pages handed out to requests
    in order; token j of a request lives at ``page[j // 16] * 16 + j % 16``.
  * ``fragmented``: a seeded token-granular permutation of all slots, cut
    into consecutive segments, one per request.

Every table entry that is not a live token (padding past ``seq_len`` and all
unused request rows) points at ``poison_slot``, a slot that no request uses;
tests fill it with NaN so that a kernel reading past ``seq_len`` is caught.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Seeds: workload k draws lengths/slots from SEED_BASE + k + 1 and values from
# SEED_BASE + k.
SEED_BASE = 184_000
PAGE = 16


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Inputs are drawn in fp32 and then stored in bf16, so the values handed to
    both sides must be exactly bf16-representable.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = np.float32("nan")
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def normal_values(shape, seed: int, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws from PCG64(seed), rounded to bf16 when dtype == 'bf16'."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        v = round_to_bf16(v)
    return v


@dataclasses.dataclass
class PagedBatch:
    """Index structures of one batch over a paged KV pool (all int32)."""

    n_layers: int
    n_slots: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str  # 'bf16' or 'f32'
    scale: float
    seq_lens: np.ndarray  # [B] keys visible to the last query, incl. new tokens
    qo_indptr: np.ndarray  # [B+1] packed new-token offsets
    req_to_token: np.ndarray  # [R, stride]
    req_pool_indices: np.ndarray  # [B]
    poison_slot: int
    live_slots: np.ndarray  # sorted unique slots referenced by some live token
    name: str = ""

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def n_new(self) -> np.ndarray:
        return np.diff(self.qo_indptr).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.n_new.max()) if self.batch else 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def kv_bytes_logical(self) -> int:
        es = 2 if self.dtype == "bf16" else 4
        return int(self.seq_lens.astype(np.int64).sum()) * self.n_kv_heads * self.head_dim * 2 * es

    def kv_bytes_unique(self) -> int:
        es = 2 if self.dtype == "bf16" else 4
        return int(self.live_slots.size) * self.n_kv_heads * self.head_dim * 2 * es


def _tables(rng, n_slots, seq_lens, slot_lists, n_rows, stride, poison):
    B = len(seq_lens)
    r2t = np.full((n_rows, stride), poison, dtype=np.int32)
    rows = rng.choice(n_rows, size=B, replace=False).astype(np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        r2t[rows[b], :L] = slot_lists[b][:L]
    return r2t, rows


def _pages16_slots(rng, n_slots, lengths, reserve):
    """Shuffled 16-slot pages, handed out in order; ``reserve`` slots at the top are kept free."""
    n_pages = (n_slots - reserve) // PAGE
    pages = rng.permutation(n_pages)
    out, cursor = [], 0
    for L in lengths:
        need = (int(L) + PAGE - 1) // PAGE
        if cursor + need > n_pages:
            raise ValueError("pool too small for the requested lengths")
        pg = pages[cursor:cursor + need]
        cursor += need
        j = np.arange(int(L))
        out.append((pg[j // PAGE] * PAGE + j % PAGE).astype(np.int32))
    return out


def _fragmented_slots(rng, n_slots, lengths, reserve):
    perm = rng.permutation(n_slots - reserve).astype(np.int32)
    out, cursor = [], 0
    for L in lengths:
        L = int(L)
        if cursor + L > perm.size:
            raise ValueError("pool too small for the requested lengths")
        out.append(perm[cursor:cursor + L])
        cursor += L
    return out


def _finish(name, n_layers, n_slots, hq, hkv, d, dtype, scale, seq_lens, n_new,
            slot_lists, rng, stride=None, n_rows=None):
    B = len(seq_lens)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    n_new = np.asarray(n_new, dtype=np.int32)
    poison = n_slots - 1
    if stride is None:
        stride = max(int(seq_lens.max()) if B else 1, 1)
    if n_rows is None:
        n_rows = max(2 * B, 1)
    r2t, rows = _tables(rng, n_slots, seq_lens, slot_lists, n_rows, stride, poison)
    qo = np.zeros(B + 1, dtype=np.int32)
    qo[1:] = np.cumsum(n_new)
    live = np.unique(np.concatenate([s[: int(L)] for s, L in zip(slot_lists, seq_lens)])) \
        if B else np.zeros(0, np.int32)
    return PagedBatch(n_layers, n_slots, hq, hkv, d, dtype, float(scale), seq_lens, qo,
                      r2t, rows, poison, live.astype(np.int32), name)


# --------------------------------------------------------------------------
# The five workloads (sizes as fixed in the design notes; "K" = 1024).
# --------------------------------------------------------------------------

def tiny_decode(poison_unused: bool = False) -> PagedBatch:
    """1 layer, B=2, 4 q / 2 KV heads, head_dim 64, fp32, seq_lens {17, 40},
    128-slot pool, slots taken from one seeded permutation, scale 1/8."""
    k = 1
    rng = np.random.default_rng(SEED_BASE + k + 1)
    n_slots = 128
    perm = rng.permutation(n_slots - 1).astype(np.int32)  # slot 127 is the poison slot
    lists = [perm[0:17], perm[17:57]]
    b = _finish("tiny_decode", 1, n_slots, 4, 2, 64, "f32", 1.0 / 8.0, [17, 40], [1, 1],
                lists, rng)
    b.name = "tiny_decode_poisoned" if poison_unused else "tiny_decode"
    return b


def b1_decode(ctx: int, n_layers: int = 1) -> PagedBatch:
    """B=1 decode, 32 q / 8 KV heads, head_dim 128, bf16, 40K-slot pool of shuffled 16-pages."""
    k = 2
    rng = np.random.default_rng(SEED_BASE + k + 1 + ctx)
    n_slots = 40 * 1024
    lists = _pages16_slots(rng, n_slots, [ctx], reserve=PAGE)
    return _finish(f"b1_decode_{ctx // 1024}k", n_layers, n_slots, 32, 8, 128, "bf16",
                   1.0 / np.sqrt(128.0), [ctx], [1], lists, rng)


def ragged_decode(batch: int, n_layers: int = 1) -> PagedBatch:
    """B in {8, 32}; seq_lens ~ U{512..8192}; a seeded quarter of the requests
    shares one 2048-token prefix (identical slots) and has L ~ U{2049..8192};
    the rest use shuffled 16-pages; pool of 2^19 slots."""
    k = 3
    rng = np.random.default_rng(SEED_BASE + k + 1 + batch)
    n_slots = 1 << 19
    lens = rng.integers(512, 8192, size=batch, endpoint=True)
    shared = np.sort(rng.choice(batch, size=batch // 4, replace=False))
    for b in shared:
        lens[b] = rng.integers(2049, 8192, endpoint=True)
    prefix_len = 2048
    # The shared prefix takes the first pages; every request's private tail follows.
    tails = [int(lens[b]) - (prefix_len if b in shared else 0) for b in range(batch)]
    lists_all = _pages16_slots(rng, n_slots, [prefix_len] + tails, reserve=PAGE)
    prefix = lists_all[0]
    lists = []
    for b in range(batch):
        tail = lists_all[1 + b]
        lists.append(np.concatenate([prefix, tail]) if b in shared else tail)
    out = _finish(f"ragged_decode_b{batch}", n_layers, n_slots, 32, 8, 128, "bf16",
                  1.0 / np.sqrt(128.0), lens, np.ones(batch, np.int32), lists, rng)
    out.shared_rows = shared  # type: ignore[attr-defined]
    out.shared_prefix = prefix_len  # type: ignore[attr-defined]
    return out


def shared_prefix_decode(batch: int = 32, prefix_len: int = 4096,
                         n_layers: int = 1) -> PagedBatch:
    """Every request of the batch shares one prefix of prefix_len keys (the
    same slots) and has a private tail of U{32..512} keys; shuffled 16-pages in
    a 2^18-slot pool; 32 q / 8 KV heads, head_dim 128, bf16. A case where the
    prefix dominates the logical K/V bytes."""
    k = 6
    rng = np.random.default_rng(SEED_BASE + k + 1 + batch)
    n_slots = 1 << 18
    tails = rng.integers(32, 512, size=batch, endpoint=True)
    lists_all = _pages16_slots(rng, n_slots, [prefix_len] + [int(t) for t in tails],
                               reserve=PAGE)
    lists = [np.concatenate([lists_all[0], lists_all[1 + b]]) for b in range(batch)]
    lens = tails + prefix_len
    out = _finish(f"shared_prefix_decode_b{batch}", n_layers, n_slots, 32, 8, 128, "bf16",
                  1.0 / np.sqrt(128.0), lens, np.ones(batch, np.int32), lists, rng)
    out.shared_rows = np.arange(batch)  # type: ignore[attr-defined]
    out.shared_prefix = prefix_len  # type: ignore[attr-defined]
    return out


def packed_prefill(n_layers: int = 1, n_req: int = 8) -> PagedBatch:
    """8 requests, new tokens n_b ~ U{64..2048}, cached prefix P_b ~ U{0..4096},
    packed by qo_indptr; 65536-slot pool of shuffled 16-pages; 32 q / 8 KV heads,
    head_dim 128, bf16, causal over the new tokens."""
    k = 4
    rng = np.random.default_rng(SEED_BASE + k + 1)
    n_slots = 1 << 16
    n_new = rng.integers(64, 2048, size=n_req, endpoint=True)
    prefix = rng.integers(0, 4096, size=n_req, endpoint=True)
    lens = prefix + n_new
    lists = _pages16_slots(rng, n_slots, lens, reserve=PAGE)
    return _finish("packed_prefill", n_layers, n_slots, 32, 8, 128, "bf16",
                   1.0 / np.sqrt(128.0), lens, n_new, lists, rng)


def large_batch_decode(n_layers: int = 1, sigma: float = 1.0,
                       layout: str = "fragmented") -> PagedBatch:
    """B=64, 64 q / 8 KV heads, head_dim 128, bf16; L = min(32768, max(1, round(4096 exp(sigma Z))));
    2^21-slot pool with token-granular (fragmented) slot assignment, or, for
    comparison, the same lengths in shuffled 16-token pages."""
    k = 5
    rng = np.random.default_rng(SEED_BASE + k + 1)
    n_slots = 1 << 21
    z = rng.standard_normal(64)
    lens = np.minimum(32768, np.maximum(1, np.rint(4096.0 * np.exp(sigma * z)))).astype(np.int64)
    if layout == "fragmented":
        lists = _fragmented_slots(rng, n_slots, lens, reserve=1)
    elif layout == "pages16":
        lists = _pages16_slots(rng, n_slots, lens, reserve=PAGE)
    else:
        raise ValueError(layout)
    return _finish("large_batch_decode", n_layers, n_slots, 64, 8, 128, "bf16",
                   1.0 / np.sqrt(128.0), lens, np.ones(64, np.int32), lists, rng)


def custom(name: str, *, n_layers: int, n_slots: int, n_q_heads: int, n_kv_heads: int,
           head_dim: int, dtype: str, seq_lens, n_new, seed: int, layout: str = "pages16",
           scale: Optional[float] = None, stride: Optional[int] = None,
           n_rows: Optional[int] = None, shared_prefix: int = 0) -> PagedBatch:
    """A seeded batch of any shape, for parity tests and edge cases.

    ``shared_prefix`` > 0 makes every request whose length exceeds it reuse the
    slots of the first such request for its first ``shared_prefix`` tokens.
    """
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    n_new = np.asarray(n_new, dtype=np.int64)
    if np.any(n_new > seq_lens) or np.any(n_new < 0):
        raise ValueError("need 0 <= n_new <= seq_len")
    if layout == "pages16":
        lists = _pages16_slots(rng, n_slots, seq_lens, reserve=PAGE)
    elif layout == "fragmented":
        lists = _fragmented_slots(rng, n_slots, seq_lens, reserve=1)
    else:
        raise ValueError(layout)
    if shared_prefix > 0:
        owner = None
        for b, L in enumerate(seq_lens):
            if L > shared_prefix:
                if owner is None:
                    owner = lists[b][:shared_prefix].copy()
                else:
                    lists[b] = lists[b].copy()
                    lists[b][:shared_prefix] = owner
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    return _finish(name, n_layers, n_slots, n_q_heads, n_kv_heads, head_dim, dtype, scale,
                   seq_lens, n_new, lists, rng, stride=stride, n_rows=n_rows)


def rope_freqs_cis(max_pos: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Input table for the rotary step: float32 [max_pos, head_dim/2, 2] holding
    (cos, sin) of angle p * base^(-2i/head_dim) for position p and pair i (the
    conventional frequency schedule; the library and the oracle both take the
    table as given)."""
    half = head_dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


# --------------------------------------------------------------------------
# Values
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Values:
    """Host values for a batch: q, the new tokens' K/V and the pools, as float32
    (exactly bf16-representable when dtype is bf16)."""

    q: np.ndarray  # [T_q, Hq, D]
    k_new: np.ndarray  # [T_q, Hkv, D]
    v_new: np.ndarray
    k_pool: np.ndarray  # [n_layers, n_slots, Hkv, D]
    v_pool: np.ndarray


def host_values(batch: PagedBatch, seed: int, poison_unreferenced: bool = True,
                layers_identical: bool = True) -> Values:
    """Draw q, k_new, v_new and fill every live slot of every layer with N(0,1).

    Slots no live token references are NaN when ``poison_unreferenced``.
    The new tokens' K/V are drawn separately; they become visible only once a
    store writes them at their cache locations.
    """
    hq, hkv, d = batch.n_q_heads, batch.n_kv_heads, batch.head_dim
    T = batch.total_q
    q = normal_values((T, hq, d), seed, batch.dtype)
    k_new = normal_values((T, hkv, d), seed + 7, batch.dtype)
    v_new = normal_values((T, hkv, d), seed + 11, batch.dtype)
    shape = (batch.n_layers, batch.n_slots, hkv, d)
    fill = np.float32("nan") if poison_unreferenced else np.float32(0.0)
    k_pool = np.full(shape, fill, dtype=np.float32)
    v_pool = np.full(shape, fill, dtype=np.float32)
    live = batch.live_slots
    n_layers_drawn = 1 if layers_identical else batch.n_layers
    for layer in range(n_layers_drawn):
        kv = normal_values((2, live.size, hkv, d), seed + 13 + layer, batch.dtype)
        k_pool[layer, live] = kv[0]
        v_pool[layer, live] = kv[1]
    if layers_identical:
        for layer in range(1, batch.n_layers):
            k_pool[layer] = k_pool[0]
            v_pool[layer] = v_pool[0]
    return Values(q, k_new, v_new, k_pool, v_pool)
