"""Python binding of libpkv: the C entry points of include/pkv.h under the same
names without the ``pkv_`` prefix.

Argument marshalling only: torch tensors are turned into device pointers and
descriptors, and the current HIP stream is passed through. Every step of the
computation runs in the library's HIP kernels; there is no Python or CPU
fallback, and a missing library raises ``LibraryMissing``.
"""

from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from . import _lib
from ._lib import BatchMeta, KVPool, SplitCfg, LibraryMissing  # noqa: F401

PKV_MODE_DECODE = _lib.PKV_MODE_DECODE
PKV_MODE_PREFILL = _lib.PKV_MODE_PREFILL


class PkvError(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name
        self.message = message


def lib():
    return _lib.load()


def _check(status: int) -> None:
    if status != _lib.PKV_OK:
        L = lib()
        raise PkvError(status, L.pkv_status_str(status).decode(), L.pkv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream: Optional[torch.cuda.Stream]):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return _lib.PKV_BF16
    if dtype == torch.float32:
        return _lib.PKV_F32
    if dtype in (torch.uint8, torch.float8_e4m3fn):
        return _lib.PKV_FP8_E4M3  # pools only: one-byte E4M3 codes
    raise TypeError(f"unsupported dtype {dtype}; use bfloat16, float32 or (pools) E4M3 bytes")


def io_dtype(pool_dtype: torch.dtype) -> torch.dtype:
    """dtype of q, the new K/V rows and the output for a pool dtype."""
    return torch.bfloat16 if dtype_code(pool_dtype) == _lib.PKV_FP8_E4M3 else pool_dtype


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def make_pool(k_pool: torch.Tensor, v_pool: torch.Tensor,
              kv_scales: Optional[torch.Tensor] = None) -> KVPool:
    """Descriptor of two contiguous [n_layers, n_slots, n_kv_heads, head_dim] pools.
    E4M3 pools (uint8 or float8_e4m3fn codes) need kv_scales: a contiguous
    float32 device tensor [n_layers, 2] of (k_scale, v_scale) per layer."""
    _need(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pools must be equal 4D tensors")
    _need(k_pool.is_contiguous() and v_pool.is_contiguous(), "pools must be contiguous")
    _need(k_pool.dtype == v_pool.dtype, "K and V pools must share a dtype")
    n_layers, n_slots, hkv, d = k_pool.shape
    code = dtype_code(k_pool.dtype)
    if code == _lib.PKV_FP8_E4M3:
        _need(kv_scales is not None and kv_scales.dtype == torch.float32 and
              kv_scales.is_contiguous() and tuple(kv_scales.shape) == (n_layers, 2),
              "an E4M3 pool needs kv_scales: contiguous float32 [n_layers, 2]")
    pool = KVPool(k_pool.data_ptr(), v_pool.data_ptr(), n_layers, n_slots, hkv, d, code, 0,
                  _ptr(kv_scales) if code == _lib.PKV_FP8_E4M3 else None)
    pool._tensors = (k_pool, v_pool, kv_scales)  # raw pointers inside: keep them alive
    return pool


def make_meta(req_to_token: torch.Tensor, req_pool_indices: torch.Tensor, seq_lens: torch.Tensor,
              qo_indptr: Optional[torch.Tensor] = None,
              kv_indptr: Optional[torch.Tensor] = None) -> BatchMeta:
    """Descriptor of the int32 batch metadata (all device tensors)."""
    for name, t in (("req_to_token", req_to_token), ("req_pool_indices", req_pool_indices),
                    ("seq_lens", seq_lens), ("qo_indptr", qo_indptr), ("kv_indptr", kv_indptr)):
        if t is not None:
            _need(t.dtype == torch.int32, f"{name} must be int32")
            _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(req_to_token.dim() == 2, "req_to_token must be 2D")
    _need(req_pool_indices.shape[0] == seq_lens.shape[0], "req_pool_indices / seq_lens length")
    _need(qo_indptr is None or qo_indptr.shape[0] == seq_lens.shape[0] + 1, "qo_indptr length")
    meta = BatchMeta(req_to_token.data_ptr(), req_to_token.stride(0), req_to_token.shape[0],
                     seq_lens.shape[0], req_pool_indices.data_ptr(), seq_lens.data_ptr(),
                     _ptr(qo_indptr), _ptr(kv_indptr))
    # the descriptor holds raw pointers: keep the tensors alive as long as it lives
    meta._tensors = (req_to_token, req_pool_indices, seq_lens, qo_indptr, kv_indptr)
    return meta


def split_cfg(max_splits: int, fixed_splits: int = 0, split_tokens: int = 256) -> SplitCfg:
    return SplitCfg(max_splits, fixed_splits, split_tokens, 0)


def choose_split(max_len: int, batch: int, n_kv_heads: int, n_cu: int = 256,
                 total_len: Optional[int] = None) -> SplitCfg:
    """The library's default split configuration for a decode batch
    (pkv_choose_split; the rule is documented in include/pkv.h). A host-only
    call: no GPU is needed."""
    out = SplitCfg()
    _check(lib().pkv_choose_split(int(max_len), int(batch),
                                  -1 if total_len is None else int(total_len), int(n_kv_heads),
                                  int(n_cu), C.byref(out)))
    return out


# ----------------------------------------------------------------- entry points

def abi_version() -> int:
    return lib().pkv_abi_version()


def kv_store(k_pool, v_pool, layer: int, k_new, v_new, loc, stream=None, kv_scales=None) -> None:
    """pool[layer, loc[t]] = new[t] for K and V (pkv_kv_store); E4M3 pools take
    bf16 rows and store their codes under the layer's scales."""
    pool = make_pool(k_pool, v_pool, kv_scales)
    io = io_dtype(k_pool.dtype)
    _need(k_new.dtype == io and v_new.dtype == io, "dtype mismatch")
    _need(k_new.is_contiguous() and v_new.is_contiguous(), "k_new / v_new must be contiguous")
    _need(loc.dtype == torch.int32 and loc.is_contiguous(), "loc must be contiguous int32")
    n = loc.shape[0]
    _need(k_new.numel() == n * k_pool.shape[2] * k_pool.shape[3], "k_new shape")
    _need(v_new.numel() == k_new.numel(), "v_new shape")
    _check(lib().pkv_kv_store(C.byref(pool), layer, k_new.data_ptr(), v_new.data_ptr(),
                              loc.data_ptr(), n, _stream(stream)))


def rope_kv_store(k_pool, v_pool, layer: int, k_new, v_new, positions, freqs_cis, loc,
                  q=None, q_out=None, interleaved: bool = True, stream=None,
                  kv_scales=None) -> None:
    """Rotary embedding of the new tokens fused with their store
    (pkv_rope_kv_store): pool[layer, loc[t]] = (rope(k_new[t]), v_new[t]) and,
    when q is given, q_out = rope(q) (q_out defaults to q: in place). E4M3
    pools take bf16 rows and store codes under the layer's scales."""
    pool = make_pool(k_pool, v_pool, kv_scales)
    io = io_dtype(k_pool.dtype)
    _need(k_new.dtype == io and v_new.dtype == io, "dtype mismatch")
    _need(k_new.is_contiguous() and v_new.is_contiguous(), "k_new / v_new must be contiguous")
    _need(loc.dtype == torch.int32 and loc.is_contiguous(), "loc must be contiguous int32")
    _need(positions.dtype == torch.int32 and positions.is_contiguous(),
          "positions must be contiguous int32")
    _need(freqs_cis.dtype == torch.float32 and freqs_cis.is_contiguous() and
          freqs_cis.dim() == 3 and freqs_cis.shape[1:] == (k_pool.shape[3] // 2, 2),
          "freqs_cis must be contiguous float32 [max_pos, head_dim/2, 2]")
    n = loc.shape[0]
    _need(positions.shape[0] == n, "positions shape")
    _need(k_new.numel() == n * k_pool.shape[2] * k_pool.shape[3], "k_new shape")
    _need(v_new.numel() == k_new.numel(), "v_new shape")
    hq = 0
    if q is not None:
        q_out = q if q_out is None else q_out
        _need(q.dtype == io and q.is_contiguous() and q_out.is_contiguous(), "q layout")
        _need(q.shape[0] == n and q_out.shape == q.shape, "q shape")
        hq = q.shape[1]
    _check(lib().pkv_rope_kv_store(C.byref(pool), layer, _ptr(q), _ptr(q_out), hq,
                                   k_new.data_ptr(), v_new.data_ptr(), positions.data_ptr(),
                                   freqs_cis.data_ptr(), freqs_cis.shape[0],
                                   1 if interleaved else 0, loc.data_ptr(), n, _stream(stream)))


def build_metadata(meta: BatchMeta, mode: int, split: Optional[SplitCfg] = None,
                   kv_indptr_out=None, loc_out=None, splits_out=None, stream=None) -> None:
    """Index step (pkv_build_metadata)."""
    split = split or split_cfg(1)
    cap = 0 if loc_out is None else loc_out.numel()
    _check(lib().pkv_build_metadata(C.byref(meta), mode, split, _ptr(kv_indptr_out),
                                    _ptr(loc_out), cap, _ptr(splits_out), _stream(stream)))


def decode_workspace_bytes(batch: int, n_q_heads: int, head_dim: int, max_splits: int) -> int:
    return int(lib().pkv_decode_workspace_bytes(batch, n_q_heads, head_dim, max_splits))


def alloc_decode_workspace(batch: int, n_q_heads: int, head_dim: int, max_splits: int,
                           device="cuda") -> torch.Tensor:
    """A byte tensor of pkv_decode_workspace_bytes (a plain tensor even under an
    inference-mode caller, so later in-place use from other threads works)."""
    n = decode_workspace_bytes(batch, n_q_heads, head_dim, max_splits)
    _need(n > 0, "invalid workspace arguments")
    with torch.inference_mode(False):
        return torch.empty(n, dtype=torch.uint8, device=device)


def workspace_views(ws: torch.Tensor, batch: int, n_q_heads: int, head_dim: int, max_splits: int):
    """(o_part, ml_part) fp32 views of a decode workspace, in the layout pkv.h documents."""
    o_elems = batch * n_q_heads * max_splits * head_dim
    ml_off = (o_elems * 4 + 255) // 256 * 256
    f = ws.view(torch.float32)
    o = f[:o_elems].view(batch, n_q_heads, max_splits, head_dim)
    ml = f[ml_off // 4: ml_off // 4 + batch * n_q_heads * max_splits * 2].view(
        batch, n_q_heads, max_splits, 2)
    return o, ml


def _q_check(q, pool: KVPool, batch_rows: int):
    _need(q.is_contiguous(), "q must be contiguous")
    _need(q.dim() == 3 and q.shape[0] == batch_rows and q.shape[2] == pool.head_dim, "q shape")
    io = _lib.PKV_BF16 if pool.dtype == _lib.PKV_FP8_E4M3 else pool.dtype
    _need(dtype_code(q.dtype) == io, "q dtype must match the pools (bf16 for E4M3 pools)")


def paged_decode_attn(q, k_pool, v_pool, layer: int, meta: BatchMeta, scale: float,
                      split: SplitCfg, workspace: torch.Tensor, out=None, stream=None,
                      kv_scales=None):
    """Split-KV paged decode (pkv_paged_decode_attn). q: [B, Hq, D]."""
    pool = make_pool(k_pool, v_pool, kv_scales)
    _q_check(q, pool, meta.batch)
    if out is None:
        out = torch.empty_like(q)
    _need(out.is_contiguous() and out.shape == q.shape and out.dtype == q.dtype, "out")
    _check(lib().pkv_paged_decode_attn(C.byref(pool), layer, q.data_ptr(), q.shape[1],
                                       C.byref(meta), scale, split, workspace.data_ptr(),
                                       workspace.numel(), out.data_ptr(), _stream(stream)))
    return out


def paged_decode_attn_noalloc(q, k_pool, v_pool, layer: int, meta: BatchMeta, scale: float,
                              split: SplitCfg, out, stream=None, kv_scales=None):
    """Split-KV paged decode with the partials in the library's own device
    scratch (pkv_paged_decode_attn_noalloc): no workspace, no allocation; ``out``
    must be given. Calls on one device must not overlap in time."""
    pool = make_pool(k_pool, v_pool, kv_scales)
    _q_check(q, pool, meta.batch)
    _need(out is not None and out.is_contiguous() and out.shape == q.shape and
          out.dtype == q.dtype, "out")
    _check(lib().pkv_paged_decode_attn_noalloc(C.byref(pool), layer, q.data_ptr(), q.shape[1],
                                               C.byref(meta), scale, split, out.data_ptr(),
                                               _stream(stream)))
    return out


def make_prefix_groups(prefix_len: torch.Tensor, group_indptr: torch.Tensor,
                       members: torch.Tensor, max_members: int) -> _lib.PrefixGroups:
    """Descriptor of the shared-prefix groups of a batch (device int32 tensors)."""
    for t, name in ((prefix_len, "prefix_len"), (group_indptr, "group_indptr"),
                    (members, "members")):
        _need(t.dtype == torch.int32 and t.is_contiguous() and t.is_cuda,
              f"{name} must be a contiguous int32 device tensor")
    g = _lib.PrefixGroups(prefix_len.data_ptr(), group_indptr.data_ptr(), members.data_ptr(),
                          group_indptr.numel() - 1, max_members, members.numel(), 0)
    g._tensors = (prefix_len, group_indptr, members)  # keep the buffers alive
    return g


def cascade_decode_attn(q, k_pool, v_pool, layer: int, meta: BatchMeta,
                        groups: _lib.PrefixGroups, scale: float, split: SplitCfg,
                        workspace: torch.Tensor, out=None, stream=None, kv_scales=None):
    """Decode with each group's shared prefix read once (pkv_cascade_decode_attn)."""
    pool = make_pool(k_pool, v_pool, kv_scales)
    _q_check(q, pool, meta.batch)
    if out is None:
        out = torch.empty_like(q)
    _need(out.is_contiguous() and out.shape == q.shape and out.dtype == q.dtype, "out")
    _check(lib().pkv_cascade_decode_attn(C.byref(pool), layer, q.data_ptr(), q.shape[1],
                                         C.byref(meta), C.byref(groups), scale, split,
                                         workspace.data_ptr(), workspace.numel(), out.data_ptr(),
                                         _stream(stream)))
    return out


def decode_step(q, k_pool, v_pool, layer: int, meta: BatchMeta, scale: float, split: SplitCfg,
                workspace: torch.Tensor, k_new=None, v_new=None, kv_indptr_out=None, loc_out=None,
                splits_out=None, out=None, stream=None, kv_scales=None):
    """Index step + store of the new tokens + decode attention in one launch
    (pkv_decode_step). k_new, v_new: [B, Hkv, D] or None."""
    pool = make_pool(k_pool, v_pool, kv_scales)
    _q_check(q, pool, meta.batch)
    if k_new is not None:
        _need(k_new.is_contiguous() and v_new is not None and v_new.is_contiguous(), "k_new/v_new")
        io = io_dtype(k_pool.dtype)
        _need(k_new.dtype == io and v_new.dtype == io, "k_new/v_new dtype")
        _need(k_new.numel() == meta.batch * pool.n_kv_heads * pool.head_dim, "k_new shape")
        _need(v_new.numel() == k_new.numel(), "v_new shape")
    for name, t, n in (("kv_indptr_out", kv_indptr_out, meta.batch + 1),
                       ("loc_out", loc_out, meta.batch), ("splits_out", splits_out, meta.batch)):
        if t is not None:
            _need(t.dtype == torch.int32 and t.is_contiguous() and t.numel() >= n, name)
    if out is None:
        out = torch.empty_like(q)
    _need(out.is_contiguous() and out.shape == q.shape and out.dtype == q.dtype, "out")
    _check(lib().pkv_decode_step(C.byref(pool), layer, q.data_ptr(), _ptr(k_new), _ptr(v_new),
                                 q.shape[1], C.byref(meta), scale, split, _ptr(kv_indptr_out),
                                 _ptr(loc_out), _ptr(splits_out), workspace.data_ptr(),
                                 workspace.numel(), out.data_ptr(), _stream(stream)))
    return out


def decode_partials(q, k_pool, v_pool, layer: int, meta: BatchMeta, scale: float,
                    split: SplitCfg, workspace: torch.Tensor, stream=None, kv_scales=None) -> None:
    pool = make_pool(k_pool, v_pool, kv_scales)
    _q_check(q, pool, meta.batch)
    _check(lib().pkv_decode_partials(C.byref(pool), layer, q.data_ptr(), q.shape[1],
                                     C.byref(meta), scale, split, workspace.data_ptr(),
                                     workspace.numel(), _stream(stream)))


def decode_merge(meta: BatchMeta, n_q_heads: int, head_dim: int, dtype: torch.dtype,
                 split: SplitCfg, workspace: torch.Tensor, out: torch.Tensor, stream=None):
    _check(lib().pkv_decode_merge(C.byref(meta), n_q_heads, head_dim, dtype_code(dtype), split,
                                  workspace.data_ptr(), workspace.numel(), out.data_ptr(),
                                  _stream(stream)))
    return out


def paged_prefill_attn(q, k_pool, v_pool, layer: int, meta: BatchMeta, max_q_len: int,
                       scale: float, causal: bool = True, out=None, stream=None, kv_scales=None):
    """Ragged packed paged prefill (pkv_paged_prefill_attn). q: [T_q, Hq, D]."""
    pool = make_pool(k_pool, v_pool, kv_scales)
    _need(q.is_contiguous() and q.dim() == 3 and q.shape[2] == pool.head_dim, "q shape")
    _need(q.dtype == io_dtype(k_pool.dtype), "q dtype must match the pools (bf16 for E4M3 pools)")
    if out is None:
        out = torch.empty_like(q)
    _need(out.is_contiguous() and out.shape == q.shape and out.dtype == q.dtype, "out")
    _check(lib().pkv_paged_prefill_attn(C.byref(pool), layer, q.data_ptr(), q.shape[1],
                                        C.byref(meta), q.shape[0], max_q_len, scale,
                                        1 if causal else 0, out.data_ptr(), _stream(stream)))
    return out


def validate_meta(meta: BatchMeta, mode: int, n_slots: int, total_q: int = 0, stream=None) -> None:
    """Synchronous debug check of the metadata contents (pkv_validate_meta)."""
    _check(lib().pkv_validate_meta(C.byref(meta), mode, n_slots, total_q, _stream(stream)))


class PreparedCall:
    """A C entry point with its arguments marshalled once, for tight loops and
    graph capture: ``call()`` re-issues the same launch with the same pointers.
    The last argument is the stream; when it was not fixed at preparation, the
    current stream is looked up at call time (so calls made under a graph
    capture land on the capturing stream)."""

    def __init__(self, fn_name: str, *args, keep=(), stream=None):
        self._fn = getattr(lib(), fn_name)
        self._args = list(args)
        self._stream = stream
        self._keep = keep  # keeps descriptor structs alive

    def __call__(self) -> None:
        s = self._stream if self._stream is not None else torch.cuda.current_stream()
        self._args[-1] = s.cuda_stream
        _check(self._fn(*self._args))


def prepare_decode(q, k_pool, v_pool, layer, meta: BatchMeta, scale, split, workspace, out,
                   stream=None, stage="all", kv_scales=None):
    pool = make_pool(k_pool, v_pool, kv_scales)
    _q_check(q, pool, meta.batch)
    s = None
    if stage == "all":
        return PreparedCall("pkv_paged_decode_attn", C.byref(pool), layer, q.data_ptr(), q.shape[1],
                            C.byref(meta), scale, split, workspace.data_ptr(), workspace.numel(),
                            out.data_ptr(), s, keep=(pool, meta), stream=stream)
    if stage == "partials":
        return PreparedCall("pkv_decode_partials", C.byref(pool), layer, q.data_ptr(), q.shape[1],
                            C.byref(meta), scale, split, workspace.data_ptr(), workspace.numel(), s,
                            keep=(pool, meta), stream=stream)
    if stage == "merge":
        return PreparedCall("pkv_decode_merge", C.byref(meta), q.shape[1], pool.head_dim,
                            dtype_code(q.dtype),
                            split, workspace.data_ptr(), workspace.numel(), out.data_ptr(), s,
                            keep=(pool, meta), stream=stream)
    raise ValueError(stage)


def prepare_decode_step(q, k_pool, v_pool, layer, meta: BatchMeta, scale, split, workspace, out,
                        k_new=None, v_new=None, kv_indptr_out=None, loc_out=None,
                        splits_out=None, stream=None, kv_scales=None):
    pool = make_pool(k_pool, v_pool, kv_scales)
    _q_check(q, pool, meta.batch)
    return PreparedCall("pkv_decode_step", C.byref(pool), layer, q.data_ptr(), _ptr(k_new),
                        _ptr(v_new), q.shape[1], C.byref(meta), scale, split,
                        _ptr(kv_indptr_out), _ptr(loc_out), _ptr(splits_out),
                        workspace.data_ptr(), workspace.numel(), out.data_ptr(), None,
                        keep=(pool, meta), stream=stream)


def prepare_cascade_decode(q, k_pool, v_pool, layer, meta: BatchMeta, groups, scale, split,
                           workspace, out, stream=None, kv_scales=None):
    pool = make_pool(k_pool, v_pool, kv_scales)
    return PreparedCall("pkv_cascade_decode_attn", C.byref(pool), layer, q.data_ptr(), q.shape[1],
                        C.byref(meta), C.byref(groups), scale, split, workspace.data_ptr(),
                        workspace.numel(), out.data_ptr(), None, keep=(pool, meta, groups),
                        stream=stream)


def prepare_kv_store(k_pool, v_pool, layer, k_new, v_new, loc, stream=None, kv_scales=None):
    pool = make_pool(k_pool, v_pool, kv_scales)
    return PreparedCall("pkv_kv_store", C.byref(pool), layer, k_new.data_ptr(), v_new.data_ptr(),
                        loc.data_ptr(), loc.shape[0], None, keep=(pool,), stream=stream)


def prepare_metadata(meta: BatchMeta, mode, split, kv_indptr_out=None, loc_out=None,
                     splits_out=None, stream=None):
    cap = 0 if loc_out is None else loc_out.numel()
    return PreparedCall("pkv_build_metadata", C.byref(meta), mode, split or split_cfg(1),
                        _ptr(kv_indptr_out), _ptr(loc_out), cap, _ptr(splits_out),
                        None, keep=(meta,), stream=stream)


def prepare_prefill(q, k_pool, v_pool, layer, meta: BatchMeta, max_q_len, scale, causal, out,
                    stream=None, kv_scales=None):
    pool = make_pool(k_pool, v_pool, kv_scales)
    return PreparedCall("pkv_paged_prefill_attn", C.byref(pool), layer, q.data_ptr(), q.shape[1],
                        C.byref(meta), q.shape[0], max_q_len, scale, 1 if causal else 0,
                        out.data_ptr(), None, keep=(pool, meta), stream=stream)
