"""GPU: index step (a1) and kv_store (a2) against the oracle, bit-exact."""

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_184_amd import ops
from paged_kv_cache_184_amd import workloads as W
from tests.gpu_util import DEV, DeviceBatch, say

pytestmark = pytest.mark.gpu


def _batches():
    yield W.tiny_decode()
    yield W.b1_decode(4096)
    yield W.ragged_decode(32)
    yield W.packed_prefill()
    yield W.custom("padded", n_layers=1, n_slots=4096, n_q_heads=4, n_kv_heads=2, head_dim=64,
                   dtype="bf16", seq_lens=[0, 17, 0, 1, 300, 16], n_new=[0, 3, 0, 1, 300, 16],
                   seed=77)
    # more requests than scan threads, to cover multi-element runs per thread
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 40, size=3000)
    yield W.custom("many", n_layers=1, n_slots=1 << 17, n_q_heads=2, n_kv_heads=1, head_dim=64,
                   dtype="bf16", seq_lens=lens, n_new=np.minimum(lens, 2), seed=78)


@pytest.mark.parametrize("batch", list(_batches()), ids=lambda b: b.name)
def test_metadata_bit_exact(batch):
    say(f"metadata {batch.name} B={batch.batch}")
    db = DeviceBatch.__new__(DeviceBatch)
    db.b = batch
    db.r2t = torch.from_numpy(batch.req_to_token).to(DEV)
    db.rows = torch.from_numpy(batch.req_pool_indices).to(DEV)
    db.lens = torch.from_numpy(batch.seq_lens).to(DEV)
    db.qo = torch.from_numpy(batch.qo_indptr).to(DEV)
    B = batch.batch
    for max_splits, fixed, tokens in [(128, 0, 256), (7, 0, 16), (64, 3, 16), (1, 0, 16)]:
        ind = torch.full((B + 1,), -7, dtype=torch.int32, device=DEV)
        loc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        spl = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        ops.build_metadata(db.meta(), ops.PKV_MODE_DECODE, ops.split_cfg(max_splits, fixed, tokens),
                           ind, loc, spl)
        torch.cuda.synchronize()
        assert np.array_equal(ind.cpu().numpy(), O.kv_indptr(batch.seq_lens))
        assert np.array_equal(loc.cpu().numpy(), O.decode_locations(
            batch.req_to_token, batch.req_pool_indices, batch.seq_lens))
        S, _ = O.split_plan(batch.seq_lens, max_splits, fixed, tokens)
        assert np.array_equal(spl.cpu().numpy(), S)
    # prefill mode: locations of the packed new tokens
    T = batch.total_q
    loc = torch.full((max(T, 1),), -7, dtype=torch.int32, device=DEV)
    ind = torch.full((B + 1,), -7, dtype=torch.int32, device=DEV)
    ops.build_metadata(db.meta(with_qo=True), ops.PKV_MODE_PREFILL, None, ind, loc, None)
    torch.cuda.synchronize()
    ref = O.prefill_locations(batch.req_to_token, batch.req_pool_indices, batch.seq_lens,
                              batch.qo_indptr)
    assert np.array_equal(loc.cpu().numpy()[:T], ref)
    assert np.array_equal(ind.cpu().numpy(), O.kv_indptr(batch.seq_lens))


def test_metadata_empty_batch():
    r2t = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
    e = torch.zeros((0,), dtype=torch.int32, device=DEV)
    meta = ops.make_meta(r2t, e, e)
    ind = torch.full((1,), 9, dtype=torch.int32, device=DEV)
    ops.build_metadata(meta, ops.PKV_MODE_DECODE, ops.split_cfg(4), ind, None, None)
    torch.cuda.synchronize()
    assert ind.item() == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_store_bit_exact(dtype):
    say(f"kv_store {dtype}")
    rng = np.random.default_rng(11)
    n_layers, n_slots, hkv, d = 3, 700, 4, 64
    shape = (n_layers, n_slots, hkv, d)
    kp = W.normal_values(shape, 1, dtype)
    vp = W.normal_values(shape, 2, dtype)
    T = 300
    kn = W.normal_values((T, hkv, d), 3, dtype)
    vn = W.normal_values((T, hkv, d), 4, dtype)
    loc = rng.permutation(n_slots)[:T].astype(np.int32)
    loc[::17] = -1  # padded rows
    loc[5] = n_slots + 3  # out of range: skipped
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    K = torch.from_numpy(kp).to(DEV, dt)
    V = torch.from_numpy(vp).to(DEV, dt)
    ops.kv_store(K, V, 1, torch.from_numpy(kn).to(DEV, dt), torch.from_numpy(vn).to(DEV, dt),
                 torch.from_numpy(loc).to(DEV))
    torch.cuda.synchronize()
    loc_o = loc.copy()
    loc_o[5] = -1  # the oracle's reading: out-of-range locations are no-ops too
    rk, rv = O.kv_store(kp, vp, 1, kn, vn, loc_o)
    # compare the stored bit patterns of the whole pools
    gk = K.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
    gv = V.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
    if dtype == "bf16":
        ek = W.bf16_bits(rk).view(np.int16)
        ev = W.bf16_bits(rv).view(np.int16)
    else:
        ek = rk.astype(np.float32).view(np.int32)
        ev = rv.astype(np.float32).view(np.int32)
    assert np.array_equal(gk, ek)
    assert np.array_equal(gv, ev)


def test_kv_store_large_prefill_rows():
    """The packed-prefill workload's new tokens, stored into a 65536-slot pool."""
    b = W.packed_prefill()
    say(f"kv_store packed_prefill T={b.total_q}")
    db = DeviceBatch(b, seed=5)
    before_k = db.k_pool.clone()
    loc = torch.from_numpy(O.prefill_locations(b.req_to_token, b.req_pool_indices, b.seq_lens,
                                               b.qo_indptr)).to(DEV)
    ops.kv_store(db.k_pool, db.v_pool, 0, db.k_new, db.v_new, loc)
    torch.cuda.synchronize()
    li = loc.long()
    assert torch.equal(db.k_pool[0, li].view(torch.int16), db.k_new.view(torch.int16))
    assert torch.equal(db.v_pool[0, li].view(torch.int16), db.v_new.view(torch.int16))
    mask = torch.ones(b.n_slots, dtype=torch.bool, device=DEV)
    mask[li] = False
    assert torch.equal(db.k_pool[0, mask].view(torch.int16), before_k[0, mask].view(torch.int16))
