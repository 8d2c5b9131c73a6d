"""GPU: packed prefill over layer pools past 32-bit byte offsets.

The prefill kernel addresses K/V through buffer descriptors (32-bit byte
offsets) while a layer's pool stays below 0xF0000000 bytes, and through
64-bit global addresses above that. These pools hold 2^32 bytes per layer
(8 KV heads of head_dim 128 or 64: 2^21 or 2^22 bf16 slots, 2^22 or 2^23
E4M3 slots), so the requests' pages, spread over the whole pool, reach
offsets near 4 GiB on the second path. Only the live slots get values (unreferenced ones hold NaN or NaN
codes); the oracle sees those slots compacted under a remapped table, which
leaves its result unchanged.
"""

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_184_amd import ops
from paged_kv_cache_184_amd import workloads as W
from tests.gpu_util import DEV, compare, say

pytestmark = pytest.mark.gpu

LENS = np.array([700, 300, 129, 1, 450])
N_NEW = np.array([200, 64, 33, 1, 90])


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return t if dtype is None else t.to(dtype)


def compact_table(b):
    """The live slots in increasing order and the table remapped onto them."""
    live = b.live_slots.astype(np.int64)
    pos = {int(s): i for i, s in enumerate(live)}
    r2t = np.zeros_like(b.req_to_token)
    for i in range(b.batch):
        r, L = int(b.req_pool_indices[i]), int(b.seq_lens[i])
        r2t[r, :L] = [pos[int(s)] for s in b.req_to_token[r, :L]]
    return live, r2t


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_pool_past_32bit_offsets(kv, d):
    # 2^32 bytes per layer: 8 heads x d elements of 2 (bf16) or 1 (E4M3) bytes per slot
    n_slots = (1 << 32) // (8 * d * (2 if kv == "bf16" else 1))
    b = W.custom(f"large_pool_{kv}_{d}", n_layers=1, n_slots=n_slots, n_q_heads=32,
                 n_kv_heads=8, head_dim=d, dtype="bf16", seq_lens=LENS, n_new=N_NEW, seed=700)
    live, r2t_c = compact_table(b)
    say(f"  {kv}, head_dim {d}: {n_slots} slots per layer, highest live slot {int(live.max())}")
    assert live.max() >= n_slots // 2
    kv_live = W.normal_values((2, live.size, 8, d), 701, "bf16")
    q = W.normal_values((b.total_q, 32, d), 702, "bf16")
    k_new = W.normal_values((b.total_q, 8, d), 703, "bf16")
    v_new = W.normal_values((b.total_q, 8, d), 704, "bf16")
    shape = (1, n_slots, 8, d)
    idx = to_dev(live)
    if kv == "bf16":
        scales = None
        k_c, v_c = kv_live[0][None], kv_live[1][None]
        kd = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        vd = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        kd[0, idx] = to_dev(k_c[0], torch.bfloat16)
        vd[0, idx] = to_dev(v_c[0], torch.bfloat16)
    else:
        scales = np.float32([[0.02, 2.0 ** -6]])
        k_c = O.quantize(kv_live[0][None], scales[0, 0])
        v_c = O.quantize(kv_live[1][None], scales[0, 1])
        kd = torch.full(shape, 0x7F, dtype=torch.uint8, device=DEV)  # NaN codes
        vd = torch.full(shape, 0x7F, dtype=torch.uint8, device=DEV)
        kd[0, idx] = to_dev(k_c[0])
        vd[0, idx] = to_dev(v_c[0])
    sd = None if scales is None else to_dev(scales)
    meta = ops.make_meta(to_dev(b.req_to_token), to_dev(b.req_pool_indices), to_dev(b.seq_lens),
                         to_dev(b.qo_indptr))
    loc = torch.empty(b.total_q, dtype=torch.int32, device=DEV)
    ops.build_metadata(meta, ops.PKV_MODE_PREFILL, None, None, loc, None)
    ops.kv_store(kd, vd, 0, to_dev(k_new, torch.bfloat16), to_dev(v_new, torch.bfloat16), loc,
                 kv_scales=sd)
    out = ops.paged_prefill_attn(to_dev(q, torch.bfloat16), kd, vd, 0, meta, b.max_q_len,
                                 b.scale, True, kv_scales=sd)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    # the stored new tokens, read back at their compacted positions
    k_after = kd[0].index_select(0, idx).cpu()
    v_after = vd[0].index_select(0, idx).cpu()
    del kd, vd, out
    torch.cuda.empty_cache()
    loc_c = O.prefill_locations(r2t_c, b.req_pool_indices, b.seq_lens, b.qo_indptr)
    if kv == "bf16":
        kp, vp = O.kv_store(k_c, v_c, 0, k_new, v_new, loc_c)
        assert np.array_equal(k_after.float().numpy(), kp[0].astype(np.float32))
        assert np.array_equal(v_after.float().numpy(), vp[0].astype(np.float32))
        ref = O.prefill_attention(q, kp, vp, 0, r2t_c, b.req_pool_indices, b.seq_lens,
                                  b.qo_indptr, b.scale, causal=True)
    else:
        kp, vp = O.kv_store_fp8(k_c, v_c, 0, k_new, v_new, loc_c, scales)
        assert np.array_equal(k_after.numpy(), kp[0]) and np.array_equal(v_after.numpy(), vp[0])
        ref = O.prefill_attention_fp8(q, kp, vp, scales, 0, r2t_c, b.req_pool_indices,
                                      b.seq_lens, b.qo_indptr, b.scale, causal=True)
    compare(got, ref, "bf16", f"prefill over a 4 GiB {kv} layer pool, head_dim {d}")
