"""Benchmark of the paged decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--ctx 32768] [--no-cpu]

A step is one pass of the whole decode hot path for one layer of a B=1 batch
(32 q / 8 KV heads, head_dim 128, bf16, 40K-slot pool of shuffled 16-token
pages): the index step (kv_indptr, new-token location, split plan), the store
of the new token's K/V, the split-KV partial kernel and the log-sum-exp merge.
Layers rotate over an 8-layer pool (1.34 GB of K+V) so that successive steps
read K/V from HBM, not from the 256 MB Infinity Cache.

The headline line is the 32K context; the other contexts (1K, 4K, 16K) are
reported under "detail". The timed region is K steps enqueued behind a short
device-side spin, so the GPU runs them back to back without host launch gaps;
ms_per_step comes from HIP events on the launch stream around the K steps, and
the partial kernel's duration from events around each of its launches.
The CPU oracle (fp64 NumPy) is timed on a bounded sample for cpu_baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--ctx", type=int, nargs="*", default=[1024, 4096, 16384, 32768])
    p.add_argument("--headline", type=int, default=32768)
    p.add_argument("--split-tokens", type=int, default=0,
                   help="tokens per split; 0 = ops.choose_split for the workload")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-batches", action="store_true", help="skip the batched decode workloads")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8 (E4M3) KV decode line")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--graph", action="store_true", help="also time HIP-graph replay")
    p.add_argument("--profile", action="store_true",
                   help="short run for hardware counters: a 256 MiB device copy (counter "
                        "calibration) then a few decode steps of the headline workload")
    return p.parse_args()


def profile_run(args):
    """A plain device-to-device copy of known size, then a few steps: the copy
    gives the scale of FETCH_SIZE / WRITE_SIZE for bytes actually moved."""
    import torch

    n = 256 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    from paged_kv_cache_184_amd import workloads as W

    db = DecodeBench(W.b1_decode(args.headline, n_layers=8), split_tokens=args.split_tokens,
                     seed=184_002)
    for i in range(max(8, args.steps)):
        db.step(i)
    torch.cuda.synchronize()
    db.run_partials(max(8, args.steps), 2)
    torch.cuda.synchronize()
    print(json.dumps({"profile": "done", "copy_bytes": n, "steps": max(8, args.steps),
                      "partial_kernel_bytes": db.partial_kernel_bytes()}), flush=True)


_SPIN_RATE = None


def spin_cycles_per_s() -> float:
    """Rate of the counter torch.cuda._sleep spins on, measured once with events."""
    global _SPIN_RATE
    if _SPIN_RATE is None:
        import torch

        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(100000)
        a.record()
        torch.cuda._sleep(2000000)
        b.record()
        torch.cuda.synchronize()
        _SPIN_RATE = 2000000 / (a.elapsed_time(b) * 1e-3)
    return _SPIN_RATE


class DecodeBench:
    """Device state of one B=1 decode workload and its prepared library calls."""

    def __init__(self, b, split_tokens: int, seed: int, kv: str = "bf16"):
        """b: a decode workload (one new token per request) with n_layers
        identical layers to rotate over. kv: "bf16" pools, or "fp8" pools of
        E4M3 codes (N(0,1) values under a scale of 1/64 per layer, saturated)."""
        import torch

        from paged_kv_cache_184_amd import ops

        self.torch, self.ops = torch, ops
        self.b = b
        self.kv = kv
        self.kv_es = 1 if kv == "fp8" else 2  # bytes per stored K/V element
        ctx = int(b.seq_lens.max())
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        shape = (b.n_layers, b.n_slots, b.n_kv_heads, b.head_dim)
        live = torch.from_numpy(b.live_slots).to(dev).long()
        vals = torch.randn((2, live.numel(), b.n_kv_heads, b.head_dim), generator=g, device=dev)
        if kv == "fp8":
            self.kv_scales = torch.full((b.n_layers, 2), 1.0 / 64, dtype=torch.float32, device=dev)
            self.k_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)  # NaN codes
            self.v_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
            vals = (vals * 64).clamp_(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            self.kv_scales = None
            self.k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
            self.v_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
            vals = vals.to(torch.bfloat16)
        for layer in range(b.n_layers):  # identical layers
            self.k_pool[layer, live] = vals[0]
            self.v_pool[layer, live] = vals[1]
        del vals
        B = b.batch
        self.q = torch.randn((B, b.n_q_heads, b.head_dim), generator=g, device=dev).to(torch.bfloat16)
        self.k_new = torch.randn((B, b.n_kv_heads, b.head_dim), generator=g, device=dev).to(torch.bfloat16)
        self.v_new = torch.randn((B, b.n_kv_heads, b.head_dim), generator=g, device=dev).to(torch.bfloat16)
        self.r2t = torch.from_numpy(b.req_to_token).to(dev)
        self.rows = torch.from_numpy(b.req_pool_indices).to(dev)
        self.lens = torch.from_numpy(b.seq_lens).to(dev)
        self.meta = ops.make_meta(self.r2t, self.rows, self.lens)
        if split_tokens > 0:
            self.split = ops.split_cfg(max(1, -(-ctx // split_tokens)), 0, split_tokens)
        else:
            self.split = ops.choose_split(ctx, b.batch, b.n_kv_heads,
                                          total_len=int(b.seq_lens.sum()))
        max_splits = self.split.max_splits
        self.ws = ops.alloc_decode_workspace(B, b.n_q_heads, b.head_dim, max_splits)
        self.out = torch.empty_like(self.q)
        self.kv_indptr = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.loc = torch.empty(B, dtype=torch.int32, device=dev)
        self.splits = torch.empty(B, dtype=torch.int32, device=dev)
        # separate path: index step, store, decode attention (merge fused inside)
        self.calls = []
        # fused path: all four rows in one launch
        self.fused = []
        for layer in range(b.n_layers):
            self.calls.append((
                ops.prepare_metadata(self.meta, ops.PKV_MODE_DECODE, self.split, self.kv_indptr,
                                     self.loc, self.splits),
                ops.prepare_kv_store(self.k_pool, self.v_pool, layer, self.k_new, self.v_new,
                                     self.loc, kv_scales=self.kv_scales),
                ops.prepare_decode(self.q, self.k_pool, self.v_pool, layer, self.meta, b.scale,
                                   self.split, self.ws, self.out, stage="all",
                                   kv_scales=self.kv_scales),
            ))
            self.fused.append(ops.prepare_decode_step(
                self.q, self.k_pool, self.v_pool, layer, self.meta, b.scale, self.split, self.ws,
                self.out, k_new=self.k_new, v_new=self.v_new, kv_indptr_out=self.kv_indptr,
                loc_out=self.loc, splits_out=self.splits, kv_scales=self.kv_scales))
        self.mode = "fused"
        # attention alone, plain or cascade (shared prefixes read once per group)
        self.attn_only = [c[2] for c in self.calls]
        self.cascade = None
        shared = getattr(b, "shared_rows", None)
        if shared is not None and len(shared) > 1 and kv == "bf16":
            P = int(b.shared_prefix)
            plen = np.zeros(B, np.int32)
            plen[shared] = P
            t = lambda x: torch.tensor(np.asarray(x, np.int32), device=dev)
            self.groups = ops.make_prefix_groups(t(plen), t([0, len(shared)]), t(shared),
                                                 len(shared))
            self.cascade = [ops.prepare_cascade_decode(self.q, self.k_pool, self.v_pool, layer,
                                                       self.meta, self.groups, b.scale,
                                                       self.split, self.ws, self.out)
                            for layer in range(b.n_layers)]

    # algorithmic bytes (K/V at kv_es bytes per element)
    def kv_bytes(self) -> int:
        return self.b.kv_bytes_logical() * self.kv_es // 2

    def kv_bytes_unique(self) -> int:
        return self.b.kv_bytes_unique() * self.kv_es // 2

    def partial_kernel_bytes(self) -> int:
        b = self.b
        L = int(b.seq_lens.sum())
        return self.kv_bytes() + b.batch * b.n_q_heads * b.head_dim * 2 + L * 4

    def step_bytes(self) -> int:
        """Algorithmic bytes of a whole step: K/V, q, slot ids, the output, and
        the new token's K/V read and stored."""
        b = self.b
        return (self.partial_kernel_bytes() + b.batch * b.n_q_heads * b.head_dim * 2 +
                2 * b.batch * b.n_kv_heads * b.head_dim * (2 + self.kv_es))

    def step(self, i: int):
        """One decode step for layer i mod n_layers."""
        if self.mode == "fused":
            self.fused[i % len(self.fused)]()
            return
        if self.mode in ("attn", "cascade"):
            calls = self.attn_only if self.mode == "attn" else self.cascade
            calls[i % len(calls)]()
            return
        for call in self.calls[i % len(self.calls)]:
            call()

    def run(self, steps: int, warmup: int):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        # host time to enqueue one step, and the device spin rate, so the hold
        # below lasts longer than enqueueing all K steps
        t = time.perf_counter()
        for i in range(8):
            self.step(i)
        enqueue_s = (time.perf_counter() - t) / 8
        torch.cuda.synchronize()
        cycles = int(min(2e9, max(1e5, 2.0 * steps * enqueue_s * spin_cycles_per_s())))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        # hold the stream so the host enqueues the K steps ahead of the GPU; the
        # start event is recorded after the hold
        torch.cuda._sleep(cycles)
        # only two events, around all K steps: an event between steps would put
        # a marker between the kernels and lengthen the step
        start.record()
        for i in range(steps):
            self.step(i)
        end.record()
        torch.cuda.synchronize()
        host_s = time.perf_counter() - t0
        return start.elapsed_time(end) / steps, host_s

    def run_partials(self, steps: int, warmup: int):
        """Average duration of the split-partial kernel alone (HIP events around
        each launch, on the launch stream), same configuration as the step."""
        torch = self.torch
        parts = [self.ops.prepare_decode(self.q, self.k_pool, self.v_pool, layer, self.meta,
                                         self.b.scale, self.split, self.ws, self.out,
                                         stage="partials", kv_scales=self.kv_scales)
                 for layer in range(self.b.n_layers)]
        for i in range(warmup):
            parts[i % len(parts)]()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))]
        t = time.perf_counter()
        for i in range(4):
            parts[i % len(parts)]()
        enqueue_s = (time.perf_counter() - t) / 4
        torch.cuda.synchronize()
        torch.cuda._sleep(int(min(2e9, max(1e5, 3.0 * steps * enqueue_s * spin_cycles_per_s()))))
        # back-to-back launches between two events: the per-launch average
        # carries no event overhead, only the (sub-microsecond) launch gaps
        evs[0][0].record()
        for i in range(steps):
            parts[i % len(parts)]()
        evs[0][1].record()
        torch.cuda.synchronize()
        return evs[0][0].elapsed_time(evs[0][1]) / steps

    def run_warm_same_layer(self, steps: int, warmup: int) -> float:
        """ms per fused step on layer 0 only (K/V cache-resident after the first)."""
        torch = self.torch
        call = self.fused[0]
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def run_graph(self, steps: int):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(len(self.calls)):
                self.step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        n_per_graph = len(self.calls)
        with torch.cuda.graph(g):
            for i in range(n_per_graph):
                self.step(i)
        torch.cuda.synchronize()
        reps = max(1, steps // n_per_graph)
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * n_per_graph)

    def oracle_inputs(self):
        b = self.b
        L = int(b.seq_lens[0])
        slots = b.req_to_token[b.req_pool_indices[0], :L]
        idx = self.torch.from_numpy(slots.astype(np.int64)).to("cuda")
        k = self.k_pool[0].index_select(0, idx).float().cpu().numpy()[None]
        v = self.v_pool[0].index_select(0, idx).float().cpu().numpy()[None]
        return (self.q[:1].float().cpu().numpy(), k, v, np.arange(L, dtype=np.int32)[None],
                np.array([0], np.int32), np.array([L], np.int32), b.scale)


def spread_us(ms_sorted):
    """[p10, p50, p90] in microseconds of sorted per-launch times in ms."""
    n = len(ms_sorted)
    pick = lambda q: ms_sorted[min(n - 1, int(q * (n - 1) + 0.5))] * 1e3
    return [round(pick(0.1), 1), round(pick(0.5), 1), round(pick(0.9), 1)]


def _time_calls(fn, steps: int) -> float:
    """Average ms of fn() over `steps` back-to-back calls between two events."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def new_token_steps(steps: int) -> dict:
    """The steps upstream of attention on the new tokens of the packed-prefill
    workload (T = 6710 tokens, 32 q / 8 KV heads, head_dim 128, bf16): the
    store of their K/V rows (a2) and the fused RoPE + store (f1, q rotated in
    place), and the same store into an E4M3 pool (quantising). GB/s counts the
    bytes each call must move: new rows read, pool rows written, q read and
    written."""
    import torch

    from paged_kv_cache_184_amd import ops
    from paged_kv_cache_184_amd import workloads as W

    b = W.packed_prefill(n_layers=1)
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(184_030)
    T, hq, hkv, d = b.total_q, b.n_q_heads, b.n_kv_heads, b.head_dim
    shape = (1, b.n_slots, hkv, d)
    kp = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    kp8 = torch.zeros(shape, dtype=torch.uint8, device=dev)
    vp8 = torch.zeros_like(kp8)
    scales = torch.full((1, 2), 1.0 / 64, dtype=torch.float32, device=dev)
    q = torch.randn((T, hq, d), generator=g, device=dev).to(torch.bfloat16)
    kn = torch.randn((T, hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((T, hkv, d), generator=g, device=dev).to(torch.bfloat16)
    loc = torch.from_numpy(np.concatenate([
        b.req_to_token[b.req_pool_indices[i], int(b.seq_lens[i] - b.n_new[i]):int(b.seq_lens[i])]
        for i in range(b.batch)]).astype(np.int32)).to(dev)
    pos = torch.from_numpy(np.concatenate([
        np.arange(int(b.seq_lens[i] - b.n_new[i]), int(b.seq_lens[i]))
        for i in range(b.batch)]).astype(np.int32)).to(dev)
    tab = torch.from_numpy(W.rope_freqs_cis(8192, d)).to(dev)
    row = hkv * d * 2  # bytes of one token's K (or V) row in bf16
    out = {}
    ms = _time_calls(lambda: ops.kv_store(kp, vp, 0, kn, vn, loc), steps)
    out["kv_store_us"] = round(ms * 1e3, 2)
    out["kv_store_gbs"] = round(4 * T * row / (ms * 1e-3) / 1e9, 1)
    ms = _time_calls(lambda: ops.rope_kv_store(kp, vp, 0, kn, vn, pos, tab, loc, q=q), steps)
    out["rope_kv_store_us"] = round(ms * 1e3, 2)
    out["rope_kv_store_gbs"] = round((4 * T * row + 2 * T * hq * d * 2) / (ms * 1e-3) / 1e9, 1)
    ms = _time_calls(lambda: ops.kv_store(kp8, vp8, 0, kn, vn, loc, kv_scales=scales), steps)
    out["kv_store_fp8_us"] = round(ms * 1e3, 2)
    out["kv_store_fp8_gbs"] = round((2 * T * row + T * row) / (ms * 1e-3) / 1e9, 1)
    out["tokens"] = int(T)
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak


class PrefillBench:
    """Packed ragged paged prefill: 8 requests, 64..2048 new tokens each over a
    0..4096-token cached prefix, 32 q / 8 KV heads, head_dim 128, bf16, causal.
    A step is the index step (new-token locations), the store of the new
    tokens' K/V and the MFMA prefill kernel, rotating over 8 layers. kv="fp8":
    E4M3 pools (N(0,1) values under a scale of 1/64, saturated) and a
    quantising store."""

    def __init__(self, n_layers: int, seed: int, kv: str = "bf16"):
        import torch

        from paged_kv_cache_184_amd import ops
        from paged_kv_cache_184_amd import workloads as W

        self.torch = torch
        b = W.packed_prefill(n_layers=n_layers)
        self.b = b
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        shape = (b.n_layers, b.n_slots, b.n_kv_heads, b.head_dim)
        live = torch.from_numpy(b.live_slots).to(dev).long()
        vals = torch.randn((2, live.numel(), b.n_kv_heads, b.head_dim), generator=g, device=dev)
        if kv == "fp8":
            self.kv_scales = torch.full((b.n_layers, 2), 1.0 / 64, dtype=torch.float32, device=dev)
            self.k_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)  # NaN codes
            self.v_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
            vals = (vals * 64).clamp_(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            self.kv_scales = None
            self.k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
            self.v_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
            vals = vals.to(torch.bfloat16)
        for layer in range(b.n_layers):
            self.k_pool[layer, live] = vals[0]
            self.v_pool[layer, live] = vals[1]
        del vals
        T = b.total_q
        self.q = torch.randn((T, b.n_q_heads, b.head_dim), generator=g, device=dev).to(torch.bfloat16)
        self.k_new = torch.randn((T, b.n_kv_heads, b.head_dim), generator=g, device=dev).to(torch.bfloat16)
        self.v_new = torch.randn((T, b.n_kv_heads, b.head_dim), generator=g, device=dev).to(torch.bfloat16)
        self.r2t = torch.from_numpy(b.req_to_token).to(dev)
        self.rows = torch.from_numpy(b.req_pool_indices).to(dev)
        self.lens = torch.from_numpy(b.seq_lens).to(dev)
        self.qo = torch.from_numpy(b.qo_indptr).to(dev)
        self.meta = ops.make_meta(self.r2t, self.rows, self.lens, self.qo)
        self.loc = torch.empty(T, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        self.calls = []
        for layer in range(b.n_layers):
            self.calls.append((
                ops.prepare_metadata(self.meta, ops.PKV_MODE_PREFILL, None, None, self.loc, None),
                ops.prepare_kv_store(self.k_pool, self.v_pool, layer, self.k_new, self.v_new,
                                     self.loc, kv_scales=self.kv_scales),
                ops.prepare_prefill(self.q, self.k_pool, self.v_pool, layer, self.meta,
                                    b.max_q_len, b.scale, True, self.out,
                                    kv_scales=self.kv_scales),
            ))

    def flops(self) -> float:
        b = self.b
        n = b.n_new.astype(np.float64)
        P = (b.seq_lens - b.n_new).astype(np.float64)
        return float(4 * b.head_dim * b.n_q_heads * np.sum(n * P + n * (n + 1) / 2))

    def run(self, steps: int, warmup: int):
        """(ms per step, mean ms per prefill launch, the launches' ms sorted).
        The warm-up runs at least 64 steps: the core clock climbs for tens of
        milliseconds of sustained MFMA work, and a launch right after a short
        warm-up runs up to 20% slower than in steady state."""
        torch = self.torch
        for i in range(max(warmup, 64)):
            for c in self.calls[i % len(self.calls)]:
                c()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            meta_call, store_call, attn_call = self.calls[i % len(self.calls)]
            meta_call()
            store_call()
            evs[i][0].record()
            attn_call()
            evs[i][1].record()
        end.record()
        torch.cuda.synchronize()
        step_ms = start.elapsed_time(end) / steps
        each = sorted(a.elapsed_time(b) for a, b in evs)
        return step_ms, float(np.mean(each)), each

    def run_kernels(self, steps: int) -> float:
        """ms per prefill launch: `steps` launches back to back (layers
        rotating) between two events on the launch stream, right after run()'s
        warm-up, so the average carries no per-launch event markers (the same
        method as the decode partial kernel's roofline figure)."""
        torch = self.torch
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            self.calls[i % len(self.calls)][2]()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_b1_32k_traffic.json")
KERNEL_SOURCES = ["paged_kv_cache_184_amd/csrc/decode_impl.hpp",
                  "paged_kv_cache_184_amd/csrc/decode_bf16_d128.hip",
                  "paged_kv_cache_184_amd/csrc/common.hpp",
                  "paged_kv_cache_184_amd/csrc/internal.hpp"]


def measured_traffic(alg_bytes: int):
    """HBM bytes per launch of the partial kernel from the committed counter
    runs, or None when the kernel sources changed since they were taken or the
    counters were taken on another workload (other algorithmic bytes)."""
    import hashlib

    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if int(rec["alg_bytes"]) != int(alg_bytes):
            return None
        h = hashlib.sha256()
        for rel in KERNEL_SOURCES:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest()[:16] != rec["source_hash"]:
            return None
        return int(round(float(rec["traffic_bytes"])))
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(db: DecodeBench, seconds: float):
    """Time the fp64 oracle on the headline workload until ``seconds`` of CPU
    work have run; report KV GB/s in the same unit as the GPU."""
    import oracle as O

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    import torch

    args = db.oracle_inputs()
    # the GPU's output for layer 0 of the same workload, checked against the
    # oracle's result from the timed calls below
    db.step(0)
    torch.cuda.synchronize()
    got = db.out[:1].float().cpu().numpy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref = O.decode_attention(args[0], args[1], args[2], 0, args[3], args[4], args[5], args[6])
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = db.kv_bytes() * reps / el / 1e9
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = None
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "host_cpus_usable": affinity,
            "blas_threads": int(threads),
            "gpu_vs_oracle_max_abs_err": float(np.abs(got - ref).max()),
            "sample": f"{reps} full oracle decode calls (B=1, ctx {db.b.seq_lens[0]}, 32 q heads) "
                      f"in {el:.1f} s; cores = BLAS threads (threadpoolctl), the only "
                      f"multi-threaded part of the oracle"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library is measured on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile:
        profile_run(args)
        return
    detail = {}
    head = None
    from paged_kv_cache_184_amd import workloads as W

    for ctx in args.ctx:
        db = DecodeBench(W.b1_decode(ctx, n_layers=8), split_tokens=args.split_tokens,
                         seed=184_002 + ctx)
        db.mode = "separate"
        sep_ms, _ = db.run(args.steps, args.warmup)
        db.mode = "fused"
        step_ms, host_s = db.run(args.steps, args.warmup)
        part_ms = db.run_partials(args.steps, args.warmup)
        entry = {
            "us_per_step": round(step_ms * 1e3, 2),
            "kv_gbs": round(db.kv_bytes() / (step_ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * db.step_bytes() / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "partial_kernel_us": round(part_ms * 1e3, 2),
            "partial_kernel_gbs": round(db.partial_kernel_bytes() / (part_ms * 1e-3) / 1e9, 1),
            "separate_calls_us_per_step": round(sep_ms * 1e3, 2),
            "splits": int(db.split.max_splits),
            "split_tokens": int(db.split.split_tokens),
        }
        if args.graph or ctx == args.headline:
            g_ms = db.run_graph(args.steps)
            entry["graph_us_per_step"] = round(g_ms * 1e3, 2)
            entry["graph_kv_gbs"] = round(db.kv_bytes() / (g_ms * 1e-3) / 1e9, 1)
        if ctx == args.headline:
            # spread: ten more timed regions of the same length, each between two events
            reps = sorted(db.run(args.steps, 2)[0] for _ in range(10))
            entry["us_per_step_repeats_p10_p50_p90"] = spread_us(reps)
            # the same step repeated on one layer: its K/V stay in the 256 MB
            # Infinity Cache between steps (labelled warm; not the headline)
            w_ms = db.run_warm_same_layer(args.steps, args.warmup)
            entry["warm_same_layer_us_per_step"] = round(w_ms * 1e3, 2)
            entry["warm_same_layer_kv_gbs"] = round(db.kv_bytes() / (w_ms * 1e-3) / 1e9, 1)
        detail[f"{ctx // 1024}k"] = entry
        print(f"# ctx {ctx}: {entry}", file=sys.stderr, flush=True)
        if ctx == args.headline:
            head = (db, step_ms, part_ms, host_s)
        else:
            del db
            torch.cuda.empty_cache()
    if not args.no_fp8 and head is not None:
        # the headline context on an FP8 (E4M3) pool: half the K/V bytes
        ctx = args.headline
        db8 = DecodeBench(W.b1_decode(ctx, n_layers=8), split_tokens=args.split_tokens,
                          seed=184_020 + ctx, kv="fp8")
        db8.mode = "fused"
        step8, _ = db8.run(args.steps, args.warmup)
        part8 = db8.run_partials(args.steps, args.warmup)
        entry = {
            "us_per_step": round(step8 * 1e3, 2),
            "kv_gbs": round(db8.kv_bytes() / (step8 * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * db8.step_bytes() / (step8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "partial_kernel_us": round(part8 * 1e3, 2),
            "partial_kernel_gbs": round(db8.partial_kernel_bytes() / (part8 * 1e-3) / 1e9, 1),
            "step_speedup_vs_bf16": round(head[1] / step8, 3),
            "splits": int(db8.split.max_splits), "split_tokens": int(db8.split.split_tokens),
        }
        detail[f"{ctx // 1024}k_fp8"] = entry
        print(f"# ctx {ctx} fp8: {entry}", file=sys.stderr, flush=True)
        del db8
        torch.cuda.empty_cache()
    if not args.no_batches:
        # batched decode workloads: ragged B=8 / B=32 with a shared 2048-token
        # prefix, B=64 lognormal lengths over a fragmented 2^21-slot pool (plus
        # the same lengths in 16-token pages, to separate the cost of the
        # token-granular scatter from the kernel's), and B=32 requests that all
        # share a 4096-token prefix (plain vs cascade attention)
        for name, make in (("ragged_b8", lambda: W.ragged_decode(8, n_layers=8)),
                           ("ragged_b32", lambda: W.ragged_decode(32, n_layers=8)),
                           ("large_b64", lambda: W.large_batch_decode(n_layers=4)),
                           ("large_b64_pages16",
                            lambda: W.large_batch_decode(n_layers=4, layout="pages16")),
                           ("shared_prefix_b32",
                            lambda: W.shared_prefix_decode(32, 4096, n_layers=8))):
            db = DecodeBench(make(), split_tokens=0, seed=184_010 + len(name))
            steps = max(10, args.steps // 4)
            db.mode = "fused"
            step_ms, _ = db.run(steps, max(2, args.warmup // 4))
            b = db.b
            detail[name] = {
                "batch": b.batch, "n_q_heads": b.n_q_heads, "sum_seq_lens": int(b.seq_lens.sum()),
                "max_seq_len": int(b.seq_lens.max()), "us_per_step": round(step_ms * 1e3, 2),
                "kv_gbs_logical": round(db.kv_bytes() / (step_ms * 1e-3) / 1e9, 1),
                "kv_gbs_unique": round(db.kv_bytes_unique() / (step_ms * 1e-3) / 1e9, 1),
                "pct_hbm_peak_unique": round(100 * (db.step_bytes() - db.kv_bytes() +
                                                    db.kv_bytes_unique()) /
                                             (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                "splits": int(db.split.max_splits), "split_tokens": int(db.split.split_tokens)}
            if db.cascade is not None:
                # attention alone: plain decode vs cascade (the shared prefix read
                # once per group); the split cap leaves room for prefix splits
                db.mode = "attn"
                attn_ms, _ = db.run(steps, 2)
                db.mode = "cascade"
                casc_ms, _ = db.run(steps, 2)
                detail[name].update({
                    "attn_us": round(attn_ms * 1e3, 2), "cascade_attn_us": round(casc_ms * 1e3, 2),
                    "cascade_kv_gbs_unique": round(db.kv_bytes_unique() / (casc_ms * 1e-3) / 1e9,
                                                   1),
                    "shared_group": len(db.b.shared_rows)})
            print(f"# {name}: {detail[name]}", file=sys.stderr, flush=True)
            del db
            torch.cuda.empty_cache()
    if not args.no_prefill:
        detail["new_token_steps"] = new_token_steps(max(20, args.steps // 4))
        print(f"# new-token steps: {detail['new_token_steps']}", file=sys.stderr, flush=True)
        pb = PrefillBench(n_layers=8, seed=184_004)
        p_step, p_ev, p_each = pb.run(max(20, args.steps // 5), args.warmup)
        p_attn = pb.run_kernels(max(20, args.steps // 5))
        tflops = pb.flops() / (p_attn * 1e-3) / 1e12
        detail["prefill"] = {
            "workload": "packed_prefill (8 requests, T_q=%d)" % pb.b.total_q,
            "us_per_step": round(p_step * 1e3, 1), "kernel_us": round(p_attn * 1e3, 1),
            "kernel_us_event_bracketed": round(p_ev * 1e3, 1),
            "kernel_us_event_bracketed_p10_p50_p90": spread_us(p_each),
            "gflop": round(pb.flops() / 1e9, 1), "tflops": round(tflops, 1),
            "mfma_util_pct": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 1)}
        print(f"# prefill: {detail['prefill']}", file=sys.stderr, flush=True)
        del pb
        torch.cuda.empty_cache()
        if not args.no_fp8:
            pb = PrefillBench(n_layers=8, seed=184_024, kv="fp8")
            p8_step, p8_ev, p8_each = pb.run(max(20, args.steps // 5), args.warmup)
            p8_attn = pb.run_kernels(max(20, args.steps // 5))
            detail["prefill_fp8"] = {
                "workload": "packed_prefill (8 requests, T_q=%d), E4M3 pools" % pb.b.total_q,
                "us_per_step": round(p8_step * 1e3, 1), "kernel_us": round(p8_attn * 1e3, 1),
                "kernel_us_event_bracketed": round(p8_ev * 1e3, 1),
                "kernel_us_event_bracketed_p10_p50_p90": spread_us(p8_each),
                "tflops": round(pb.flops() / (p8_attn * 1e-3) / 1e12, 1),
                "kernel_vs_bf16": round(p_attn / p8_attn, 3)}
            print(f"# prefill fp8: {detail['prefill_fp8']}", file=sys.stderr, flush=True)
            del pb
            torch.cuda.empty_cache()
    if head is None:
        raise SystemExit("--headline must be one of --ctx")
    db, step_ms, part_ms, host_s = head
    kv_gbs = db.kv_bytes() / (step_ms * 1e-3) / 1e9
    achieved = db.partial_kernel_bytes() / (part_ms * 1e-3) / 1e9
    line = {
        "metric": "paged decode attn KV GB/s (% HBM peak) + us/step, B=1..64, 1K-32K ctx",
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"b1_decode_{args.headline // 1024}k", "batch": 1,
                   "context": args.headline, "n_q_heads": 32, "n_kv_heads": 8, "head_dim": 128,
                   "kv_dtype": "bf16", "pool_slots": 40960, "layers_rotated": 8,
                   "slot_layout": "shuffled 16-token pages",
                   "split_tokens": int(db.split.split_tokens)},
        "pct_hbm_peak": detail[f"{args.headline // 1024}k"]["pct_hbm_peak"],
        "us_per_step": round(step_ms * 1e3, 2),
        "host_s_timed_region": round(host_s, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(db.partial_kernel_bytes()), "traffic_unit": "bytes per launch",
                     "algorithmic_bytes_per_launch": db.partial_kernel_bytes(),
                     "kernel": "decode_partial_kernel<bf16,128,4>"},
        "detail": detail,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(db, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
