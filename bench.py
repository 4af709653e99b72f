"""Benchmark of the paged-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the decode path over one batch: the K/V write of the
step's new token (kv_store), the split-KV paged decode and the merge.  The
headline workload is the Llama-3-8B-shaped single-request decode at the
longest sweep context (32 query / 8 kv heads, head_dim 128, bf16, 65536-slot
pool, 32 layers, seq_len 32768).  Successive steps attend successive layers
(31, 30, ..., 0, 31, ...) of the 32-layer pool, as a model forward does, so
each step's K/V come from HBM rather than from the 256 MB last-level cache.
The K timed steps are replayed from one captured HIP graph.

Printed as ONE JSON line (rank 0): value = algorithmic bytes per step /
time per step (GB/s).  Extra fields: the B=1 decode latency sweep
(1K..32K), the ragged causal prefill (TFLOP/s), the batched prefix-sharing
and long-context decodes (GB/s), the roofline of the dominant kernel
(paged_decode's split kernel, timed per launch with HIP events on its
stream), and the CPU fp64 oracle's throughput on a bounded sample.
"""

from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 matrix
METRIC = "paged decode achieved HBM GB/s (% peak) + prefill TFLOP/s; B=1 decode µs @1K–32K"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# launch plumbing: prebuilt ctypes arguments, direct calls into libpkv
# ---------------------------------------------------------------------------
class DecodeRunner:
    """One decode workload on the device with its C-ABI arguments prebuilt."""

    def __init__(self, case, fill_all_layers=True, num_splits=None, load_policy=0):
        import torch
        import workloads as W
        from paged_kv_attention_12_amd import api, binding as B
        self.torch = torch
        self.case = case
        self.lib = B.load()
        t = W.make_tensors(case, device="cuda", poison=not fill_all_layers)
        if fill_all_layers and case.n_layers > 1:
            g = torch.Generator(device="cuda")
            g.manual_seed(case.seed + 99)
            for layer in range(case.n_layers):
                if layer != case.layer_id:
                    W._fill_normal(t["k_buffer"][layer], g, case.k_scale)
                    W._fill_normal(t["v_buffer"][layer], g)
        self.t = t
        self.step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token,
                                   page_size=case.page_size)
        H, d = case.n_heads, case.head_dim
        self.num_splits = num_splits or B.pkv_decode_pick_splits(
            case.batch, case.n_kv_heads, H, self.step.max_len, self.step.total_len)
        self.ws = api.decode_workspace(case.batch, H, d, self.num_splits)
        self.ws_bytes = self.ws.numel() * 4
        self.out = torch.empty_like(t["q"])
        self.pool = B.make_pool(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.page_size,
                                load_policy)
        self.pool_ref = C.byref(self.pool)
        self.step_ref = C.byref(self.step.c)
        self.out_dtype = B.dtype_code(self.out)
        self.scale = case.sm_scale
        self.ptr = {k: t[k].data_ptr() for k in ("q", "k_new", "v_new")}
        self.loc = self.step.out_cache_loc.data_ptr()

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def store(self, layer, st):
        r = self.lib.pkv_kv_store(self.pool_ref, layer, self.ptr["k_new"], self.ptr["v_new"],
                                  self.loc, self.step.n_new, st)
        assert r == 0, r

    def decode(self, layer, st):
        r = self.lib.pkv_paged_decode(self.pool_ref, layer, self.step_ref, self.ptr["q"],
                                      self.case.n_heads, self.scale, self.num_splits,
                                      self.ws.data_ptr(), self.ws_bytes, st)
        assert r == 0, r

    def merge(self, st):
        r = self.lib.pkv_paged_decode_merge(self.case.batch, self.case.n_heads,
                                            self.case.head_dim, self.out_dtype, self.num_splits,
                                            self.ws.data_ptr(), self.ws_bytes,
                                            self.out.data_ptr(), st)
        assert r == 0, r

    def run_step(self, layer):
        st = self.stream()
        self.store(layer, st)
        self.decode(layer, st)
        self.merge(st)


    def layer_of(self, k):
        n = self.case.n_layers
        return (self.case.layer_id - k) % n

    # ---- algorithmic work ----
    def table_bytes(self):
        """Table entries the step needs: one slot id per token, or one page id
        per page of page_size tokens."""
        ps = self.case.page_size
        return 4 * int(sum((int(L) + ps - 1) // ps for L in self.case.seq_lens))

    def kernel_bytes(self):
        """Split kernel per launch: every key/value row of every request once,
        the table entries, and q."""
        c = self.case
        row = c.n_kv_heads * c.head_dim * 2
        L = int(c.seq_lens.sum())
        return L * 2 * row + self.table_bytes() + c.batch * c.n_heads * c.head_dim * 2

    def unique_kernel_bytes(self):
        c = self.case
        row = c.n_kv_heads * c.head_dim * 2
        uniq = len(c.referenced_slots())
        return uniq * 2 * row + int(c.seq_lens.sum()) * 4 + c.batch * c.n_heads * c.head_dim * 2

    def step_bytes(self):
        """kv_store (new rows read + written) + split kernel + merged output."""
        c = self.case
        row = c.n_kv_heads * c.head_dim * 2
        return self.kernel_bytes() + 4 * c.batch * row + c.batch * c.n_heads * c.head_dim * 2


class FusedDecodeRunner(DecodeRunner):
    """The same workload stepped through pkv_paged_decode_step: one launch for
    the K/V write, the split attention and the merge."""

    def __init__(self, case, fill_all_layers=True, num_splits=None):
        from paged_kv_attention_12_amd import api, binding as B
        super().__init__(case, fill_all_layers)
        c = self.case
        self.num_splits = num_splits or B.pkv_decode_step_pick_splits(
            c.batch, c.n_kv_heads, c.n_heads, self.step.max_len, self.step.total_len)
        self.ws = api.decode_workspace(c.batch, c.n_heads, c.head_dim, self.num_splits)
        self.ws_bytes = self.ws.numel() * 4
        self.sync = api.decode_sync(c.batch, c.n_heads)

    def run_step(self, layer):
        r = self.lib.pkv_paged_decode_step(
            self.pool_ref, layer, self.step_ref, self.ptr["q"], self.ptr["k_new"],
            self.ptr["v_new"], self.case.n_heads, self.scale, self.num_splits, self.ws.data_ptr(),
            self.ws_bytes, self.sync.data_ptr(), self.sync.numel(), self.out.data_ptr(),
            self.stream())
        assert r == 0, r


class StoredDecodeRunner(DecodeRunner):
    """The same workload stepped through pkv_paged_decode_store: two launches,
    the split kernel with the new token's K/V write folded in, then the merge.
    decode() (used for the split-kernel timing) is the plain split kernel."""

    def run_step(self, layer):
        r = self.lib.pkv_paged_decode_store(
            self.pool_ref, layer, self.step_ref, self.ptr["q"], self.ptr["k_new"],
            self.ptr["v_new"], self.case.n_heads, self.scale, self.num_splits, self.ws.data_ptr(),
            self.ws_bytes, self.out.data_ptr(), self.stream())
        assert r == 0, r


class SharedDecodeRunner(DecodeRunner):
    """The same workload stepped through pkv_paged_decode_shared: each prefix
    group's shared keys read once (groups from pkv_decode_prefix_groups on the
    host table), the requests' own keys with the new-token K/V write, the
    merge.  decode() is the whole shared step (three launches)."""

    def __init__(self, case, fill_all_layers=True, min_prefix=256):
        from paged_kv_attention_12_amd import api, binding as B
        super().__init__(case, fill_all_layers)
        c = self.case
        self.groups = api.PrefixGroups(self.step, c.req_pool_indices, c.seq_lens,
                                       c.req_to_token, min_prefix=min_prefix)
        self.num_splits, self.prefix_splits = self.groups.pick_splits(self.step, c.n_kv_heads,
                                                                      c.n_heads)
        self.ws = api.decode_workspace(c.batch, c.n_heads, c.head_dim,
                                       self.num_splits + self.prefix_splits)
        self.ws_bytes = self.ws.numel() * 4
        self.groups_ref = C.byref(self.groups.c)

    def run_step(self, layer):
        r = self.lib.pkv_paged_decode_shared(
            self.pool_ref, layer, self.step_ref, self.groups_ref, self.ptr["q"], self.ptr["k_new"],
            self.ptr["v_new"], self.case.n_heads, self.scale, self.num_splits, self.prefix_splits,
            self.ws.data_ptr(), self.ws_bytes, self.out.data_ptr(), self.stream())
        assert r == 0, r

    def decode(self, layer, st):
        self.run_step(layer)


def graph_steps(runner, n, start=0):
    """Capture n consecutive steps (layer rotation from step `start`) in one graph."""
    torch = runner.torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        runner.run_step(runner.layer_of(start))  # touch everything once outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for k in range(start, start + n):
            runner.run_step(runner.layer_of(k))
    torch.cuda.synchronize()
    return g


def timed_graph(runner, steps, warmup):
    """W warm-up steps, then exactly K steps replayed from one graph, with a
    device synchronize on both sides of the timed replay."""
    torch = runner.torch
    gw = graph_steps(runner, max(1, warmup))
    gk = graph_steps(runner, steps, start=max(1, warmup))
    gw.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gk.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # the graph's result equals an eager run of the same last step
    ref = runner.out.clone()
    runner.run_step(runner.layer_of(max(1, warmup) + steps - 1))
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(ref, runner.out))
    del gw, gk
    return dt / steps, graph_ok


def kernel_event_times(runner, launches, reps=3):
    """Average duration of the split kernel: HIP events on its stream bracket
    the replay of a graph holding `launches` back-to-back split-kernel
    launches (successive layers); returns one average per replay."""
    torch = runner.torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        runner.run_step(runner.layer_of(0))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st = runner.stream()
        for k in range(launches):
            runner.decode(runner.layer_of(k), st)
    torch.cuda.synchronize()
    g.replay()  # warm
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(cur)
        g.replay()
        b.record(cur)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e-3 / launches)
    del g
    return np.array(out)


def kernel_launch_spread(runner, launches=100, warm=False):
    """Per-launch durations of the split kernel: a HIP event pair on its stream
    around each of `launches` eager launches; successive layers (cold: K/V
    from HBM) or, with warm, the same layer every time (its 134 MB stay in the
    last-level cache).  Returns (p10, p50, p90) in seconds."""
    torch = runner.torch
    st = runner.stream()
    cur = torch.cuda.current_stream()
    for k in range(3):
        runner.decode(runner.layer_of(0 if warm else k), st)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    for k, (a, b) in enumerate(ev):
        a.record(cur)
        runner.decode(runner.layer_of(0 if warm else k), st)
        b.record(cur)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    return tuple(float(np.percentile(t, q)) for q in (10, 50, 90))


def flushed_step_times(runner, n=20, flush_bytes=1 << 30, write=False):
    """Per-step durations with the caches flushed first: before each step a
    1 GiB device buffer (more than the L2s and the last-level cache hold) is
    read by a sum, which leaves the caches holding clean lines of it, then a
    HIP event pair on the step's stream brackets one step (successive
    layers).  With write, the buffer is written instead: the step then also
    pays for writing the flush's dirty lines back to HBM.  Returns (p10,
    p50, p90) in seconds."""
    torch = runner.torch
    scratch = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda")
    cur = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    runner.run_step(runner.layer_of(0))
    for k, (a, b) in enumerate(ev):
        if write:
            scratch.fill_(k)
        else:
            scratch.sum()
        a.record(cur)
        runner.run_step(runner.layer_of(k))
        b.record(cur)
    torch.cuda.synchronize()
    del scratch
    t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    return tuple(float(np.percentile(t, q)) for q in (10, 50, 90))


# ---------------------------------------------------------------------------
# graph-captured decode loop: one token of a 32-layer forward per replay
# ---------------------------------------------------------------------------
def bench_decode_loop(L, tokens=8, fused=True):
    """Per token, for every layer (31 .. 0): the rotary embedding of the new
    token with its K/V write, the split attention and the merge; then the
    in-place advance of the step metadata (seq_lens, position_ids,
    out_cache_loc, kv_indptr).  fused: the rotation and the write inside the
    split kernel (pkv_paged_decode_rope_store, two launches a layer); else
    pkv_rope_kv_store, then the split and merge launches (three a layer).
    Captured once, replayed token after token.  The request starts at
    position L - tokens - 1, so the table row (L positions) covers every
    token and the last advance.  Also timed: the same launches issued
    eagerly from Python through the C ABI."""
    import torch
    import workloads as W
    from paged_kv_attention_12_amd import api
    r = DecodeRunner(W.llama_b1_decode(L))
    c = r.case
    t = r.t
    p0 = L - tokens - 1
    step = api.DeviceStep(c.req_pool_indices, np.array([p0 + 1], np.int32), c.req_to_token,
                          max_len=L)
    freqs = W.rope_table(L, c.head_dim, device="cuda")
    ns = r.num_splits
    ws = api.decode_workspace(1, c.n_heads, c.head_dim, ns)
    q_rot = torch.empty_like(t["q"])
    out = torch.empty_like(t["q"])
    kb, vb, tab = t["k_buffer"], t["v_buffer"], t["req_to_token"]

    def one_token():
        for layer in range(c.n_layers - 1, -1, -1):
            if fused:
                api.rope_decode_step(kb, vb, tab, layer, step, t["q"], t["k_new"], t["v_new"],
                                     freqs, c.sm_scale, num_splits=ns, workspace=ws, out=out)
                continue
            api.rope_kv_store(kb, vb, tab, layer, step, t["q"], t["k_new"], t["v_new"], freqs,
                              q_out=q_rot)
            api.decode_step(kb, vb, tab, layer, step, q_rot, None, None, c.sm_scale,
                            num_splits=ns, workspace=ws, out=out, write_kv=False)
        api.advance_decode(kb, vb, tab, step)

    def reset():
        step.seq_lens.fill_(p0 + 1)
        step.position_ids.fill_(p0)
        step.kv_indptr[1:].fill_(p0 + 1)
        step.out_cache_loc.fill_(int(c.req_to_token[int(c.req_pool_indices[0]), p0]))

    # eager: every launch from Python
    one_token()
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(tokens):
        one_token()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / tokens
    # graph: one token's launches captured once (nothing runs while capturing)
    reset()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            one_token()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g.replay()  # warm: the first token
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(tokens):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / tokens
    advanced = int(step.seq_lens.item()) == p0 + 1 + tokens
    del g, r
    torch.cuda.empty_cache()
    n = c.n_layers
    return {"form": "rope_in_step" if fused else "rope_then_step", "tokens": tokens,
            "layers": n, "context": [p0 + 1, p0 + tokens],
            "graph_us_per_token": graph * 1e6, "graph_us_per_layer": graph / n * 1e6,
            "eager_us_per_token": eager * 1e6, "eager_us_per_layer": eager / n * 1e6,
            "metadata_advanced": advanced}


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def prefill_flops(case):
    d, H = case.head_dim, case.n_heads
    tot = 0
    for L, q in zip(case.seq_lens.astype(np.int64), case.q_lens.astype(np.int64)):
        p = L - q
        tot += q * p + q * (q + 1) // 2
    return 4 * d * H * int(tot)


def bench_prefill(reps=20, case=None):
    import torch
    import workloads as W
    from paged_kv_attention_12_amd import api, binding as B
    case = case or W.ragged_prefill()
    t = W.make_tensors(case, device="cuda", poison=False)
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens,
                          page_size=case.page_size)
    step.set_prefill_blocks(case.n_heads, case.n_kv_heads)   # launch schedule of this step
    out = torch.empty_like(t["q"])
    lib = B.load()
    pool = B.make_pool(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.page_size)
    st = torch.cuda.current_stream().cuda_stream
    cur = torch.cuda.current_stream()

    def store():
        assert lib.pkv_kv_store(C.byref(pool), 0, t["k_new"].data_ptr(), t["v_new"].data_ptr(),
                                step.out_cache_loc.data_ptr(), step.n_new, st) == 0

    def attend():
        assert lib.pkv_paged_prefill(C.byref(pool), 0, C.byref(step.c), t["q"].data_ptr(),
                                     case.n_heads, case.sm_scale, 1, out.data_ptr(), st) == 0

    freqs = W.rope_table(case.max_ctx_len, case.head_dim, device="cuda")
    q_rot = torch.empty_like(t["q"])

    def rope():
        assert lib.pkv_rope_kv_store(C.byref(pool), 0, t["q"].data_ptr(), q_rot.data_ptr(),
                                     case.n_heads, t["k_new"].data_ptr(), t["v_new"].data_ptr(),
                                     step.position_ids.data_ptr(), freqs.data_ptr(),
                                     freqs.shape[0], step.out_cache_loc.data_ptr(), step.n_new,
                                     st) == 0

    for _ in range(3):
        store()
        attend()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b, c in ev:
        a.record(cur)
        store()
        b.record(cur)
        attend()
        c.record(cur)
    torch.cuda.synchronize()
    t_store = np.array([a.elapsed_time(b) for a, b, _ in ev]) * 1e-3
    t_pre = np.array([b.elapsed_time(c) for _, b, c in ev]) * 1e-3
    for _ in range(3):
        rope()
    torch.cuda.synchronize()
    evr = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evr:
        a.record(cur)
        rope()
        b.record(cur)
    torch.cuda.synchronize()
    t_rope = float(np.median([a.elapsed_time(b) for a, b in evr])) * 1e-3
    n = step.n_new
    # q, k, v rows read and written once, positions and slots read, one
    # table row (head_dim / 2 [cos, sin] f32 pairs) per token
    rope_bytes = (2 * n * (case.n_heads + 2 * case.n_kv_heads) * case.head_dim * 2 + 8 * n
                  + n * case.head_dim * 4)
    flops = prefill_flops(case)
    med = float(np.median(t_pre))
    row = case.n_kv_heads * case.head_dim * 2
    return {
        "workload": "ragged_causal_prefill_16req" + (
            f"_pages{case.page_size}" if case.page_size > 1 else ""),
        "n_new_tokens": int(case.q_lens.sum()), "kv_tokens": int(case.seq_lens.sum()),
        "flops": flops, "prefill_ms": med * 1e3, "prefill_ms_p10_p90":
            [float(np.percentile(t_pre, 10)) * 1e3, float(np.percentile(t_pre, 90)) * 1e3],
        "tflops": flops / med / 1e12, "frac_of_bf16_peak": flops / med / 1e12 / BF16_PEAK_TFLOPS,
        "kv_store_ms": float(np.median(t_store)) * 1e3,
        "kv_store_gbps": 4 * step.n_new * row / float(np.median(t_store)) / 1e9,
        "rope_kv_store_ms": t_rope * 1e3, "rope_kv_store_bytes": rope_bytes,
        "rope_kv_store_gbps": rope_bytes / t_rope / 1e9,
        "rope_kv_store_frac_of_hbm_peak": rope_bytes / t_rope / 1e9 / HBM_PEAK_GBPS,
    }


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the headline workload)
# ---------------------------------------------------------------------------
def _threads():
    """(os.cpu_count(), BLAS threads numpy uses)."""
    n = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = n
    return int(n), int(blas)


def _host_layer(t, case, slots):
    """Host float32 copies of the attended layer's rows at `slots` (sorted),
    and the request table renumbered onto them."""
    import torch
    idx = torch.from_numpy(slots).cuda()
    layer = case.layer_id
    k = t["k_buffer"][layer].index_select(0, idx).float().cpu().numpy()[None]
    v = t["v_buffer"][layer].index_select(0, idx).float().cpu().numpy()[None]
    table = np.zeros_like(case.req_to_token)
    for b in range(case.batch):
        r = int(case.req_pool_indices[b])
        L = int(case.seq_lens[b])
        table[r, :L] = np.searchsorted(slots, case.req_to_token[r, :L])
    return k, v, table


def cpu_baseline(runner, budget_s=10.0):
    """The oracle on the headline decode step: whole steps (write + attention
    of every head), repeated for about budget_s."""
    import oracle
    case = runner.case
    k, v, table = _host_layer(runner.t, case, case.referenced_slots())
    q = runner.t["q"].float().cpu().numpy()
    kn = runner.t["k_new"].float().cpu().numpy()
    vn = runner.t["v_new"].float().cpu().numpy()
    n_cpu, blas = _threads()
    n = 0
    t0 = time.perf_counter()
    while True:
        md = oracle.build_step(case.req_pool_indices, case.seq_lens, table)
        k2, v2 = oracle.kv_store(k, v, 0, md["out_cache_loc"], kn, vn)
        oracle.decode(k2, v2, 0, table, case.req_pool_indices, case.seq_lens, q, case.sm_scale)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or n >= 200:
            break
    per = dt / n
    return {"value": runner.step_bytes() / per / 1e9, "unit": "GB/s", "cores": blas,
            "kind": "oracle", "os_cpu_count": n_cpu, "blas_threads": blas,
            "sample": f"{n} full decode steps of {case.name} (kv_store + attention of all "
                      f"{case.n_heads} heads over {int(case.seq_lens[0])} keys), numpy fp64, "
                      f"{per * 1e3:.1f} ms/step"}


def cpu_baseline_long_context(runner, budget_s=8.0):
    """The oracle on the long-context decode: (request, query head) rows of
    one kv-head group at a time (all 131072 keys each), repeated over
    requests for about budget_s; reported on the K/V bytes those rows read."""
    import oracle
    case = runner.case
    G = case.n_heads // case.n_kv_heads
    n_cpu, blas = _threads()
    rows = 0
    groups = 0
    t_work = 0.0
    for b in range(case.batch):
        slots = np.unique(case.req_to_token[int(case.req_pool_indices[b]),
                                            :int(case.seq_lens[b])].astype(np.int64))
        k, v, table = _host_layer(runner.t, case, slots)
        q = runner.t["q"][b:b + 1].float().cpu().numpy()
        for hk in range(case.n_kv_heads):
            pairs = [(0, hk * G + g) for g in range(G)]
            t0 = time.perf_counter()
            oracle.decode_pairs(k, v, 0, table, case.req_pool_indices[b:b + 1],
                                case.seq_lens[b:b + 1], q, case.sm_scale, pairs)
            t_work += time.perf_counter() - t0
            rows += G
            groups += 1
            if t_work >= budget_s:
                break
        del k, v
        if t_work >= budget_s:
            break
    L = int(case.seq_lens[0])
    sampled = groups * L * (2 * case.head_dim * 2 + 4)   # K+V row of one kv-head + slot id
    return {"value": sampled / t_work / 1e9, "unit": "GB/s", "cores": blas, "kind": "oracle",
            "os_cpu_count": n_cpu, "blas_threads": blas,
            "sample": f"{rows} (request, head) rows = {groups} kv-head groups x {L} keys of "
                      f"{case.name}, numpy fp64, {t_work:.1f} s; rate on the K/V bytes they read",
            "full_call_s_extrapolated": t_work / groups * case.batch * case.n_kv_heads}


def cpu_baseline_prefill(budget_s=8.0, seed=7):
    """The oracle on the ragged prefill: all query heads of random new tokens
    of every request, in rounds, for about budget_s; reported in TFLOP/s on
    the unmasked (query, key) pairs of the rows evaluated."""
    import oracle
    import workloads as W
    case = W.ragged_prefill()
    t = W.make_tensors(case, device="cuda", poison=False)
    k, v, table = _host_layer(t, case, case.referenced_slots())
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, table, case.q_lens)
    k, v = oracle.kv_store(k, v, 0, md["out_cache_loc"], t["k_new"].float().cpu().numpy(),
                           t["v_new"].float().cpu().numpy())
    q = t["q"].float().cpu().numpy()
    del t
    qo = md["qo_indptr"]
    rng = np.random.default_rng(seed)
    n_cpu, blas = _threads()
    d, H = case.head_dim, case.n_heads
    flops = 0
    n_rows = 0
    t_work = 0.0
    while t_work < budget_s:
        rows = []
        for i in range(case.batch):
            q0, q1 = int(qo[i]), int(qo[i + 1])
            if q1 == q0:
                continue
            tok = int(rng.integers(q0, q1))
            p = int(case.seq_lens[i]) - (q1 - q0)
            flops += 4 * d * H * (p + tok - q0 + 1)
            rows += [(tok, h) for h in range(H)]
        t0 = time.perf_counter()
        oracle.prefill_rows(k, v, 0, table, case.req_pool_indices, case.seq_lens, qo, q,
                            case.sm_scale, rows)
        t_work += time.perf_counter() - t0
        n_rows += len(rows)
    rate = flops / t_work
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "os_cpu_count": n_cpu, "blas_threads": blas,
            "sample": f"{n_rows} (token, head) rows of ragged_causal_prefill_16req (one random "
                      f"new token per request per round, all {H} heads), numpy fp64, "
                      f"{t_work:.1f} s; FLOPs of their unmasked (query, key) pairs",
            "full_call_s_extrapolated": prefill_flops(case) / rate}


# ---------------------------------------------------------------------------
def counters_for(kernel_src_hash):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "decode_split_mfma_llama_b1_L32768.counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("source_sha256") != kernel_src_hash:
        return None
    return d.get("traffic_bytes_per_launch")


def src_hash():
    h = hashlib.sha256()
    for f in ("decode.hip", "device.hpp"):
        h.update(open(os.path.join(ROOT, "paged_kv_attention_12_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true",
                    help="skip the sweep, prefill and the other decode workloads")
    ap.add_argument("--kernel-launches", type=int, default=64)
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the ragged prefill measurement and print it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        log(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
            "(the path is single-GPU; see the sharding design notes)")
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py runs as a single process on one GPU")
        sys.exit(2)

    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    from paged_kv_attention_12_amd import binding as B
    B.load()

    if args.copy_calibration:
        # A plain copy of known size: its HBM counters give the scale between
        # counter units and bytes on this machine.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies (read 1 GiB + write 1 GiB each)")
        del src, dst

    if args.only_prefill:
        print(json.dumps(bench_prefill()), flush=True)
        return

    # ---- headline: Llama-3-8B-shaped B=1 decode, seq_len 32768 ----
    L_head = W.LLAMA_SWEEP[-1]
    log(f"headline: llama B=1 decode L={L_head}")
    head = StoredDecodeRunner(W.llama_b1_decode(L_head))
    sec_per_step, graph_ok = timed_graph(head, args.steps, args.warmup)
    step_bytes = head.step_bytes()
    value = step_bytes / sec_per_step / 1e9
    kt = kernel_event_times(head, args.kernel_launches)
    k_avg = float(kt.mean())
    k_bytes = head.kernel_bytes()
    achieved = k_bytes / k_avg / 1e9
    traffic = counters_for(src_hash())
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                "kernel": "decode_split_mfma_kernel", "bytes_per_launch": k_bytes,
                "avg_launch_us": k_avg * 1e6, "launches": int(len(kt)) * args.kernel_launches,
                "timing": "HIP events around a graph of back-to-back split-kernel launches",
                "num_splits": head.num_splits,
                "row_loads": ("non-temporal" if B.pkv_decode_load_kind(
                    head.pool, 1, head.step.max_len) == 1 else "cached") + " (PKV_LOAD_AUTO)"}
    log(f"  step {sec_per_step * 1e6:.1f} us  {value:.0f} GB/s; split kernel {k_avg * 1e6:.1f} us "
        f"{achieved:.0f} GB/s ({achieved / HBM_PEAK_GBPS:.1%})  graph_ok={graph_ok}")
    cold = kernel_launch_spread(head)
    warm = kernel_launch_spread(head, warm=True)
    roofline["eager_launch_us_p10_p50_p90"] = [x * 1e6 for x in cold]
    roofline["warm_launch_us_p10_p50_p90"] = [x * 1e6 for x in warm]
    log(f"  split kernel per eager launch p10/p50/p90: {cold[0] * 1e6:.1f} / {cold[1] * 1e6:.1f} / "
        f"{cold[2] * 1e6:.1f} us; warm (one layer, cached): {warm[1] * 1e6:.1f} us")

    extra = {}
    cpu_long = None
    if not args.only_headline:
        sweep = {}
        for L in W.LLAMA_SWEEP:
            r = head if L == L_head else StoredDecodeRunner(W.llama_b1_decode(L))
            spp, ok = timed_graph(r, 50, 5)
            kt_l = kernel_event_times(r, 32, reps=2)
            fl = flushed_step_times(r)
            sweep[str(L)] = {"step_us": spp * 1e6, "split_kernel_us": float(kt_l.mean()) * 1e6,
                             "step_gbps": r.step_bytes() / spp / 1e9,
                             "split_kernel_gbps": r.kernel_bytes() / float(kt_l.mean()) / 1e9,
                             "flushed_step_us_p10_p50_p90": [x * 1e6 for x in fl],
                             "num_splits": r.num_splits, "graph_ok": ok}
            if r is not head:
                del r
                torch.cuda.empty_cache()
            r3 = DecodeRunner(W.llama_b1_decode(L))
            sp3, ok3 = timed_graph(r3, 50, 5)
            sweep[str(L)].update({"three_launch_step_us": sp3 * 1e6, "three_launch_graph_ok": ok3})
            del r3
            torch.cuda.empty_cache()
            rf = FusedDecodeRunner(W.llama_b1_decode(L))
            spf, okf = timed_graph(rf, 50, 5)
            sweep[str(L)].update({"fused_step_us": spf * 1e6, "fused_num_splits": rf.num_splits,
                                  "fused_graph_ok": okf})
            del rf
            torch.cuda.empty_cache()
            log(f"  B=1 L={L}: step {spp * 1e6:.1f} us (three launches {sp3 * 1e6:.1f} us, "
                f"one launch {spf * 1e6:.1f} us), split kernel {kt_l.mean() * 1e6:.1f} us; "
                f"caches flushed before each step: median {fl[1] * 1e6:.1f} us")
        extra["b1_decode_us"] = {L: v["step_us"] for L, v in sweep.items()}
        extra["b1_decode_three_launch_step_us"] = {L: v["three_launch_step_us"]
                                                   for L, v in sweep.items()}
        extra["b1_decode_fused_step_us"] = {L: v["fused_step_us"] for L, v in sweep.items()}
        extra["b1_decode_sweep"] = sweep

        log("batched prefix-sharing decode")
        rb = DecodeRunner(W.batched_prefix_decode())
        spp, ok = timed_graph(rb, 20, 3)
        ktb = kernel_event_times(rb, 8, reps=2)
        extra["batched_prefix_decode"] = {
            "step_us": spp * 1e6, "split_kernel_us": float(ktb.mean()) * 1e6,
            "gbps_unique": rb.unique_kernel_bytes() / float(ktb.mean()) / 1e9,
            "gbps_logical": rb.kernel_bytes() / float(ktb.mean()) / 1e9,
            "num_splits": rb.num_splits, "graph_ok": ok}
        del rb
        torch.cuda.empty_cache()
        rs = SharedDecodeRunner(W.batched_prefix_decode())
        sps, oks = timed_graph(rs, 20, 3)
        kts = kernel_event_times(rs, 8, reps=2)
        extra["batched_prefix_decode"]["shared_prefix"] = {
            "step_us": sps * 1e6, "step_event_us": float(kts.mean()) * 1e6,
            "gbps_unique": rs.unique_kernel_bytes() / sps / 1e9,
            "frac_of_hbm_peak_unique": rs.unique_kernel_bytes() / sps / 1e9 / HBM_PEAK_GBPS,
            "gbps_logical": rs.kernel_bytes() / sps / 1e9,
            "num_splits": rs.num_splits, "prefix_splits": rs.prefix_splits,
            "n_groups": rs.groups.n_groups, "graph_ok": oks,
            "step": "pkv_paged_decode_shared: shared keys once per group + own keys with the "
                    "K/V write + merge"}
        log(f"  shared-prefix step {sps * 1e6:.1f} us ({rs.groups.n_groups} groups), plain step "
            f"{extra['batched_prefix_decode']['step_us']:.1f} us")
        del rs
        torch.cuda.empty_cache()

        log("long-context decode")
        # its table is a permutation of the pool: no slot is shared between
        # requests, so the rows are read once per step (PKV_LOAD_STREAM)
        rl = DecodeRunner(W.long_context_decode(), load_policy=2)
        spp, ok = timed_graph(rl, 10, 2)
        ktl = kernel_event_times(rl, 4, reps=2)
        extra["long_context_decode"] = {
            "step_us": spp * 1e6, "split_kernel_us": float(ktl.mean()) * 1e6,
            "gbps": rl.kernel_bytes() / float(ktl.mean()) / 1e9,
            "frac_of_hbm_peak": rl.kernel_bytes() / float(ktl.mean()) / 1e9 / HBM_PEAK_GBPS,
            "num_splits": rl.num_splits, "graph_ok": ok,
            "row_loads": "non-temporal (PKV_LOAD_STREAM: no slot shared between requests)"}
        if not args.no_cpu_baseline:
            log("cpu oracle baseline: long-context decode sample")
            cpu_long = cpu_baseline_long_context(rl)
        del rl
        torch.cuda.empty_cache()

        log("ragged prefill")
        extra["prefill"] = bench_prefill()
        log(f"  prefill {extra['prefill']['prefill_ms']:.3f} ms "
            f"{extra['prefill']['tflops']:.1f} TFLOP/s")

        log("graph-captured decode loop")
        extra["decode_loop"] = {str(L): bench_decode_loop(L) for L in (1024, 32768)}
        extra["decode_loop_rope_then_step"] = {str(L): bench_decode_loop(L, fused=False)
                                               for L in (1024, 32768)}
        for key in ("decode_loop", "decode_loop_rope_then_step"):
            for L, v in extra[key].items():
                log(f"  {v['form']} L={L}: graph {v['graph_us_per_layer']:.1f} us/layer, eager "
                    f"{v['eager_us_per_layer']:.1f} us/layer, advanced={v['metadata_advanced']}")

        # the same workloads on pools of 64-token pages
        log("paged pools (64-token pages)")
        rp = StoredDecodeRunner(W.llama_b1_decode_paged(L_head, page_size=64))
        spp, ok = timed_graph(rp, 50, 5)
        ktp = kernel_event_times(rp, 32, reps=2)
        pre_p = bench_prefill(case=W.ragged_prefill_paged(64))
        extra["pages64"] = {
            "b1_decode_L32768": {
                "step_us": spp * 1e6, "split_kernel_us": float(ktp.mean()) * 1e6,
                "step_gbps": rp.step_bytes() / spp / 1e9,
                "split_kernel_gbps": rp.kernel_bytes() / float(ktp.mean()) / 1e9,
                "frac_of_hbm_peak": rp.kernel_bytes() / float(ktp.mean()) / 1e9 / HBM_PEAK_GBPS,
                "num_splits": rp.num_splits, "graph_ok": ok},
            "prefill": {k: pre_p[k] for k in ("workload", "flops", "prefill_ms", "tflops",
                                              "frac_of_bf16_peak")},
        }
        del rp
        torch.cuda.empty_cache()
        log(f"  B=1 L={L_head} pages of 64: step {spp * 1e6:.1f} us, split kernel "
            f"{ktp.mean() * 1e6:.1f} us; prefill {pre_p['prefill_ms']:.3f} ms "
            f"{pre_p['tflops']:.1f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu oracle baseline: headline decode")
        cpu = cpu_baseline(head)
        if not args.only_headline:
            cpu["long_context_decode"] = cpu_long
            log("cpu oracle baseline: prefill sample")
            cpu["prefill"] = cpu_baseline_prefill()

    rec = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": sec_per_step * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3_8b_shape_b1_decode_L{L_head}", "batch": 1,
                   "n_heads": 32, "n_kv_heads": 8, "head_dim": 128, "seq_len": L_head,
                   "pool_slots": 65536, "n_layers": 32,
                   "step": "paged_decode_store (split attention with the new-token K/V write) "
                           "+ merge",
                   "layer_rotation": "31,30,...,0", "timing": "one HIP graph of K steps",
                   "num_splits": head.num_splits, "bytes_per_step": step_bytes},
        "hbm_frac": value / HBM_PEAK_GBPS,
        "graph_replay_matches_eager": graph_ok,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
