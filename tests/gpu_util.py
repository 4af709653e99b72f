"""Helpers for GPU parity tests: seeded inputs on the device, the oracle's own
host copy of what it needs (taken before any libpkv call), and the tolerances.

The oracle never sees a value the HIP path produced: host copies are made
with torch (copy / index_select) before the K/V write, and the oracle applies
the write itself."""

from __future__ import annotations

import sys
from typing import Iterable, Optional, Sequence

import numpy as np

import oracle
import workloads as W

# Tolerances stated for this path: fp32 inputs max-abs 1e-5; bf16 inputs
# (fp32 accumulate) |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise.
F32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_RTOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        worst = float(err.max(initial=0.0))
        assert worst <= F32_ATOL, f"{what}: max abs err {worst:.3e} > {F32_ATOL}"
        return worst
    bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, "
                           f"worst {float((err - bound).max()):.3e} over the bound")
    return float(err.max(initial=0.0))


def to_np(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


class HostView:
    """The oracle's copy of one layer, restricted to the slots some checked
    request reads; slots are renumbered 0 .. n-1 in sorted order."""

    def __init__(self, case: W.Case, t: dict, requests: Optional[Sequence[int]] = None):
        import torch
        reqs = range(case.batch) if requests is None else requests
        self.requests = list(reqs)
        parts = [case.req_to_token[int(case.req_pool_indices[b]), :int(case.seq_lens[b])]
                 for b in self.requests]
        self.slots = np.unique(np.concatenate(parts).astype(np.int64))
        idx = torch.from_numpy(self.slots).to(t["k_buffer"].device)
        layer = case.layer_id
        self.k = to_np(t["k_buffer"][layer].index_select(0, idx))[None]
        self.v = to_np(t["v_buffer"][layer].index_select(0, idx))[None]
        table = np.zeros_like(case.req_to_token)
        for b in self.requests:
            r = int(case.req_pool_indices[b])
            L = int(case.seq_lens[b])
            table[r, :L] = np.searchsorted(self.slots, case.req_to_token[r, :L])
        self.table = table
        self.q = to_np(t["q"])
        self.k_new = to_np(t["k_new"])
        self.v_new = to_np(t["v_new"])
        # step metadata on the real slots; the oracle then applies the step's
        # write to its own copy, for the checked requests' new tokens only
        md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token,
                               None if case.is_decode else case.q_lens)
        self.md = md
        qo = md["qo_indptr"]
        rows = [t for b in self.requests for t in range(int(qo[b]), int(qo[b + 1]))]
        locs = np.searchsorted(self.slots, md["out_cache_loc"][rows]).astype(np.int64)
        self.k, self.v = oracle.kv_store(self.k, self.v, 0, locs, self.k_new[rows],
                                         self.v_new[rows])

    def decode_pairs(self, case: W.Case, pairs: Iterable, sm_scale=None) -> np.ndarray:
        return oracle.decode_pairs(self.k, self.v, 0, self.table, case.req_pool_indices,
                                   case.seq_lens, self.q, case.sm_scale if sm_scale is None
                                   else sm_scale, pairs)

    def decode_all(self, case: W.Case) -> np.ndarray:
        return oracle.decode(self.k, self.v, 0, self.table, case.req_pool_indices,
                             case.seq_lens, self.q, case.sm_scale)

    def prefill_all(self, case: W.Case, causal=True) -> np.ndarray:
        return oracle.prefill(self.k, self.v, 0, self.table, case.req_pool_indices,
                              case.seq_lens, self.md["qo_indptr"], self.q, case.sm_scale,
                              causal=causal)

    def prefill_rows(self, case: W.Case, rows, causal=True) -> np.ndarray:
        return oracle.prefill_rows(self.k, self.v, 0, self.table, case.req_pool_indices,
                                   case.seq_lens, self.md["qo_indptr"], self.q, case.sm_scale,
                                   rows, causal=causal)
