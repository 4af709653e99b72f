"""Plain CPU fp64 restatement of paged-KV attention (page_size = 1).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Sources (AstrAI project pages):
  * "Inference" guide, section "KV Cache": the decode attention equation
    o_n = sum_j softmax(q_n . k_j / sqrt(d_k)) v_j, and the rule that cached
    K/V are already rotated (no rotation happens here).
  * "Inference" guide, section "KVCache System": the flat pool
    k_buffer/v_buffer [n_layers, size, n_kv_heads, head_dim], the
    req_to_token [num_reqs, max_ctx_len] slot table, the per-step fields
    req_pool_indices, seq_lens, out_cache_loc, max_len, kv_indptr, qo_indptr,
    and the raw indexing used to write (buffer[layer, out_cache_loc] = k) and
    to gather (buffer[layer, indices]).
  * "Inference" guide, section "Attention Backend": decode writes K/V first,
    then attends with req_to_token as a page table of one-token pages; prefill
    writes K/V, then attends over a ragged batch addressed by qo_indptr and
    kv_indptr.
  * Commit history of tests/inference/test_cache.py: indices are int32; the
    decode kernel produces per-split partial outputs and (max, sum) pairs
    into a workspace, which a merge pass combines.

Readings where the pages are silent:
  * GQA head map: query head h reads kv-head h // G with G = n_heads / n_kv_heads.
  * sm_scale is a parameter; the equation's value is 1/sqrt(head_dim).
  * Prefill is causal with the new tokens aligned to the end of the context:
    new token t of a request with prefix p sees keys 0 .. p + t.
  * A split partial is (m, l, o) with m = max score, l = sum exp(score - m),
    o = (sum exp(score - m) v) / l; empty splits are (-inf, 0, 0).

No blocking, fusion or reordering: every output row is the definition applied
to the rows the slot table names, in logical order.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step metadata ("Inference" guide, section "KVCache System": seq_lens,
# out_cache_loc, max_len, kv_indptr, qo_indptr; commit history: int32 indices)
# ---------------------------------------------------------------------------
def build_step(req_pool_indices: Sequence[int], seq_lens: Sequence[int],
               req_to_token: np.ndarray, q_lens: Optional[Sequence[int]] = None):
    """Per-step metadata for one batch.

    kv_indptr is the exclusive prefix sum of seq_lens, qo_indptr that of the
    per-request new-token counts (decode: one new token per request), and
    out_cache_loc lists, in qo order, the physical slot of every new token:
    request b's new tokens sit at the last q_len_b logical positions of its
    context, so token t maps to req_to_token[r_b, seq_len_b - q_len_b + t].
    prefill_order lists the requests longest context first (ties in batch
    order); it only schedules work.  position_ids lists, in qo order, the
    logical position seq_len_b - q_len_b + t of every new token: the row of
    the rotary table its query and key use ("Inference" guide, section
    "Rotary Embedding Backend").  Returns a dict of int32 arrays and ints.
    """
    B = len(seq_lens)
    if q_lens is None:
        q_lens = [1] * B
    kv_indptr = [0]
    qo_indptr = [0]
    locs: List[int] = []
    poss: List[int] = []
    for b in range(B):
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        ql = int(q_lens[b])
        kv_indptr.append(kv_indptr[-1] + L)
        qo_indptr.append(qo_indptr[-1] + ql)
        for t in range(ql):
            locs.append(int(req_to_token[r, L - ql + t]))
            poss.append(L - ql + t)
    # processing order for prefill: longest context first, ties in batch order
    order = sorted(range(B), key=lambda b: (-int(seq_lens[b]), b))
    return {
        "kv_indptr": np.array(kv_indptr, dtype=np.int32),
        "qo_indptr": np.array(qo_indptr, dtype=np.int32),
        "out_cache_loc": np.array(locs, dtype=np.int32),
        "position_ids": np.array(poss, dtype=np.int32),
        "prefill_order": np.array(order, dtype=np.int32),
        "max_len": max([int(x) for x in seq_lens], default=0),
        "max_q_len": max([int(x) for x in q_lens], default=0),
        "n_new": len(locs),
    }


def validate_step(size: int, num_reqs: int, max_ctx_len: int,
                  req_to_token: np.ndarray, req_pool_indices, seq_lens,
                  kv_indptr, qo_indptr, out_cache_loc) -> Tuple[bool, str]:
    """Checked-mode consistency test of one step's metadata.

    A step is well formed when every request row is in range, every context
    length is in [1, max_ctx_len], every new-token count is in [0, seq_len],
    the two indptr arrays are the exclusive prefix sums of the lengths,
    every slot the step will read or write lies in [0, size), the write
    slots are pairwise distinct, and each write slot is the slot table's
    entry for that token's logical position.
    """
    B = len(seq_lens)
    if len(req_pool_indices) != B or len(kv_indptr) != B + 1 or len(qo_indptr) != B + 1:
        return False, "array lengths"
    if kv_indptr[0] != 0 or qo_indptr[0] != 0:
        return False, "indptr start"
    if len(out_cache_loc) != qo_indptr[B]:
        return False, "out_cache_loc length"
    seen = set()
    for b in range(B):
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        if not (0 <= r < num_reqs):
            return False, f"request row {b}"
        if not (1 <= L <= max_ctx_len):
            return False, f"seq_len {b}"
        if int(kv_indptr[b + 1]) - int(kv_indptr[b]) != L:
            return False, f"kv_indptr {b}"
        ql = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        if not (0 <= ql <= L):
            return False, f"q_len {b}"
        for j in range(L):
            s = int(req_to_token[r, j])
            if not (0 <= s < size):
                return False, f"slot ({b},{j})"
        for t in range(ql):
            loc = int(out_cache_loc[int(qo_indptr[b]) + t])
            if not (0 <= loc < size):
                return False, f"out_cache_loc range ({b},{t})"
            if loc in seen:
                return False, f"out_cache_loc duplicate ({b},{t})"
            seen.add(loc)
            if loc != int(req_to_token[r, L - ql + t]):
                return False, f"out_cache_loc mismatch ({b},{t})"
    return True, "ok"


# ---------------------------------------------------------------------------
# KV write ("Inference" guide, section "KVCache System": buffer[layer,
# out_cache_loc] = k; section "Attention Backend": written before attention)
# ---------------------------------------------------------------------------
def kv_store(k_buffer: np.ndarray, v_buffer: np.ndarray, layer_id: int,
             out_cache_loc: Sequence[int], k_new: np.ndarray, v_new: np.ndarray):
    """Return copies of both pools with row i of k_new / v_new placed at slot
    out_cache_loc[i] of layer layer_id.  A pure copy: values keep their dtype
    and bits; nothing else in the pools changes."""
    k_out = k_buffer.copy()
    v_out = v_buffer.copy()
    for i, loc in enumerate(out_cache_loc):
        k_out[layer_id, int(loc)] = k_new[i]
        v_out[layer_id, int(loc)] = v_new[i]
    return k_out, v_out


# ---------------------------------------------------------------------------
# The attention equation ("Inference" guide, section "KV Cache")
# ---------------------------------------------------------------------------
def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float,
           n_keys: Optional[Sequence[int]] = None) -> np.ndarray:
    """o_r = sum_j softmax_j(sm_scale * q_r . k_j) v_j over keys j < n_keys[r].

    q_rows [R, d]; K, V [n, d] are the gathered key / value rows in logical
    order.  n_keys defaults to n for every row.  fp64; softmax is taken with
    the row maximum subtracted, which leaves its value unchanged.
    """
    q = _f64(q_rows)
    if q.ndim == 1:
        q = q[None, :]
    K = _f64(K)
    V = _f64(V)
    R = q.shape[0]
    n = K.shape[0]
    if n_keys is None:
        n_keys = [n] * R
    out = np.zeros((R, V.shape[1]), dtype=np.float64)
    scores = (q @ K.T) * float(sm_scale)  # [R, n]
    for r in range(R):
        nk = int(n_keys[r])
        if nk <= 0:
            continue
        s = scores[r, :nk]
        m = s.max()
        w = np.exp(s - m)
        out[r] = (w @ V[:nk]) / w.sum()
    return out


def _gather(buffer: np.ndarray, layer_id: int, slots: np.ndarray, hk: int) -> np.ndarray:
    # buffer[layer_id, indices] restricted to one kv-head
    return buffer[layer_id, slots, hk, :]


def decode(k_buffer, v_buffer, layer_id, req_to_token, req_pool_indices,
           seq_lens, q, sm_scale) -> np.ndarray:
    """Decode attention: one query row per request and head, attending to all
    seq_len cached keys of that request (the just-written token included),
    gathered through req_to_token.  q [B, H, dk] -> out [B, H, dv] fp64, dv the
    width of the value rows (keys and queries share dk)."""
    q = _f64(q)
    B, H, _ = q.shape
    Hk = k_buffer.shape[2]
    G = H // Hk
    dv = v_buffer.shape[3]   # outputs have the value rows' width
    out = np.zeros((B, H, dv), dtype=np.float64)
    for b in range(B):
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        slots = np.asarray(req_to_token[r, :L], dtype=np.int64)
        for hk in range(Hk):
            K = _gather(k_buffer, layer_id, slots, hk)
            V = _gather(v_buffer, layer_id, slots, hk)
            heads = list(range(hk * G, (hk + 1) * G))
            out[b, heads] = attend(q[b, heads], K, V, sm_scale)
    return out


def decode_pairs(k_buffer, v_buffer, layer_id, req_to_token, req_pool_indices,
                 seq_lens, q, sm_scale, pairs: Iterable[Tuple[int, int]]) -> np.ndarray:
    """decode() evaluated only at the (b, h) pairs listed; returns [n_pairs, d]."""
    q = _f64(q)
    H = q.shape[1]
    Hk = k_buffer.shape[2]
    G = H // Hk
    rows = []
    for b, h in pairs:
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        slots = np.asarray(req_to_token[r, :L], dtype=np.int64)
        hk = h // G
        K = _gather(k_buffer, layer_id, slots, hk)
        V = _gather(v_buffer, layer_id, slots, hk)
        rows.append(attend(q[b, h], K, V, sm_scale)[0])
    return np.stack(rows) if rows else np.zeros((0, v_buffer.shape[3]))


# ---------------------------------------------------------------------------
# Split partials and their merge (commit history of
# tests/inference/test_cache.py: per-split output and (max, sum) workspace
# buffers combined by a merge pass)
# ---------------------------------------------------------------------------
def split_partial(q_row, K, V, sm_scale, lo: int, hi: int):
    """(m, l, o) of one split covering logical keys [lo, hi).

    m = max score, l = sum_j exp(score_j - m), o = sum_j exp(score_j - m) v_j / l.
    An empty split is (-inf, 0, 0)."""
    d = V.shape[1]
    if hi <= lo:
        return NEG_INF, 0.0, np.zeros(d, dtype=np.float64)
    s = (_f64(K[lo:hi]) @ _f64(q_row)) * float(sm_scale)
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    o = (w @ _f64(V[lo:hi])) / l
    return float(m), float(l), o


def merge_partials(ms: Sequence[float], ls: Sequence[float], os: Sequence[np.ndarray]) -> np.ndarray:
    """Combine split partials: with M = max_s m_s and w_s = l_s exp(m_s - M),
    out = sum_s w_s o_s / sum_s w_s.  Empty splits (l_s = 0) weigh zero."""
    finite = [m for m, l in zip(ms, ls) if l > 0]
    d = len(os[0])
    if not finite:
        return np.zeros(d, dtype=np.float64)
    M = max(finite)
    num = np.zeros(d, dtype=np.float64)
    den = 0.0
    for m, l, o in zip(ms, ls, os):
        if l <= 0:
            continue
        w = l * math.exp(m - M)
        num += w * _f64(o)
        den += w
    return num / den


def decode_split(k_buffer, v_buffer, layer_id, req_to_token, req_pool_indices,
                 seq_lens, q, sm_scale, boundaries_for) -> np.ndarray:
    """Decode computed as per-split partials plus merge.

    boundaries_for(b) returns the split edges [0 = e_0 <= e_1 <= ... <= e_S =
    seq_len_b] for request b; split s covers logical keys [e_s, e_{s+1}).
    Mathematically equal to decode(); used to pin split independence."""
    q = _f64(q)
    B, H, _ = q.shape
    Hk = k_buffer.shape[2]
    G = H // Hk
    dv = v_buffer.shape[3]   # outputs have the value rows' width
    out = np.zeros((B, H, dv), dtype=np.float64)
    for b in range(B):
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        slots = np.asarray(req_to_token[r, :L], dtype=np.int64)
        edges = list(boundaries_for(b))
        assert edges[0] == 0 and edges[-1] == L
        for h in range(H):
            hk = h // G
            K = _gather(k_buffer, layer_id, slots, hk)
            V = _gather(v_buffer, layer_id, slots, hk)
            parts = [split_partial(q[b, h], K, V, sm_scale, lo, hi)
                     for lo, hi in zip(edges[:-1], edges[1:])]
            out[b, h] = merge_partials([p[0] for p in parts], [p[1] for p in parts],
                                       [p[2] for p in parts])
    return out


# ---------------------------------------------------------------------------
# Ragged paged prefill ("Inference" guide, section "Attention Backend")
# ---------------------------------------------------------------------------
def prefill_rows(k_buffer, v_buffer, layer_id, req_to_token, req_pool_indices,
                 seq_lens, qo_indptr, q, sm_scale, rows: Iterable[Tuple[int, int]],
                 causal: bool = True) -> np.ndarray:
    """Prefill output at selected (token, head) rows; token indexes the packed
    [n_new, H, d] query.  Request i owns tokens qo_indptr[i] .. qo_indptr[i+1]-1;
    its t-th new token sits at logical position p_i + t with
    p_i = seq_len_i - q_len_i and, when causal, sees keys 0 .. p_i + t.

    Rows that share a request and a kv-head are evaluated together, so that
    their keys are gathered once; each row still attends its own visible
    keys.  Results come back in the order of ``rows``."""
    q = _f64(q)
    H = q.shape[1]
    Hk = k_buffer.shape[2]
    G = H // Hk
    qo = [int(x) for x in qo_indptr]
    rows = [(int(tok), int(h)) for tok, h in rows]
    out = np.zeros((len(rows), v_buffer.shape[3]), dtype=np.float64)
    groups = {}
    for n, (tok, h) in enumerate(rows):
        i = int(np.searchsorted(qo, tok, side="right")) - 1
        groups.setdefault((i, h // G), []).append(n)
    for (i, hk), members in groups.items():
        r = int(req_pool_indices[i])
        L = int(seq_lens[i])
        ql = qo[i + 1] - qo[i]
        slots = np.asarray(req_to_token[r, :L], dtype=np.int64)
        K = _gather(k_buffer, layer_id, slots, hk)
        V = _gather(v_buffer, layer_id, slots, hk)
        qs, nks = [], []
        for n in members:
            tok, h = rows[n]
            t = tok - qo[i]
            nks.append((L - ql + t + 1) if causal else L)
            qs.append(q[tok, h])
        out[members] = attend(np.stack(qs), K, V, sm_scale, nks)
    return out


def prefill(k_buffer, v_buffer, layer_id, req_to_token, req_pool_indices,
            seq_lens, qo_indptr, q, sm_scale, causal: bool = True,
            row_block: int = 512) -> np.ndarray:
    """Prefill output for every new token and head: q [n_new, H, dk] -> [n_new, H, dv].

    Per request and head, the gathered K/V rows are shared by all of that
    request's new tokens; each row keeps its own visible-key count.  Rows are
    evaluated in groups of row_block only to bound memory."""
    q = _f64(q)
    n_new, H, _ = q.shape
    Hk = k_buffer.shape[2]
    G = H // Hk
    dv = v_buffer.shape[3]   # outputs have the value rows' width
    out = np.zeros((n_new, H, dv), dtype=np.float64)
    B = len(seq_lens)
    for i in range(B):
        r = int(req_pool_indices[i])
        L = int(seq_lens[i])
        q0 = int(qo_indptr[i])
        ql = int(qo_indptr[i + 1]) - q0
        if ql == 0:
            continue
        p = L - ql
        slots = np.asarray(req_to_token[r, :L], dtype=np.int64)
        for hk in range(Hk):
            K = _gather(k_buffer, layer_id, slots, hk)
            V = _gather(v_buffer, layer_id, slots, hk)
            for h in range(hk * G, (hk + 1) * G):
                for t0 in range(0, ql, row_block):
                    t1 = min(ql, t0 + row_block)
                    nk = [(p + t + 1) if causal else L for t in range(t0, t1)]
                    out[q0 + t0:q0 + t1, h] = attend(q[q0 + t0:q0 + t1, h], K, V,
                                                     sm_scale, nk)
    return out
