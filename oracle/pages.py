"""Plain CPU fp64 restatement of attention over a KV pool whose pages hold
page_size > 1 tokens.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library and never imports it.

Sources (AstrAI project pages):
  * "Inference" guide, section "KVCache System": the pool runs in paged mode
    with page_size 1 or larger, and req_to_token maps a request's logical
    positions to physical storage.
  * Compare page v1.3.3 -> v1.3.4, class PagedCache: the caches have shape
    [n_layers, n_pages, page_size, n_kv_heads, head_dim]; a request's page
    table lists its physical pages in logical order; the write puts logical
    position pos in logical page pos // page_size, at offset
    pos - (pos // page_size) * page_size of that page's physical page; the
    gather concatenates the request's physical pages in logical order.
  * "Inference" guide, section "KV Cache": the attention equation, evaluated
    here by ``oracle.attention.attend`` on the gathered rows.

Readings where the pages are silent:
  * The flat pool k_buffer [n_layers, size, n_kv_heads, head_dim] with
    size = n_pages * page_size is the same memory as the page view
    [n_layers, n_pages, page_size, n_kv_heads, head_dim]; a flat slot index
    (out_cache_loc) of position pos is therefore
    page * page_size + offset.  Gathers below index the page view directly.
  * With pages, req_to_token is [num_reqs, ceil(max_ctx_len / page_size)]
    and holds physical page ids.
  * page_size = 1 is the one-token case of ``oracle.attention``.

Pins: tests/test_oracle_pages.py (torch SDPA on the pages' concatenated
gather, page_size 1 against the one-token oracle, physical page permutation,
contiguous layout, a hand-worked fixture, planted mistakes).
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .attention import attend


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def page_view(buffer: np.ndarray, page_size: int) -> np.ndarray:
    """[n_layers, size, Hk, d] -> [n_layers, size // page_size, page_size, Hk, d]."""
    n_layers, size = buffer.shape[0], buffer.shape[1]
    assert size % page_size == 0, "pool size must be whole pages"
    return buffer.reshape((n_layers, size // page_size, page_size) + buffer.shape[2:])


def gather_rows(cache5: np.ndarray, layer_id: int, page_row: Sequence[int], n_tokens: int,
                hk: int) -> np.ndarray:
    """Rows of logical positions 0 .. n_tokens-1 of one request and kv-head:
    position pos comes from physical page page_row[pos // page_size] at
    offset pos % page_size (the page write's placement)."""
    ps = cache5.shape[2]
    rows = []
    for pos in range(n_tokens):
        page = int(page_row[pos // ps])
        rows.append(cache5[layer_id, page, pos % ps, hk])
    if not rows:
        return np.zeros((0, cache5.shape[-1]), dtype=cache5.dtype)
    return np.stack(rows)


def build_step(req_pool_indices: Sequence[int], seq_lens: Sequence[int],
               page_table: np.ndarray, page_size: int,
               q_lens: Optional[Sequence[int]] = None):
    """Step metadata of a paged pool: kv_indptr / qo_indptr as exclusive prefix
    sums of seq_lens and of the new-token counts, and out_cache_loc, in qo
    order, the flat slot page * page_size + offset of each new token (new token
    t of request b sits at position seq_len_b - q_len_b + t)."""
    B = len(seq_lens)
    if q_lens is None:
        q_lens = [1] * B
    kv_indptr = [0]
    qo_indptr = [0]
    locs: List[int] = []
    for b in range(B):
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        ql = int(q_lens[b])
        kv_indptr.append(kv_indptr[-1] + L)
        qo_indptr.append(qo_indptr[-1] + ql)
        for t in range(ql):
            pos = L - ql + t
            page = int(page_table[r, pos // page_size])
            locs.append(page * page_size + pos % page_size)
    return {
        "kv_indptr": np.array(kv_indptr, dtype=np.int32),
        "qo_indptr": np.array(qo_indptr, dtype=np.int32),
        "out_cache_loc": np.array(locs, dtype=np.int32),
        "max_len": max([int(x) for x in seq_lens], default=0),
        "max_q_len": max([int(x) for x in q_lens], default=0),
        "n_new": len(locs),
    }


def write(k_buffer: np.ndarray, v_buffer: np.ndarray, layer_id: int, page_table: np.ndarray,
          page_size: int, req_pool_indices, seq_lens, q_lens, k_new: np.ndarray,
          v_new: np.ndarray):
    """The page write: copies of both pools with new token t of request b (its
    row qo_b + t of k_new / v_new) stored at physical page
    page_table[r_b, pos // page_size], offset pos % page_size, where
    pos = seq_len_b - q_len_b + t.  A bitwise copy; nothing else changes."""
    k_out = k_buffer.copy()
    v_out = v_buffer.copy()
    k5 = page_view(k_out, page_size)
    v5 = page_view(v_out, page_size)
    i = 0
    for b in range(len(seq_lens)):
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        ql = int(q_lens[b])
        for t in range(ql):
            pos = L - ql + t
            page = int(page_table[r, pos // page_size])
            k5[layer_id, page, pos % page_size] = k_new[i]
            v5[layer_id, page, pos % page_size] = v_new[i]
            i += 1
    return k_out, v_out


def decode(k_buffer, v_buffer, layer_id, page_table, page_size, req_pool_indices, seq_lens,
           q, sm_scale) -> np.ndarray:
    """Decode over a paged pool: each request's query rows attend its seq_len
    positions gathered page by page.  q [B, H, dk] -> [B, H, dv] fp64 (dv: the
    value rows' width)."""
    q = _f64(q)
    B, H, _ = q.shape
    Hk = k_buffer.shape[2]
    G = H // Hk
    k5 = page_view(k_buffer, page_size)
    v5 = page_view(v_buffer, page_size)
    out = np.zeros((B, H, v_buffer.shape[3]), dtype=np.float64)
    for b in range(B):
        row = page_table[int(req_pool_indices[b])]
        L = int(seq_lens[b])
        for hk in range(Hk):
            K = gather_rows(k5, layer_id, row, L, hk)
            V = gather_rows(v5, layer_id, row, L, hk)
            heads = list(range(hk * G, (hk + 1) * G))
            out[b, heads] = attend(q[b, heads], K, V, sm_scale)
    return out


def decode_pairs(k_buffer, v_buffer, layer_id, page_table, page_size, req_pool_indices,
                 seq_lens, q, sm_scale, pairs: Iterable[Tuple[int, int]]) -> np.ndarray:
    """decode() at the listed (b, h) pairs only; returns [n_pairs, d]."""
    q = _f64(q)
    H = q.shape[1]
    Hk = k_buffer.shape[2]
    G = H // Hk
    k5 = page_view(k_buffer, page_size)
    v5 = page_view(v_buffer, page_size)
    rows = []
    for b, h in pairs:
        row = page_table[int(req_pool_indices[b])]
        L = int(seq_lens[b])
        K = gather_rows(k5, layer_id, row, L, h // G)
        V = gather_rows(v5, layer_id, row, L, h // G)
        rows.append(attend(q[b, h], K, V, sm_scale)[0])
    return np.stack(rows) if rows else np.zeros((0, v_buffer.shape[3]))


def prefill(k_buffer, v_buffer, layer_id, page_table, page_size, req_pool_indices, seq_lens,
            qo_indptr, q, sm_scale, causal: bool = True) -> np.ndarray:
    """Ragged prefill over a paged pool: new token t of request i (prefix
    p_i = seq_len_i - q_len_i) attends positions 0 .. p_i + t when causal,
    else all seq_len_i positions.  q [n_new, H, dk] -> [n_new, H, dv] fp64."""
    q = _f64(q)
    n_new, H, _ = q.shape
    Hk = k_buffer.shape[2]
    G = H // Hk
    k5 = page_view(k_buffer, page_size)
    v5 = page_view(v_buffer, page_size)
    out = np.zeros((n_new, H, v_buffer.shape[3]), dtype=np.float64)
    for i in range(len(seq_lens)):
        row = page_table[int(req_pool_indices[i])]
        L = int(seq_lens[i])
        q0 = int(qo_indptr[i])
        ql = int(qo_indptr[i + 1]) - q0
        if ql == 0:
            continue
        p = L - ql
        for hk in range(Hk):
            K = gather_rows(k5, layer_id, row, L, hk)
            V = gather_rows(v5, layer_id, row, L, hk)
            nk = [(p + t + 1) if causal else L for t in range(ql)]
            for h in range(hk * G, (hk + 1) * G):
                out[q0:q0 + ql, h] = attend(q[q0:q0 + ql, h], K, V, sm_scale, nk)
    return out


def prefill_rows(k_buffer, v_buffer, layer_id, page_table, page_size, req_pool_indices,
                 seq_lens, qo_indptr, q, sm_scale, rows: Iterable[Tuple[int, int]],
                 causal: bool = True) -> np.ndarray:
    """prefill() at the listed (token, head) rows only; token indexes the packed
    [n_new, H, d] query.  Returns [n_rows, d]."""
    q = _f64(q)
    H = q.shape[1]
    G = H // k_buffer.shape[2]
    k5 = page_view(k_buffer, page_size)
    v5 = page_view(v_buffer, page_size)
    qo = [int(x) for x in qo_indptr]
    out = []
    for tok, h in rows:
        i = int(np.searchsorted(qo, tok, side="right")) - 1
        row = page_table[int(req_pool_indices[i])]
        L = int(seq_lens[i])
        t = tok - qo[i]
        nk = (L - (qo[i + 1] - qo[i]) + t + 1) if causal else L
        K = gather_rows(k5, layer_id, row, nk, h // G)
        V = gather_rows(v5, layer_id, row, nk, h // G)
        out.append(attend(q[tok, h], K, V, sm_scale)[0])
    return np.stack(out) if out else np.zeros((0, v_buffer.shape[3]))


def validate_step(size: int, page_size: int, page_table: np.ndarray, req_pool_indices,
                  seq_lens, kv_indptr, qo_indptr, out_cache_loc) -> Tuple[bool, str]:
    """Checked mode for a paged pool ("Inference" guide, section "KVCache
    System": kv_indptr and qo_indptr are the exclusive prefix sums of seq_lens
    and of the new-token counts; out_cache_loc holds the write slots).  A step
    is well formed when the pool is whole pages, every request row is a row of
    the page table, every length is in [1, max_ctx_len] (max_ctx_len = table
    width x page_size), both indptr arrays are those prefix sums, every
    new-token count is in [0, seq_len], every page a request reads is a
    physical page of the pool, and each write slot is the flat slot of its
    token's position, the write slots pairwise distinct."""
    B = len(seq_lens)
    if size % page_size != 0:
        return False, "pool size not whole pages"
    n_pages = size // page_size
    if len(req_pool_indices) != B or len(kv_indptr) != B + 1 or len(qo_indptr) != B + 1:
        return False, "array lengths"
    if int(kv_indptr[0]) != 0 or int(qo_indptr[0]) != 0:
        return False, "indptr start"
    if len(out_cache_loc) != int(qo_indptr[B]):
        return False, "out_cache_loc length"
    seen = set()
    for b in range(B):
        r = int(req_pool_indices[b])
        L = int(seq_lens[b])
        if not (0 <= r < page_table.shape[0]) or not (1 <= L <= page_table.shape[1] * page_size):
            return False, f"request {b}"
        if int(kv_indptr[b + 1]) - int(kv_indptr[b]) != L:
            return False, f"kv_indptr {b}"
        for lp in range((L + page_size - 1) // page_size):
            if not (0 <= int(page_table[r, lp]) < n_pages):
                return False, f"page ({b},{lp})"
        q0 = int(qo_indptr[b])
        ql = int(qo_indptr[b + 1]) - q0
        if not (0 <= ql <= L):
            return False, f"q_len {b}"
        for t in range(ql):
            pos = L - ql + t
            loc = int(out_cache_loc[q0 + t])
            want = int(page_table[r, pos // page_size]) * page_size + pos % page_size
            if loc != want:
                return False, f"out_cache_loc mismatch ({b},{t})"
            if loc in seen:
                return False, f"out_cache_loc duplicate ({b},{t})"
            seen.add(loc)
    return True, "ok"
