"""Seeded synthetic inputs for paged-KV attention, shared by tests and bench.

This module only draws random numbers and lays them out: request lengths,
slot permutations, slot tables and pool / query contents.  It holds none of
the attention arithmetic and derives no step metadata (prefix sums and write
slots are computed separately by the library and by the oracle).

Host-side structures are numpy int32 arrays drawn with
``numpy.random.default_rng(seed)``; tensor contents are drawn with a seeded
``torch.Generator`` on the target device, in chunks, so that multi-GiB pools
can be filled on the GPU.  Poisoning: every pool slot of the attended layer
that no request references, every other layer, and the slot that unused
slot-table entries point at, hold NaN, so any stray read shows up as NaN.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "bf16")


@dataclass
class Case:
    """One attention step over a paged pool (decode when q_lens are all 1)."""

    name: str
    dtype: str                 # "f32" | "bf16"
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    layer_id: int
    size: int                  # pool slots per layer
    req_to_token: np.ndarray   # int32 [num_reqs, max_ctx_len]
    req_pool_indices: np.ndarray  # int32 [B]
    seq_lens: np.ndarray       # int32 [B], context length incl. new tokens
    q_lens: np.ndarray         # int32 [B], new tokens this step
    seed: int
    k_scale: float = 1.0
    poison_slot: Optional[int] = None
    notes: Dict[str, object] = field(default_factory=dict)
    # Tokens per page.  1: req_to_token holds slots.  >1: req_to_token is the
    # page table [num_reqs, max_pages] of physical page ids, the pool holds
    # size / page_size pages, and poison_slot is unused (poison_page instead).
    page_size: int = 1
    poison_page: Optional[int] = None
    # Width of the value rows when it differs from the key rows (MLA-shaped
    # layers: keys qk_nope + qk_rope wide, values v_head_dim); None: head_dim.
    v_head_dim: Optional[int] = None

    @property
    def dv(self) -> int:
        return int(self.v_head_dim or self.head_dim)

    @property
    def batch(self) -> int:
        return int(len(self.seq_lens))

    @property
    def num_reqs(self) -> int:
        return int(self.req_to_token.shape[0])

    @property
    def max_ctx_len(self) -> int:
        return int(self.req_to_token.shape[1]) * self.page_size

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.q_lens == 1))

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    def referenced_pages(self) -> np.ndarray:
        """Paged pools: sorted unique physical pages some request reads."""
        ps = self.page_size
        parts = [self.req_to_token[int(r), : (int(L) + ps - 1) // ps]
                 for r, L in zip(self.req_pool_indices, self.seq_lens)]
        if not parts:
            return np.zeros(0, dtype=np.int64)
        return np.unique(np.concatenate(parts).astype(np.int64))

    def referenced_slots(self) -> np.ndarray:
        """Sorted unique slots that some request reads (positions < seq_len)."""
        assert self.page_size == 1, "slot table only"
        parts = [self.req_to_token[int(r), : int(L)]
                 for r, L in zip(self.req_pool_indices, self.seq_lens)]
        if not parts:
            return np.zeros(0, dtype=np.int64)
        return np.unique(np.concatenate(parts).astype(np.int64))


def _table(num_reqs: int, max_ctx_len: int, fill: int) -> np.ndarray:
    return np.full((num_reqs, max_ctx_len), fill, dtype=np.int32)


# ---------------------------------------------------------------------------
# Generic builders
# ---------------------------------------------------------------------------
def random_case(seed: int, seq_lens: Sequence[int], q_lens: Optional[Sequence[int]] = None,
                n_heads: int = 4, n_kv_heads: int = 2, head_dim: int = 64,
                dtype: str = "f32", size: Optional[int] = None, n_layers: int = 1,
                layer_id: int = 0, num_reqs: Optional[int] = None,
                max_ctx_len: Optional[int] = None, k_scale: float = 1.0,
                name: str = "random", v_head_dim: Optional[int] = None) -> Case:
    """Requests with the given lengths; each request's logical positions map to
    distinct slots drawn from one random permutation of the pool; request rows
    are a random subset of num_reqs table rows; unused table entries point at a
    reserved poison slot."""
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.ones(B, dtype=np.int32) if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    total = int(seq_lens.sum())
    if size is None:
        size = total + 8
    if num_reqs is None:
        num_reqs = B + 2
    if max_ctx_len is None:
        max_ctx_len = max(int(seq_lens.max(initial=1)), 1)
    assert size >= total + 1, "pool too small for distinct slots plus a poison slot"
    perm = rng.permutation(size).astype(np.int32)
    poison = int(perm[total])
    table = _table(num_reqs, max_ctx_len, poison)
    rows = rng.permutation(num_reqs)[:B].astype(np.int32)
    off = 0
    for b in range(B):
        L = int(seq_lens[b])
        table[rows[b], :L] = perm[off:off + L]
        off += L
    return Case(name=name, dtype=dtype, n_heads=n_heads, n_kv_heads=n_kv_heads,
                head_dim=head_dim, n_layers=n_layers, layer_id=layer_id, size=size,
                req_to_token=table, req_pool_indices=rows, seq_lens=seq_lens,
                q_lens=q_lens, seed=seed, k_scale=k_scale, poison_slot=poison,
                v_head_dim=v_head_dim)


def random_paged_case(seed: int, seq_lens: Sequence[int], page_size: int,
                      q_lens: Optional[Sequence[int]] = None, n_heads: int = 4,
                      n_kv_heads: int = 2, head_dim: int = 64, dtype: str = "f32",
                      n_pages: Optional[int] = None, n_layers: int = 1, layer_id: int = 0,
                      num_reqs: Optional[int] = None, max_pages: Optional[int] = None,
                      shared_pages: int = 0, k_scale: float = 1.0,
                      name: str = "random_paged", v_head_dim: Optional[int] = None) -> Case:
    """Requests with the given lengths on a pool of n_pages pages of page_size
    tokens.  Each request's logical pages map to distinct physical pages taken
    in order from one random permutation of the pages, except that the first
    shared_pages logical pages of every request map to the same physical pages
    (a shared prefix; each request must be longer than that prefix so its new
    tokens stay on private pages).  Request rows are a random subset of
    num_reqs table rows; unused table entries point at a reserved poison
    page."""
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.ones(B, dtype=np.int32) if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    need = [-(-int(L) // page_size) for L in seq_lens]
    assert all(int(L) - int(ql) >= shared_pages * page_size for L, ql in zip(seq_lens, q_lens)), \
        "new tokens must not land on shared pages"
    total = shared_pages + sum(n - shared_pages for n in need)
    if n_pages is None:
        n_pages = total + 4
    if num_reqs is None:
        num_reqs = B + 2
    if max_pages is None:
        max_pages = max(need + [1])
    assert n_pages >= total + 1, "pool too small for distinct pages plus a poison page"
    perm = rng.permutation(n_pages).astype(np.int32)
    poison = int(perm[total])
    table = _table(num_reqs, max_pages, poison)
    rows = rng.permutation(num_reqs)[:B].astype(np.int32)
    off = shared_pages
    for b in range(B):
        n = need[b]
        table[rows[b], :shared_pages] = perm[:shared_pages]
        table[rows[b], shared_pages:n] = perm[off:off + n - shared_pages]
        off += n - shared_pages
    return Case(name=name, dtype=dtype, n_heads=n_heads, n_kv_heads=n_kv_heads,
                head_dim=head_dim, n_layers=n_layers, layer_id=layer_id,
                size=n_pages * page_size, req_to_token=table, req_pool_indices=rows,
                seq_lens=seq_lens, q_lens=q_lens, seed=seed, k_scale=k_scale,
                page_size=page_size, poison_page=poison, v_head_dim=v_head_dim)


def contiguous_case(seed: int, seq_lens: Sequence[int], max_seq_len: int, **kw) -> Case:
    """Contiguous-mode slot table: slot = request_row * max_seq_len + position
    ("Inference" guide, section "KVCache System", contiguous mode)."""
    B = len(seq_lens)
    num_reqs = B
    size = num_reqs * max_seq_len
    table = np.zeros((num_reqs, max_seq_len), dtype=np.int32)
    for r in range(num_reqs):
        table[r] = np.arange(r * max_seq_len, (r + 1) * max_seq_len, dtype=np.int32)
    q_lens = kw.pop("q_lens", None)
    c = Case(name=kw.pop("name", "contiguous"), dtype=kw.pop("dtype", "f32"),
             n_heads=kw.pop("n_heads", 4), n_kv_heads=kw.pop("n_kv_heads", 2),
             head_dim=kw.pop("head_dim", 64), n_layers=1, layer_id=0, size=size,
             req_to_token=table, req_pool_indices=np.arange(B, dtype=np.int32),
             seq_lens=np.asarray(seq_lens, dtype=np.int32),
             q_lens=np.ones(B, dtype=np.int32) if q_lens is None else np.asarray(q_lens, dtype=np.int32),
             seed=seed, poison_slot=None)
    assert not kw, kw
    return c


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------
def tiny_decode_f32(seed: int = 1) -> Case:
    """Tiny decode, fp32: B=2, 4 query / 2 kv heads, head_dim 64, one layer,
    64-slot pool, seq_lens {5, 17}; rows are a random 2-subset of 4 table rows
    and take the first 5 and the next 17 entries of one slot permutation."""
    rng = np.random.default_rng(seed)
    size, lens = 64, (5, 17)
    perm = rng.permutation(size).astype(np.int32)
    poison = int(perm[sum(lens)])
    table = _table(4, 17, poison)
    rows = rng.permutation(4)[:2].astype(np.int32)
    table[rows[0], :5] = perm[:5]
    table[rows[1], :17] = perm[5:22]
    return Case(name="tiny_decode_f32", dtype="f32", n_heads=4, n_kv_heads=2, head_dim=64,
                n_layers=1, layer_id=0, size=size, req_to_token=table,
                req_pool_indices=rows, seq_lens=np.array(lens, dtype=np.int32),
                q_lens=np.ones(2, dtype=np.int32), seed=seed, poison_slot=poison)


LLAMA_SWEEP = (1024, 4096, 16384, 32768)


def llama_b1_decode(seq_len: int, seed: int = 2, n_layers: int = 32, layer_id: int = 31) -> Case:
    """Llama-3-8B-shaped single-request decode, bf16: 32 query / 8 kv heads,
    head_dim 128, 32 layers (layer 31 attended), 65536-slot pool, the request's
    positions on the first seq_len entries of a random slot permutation."""
    rng = np.random.default_rng(seed * 100003 + seq_len)
    size = 65536
    perm = rng.permutation(size).astype(np.int32)
    poison = int(perm[seq_len]) if seq_len < size else None
    table = _table(1, seq_len, 0)
    table[0, :] = perm[:seq_len]
    return Case(name=f"llama_b1_decode_L{seq_len}", dtype="bf16", n_heads=32, n_kv_heads=8,
                head_dim=128, n_layers=n_layers, layer_id=layer_id, size=size,
                req_to_token=table, req_pool_indices=np.zeros(1, dtype=np.int32),
                seq_lens=np.array([seq_len], dtype=np.int32), q_lens=np.ones(1, dtype=np.int32),
                seed=seed, poison_slot=poison)


def batched_prefix_decode(seed: int = 3, B: int = 64, lo: int = 128, hi: int = 8192,
                          group: int = 8, shared: int = 1024, size: int = 600_000) -> Case:
    """Batched ragged decode with prefix sharing, bf16: 64 requests, 32/8/128
    heads, seq_lens uniform in [128, 8192]; requests 8g .. 8g+7 map their first
    min(1024, seq_len - 1) positions onto the same 1024 physical slots (a
    prefix-cache hit), and every other position, the current token's included,
    onto a private slot of a 600K-slot pool."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    perm = rng.permutation(size).astype(np.int32)
    n_groups = (B + group - 1) // group
    shared_slots = perm[: n_groups * shared].reshape(n_groups, shared)
    off = n_groups * shared
    private_needed = int(sum(int(L) - min(shared, int(L) - 1) for L in lens))
    assert off + private_needed + 1 <= size
    poison = int(perm[off + private_needed])
    table = _table(B, hi, poison)
    for b in range(B):
        L = int(lens[b])
        ns = min(shared, L - 1)
        table[b, :ns] = shared_slots[b // group, :ns]
        npriv = L - ns
        table[b, ns:L] = perm[off:off + npriv]
        off += npriv
    c = Case(name="batched_prefix_decode", dtype="bf16", n_heads=32, n_kv_heads=8, head_dim=128,
             n_layers=1, layer_id=0, size=size, req_to_token=table,
             req_pool_indices=np.arange(B, dtype=np.int32), seq_lens=lens,
             q_lens=np.ones(B, dtype=np.int32), seed=seed, poison_slot=poison)
    return c


def ragged_prefill(seed: int = 4, n_req: int = 16, q_hi: int = 2048, p_hi: int = 4096,
                   size: int = 131072, n_heads: int = 32, n_kv_heads: int = 8,
                   head_dim: int = 128, dtype: str = "bf16") -> Case:
    """Ragged causal paged prefill, bf16: 16 requests, 32/8/128 heads, q_len
    uniform in [1, 2048], cached prefix uniform in [0, 4096], kv_len = prefix +
    q_len; every request's positions on disjoint slots of one permutation of a
    131072-slot pool."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, q_hi + 1, size=n_req).astype(np.int32)
    prefix = rng.integers(0, p_hi + 1, size=n_req).astype(np.int32)
    lens = (prefix + q_lens).astype(np.int32)
    c = random_case(seed + 1, lens, q_lens, n_heads=n_heads, n_kv_heads=n_kv_heads,
                    head_dim=head_dim, dtype=dtype, size=size, num_reqs=n_req,
                    max_ctx_len=int(lens.max()), name="ragged_prefill")
    return c


def llama_b1_decode_paged(seq_len: int, page_size: int = 64, seed: int = 2, n_layers: int = 32,
                          layer_id: int = 31) -> Case:
    """The Llama-3-8B-shaped single-request decode on a pool of page_size-token
    pages: 32 query / 8 kv heads, head_dim 128, bf16, 32 layers (layer 31
    attended), 65536 slots = 65536 / page_size pages; the request's logical
    pages on the first ceil(seq_len / page_size) pages of a random page
    permutation."""
    c = random_paged_case(seed * 100003 + seq_len, [seq_len], page_size, n_heads=32,
                          n_kv_heads=8, head_dim=128, dtype="bf16",
                          n_pages=65536 // page_size, n_layers=n_layers, layer_id=layer_id,
                          num_reqs=1, name=f"llama_b1_decode_paged{page_size}_L{seq_len}")
    return c


def ragged_prefill_paged(page_size: int = 64, seed: int = 4, n_req: int = 16, q_hi: int = 2048,
                         p_hi: int = 4096, size: int = 131072) -> Case:
    """The ragged causal prefill (same length draws as ragged_prefill) on a
    pool of page_size-token pages: 131072 slots = 131072 / page_size pages;
    every request's logical pages on disjoint pages of one page permutation."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, q_hi + 1, size=n_req).astype(np.int32)
    prefix = rng.integers(0, p_hi + 1, size=n_req).astype(np.int32)
    lens = (prefix + q_lens).astype(np.int32)
    return random_paged_case(seed + 1, lens, page_size, q_lens=q_lens, n_heads=32, n_kv_heads=8,
                             head_dim=128, dtype="bf16", n_pages=size // page_size,
                             num_reqs=n_req, name=f"ragged_prefill_paged{page_size}")


def long_context_decode(seed: int = 5, B: int = 8, seq_len: int = 131072,
                        size: int = 1 << 20, n_layers: int = 4, layer_id: int = 3) -> Case:
    """Long-context split-KV stress, bf16: 8 requests of 131072 tokens, 64 query
    / 8 kv heads, head_dim 128, 4 layers (layer 3 attended), the slot table a
    random permutation of the 2^20-slot pool reshaped to [8, 131072]; keys are
    drawn as 4 * N(0, 1) to sharpen the softmax."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(size).astype(np.int32)
    table = perm[: B * seq_len].reshape(B, seq_len).copy()
    return Case(name="long_context_decode", dtype="bf16", n_heads=64, n_kv_heads=8,
                head_dim=128, n_layers=n_layers, layer_id=layer_id, size=size,
                req_to_token=table, req_pool_indices=np.arange(B, dtype=np.int32),
                seq_lens=np.full(B, seq_len, dtype=np.int32), q_lens=np.ones(B, dtype=np.int32),
                seed=seed, k_scale=4.0, poison_slot=None)


# ---------------------------------------------------------------------------
# Tensor contents
# ---------------------------------------------------------------------------
def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _fill_normal(t, gen, scale: float = 1.0, chunk: int = 1 << 26) -> None:
    import torch
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=gen, device=t.device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[s:e].copy_(x)


def make_tensors(case: Case, device="cpu", poison: bool = True) -> Dict[str, object]:
    """Allocate and fill the pool and the step's activations.

    Returns k_buffer, v_buffer [n_layers, size, Hk, d]; q [n_new, H, d] (for
    decode n_new = B, so q is also [B, H, d]); k_new, v_new [n_new, Hk, d];
    req_to_token, req_pool_indices, seq_lens, q_lens as int32 tensors.
    The attended layer holds N(0,1) (keys times k_scale); when poison is set,
    the other layers, the unreferenced slots and the poison slot hold NaN."""
    import torch
    dt = torch_dtype(case.dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(case.seed * 7919 + 17)
    shape = (case.n_layers, case.size, case.n_kv_heads, case.head_dim)
    kb = torch.empty(shape, dtype=dt, device=device)
    vb = torch.empty(shape[:3] + (case.dv,), dtype=dt, device=device)
    if poison and case.n_layers > 1:
        kb.fill_(float("nan"))
        vb.fill_(float("nan"))
    _fill_normal(kb[case.layer_id], gen, case.k_scale)
    _fill_normal(vb[case.layer_id], gen, 1.0)
    if poison and case.page_size > 1:
        # Page view [n_pages, page_size, Hk, d] of the attended layer: NaN in
        # every page no request reads and in the unused tail of each
        # request's last page.
        ps = case.page_size
        kv5 = [x[case.layer_id].view(case.size // ps, ps, case.n_kv_heads, x.shape[-1])
               for x in (kb, vb)]
        keep = torch.zeros(case.size // ps, dtype=torch.bool)
        keep[torch.from_numpy(case.referenced_pages())] = True
        drop = (~keep).nonzero().view(-1).to(device)
        for x in kv5:
            x.index_fill_(0, drop, float("nan"))
        for r, L in zip(case.req_pool_indices, case.seq_lens):
            used = int(L) % ps
            if used:
                last = int(case.req_to_token[int(r), (int(L) - 1) // ps])
                for x in kv5:
                    x[last, used:] = float("nan")
    elif poison:
        ref = case.referenced_slots()
        if ref.size < case.size:
            keep = torch.zeros(case.size, dtype=torch.bool)
            keep[torch.from_numpy(ref)] = True
            drop = (~keep).nonzero().view(-1).to(device)
            kb[case.layer_id].index_fill_(0, drop, float("nan"))
            vb[case.layer_id].index_fill_(0, drop, float("nan"))
    n_new = int(case.q_lens.sum())
    q = torch.empty((n_new, case.n_heads, case.head_dim), dtype=dt, device=device)
    k_new = torch.empty((n_new, case.n_kv_heads, case.head_dim), dtype=dt, device=device)
    v_new = torch.empty((n_new, case.n_kv_heads, case.dv), dtype=dt, device=device)
    _fill_normal(q, gen)
    _fill_normal(k_new, gen, case.k_scale)
    _fill_normal(v_new, gen)
    return {
        "k_buffer": kb, "v_buffer": vb, "q": q, "k_new": k_new, "v_new": v_new,
        "req_to_token": torch.from_numpy(case.req_to_token).to(device),
        "req_pool_indices": torch.from_numpy(case.req_pool_indices).to(device),
        "seq_lens": torch.from_numpy(case.seq_lens).to(device),
        "q_lens": torch.from_numpy(case.q_lens).to(device),
    }


def rope_table(max_pos: int, head_dim: int, base: float = 10000.0, device="cpu"):
    """A rotary table input, float32 [max_pos, head_dim / 2, 2] of [cos, sin]
    for the angles p * base^(-2j / head_dim) (how a model fills its table is
    outside the rotary step; this is the usual construction)."""
    import torch
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * j / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    t = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    return torch.from_numpy(t).to(device)


def mla_decode(seed: int = 6, seq_lens: Sequence[int] = (4096, 1000, 7000, 333),
               n_heads: int = 16, n_kv_heads: int = 16, qk_nope: int = 128, qk_rope: int = 64,
               v_head_dim: int = 128, q_lens: Optional[Sequence[int]] = None) -> Case:
    """An MLA-shaped layer (class MLA of the v1.3.4 compare page): per-head
    keys of qk_nope + qk_rope dims and values of v_head_dim, in a one-token
    page pool with random slots; decode unless q_lens are given."""
    total = int(np.sum(seq_lens))
    c = random_case(seed, list(seq_lens), q_lens, n_heads=n_heads, n_kv_heads=n_kv_heads,
                    head_dim=qk_nope + qk_rope, dtype="bf16", size=total + 64,
                    name="mla_decode" if q_lens is None else "mla_prefill",
                    v_head_dim=v_head_dim)
    c.notes.update({"qk_nope_head_dim": qk_nope, "qk_rope_head_dim": qk_rope})
    return c


def named_cases() -> List[str]:
    return ["tiny_decode_f32", "llama_b1_decode", "batched_prefix_decode",
            "ragged_prefill", "long_context_decode"]
