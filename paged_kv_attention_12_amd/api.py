"""Convenience layer over the C entry points: one step's metadata on the
device, and the decode / prefill step sequences (write, attend, merge).
Marshalling only: every stage runs in libpkv's kernels."""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import binding as B


class DeviceStep:
    """Metadata of one step, built on the host by pkv_build_step and copied to
    the device once (int32 kv_indptr, qo_indptr, out_cache_loc, plus the
    request rows and lengths), with the host scalars kept alongside."""

    def __init__(self, req_pool_indices, seq_lens, req_to_token_host, q_lens=None,
                 device="cuda", max_len: Optional[int] = None, page_size: int = 1):
        import torch
        md = B.pkv_build_step(req_pool_indices, seq_lens, req_to_token_host, q_lens, page_size)
        self.host = md
        self.page_size = int(page_size)   # req_to_token is a page table when > 1
        self.batch = len(md["kv_indptr"]) - 1
        self.n_new = md["n_new"]
        # decode: a larger bound lets graph replays grow seq_lens in place
        self.max_len = md["max_len"] if max_len is None else max(int(max_len), md["max_len"])
        self.max_q_len = md["max_q_len"]
        self.total_len = int(md["kv_indptr"][-1])
        self.decode = q_lens is None
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        self.req_pool_indices = to(B._host_i32(req_pool_indices, "req_pool_indices"))
        self.seq_lens = to(B._host_i32(seq_lens, "seq_lens"))
        self.kv_indptr = to(md["kv_indptr"])
        self.qo_indptr = to(md["qo_indptr"])
        self.out_cache_loc = to(md["out_cache_loc"]) if self.n_new else \
            torch.zeros(0, dtype=torch.int32, device=device)
        self.prefill_order = to(md["prefill_order"]) if self.batch else None
        # logical positions of the new tokens (rows of the rotary table)
        self.position_ids = to(B.pkv_build_positions(seq_lens, q_lens)) if self.n_new else \
            torch.zeros(0, dtype=torch.int32, device=device)
        self.q_lens_host = None if q_lens is None else B._host_i32(q_lens, "q_lens")
        self.prefill_blocks = None      # device schedule, set for given head counts
        self.prefill_heads = None
        self._make_c()

    def _make_c(self):
        self.c = B.make_step(self.batch, self.req_pool_indices, self.seq_lens, self.kv_indptr,
                             None if self.decode else self.qo_indptr,
                             self.out_cache_loc if self.n_new else None, self.n_new,
                             self.max_len, self.max_q_len,
                             None if self.decode else self.prefill_order,
                             self.prefill_blocks)

    def set_prefill_blocks(self, n_heads: int, n_kv_heads: int) -> None:
        """Build the prefill launch schedule (pkv_prefill_blocks) for these head
        counts, copy it to the device once and attach it to the step."""
        import torch
        if self.decode or self.prefill_heads == (n_heads, n_kv_heads):
            return
        blocks = B.pkv_prefill_blocks(self.q_lens_host, self.host["prefill_order"], n_heads,
                                      n_kv_heads)
        self.prefill_blocks = (torch.from_numpy(np.ascontiguousarray(blocks.reshape(-1)))
                               .to(self.req_pool_indices.device) if len(blocks) else None)
        self.prefill_heads = (n_heads, n_kv_heads)
        self._make_c()


def decode_workspace(batch: int, n_heads: int, head_dim: int, num_splits: int, device="cuda"):
    import torch
    nbytes = B.pkv_decode_workspace_bytes(batch, n_heads, head_dim, num_splits)
    return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device)


def decode_step(k_buffer, v_buffer, req_to_token, layer_id: int, step: DeviceStep, q, k_new,
                v_new, sm_scale: float, num_splits: Optional[int] = None, workspace=None,
                out=None, write_kv: bool = True):
    """K/V write of the step's new tokens, split decode, merge.  Returns out."""
    import torch
    H, d = int(q.shape[1]), int(v_buffer.shape[3])   # outputs: value width
    if num_splits is None:
        num_splits = B.pkv_decode_pick_splits(step.batch, int(k_buffer.shape[2]), H,
                                              step.max_len, step.total_len)
    if workspace is None:
        workspace = decode_workspace(step.batch, H, d, num_splits, q.device)
    if out is None:
        out = q.new_empty((q.shape[0], q.shape[1], v_buffer.shape[3]))
    if write_kv:
        B.pkv_kv_store(k_buffer, v_buffer, req_to_token, layer_id, k_new, v_new,
                       step.out_cache_loc, page_size=step.page_size)
    B.pkv_paged_decode(k_buffer, v_buffer, req_to_token, layer_id, step.c, q, sm_scale,
                       num_splits, workspace, page_size=step.page_size)
    B.pkv_paged_decode_merge(step.batch, H, d, num_splits, workspace, out)
    return out


def decode_sync(batch: int, n_heads: int, device="cuda"):
    """Ticket counters of the fused decode step (zero; every call leaves them zero)."""
    import torch
    return torch.zeros(batch * n_heads, dtype=torch.int32, device=device)


def fused_decode_step(k_buffer, v_buffer, req_to_token, layer_id: int, step: DeviceStep, q,
                      k_new, v_new, sm_scale: float, num_splits: Optional[int] = None,
                      workspace=None, sync=None, out=None):
    """The decode step (K/V write, split attention, merge) in one library call:
    one launch for bf16 pools with head_dim 128.  Returns out."""
    import torch
    H, d = int(q.shape[1]), int(v_buffer.shape[3])   # outputs: value width
    if num_splits is None:
        num_splits = B.pkv_decode_step_pick_splits(step.batch, int(k_buffer.shape[2]), H,
                                                   step.max_len, step.total_len)
    if workspace is None:
        workspace = decode_workspace(step.batch, H, d, num_splits, q.device)
    if sync is None:
        sync = decode_sync(step.batch, H, q.device)
    if out is None:
        out = q.new_empty((q.shape[0], q.shape[1], v_buffer.shape[3]))
    B.pkv_paged_decode_step(k_buffer, v_buffer, req_to_token, layer_id, step.c, q, k_new, v_new,
                            sm_scale, num_splits, workspace, sync, out,
                            page_size=step.page_size)
    return out


def stored_decode_step(k_buffer, v_buffer, req_to_token, layer_id: int, step: DeviceStep, q,
                       k_new, v_new, sm_scale: float, num_splits: Optional[int] = None,
                       workspace=None, out=None):
    """The decode step (K/V write, split attention, merge) in two launches: the
    split kernel also writes the new token's K/V (bf16 pools with head_dim
    128).  Returns out."""
    import torch
    H, d = int(q.shape[1]), int(v_buffer.shape[3])   # outputs: value width
    if num_splits is None:
        num_splits = B.pkv_decode_pick_splits(step.batch, int(k_buffer.shape[2]), H,
                                              step.max_len, step.total_len)
    if workspace is None:
        workspace = decode_workspace(step.batch, H, d, num_splits, q.device)
    if out is None:
        out = q.new_empty((q.shape[0], q.shape[1], v_buffer.shape[3]))
    B.pkv_paged_decode_store(k_buffer, v_buffer, req_to_token, layer_id, step.c, q, k_new, v_new,
                             sm_scale, num_splits, workspace, out, page_size=step.page_size)
    return out


def rope_decode_step(k_buffer, v_buffer, req_to_token, layer_id: int, step: DeviceStep, q,
                     k_new, v_new, freqs_cis, sm_scale: float, num_splits: Optional[int] = None,
                     workspace=None, out=None):
    """The decode step with the rotary turn of q and k_new folded into the
    split kernel, then the merge (pkv_paged_decode_rope_store): q and k_new
    unrotated, positions step.position_ids.  Returns out."""
    H, d = int(q.shape[1]), int(v_buffer.shape[3])
    if num_splits is None:
        num_splits = B.pkv_decode_pick_splits(step.batch, int(k_buffer.shape[2]), H,
                                              step.max_len, step.total_len)
    if workspace is None:
        workspace = decode_workspace(step.batch, H, d, num_splits, q.device)
    if out is None:
        out = q.new_empty((q.shape[0], q.shape[1], v_buffer.shape[3]))
    B.pkv_paged_decode_rope_store(k_buffer, v_buffer, req_to_token, layer_id, step.c, q, k_new,
                                  v_new, step.position_ids, freqs_cis, sm_scale, num_splits,
                                  workspace, out, page_size=step.page_size)
    return out


class PrefixGroups:
    """The prefix groups of one decode step (pkv_decode_prefix_groups on the
    host copies of its metadata and table), copied to the device once."""

    def __init__(self, step: "DeviceStep", req_pool_indices, seq_lens, req_to_token_host,
                 min_prefix: int = 256, device="cuda"):
        import torch
        h = B.pkv_decode_prefix_groups(req_pool_indices, seq_lens, req_to_token_host,
                                       step.page_size, min_prefix)
        self.host = h
        self.n_groups = h["n_groups"]
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        self.groups = to(h["groups"].reshape(-1)) if self.n_groups else \
            torch.zeros(B.PKV_PREFIX_GROUP_INTS, dtype=torch.int32, device=device)
        self.kv_start = to(h["kv_start"])
        self.c = B.make_prefix_groups(self.groups, self.kv_start, self.n_groups, h["max_prefix"],
                                      h["max_members"], h["max_suffix"])
        self.suffix_total = int(np.sum(np.asarray(seq_lens, dtype=np.int64) - h["kv_start"]))

    def pick_splits(self, step: "DeviceStep", n_kv_heads: int, n_heads: int):
        """(num_splits, prefix_splits): the split heuristic on the requests'
        own keys, and prefix splits of about 256 shared keys."""
        ns = B.pkv_decode_pick_splits(step.batch, n_kv_heads, n_heads,
                                      max(self.host["max_suffix"], 1), self.suffix_total)
        ps = max(1, -(-self.host["max_prefix"] // 256)) if self.n_groups else 1
        return ns, ps


def shared_decode_step(k_buffer, v_buffer, req_to_token, layer_id: int, step: DeviceStep,
                       groups: PrefixGroups, q, k_new, v_new, sm_scale: float,
                       num_splits: Optional[int] = None, prefix_splits: Optional[int] = None,
                       workspace=None, out=None):
    """The decode step with each prefix group's shared keys read once
    (pkv_paged_decode_shared).  Returns out."""
    import torch
    H, d = int(q.shape[1]), int(v_buffer.shape[3])   # outputs: value width
    ns, ps = groups.pick_splits(step, int(k_buffer.shape[2]), H)
    num_splits = ns if num_splits is None else num_splits
    prefix_splits = ps if prefix_splits is None else prefix_splits
    if workspace is None:
        workspace = decode_workspace(step.batch, H, d, num_splits + prefix_splits, q.device)
    if out is None:
        out = q.new_empty((q.shape[0], q.shape[1], v_buffer.shape[3]))
    B.pkv_paged_decode_shared(k_buffer, v_buffer, req_to_token, layer_id, step.c, groups.c, q,
                              k_new, v_new, sm_scale, num_splits, prefix_splits, workspace, out,
                              page_size=step.page_size)
    return out


def advance_decode(k_buffer, v_buffer, req_to_token, step: DeviceStep) -> None:
    """Move a decode step's device metadata to the next token in place (one
    launch; graph-capturable).  step.max_len must already bound the lengths
    the coming steps reach (DeviceStep(..., max_len=...))."""
    B.pkv_decode_advance(k_buffer, v_buffer, req_to_token, step.req_pool_indices, step.seq_lens,
                         step.kv_indptr, step.out_cache_loc, step.position_ids,
                         page_size=step.page_size)


def rope_kv_store(k_buffer, v_buffer, req_to_token, layer_id: int, step: DeviceStep, q, k_new,
                  v_new, freqs_cis, q_out=None, rope_dim: Optional[int] = None):
    """Rotate the step's new queries and keys by their positions' rows of the
    rotary table freqs_cis [max_pos, head_dim / 2, 2] (f32 [cos, sin]) and
    write the rotated keys and the values to the pool, in one launch.  With
    rope_dim (MLA-shaped rows) only the last rope_dim dims turn and the table
    is [max_pos, rope_dim / 2, 2].  Returns the rotated queries (q_out; pass
    q_out=q to rotate in place)."""
    import torch
    if q_out is None:
        q_out = torch.empty_like(q)
    B.pkv_rope_kv_store(k_buffer, v_buffer, req_to_token, layer_id, q, q_out, k_new, v_new,
                        step.position_ids, freqs_cis, step.out_cache_loc,
                        page_size=step.page_size, rope_dim=rope_dim)
    return q_out


def prefill_step(k_buffer, v_buffer, req_to_token, layer_id: int, step: DeviceStep, q, k_new,
                 v_new, sm_scale: float, causal: bool = True, out=None, write_kv: bool = True,
                 schedule: bool = True):
    """K/V write of the step's new tokens, then ragged paged prefill (with the
    step's launch schedule of non-empty row blocks unless schedule=False)."""
    import torch
    if out is None:
        out = q.new_empty((q.shape[0], q.shape[1], v_buffer.shape[3]))
    if write_kv:
        B.pkv_kv_store(k_buffer, v_buffer, req_to_token, layer_id, k_new, v_new,
                       step.out_cache_loc, page_size=step.page_size)
    if schedule:
        step.set_prefill_blocks(int(q.shape[1]), int(k_buffer.shape[2]))
    B.pkv_paged_prefill(k_buffer, v_buffer, req_to_token, layer_id, step.c, q, sm_scale,
                        causal, out, page_size=step.page_size)
    return out
