"""Randomised GPU parity: seeded draws of decode and prefill configurations
(head counts and group sizes, head_dim, dtype, page size, ragged lengths,
split counts, causal or not), each run through the C ABI and compared with
the oracle (one-token pages: oracle.attention; larger pages: oracle.pages)
at the stated tolerances.  Every draw is printed before it runs."""

import numpy as np
import pytest
import torch

import oracle
import oracle.pages as OP
import workloads as W
from paged_kv_attention_12_amd import api
from tests.gpu_util import assert_close, say, to_np

pytestmark = pytest.mark.gpu

GROUPS = [(4, 4), (8, 2), (12, 4), (16, 2), (32, 8), (6, 1)]


def draw_case(rng, prefill: bool):
    H, Hk = GROUPS[int(rng.integers(0, len(GROUPS)))]
    d = int(rng.choice([64, 128]))
    dtype = "bf16" if prefill else str(rng.choice(["f32", "bf16"]))
    ps = int(rng.choice([1, 1, 2, 16, 64]))
    B = int(rng.integers(1, 6))
    if prefill:
        q_lens = rng.integers(0, 90, size=B)
        q_lens[int(rng.integers(0, B))] = max(1, q_lens.max())   # at least one row
        lens = (q_lens + rng.integers(0, 200, size=B)).clip(min=1)
    else:
        q_lens = np.ones(B, dtype=np.int64)
        lens = rng.integers(1, 700, size=B)
    seed = int(rng.integers(0, 1 << 20))
    if ps == 1:
        case = W.random_case(seed, lens.tolist(), q_lens.tolist(), n_heads=H, n_kv_heads=Hk,
                             head_dim=d, dtype=dtype, n_layers=2, layer_id=1)
    else:
        case = W.random_paged_case(seed, lens.tolist(), ps, q_lens=q_lens.tolist(), n_heads=H,
                                   n_kv_heads=Hk, head_dim=d, dtype=dtype, n_layers=2,
                                   layer_id=1)
    return case


def oracle_out(case, t, prefill, causal, q=None, kn=None):
    """The oracle's output for the case's tensors; q / kn replace the query
    and new-key rows when given (the rotated rows of a rotary step)."""
    sl = slice(case.layer_id, case.layer_id + 1)
    kb0, vb0 = to_np(t["k_buffer"][sl]), to_np(t["v_buffer"][sl])
    q = to_np(t["q"]) if q is None else q
    kn = to_np(t["k_new"]) if kn is None else kn
    vn = to_np(t["v_new"])
    ps = case.page_size
    if ps == 1:
        md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token,
                               case.q_lens)
        kb, vb = oracle.kv_store(kb0, vb0, 0, md["out_cache_loc"], kn, vn)
        if prefill:
            return oracle.prefill(kb, vb, 0, case.req_to_token, case.req_pool_indices,
                                  case.seq_lens, md["qo_indptr"], q, case.sm_scale, causal)
        return oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices,
                             case.seq_lens, q, case.sm_scale)
    md = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, ps, case.q_lens)
    kb, vb = OP.write(kb0, vb0, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                      case.q_lens, kn, vn)
    if prefill:
        return OP.prefill(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices,
                          case.seq_lens, md["qo_indptr"], q, case.sm_scale, causal)
    return OP.decode(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens, q,
                     case.sm_scale)


@pytest.mark.parametrize("draw", range(24))
def test_random_decode(draw):
    rng = np.random.default_rng(7000 + draw)
    case = draw_case(rng, prefill=False)
    kind = str(rng.choice(["three_launch", "stored", "fused"]))
    ns = int(rng.choice([0, 1, 3, 17]))
    say("random decode", draw, kind, case.dtype, case.n_heads, case.n_kv_heads, case.head_dim,
        "pages", case.page_size, "lens", case.seq_lens.tolist(), "splits", ns or "auto")
    t = W.make_tensors(case, device="cuda")
    ref = oracle_out(case, t, prefill=False, causal=True)
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token,
                          page_size=case.page_size)
    fn = {"three_launch": api.decode_step, "stored": api.stored_decode_step,
          "fused": api.fused_decode_step}[kind]
    out = fn(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id, step, t["q"],
             t["k_new"], t["v_new"], case.sm_scale, num_splits=ns or None)
    torch.cuda.synchronize()
    assert_close(to_np(out), ref, case.dtype, f"random decode {draw} ({kind})")


@pytest.mark.parametrize("draw", range(12))
def test_random_prefill(draw):
    rng = np.random.default_rng(8000 + draw)
    case = draw_case(rng, prefill=True)
    causal = bool(rng.integers(0, 4))   # mostly causal
    say("random prefill", draw, case.n_heads, case.n_kv_heads, case.head_dim, "pages",
        case.page_size, "q_lens", case.q_lens.tolist(), "lens", case.seq_lens.tolist(),
        "causal", causal)
    t = W.make_tensors(case, device="cuda")
    ref = oracle_out(case, t, prefill=True, causal=causal)
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens,
                          page_size=case.page_size)
    out = api.prefill_step(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id, step,
                           t["q"], t["k_new"], t["v_new"], case.sm_scale, causal=causal)
    torch.cuda.synchronize()
    assert_close(to_np(out), ref, "bf16", f"random prefill {draw}")


ROPE_GROUPS = [(4, 4), (8, 2), (12, 4), (16, 1), (32, 8), (6, 1), (32, 2)]


@pytest.mark.parametrize("draw", range(12))
def test_random_rope_decode(draw):
    """The decode step with the rotary turn folded in
    (pkv_paged_decode_rope_store; bf16 pools with 128-wide rows and up to 16
    query heads per kv-head) on seeded draws of group size, page size, batch,
    lengths and split count, against the oracle: q and k_new turned by
    oracle.rope_rotate at position seq_lens - 1 and rounded to bf16, then the
    write and the attention."""
    rng = np.random.default_rng(9000 + draw)
    H, Hk = ROPE_GROUPS[int(rng.integers(0, len(ROPE_GROUPS)))]
    ps = int(rng.choice([1, 1, 2, 16, 64]))
    B = int(rng.integers(1, 7))
    lens = rng.integers(1, 900, size=B)
    ns = int(rng.choice([0, 1, 5, 33]))
    seed = int(rng.integers(0, 1 << 20))
    kw = dict(n_heads=H, n_kv_heads=Hk, head_dim=128, dtype="bf16", n_layers=2, layer_id=1)
    if ps == 1:
        case = W.random_case(seed, lens.tolist(), **kw)
    else:
        case = W.random_paged_case(seed, lens.tolist(), ps, **kw)
    say("random rope decode", draw, H, Hk, "pages", ps, "lens", case.seq_lens.tolist(),
        "splits", ns or "auto")
    t = W.make_tensors(case, device="cuda")
    max_pos = int(case.seq_lens.max()) + int(rng.integers(0, 50))
    freqs = W.rope_table(max_pos, 128, device="cuda")
    pos = np.asarray(case.seq_lens) - 1
    f0 = freqs.cpu().numpy()
    q_rot = oracle.to_dtype(oracle.rope_rotate(to_np(t["q"]), pos, f0), "bf16")
    k_rot = oracle.to_dtype(oracle.rope_rotate(to_np(t["k_new"]), pos, f0), "bf16")
    ref = oracle_out(case, t, prefill=False, causal=True, q=q_rot, kn=k_rot)
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token,
                          page_size=case.page_size)
    out = api.rope_decode_step(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id,
                               step, t["q"], t["k_new"], t["v_new"], freqs, case.sm_scale,
                               num_splits=ns or None)
    torch.cuda.synchronize()
    assert_close(to_np(out), ref, "bf16", f"random rope decode {draw}")
