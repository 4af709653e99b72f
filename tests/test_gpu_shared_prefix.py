"""GPU parity of the decode step with shared prefixes read once per group
(pkv_paged_decode_shared) against the oracle: the same per-head attention
over every request's seq_lens keys as plain decode, whatever the grouping.
Also its pool write (bit for bit), graph replay, and the fall-back to the
plain step when nothing is shared."""

import numpy as np
import pytest
import torch

import oracle.pages as OP
import workloads as W
from paged_kv_attention_12_amd import api, binding as B
from tests.gpu_util import HostView, assert_close, say, to_np
from tests.test_gpu_pages import host_layer, oracle_written, step_of

pytestmark = pytest.mark.gpu


def bits(t):
    t = t.contiguous()
    return (t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)).cpu().numpy()


def shared_step(case, t, step, min_prefix=16, num_splits=None, prefix_splits=None):
    groups = api.PrefixGroups(step, case.req_pool_indices, case.seq_lens, case.req_to_token,
                              min_prefix=min_prefix)
    out = api.shared_decode_step(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id,
                                 step, groups, t["q"], t["k_new"], t["v_new"], case.sm_scale,
                                 num_splits=num_splits, prefix_splits=prefix_splits)
    return out, groups


def test_shared_batched_prefix_workload_whole_batch():
    case = W.batched_prefix_decode()
    say("shared prefix: batched workload")
    t = W.make_tensors(case, device="cuda")
    hv = HostView(case, t)
    ref = hv.decode_all(case)
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token)
    out, groups = shared_step(case, t, step, min_prefix=256)
    assert groups.n_groups == 8
    assert_close(to_np(out), ref, "bf16", "shared prefix batched")


def partly_shared_case(seed, lens, shares, H, Hk):
    """One-token pages; shares lists (b, src, P): request b reads request
    src's slots for its first P positions (P < seq_len of both), so the
    requests share prefixes of different lengths and some share nothing."""
    case = W.random_case(seed, lens, n_heads=H, n_kv_heads=Hk, head_dim=128, dtype="bf16",
                         n_layers=2, layer_id=1)
    tab = case.req_to_token
    for b, src, P in shares:
        assert P < lens[b] and P < lens[src]
        tab[case.req_pool_indices[b], :P] = tab[case.req_pool_indices[src], :P]
    return case


CASES = [
    # (page_size, H, Hk, seq_lens, shared_pages, num_splits, prefix_splits)
    (1, 32, 8, [300, 70, 129, 500, 65, 900], 64, None, None),      # G = 4, all in one group
    (16, 12, 2, [200, 330, 129, 1200], 8, 2, 1),                  # G = 6, 16-token pages
    (64, 8, 8, [70, 200, 129, 500, 1000, 65], 1, None, 3),        # G = 1 (MHA), 64-token pages
    (1, 40, 2, [2000, 2100, 2200], 1500, 5, 2),                   # G = 20: two column chunks
    (4, 32, 8, [17] * 20, 4, 1, 1),                               # 20 members: two groups
    (1, 16, 2, [1000, 1001, 2000, 40, 3000], None, 3, 7),         # G = 8, partly shared
]


@pytest.mark.parametrize("ps,H,Hk,lens,shared,ns,pfx", CASES,
                         ids=["g4", "g6_p16", "mha_p64", "g20", "twenty", "g8_partly"])
def test_shared_prefix_matches_oracle(ps, H, Hk, lens, shared, ns, pfx):
    if shared is None:
        case = partly_shared_case(600 + H, lens, [(1, 0, 900), (2, 0, 990), (4, 0, 500)], H, Hk)
    else:
        case = W.random_paged_case(600 + ps + H, lens, ps, n_heads=H, n_kv_heads=Hk,
                                   head_dim=128, dtype="bf16", n_layers=2, layer_id=1,
                                   shared_pages=shared)
    say("shared prefix", ps, H, Hk, lens, shared, ns, pfx)
    t = W.make_tensors(case, device="cuda")
    h = host_layer(case, t)
    step = step_of(case)
    out, groups = shared_step(case, t, step, min_prefix=8, num_splits=ns, prefix_splits=pfx)
    assert groups.n_groups >= 1
    torch.cuda.synchronize()
    kb, vb = oracle_written(case, h)
    ref = OP.decode(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                    h["q"], case.sm_scale)
    assert_close(to_np(out), ref, "bf16", f"shared {ps}/{H}/{Hk}")


def test_shared_prefix_pool_write_bit_exact():
    case = W.random_paged_case(650, [400, 401, 300, 90], 1, n_heads=32, n_kv_heads=8,
                               head_dim=128, dtype="bf16", n_layers=2, layer_id=0,
                               shared_pages=80)
    t = W.make_tensors(case, device="cuda")
    k0, v0 = bits(t["k_buffer"]), bits(t["v_buffer"])
    md = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, 1)
    step = step_of(case)
    shared_step(case, t, step, min_prefix=8)
    torch.cuda.synchronize()
    k1, v1 = bits(t["k_buffer"]), bits(t["v_buffer"])
    kn, vn = bits(t["k_new"]), bits(t["v_new"])
    for i, loc in enumerate(md["out_cache_loc"]):
        k0[0, loc] = kn[i]
        v0[0, loc] = vn[i]
    assert np.array_equal(k1, k0) and np.array_equal(v1, v0)


def test_shared_prefix_without_groups_is_the_plain_step():
    case = W.random_case(651, [100, 2000, 37], n_heads=32, n_kv_heads=8, head_dim=128,
                         dtype="bf16")
    t1 = W.make_tensors(case, device="cuda")
    t2 = W.make_tensors(case, device="cuda")
    s1 = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token)
    s2 = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token)
    o1, groups = shared_step(case, t1, s1, num_splits=6)
    assert groups.n_groups == 0
    o2 = api.stored_decode_step(t2["k_buffer"], t2["v_buffer"], t2["req_to_token"], 0, s2,
                                t2["q"], t2["k_new"], t2["v_new"], case.sm_scale, num_splits=6)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_shared_prefix_graph_replay_matches_eager():
    case = W.random_paged_case(652, [700, 800, 900, 1000], 1, n_heads=32, n_kv_heads=8,
                               head_dim=128, dtype="bf16", shared_pages=512)
    t = W.make_tensors(case, device="cuda")
    step = step_of(case)
    groups = api.PrefixGroups(step, case.req_pool_indices, case.seq_lens, case.req_to_token)
    ns, ps = groups.pick_splits(step, case.n_kv_heads, case.n_heads)
    ws = api.decode_workspace(case.batch, case.n_heads, case.head_dim, ns + ps)
    out = torch.empty_like(t["q"])
    run = lambda: api.shared_decode_step(t["k_buffer"], t["v_buffer"], t["req_to_token"], 0,
                                         step, groups, t["q"], t["k_new"], t["v_new"],
                                         case.sm_scale, num_splits=ns, prefix_splits=ps,
                                         workspace=ws, out=out)
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        run()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
