"""A decode loop captured once in a HIP graph and replayed token after token,
with the step metadata advanced in place on the device between replays
(seq_lens, position_ids, out_cache_loc).  The captured work is the rotary
embedding fused with the K/V write, the split attention and the merge; the
metadata advance (pkv_decode_advance) is captured too.  Every replay is
checked against the oracle run on the same inputs."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from paged_kv_attention_12_amd import api
from paged_kv_attention_12_amd import binding as B
from tests.gpu_util import assert_close, say, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", ["three_requests", "one_request_streamed"])
@pytest.mark.parametrize("form", ["rope_then_step", "rope_in_step"])
def test_graph_captured_decode_loop_advances_metadata_in_place(form, shape):
    """rope_then_step: the rotary write, then split attention and merge;
    rope_in_step: the rotary turn folded into the split kernel
    (pkv_paged_decode_rope_store), then the merge.  one_request_streamed: a
    single request of ~3000 keys on a 32-layer pool, whose K/V over all
    layers exceed the last-level cache, so the default load policy reads its
    rows with non-temporal loads (checked with pkv_decode_load_kind)."""
    steps = 6
    if shape == "three_requests":
        start = np.array([300, 451, 17], dtype=np.int32)   # position of each request's first token
        n_layers = 1
    else:
        start = np.array([2990], dtype=np.int32)
        n_layers = 32
    H, Hk, d = 32, 8, 128
    # table rows hold every position the loop reaches, including the one the
    # last metadata advance looks up (start + steps)
    case = W.random_case(960, list(start + steps + 1), n_heads=H, n_kv_heads=Hk, head_dim=d,
                         dtype="bf16", n_layers=n_layers)
    t = W.make_tensors(case, device="cuda", poison=False)
    pool = B.make_pool(t["k_buffer"], t["v_buffer"], t["req_to_token"])
    streamed = B.pkv_decode_load_kind(pool, case.batch, int((start + steps).max()))
    assert streamed == (1 if shape == "one_request_streamed" else 0)
    B_ = case.batch
    rpi = case.req_pool_indices
    # the first step: each request's token at position start_b (seq_len start_b + 1); the host
    # bound max_len covers every later length
    step = api.DeviceStep(rpi, start + 1, case.req_to_token, max_len=int((start + steps).max()))
    freqs = W.rope_table(case.max_ctx_len, d, device="cuda")
    q = torch.empty((B_, H, d), dtype=torch.bfloat16, device="cuda")
    k_new = torch.empty((B_, Hk, d), dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    q_rot = torch.empty_like(q)
    out = torch.empty_like(q)
    ns = 8
    ws = api.decode_workspace(B_, H, d, ns)

    def one_step():
        if form == "rope_in_step":
            api.rope_decode_step(t["k_buffer"], t["v_buffer"], t["req_to_token"], 0, step, q,
                                 k_new, v_new, freqs, case.sm_scale, num_splits=ns, workspace=ws,
                                 out=out)
            return
        api.rope_kv_store(t["k_buffer"], t["v_buffer"], t["req_to_token"], 0, step, q, k_new,
                          v_new, freqs, q_out=q_rot)
        api.decode_step(t["k_buffer"], t["v_buffer"], t["req_to_token"], 0, step, q_rot, None,
                        None, case.sm_scale, num_splits=ns, workspace=ws, out=out, write_kv=False)

    def advance():
        api.advance_decode(t["k_buffer"], t["v_buffer"], t["req_to_token"], step)

    # capture on a side stream (nothing runs while capturing)
    q.zero_(), k_new.zero_(), v_new.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            one_step()
            advance()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # capture ran nothing: the metadata is still the first step's
    assert step.seq_lens.cpu().numpy().tolist() == (start + 1).tolist()

    kb = to_np(t["k_buffer"][0]).astype(np.float64)[None]
    vb = to_np(t["v_buffer"][0]).astype(np.float64)[None]
    f0 = freqs.cpu().numpy()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(961)
    for k in range(steps):
        for x in (q, k_new, v_new):
            x.copy_(torch.randn(x.shape, generator=gen, device="cuda"))
        q0, kn0, vn0 = to_np(q), to_np(k_new), to_np(v_new)
        say("graph loop step", form, shape, k)
        g.replay()
        torch.cuda.synchronize()
        pos = start + k
        locs = case.req_to_token[rpi, pos]
        q_ref, kb, vb = oracle.rope_kv_store(kb, vb, 0, locs, q0, kn0, vn0, pos, f0, "bf16")
        ref = oracle.decode(kb, vb, 0, case.req_to_token, rpi, pos + 1, q_ref, case.sm_scale)
        assert_close(to_np(out), ref, "bf16", f"graph loop step {k}")
        assert step.seq_lens.cpu().numpy().tolist() == (pos + 2).tolist()


def test_decode_advance_matches_the_next_steps_metadata():
    """pkv_decode_advance against the oracle's metadata of the next steps:
    seq_lens, position_ids, out_cache_loc and kv_indptr, bit for bit."""
    start = np.array([5, 1, 90, 33], dtype=np.int32)
    case = W.random_case(962, list(start + 5), n_heads=4, n_kv_heads=2, head_dim=64, dtype="bf16")
    t = W.make_tensors(case, device="cuda", poison=False)
    step = api.DeviceStep(case.req_pool_indices, start, case.req_to_token,
                          max_len=int((start + 5).max()))
    for k in range(1, 5):
        api.advance_decode(t["k_buffer"], t["v_buffer"], t["req_to_token"], step)
        torch.cuda.synchronize()
        md = oracle.build_step(case.req_pool_indices, start + k, case.req_to_token)
        assert step.seq_lens.cpu().numpy().tolist() == (start + k).tolist()
        assert np.array_equal(step.kv_indptr.cpu().numpy(), md["kv_indptr"])
        assert np.array_equal(step.out_cache_loc.cpu().numpy(), md["out_cache_loc"])
        assert np.array_equal(step.position_ids.cpu().numpy(), md["position_ids"])
