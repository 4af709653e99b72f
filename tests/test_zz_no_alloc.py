"""The allocation-free decode step (pkv_paged_decode_store_noalloc: split
partials in the library's static per-device scratch array) against
pkv_paged_decode_store with a caller workspace, through the C ABI: output and
pool bit for bit, two calls in a row with the second one smaller, against the
oracle too, and the scratch limit."""

import numpy as np
import pytest
import torch

import workloads as W
from paged_kv_attention_12_amd import api
from paged_kv_attention_12_amd import binding as B
from tests.gpu_util import HostView, assert_close, say, to_np

pytestmark = pytest.mark.gpu


def bits(t):
    t = t.contiguous()
    return (t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)).cpu().numpy()


def both(case, num_splits):
    """The same step through both entry points on two identical copies of the
    inputs; returns (out_noalloc, out_workspace, tensors_noalloc, tensors_ws)."""
    t1 = W.make_tensors(case, device="cuda")
    t2 = W.make_tensors(case, device="cuda")
    step1 = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token)
    step2 = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token)
    ns = num_splits if num_splits is not None else B.pkv_decode_pick_splits(
        step1.batch, case.n_kv_heads, case.n_heads, step1.max_len, step1.total_len)
    o1 = torch.empty_like(t1["q"])
    B.pkv_paged_decode_store_noalloc(t1["k_buffer"], t1["v_buffer"], t1["req_to_token"],
                                     case.layer_id, step1.c, t1["q"], t1["k_new"], t1["v_new"],
                                     case.sm_scale, ns, o1)
    o2 = api.stored_decode_step(t2["k_buffer"], t2["v_buffer"], t2["req_to_token"],
                                case.layer_id, step2, t2["q"], t2["k_new"], t2["v_new"],
                                case.sm_scale, num_splits=ns)
    torch.cuda.synchronize()
    return o1, o2, t1, t2


def check_pair(case, num_splits, with_oracle=True):
    o1, o2, t1, t2 = both(case, num_splits)
    assert torch.equal(o1, o2)
    assert np.array_equal(bits(t1["k_buffer"]), bits(t2["k_buffer"]))
    assert np.array_equal(bits(t1["v_buffer"]), bits(t2["v_buffer"]))
    if with_oracle:
        t = W.make_tensors(case, device="cuda")
        ref = HostView(case, t).decode_all(case)
        assert_close(to_np(o1), ref, case.dtype, "noalloc step")


def test_noalloc_matches_workspace_step_two_calls_second_smaller():
    big = W.random_case(900, [3000, 17, 1200, 1], n_heads=32, n_kv_heads=8, head_dim=128,
                        dtype="bf16", n_layers=2, layer_id=1)
    small = W.random_case(901, [40, 5], n_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16")
    say("noalloc big", big.seq_lens.tolist())
    check_pair(big, 24)
    say("noalloc small", small.seq_lens.tolist())
    check_pair(small, 3)


def test_noalloc_other_shapes_run_the_three_launches():
    # f32 and head_dim 64 pools go through kv_store + split + merge
    for seed, d, dtype in ((902, 128, "f32"), (903, 64, "bf16")):
        case = W.random_case(seed, [33, 129], n_heads=8, n_kv_heads=2, head_dim=d, dtype=dtype)
        say("noalloc", d, dtype)
        check_pair(case, 4)


def test_noalloc_llama_b1_long_context_then_tiny():
    case = W.llama_b1_decode(32768)
    say("noalloc llama b1 32768")
    check_pair(case, None, with_oracle=False)
    tiny = W.random_case(904, [2], n_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16")
    check_pair(tiny, 1)


def test_noalloc_rejects_sizes_past_the_scratch():
    case = W.random_case(905, [64], n_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16")
    t = W.make_tensors(case, device="cuda")
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token)
    limit = 32 << 20
    per_split = B.pkv_decode_workspace_bytes(1, 32, 128, 1)
    too_many = limit // per_split + 1
    assert B.pkv_decode_workspace_bytes(1, 32, 128, too_many) > limit
    before = bits(t["k_buffer"])
    out = torch.zeros_like(t["q"])
    with pytest.raises(B.PkvError) as e:
        B.pkv_paged_decode_store_noalloc(t["k_buffer"], t["v_buffer"], t["req_to_token"], 0,
                                         step.c, t["q"], t["k_new"], t["v_new"], case.sm_scale,
                                         too_many, out)
    assert e.value.status == B.PKV_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert np.array_equal(bits(t["k_buffer"]), before)   # nothing launched
    assert not out.any()
