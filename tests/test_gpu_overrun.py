"""Decode lengths that outgrow the step's bounds on the device, as they do when
a captured step is replayed with pkv_decode_advance moving the metadata:

  * past num_splits * split size (the host max_len was too small): the last
    split takes the excess and the output still equals the oracle's;
  * past max_ctx_len (the table row cannot address the position): every head
    of that request is NaN, the other requests are unaffected, and the one-
    and two-launch steps leave the pool untouched."""

import numpy as np
import pytest
import torch

import workloads as W
from paged_kv_attention_12_amd import api
from paged_kv_attention_12_amd import binding as B
from tests.gpu_util import HostView, assert_close, say, to_np

pytestmark = pytest.mark.gpu

FORMS = ["three", "stored", "fused"]


def bits(t):
    t = t.contiguous()
    return (t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)).cpu().numpy()


def run_form(form, case, t, step, ns):
    args = (t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id, step, t["q"],
            t["k_new"], t["v_new"], case.sm_scale)
    if form == "three":
        return api.decode_step(*args, num_splits=ns)
    if form == "stored":
        return api.stored_decode_step(*args, num_splits=ns)
    return api.fused_decode_step(*args, num_splits=ns)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("H,Hk,d,dtype", [(32, 8, 128, "bf16"), (8, 2, 64, "bf16"),
                                          (8, 2, 128, "f32")])
def test_lengths_past_the_split_bound_are_attended_whole(form, H, Hk, d, dtype):
    case = W.random_case(950 + H + d, [140, 60, 333], n_heads=H, n_kv_heads=Hk, head_dim=d,
                         dtype=dtype, n_layers=2, layer_id=1)
    say("overrun split bound", form, H, Hk, d, dtype)
    t = W.make_tensors(case, device="cuda")
    hv = HostView(case, t)
    ref = hv.decode_all(case)
    grow = 45
    lens = [int(L) - grow for L in case.seq_lens]
    step = api.DeviceStep(case.req_pool_indices, lens, case.req_to_token)
    assert step.max_len == max(lens)
    for _ in range(grow):
        api.advance_decode(t["k_buffer"], t["v_buffer"], t["req_to_token"], step)
    torch.cuda.synchronize()
    assert step.seq_lens.cpu().tolist() == [int(x) for x in case.seq_lens]
    ns = 4
    # the split size comes from the stale host max_len: 4 splits of it cover
    # less than the longest request now holds
    chunk = max(16, (-(-step.max_len // ns) + 15) // 16 * 16)
    assert ns * chunk < int(max(case.seq_lens))
    out = run_form(form, case, t, step, ns)
    assert_close(to_np(out), ref, dtype, f"{form} past the split bound")


@pytest.mark.parametrize("form", FORMS)
def test_length_past_max_ctx_len_gives_nan_and_no_write(form):
    # request 0's table row holds exactly 50 positions; request 1 has room
    case = W.random_case(960, [50, 30], n_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
                         max_ctx_len=50)
    say("overrun max_ctx_len", form)
    t = W.make_tensors(case, device="cuda")
    lens = [50, 29]
    step = api.DeviceStep(case.req_pool_indices, lens, case.req_to_token)
    api.advance_decode(t["k_buffer"], t["v_buffer"], t["req_to_token"], step)
    torch.cuda.synchronize()
    assert step.seq_lens.cpu().tolist() == [51, 30]
    # the oracle's reference for request 1 (length 30, its new token written)
    case1 = W.random_case(960, [50, 30], n_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
                          max_ctx_len=50)
    hv = HostView(case1, t, requests=[1])
    ref1 = hv.decode_pairs(case1, [(1, h) for h in range(32)])
    k_before, v_before = bits(t["k_buffer"]), bits(t["v_buffer"])
    out = run_form(form, case, t, step, 3)
    torch.cuda.synchronize()
    o = to_np(out)
    assert np.isnan(o[0]).all(), "request past max_ctx_len must come out NaN"
    assert_close(o[1], ref1, "bf16", f"{form}: the other request")
    if form in ("stored", "fused"):
        # no write for the request past its row; request 1's new token written
        kb, vb = bits(t["k_buffer"]), bits(t["v_buffer"])
        loc1 = int(case.req_to_token[case.req_pool_indices[1], 29])
        changed = np.nonzero((kb != k_before).any(axis=(2, 3)).ravel())[0].tolist()
        assert changed in ([], [loc1]), changed
        assert np.array_equal(np.delete(kb[0], loc1, axis=0), np.delete(k_before[0], loc1, axis=0))
        assert np.array_equal(np.delete(vb[0], loc1, axis=0), np.delete(v_before[0], loc1, axis=0))
