"""K/V rows read with non-temporal loads (pkv_pool.load_policy =
PKV_LOAD_STREAM) against cached loads (PKV_LOAD_CACHED), through the C ABI:
the load kind is a cache hint only, so

  * the split partials and the merged output of pkv_paged_decode +
    pkv_paged_decode_merge,
  * the output and both pools after pkv_paged_decode_store (split kernel with
    the new token's write, then the merge),
  * the output and both pools after pkv_paged_decode_rope_store (the same
    with the rotary turn folded in)

are the same bits under both policies, on ragged and single requests,
16-token pages, MLA-shaped keys (192 wide, values 128) and an fp32 pool of
64-wide rows (whose vector kernels ignore the policy); the streamed output
meets the CPU fp64 oracle at the pool dtype's tolerance; and the headline
shape (one request of 32768 keys on a 32-layer pool), where PKV_LOAD_AUTO
streams, gives the bits of PKV_LOAD_CACHED."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from paged_kv_attention_12_amd import api
from paged_kv_attention_12_amd import binding as B
from tests.gpu_util import assert_close, say, to_np

pytestmark = pytest.mark.gpu


def bits(t):
    t = t.contiguous()
    return (t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)).cpu().numpy()


CASES = {
    "ragged": (lambda: W.random_case(1200, [1, 40, 900, 3000], n_heads=32, n_kv_heads=8,
                                     head_dim=128, dtype="bf16"), 9),
    "single": (lambda: W.random_case(1201, [4097], n_heads=32, n_kv_heads=8, head_dim=128,
                                     dtype="bf16"), 16),
    "pages16": (lambda: W.random_paged_case(1202, [16, 33, 700], 16, n_heads=16, n_kv_heads=4,
                                            head_dim=128, dtype="bf16"), 5),
    "mla": (lambda: W.random_case(1203, [300, 77], n_heads=16, n_kv_heads=16, head_dim=192,
                                  v_head_dim=128, dtype="bf16"), 4),
    # the vector kernels (fp32, head_dim 64) read cached under every policy
    "f32_d64": (lambda: W.random_case(1204, [5, 130, 999], n_heads=8, n_kv_heads=2, head_dim=64,
                                      dtype="f32"), 6),
}


def run(case, form, policy, ns):
    t = W.make_tensors(case, device="cuda")
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token,
                          page_size=case.page_size)
    H = case.n_heads
    dv = int(t["v_buffer"].shape[3])
    ws = api.decode_workspace(case.batch, H, dv, ns)
    out = torch.empty((case.batch, H, dv), dtype=t["q"].dtype, device="cuda")
    args = (t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id, step.c)
    kw = dict(page_size=case.page_size, load_policy=policy)
    if form == "split":
        B.pkv_paged_decode(*args, t["q"], case.sm_scale, ns, ws, **kw)
        B.pkv_paged_decode_merge(case.batch, H, dv, ns, ws, out)
    elif form == "store":
        B.pkv_paged_decode_store(*args, t["q"], t["k_new"], t["v_new"], case.sm_scale, ns, ws,
                                 out, **kw)
    else:
        freqs = W.rope_table(int(case.seq_lens.max()), case.head_dim, device="cuda")
        B.pkv_paged_decode_rope_store(*args, t["q"], t["k_new"], t["v_new"], step.position_ids,
                                      freqs, case.sm_scale, ns, ws, out, **kw)
    torch.cuda.synchronize()
    res = {"out": bits(out), "k": bits(t["k_buffer"]), "v": bits(t["v_buffer"])}
    if form == "split":
        res["ws"] = bits(ws)
    return res, t, out


# the rotary step takes bf16 pools with 128-wide keys and values only
PAIRS = [(n, f) for n in CASES for f in ("split", "store", "rope")
         if not (n in ("mla", "f32_d64") and f == "rope")]


@pytest.mark.parametrize("name,form", PAIRS)
def test_streamed_rows_give_the_bits_of_cached_rows(name, form):
    make, ns = CASES[name]
    case = make()
    say("load policy", name, form, "splits", ns)
    cached, _, _ = run(case, form, B.PKV_LOAD_CACHED, ns)
    streamed, t, out = run(case, form, B.PKV_LOAD_STREAM, ns)
    for k in cached:
        assert np.array_equal(cached[k], streamed[k]), f"{name} {form}: {k} differs"
    if form == "store":
        # and against the oracle: the write, then the attention
        t0 = W.make_tensors(case, device="cuda")   # the same seeded pools, before the write
        kb0 = to_np(t0["k_buffer"][case.layer_id])[None]
        vb0 = to_np(t0["v_buffer"][case.layer_id])[None]
        del t0
        if case.page_size == 1:
            md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token)
            kb, vb = oracle.kv_store(kb0, vb0, 0, md["out_cache_loc"], to_np(t["k_new"]),
                                     to_np(t["v_new"]))
            ref = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices,
                                case.seq_lens, to_np(t["q"]), case.sm_scale)
        else:
            import oracle.pages as OP
            kb, vb = OP.write(kb0, vb0, 0, case.req_to_token, case.page_size,
                              case.req_pool_indices, case.seq_lens, np.ones(case.batch, np.int64),
                              to_np(t["k_new"]), to_np(t["v_new"]))
            ref = OP.decode(kb, vb, 0, case.req_to_token, case.page_size, case.req_pool_indices,
                            case.seq_lens, to_np(t["q"]), case.sm_scale)
        assert_close(to_np(out), ref, case.dtype, f"{name} streamed store step vs oracle")


def test_auto_policy_at_the_headline_shape():
    """One request of 32768 keys on a 32-layer Llama-shaped pool: AUTO picks
    non-temporal loads (its K/V over all layers are 4.3 GB), and the two-launch
    step gives the bits of the cached form."""
    case = W.llama_b1_decode(32768)
    t = W.make_tensors(case, device="cuda", poison=False)
    pool = B.make_pool(t["k_buffer"], t["v_buffer"], t["req_to_token"])
    assert B.pkv_decode_load_kind(pool, 1, 32768) == 1
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token)
    ns = B.pkv_decode_pick_splits(1, case.n_kv_heads, case.n_heads, step.max_len, step.total_len)
    ws = api.decode_workspace(1, case.n_heads, case.head_dim, ns)
    outs = []
    for policy in (B.PKV_LOAD_AUTO, B.PKV_LOAD_CACHED):
        out = torch.empty_like(t["q"])
        B.pkv_paged_decode_store(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id,
                                 step.c, t["q"], t["k_new"], t["v_new"], case.sm_scale, ns, ws,
                                 out, load_policy=policy)
        torch.cuda.synchronize()
        outs.append(bits(out))
    assert np.array_equal(outs[0], outs[1])
