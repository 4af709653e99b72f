"""Parity of the fused rotary + K/V write (pkv_rope_kv_store) against the
oracle (oracle/rope.py) on the same seeded inputs.

Tolerance: the kernel rotates in fp32 and rounds once to the pool dtype; the
oracle rotates in fp64 and rounds once.  The two may differ only where the
fp32 error moves a value across a rounding boundary: bf16 results within one
bf16 step of the oracle (plus 2^-20 of the row's largest input, for
cancellation), fp32 results within 2^-22 of the row's largest input; at
least 99.9% of bf16 elements are identical.  Values are copied bit for bit,
and no other byte of the pool changes."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from paged_kv_attention_12_amd import api
from tests.gpu_util import say, to_np

pytestmark = pytest.mark.gpu


def bits(t):
    t = t.contiguous()
    return (t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)).cpu().numpy()


def check_rotated(got, ref, x_in, dtype, what):
    """got, ref, x_in: [n, heads, d] fp64 arrays (x_in the unrotated input)."""
    scale = np.abs(x_in).max(axis=-1, keepdims=True)
    err = np.abs(got - ref)
    if dtype == "bf16":
        mag = np.maximum(np.abs(ref), 2.0 ** -126)
        step = np.ldexp(1.0, np.frexp(mag)[1] - 8)      # bf16 spacing at ref
        bound = step + 2.0 ** -20 * scale
        exact = float((got == ref).mean()) if got.size else 1.0
        assert exact >= 0.999, f"{what}: only {exact:.5f} of elements identical"
    else:
        bound = 2.0 ** -22 * scale + 1e-30
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the bound, worst {err.max():.3e}"


def run_case(case, max_pos=None, in_place=False):
    t = W.make_tensors(case, device="cuda")
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token,
                          None if case.is_decode else case.q_lens)
    max_pos = max_pos or case.max_ctx_len
    freqs = W.rope_table(max_pos, case.head_dim, device="cuda")
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token,
                           None if case.is_decode else case.q_lens)
    # the oracle's inputs, copied before any library call
    kb0, vb0 = bits(t["k_buffer"]), bits(t["v_buffer"])
    q0, kn0, vn0 = to_np(t["q"]), to_np(t["k_new"]), to_np(t["v_new"])
    f0 = freqs.cpu().numpy()
    q_out = t["q"] if in_place else torch.empty_like(t["q"])
    api.rope_kv_store(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id, step, t["q"],
                      t["k_new"], t["v_new"], freqs, q_out=q_out)
    torch.cuda.synchronize()
    pos = md["position_ids"]
    locs = md["out_cache_loc"]
    q_ref = oracle.to_dtype(oracle.rope_rotate(q0, pos, f0), case.dtype)
    k_ref = oracle.to_dtype(oracle.rope_rotate(kn0, pos, f0), case.dtype)
    what = f"{case.name} {case.dtype} H={case.n_heads} Hk={case.n_kv_heads} d={case.head_dim}"
    check_rotated(to_np(q_out).astype(np.float64), q_ref, q0, case.dtype, what + " q")
    kb = t["k_buffer"][case.layer_id].index_select(0, torch.from_numpy(locs.astype(np.int64)).cuda())
    check_rotated(to_np(kb).astype(np.float64), k_ref, kn0, case.dtype, what + " k")
    # values bit for bit, and no other byte of either pool changed
    kb1, vb1 = bits(t["k_buffer"]), bits(t["v_buffer"])
    vn_bits = bits(t["v_new"])
    assert np.array_equal(vb1[case.layer_id, locs], vn_bits)
    keep = np.ones(case.size, dtype=bool)
    keep[locs] = False
    for L in range(case.n_layers):
        rows = keep if L == case.layer_id else slice(None)
        assert np.array_equal(kb1[L, rows], kb0[L, rows]), f"{what}: k pool changed outside the write"
        assert np.array_equal(vb1[L, rows], vb0[L, rows]), f"{what}: v pool changed outside the write"
    return t, q_out


MATRIX = [
    # (H, Hk, d, dtype, seq_lens, q_lens)
    (32, 8, 128, "bf16", [1, 100, 2049], None),              # decode
    (32, 8, 128, "bf16", [300, 40, 1000], [300, 7, 129]),    # ragged prefill with prefixes
    (8, 2, 64, "bf16", [17, 5, 64], [17, 1, 33]),
    (12, 2, 128, "f32", [33, 9], [4, 9]),
    (4, 4, 64, "f32", [1, 2, 3], None),
]


@pytest.mark.parametrize("H,Hk,d,dtype,lens,qls", MATRIX)
def test_rope_kv_store_matches_oracle(H, Hk, d, dtype, lens, qls):
    case = W.random_case(900 + H + d + len(lens), lens, qls, n_heads=H, n_kv_heads=Hk, head_dim=d,
                         dtype=dtype, n_layers=2, layer_id=1)
    say("rope", H, Hk, d, dtype, lens, qls)
    run_case(case)


def test_rope_in_place_queries():
    case = W.random_case(950, [50, 3], [50, 1], n_heads=16, n_kv_heads=4, head_dim=128,
                         dtype="bf16")
    run_case(case, in_place=True)


def test_rope_last_table_row():
    """Positions up to max_pos - 1: a table exactly as long as the longest
    context."""
    case = W.random_case(951, [64, 64], [64, 1], n_heads=8, n_kv_heads=2, head_dim=64, dtype="bf16")
    run_case(case, max_pos=64)


def test_rope_empty_step_is_a_no_op():
    case = W.random_case(952, [5], [0], n_heads=8, n_kv_heads=2, head_dim=64, dtype="bf16")
    t = W.make_tensors(case, device="cuda")
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    kb0 = bits(t["k_buffer"])
    freqs = W.rope_table(8, 64, device="cuda")
    api.rope_kv_store(t["k_buffer"], t["v_buffer"], t["req_to_token"], 0, step, t["q"],
                      t["k_new"], t["v_new"], freqs)
    torch.cuda.synchronize()
    assert np.array_equal(bits(t["k_buffer"]), kb0)


def test_rope_graph_replay_matches_eager():
    case = W.random_case(953, [700, 30], [700, 1], n_heads=32, n_kv_heads=8, head_dim=128,
                         dtype="bf16")
    t = W.make_tensors(case, device="cuda")
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    freqs = W.rope_table(case.max_ctx_len, 128, device="cuda")
    q_out = torch.empty_like(t["q"])
    run = lambda: api.rope_kv_store(t["k_buffer"], t["v_buffer"], t["req_to_token"], 0, step,
                                    t["q"], t["k_new"], t["v_new"], freqs, q_out=q_out)
    run()
    torch.cuda.synchronize()
    eager_q, eager_k = q_out.clone(), bits(t["k_buffer"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        q_out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_out, eager_q)
        assert np.array_equal(bits(t["k_buffer"]), eager_k)
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_rope_ragged_prefill_workload_sampled():
    """The 16-request prefill workload at full size; every key row and a
    sample of query rows against the oracle."""
    case = W.ragged_prefill()
    say("rope ragged prefill workload")
    t = W.make_tensors(case, device="cuda", poison=False)
    step = api.DeviceStep(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    freqs = W.rope_table(case.max_ctx_len, case.head_dim, device="cuda")
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(step.n_new, size=min(step.n_new, 512), replace=False))
    q0 = to_np(t["q"][torch.from_numpy(rows).cuda()])
    kn0 = to_np(t["k_new"])
    f0 = freqs.cpu().numpy()
    q_out = api.rope_kv_store(t["k_buffer"], t["v_buffer"], t["req_to_token"], case.layer_id, step,
                              t["q"], t["k_new"], t["v_new"], freqs)
    torch.cuda.synchronize()
    pos = md["position_ids"]
    q_ref = oracle.to_dtype(oracle.rope_rotate(q0, pos[rows], f0), case.dtype)
    check_rotated(to_np(q_out[torch.from_numpy(rows).cuda()]).astype(np.float64), q_ref, q0,
                  case.dtype, "prefill workload q")
    k_ref = oracle.to_dtype(oracle.rope_rotate(kn0, pos, f0), case.dtype)
    locs = torch.from_numpy(md["out_cache_loc"].astype(np.int64)).cuda()
    kb = to_np(t["k_buffer"][case.layer_id].index_select(0, locs)).astype(np.float64)
    check_rotated(kb, k_ref, kn0, case.dtype, "prefill workload k")
