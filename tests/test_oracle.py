"""Pins for the CPU fp64 oracle (no GPU).

Each test ties the oracle to something other than itself: a library routine
(torch's scaled_dot_product_attention and causal_lower_right bias in fp64, torch
index_put, numpy cumsum), a closed form, a hand-derived fixture under
tests/golden/, or an invariant the mathematics fixes (slot permutation,
contiguous vs paged mapping, split independence, GQA = MHA on repeated heads).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def np_tensors(case, poison=True):
    t = W.make_tensors(case, device="cpu", poison=poison)
    out = {}
    for k, v in t.items():
        if v.dtype == torch.bfloat16:
            v = v.float()
        out[k] = v.numpy()
    return out


def store_new(case, t):
    """Apply the step's K/V write so the pool holds the new tokens."""
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    kb, vb = oracle.kv_store(t["k_buffer"], t["v_buffer"], case.layer_id, md["out_cache_loc"],
                             t["k_new"], t["v_new"])
    return kb, vb, md


def run_decode(case, t):
    kb, vb, _ = store_new(case, t)
    return oracle.decode(kb, vb, case.layer_id, case.req_to_token, case.req_pool_indices,
                         case.seq_lens, t["q"], case.sm_scale)


def sdpa_dense(q, K, V, scale, causal=False, lower_right=False):
    """torch SDPA in fp64 on CPU. q [H, R, d], K/V [Hk, n, d]."""
    q = torch.from_numpy(np.asarray(q, np.float64))[None]
    K = torch.from_numpy(np.asarray(K, np.float64))[None]
    V = torch.from_numpy(np.asarray(V, np.float64))[None]
    mask = None
    if lower_right:
        from torch.nn.attention.bias import causal_lower_right
        mask = causal_lower_right(q.shape[2], K.shape[2])
        out = F.scaled_dot_product_attention(
            q, torch.repeat_interleave(K, q.shape[1] // K.shape[1], dim=1),
            torch.repeat_interleave(V, q.shape[1] // K.shape[1], dim=1), attn_mask=mask,
            scale=scale)
        return out[0].numpy()
    out = F.scaled_dot_product_attention(q, K, V, is_causal=causal, scale=scale, enable_gqa=True)
    return out[0].numpy()


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,Hk,d", [(4, 2, 64), (8, 8, 32), (8, 2, 16), (12, 2, 8), (16, 2, 128)])
def test_decode_matches_sdpa_fp64(H, Hk, d):
    case = W.random_case(11 + H + d, [1, 7, 33, 70], n_heads=H, n_kv_heads=Hk, head_dim=d)
    t = np_tensors(case)
    out = run_decode(case, t)
    kb, vb, _ = store_new(case, t)
    for b in range(case.batch):
        r, L = case.req_pool_indices[b], case.seq_lens[b]
        slots = case.req_to_token[r, :L]
        K = kb[0, slots].transpose(1, 0, 2)  # [Hk, L, d]
        V = vb[0, slots].transpose(1, 0, 2)
        ref = sdpa_dense(t["q"][b][:, None, :], K, V, case.sm_scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_decode_tiny_config_matches_sdpa_and_is_finite():
    case = W.tiny_decode_f32()
    t = np_tensors(case)
    assert np.isnan(t["k_buffer"][0, case.poison_slot]).all()
    out = run_decode(case, t)
    assert np.isfinite(out).all()
    kb, vb, _ = store_new(case, t)
    for b in range(2):
        slots = case.req_to_token[case.req_pool_indices[b], :case.seq_lens[b]]
        ref = sdpa_dense(t["q"][b][:, None, :], kb[0, slots].transpose(1, 0, 2),
                         vb[0, slots].transpose(1, 0, 2), case.sm_scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_decode_slot_permutation_bitwise():
    case = W.random_case(5, [3, 17, 40], n_heads=8, n_kv_heads=2, head_dim=32, size=80)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    rng = np.random.default_rng(0)
    pi = rng.permutation(case.size)           # new slot of old slot s is pi[s]
    kb2 = np.empty_like(kb)
    vb2 = np.empty_like(vb)
    kb2[:, pi] = kb
    vb2[:, pi] = vb
    table2 = pi[case.req_to_token].astype(np.int32)
    out2 = oracle.decode(kb2, vb2, 0, table2, case.req_pool_indices, case.seq_lens,
                         t["q"], case.sm_scale)
    assert np.array_equal(out, out2)


def test_contiguous_mapping_equals_paged_bitwise():
    lens = [5, 12, 9]
    maxs = 16
    cont = W.contiguous_case(3, lens, maxs, n_heads=4, n_kv_heads=2, head_dim=16)
    paged = W.random_case(3, lens, n_heads=4, n_kv_heads=2, head_dim=16, size=64)
    tc = np_tensors(cont, poison=False)
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 4, 16))
    # identical logical K/V in both layouts
    kp = np.full((1, paged.size, 2, 16), np.nan)
    vp = np.full((1, paged.size, 2, 16), np.nan)
    kc = tc["k_buffer"]
    vc = tc["v_buffer"]
    for b in range(3):
        for j in range(lens[b]):
            kp[0, paged.req_to_token[paged.req_pool_indices[b], j]] = kc[0, b * maxs + j]
            vp[0, paged.req_to_token[paged.req_pool_indices[b], j]] = vc[0, b * maxs + j]
    o1 = oracle.decode(kc, vc, 0, cont.req_to_token, cont.req_pool_indices, cont.seq_lens, q, 0.25)
    o2 = oracle.decode(kp, vp, 0, paged.req_to_token, paged.req_pool_indices, paged.seq_lens, q, 0.25)
    assert np.array_equal(o1, o2)


def test_single_token_context_returns_v():
    case = W.random_case(9, [1, 1], n_heads=6, n_kv_heads=3, head_dim=32)
    t = np_tensors(case)
    kb, vb, md = store_new(case, t)
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    for b in range(2):
        for h in range(6):
            assert np.array_equal(out[b, h], t["v_new"][b, h // 2].astype(np.float64))


def test_constant_v_returns_constant():
    case = W.random_case(4, [50, 300], n_heads=4, n_kv_heads=2, head_dim=8)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    vb[...] = 0.375
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"] * 3, case.sm_scale)
    assert np.max(np.abs(out - 0.375)) <= 1e-15 * 300


def test_zero_query_gives_mean_of_values():
    case = W.random_case(8, [13, 29], n_heads=4, n_kv_heads=4, head_dim=16)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    q = np.zeros_like(t["q"])
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        q, case.sm_scale)
    for b in range(2):
        slots = case.req_to_token[case.req_pool_indices[b], :case.seq_lens[b]]
        mean = vb[0, slots].astype(np.float64).mean(axis=0)  # [Hk, d]
        np.testing.assert_allclose(out[b], mean, rtol=0, atol=1e-14)


def test_two_keys_sigmoid_closed_form():
    rng = np.random.default_rng(3)
    d = 32
    q = rng.standard_normal(d)
    k = rng.standard_normal((2, d))
    v = rng.standard_normal((2, d))
    scale = 1 / math.sqrt(d)
    s0, s1 = scale * q @ k[0], scale * q @ k[1]
    sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    expect = sig * v[0] + (1 - sig) * v[1]
    np.testing.assert_allclose(oracle.attend(q, k, v, scale)[0], expect, rtol=0, atol=1e-14)


def test_gqa_equals_mha_on_repeated_kv_heads():
    case = W.random_case(12, [9, 21], n_heads=8, n_kv_heads=2, head_dim=16, size=64)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    # expand kv-head c to heads 4c .. 4c+3 and run as MHA
    kb_m = np.repeat(kb, 4, axis=2)
    vb_m = np.repeat(vb, 4, axis=2)
    out_m = oracle.decode(kb_m, vb_m, 0, case.req_to_token, case.req_pool_indices,
                          case.seq_lens, t["q"], case.sm_scale)
    # the oracle batches a kv-head's query heads into one product, so only the
    # summation order may differ
    np.testing.assert_allclose(out, out_m, rtol=0, atol=1e-14)


@pytest.mark.parametrize("S", [1, 2, 7, 64, "L", "random"])
def test_split_independence(S):
    case = W.random_case(21, [1, 5, 64, 150], n_heads=4, n_kv_heads=2, head_dim=16)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    ref = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    rng = np.random.default_rng(1)

    def edges(b):
        L = int(case.seq_lens[b])
        if S == "L":
            return list(range(L + 1))
        if S == "random":
            cuts = sorted(rng.integers(0, L + 1, size=6).tolist())  # may repeat: empty splits
            return [0] + cuts + [L, L]
        chunk = -(-L // S) if S else L
        e = [min(L, i * chunk) for i in range(S + 1)]
        e[-1] = L
        return e

    out = oracle.decode_split(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                              t["q"], case.sm_scale, edges)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_merge_ignores_empty_splits():
    o = np.arange(4.0)
    out = oracle.merge_partials([oracle.NEG_INF, 1.5, oracle.NEG_INF], [0.0, 2.0, 0.0],
                                [np.full(4, np.nan), o, np.full(4, np.nan)])
    assert np.array_equal(out, o)


def test_hand_derived_golden_decode():
    g = json.load(open(os.path.join(GOLDEN, "decode_two_keys.json")))
    d = g["head_dim"]
    kb = np.full((1, g["pool_size"], 1, d), np.nan)
    vb = np.full((1, g["pool_size"], 1, d), np.nan)
    for s, row in g["k_slots"].items():
        kb[0, int(s), 0] = row
    for s, row in g["v_slots"].items():
        vb[0, int(s), 0] = row
    q = np.array(g["q_ln3_multiple"], dtype=np.float64)[None, None, :] * math.log(3.0)
    out = oracle.decode(kb, vb, 0, np.array(g["req_to_token"]), g["req_pool_indices"],
                        g["seq_lens"], q, g["sm_scale"])
    np.testing.assert_allclose(out[0, 0], g["expected_out"], rtol=0, atol=1e-13)


def test_oracle_never_reads_past_seq_len():
    case = W.random_case(31, [4, 9], n_heads=2, n_kv_heads=1, head_dim=8, size=40, max_ctx_len=30)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    # every unreferenced slot, and the poison slot unused table entries point at, is NaN
    assert np.isnan(kb[0, case.poison_slot]).all()
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    assert np.isfinite(out).all()


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def prefill_case(seed, q_lens, prefix, H=4, Hk=2, d=16):
    lens = [a + b for a, b in zip(q_lens, prefix)]
    return W.random_case(seed, lens, q_lens, n_heads=H, n_kv_heads=Hk, head_dim=d)


def run_prefill(case, t, causal=True):
    kb, vb, md = store_new(case, t)
    out = oracle.prefill(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                         md["qo_indptr"], t["q"], case.sm_scale, causal=causal)
    return out, kb, vb, md


def test_prefill_no_prefix_equals_causal_sdpa():
    case = prefill_case(41, [7, 1, 30], [0, 0, 0], H=6, Hk=2)
    t = np_tensors(case)
    out, kb, vb, md = run_prefill(case, t)
    qo = md["qo_indptr"]
    for i in range(case.batch):
        slots = case.req_to_token[case.req_pool_indices[i], :case.seq_lens[i]]
        qi = t["q"][qo[i]:qo[i + 1]].transpose(1, 0, 2)
        ref = sdpa_dense(qi, kb[0, slots].transpose(1, 0, 2), vb[0, slots].transpose(1, 0, 2),
                         case.sm_scale, causal=True)
        np.testing.assert_allclose(out[qo[i]:qo[i + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_prefill_with_prefix_equals_lower_right_causal_sdpa():
    case = prefill_case(42, [5, 16, 3, 1], [9, 4, 0, 20], H=8, Hk=2)
    t = np_tensors(case)
    out, kb, vb, md = run_prefill(case, t)
    qo = md["qo_indptr"]
    for i in range(case.batch):
        slots = case.req_to_token[case.req_pool_indices[i], :case.seq_lens[i]]
        qi = t["q"][qo[i]:qo[i + 1]].transpose(1, 0, 2)
        ref = sdpa_dense(qi, kb[0, slots].transpose(1, 0, 2), vb[0, slots].transpose(1, 0, 2),
                         case.sm_scale, lower_right=True)
        np.testing.assert_allclose(out[qo[i]:qo[i + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_prefill_non_causal_equals_sdpa():
    case = prefill_case(43, [6, 2], [3, 11])
    t = np_tensors(case)
    out, kb, vb, md = run_prefill(case, t, causal=False)
    qo = md["qo_indptr"]
    for i in range(case.batch):
        slots = case.req_to_token[case.req_pool_indices[i], :case.seq_lens[i]]
        qi = t["q"][qo[i]:qo[i + 1]].transpose(1, 0, 2)
        ref = sdpa_dense(qi, kb[0, slots].transpose(1, 0, 2), vb[0, slots].transpose(1, 0, 2),
                         case.sm_scale)
        np.testing.assert_allclose(out[qo[i]:qo[i + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_prefill_rows_equal_decode_at_each_position():
    case = prefill_case(44, [6, 1, 11], [5, 0, 2], H=4, Hk=1)
    t = np_tensors(case)
    out, kb, vb, md = run_prefill(case, t)
    qo = md["qo_indptr"]
    for i in range(case.batch):
        p = int(case.seq_lens[i] - case.q_lens[i])
        for tt in range(int(case.q_lens[i])):
            dec = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices[i:i + 1],
                                [p + tt + 1], t["q"][qo[i] + tt][None], case.sm_scale)
            assert np.array_equal(out[qo[i] + tt], dec[0])


def test_prefill_rows_sampler_matches_full():
    case = prefill_case(45, [9, 4], [3, 6], H=4, Hk=2)
    t = np_tensors(case)
    out, kb, vb, md = run_prefill(case, t)
    rows = [(0, 0), (3, 1), (8, 3), (9, 2), (12, 0)]
    got = oracle.prefill_rows(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                              md["qo_indptr"], t["q"], case.sm_scale, rows)
    for n, (tok, h) in enumerate(rows):
        np.testing.assert_allclose(got[n], out[tok, h], rtol=0, atol=1e-14)


def test_prefill_empty_request_rows():
    case = prefill_case(46, [0, 5, 0], [4, 2, 7])
    t = np_tensors(case)
    out, *_ = run_prefill(case, t)
    assert out.shape[0] == 5 and np.isfinite(out).all()


# ---------------------------------------------------------------------------
# kv_store and step metadata
# ---------------------------------------------------------------------------
def test_kv_store_matches_index_put_and_leaves_rest_untouched():
    case = W.random_case(51, [3, 8, 2], [2, 3, 1], n_heads=4, n_kv_heads=2, head_dim=8,
                         n_layers=3, layer_id=1)
    t = W.make_tensors(case, poison=False)
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    kb, vb = oracle.kv_store(t["k_buffer"].numpy(), t["v_buffer"].numpy(), 1, md["out_cache_loc"],
                             t["k_new"].numpy(), t["v_new"].numpy())
    ref_k = t["k_buffer"].clone()
    ref_k[1].index_put_((torch.from_numpy(md["out_cache_loc"]).long(),), t["k_new"])
    assert kb.tobytes() == ref_k.numpy().tobytes()
    # rows not written keep their bytes; written rows equal the inputs bitwise
    loc = set(md["out_cache_loc"].tolist())
    for layer in range(3):
        for s in range(case.size):
            if layer == 1 and s in loc:
                continue
            assert kb[layer, s].tobytes() == t["k_buffer"][layer, s].numpy().tobytes()
            assert vb[layer, s].tobytes() == t["v_buffer"][layer, s].numpy().tobytes()
    for i, s in enumerate(md["out_cache_loc"]):
        assert vb[1, s].tobytes() == t["v_new"][i].numpy().tobytes()


def test_build_step_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "step_metadata.json")))
    md = oracle.build_step(g["req_pool_indices"], g["seq_lens"], np.array(g["req_to_token"]),
                           g["q_lens"])
    for key in ("kv_indptr", "qo_indptr", "out_cache_loc", "prefill_order"):
        assert md[key].tolist() == g[key], key
        assert md[key].dtype == np.int32
    for key in ("max_len", "max_q_len", "n_new"):
        assert md[key] == g[key]


def test_build_step_prefix_sums_match_numpy_cumsum():
    case = W.batched_prefix_decode(B=16, hi=600, lo=10, shared=64, size=20000)
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token)
    assert md["kv_indptr"].tolist() == [0] + np.cumsum(case.seq_lens).tolist()
    assert md["qo_indptr"].tolist() == list(range(17))
    # decode writes the last position, which is always a private slot
    shared = set()
    for b in range(16):
        shared |= set(case.req_to_token[b, :min(64, int(case.seq_lens[b]) - 1)].tolist())
    assert not (set(md["out_cache_loc"].tolist()) & shared)


def test_validate_step_accepts_good_and_rejects_each_corruption():
    case = W.random_case(61, [4, 9, 6], [1, 3, 6], n_heads=4, n_kv_heads=2, head_dim=8)
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)

    def check(**over):
        a = dict(size=case.size, num_reqs=case.num_reqs, max_ctx_len=case.max_ctx_len,
                 req_to_token=case.req_to_token, req_pool_indices=case.req_pool_indices,
                 seq_lens=case.seq_lens, kv_indptr=md["kv_indptr"], qo_indptr=md["qo_indptr"],
                 out_cache_loc=md["out_cache_loc"])
        a.update(over)
        return oracle.validate_step(**a)[0]

    assert check()
    bad_loc = md["out_cache_loc"].copy(); bad_loc[1] = bad_loc[0]
    assert not check(out_cache_loc=bad_loc)
    bad_loc = md["out_cache_loc"].copy(); bad_loc[2] = case.size
    assert not check(out_cache_loc=bad_loc)
    bad_kv = md["kv_indptr"].copy(); bad_kv[2] += 1
    assert not check(kv_indptr=bad_kv)
    bad_rows = case.req_pool_indices.copy(); bad_rows[0] = case.num_reqs
    assert not check(req_pool_indices=bad_rows)
    bad_lens = case.seq_lens.copy(); bad_lens[0] = 0
    assert not check(seq_lens=bad_lens)
    bad_table = case.req_to_token.copy(); bad_table[case.req_pool_indices[1], 0] = -1
    assert not check(req_to_token=bad_table)
    bad_qo = md["qo_indptr"].copy(); bad_qo[1] = 5   # q_len 5 > seq_len 4
    assert not check(qo_indptr=bad_qo)
