"""Pins for the oracle on MLA-shaped layers (no GPU): keys and queries of
qk_nope + qk_rope dims, values of their own width, rotation on the last
qk_rope dims only.

Ties: torch scaled_dot_product_attention in fp64 with a value width unlike
the key width (decode, causal and non-causal prefill, GQA and MHA), a
hand-worked fixture (tests/golden/mla_two_keys_partial_rope.json), the
full-row rotation restricted to the tail (and equal to it when the tail is
the whole row), and planted mistakes that must fail.
"""

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as OA
import oracle.rope as OR
import workloads as W
from tests.test_oracle import GOLDEN, np_tensors, store_new


def sdpa(q, K, V, scale, lower_right=False):
    """q [H, R, dk], K [Hk, n, dk], V [Hk, n, dv] -> [H, R, dv], torch fp64 CPU."""
    q = torch.from_numpy(np.asarray(q, np.float64))[None]
    K = torch.from_numpy(np.asarray(K, np.float64))[None]
    V = torch.from_numpy(np.asarray(V, np.float64))[None]
    G = q.shape[1] // K.shape[1]
    K = torch.repeat_interleave(K, G, dim=1)
    V = torch.repeat_interleave(V, G, dim=1)
    mask = None
    if lower_right:
        from torch.nn.attention.bias import causal_lower_right
        mask = causal_lower_right(q.shape[2], K.shape[2])
    return F.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=scale)[0].numpy()


@pytest.mark.parametrize("H,Hk", [(4, 4), (8, 2)])
def test_mla_decode_equals_sdpa(H, Hk):
    case = W.random_case(501, [1, 9, 40], n_heads=H, n_kv_heads=Hk, head_dim=24, v_head_dim=16)
    t = np_tensors(case)
    assert t["v_buffer"].shape[-1] == 16 and t["k_buffer"].shape[-1] == 24
    kb, vb, _ = store_new(case, t)
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    assert out.shape == (3, H, 16)
    for b in range(case.batch):
        slots = case.req_to_token[case.req_pool_indices[b], :case.seq_lens[b]]
        ref = sdpa(t["q"][b][:, None, :], kb[0, slots].transpose(1, 0, 2),
                   vb[0, slots].transpose(1, 0, 2), case.sm_scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_mla_prefill_equals_sdpa(causal):
    q_lens, prefix = [5, 1, 7], [0, 12, 3]
    lens = [a + b for a, b in zip(q_lens, prefix)]
    case = W.random_case(502, lens, q_lens, n_heads=6, n_kv_heads=2, head_dim=24, v_head_dim=8)
    t = np_tensors(case)
    kb, vb, md = store_new(case, t)
    out = oracle.prefill(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                         md["qo_indptr"], t["q"], case.sm_scale, causal=causal)
    assert out.shape == (md["n_new"], 6, 8)
    qo = md["qo_indptr"]
    for i in range(case.batch):
        slots = case.req_to_token[case.req_pool_indices[i], :case.seq_lens[i]]
        ref = sdpa(t["q"][qo[i]:qo[i + 1]].transpose(1, 0, 2), kb[0, slots].transpose(1, 0, 2),
                   vb[0, slots].transpose(1, 0, 2), case.sm_scale, lower_right=causal)
        np.testing.assert_allclose(out[qo[i]:qo[i + 1]], ref.transpose(1, 0, 2), rtol=0,
                                   atol=1e-12)
    rows = [(0, 0), (5, 3), (12, 5)]
    got = oracle.prefill_rows(kb, vb, 0, case.req_to_token, case.req_pool_indices,
                              case.seq_lens, qo, t["q"], case.sm_scale, rows, causal=causal)
    np.testing.assert_allclose(got, np.stack([out[a, h] for a, h in rows]), rtol=0, atol=1e-14)


def golden():
    return json.load(open(os.path.join(GOLDEN, "mla_two_keys_partial_rope.json")))


def golden_attention_holds() -> bool:
    g = golden()
    kb = np.full((1, g["pool_size"], 1, g["head_dim"]), np.nan)
    vb = np.full((1, g["pool_size"], 1, g["v_head_dim"]), np.nan)
    for s, row in g["k_slots"].items():
        kb[0, int(s), 0] = row
    for s, row in g["v_slots"].items():
        vb[0, int(s), 0] = row
    q = np.array(g["q_ln3_multiple"])[None, None, :] * np.log(3.0)
    out = oracle.decode(kb, vb, 0, np.array(g["req_to_token"]), g["req_pool_indices"],
                        g["seq_lens"], q, 1.0)
    return bool(np.allclose(out[0, 0], g["expected_out"], rtol=0, atol=1e-13))


def golden_rope_holds() -> bool:
    g = golden()
    x = np.array(g["rope_row"])[None, None, :]
    f = np.array(g["rope_table_row"])[None]
    got = oracle.rope_rotate_tail(x, [0], f, g["rope_dim"])
    return bool(np.allclose(got[0, 0], g["rope_expected"], rtol=0, atol=1e-15))


def test_mla_golden():
    assert golden_attention_holds()
    assert golden_rope_holds()


def test_tail_rotation_is_the_full_rotation_of_the_tail():
    rng = np.random.default_rng(503)
    x = rng.standard_normal((5, 3, 24))
    table = W.rope_table(40, 8).numpy()
    pos = [0, 3, 39, 17, 8]
    got = oracle.rope_rotate_tail(x, pos, table, 8)
    assert np.array_equal(got[:, :, :16], x[:, :, :16])          # qk_nope untouched
    assert np.array_equal(got[:, :, 16:], oracle.rope_rotate(x[:, :, 16:], pos, table))
    full = W.rope_table(40, 24).numpy()
    assert np.array_equal(oracle.rope_rotate_tail(x, pos, full, 24),
                          oracle.rope_rotate(x, pos, full))
    # rotation keeps the norm of every rope pair (to the fp32 table's c^2 + s^2)
    a, b = got[:, :, 16::2], got[:, :, 17::2]
    np.testing.assert_allclose(a * a + b * b, x[:, :, 16::2] ** 2 + x[:, :, 17::2] ** 2,
                               rtol=1e-6)


def test_partial_rope_kv_store_writes_rotated_keys_and_plain_values():
    case = W.random_case(504, [3, 6], [1, 2], n_heads=4, n_kv_heads=2, head_dim=24,
                         v_head_dim=16)
    t = np_tensors(case)
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    table = W.rope_table(8, 8).numpy()
    q_rot, kb, vb = oracle.rope_kv_store(t["k_buffer"], t["v_buffer"], 0, md["out_cache_loc"],
                                         t["q"], t["k_new"], t["v_new"], md["position_ids"],
                                         table, "f32", rope_dim=8)
    for i, loc in enumerate(md["out_cache_loc"]):
        p = [md["position_ids"][i]]
        want = oracle.to_dtype(oracle.rope_rotate_tail(t["k_new"][i:i + 1], p, table, 8), "f32")
        assert np.array_equal(kb[0, loc], want[0])
        assert np.array_equal(vb[0, loc], t["v_new"][i])
    np.testing.assert_array_equal(q_rot[:, :, :16], t["q"][:, :, :16])


# planted mistakes ------------------------------------------------------------
def test_planted_mla_mistakes_are_caught(monkeypatch):
    _rot = OR.rope_rotate

    def head_instead_of_tail(x, positions, freqs_cis, rope_dim):
        x = np.asarray(x, np.float64)
        out = x.copy()
        out[:, :, :rope_dim] = _rot(x[:, :, :rope_dim], positions, freqs_cis)
        return out
    monkeypatch.setattr(oracle, "rope_rotate_tail", head_instead_of_tail)
    assert not golden_rope_holds()
    monkeypatch.undo()

    _attend = OA.attend

    def values_cut_to_key_width(q, K, V, s, n_keys=None):
        # a plausible slip: value rows read with the key width's split point
        return _attend(q, K, V[:, ::-1], s, n_keys)
    monkeypatch.setattr(OA, "attend", values_cut_to_key_width)
    assert not golden_attention_holds()
