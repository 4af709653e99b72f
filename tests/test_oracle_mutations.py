"""Mistakes planted in the oracle (on the CPU) must be caught by its pins.

Each mutant patches one step of ``oracle.attention`` with a plausible error
(dropped scale, wrong GQA head, dropped or extra key, swapped operands, wrong
causal alignment, wrong merge weight, wrong write position) and checks that a
pin from test_oracle.py, re-run against the mutant, fails.
"""

import json
import os

import numpy as np
import pytest

import oracle
import oracle.attention as OA
import workloads as W
from tests.test_oracle import GOLDEN, np_tensors, sdpa_dense, store_new


def decode_matches_sdpa() -> bool:
    case = W.random_case(77, [1, 6, 40], n_heads=8, n_kv_heads=2, head_dim=16)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    out = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    for b in range(case.batch):
        slots = case.req_to_token[case.req_pool_indices[b], :case.seq_lens[b]]
        ref = sdpa_dense(t["q"][b][:, None, :], kb[0, slots].transpose(1, 0, 2),
                         vb[0, slots].transpose(1, 0, 2), case.sm_scale)[:, 0, :]
        if not np.allclose(out[b], ref, rtol=0, atol=1e-12):
            return False
    return True


def prefill_matches_lower_right() -> bool:
    case = W.random_case(78, [9, 20], [5, 16], n_heads=4, n_kv_heads=2, head_dim=16)
    t = np_tensors(case)
    kb, vb, md = store_new(case, t)
    out = oracle.prefill(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                         md["qo_indptr"], t["q"], case.sm_scale)
    qo = md["qo_indptr"]
    for i in range(case.batch):
        slots = case.req_to_token[case.req_pool_indices[i], :case.seq_lens[i]]
        ref = sdpa_dense(t["q"][qo[i]:qo[i + 1]].transpose(1, 0, 2),
                         kb[0, slots].transpose(1, 0, 2), vb[0, slots].transpose(1, 0, 2),
                         case.sm_scale, lower_right=True)
        if not np.allclose(out[qo[i]:qo[i + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12):
            return False
    return True


def split_independent() -> bool:
    case = W.random_case(79, [33, 90], n_heads=2, n_kv_heads=1, head_dim=8)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    ref = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"], case.sm_scale)
    out = oracle.decode_split(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                              t["q"], case.sm_scale,
                              lambda b: [0, 5, 5, int(case.seq_lens[b]) // 2, int(case.seq_lens[b])])
    return bool(np.allclose(out, ref, rtol=1e-12, atol=1e-13))


def golden_metadata_holds() -> bool:
    g = json.load(open(os.path.join(GOLDEN, "step_metadata.json")))
    md = oracle.build_step(g["req_pool_indices"], g["seq_lens"], np.array(g["req_to_token"]),
                           g["q_lens"])
    return md["out_cache_loc"].tolist() == g["out_cache_loc"] and \
        md["kv_indptr"].tolist() == g["kv_indptr"]


def golden_decode_holds() -> bool:
    g = json.load(open(os.path.join(GOLDEN, "decode_two_keys.json")))
    d = g["head_dim"]
    kb = np.full((1, g["pool_size"], 1, d), np.nan)
    vb = np.full((1, g["pool_size"], 1, d), np.nan)
    for s, row in g["k_slots"].items():
        kb[0, int(s), 0] = row
    for s, row in g["v_slots"].items():
        vb[0, int(s), 0] = row
    q = np.array(g["q_ln3_multiple"], dtype=np.float64)[None, None, :] * np.log(3.0)
    out = oracle.decode(kb, vb, 0, np.array(g["req_to_token"]), g["req_pool_indices"],
                        g["seq_lens"], q, g["sm_scale"])
    return bool(np.allclose(out[0, 0], g["expected_out"], rtol=0, atol=1e-13))


def test_unmutated_oracle_passes_every_pin():
    assert decode_matches_sdpa()
    assert prefill_matches_lower_right()
    assert split_independent()
    assert golden_metadata_holds()
    assert golden_decode_holds()


_attend = OA.attend
_gather = OA._gather
_split = OA.split_partial
_merge = OA.merge_partials
_build = OA.build_step


def m_no_scale(q, K, V, s, n_keys=None):
    return _attend(q, K, V, 1.0, n_keys)


def m_drop_last_key(q, K, V, s, n_keys=None):
    if n_keys is None:
        return _attend(q, K[:-1], V[:-1], s) if K.shape[0] > 1 else _attend(q, K, V, s)
    return _attend(q, K, V, s, [max(1, n - 1) for n in n_keys])


def m_swap_kv(q, K, V, s, n_keys=None):
    return _attend(q, V, K, s, n_keys)


def m_sign(q, K, V, s, n_keys=None):
    return _attend(q, K, V, -s, n_keys)


def m_head_map(buffer, layer_id, slots, hk):
    return _gather(buffer, layer_id, slots, (hk + 1) % buffer.shape[2])


def m_top_left(q, K, V, s, n_keys=None):
    # causal alignment to the start instead of the end of the context
    if n_keys is None or len(n_keys) < 2:
        return _attend(q, K, V, s, n_keys)
    base = min(n_keys) - 1
    return _attend(q, K, V, s, [n - base for n in n_keys])


def m_causal_off_by_one(q, K, V, s, n_keys=None):
    if n_keys is None or len(n_keys) < 2:
        return _attend(q, K, V, s, n_keys)
    return _attend(q, K, V, s, [n - 1 if n > 1 else n for n in n_keys])


def m_split_unnormalised(q, K, V, s, lo, hi):
    m, l, o = _split(q, K, V, s, lo, hi)
    return m, 1.0 if l > 0 else 0.0, o


def m_merge_no_exp(ms, ls, os):
    return _merge([0.0 if np.isfinite(m) else m for m in ms], ls, os)


def m_write_pos(req_pool_indices, seq_lens, req_to_token, q_lens=None):
    md = _build(req_pool_indices, seq_lens, req_to_token, q_lens)
    B = len(seq_lens)
    ql = [1] * B if q_lens is None else q_lens
    locs = []
    for b in range(B):
        for t in range(int(ql[b])):   # writes at the first positions instead of the last
            locs.append(int(req_to_token[int(req_pool_indices[b]), t]))
    md["out_cache_loc"] = np.array(locs, dtype=np.int32)
    return md


MUTANTS = [
    ("attend", m_no_scale, [decode_matches_sdpa, golden_decode_holds]),
    ("attend", m_drop_last_key, [decode_matches_sdpa, golden_decode_holds]),
    ("attend", m_swap_kv, [decode_matches_sdpa]),
    ("attend", m_sign, [decode_matches_sdpa, golden_decode_holds]),
    ("_gather", m_head_map, [decode_matches_sdpa]),
    ("attend", m_top_left, [prefill_matches_lower_right]),
    ("attend", m_causal_off_by_one, [prefill_matches_lower_right]),
    ("split_partial", m_split_unnormalised, [split_independent]),
    ("merge_partials", m_merge_no_exp, [split_independent]),
    ("build_step", m_write_pos, [golden_metadata_holds]),
]


@pytest.mark.parametrize("target,mutant,pins", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant, pins):
    monkeypatch.setattr(OA, target, mutant)
    if target == "build_step":
        monkeypatch.setattr(oracle, "build_step", mutant)
    for pin in pins:
        assert not pin(), f"{mutant.__name__} survived {pin.__name__}"
