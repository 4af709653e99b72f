"""Pins for the paged-pool oracle (page_size > 1), no GPU.

Each test ties ``oracle.pages`` to something other than itself: torch's
scaled_dot_product_attention in fp64 on K/V gathered the way the PagedCache of
the v1.3.3 -> v1.3.4 compare page gathers them (torch.cat of the request's
physical pages of a 5-D [n_layers, n_pages, page_size, Hk, d] cache, in
logical order), the one-token oracle at page_size 1, the contiguous layout,
invariance under a permutation of physical pages, a hand-worked fixture, and
planted mistakes that these pins must catch.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.pages as OP
import workloads as W
from tests.test_oracle import GOLDEN, np_tensors, sdpa_dense


def paged_store(case, t):
    kb, vb = OP.write(t["k_buffer"], t["v_buffer"], case.layer_id, case.req_to_token,
                      case.page_size, case.req_pool_indices, case.seq_lens, case.q_lens,
                      t["k_new"], t["v_new"])
    md = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token,
                       case.page_size, case.q_lens)
    return kb, vb, md


def torch_page_gather(buffer, layer_id, page_row, n_pages_used, page_size, L):
    """The pages' gather: concatenate the request's physical pages of the 5-D
    cache in logical order, then keep the first L positions.  -> [Hk, L, d]"""
    t = torch.from_numpy(np.ascontiguousarray(buffer))
    cache5 = t.view(t.shape[0], t.shape[1] // page_size, page_size, t.shape[2], t.shape[3])
    parts = [cache5[layer_id, int(page_row[p])] for p in range(n_pages_used)]
    kv = torch.cat(parts, dim=0)[:L]           # [L, Hk, d]
    return kv.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("ps,H,Hk,d", [(4, 4, 2, 16), (16, 8, 2, 32), (64, 6, 3, 8), (2, 8, 8, 16)])
def test_paged_decode_matches_sdpa_on_page_gather(ps, H, Hk, d):
    lens = [1, ps - 1 if ps > 1 else 1, ps, ps + 1, 3 * ps + 5]
    case = W.random_paged_case(20 + ps, lens, ps, n_heads=H, n_kv_heads=Hk, head_dim=d)
    t = np_tensors(case)
    kb, vb, _ = paged_store(case, t)
    out = OP.decode(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                    t["q"], case.sm_scale)
    assert np.isfinite(out).all()
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        row = case.req_to_token[case.req_pool_indices[b]]
        npg = -(-L // ps)
        K = torch_page_gather(kb, 0, row, npg, ps, L)
        V = torch_page_gather(vb, 0, row, npg, ps, L)
        ref = sdpa_dense(t["q"][b][:, None, :], K, V, case.sm_scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_paged_prefill_matches_lower_right_sdpa():
    ps = 8
    q_lens = [5, 16, 3, 1, 9]
    prefix = [9, 4, 0, 20, 16]
    lens = [p + q for p, q in zip(prefix, q_lens)]
    case = W.random_paged_case(31, lens, ps, q_lens=q_lens, n_heads=8, n_kv_heads=2, head_dim=16)
    t = np_tensors(case)
    kb, vb, md = paged_store(case, t)
    qo = md["qo_indptr"]
    out = OP.prefill(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                     qo, t["q"], case.sm_scale)
    full = OP.prefill(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                      qo, t["q"], case.sm_scale, causal=False)
    for i in range(case.batch):
        L = int(case.seq_lens[i])
        row = case.req_to_token[case.req_pool_indices[i]]
        K = torch_page_gather(kb, 0, row, -(-L // ps), ps, L)
        V = torch_page_gather(vb, 0, row, -(-L // ps), ps, L)
        qi = t["q"][qo[i]:qo[i + 1]].transpose(1, 0, 2)
        ref = sdpa_dense(qi, K, V, case.sm_scale, lower_right=True)
        np.testing.assert_allclose(out[qo[i]:qo[i + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)
        ref_full = sdpa_dense(qi, K, V, case.sm_scale)
        np.testing.assert_allclose(full[qo[i]:qo[i + 1]], ref_full.transpose(1, 0, 2), rtol=0,
                                   atol=1e-12)


def test_page_size_one_is_the_one_token_oracle_bitwise():
    case = W.random_case(5, [3, 17, 40], [1, 4, 2], n_heads=8, n_kv_heads=2, head_dim=32)
    t = np_tensors(case)
    md1 = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    mdp = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, 1, case.q_lens)
    for key in ("kv_indptr", "qo_indptr", "out_cache_loc"):
        assert np.array_equal(md1[key], mdp[key])
    kb1, vb1 = oracle.kv_store(t["k_buffer"], t["v_buffer"], 0, md1["out_cache_loc"],
                               t["k_new"], t["v_new"])
    kbp, vbp = OP.write(t["k_buffer"], t["v_buffer"], 0, case.req_to_token, 1,
                        case.req_pool_indices, case.seq_lens, case.q_lens, t["k_new"], t["v_new"])
    assert np.array_equal(kb1, kbp, equal_nan=True) and np.array_equal(vb1, vbp, equal_nan=True)
    dec = oracle.decode(kb1, vb1, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                        t["q"][:3], case.sm_scale)
    decp = OP.decode(kbp, vbp, 0, case.req_to_token, 1, case.req_pool_indices, case.seq_lens,
                     t["q"][:3], case.sm_scale)
    assert np.array_equal(dec, decp)
    pre = oracle.prefill(kb1, vb1, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                         md1["qo_indptr"], t["q"], case.sm_scale)
    prep = OP.prefill(kbp, vbp, 0, case.req_to_token, 1, case.req_pool_indices, case.seq_lens,
                      mdp["qo_indptr"], t["q"], case.sm_scale)
    assert np.array_equal(pre, prep)


def test_write_matches_flat_kv_store_at_build_step_slots():
    """The page write and the flat write k_buffer[layer, out_cache_loc] = k put
    every new row in the same place: out_cache_loc names the flat slot."""
    case = W.random_paged_case(8, [7, 16, 33, 40], 16, q_lens=[7, 2, 17, 1], n_heads=4,
                               n_kv_heads=2, head_dim=8)
    t = np_tensors(case)
    kbp, vbp, md = paged_store(case, t)
    kb1, vb1 = oracle.kv_store(t["k_buffer"], t["v_buffer"], 0, md["out_cache_loc"],
                               t["k_new"], t["v_new"])
    assert np.array_equal(kbp, kb1, equal_nan=True) and np.array_equal(vbp, vb1, equal_nan=True)
    assert len(set(md["out_cache_loc"].tolist())) == md["n_new"]
    ok, why = OP.validate_step(case.size, 16, case.req_to_token, case.req_pool_indices,
                               case.seq_lens, md["kv_indptr"], md["qo_indptr"],
                               md["out_cache_loc"])
    assert ok, why


def test_physical_page_permutation_bitwise():
    ps = 4
    case = W.random_paged_case(12, [3, 9, 21], ps, n_heads=4, n_kv_heads=2, head_dim=16)
    t = np_tensors(case)
    kb, vb, _ = paged_store(case, t)
    out = OP.decode(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                    t["q"], case.sm_scale)
    n_pages = case.size // ps
    pi = np.random.default_rng(3).permutation(n_pages)   # page p moves to pi[p]
    k5 = OP.page_view(kb, ps)
    v5 = OP.page_view(vb, ps)
    k2 = np.empty_like(k5)
    v2 = np.empty_like(v5)
    k2[:, pi] = k5
    v2[:, pi] = v5
    table2 = pi[case.req_to_token].astype(np.int32)
    out2 = OP.decode(k2.reshape(kb.shape), v2.reshape(vb.shape), 0, table2, ps,
                     case.req_pool_indices, case.seq_lens, t["q"], case.sm_scale)
    assert np.array_equal(out, out2)


def test_contiguous_pages_equal_contiguous_slots_bitwise():
    """Contiguous mode (slot = row * max_seq_len + pos) is the paged pool whose
    page table row r lists pages r * P .. r * P + P - 1 (P = max_seq_len / ps)."""
    ps, maxs, lens = 8, 32, [5, 32, 17]
    cont = W.contiguous_case(4, lens, maxs, n_heads=4, n_kv_heads=2, head_dim=16)
    t = np_tensors(cont, poison=False)
    P = maxs // ps
    table = np.arange(len(lens) * P, dtype=np.int32).reshape(len(lens), P)
    q = np.random.default_rng(9).standard_normal((3, 4, 16))
    o1 = oracle.decode(t["k_buffer"], t["v_buffer"], 0, cont.req_to_token, cont.req_pool_indices,
                       cont.seq_lens, q, 0.25)
    o2 = OP.decode(t["k_buffer"], t["v_buffer"], 0, table, ps, cont.req_pool_indices,
                   cont.seq_lens, q, 0.25)
    assert np.array_equal(o1, o2)


def test_shared_prefix_pages_read_the_same_rows():
    ps = 4
    case = W.random_paged_case(14, [9, 13, 10], ps, n_heads=2, n_kv_heads=1, head_dim=8,
                               shared_pages=2)
    rows = case.req_to_token[case.req_pool_indices]
    assert (rows[:, :2] == rows[0, :2]).all()
    t = np_tensors(case)
    kb, vb, md = paged_store(case, t)
    # the written slots avoid the shared pages
    shared = {int(p) * ps + o for p in rows[0, :2] for o in range(ps)}
    assert not shared & set(md["out_cache_loc"].tolist())
    k5 = OP.page_view(kb, ps)
    for b in range(case.batch):
        K = OP.gather_rows(k5, 0, case.req_to_token[case.req_pool_indices[b]], 8, 0)
        K0 = OP.gather_rows(k5, 0, case.req_to_token[case.req_pool_indices[0]], 8, 0)
        assert np.array_equal(K, K0)


def test_paged_oracle_never_reads_past_seq_len():
    ps = 16
    case = W.random_paged_case(15, [5, 17, 32], ps, n_heads=4, n_kv_heads=2, head_dim=16)
    t = np_tensors(case)
    kb, vb, _ = paged_store(case, t)
    # the tails of the last pages and the unused pages hold NaN
    k5 = OP.page_view(kb, ps)
    last = case.req_to_token[case.req_pool_indices[0], 0]
    assert np.isnan(k5[0, last, 5:]).all()
    out = OP.decode(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                    t["q"], case.sm_scale)
    assert np.isfinite(out).all()


def test_paged_golden_metadata():
    g = json.load(open(os.path.join(GOLDEN, "paged_step_metadata.json")))
    md = OP.build_step(g["req_pool_indices"], g["seq_lens"], np.array(g["page_table"]),
                       g["page_size"], g["q_lens"])
    assert md["out_cache_loc"].tolist() == g["out_cache_loc"]
    assert md["kv_indptr"].tolist() == g["kv_indptr"]
    assert md["qo_indptr"].tolist() == g["qo_indptr"]


def test_paged_validate_rejects_each_corruption():
    ps = 4
    case = W.random_paged_case(16, [6, 9], ps, q_lens=[2, 1], n_heads=2, n_kv_heads=1, head_dim=8)
    md = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, ps, case.q_lens)
    args = (case.size, ps, case.req_to_token, case.req_pool_indices, case.seq_lens,
            md["kv_indptr"], md["qo_indptr"], md["out_cache_loc"])
    assert OP.validate_step(*args)[0]
    bad_loc = md["out_cache_loc"].copy()
    bad_loc[0] += 1
    assert not OP.validate_step(*args[:7], bad_loc)[0]
    dup = md["out_cache_loc"].copy()
    dup[1] = dup[0]
    assert not OP.validate_step(*args[:7], dup)[0]
    table = case.req_to_token.copy()
    table[case.req_pool_indices[0], 0] = case.size // ps
    assert not OP.validate_step(case.size, ps, table, *args[3:])[0]
    assert not OP.validate_step(case.size + 1, ps, *args[2:])[0]
    kv = md["kv_indptr"].copy()
    kv[1] += 1
    assert not OP.validate_step(*args[:5], kv, *args[6:])[0]
    qo = md["qo_indptr"].copy()
    qo[0] = 1
    assert not OP.validate_step(*args[:6], qo, args[7])[0]


# ---------------------------------------------------------------------------
# planted mistakes: each must fail one of the pins above
# ---------------------------------------------------------------------------
def _pins_hold() -> bool:
    try:
        test_paged_decode_matches_sdpa_on_page_gather(4, 4, 2, 16)
        test_paged_prefill_matches_lower_right_sdpa()
        test_write_matches_flat_kv_store_at_build_step_slots()
        test_paged_golden_metadata()
        test_paged_oracle_never_reads_past_seq_len()
    except AssertionError:
        return False
    return True


def test_unmutated_paged_oracle_passes_its_pins():
    assert _pins_hold()


def _gather_offset_swapped(cache5, layer_id, page_row, n_tokens, hk):
    ps = cache5.shape[2]
    rows = [cache5[layer_id, int(page_row[pos % ps]) if pos % ps < len(page_row) else 0,
                   pos // ps if pos // ps < ps else 0, hk] for pos in range(n_tokens)]
    return np.stack(rows)


def _gather_next_page(cache5, layer_id, page_row, n_tokens, hk):
    ps = cache5.shape[2]
    rows = [cache5[layer_id, int(page_row[min(pos // ps + (pos % ps == ps - 1), len(page_row) - 1)]),
                   pos % ps, hk] for pos in range(n_tokens)]
    return np.stack(rows)


def _build_step_page_not_scaled(req_pool_indices, seq_lens, page_table, page_size, q_lens=None):
    md = _orig_build(req_pool_indices, seq_lens, page_table, page_size, q_lens)
    md["out_cache_loc"] = np.array([int(page_table[int(req_pool_indices[0]), 0]) + (x % page_size)
                                    for x in md["out_cache_loc"]], dtype=np.int32)
    return md


def _write_offset_from_start(k_buffer, v_buffer, layer_id, page_table, page_size,
                             req_pool_indices, seq_lens, q_lens, k_new, v_new):
    # new tokens placed as if the context started empty (position t, not L - ql + t)
    return _orig_write(k_buffer, v_buffer, layer_id, page_table, page_size, req_pool_indices,
                       [int(q) for q in q_lens], q_lens, k_new, v_new)


_orig_build = OP.build_step
_orig_write = OP.write


@pytest.mark.parametrize("name,target,mutant", [
    ("offset and page swapped", "gather_rows", _gather_offset_swapped),
    ("page index off by one at page ends", "gather_rows", _gather_next_page),
    ("slot not scaled by page_size", "build_step", _build_step_page_not_scaled),
    ("write position from the context start", "write", _write_offset_from_start),
])
def test_planted_paging_mistake_is_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(OP, target, mutant)
    assert not _pins_hold(), name


def test_paged_prefill_rows_sampler_matches_full():
    ps = 4
    case = W.random_paged_case(17, [9, 14], ps, q_lens=[4, 6], n_heads=4, n_kv_heads=2,
                               head_dim=8)
    t = np_tensors(case)
    kb, vb, md = paged_store(case, t)
    full = OP.prefill(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                      md["qo_indptr"], t["q"], case.sm_scale)
    rows = [(0, 0), (3, 3), (4, 1), (9, 2)]
    sub = OP.prefill_rows(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                          md["qo_indptr"], t["q"], case.sm_scale, rows)
    assert np.array_equal(sub, full[[r for r, _ in rows], [h for _, h in rows]])
