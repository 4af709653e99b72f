"""Pins for the oracle's sampled evaluators (no GPU).

``oracle.decode_pairs`` and ``oracle.pages.decode_pairs`` evaluate decode at
chosen (request, query head) pairs with a gather and a GQA head map of their
own; the large-workload GPU tests use them as their reference.  Here they are
tied to the full ``decode()`` of the same module (itself pinned by torch SDPA
in fp64): every (b, h) pair of a G = 4 and a G = 6 batch, on one-token pages
and on 16-token pages, must give decode()'s row.  Mistakes planted in copies
of the samplers (head map h % Hk, the slot row cut one short, the pair's
request taken as its table row) must fail the same comparison.
``oracle.prefill_rows`` (which groups its rows by request and kv-head) is
held to the full ``prefill()`` the same way, causal and not, with rows asked
for in a shuffled order; copies with a wrong head map or a causal limit one
key short fail.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as OA
import oracle.pages as OP
import workloads as W
from tests.test_oracle import np_tensors, store_new
from tests.test_oracle_pages import paged_store

# Requests with distinct lengths, table rows a random subset, so that a wrong
# head, a wrong request row or a missing key all change the result.
SHAPES = [(8, 2), (12, 2)]   # (n_heads, n_kv_heads): G = 4 and G = 6
LENS = [1, 7, 33, 18]


def _flat_case(seed, H, Hk):
    case = W.random_case(seed, LENS, n_heads=H, n_kv_heads=Hk, head_dim=16)
    t = np_tensors(case)
    kb, vb, _ = store_new(case, t)
    full = oracle.decode(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                         t["q"], case.sm_scale)
    return case, t, kb, vb, full


def _paged_case(seed, H, Hk, ps=16):
    case = W.random_paged_case(seed, LENS, ps, n_heads=H, n_kv_heads=Hk, head_dim=16)
    t = np_tensors(case)
    kb, vb, _ = paged_store(case, t)
    full = OP.decode(kb, vb, 0, case.req_to_token, ps, case.req_pool_indices, case.seq_lens,
                     t["q"], case.sm_scale)
    return case, t, kb, vb, full


def _all_pairs(case):
    return [(b, h) for b in range(case.batch) for h in range(case.n_heads)]


def _flat_sampler_matches(fn, seed, H, Hk) -> bool:
    case, t, kb, vb, full = _flat_case(seed, H, Hk)
    pairs = _all_pairs(case)
    got = fn(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens, t["q"],
             case.sm_scale, pairs)
    want = np.stack([full[b, h] for b, h in pairs])
    return got.shape == want.shape and bool(np.allclose(got, want, rtol=0, atol=1e-14))


def _paged_sampler_matches(fn, seed, H, Hk) -> bool:
    case, t, kb, vb, full = _paged_case(seed, H, Hk)
    pairs = _all_pairs(case)
    got = fn(kb, vb, 0, case.req_to_token, case.page_size, case.req_pool_indices, case.seq_lens,
             t["q"], case.sm_scale, pairs)
    want = np.stack([full[b, h] for b, h in pairs])
    return got.shape == want.shape and bool(np.allclose(got, want, rtol=0, atol=1e-14))


@pytest.mark.parametrize("H,Hk", SHAPES)
def test_decode_pairs_equals_decode_every_pair(H, Hk):
    case, t, kb, vb, full = _flat_case(101, H, Hk)
    pairs = _all_pairs(case)
    got = oracle.decode_pairs(kb, vb, 0, case.req_to_token, case.req_pool_indices,
                              case.seq_lens, t["q"], case.sm_scale, pairs)
    want = np.stack([full[b, h] for b, h in pairs])
    # Same gather and the same attend(); only the row count of the score
    # product differs, so any difference is last-bit BLAS rounding.
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("H,Hk", SHAPES)
def test_paged_decode_pairs_equals_decode_every_pair(H, Hk):
    case, t, kb, vb, full = _paged_case(102, H, Hk)
    assert case.page_size == 16 and max(LENS) > 16   # requests span several pages
    pairs = _all_pairs(case)
    got = OP.decode_pairs(kb, vb, 0, case.req_to_token, case.page_size, case.req_pool_indices,
                          case.seq_lens, t["q"], case.sm_scale, pairs)
    want = np.stack([full[b, h] for b, h in pairs])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_decode_pairs_any_order_and_repeats():
    case, t, kb, vb, full = _flat_case(103, 12, 2)
    pairs = [(3, 11), (0, 0), (3, 11), (1, 6), (2, 5)]
    got = oracle.decode_pairs(kb, vb, 0, case.req_to_token, case.req_pool_indices,
                              case.seq_lens, t["q"], case.sm_scale, pairs)
    np.testing.assert_allclose(got, np.stack([full[b, h] for b, h in pairs]), rtol=0, atol=1e-14)
    empty = oracle.decode_pairs(kb, vb, 0, case.req_to_token, case.req_pool_indices,
                                case.seq_lens, t["q"], case.sm_scale, [])
    assert empty.shape == (0, 16)


# ---------------------------------------------------------------------------
# Planted mistakes: copies of the samplers with one plausible error each.
# ---------------------------------------------------------------------------
def _flat_mutant(head_of, cut, row_of):
    def fn(k_buffer, v_buffer, layer_id, req_to_token, req_pool_indices, seq_lens, q, sm_scale,
           pairs):
        q = np.asarray(q, np.float64)
        H, Hk = q.shape[1], k_buffer.shape[2]
        G = H // Hk
        rows = []
        for b, h in pairs:
            r = row_of(b, req_pool_indices)
            L = int(seq_lens[b]) - cut
            slots = np.asarray(req_to_token[r, :max(L, 1)], dtype=np.int64)
            hk = head_of(h, G, Hk)
            K = k_buffer[layer_id, slots, hk, :]
            V = v_buffer[layer_id, slots, hk, :]
            rows.append(OA.attend(q[b, h], K, V, sm_scale)[0])
        return np.stack(rows)
    return fn


def _paged_mutant(head_of, cut, row_of):
    def fn(k_buffer, v_buffer, layer_id, page_table, page_size, req_pool_indices, seq_lens, q,
           sm_scale, pairs):
        q = np.asarray(q, np.float64)
        H, Hk = q.shape[1], k_buffer.shape[2]
        G = H // Hk
        k5 = OP.page_view(k_buffer, page_size)
        v5 = OP.page_view(v_buffer, page_size)
        rows = []
        for b, h in pairs:
            row = page_table[row_of(b, req_pool_indices)]
            L = max(int(seq_lens[b]) - cut, 1)
            hk = head_of(h, G, Hk)
            K = OP.gather_rows(k5, layer_id, row, L, hk)
            V = OP.gather_rows(v5, layer_id, row, L, hk)
            rows.append(OA.attend(q[b, h], K, V, sm_scale)[0])
        return np.stack(rows)
    return fn


_RIGHT_HEAD = lambda h, G, Hk: h // G           # noqa: E731
_MOD_HEAD = lambda h, G, Hk: h % Hk             # noqa: E731
_RIGHT_ROW = lambda b, rpi: int(rpi[b])         # noqa: E731
_BATCH_ROW = lambda b, rpi: b                   # noqa: E731

MUTANTS = [
    ("head map h % Hk", _MOD_HEAD, 0, _RIGHT_ROW),
    ("slot row cut one short", _RIGHT_HEAD, 1, _RIGHT_ROW),
    ("batch index used as table row", _RIGHT_HEAD, 0, _BATCH_ROW),
]


def test_unmutated_sampler_copies_pass():
    # the copies without a planted error pass the pins, so a failure below is
    # the planted error's doing
    for H, Hk in SHAPES:
        assert _flat_sampler_matches(_flat_mutant(_RIGHT_HEAD, 0, _RIGHT_ROW), 104, H, Hk)
        assert _paged_sampler_matches(_paged_mutant(_RIGHT_HEAD, 0, _RIGHT_ROW), 105, H, Hk)


@pytest.mark.parametrize("name,head_of,cut,row_of", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_sampler_mistake_is_caught(name, head_of, cut, row_of):
    for H, Hk in SHAPES:
        assert not _flat_sampler_matches(_flat_mutant(head_of, cut, row_of), 104, H, Hk), name
        assert not _paged_sampler_matches(_paged_mutant(head_of, cut, row_of), 105, H, Hk), name


# ---------------------------------------------------------------------------
# prefill_rows: every (token, head) row of a G = 4 and a G = 6 ragged batch,
# asked for in a shuffled order, equals the full prefill's row.
# ---------------------------------------------------------------------------
def _prefill_case(seed, H, Hk):
    q_lens, prefix = [5, 1, 0, 9], [3, 12, 4, 0]
    lens = [a + b for a, b in zip(q_lens, prefix)]
    case = W.random_case(seed, lens, q_lens, n_heads=H, n_kv_heads=Hk, head_dim=16)
    t = np_tensors(case)
    kb, vb, md = store_new(case, t)
    return case, t, kb, vb, md


def _prefill_rows_match(fn, seed, H, Hk, causal) -> bool:
    case, t, kb, vb, md = _prefill_case(seed, H, Hk)
    full = oracle.prefill(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
                          md["qo_indptr"], t["q"], case.sm_scale, causal=causal)
    rows = [(tok, h) for tok in range(md["n_new"]) for h in range(H)]
    np.random.default_rng(seed).shuffle(rows)
    got = fn(kb, vb, 0, case.req_to_token, case.req_pool_indices, case.seq_lens,
             md["qo_indptr"], t["q"], case.sm_scale, rows, causal=causal)
    want = np.stack([full[tok, h] for tok, h in rows])
    return got.shape == want.shape and bool(np.allclose(got, want, rtol=0, atol=1e-14))


@pytest.mark.parametrize("H,Hk", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_rows_equals_prefill_every_row(H, Hk, causal):
    assert _prefill_rows_match(oracle.prefill_rows, 106, H, Hk, causal)


def _prefill_rows_mutant(head_of, causal_shift):
    def fn(k_buffer, v_buffer, layer_id, req_to_token, req_pool_indices, seq_lens, qo_indptr, q,
           sm_scale, rows, causal=True):
        q = np.asarray(q, np.float64)
        H, Hk = q.shape[1], k_buffer.shape[2]
        G = H // Hk
        qo = [int(x) for x in qo_indptr]
        out = []
        for tok, h in rows:
            i = int(np.searchsorted(qo, tok, side="right")) - 1
            L, ql, t = int(seq_lens[i]), qo[i + 1] - qo[i], tok - qo[i]
            nk = (L - ql + t + 1 - causal_shift) if causal else L
            slots = np.asarray(req_to_token[int(req_pool_indices[i]), :max(nk, 1)], np.int64)
            hk = head_of(h, G, Hk)
            out.append(OA.attend(q[tok, h], k_buffer[layer_id, slots, hk, :],
                                 v_buffer[layer_id, slots, hk, :], sm_scale)[0])
        return np.stack(out)
    return fn


def test_prefill_rows_planted_mistakes_are_caught():
    assert _prefill_rows_match(_prefill_rows_mutant(_RIGHT_HEAD, 0), 107, 12, 2, True)
    assert not _prefill_rows_match(_prefill_rows_mutant(_MOD_HEAD, 0), 107, 12, 2, True)
    assert not _prefill_rows_match(_prefill_rows_mutant(_RIGHT_HEAD, 1), 107, 12, 2, True)
