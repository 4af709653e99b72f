"""Pins of the rotary oracle (oracle/rope.py) against what the pages and the
mathematics fix, with no GPU:

* the hand-derived golden example (tests/golden/rope_quarter_turn.json);
* the complex-multiply formulation the pages name for the torch path, done
  independently with numpy complex128;
* rotations preserve every pair's length, and scores of rotated queries and
  keys depend only on the position difference (for a table of angles p th_j);
* the bf16 rounding: worked tie cases and agreement with torch's own
  float32 -> bfloat16 conversion;
* the fused write: rotated keys land at out_cache_loc, values unrotated,
  every other row untouched; positions in the step metadata.

Planted mistakes (wrong sign, wrong pairing, off-by-one position, keys left
unrotated, ties rounded away from zero) must each fail one of these pins.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.rope as OR
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def angle_table(max_pos: int, d: int, base: float = 10000.0) -> np.ndarray:
    """A table of angles p * base^(-2j/d) as [cos, sin] in float32 (test input)."""
    j = np.arange(d // 2, dtype=np.float64)
    th = base ** (-2.0 * j / d)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * th[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def random_table(rng, max_pos: int, d: int) -> np.ndarray:
    ang = rng.uniform(-np.pi, np.pi, size=(max_pos, d // 2))
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


# ---------------------------------------------------------------- pin functions
def golden_holds() -> bool:
    g = json.load(open(os.path.join(GOLDEN, "rope_quarter_turn.json")))
    out = oracle.rope_rotate(np.array(g["x"], dtype=np.float64), g["position_ids"],
                             np.array(g["freqs_cis"], dtype=np.float64))
    return bool(np.allclose(out, np.array(g["expected"]), rtol=0, atol=1e-15))


def complex_multiply_holds() -> bool:
    rng = np.random.default_rng(11)
    n, H, d, P = 7, 3, 16, 20
    x = rng.standard_normal((n, H, d))
    f = random_table(rng, P, d)
    pos = rng.integers(0, P, size=n)
    out = oracle.rope_rotate(x, pos, f)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    w = f[pos, :, 0].astype(np.float64) + 1j * f[pos, :, 1].astype(np.float64)
    ref = z * w[:, None, :]
    return bool(np.allclose(out[..., 0::2], ref.real, rtol=0, atol=1e-13) and
                np.allclose(out[..., 1::2], ref.imag, rtol=0, atol=1e-13))


def relative_position_holds() -> bool:
    rng = np.random.default_rng(12)
    d, P = 32, 64
    f = angle_table(P, d)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    s0 = float(np.sum(oracle.rope_rotate(q, [9], f) * oracle.rope_rotate(k, [4], f)))
    s1 = float(np.sum(oracle.rope_rotate(q, [40], f) * oracle.rope_rotate(k, [35], f)))
    s2 = float(np.sum(oracle.rope_rotate(q, [9], f) * oracle.rope_rotate(k, [5], f)))
    # same difference -> same score (up to the f32 table); another one differs
    return abs(s0 - s1) < 1e-4 * (1 + abs(s0)) and abs(s0 - s2) > 1e-3


def fused_write_holds() -> bool:
    rng = np.random.default_rng(13)
    n_layers, size, Hk, H, d, P = 2, 12, 2, 4, 8, 10
    kb = rng.standard_normal((n_layers, size, Hk, d))
    vb = rng.standard_normal((n_layers, size, Hk, d))
    q = rng.standard_normal((3, H, d))
    kn = rng.standard_normal((3, Hk, d))
    vn = rng.standard_normal((3, Hk, d))
    f = random_table(rng, P, d)
    loc, pos = [7, 2, 9], [0, 5, 9]
    q_rot, k_out, v_out = oracle.rope_kv_store(kb, vb, 1, loc, q, kn, vn, pos, f, "f32")
    # the step written out by hand: rotate each key pair as a complex product
    k_ref = kb.copy()
    v_ref = vb.copy()
    for i in range(3):
        w = f[pos[i], :, 0].astype(np.float64) + 1j * f[pos[i], :, 1].astype(np.float64)
        z = (kn[i, :, 0::2] + 1j * kn[i, :, 1::2]) * w[None, :]
        row = np.empty((Hk, d))
        row[:, 0::2], row[:, 1::2] = z.real, z.imag
        k_ref[1, loc[i]] = row.astype(np.float32)
        v_ref[1, loc[i]] = vn[i]
    zq = (q[..., 0::2] + 1j * q[..., 1::2]) * \
        (f[pos, :, 0].astype(np.float64) + 1j * f[pos, :, 1].astype(np.float64))[:, None, :]
    q_ref = np.empty_like(q)
    q_ref[..., 0::2], q_ref[..., 1::2] = zq.real, zq.imag
    return bool(np.array_equal(k_out, k_ref) and np.array_equal(v_out, v_ref) and
                np.array_equal(q_rot, q_ref.astype(np.float32)))


def bf16_ties_hold() -> bool:
    cases = {
        1.0: 1.0,
        1.0 + 2.0 ** -8: 1.0,                    # halfway, down to the even neighbour
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,    # halfway, up to the even neighbour
        1.0 + 2.0 ** -8 + 2.0 ** -30: 1.0 + 2.0 ** -7,  # just above halfway
        -(1.0 + 2.0 ** -8): -1.0,
        3.0 * 2.0 ** -130: 3.0 * 2.0 ** -130,    # subnormal range, exact
        0.0: 0.0,
    }
    got = oracle.round_to_bf16(np.array(list(cases.keys())))
    return bool(np.array_equal(got, np.array(list(cases.values()))))


# --------------------------------------------------------------------- the pins
def test_golden_quarter_turn():
    assert golden_holds()


def test_matches_complex_multiply():
    assert complex_multiply_holds()


def test_pair_lengths_are_preserved():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((5, 4, 64))
    f = random_table(rng, 30, 64)
    out = oracle.rope_rotate(x, rng.integers(0, 30, size=5), f)
    n_in = np.hypot(x[..., 0::2], x[..., 1::2])
    n_out = np.hypot(out[..., 0::2], out[..., 1::2])
    # |cos + i sin| is 1 up to the f32 rounding of the table
    assert np.allclose(n_out, n_in, rtol=2e-7, atol=0)


def test_scores_depend_on_position_difference_only():
    assert relative_position_holds()


def test_zero_angle_row_is_the_identity():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((3, 2, 8))
    f = angle_table(4, 8)          # row 0: cos 1, sin 0
    assert np.array_equal(oracle.rope_rotate(x, [0, 0, 0], f), x)


def test_round_to_bf16_ties():
    assert bf16_ties_hold()


def test_round_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(16)
    x = np.concatenate([rng.standard_normal(100000),
                        rng.standard_normal(1000) * 1e30,
                        rng.standard_normal(1000) * 1e-38]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), ref)


def test_fused_write():
    assert fused_write_holds()


def test_rope_kv_store_leaves_other_rows_and_layers():
    rng = np.random.default_rng(17)
    kb = rng.standard_normal((3, 16, 2, 8))
    vb = rng.standard_normal((3, 16, 2, 8))
    q_rot, k_out, v_out = oracle.rope_kv_store(
        kb, vb, 2, [3, 11], rng.standard_normal((2, 4, 8)), rng.standard_normal((2, 2, 8)),
        rng.standard_normal((2, 2, 8)), [1, 2], angle_table(4, 8), "bf16")
    keep = np.ones(16, dtype=bool)
    keep[[3, 11]] = False
    assert np.array_equal(k_out[:2], kb[:2]) and np.array_equal(v_out[:2], vb[:2])
    assert np.array_equal(k_out[2, keep], kb[2, keep]) and np.array_equal(v_out[2, keep], vb[2, keep])
    assert np.array_equal(oracle.round_to_bf16(k_out[2, [3, 11]]), k_out[2, [3, 11]])


def test_step_positions_are_the_new_tokens_logical_positions():
    case = W.random_case(18, [5, 1, 9], [2, 1, 9], n_heads=2, n_kv_heads=1, head_dim=4)
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    assert md["position_ids"].tolist() == [3, 4, 0, 0, 1, 2, 3, 4, 5, 6, 7, 8]
    # each new token's slot is the table entry at its position
    r = np.repeat(case.req_pool_indices, case.q_lens)
    assert np.array_equal(case.req_to_token[r, md["position_ids"]], md["out_cache_loc"])


# ------------------------------------------------------------ planted mistakes
_rotate = OR.rope_rotate
_round = OR.round_to_bf16


def m_sin_sign(x, positions, f):
    f = np.array(f, dtype=np.float64, copy=True)
    f[..., 1] = -f[..., 1]
    return _rotate(x, positions, f)


def m_half_split(x, positions, f):
    # pairs (j, j + d/2) instead of adjacent elements
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    perm = np.empty(d, dtype=np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    out = _rotate(x[..., perm], positions, f)
    back = np.empty_like(out)
    back[..., perm] = out
    return back


def m_position_plus_one(x, positions, f):
    f = np.asarray(f)
    return _rotate(x, [min(int(p) + 1, f.shape[0] - 1) for p in positions], f)


def m_keys_unrotated(k_buffer, v_buffer, layer_id, out_cache_loc, q, k_new, v_new, positions,
                     freqs_cis, dtype):
    q_rot = OR.to_dtype(_rotate(q, positions, freqs_cis), dtype)
    k_out = np.asarray(k_buffer, dtype=np.float64).copy()
    v_out = np.asarray(v_buffer, dtype=np.float64).copy()
    for i, loc in enumerate(out_cache_loc):
        k_out[layer_id, int(loc)] = OR.to_dtype(np.asarray(k_new[i], dtype=np.float64), dtype)
        v_out[layer_id, int(loc)] = v_new[i]
    return q_rot, k_out, v_out


def m_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    out[fin] = np.sign(x[fin]) * np.floor(np.abs(x[fin]) / q + 0.5) * q
    return out


MUTANTS = [
    ("rope_rotate", m_sin_sign, [golden_holds, complex_multiply_holds]),
    ("rope_rotate", m_half_split, [golden_holds, complex_multiply_holds]),
    ("rope_rotate", m_position_plus_one, [golden_holds, complex_multiply_holds]),
    ("rope_kv_store", m_keys_unrotated, [fused_write_holds]),
    ("round_to_bf16", m_ties_away, [bf16_ties_hold]),
]


def test_unmutated_rope_oracle_passes_every_pin():
    for pin in (golden_holds, complex_multiply_holds, relative_position_holds, fused_write_holds,
                bf16_ties_hold):
        assert pin(), pin.__name__


@pytest.mark.parametrize("target,mutant,pins", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_rope_mistake_is_caught(monkeypatch, target, mutant, pins):
    monkeypatch.setattr(OR, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    for pin in pins:
        assert not pin(), f"{mutant.__name__} survived {pin.__name__}"
