"""Plain CPU fp64 restatement of the rotary embedding fused with the K/V write.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library and never imports it.

Sources (AstrAI project pages):
  * "Inference" guide, section "Rotary Embedding Backend": the rotary table
    ``freqs_cis`` has shape [max_len, dim/2, 2] in f32 and holds [cos, sin]
    pairs; the rows used by a token are selected by its entry of
    ``position_ids``; the reference (torch) path views the last dimension of
    the input as complex numbers (adjacent elements 2j, 2j+1 form pair j) and
    multiplies them by the table's complex entries cos + i sin.
  * "Inference" guide, section "KV Cache": the rotation is applied to the keys
    before they are written to the cache (and to the queries before they
    attend); values are not rotated.
  * "Inference" guide, section "KVCache System": the write is
    buffer[layer, out_cache_loc] = k.

  * Compare page v1.3.3 -> v1.3.4, class MLA: its queries and keys have
    qk_nope_head_dim + qk_rope_head_dim dims and its values their own width;
    only the qk_rope part carries the rotation.

Readings where the pages are silent:
  * The table is an input; how it was filled (base frequency) is not part of
    this step.
  * MLA rows: the rotated (qk_rope) part is the last qk_rope_head_dim dims of
    each query and key row, after the qk_nope part (the order the class lists
    them); its pairs are (2j, 2j+1) counted within that part, and the table
    is [max_len, qk_rope_head_dim / 2, 2].  The qk_nope dims pass unchanged.
  * The rotated values are rounded once to the pool dtype (bf16: round to
    nearest, ties to even, from the exact fp64 value).
"""

from __future__ import annotations

from typing import Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rope_rotate(x, positions: Sequence[int], freqs_cis) -> np.ndarray:
    """Rotate every head row of every token ("Rotary Embedding Backend").

    x: [n, heads, d] (any float dtype, upcast exactly); positions: [n] table
    rows; freqs_cis: [max_pos, d/2, 2] with [cos, sin] in the last axis.
    Pair j of a row is (x[2j], x[2j+1]); with (c, s) = freqs_cis[p, j] it
    becomes (x[2j] c - x[2j+1] s, x[2j] s + x[2j+1] c), the product of
    x[2j] + i x[2j+1] and c + i s.  Returns fp64 [n, heads, d].
    """
    x = _f64(x)
    f = _f64(freqs_cis)
    n, heads, d = x.shape
    assert d % 2 == 0 and f.shape[1] == d // 2 and f.shape[2] == 2
    out = np.empty_like(x)
    for i in range(n):
        p = int(positions[i])
        assert 0 <= p < f.shape[0], "position outside the table"
        c = f[p, :, 0]
        s = f[p, :, 1]
        a = x[i, :, 0::2]
        b = x[i, :, 1::2]
        out[i, :, 0::2] = a * c - b * s
        out[i, :, 1::2] = a * s + b * c
    return out


def round_to_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits, ties to
    even, the exponent range of fp32), returned as fp64.  Values whose bf16
    rounding overflows become +-inf; NaN stays NaN."""
    x = _f64(x)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])              # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)              # below 2^-126 the spacing stays 2^-133
    q = np.ldexp(1.0, e - 8)             # spacing of bf16 values near x
    r = np.rint(x[fin] / q) * q          # np.rint: half to even
    r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
    out[fin] = r
    return out


def to_dtype(x, dtype: str) -> np.ndarray:
    """The pool dtype's value of fp64 results: "bf16" rounds as above, "f32"
    rounds to the nearest float32 (numpy's conversion, ties to even)."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return _f64(x).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def rope_rotate_tail(x, positions: Sequence[int], freqs_cis, rope_dim: int) -> np.ndarray:
    """MLA rows (class MLA): the last rope_dim dims of every head row are
    rotated as rope_rotate does a whole row (pairs counted within that part,
    freqs_cis [max_pos, rope_dim/2, 2]); the first d - rope_dim dims are
    returned unchanged.  Returns fp64 [n, heads, d]."""
    x = _f64(x)
    d = x.shape[2]
    assert 0 < rope_dim <= d and rope_dim % 2 == 0
    out = x.copy()
    out[:, :, d - rope_dim:] = rope_rotate(x[:, :, d - rope_dim:], positions, freqs_cis)
    return out


def rope_kv_store(k_buffer, v_buffer, layer_id: int, out_cache_loc: Sequence[int], q, k_new,
                  v_new, positions: Sequence[int], freqs_cis, dtype: str, rope_dim=None):
    """The rotary step of one forward fused with its K/V write ("KV Cache":
    rotate first, then write).

    Returns (q_rot, k_pool, v_pool): the rotated queries rounded to ``dtype``,
    and copies of both pools (fp64 values) in which slot out_cache_loc[i] of
    layer layer_id holds the rotated, rounded key row i and the unrotated
    value row i.  Nothing else changes.  With rope_dim (MLA rows), only the
    last rope_dim dims of each query and key row are rotated.
    """
    if rope_dim is None:
        q_rot = to_dtype(rope_rotate(q, positions, freqs_cis), dtype)
        k_rot = to_dtype(rope_rotate(k_new, positions, freqs_cis), dtype)
    else:
        q_rot = to_dtype(rope_rotate_tail(q, positions, freqs_cis, rope_dim), dtype)
        k_rot = to_dtype(rope_rotate_tail(k_new, positions, freqs_cis, rope_dim), dtype)
    k_out = _f64(k_buffer).copy()
    v_out = _f64(v_buffer).copy()
    v_new = _f64(v_new)
    for i, loc in enumerate(out_cache_loc):
        k_out[layer_id, int(loc)] = k_rot[i]
        v_out[layer_id, int(loc)] = v_new[i]
    return q_rot, k_out, v_out
