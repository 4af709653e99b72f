"""Host-side checks of libpkv (no GPU): exported symbols, step metadata and
checked mode against the oracle (bit-exact), and argument errors that are
reported before anything is launched."""

import ctypes as C
import json
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W
from paged_kv_attention_12_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        pytest.skip("libpkv.so not built")
    return B.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "pkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTED) == set(names)


def test_status_strings(lib):
    for s in range(9):
        assert lib.pkv_status_string(s)
    assert B.status_string(B.PKV_ERR_SCRATCH_LIMIT).startswith("workspace needed exceeds")
    assert B.status_string(B.PKV_ERR_WORKSPACE_TOO_SMALL) == "workspace too small"


def test_build_step_golden(lib):
    g = json.load(open(os.path.join(GOLDEN, "step_metadata.json")))
    md = B.pkv_build_step(g["req_pool_indices"], g["seq_lens"], np.array(g["req_to_token"]),
                          g["q_lens"])
    for k in ("kv_indptr", "qo_indptr", "out_cache_loc", "prefill_order"):
        assert md[k].tolist() == g[k]
    assert (md["n_new"], md["max_len"], md["max_q_len"]) == (g["n_new"], g["max_len"],
                                                             g["max_q_len"])


@pytest.mark.parametrize("maker", [
    lambda: W.tiny_decode_f32(),
    lambda: W.batched_prefix_decode(),
    lambda: W.ragged_prefill(),
    lambda: W.random_case(3, [1, 9, 40, 2], [0, 4, 40, 1], n_heads=8, n_kv_heads=2, head_dim=64),
])
def test_build_step_matches_oracle_bitwise(lib, maker):
    case = maker()
    ql = None if case.is_decode else case.q_lens
    got = B.pkv_build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, ql)
    ref = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, ql)
    for k in ("kv_indptr", "qo_indptr", "out_cache_loc", "prefill_order"):
        assert got[k].dtype == np.int32
        assert got[k].tobytes() == ref[k].tobytes(), k
    for k in ("n_new", "max_len", "max_q_len"):
        assert got[k] == ref[k]


def test_build_step_rejects_bad_rows(lib):
    case = W.random_case(5, [3, 4], n_heads=2, n_kv_heads=1, head_dim=64)
    rows = case.req_pool_indices.copy()
    rows[1] = case.num_reqs
    with pytest.raises(B.PkvError) as e:
        B.pkv_build_step(rows, case.seq_lens, case.req_to_token)
    assert e.value.status == B.PKV_ERR_BAD_METADATA
    with pytest.raises(B.PkvError):
        B.pkv_build_step(case.req_pool_indices, [3, 0], case.req_to_token)


def _validate_both(case, md, **over):
    a = dict(size=case.size, req_to_token=case.req_to_token,
             req_pool_indices=case.req_pool_indices, seq_lens=case.seq_lens,
             kv_indptr=md["kv_indptr"], qo_indptr=md["qo_indptr"],
             out_cache_loc=md["out_cache_loc"])
    a.update(over)
    lib_ok = B.pkv_validate_step(**a) == B.PKV_OK
    ref_ok, _ = oracle.validate_step(num_reqs=case.num_reqs, max_ctx_len=case.max_ctx_len, **a)
    return lib_ok, ref_ok


def test_validate_step_agrees_with_oracle(lib):
    case = W.random_case(61, [4, 9, 6, 1], [1, 3, 6, 1], n_heads=4, n_kv_heads=2, head_dim=64)
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    assert _validate_both(case, md) == (True, True)
    corrupt = []
    x = md["out_cache_loc"].copy(); x[1] = x[0]; corrupt.append(dict(out_cache_loc=x))
    x = md["out_cache_loc"].copy(); x[2] = case.size; corrupt.append(dict(out_cache_loc=x))
    x = md["out_cache_loc"].copy(); x[3] = -1; corrupt.append(dict(out_cache_loc=x))
    x = md["kv_indptr"].copy(); x[2] += 1; corrupt.append(dict(kv_indptr=x))
    x = case.req_pool_indices.copy(); x[0] = case.num_reqs; corrupt.append(dict(req_pool_indices=x))
    x = case.seq_lens.copy(); x[0] = 0; corrupt.append(dict(seq_lens=x))
    x = case.seq_lens.copy(); x[1] = case.max_ctx_len + 1; corrupt.append(dict(seq_lens=x))
    x = case.req_to_token.copy(); x[case.req_pool_indices[1], 0] = case.size
    corrupt.append(dict(req_to_token=x))
    x = md["qo_indptr"].copy(); x[1] = 5; corrupt.append(dict(qo_indptr=x))
    for c in corrupt:
        assert _validate_both(case, md, **c) == (False, False), list(c)


def test_validate_checks_prefill_order(lib):
    case = W.random_case(62, [4, 9, 6], [1, 3, 6], n_heads=4, n_kv_heads=2, head_dim=64)
    md = B.pkv_build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, case.q_lens)
    args = (case.size, case.req_to_token, case.req_pool_indices, case.seq_lens, md["kv_indptr"],
            md["qo_indptr"], md["out_cache_loc"])
    assert md["prefill_order"].tolist() == [1, 2, 0]
    assert B.pkv_validate_step(*args, prefill_order=md["prefill_order"]) == B.PKV_OK
    for bad in ([1, 1, 0], [0, 1, 3], [2, 1], [-1, 0, 1]):
        assert B.pkv_validate_step(*args, prefill_order=np.array(bad)) == B.PKV_ERR_BAD_METADATA


def test_validate_decode_with_null_qo_indptr(lib):
    case = W.tiny_decode_f32()
    md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token)
    st = B.pkv_validate_step(case.size, case.req_to_token, case.req_pool_indices, case.seq_lens,
                             md["kv_indptr"], None, md["out_cache_loc"])
    assert st == B.PKV_OK


def test_workspace_bytes_and_split_choice(lib):
    assert B.pkv_decode_workspace_bytes(8, 64, 128, 64) == 8 * 64 * 64 * (128 + 2) * 4
    assert B.pkv_decode_workspace_bytes(0, 64, 128, 64) == 0
    for args in [(1, 8, 32, 1024), (1, 8, 32, 32768), (64, 8, 32, 8192), (8, 8, 64, 131072),
                 (2, 2, 4, 17)]:
        s = B.pkv_decode_pick_splits(*args, max_splits=512)
        assert 1 <= s <= 512
        assert s <= max(1, (args[3] + 15) // 16)   # never below 16 tokens per split
    assert B.pkv_decode_pick_splits(1, 8, 32, 32768, max_splits=4) == 4
    # the measured choices: B=1 Llama shapes, long context, ragged batch
    assert B.pkv_decode_pick_splits(1, 8, 32, 32768, 32768) == 128
    assert B.pkv_decode_pick_splits(1, 8, 32, 1024, 1024) == 64
    assert B.pkv_decode_pick_splits(8, 8, 64, 131072, 8 * 131072) == 64
    # ragged: 266000 * 8 / 4096 = 519 wavefront-tokens, capped at 512 tokens
    # per split: 16 splits, one more: an odd count spreads a request's
    # 2 x 17 workgroups over the most XCD offsets
    assert B.pkv_decode_pick_splits(64, 8, 32, 8192, 266000) == 17
    rng = np.random.default_rng(5)
    for _ in range(200):
        batch = int(rng.integers(2, 200))
        hk = int(rng.choice([1, 2, 4, 8, 16]))
        heads = hk * int(rng.choice([1, 2, 4, 8, 24]))
        max_len = int(rng.integers(16, 200000))
        total = int(rng.integers(max_len, max_len * batch // 2 + max_len + 1))
        s = B.pkv_decode_pick_splits(batch, hk, heads, max_len, total, max_splits=65535)
        ragged = batch * max_len > total + total // 4
        wgs = (hk * ((heads // hk + 15) // 16) + 3) // 4
        if ragged and 1 < s < 65535 and wgs % 8:
            assert s % 2 == 1, (batch, hk, heads, max_len, total, s)


def _fake_pool(dtype=B.PKV_BF16, head_dim=128, n_layers=2):
    p = B.pkv_pool()
    p.k_buffer, p.v_buffer, p.req_to_token = 0x1000, 0x2000, 0x3000
    p.n_layers, p.size, p.num_reqs, p.max_ctx_len = n_layers, 64, 4, 32
    p.n_kv_heads, p.head_dim, p.dtype = 2, head_dim, dtype
    return p


def test_argument_errors_before_launch(lib):
    """Every call below fails a host check, so nothing reaches the device."""
    p = _fake_pool()
    s = B.pkv_step()
    s.batch, s.req_pool_indices, s.seq_lens, s.max_len = 2, 0x10, 0x20, 8
    fake = C.c_void_p(0x4000)
    # null / range / dtype checks
    assert lib.pkv_kv_store(None, 0, fake, fake, fake, 4, None) == B.PKV_ERR_NULL
    assert lib.pkv_kv_store(C.byref(p), 2, fake, fake, fake, 4, None) == B.PKV_ERR_SHAPE
    assert lib.pkv_kv_store(C.byref(p), -1, fake, fake, fake, 4, None) == B.PKV_ERR_SHAPE
    assert lib.pkv_kv_store(C.byref(p), 0, None, fake, fake, 4, None) == B.PKV_ERR_NULL
    assert lib.pkv_kv_store(C.byref(p), 0, fake, fake, fake, -1, None) == B.PKV_ERR_SHAPE
    assert lib.pkv_kv_store(C.byref(p), 0, fake, fake, fake, 0, None) == B.PKV_OK
    bad = _fake_pool(dtype=7)
    assert lib.pkv_kv_store(C.byref(bad), 0, fake, fake, fake, 4, None) == B.PKV_ERR_DTYPE
    # decode: heads not a multiple of kv-heads, unsupported head_dim, workspace too small
    assert lib.pkv_paged_decode(C.byref(p), 0, C.byref(s), fake, 3, 0.1, 1, fake, 1 << 20,
                                None) == B.PKV_ERR_SHAPE
    p96 = _fake_pool(head_dim=96)
    assert lib.pkv_paged_decode(C.byref(p96), 0, C.byref(s), fake, 4, 0.1, 1, fake, 1 << 20,
                                None) == B.PKV_ERR_UNSUPPORTED
    need = lib.pkv_decode_workspace_bytes(2, 4, 128, 4)
    assert lib.pkv_paged_decode(C.byref(p), 0, C.byref(s), fake, 4, 0.1, 4, fake, need - 1,
                                None) == B.PKV_ERR_WORKSPACE_TOO_SMALL
    assert lib.pkv_paged_decode(C.byref(p), 0, C.byref(s), fake, 4, float("nan"), 4, fake,
                                need, None) == B.PKV_ERR_SHAPE
    assert lib.pkv_paged_decode(C.byref(p), 0, C.byref(s), fake, 4, 0.1, 0, fake, need,
                                None) == B.PKV_ERR_SHAPE
    s_long = B.pkv_step()
    s_long.batch, s_long.req_pool_indices, s_long.seq_lens, s_long.max_len = 2, 0x10, 0x20, 33
    assert lib.pkv_paged_decode(C.byref(p), 0, C.byref(s_long), fake, 4, 0.1, 4, fake, need,
                                None) == B.PKV_ERR_SHAPE
    assert lib.pkv_paged_decode_merge(2, 4, 128, B.PKV_BF16, 4, fake, need - 4, fake,
                                      None) == B.PKV_ERR_WORKSPACE_TOO_SMALL
    assert lib.pkv_paged_decode_merge(2, 4, 128, 9, 4, fake, need, fake,
                                      None) == B.PKV_ERR_DTYPE
    # prefill: fp32 pools are rejected, missing qo_indptr is a null error
    pf = _fake_pool(dtype=B.PKV_F32)
    sp = B.pkv_step()
    sp.batch, sp.req_pool_indices, sp.seq_lens, sp.max_len, sp.n_new, sp.max_q_len = \
        2, 0x10, 0x20, 8, 4, 2
    assert lib.pkv_paged_prefill(C.byref(pf), 0, C.byref(sp), fake, 4, 0.1, 1, fake,
                                 None) == B.PKV_ERR_DTYPE
    assert lib.pkv_paged_prefill(C.byref(p), 0, C.byref(sp), fake, 4, 0.1, 1, fake,
                                 None) == B.PKV_ERR_NULL
    # prefill ranks raw scores, so the scale must be positive
    for bad_scale in (0.0, -0.1, float("inf")):
        assert lib.pkv_paged_prefill(C.byref(p), 0, C.byref(sp), fake, 4, bad_scale, 1, fake,
                                     None) == B.PKV_ERR_SHAPE


def test_decode_load_kind(lib):
    """pkv_pool.load_policy: AUTO streams a one-request step whose K/V over
    all layers exceed the 256 MiB last-level cache; CACHED and STREAM
    override; invalid fields give -1 and entry points refuse them."""
    p = _fake_pool(n_layers=32)
    p.n_kv_heads = 8                     # rows of 8 * (128 + 128) * 2 = 4096 bytes
    assert p.load_policy == B.PKV_LOAD_AUTO
    # 32 layers * L * 4096 bytes against 256 MiB: the boundary is L = 2048
    assert B.pkv_decode_load_kind(p, 1, 2048) == 0
    assert B.pkv_decode_load_kind(p, 1, 2049) == 1
    assert B.pkv_decode_load_kind(p, 1, 32768) == 1
    assert B.pkv_decode_load_kind(p, 1, 1024) == 0
    for batch in (0, 2, 8, 64):        # requests may share slots: cached
        assert B.pkv_decode_load_kind(p, batch, 131072) == 0
    one = _fake_pool(n_layers=1)
    one.n_kv_heads = 8
    assert B.pkv_decode_load_kind(one, 1, 32768) == 0   # 134 MB fit the cache
    mla = _fake_pool(head_dim=192, n_layers=32)
    mla.v_head_dim, mla.n_kv_heads = 128, 8           # rows of 8 * 320 * 2 bytes
    assert B.pkv_decode_load_kind(mla, 1, 1638) == 0  # 32 * 1638 * 5120 < 2^28
    assert B.pkv_decode_load_kind(mla, 1, 1639) == 1
    p.load_policy = B.PKV_LOAD_CACHED
    assert B.pkv_decode_load_kind(p, 1, 131072) == 0
    p.load_policy = B.PKV_LOAD_STREAM
    assert B.pkv_decode_load_kind(p, 64, 16) == 1
    for bad in (-1, 3):
        p.load_policy = bad
        assert B.pkv_decode_load_kind(p, 1, 32768) == -1
        fake = C.c_void_p(0x4000)
        assert lib.pkv_kv_store(C.byref(p), 0, fake, fake, fake, 4, None) == B.PKV_ERR_SHAPE
    assert lib.pkv_decode_load_kind(None, 1, 32768) == -1


def test_fused_step_split_choice(lib):
    # a quarter of the single-wave choice (four waves share a split), at least 1
    for args in [(1, 8, 32, 1024, 1024), (1, 8, 32, 32768, 32768), (8, 8, 64, 131072, 8 * 131072),
                 (64, 8, 32, 8192, 266000), (2, 2, 4, 17, 22)]:
        s1 = B.pkv_decode_pick_splits(*args, max_splits=65535)
        assert B.pkv_decode_step_pick_splits(*args) == max(1, (s1 + 3) // 4)
    assert B.pkv_decode_step_pick_splits(1, 8, 32, 32768, 32768) == 32
    assert B.pkv_decode_step_pick_splits(1, 8, 32, 32768, 32768, max_splits=5) == 5


def test_fused_step_argument_errors(lib):
    """Host checks of pkv_paged_decode_step; nothing reaches the device."""
    p = _fake_pool()
    s = B.pkv_step()
    s.batch, s.req_pool_indices, s.seq_lens, s.max_len = 2, 0x10, 0x20, 8
    s.out_cache_loc, s.n_new = 0x30, 2
    fake = C.c_void_p(0x4000)
    sync = C.c_void_p(0x5000)
    need = lib.pkv_decode_workspace_bytes(2, 4, 128, 4)
    call = lambda step=s, pool=p, sync_ptr=sync, sync_len=8, ws=need, ns=4: \
        lib.pkv_paged_decode_step(C.byref(pool), 0, C.byref(step), fake, fake, fake, 4, 0.1, ns,
                                  fake, ws, sync_ptr, sync_len, fake, None)
    assert call(sync_ptr=None) == B.PKV_ERR_NULL
    assert call(sync_len=7) == B.PKV_ERR_SHAPE          # needs batch * n_heads counters
    assert call(ws=need - 1) == B.PKV_ERR_WORKSPACE_TOO_SMALL
    assert call(ns=0) == B.PKV_ERR_SHAPE
    s3 = B.pkv_step()
    s3.batch, s3.req_pool_indices, s3.seq_lens, s3.max_len = 2, 0x10, 0x20, 8
    s3.out_cache_loc, s3.n_new = 0x30, 3                  # not one new token per request
    assert call(step=s3) == B.PKV_ERR_SHAPE
    s0 = B.pkv_step()
    s0.batch, s0.req_pool_indices, s0.seq_lens, s0.max_len = 2, 0x10, 0x20, 8
    s0.n_new = 2                                          # no out_cache_loc
    assert call(step=s0) == B.PKV_ERR_NULL
    assert call(pool=_fake_pool(head_dim=96)) == B.PKV_ERR_UNSUPPORTED


def test_stored_step_argument_errors(lib):
    """Host checks of pkv_paged_decode_store; nothing reaches the device."""
    p = _fake_pool()
    s = B.pkv_step()
    s.batch, s.req_pool_indices, s.seq_lens, s.max_len = 2, 0x10, 0x20, 8
    s.out_cache_loc, s.n_new = 0x30, 2
    fake = C.c_void_p(0x4000)
    need = lib.pkv_decode_workspace_bytes(2, 4, 128, 4)
    call = lambda step=s, pool=p, ws=need, ns=4, out=fake, knew=fake: \
        lib.pkv_paged_decode_store(C.byref(pool), 0, C.byref(step), fake, knew, fake, 4, 0.1, ns,
                                   fake, ws, out, None)
    assert call(out=None) == B.PKV_ERR_NULL
    assert call(knew=None) == B.PKV_ERR_NULL
    assert call(ws=need - 1) == B.PKV_ERR_WORKSPACE_TOO_SMALL
    assert call(ns=0) == B.PKV_ERR_SHAPE
    s3 = B.pkv_step()
    s3.batch, s3.req_pool_indices, s3.seq_lens, s3.max_len = 2, 0x10, 0x20, 8
    s3.out_cache_loc, s3.n_new = 0x30, 3                  # not one new token per request
    assert call(step=s3) == B.PKV_ERR_SHAPE
    s0 = B.pkv_step()
    s0.batch, s0.req_pool_indices, s0.seq_lens, s0.max_len = 2, 0x10, 0x20, 8
    s0.n_new = 2                                          # no out_cache_loc
    assert call(step=s0) == B.PKV_ERR_NULL
    assert call(pool=_fake_pool(head_dim=96)) == B.PKV_ERR_UNSUPPORTED
    sb = B.pkv_step()
    sb.batch = 0                                          # empty step: nothing to do
    assert call(step=sb) == B.PKV_OK


def test_build_positions_matches_oracle():
    import oracle
    import workloads as W
    for seed, lens, qls in [(1, [5, 1, 9], [2, 1, 9]), (2, [7, 300, 64], None), (3, [4, 4], [0, 4])]:
        case = W.random_case(seed, lens, qls, n_heads=2, n_kv_heads=1, head_dim=4)
        md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token,
                               None if qls is None else case.q_lens)
        got = B.pkv_build_positions(case.seq_lens, None if qls is None else case.q_lens)
        assert np.array_equal(got, md["position_ids"])


def test_build_positions_errors(lib):
    sl = np.array([3, 2], dtype=np.int32)
    bad = np.array([1, 3], dtype=np.int32)        # q_len above seq_len
    out = np.zeros(8, dtype=np.int32)
    n = C.c_int64(0)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    assert lib.pkv_build_positions(2, p(sl), p(bad), p(out), 8, C.byref(n)) == B.PKV_ERR_BAD_METADATA
    assert lib.pkv_build_positions(2, p(sl), None, p(out), 1, C.byref(n)) == B.PKV_ERR_SHAPE
    assert lib.pkv_build_positions(2, None, None, p(out), 8, C.byref(n)) == B.PKV_ERR_NULL
    assert lib.pkv_build_positions(-1, p(sl), None, p(out), 8, C.byref(n)) == B.PKV_ERR_SHAPE
    assert lib.pkv_build_positions(2, p(sl), None, p(out), 8, C.byref(n)) == B.PKV_OK
    assert n.value == 2 and out[:2].tolist() == [2, 1]


def test_rope_kv_store_argument_errors(lib):
    """Host checks of pkv_rope_kv_store; nothing reaches the device."""
    p = _fake_pool()
    fake = C.c_void_p(0x4000)
    mis = C.c_void_p(0x4008)                       # 8-byte, not 16-byte, aligned
    call = lambda pool=p, q=fake, qo=fake, H=4, kn=fake, pos=fake, fr=fake, mp=16, n=3: \
        lib.pkv_rope_kv_store(C.byref(pool), 0, q, qo, H, kn, fake, pos, fr, mp, fake, n, None)
    assert call(q=None) == B.PKV_ERR_NULL
    assert call(pos=None) == B.PKV_ERR_NULL
    assert call(fr=None) == B.PKV_ERR_NULL
    assert call(q=mis) == B.PKV_ERR_SHAPE
    assert call(fr=mis) == B.PKV_ERR_SHAPE
    assert call(mp=0) == B.PKV_ERR_SHAPE
    assert call(H=3) == B.PKV_ERR_SHAPE               # not a multiple of n_kv_heads
    assert call(n=-1) == B.PKV_ERR_SHAPE
    assert call(pool=_fake_pool(head_dim=96)) == B.PKV_ERR_UNSUPPORTED
    assert call(n=0) == B.PKV_OK                      # empty step: nothing to do


def test_decode_advance_argument_errors(lib):
    """Host checks of pkv_decode_advance; nothing reaches the device."""
    p = _fake_pool()
    fake = C.c_void_p(0x4000)
    call = lambda n=2, rpi=fake, sl=fake, loc=fake: \
        lib.pkv_decode_advance(C.byref(p), n, rpi, sl, None, loc, None, None)
    assert call(rpi=None) == B.PKV_ERR_NULL
    assert call(sl=None) == B.PKV_ERR_NULL
    assert call(loc=None) == B.PKV_ERR_NULL
    assert call(n=-1) == B.PKV_ERR_SHAPE
    assert call(n=0) == B.PKV_OK


# ---------------------------------------------------------------------------
# pools of page_size > 1 tokens
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ps", [2, 16, 64])
def test_paged_build_step_matches_paged_oracle(lib, ps):
    import oracle.pages as OP
    lens = [1, ps, ps + 1, 5 * ps + 3]
    q_lens = [1, ps, 2, 3 * ps]
    case = W.random_paged_case(70 + ps, lens, ps, q_lens=q_lens)
    got = B.pkv_build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, q_lens, ps)
    ref = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, ps, q_lens)
    for k in ("kv_indptr", "qo_indptr", "out_cache_loc"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["max_len"] == ref["max_len"] and got["n_new"] == ref["n_new"]


def test_paged_golden_build_step(lib):
    g = json.load(open(os.path.join(GOLDEN, "paged_step_metadata.json")))
    md = B.pkv_build_step(g["req_pool_indices"], g["seq_lens"], np.array(g["page_table"]),
                          g["q_lens"], g["page_size"])
    assert md["out_cache_loc"].tolist() == g["out_cache_loc"]
    assert md["kv_indptr"].tolist() == g["kv_indptr"]


def test_paged_validate_agrees_with_paged_oracle(lib):
    import oracle.pages as OP
    ps = 8
    case = W.random_paged_case(80, [7, 8, 9, 30], ps, q_lens=[7, 1, 2, 9])
    md = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, ps, case.q_lens)

    def both(table=case.req_to_token, loc=md["out_cache_loc"], size=case.size):
        lib_ok = B.pkv_validate_step(size, table, case.req_pool_indices, case.seq_lens,
                                     md["kv_indptr"], md["qo_indptr"], loc,
                                     page_size=ps) == B.PKV_OK
        ref_ok, _ = OP.validate_step(size, ps, table, case.req_pool_indices, case.seq_lens,
                                     md["kv_indptr"], md["qo_indptr"], loc)
        return lib_ok, ref_ok

    assert both() == (True, True)
    x = md["out_cache_loc"].copy(); x[0] += 1
    assert both(loc=x) == (False, False)
    x = md["out_cache_loc"].copy(); x[1] = x[0]
    assert both(loc=x) == (False, False)
    t = case.req_to_token.copy(); t[case.req_pool_indices[3], 2] = case.size // ps
    assert both(table=t) == (False, False)
    t = case.req_to_token.copy(); t[case.req_pool_indices[0], 0] = -1
    assert both(table=t) == (False, False)


def test_page_size_argument_errors(lib):
    case = W.random_paged_case(81, [5, 9], 4)
    for bad in (3, 6, 1 << 17, -4):
        with pytest.raises(B.PkvError):
            B.pkv_build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, None, bad)
    md = B.pkv_build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, None, 4)
    st = B.pkv_validate_step(case.size + 2, case.req_to_token, case.req_pool_indices,
                             case.seq_lens, md["kv_indptr"], None, md["out_cache_loc"],
                             page_size=4)
    assert st == B.PKV_ERR_SHAPE


def test_pool_page_size_checks_before_launch(lib):
    """A pool whose page size is not a power of two, or does not divide the
    slot count, is refused by every pool-taking entry point before launch."""
    fake = C.c_void_p(0x4000)
    s = B.pkv_step()
    s.batch, s.req_pool_indices, s.seq_lens, s.max_len = 2, 0x10, 0x20, 8
    for ps, size in ((3, 48), (6, 48), (1 << 17, 1 << 17), (-2, 48), (16, 40)):
        p = _fake_pool()
        p.page_size, p.size = ps, size
        assert lib.pkv_kv_store(C.byref(p), 0, fake, fake, fake, 4, None) == B.PKV_ERR_SHAPE
        assert lib.pkv_paged_decode(C.byref(p), 0, C.byref(s), fake, 8, 0.1, 1, fake, 1 << 20,
                                    None) == B.PKV_ERR_SHAPE
    p = _fake_pool()
    p.page_size, p.size = 16, 48
    assert lib.pkv_kv_store(C.byref(p), 0, fake, fake, fake, 0, None) == B.PKV_OK


def test_c_caller_of_the_header(lib, tmp_path):
    """include/pkv.h compiles as C99 with gcc and a C program linked against
    libpkv.so gets the hand-worked step metadata (one-token and 4-token pages)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "host_abi")
    libdir = os.path.dirname(B.lib_path())
    src = os.path.join(ROOT, "tests", "c", "host_abi.c")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    src, "-L", libdir, "-lpkv", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    layout = [str(C.sizeof(B.pkv_pool)), str(B.pkv_pool.load_policy.offset),
              str(C.sizeof(B.pkv_step))]
    r = subprocess.run([exe, *layout], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.parametrize("ps", [1, 4])
def test_validate_step_random_corruptions_agree_with_oracle(lib, ps):
    """Randomised agreement of the library's checked mode with the oracle's on
    one well-formed step and many single-field corruptions of it (slot or page
    table entries, write slots, lengths, request rows, prefix sums)."""
    import oracle.pages as OP
    rng = np.random.default_rng(900 + ps)
    lens = [3, 9, 1, 14]
    q_lens = [1, 4, 1, 6]
    if ps == 1:
        case = W.random_case(91, lens, q_lens)
        md = oracle.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, q_lens)
    else:
        case = W.random_paged_case(91, lens, ps, q_lens=q_lens)
        md = OP.build_step(case.req_pool_indices, case.seq_lens, case.req_to_token, ps, q_lens)
    base = dict(req_to_token=case.req_to_token, req_pool_indices=case.req_pool_indices,
                seq_lens=case.seq_lens, kv_indptr=md["kv_indptr"], qo_indptr=md["qo_indptr"],
                out_cache_loc=md["out_cache_loc"])

    def both(a):
        lib_ok = B.pkv_validate_step(case.size, page_size=ps, **a) == B.PKV_OK
        if ps == 1:
            ref_ok, _ = oracle.validate_step(case.size, case.num_reqs, case.max_ctx_len, **a)
        else:
            ref_ok, _ = OP.validate_step(case.size, ps, a["req_to_token"], a["req_pool_indices"],
                                         a["seq_lens"], a["kv_indptr"], a["qo_indptr"],
                                         a["out_cache_loc"])
        return lib_ok, ref_ok

    assert both(base) == (True, True)
    n_bad = 0
    for _ in range(300):
        a = {k: np.array(v, copy=True) for k, v in base.items()}
        field = rng.choice(list(a))
        arr = a[field]
        flat = arr.reshape(-1)
        i = int(rng.integers(0, flat.size))
        flat[i] = flat[i] + int(rng.choice([-2, -1, 1, 2, 7, -100, 100000]))
        lib_ok, ref_ok = both(a)
        assert lib_ok == ref_ok, (field, i, flat[i])
        n_bad += not lib_ok
    assert n_bad > 100


def test_prefill_blocks_schedule(lib):
    """pkv_prefill_blocks lists every non-empty row block of PKV_PREFILL_BLOCK_ROWS
    query rows (token x group head), requests in the given order, the block of
    the last rows first; errors for bad head counts, orders and q_lens."""
    q_lens = [300, 0, 64, 65, 1]
    order = [3, 0, 4, 2, 1]
    got = B.pkv_prefill_blocks(q_lens, order, 32, 8)         # G = 4: 64 tokens per block
    want = []
    for i in order:
        nblk = -(-q_lens[i] * 4 // 256)
        want += [(i, nblk - 1 - x) for x in range(nblk)]
    assert [tuple(x) for x in got.tolist()] == want
    assert len(got) == 2 + 5 + 1 + 1
    got1 = B.pkv_prefill_blocks(q_lens, None, 8, 8)          # G = 1: 256 tokens per block
    assert [tuple(x) for x in got1.tolist()] == [(0, 1), (0, 0), (2, 0), (3, 0), (4, 0)]
    for bad in (dict(n_heads=30, n_kv_heads=8), dict(n_heads=0, n_kv_heads=8)):
        with pytest.raises(B.PkvError):
            B.pkv_prefill_blocks(q_lens, order, **bad)
    with pytest.raises(B.PkvError):
        B.pkv_prefill_blocks(q_lens, [0, 0, 1, 2, 3], 32, 8)
    with pytest.raises(B.PkvError):
        B.pkv_prefill_blocks([5, -1], None, 32, 8)
