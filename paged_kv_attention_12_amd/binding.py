"""ctypes binding of libpkv (include/pkv.h): argument marshalling only.

Functions carry the C names.  Device arrays are torch tensors on the current
HIP device (their data_ptr() is passed); host arrays are numpy arrays or
CPU tensors.  Kernels are enqueued on torch's current stream.  Every non-OK
status raises PkvError.  There is no fallback: if libpkv.so is missing, the
first call raises.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK = 0
PKV_ERR_NULL = 1
PKV_ERR_SHAPE = 2
PKV_ERR_DTYPE = 3
PKV_ERR_WORKSPACE_TOO_SMALL = 4
PKV_ERR_BAD_METADATA = 5
PKV_ERR_HIP = 6
PKV_ERR_UNSUPPORTED = 7
PKV_ERR_SCRATCH_LIMIT = 8

PKV_F32 = 0
PKV_BF16 = 1

PKV_LOAD_AUTO = 0
PKV_LOAD_CACHED = 1
PKV_LOAD_STREAM = 2

EXPORTED = (
    "pkv_status_string", "pkv_last_hip_error", "pkv_build_step", "pkv_validate_step",
    "pkv_kv_store", "pkv_decode_workspace_bytes", "pkv_decode_pick_splits",
    "pkv_paged_decode", "pkv_paged_decode_merge", "pkv_paged_prefill",
    "pkv_paged_decode_step", "pkv_decode_step_pick_splits", "pkv_paged_decode_store",
    "pkv_build_positions", "pkv_rope_kv_store", "pkv_decode_advance", "pkv_prefill_blocks",
    "pkv_paged_decode_store_noalloc", "pkv_decode_prefix_groups", "pkv_paged_decode_shared",
    "pkv_rope_kv_store_partial", "pkv_paged_decode_rope_store", "pkv_decode_load_kind",
)

PKV_PREFIX_GROUP_MAX = 16
PKV_PREFIX_GROUP_INTS = 2 + PKV_PREFIX_GROUP_MAX


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class pkv_pool(C.Structure):
    _fields_ = [
        ("k_buffer", C.c_void_p), ("v_buffer", C.c_void_p), ("req_to_token", C.c_void_p),
        ("n_layers", C.c_int64), ("size", C.c_int64), ("num_reqs", C.c_int64),
        ("max_ctx_len", C.c_int64), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("dtype", C.c_int32), ("page_size", C.c_int32), ("v_head_dim", C.c_int32),
        ("load_policy", C.c_int32),
    ]


class pkv_step(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("req_pool_indices", C.c_void_p), ("seq_lens", C.c_void_p),
        ("kv_indptr", C.c_void_p), ("qo_indptr", C.c_void_p), ("out_cache_loc", C.c_void_p),
        ("n_new", C.c_int64), ("max_len", C.c_int32), ("max_q_len", C.c_int32),
        ("prefill_order", C.c_void_p), ("prefill_blocks", C.c_void_p),
        ("n_prefill_blocks", C.c_int64),
    ]


class pkv_prefix_groups(C.Structure):
    _fields_ = [
        ("groups", C.c_void_p), ("kv_start", C.c_void_p), ("n_groups", C.c_int32),
        ("max_prefix", C.c_int32), ("max_members", C.c_int32), ("max_suffix", C.c_int32),
    ]


_lib: Optional[C.CDLL] = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> C.CDLL:
    """Load libpkv.so (built in-tree by paged_kv_attention_12_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libpkv.so not built at {_LIB_PATH}; run "
                          "`python -m paged_kv_attention_12_amd.build`")
    try:  # let torch bring its HIP runtime in first, so both share one runtime
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(_LIB_PATH)
    P = C.c_void_p
    i32, i64, f32, sz = C.c_int32, C.c_int64, C.c_float, C.c_size_t
    sig = {
        "pkv_status_string": (C.c_char_p, [C.c_int]),
        "pkv_last_hip_error": (i32, []),
        "pkv_build_step": (C.c_int, [i32, P, P, P, P, i64, i64, i32, P, P, P, i64, P, P, P, P]),
        "pkv_validate_step": (C.c_int, [i64, i64, i64, i32, P, i32, P, P, P, P, P, i64, P]),
        "pkv_kv_store": (C.c_int, [C.POINTER(pkv_pool), i32, P, P, P, i64, P]),
        "pkv_decode_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "pkv_decode_pick_splits": (i32, [i32, i32, i32, i32, i64, i32]),
        "pkv_decode_load_kind": (i32, [C.POINTER(pkv_pool), i32, i32]),
        "pkv_paged_decode": (C.c_int, [C.POINTER(pkv_pool), i32, C.POINTER(pkv_step), P, i32,
                                       f32, i32, P, sz, P]),
        "pkv_paged_decode_merge": (C.c_int, [i32, i32, i32, C.c_int, i32, P, sz, P, P]),
        "pkv_paged_prefill": (C.c_int, [C.POINTER(pkv_pool), i32, C.POINTER(pkv_step), P, i32,
                                        f32, i32, P, P]),
        "pkv_paged_decode_step": (C.c_int, [C.POINTER(pkv_pool), i32, C.POINTER(pkv_step), P, P,
                                            P, i32, f32, i32, P, sz, P, i64, P, P]),
        "pkv_decode_step_pick_splits": (i32, [i32, i32, i32, i32, i64, i32]),
        "pkv_paged_decode_store": (C.c_int, [C.POINTER(pkv_pool), i32, C.POINTER(pkv_step), P, P,
                                             P, i32, f32, i32, P, sz, P, P]),
        "pkv_paged_decode_store_noalloc": (C.c_int, [C.POINTER(pkv_pool), i32,
                                                     C.POINTER(pkv_step), P, P, P, i32, f32, i32,
                                                     P, P]),
        "pkv_decode_prefix_groups": (C.c_int, [i32, P, P, P, i64, i64, i32, i32, P, i64,
                                               C.POINTER(C.c_int64), P, P, P, P]),
        "pkv_paged_decode_shared": (C.c_int, [C.POINTER(pkv_pool), i32, C.POINTER(pkv_step),
                                              C.POINTER(pkv_prefix_groups), P, P, P, i32, f32,
                                              i32, i32, P, sz, P, P]),
        "pkv_build_positions": (C.c_int, [i32, P, P, P, i64, C.POINTER(C.c_int64)]),
        "pkv_rope_kv_store": (C.c_int, [C.POINTER(pkv_pool), i32, P, P, i32, P, P, P, P, i64, P,
                                        i64, P]),
        "pkv_rope_kv_store_partial": (C.c_int, [C.POINTER(pkv_pool), i32, P, P, i32, P, P, P, P,
                                                i64, i32, P, i64, P]),
        "pkv_decode_advance": (C.c_int, [C.POINTER(pkv_pool), i32, P, P, P, P, P, P]),
        "pkv_prefill_blocks": (C.c_int, [i32, P, P, i32, i32, P, i64, C.POINTER(C.c_int64)]),
        "pkv_paged_decode_rope_store": (C.c_int, [C.POINTER(pkv_pool), i32, C.POINTER(pkv_step),
                                                  P, P, P, P, P, i64, i32, f32, i32, P, sz, P,
                                                  P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().pkv_status_string(int(status)).decode()
    except ImportError:
        return "?"


def _check(status: int, what: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, what)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _dev_ptr(t, name: str, dtype=None) -> int:
    import torch
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _host_i32(x, name: str) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):
        if x.is_cuda:
            raise TypeError(f"{name} must be host memory")
        x = x.detach().numpy()
    a = np.ascontiguousarray(np.asarray(x), dtype=np.int32)
    return a


def _hp(a: Optional[np.ndarray]) -> int:
    return 0 if a is None else a.ctypes.data


def _stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_q_out(q, out, k_buffer, v_buffer, rows: int) -> None:
    """q [rows, n_heads, head_dim] and out [rows, n_heads, v_head_dim] in the pool dtype."""
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != k_buffer.shape[3] \
            or q.dtype != k_buffer.dtype or out.dim() != 3 \
            or tuple(out.shape) != (q.shape[0], q.shape[1], v_buffer.shape[3]) \
            or out.dtype != q.dtype:
        raise ValueError("q must be [rows, n_heads, head_dim] and out [rows, n_heads, "
                         "v_head_dim] in the pool dtype")


def _check_new(k_new, v_new, k_buffer, v_buffer, rows: int) -> None:
    """k_new [rows, n_kv_heads, head_dim], v_new [rows, n_kv_heads, v_head_dim]."""
    if tuple(k_new.shape) != (rows,) + tuple(k_buffer.shape[2:]) \
            or tuple(v_new.shape) != (rows,) + tuple(v_buffer.shape[2:]) \
            or k_new.dtype != k_buffer.dtype or v_new.dtype != k_buffer.dtype:
        raise ValueError("k_new / v_new must be [rows, n_kv_heads, head_dim / v_head_dim] in "
                         "the pool dtype")


def make_pool(k_buffer, v_buffer, req_to_token, page_size: int = 1,
              load_policy: int = PKV_LOAD_AUTO) -> pkv_pool:
    """pkv_pool view of device tensors k_buffer / v_buffer [n_layers, size,
    n_kv_heads, head_dim] and req_to_token int32 [num_reqs, entries]: slots
    (page_size 1, max_ctx_len = entries) or physical page ids of pages of
    page_size tokens (max_ctx_len = entries * page_size).  load_policy: how
    the decode kernels read K/V rows (PKV_LOAD_*)."""
    import torch
    if k_buffer.shape[:3] != v_buffer.shape[:3] or k_buffer.dtype != v_buffer.dtype:
        raise ValueError("k_buffer and v_buffer differ in layers, slots, heads or dtype")
    if k_buffer.dim() != 4 or req_to_token.dim() != 2:
        raise ValueError("pool must be 4-D and req_to_token 2-D")
    p = pkv_pool()
    p.k_buffer = _dev_ptr(k_buffer, "k_buffer")
    p.v_buffer = _dev_ptr(v_buffer, "v_buffer")
    p.req_to_token = _dev_ptr(req_to_token, "req_to_token", torch.int32)
    p.n_layers, p.size, p.n_kv_heads, p.head_dim = (int(s) for s in k_buffer.shape)
    p.v_head_dim = int(v_buffer.shape[3])
    p.num_reqs = int(req_to_token.shape[0])
    p.max_ctx_len = int(req_to_token.shape[1]) * max(int(page_size), 1)
    p.page_size = int(page_size)
    p.dtype = dtype_code(k_buffer)
    p.load_policy = int(load_policy)
    return p


def make_step(batch: int, req_pool_indices, seq_lens, kv_indptr=None, qo_indptr=None,
              out_cache_loc=None, n_new: Optional[int] = None, max_len: int = 0,
              max_q_len: int = 1, prefill_order=None, prefill_blocks=None) -> pkv_step:
    """pkv_step view of device int32 tensors plus the host scalars."""
    import torch
    s = pkv_step()
    s.batch = int(batch)
    s.req_pool_indices = _dev_ptr(req_pool_indices, "req_pool_indices", torch.int32)
    s.seq_lens = _dev_ptr(seq_lens, "seq_lens", torch.int32)
    s.kv_indptr = _dev_ptr(kv_indptr, "kv_indptr", torch.int32)
    s.qo_indptr = _dev_ptr(qo_indptr, "qo_indptr", torch.int32)
    s.out_cache_loc = _dev_ptr(out_cache_loc, "out_cache_loc", torch.int32)
    s.n_new = int(batch if n_new is None else n_new)
    s.max_len = int(max_len)
    s.max_q_len = int(max_q_len)
    s.prefill_order = _dev_ptr(prefill_order, "prefill_order", torch.int32)
    s.prefill_blocks = _dev_ptr(prefill_blocks, "prefill_blocks", torch.int32)
    s.n_prefill_blocks = 0 if prefill_blocks is None else int(prefill_blocks.numel()) // 2
    return s


# ---------------------------------------------------------------------------
# entry points (C names)
# ---------------------------------------------------------------------------
def pkv_build_step(req_pool_indices, seq_lens, req_to_token, q_lens=None,
                   page_size: int = 1) -> dict:
    """Host step metadata: returns dict of int32 numpy arrays kv_indptr,
    qo_indptr, out_cache_loc and ints n_new, max_len, max_q_len.  With
    page_size > 1, req_to_token is the page table."""
    rpi = _host_i32(req_pool_indices, "req_pool_indices")
    sl = _host_i32(seq_lens, "seq_lens")
    ql = _host_i32(q_lens, "q_lens")
    table = _host_i32(req_to_token, "req_to_token")
    if table.ndim != 2:
        raise ValueError("req_to_token must be 2-D")
    B = len(sl)
    if len(rpi) != B or (ql is not None and len(ql) != B):
        raise ValueError("batch arrays differ in length")
    cap = int(ql.sum()) if ql is not None else B
    kv = np.zeros(B + 1, dtype=np.int32)
    qo = np.zeros(B + 1, dtype=np.int32)
    loc = np.zeros(max(cap, 1), dtype=np.int32)
    order = np.zeros(max(B, 1), dtype=np.int32)
    n_new, ml, mq = C.c_int64(0), C.c_int32(0), C.c_int32(0)
    ps = int(page_size)
    st = load().pkv_build_step(B, _hp(rpi), _hp(sl), _hp(ql), _hp(table), table.shape[0],
                               table.shape[1] * max(ps, 1), ps, _hp(kv), _hp(qo), _hp(loc), cap,
                               C.byref(n_new), C.byref(ml), C.byref(mq), _hp(order))
    _check(st, "pkv_build_step")
    return {"kv_indptr": kv, "qo_indptr": qo, "out_cache_loc": loc[:n_new.value].copy(),
            "n_new": n_new.value, "max_len": ml.value, "max_q_len": mq.value,
            "prefill_order": order[:B].copy()}


def pkv_prefill_blocks(q_lens, order, n_heads: int, n_kv_heads: int) -> np.ndarray:
    """Host: the prefill launch schedule, int32 [n_blocks, 2] of (request,
    row block) pairs in launch order (order None: batch order)."""
    ql = _host_i32(q_lens, "q_lens")
    od = _host_i32(order, "order")
    B = len(ql)
    if od is not None and len(od) != B:
        raise ValueError("order must hold one entry per request")
    G = max(int(n_heads) // max(int(n_kv_heads), 1), 1)
    cap = int(sum(-(-max(int(x), 0) * G // 256) for x in ql))
    out = np.zeros((max(cap, 1), 2), dtype=np.int32)
    n = C.c_int64(0)
    st = load().pkv_prefill_blocks(B, _hp(ql), _hp(od), int(n_heads), int(n_kv_heads),
                                   _hp(out), cap, C.byref(n))
    _check(st, "pkv_prefill_blocks")
    return out[:n.value].copy()


def pkv_build_positions(seq_lens, q_lens=None) -> np.ndarray:
    """Host: logical position of every new token, in qo order (int32)."""
    sl = _host_i32(seq_lens, "seq_lens")
    ql = _host_i32(q_lens, "q_lens")
    B = len(sl)
    if ql is not None and len(ql) != B:
        raise ValueError("batch arrays differ in length")
    cap = int(ql.sum()) if ql is not None else B
    pos = np.zeros(max(cap, 1), dtype=np.int32)
    n_new = C.c_int64(0)
    st = load().pkv_build_positions(B, _hp(sl), _hp(ql), _hp(pos), cap, C.byref(n_new))
    _check(st, "pkv_build_positions")
    return pos[:n_new.value].copy()


def pkv_validate_step(size: int, req_to_token, req_pool_indices, seq_lens, kv_indptr,
                      qo_indptr, out_cache_loc, prefill_order=None, page_size: int = 1) -> int:
    """Checked mode on host copies; returns the status (0 = well formed)."""
    table = _host_i32(req_to_token, "req_to_token")
    rpi = _host_i32(req_pool_indices, "req_pool_indices")
    sl = _host_i32(seq_lens, "seq_lens")
    kv = _host_i32(kv_indptr, "kv_indptr")
    qo = _host_i32(qo_indptr, "qo_indptr")
    loc = _host_i32(out_cache_loc, "out_cache_loc")
    order = _host_i32(prefill_order, "prefill_order")
    B = len(sl)
    if order is not None and len(order) != B:
        return PKV_ERR_BAD_METADATA
    if len(rpi) != B or len(kv) != B + 1 or (qo is not None and len(qo) != B + 1):
        return PKV_ERR_BAD_METADATA
    ps = int(page_size)
    return int(load().pkv_validate_step(int(size), table.shape[0], table.shape[1] * max(ps, 1), ps,
                                        _hp(table),
                                        B, _hp(rpi), _hp(sl), _hp(kv), _hp(qo), _hp(loc),
                                        0 if loc is None else len(loc), _hp(order)))


def pkv_kv_store(k_buffer, v_buffer, req_to_token, layer_id: int, k_new, v_new,
                 out_cache_loc, page_size: int = 1) -> None:
    import torch
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size)
    n_new = int(out_cache_loc.numel())
    if n_new:
        _check_new(k_new, v_new, k_buffer, v_buffer, n_new)
    st = load().pkv_kv_store(C.byref(pool), int(layer_id),
                             _dev_ptr(k_new, "k_new") if n_new else 0,
                             _dev_ptr(v_new, "v_new") if n_new else 0,
                             _dev_ptr(out_cache_loc, "out_cache_loc", torch.int32) if n_new else 0,
                             n_new, _stream())
    _check(st, "pkv_kv_store")


def pkv_decode_workspace_bytes(max_batch: int, n_heads: int, head_dim: int,
                               num_splits: int) -> int:
    return int(load().pkv_decode_workspace_bytes(max_batch, n_heads, head_dim, num_splits))


def pkv_decode_load_kind(pool: pkv_pool, batch: int, max_len: int) -> int:
    """1 if the decode kernels read this step's K/V rows with non-temporal
    loads under pool.load_policy, 0 if cached, -1 for invalid fields."""
    return int(load().pkv_decode_load_kind(C.byref(pool), int(batch), int(max_len)))


def pkv_decode_pick_splits(batch: int, n_kv_heads: int, n_heads: int, max_len: int,
                           total_len: int = 0, max_splits: int = 1024) -> int:
    return int(load().pkv_decode_pick_splits(batch, n_kv_heads, n_heads, max_len,
                                             int(total_len), max_splits))


def pkv_paged_decode(k_buffer, v_buffer, req_to_token, layer_id: int, step: pkv_step, q,
                     sm_scale: float, num_splits: int, workspace, page_size: int = 1,
                     load_policy: int = PKV_LOAD_AUTO) -> None:
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size, load_policy)
    if q.dim() != 3 or q.shape[0] != step.batch or q.shape[2] != k_buffer.shape[3] \
            or q.dtype != k_buffer.dtype:
        raise ValueError("q must be [batch, n_heads, head_dim] in the pool dtype")
    st = load().pkv_paged_decode(C.byref(pool), int(layer_id), C.byref(step),
                                 _dev_ptr(q, "q"), int(q.shape[1]), float(sm_scale),
                                 int(num_splits), _dev_ptr(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream())
    _check(st, "pkv_paged_decode")


def pkv_paged_decode_merge(batch: int, n_heads: int, head_dim: int, num_splits: int,
                           workspace, out) -> None:
    if out.dim() != 3 or tuple(out.shape) != (batch, n_heads, head_dim):
        raise ValueError("out must be [batch, n_heads, head_dim]")
    st = load().pkv_paged_decode_merge(int(batch), int(n_heads), int(head_dim), dtype_code(out),
                                       int(num_splits), _dev_ptr(workspace, "workspace"),
                                       workspace.numel() * workspace.element_size(),
                                       _dev_ptr(out, "out"), _stream())
    _check(st, "pkv_paged_decode_merge")


def pkv_decode_step_pick_splits(batch: int, n_kv_heads: int, n_heads: int, max_len: int,
                                total_len: int = 0, max_splits: int = 1024) -> int:
    return int(load().pkv_decode_step_pick_splits(batch, n_kv_heads, n_heads, max_len,
                                                  int(total_len), max_splits))


def pkv_paged_decode_step(k_buffer, v_buffer, req_to_token, layer_id: int, step: pkv_step, q,
                          k_new, v_new, sm_scale: float, num_splits: int, workspace, sync,
                          out, page_size: int = 1) -> None:
    import torch
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size)
    _check_q_out(q, out, k_buffer, v_buffer, step.batch)
    _check_new(k_new, v_new, k_buffer, v_buffer, step.batch)
    st = load().pkv_paged_decode_step(
        C.byref(pool), int(layer_id), C.byref(step), _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"),
        _dev_ptr(v_new, "v_new"), int(q.shape[1]), float(sm_scale), int(num_splits),
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dev_ptr(sync, "sync", torch.int32), int(sync.numel()), _dev_ptr(out, "out"), _stream())
    _check(st, "pkv_paged_decode_step")


def pkv_paged_decode_store(k_buffer, v_buffer, req_to_token, layer_id: int, step: pkv_step, q,
                           k_new, v_new, sm_scale: float, num_splits: int, workspace,
                           out, page_size: int = 1,
                           load_policy: int = PKV_LOAD_AUTO) -> None:
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size, load_policy)
    _check_q_out(q, out, k_buffer, v_buffer, step.batch)
    _check_new(k_new, v_new, k_buffer, v_buffer, step.batch)
    st = load().pkv_paged_decode_store(
        C.byref(pool), int(layer_id), C.byref(step), _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"),
        _dev_ptr(v_new, "v_new"), int(q.shape[1]), float(sm_scale), int(num_splits),
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dev_ptr(out, "out"), _stream())
    _check(st, "pkv_paged_decode_store")


def pkv_paged_decode_rope_store(k_buffer, v_buffer, req_to_token, layer_id: int,
                                step: pkv_step, q, k_new, v_new, position_ids, freqs_cis,
                                sm_scale: float, num_splits: int, workspace, out,
                                page_size: int = 1,
                                load_policy: int = PKV_LOAD_AUTO) -> None:
    """The two-launch decode step with the rotary turn of q and k_new folded
    in (pkv_paged_decode_rope_store)."""
    import torch
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size, load_policy)
    _check_q_out(q, out, k_buffer, v_buffer, step.batch)
    _check_new(k_new, v_new, k_buffer, v_buffer, step.batch)
    if freqs_cis.dim() != 3 or tuple(freqs_cis.shape[1:]) != (int(k_buffer.shape[3]) // 2, 2) \
            or freqs_cis.dtype != torch.float32:
        raise ValueError("freqs_cis must be float32 [max_pos, head_dim / 2, 2]")
    if position_ids.numel() != step.batch:
        raise ValueError("position_ids must hold one entry per request")
    st = load().pkv_paged_decode_rope_store(
        C.byref(pool), int(layer_id), C.byref(step), _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"),
        _dev_ptr(v_new, "v_new"), _dev_ptr(position_ids, "position_ids", torch.int32),
        _dev_ptr(freqs_cis, "freqs_cis", torch.float32), int(freqs_cis.shape[0]),
        int(q.shape[1]), float(sm_scale), int(num_splits), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _dev_ptr(out, "out"), _stream())
    _check(st, "pkv_paged_decode_rope_store")


def pkv_paged_decode_store_noalloc(k_buffer, v_buffer, req_to_token, layer_id: int,
                                   step: pkv_step, q, k_new, v_new, sm_scale: float,
                                   num_splits: int, out, page_size: int = 1) -> None:
    """pkv_paged_decode_store with the split partials in the library's static
    per-device scratch array instead of a caller workspace."""
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size)
    _check_q_out(q, out, k_buffer, v_buffer, step.batch)
    _check_new(k_new, v_new, k_buffer, v_buffer, step.batch)
    st = load().pkv_paged_decode_store_noalloc(
        C.byref(pool), int(layer_id), C.byref(step), _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"),
        _dev_ptr(v_new, "v_new"), int(q.shape[1]), float(sm_scale), int(num_splits),
        _dev_ptr(out, "out"), _stream())
    _check(st, "pkv_paged_decode_store_noalloc")


def pkv_decode_prefix_groups(req_pool_indices, seq_lens, req_to_token, page_size: int = 1,
                             min_prefix: int = 256) -> dict:
    """Host prefix groups of a decode step: dict with groups (int32
    [n_groups, PKV_PREFIX_GROUP_INTS]), kv_start (int32 [batch]) and the ints
    n_groups, max_prefix, max_members, max_suffix."""
    rpi = _host_i32(req_pool_indices, "req_pool_indices")
    sl = _host_i32(seq_lens, "seq_lens")
    table = _host_i32(req_to_token, "req_to_token")
    if table.ndim != 2 or len(rpi) != len(sl):
        raise ValueError("req_to_token must be 2-D and the batch arrays equal in length")
    B = len(sl)
    cap = max(B // 2, 1)
    groups = np.zeros((cap, PKV_PREFIX_GROUP_INTS), dtype=np.int32)
    kv_start = np.zeros(max(B, 1), dtype=np.int32)
    ng = C.c_int64(0)
    mp, mm, ms = (np.zeros(1, dtype=np.int32) for _ in range(3))
    st = load().pkv_decode_prefix_groups(
        B, _hp(rpi), _hp(sl), _hp(table), table.shape[0], table.shape[1] * max(page_size, 1),
        int(page_size), int(min_prefix), _hp(groups), cap, C.byref(ng), _hp(kv_start), _hp(mp),
        _hp(mm), _hp(ms))
    _check(st, "pkv_decode_prefix_groups")
    return {"groups": groups[:ng.value].copy(), "kv_start": kv_start[:B].copy(),
            "n_groups": int(ng.value), "max_prefix": int(mp[0]), "max_members": int(mm[0]),
            "max_suffix": int(ms[0])}


def make_prefix_groups(groups_dev, kv_start_dev, n_groups: int, max_prefix: int,
                       max_members: int, max_suffix: int) -> pkv_prefix_groups:
    import torch
    g = pkv_prefix_groups()
    g.groups = _dev_ptr(groups_dev, "groups", torch.int32)
    g.kv_start = _dev_ptr(kv_start_dev, "kv_start", torch.int32)
    g.n_groups, g.max_prefix = int(n_groups), int(max_prefix)
    g.max_members, g.max_suffix = int(max_members), int(max_suffix)
    return g


def pkv_paged_decode_shared(k_buffer, v_buffer, req_to_token, layer_id: int, step: pkv_step,
                            groups: Optional[pkv_prefix_groups], q, k_new, v_new,
                            sm_scale: float, num_splits: int, prefix_splits: int, workspace,
                            out, page_size: int = 1) -> None:
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size)
    _check_q_out(q, out, k_buffer, v_buffer, step.batch)
    _check_new(k_new, v_new, k_buffer, v_buffer, step.batch)
    st = load().pkv_paged_decode_shared(
        C.byref(pool), int(layer_id), C.byref(step), C.byref(groups) if groups is not None else None,
        _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"), int(q.shape[1]),
        float(sm_scale), int(num_splits), int(prefix_splits), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _dev_ptr(out, "out"), _stream())
    _check(st, "pkv_paged_decode_shared")


def pkv_rope_kv_store(k_buffer, v_buffer, req_to_token, layer_id: int, q, q_out, k_new, v_new,
                      position_ids, freqs_cis, out_cache_loc, page_size: int = 1,
                      rope_dim: Optional[int] = None) -> None:
    """Rotary write of the new tokens (pkv_rope_kv_store); with rope_dim, only
    the last rope_dim dims of each query / key row turn
    (pkv_rope_kv_store_partial, freqs_cis [max_pos, rope_dim / 2, 2])."""
    import torch
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size)
    n_new = int(k_new.shape[0])
    if q.dim() != 3 or q.shape[0] != n_new or q.shape[2] != k_buffer.shape[3] \
            or q.dtype != k_buffer.dtype or q_out.shape != q.shape or q_out.dtype != q.dtype:
        raise ValueError("q / q_out must be [n_new, n_heads, head_dim] in the pool dtype")
    _check_new(k_new, v_new, k_buffer, v_buffer, n_new)
    R = int(k_buffer.shape[3]) if rope_dim is None else int(rope_dim)
    if freqs_cis.dim() != 3 or tuple(freqs_cis.shape[1:]) != (R // 2, 2) \
            or freqs_cis.dtype != torch.float32:
        raise ValueError("freqs_cis must be float32 [max_pos, rotated dims / 2, 2]")
    if position_ids.numel() != n_new or out_cache_loc.numel() != n_new:
        raise ValueError("position_ids / out_cache_loc must hold n_new entries")
    args = [C.byref(pool), int(layer_id), _dev_ptr(q, "q"), _dev_ptr(q_out, "q_out"),
            int(q.shape[1]), _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"),
            _dev_ptr(position_ids, "position_ids", torch.int32),
            _dev_ptr(freqs_cis, "freqs_cis", torch.float32), int(freqs_cis.shape[0])]
    tail = [_dev_ptr(out_cache_loc, "out_cache_loc", torch.int32), n_new, _stream()]
    if rope_dim is None:
        st = load().pkv_rope_kv_store(*args, *tail)
        _check(st, "pkv_rope_kv_store")
    else:
        st = load().pkv_rope_kv_store_partial(*args, R, *tail)
        _check(st, "pkv_rope_kv_store_partial")


def pkv_decode_advance(k_buffer, v_buffer, req_to_token, req_pool_indices, seq_lens, kv_indptr,
                       out_cache_loc, position_ids, page_size: int = 1) -> None:
    import torch
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size)
    n = int(seq_lens.numel())
    if req_pool_indices.numel() != n or out_cache_loc.numel() != n or \
            (position_ids is not None and position_ids.numel() != n) or \
            (kv_indptr is not None and kv_indptr.numel() != n + 1):
        raise ValueError("decode metadata arrays disagree in length")
    st = load().pkv_decode_advance(
        C.byref(pool), n, _dev_ptr(req_pool_indices, "req_pool_indices", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), _dev_ptr(kv_indptr, "kv_indptr", torch.int32),
        _dev_ptr(out_cache_loc, "out_cache_loc", torch.int32),
        _dev_ptr(position_ids, "position_ids", torch.int32), _stream())
    _check(st, "pkv_decode_advance")


def pkv_paged_prefill(k_buffer, v_buffer, req_to_token, layer_id: int, step: pkv_step, q,
                      sm_scale: float, causal: bool, out, page_size: int = 1) -> None:
    pool = make_pool(k_buffer, v_buffer, req_to_token, page_size)
    _check_q_out(q, out, k_buffer, v_buffer, step.n_new)
    st = load().pkv_paged_prefill(C.byref(pool), int(layer_id), C.byref(step), _dev_ptr(q, "q"),
                                  int(q.shape[1]), float(sm_scale), 1 if causal else 0,
                                  _dev_ptr(out, "out"), _stream())
    _check(st, "pkv_paged_prefill")
