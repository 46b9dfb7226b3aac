"""ctypes binding of libhstu (include/hstu.h), function for function.

Argument marshalling only: every step of the HSTU path runs in the library's
HIP kernels.  Device buffers are passed as integer addresses (e.g. a torch
tensor's data_ptr()), streams as the raw hipStream_t handle.  Loading fails
loudly when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# HSTU_LIBRARY names another build of the same ABI (the tests' host-only
# sanitizer build); by default the in-tree HIP library
LIB_PATH = os.environ.get("HSTU_LIBRARY") or os.path.join(PKG, "libhstu.so")

HSTU_OK, HSTU_ERR_INVALID, HSTU_ERR_NO_SPACE, HSTU_ERR_UNKNOWN_USER, HSTU_ERR_DEVICE, \
    HSTU_ERR_UNSUPPORTED = range(6)
HSTU_F32, HSTU_BF16 = 0, 1

c_i32, c_i64, c_f32, c_size, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
P_i32, P_i64, P_f32 = ctypes.POINTER(c_i32), ctypes.POINTER(c_i64), ctypes.POINTER(c_f32)


class HstuError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hstu status {status}: {msg}")
        self.status = status


class hstu_kv_cache_desc(ctypes.Structure):
    _fields_ = [("num_layers", c_i32), ("num_heads", c_i32), ("head_dim", c_i32), ("page_size", c_i32),
                ("num_pages", c_i32), ("dtype", c_i32), ("k_pool", c_vp), ("v_pool", c_vp),
                ("initial_free_order", P_i32)]


class hstu_batch_desc(ctypes.Structure):
    _fields_ = [("B", c_i32), ("num_heads", c_i32), ("head_dim", c_i32), ("new_len", P_i32),
                ("cached_len", P_i32), ("n_targets", P_i32), ("norm_n", P_f32), ("page_size", c_i32),
                ("max_pages", c_i32)]


class hstu_plan_info(ctypes.Structure):
    _fields_ = [("n_new_total", c_i32), ("n_work_items", c_i32), ("n_partial_slots", c_i32),
                ("pairs", c_i64), ("meta_bytes", c_size), ("attn_workspace_bytes", c_size)]


class hstu_attn_args(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("plan", c_vp), ("q", c_vp), ("q_row_stride", c_i64), ("k", c_vp),
                ("v", c_vp), ("kv_row_stride", c_i64), ("cache", c_vp), ("layer", c_i32),
                ("d_page_table", c_vp), ("rab", c_vp), ("num_buckets", c_i32), ("out", c_vp),
                ("workspace", c_vp), ("workspace_bytes", c_size)]


class hstu_layer_args(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("d_model", c_i32), ("eps", c_f32), ("plan", c_vp), ("x", c_vp),
                ("y", c_vp), ("w1", c_vp), ("w2", c_vp), ("rab", c_vp), ("num_buckets", c_i32),
                ("cache", c_vp), ("layer", c_i32), ("d_page_table", c_vp), ("workspace", c_vp),
                ("workspace_bytes", c_size), ("uvqk_out", c_vp), ("o_out", c_vp), ("g_out", c_vp),
                ("s_out", c_vp), ("w1_colsum", c_vp),
                ("x_stats", c_vp), ("y_stats", c_vp), ("row_slots", c_vp)]


class hstu_layer_bwd_args(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("d_model", c_i32), ("eps", c_f32), ("plan", c_vp), ("x", c_vp),
                ("w1t", c_vp), ("w2t", c_vp), ("rab", c_vp), ("num_buckets", c_i32), ("uvqk", c_vp), ("s", c_vp),
                ("o", c_vp), ("dy", c_vp), ("dx", c_vp), ("dw1", c_vp), ("dw2", c_vp), ("drab", c_vp),
                ("workspace", c_vp), ("workspace_bytes", c_size)]


class hstu_head_args(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("d_model", c_i32), ("num_tasks", c_i32), ("hidden", c_i32), ("y", c_vp),
                ("y_rows", c_i32), ("d_rows", c_vp), ("n_rows", c_i32), ("w_hidden", c_vp), ("b_hidden", c_vp),
                ("w_out", c_vp), ("b_out", c_vp), ("logits", c_vp), ("workspace", c_vp),
                ("workspace_bytes", c_size)]


class hstu_batcher_desc(ctypes.Structure):
    _fields_ = [("max_batch", c_i32), ("max_delay_us", c_i64), ("max_tokens", c_i64)]


# name -> (restype, argtypes); every symbol include/hstu.h declares
SIGNATURES = {
    "hstu_last_error": (ctypes.c_char_p, []),
    "hstu_abi_version": (c_i32, []),
    "kv_cache_create": (c_i32, [ctypes.POINTER(hstu_kv_cache_desc), ctypes.POINTER(c_vp)]),
    "kv_cache_destroy": (c_i32, [c_vp]),
    "kv_lookup": (c_i32, [c_vp, P_i64, c_i32, P_i32]),
    "kv_evict_lru": (c_i32, [c_vp, c_i32, P_i64, c_i32, P_i64, c_i32, P_i32]),
    "kv_lru_victims": (c_i32, [c_vp, c_i32, P_i64, c_i32, P_i64, c_i32, P_i32]),
    "kv_page_alloc": (c_i32, [c_vp, P_i64, P_i32, c_i32, P_i32, c_i32, P_i32]),
    "kv_truncate": (c_i32, [c_vp, c_i64, c_i32]),
    "kv_free_pages": (c_i32, [c_vp, P_i32]),
    "kv_page_table": (c_i32, [c_vp, P_i64, c_i32, P_i32, c_i32, P_i32]),
    "kv_state_dump": (c_i32, [c_vp, c_vp, c_size, ctypes.POINTER(c_size)]),
    "kv_state_load": (c_i32, [c_vp, c_vp, c_size]),
    "kv_host_attach": (c_i32, [c_vp, c_vp, c_vp, c_i32]),
    "kv_residency": (c_i32, [c_vp, P_i64, c_i32, P_i32, P_i32]),
    "kv_offload": (c_i32, [c_vp, P_i64, c_i32, P_i64, c_i32, c_vp, P_i64, c_i32, P_i32]),
    "kv_onboard": (c_i32, [c_vp, P_i64, c_i32, c_vp]),
    "kv_page_append": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i64, c_i32, c_vp]),
    "kv_page_gather": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "hstu_plan_create": (c_i32, [ctypes.POINTER(hstu_batch_desc), ctypes.POINTER(c_vp)]),
    "hstu_plan_destroy": (c_i32, [c_vp]),
    "hstu_plan_get_info": (c_i32, [c_vp, ctypes.POINTER(hstu_plan_info)]),
    "hstu_plan_upload": (c_i32, [c_vp, c_vp, c_size, c_vp]),
    "hstu_plan_get_items": (c_i32, [c_vp, P_i32, c_i32, P_i32]),
    "hstu_attn_fwd": (c_i32, [ctypes.POINTER(hstu_attn_args), c_vp]),
    "hstu_attn_fwd_static": (c_i32, [ctypes.POINTER(hstu_attn_args), c_vp]),
    "hstu_attn_static_scratch_bytes": (c_size, []),
    "hstu_layer_workspace_size": (c_i32, [ctypes.POINTER(hstu_layer_args), ctypes.POINTER(c_size)]),
    "hstu_layer_forward": (c_i32, [ctypes.POINTER(hstu_layer_args), c_vp]),
    "hstu_stack_forward": (c_i32, [ctypes.POINTER(hstu_layer_args), c_i32, c_vp]),
    "hstu_w1_colsum": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp]),
    "hstu_layer_backward_workspace_size": (c_i32, [ctypes.POINTER(hstu_layer_bwd_args), ctypes.POINTER(c_size)]),
    "hstu_layer_backward": (c_i32, [ctypes.POINTER(hstu_layer_bwd_args), c_vp]),
    "hstu_head_workspace_size": (c_i32, [ctypes.POINTER(hstu_head_args), ctypes.POINTER(c_size)]),
    "hstu_head_forward": (c_i32, [ctypes.POINTER(hstu_head_args), c_vp]),
    "hstu_batcher_create": (c_i32, [ctypes.POINTER(hstu_batcher_desc), ctypes.POINTER(c_vp)]),
    "hstu_batcher_destroy": (c_i32, [c_vp]),
    "hstu_batcher_submit": (c_i32, [c_vp, c_i64, c_i64, c_i32, c_i64]),
    "hstu_batcher_next": (c_i32, [c_vp, c_i64, P_i64, c_i32, P_i32, P_i64]),
    "hstu_batcher_pending": (c_i32, [c_vp, P_i32]),
    "hstu_timing_enable": (c_i32, [c_i32]),
    "hstu_attn_stamps": (c_i32, [c_vp, c_i64]),
    "hstu_ceiling_mfma": (c_i32, [c_i32, c_i32, c_vp, c_vp]),
    "hstu_ceiling_read": (c_i32, [c_vp, c_i64, c_vp, c_vp]),
    "hstu_ceiling_copy": (c_i32, [c_vp, c_vp, c_i64, c_vp]),
    "hstu_timing_read": (c_i32, [ctypes.c_char_p, P_i32, ctypes.POINTER(ctypes.c_double)]),
}

TIMED_KERNELS = ("layer_norm", "f1_gemm", "append", "attention", "reduce_gate", "f2_gemm", "gather", "head",
                 "bwd_attention", "bwd_gemm", "bwd_rows", "attention_cached", "attention_prefill")

_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m generative_recommender_sequence_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != HSTU_OK:
        msg = lib().hstu_last_error().decode()
        raise HstuError(status, f"{what}: {msg}")


def _arr(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


# ---------------------------------------------------------------------------
# KV cache
# ---------------------------------------------------------------------------

def kv_cache_create(num_layers, num_heads, head_dim, page_size, num_pages, dtype,
                    k_pool: int = 0, v_pool: int = 0, initial_free_order=None) -> int:
    fo = None if initial_free_order is None else _arr(initial_free_order, np.int32)
    d = hstu_kv_cache_desc(num_layers, num_heads, head_dim, page_size, num_pages, dtype,
                           k_pool or None, v_pool or None, None if fo is None else _ptr(fo, c_i32))
    h = c_vp()
    _check(lib().kv_cache_create(ctypes.byref(d), ctypes.byref(h)), "kv_cache_create")
    return h.value


def kv_cache_destroy(h: int):
    _check(lib().kv_cache_destroy(h), "kv_cache_destroy")


def kv_lookup(h: int, users) -> np.ndarray:
    u = _arr(users, np.int64)
    out = np.zeros(max(len(u), 1), np.int32)
    _check(lib().kv_lookup(h, _ptr(u, c_i64), len(u), _ptr(out, c_i32)), "kv_lookup")
    return out[:len(u)]


def kv_evict_lru(h: int, pages_needed: int, pinned, cap: int = 1 << 16) -> np.ndarray:
    p = _arr(pinned, np.int64) if len(pinned) else np.zeros(1, np.int64)
    ev = np.zeros(max(cap, 1), np.int64)
    n = c_i32(0)
    _check(lib().kv_evict_lru(h, int(pages_needed), _ptr(p, c_i64), len(pinned), _ptr(ev, c_i64), cap,
                              ctypes.byref(n)), "kv_evict_lru")
    return ev[:n.value].copy()


def kv_lru_victims(h: int, pages_needed: int, pinned, cap: int = 1 << 16) -> np.ndarray:
    p = _arr(pinned, np.int64) if len(pinned) else np.zeros(1, np.int64)
    ev = np.zeros(max(cap, 1), np.int64)
    n = c_i32(0)
    _check(lib().kv_lru_victims(h, int(pages_needed), _ptr(p, c_i64), len(pinned), _ptr(ev, c_i64), cap,
                                ctypes.byref(n)), "kv_lru_victims")
    return ev[:n.value].copy()


def kv_page_alloc(h: int, users, n_new, max_pages: int):
    u = _arr(users, np.int64)
    nn = _arr(n_new, np.int32)
    pt = np.zeros((max(len(u), 1), max(max_pages, 1)), np.int32)
    kl = np.zeros(max(len(u), 1), np.int32)
    _check(lib().kv_page_alloc(h, _ptr(u, c_i64), _ptr(nn, c_i32), len(u), _ptr(pt, c_i32), max_pages,
                               _ptr(kl, c_i32)), "kv_page_alloc")
    return pt[:len(u), :max_pages].copy(), kl[:len(u)].copy()


def kv_truncate(h: int, user: int, new_len: int):
    _check(lib().kv_truncate(h, int(user), int(new_len)), "kv_truncate")


def kv_free_pages(h: int) -> int:
    n = c_i32(0)
    _check(lib().kv_free_pages(h, ctypes.byref(n)), "kv_free_pages")
    return n.value


def kv_page_table(h: int, users, max_pages: int):
    u = _arr(users, np.int64)
    pt = np.zeros((max(len(u), 1), max(max_pages, 1)), np.int32)
    kl = np.zeros(max(len(u), 1), np.int32)
    _check(lib().kv_page_table(h, _ptr(u, c_i64), len(u), _ptr(pt, c_i32), max_pages, _ptr(kl, c_i32)),
           "kv_page_table")
    return pt[:len(u), :max_pages].copy(), kl[:len(u)].copy()


def kv_state_dump(h: int) -> bytes:
    need = c_size(0)
    _check(lib().kv_state_dump(h, None, 0, ctypes.byref(need)), "kv_state_dump")
    buf = (ctypes.c_uint8 * max(need.value, 1))()
    _check(lib().kv_state_dump(h, buf, need.value, ctypes.byref(need)), "kv_state_dump")
    return bytes(buf)[:need.value]


def kv_state_load(h: int, data: bytes):
    buf = (ctypes.c_uint8 * max(len(data), 1)).from_buffer_copy(data if data else b"\0")
    _check(lib().kv_state_load(h, buf, len(data)), "kv_state_load")


def kv_host_attach(h: int, host_pages: int, host_k_pool: int = 0, host_v_pool: int = 0):
    _check(lib().kv_host_attach(h, host_k_pool or None, host_v_pool or None, int(host_pages)),
           "kv_host_attach")


def kv_residency(h: int, users):
    u = _arr(users, np.int64)
    where = np.zeros(max(len(u), 1), np.int32)
    ln = np.zeros(max(len(u), 1), np.int32)
    _check(lib().kv_residency(h, _ptr(u, c_i64), len(u), _ptr(where, c_i32), _ptr(ln, c_i32)),
           "kv_residency")
    return where[:len(u)].copy(), ln[:len(u)].copy()


def kv_offload(h: int, users, stream: int = 0, pinned=(), cap: int = 1 << 16) -> np.ndarray:
    u = _arr(users, np.int64) if len(users) else np.zeros(1, np.int64)
    p = _arr(pinned, np.int64) if len(pinned) else np.zeros(1, np.int64)
    ev = np.zeros(max(cap, 1), np.int64)
    n = c_i32(0)
    _check(lib().kv_offload(h, _ptr(u, c_i64), len(users), _ptr(p, c_i64), len(pinned), stream or None,
                            _ptr(ev, c_i64), cap, ctypes.byref(n)), "kv_offload")
    return ev[:n.value].copy()


def kv_onboard(h: int, users, stream: int = 0):
    u = _arr(users, np.int64) if len(users) else np.zeros(1, np.int64)
    _check(lib().kv_onboard(h, _ptr(u, c_i64), len(users), stream or None), "kv_onboard")


def kv_page_append(h: int, layer: int, B: int, d_new_offsets: int, d_start_pos: int, d_page_table: int,
                   max_pages: int, k_new: int, v_new: int, row_stride: int, n_new_total: int, stream: int):
    _check(lib().kv_page_append(h, layer, B, d_new_offsets, d_start_pos, d_page_table, max_pages, k_new,
                                v_new, row_stride, n_new_total, stream), "kv_page_append")


def kv_page_gather(h: int, layer: int, B: int, d_page_table: int, max_pages: int, d_kv_len: int,
                   d_out_offsets: int, n_out_total: int, k_out: int, v_out: int, stream: int):
    _check(lib().kv_page_gather(h, layer, B, d_page_table, max_pages, d_kv_len, d_out_offsets,
                                n_out_total, k_out, v_out, stream), "kv_page_gather")


class KVCache:
    """Owning wrapper of an hstu_kv_cache handle (host metadata only)."""

    def __init__(self, handle: int):
        self.h = handle

    @classmethod
    def host_only(cls, num_pages, page_size, free_order=None, num_layers=1, num_heads=1, head_dim=8,
                  dtype=HSTU_BF16):
        return cls(kv_cache_create(num_layers, num_heads, head_dim, page_size, num_pages, dtype, 0, 0,
                                   free_order))

    def __del__(self):
        if getattr(self, "h", None):
            lib().kv_cache_destroy(self.h)
            self.h = None

    # the (rc, ...) convention of the cross-implementation allocator tests
    def lookup(self, users):
        try:
            return HSTU_OK, kv_lookup(self.h, users)
        except HstuError as e:
            return e.status, None

    def evict_lru(self, pages_needed, pinned, cap=1 << 16):
        try:
            return HSTU_OK, kv_evict_lru(self.h, pages_needed, pinned, cap)
        except HstuError as e:
            return e.status, []

    def lru_victims(self, pages_needed, pinned, cap=1 << 16):
        try:
            return HSTU_OK, kv_lru_victims(self.h, pages_needed, pinned, cap)
        except HstuError as e:
            return e.status, []

    def alloc(self, users, n_new, max_pages):
        try:
            pt, kl = kv_page_alloc(self.h, users, n_new, max_pages)
            return HSTU_OK, pt, kl
        except HstuError as e:
            return e.status, None, None

    def truncate(self, user, new_len):
        try:
            kv_truncate(self.h, user, new_len)
            return HSTU_OK
        except HstuError as e:
            return e.status

    def host_attach(self, host_pages, host_k_pool: int = 0, host_v_pool: int = 0):
        try:
            kv_host_attach(self.h, host_pages, host_k_pool, host_v_pool)
            return HSTU_OK
        except HstuError as e:
            return e.status

    def residency(self, users):
        try:
            where, ln = kv_residency(self.h, users)
            return HSTU_OK, [int(x) for x in where], [int(x) for x in ln]
        except HstuError as e:
            return e.status, None, None

    def offload(self, users, pinned=(), cap=1 << 16, stream: int = 0):
        try:
            return HSTU_OK, kv_offload(self.h, users, stream, pinned, cap)
        except HstuError as e:
            return e.status, []

    def onboard(self, users, stream: int = 0):
        try:
            kv_onboard(self.h, users, stream)
            return HSTU_OK
        except HstuError as e:
            return e.status

    def dump(self) -> bytes:
        return kv_state_dump(self.h)

    def load(self, data: bytes):
        kv_state_load(self.h, data)

    def free_pages(self) -> int:
        return kv_free_pages(self.h)


# ---------------------------------------------------------------------------
# plan, attention, layer
# ---------------------------------------------------------------------------

def hstu_plan_create(num_heads, head_dim, new_len, cached_len, n_targets, norm_n=None,
                     page_size: int = 0, max_pages: int = 0) -> int:
    nl, cl, nt = _arr(new_len, np.int32), _arr(cached_len, np.int32), _arr(n_targets, np.int32)
    nn = None if norm_n is None else _arr(norm_n, np.float32)
    B = len(nl)
    keep = [np.zeros(1, np.int32) if B == 0 else a for a in (nl, cl, nt)]
    d = hstu_batch_desc(B, num_heads, head_dim, _ptr(keep[0], c_i32), _ptr(keep[1], c_i32),
                        _ptr(keep[2], c_i32), None if nn is None else _ptr(nn, c_f32), page_size, max_pages)
    h = c_vp()
    _check(lib().hstu_plan_create(ctypes.byref(d), ctypes.byref(h)), "hstu_plan_create")
    return h.value


def hstu_plan_destroy(h: int):
    _check(lib().hstu_plan_destroy(h), "hstu_plan_destroy")


def hstu_plan_get_info(h: int) -> hstu_plan_info:
    info = hstu_plan_info()
    _check(lib().hstu_plan_get_info(h, ctypes.byref(info)), "hstu_plan_get_info")
    return info


def hstu_plan_get_items(h: int) -> np.ndarray:
    """The plan's attention work items in launch order: int32 [n][6] =
    (user, head, q-block, first key tile, end key tile, slot; -1 = padding)."""
    n = c_i32()
    _check(lib().hstu_plan_get_items(h, None, 0, ctypes.byref(n)), "hstu_plan_get_items")
    out = np.zeros((max(n.value, 1), 6), np.int32)
    _check(lib().hstu_plan_get_items(h, _ptr(out, c_i32), n.value, ctypes.byref(n)), "hstu_plan_get_items")
    return out[:n.value]


def hstu_plan_upload(h: int, d_meta: int, nbytes: int, stream: int):
    _check(lib().hstu_plan_upload(h, d_meta, nbytes, stream), "hstu_plan_upload")


def hstu_attn_fwd(args: hstu_attn_args, stream: int):
    _check(lib().hstu_attn_fwd(ctypes.byref(args), stream), "hstu_attn_fwd")


def hstu_attn_fwd_static(args: hstu_attn_args, stream: int):
    _check(lib().hstu_attn_fwd_static(ctypes.byref(args), stream), "hstu_attn_fwd_static")


def hstu_attn_static_scratch_bytes() -> int:
    return int(lib().hstu_attn_static_scratch_bytes())


def hstu_layer_workspace_size(args: hstu_layer_args) -> int:
    n = c_size(0)
    _check(lib().hstu_layer_workspace_size(ctypes.byref(args), ctypes.byref(n)), "hstu_layer_workspace_size")
    return n.value


def hstu_layer_forward(args: hstu_layer_args, stream: int):
    _check(lib().hstu_layer_forward(ctypes.byref(args), stream), "hstu_layer_forward")


def hstu_stack_forward(layers, stream: int):
    """layers: a sequence (or ctypes array) of hstu_layer_args."""
    if not isinstance(layers, ctypes.Array):
        arr = (hstu_layer_args * len(layers))(*layers)
    else:
        arr = layers
    _check(lib().hstu_stack_forward(arr, len(arr), stream), "hstu_stack_forward")


def hstu_w1_colsum(w1: int, rows: int, d_model: int, out: int, stream: int):
    _check(lib().hstu_w1_colsum(w1, rows, d_model, out, stream or None), "hstu_w1_colsum")


def hstu_layer_backward_workspace_size(args: hstu_layer_bwd_args) -> int:
    n = c_size(0)
    _check(lib().hstu_layer_backward_workspace_size(ctypes.byref(args), ctypes.byref(n)),
           "hstu_layer_backward_workspace_size")
    return n.value


def hstu_layer_backward(args: hstu_layer_bwd_args, stream: int):
    _check(lib().hstu_layer_backward(ctypes.byref(args), stream or None), "hstu_layer_backward")


def hstu_head_workspace_size(args: hstu_head_args) -> int:
    n = c_size(0)
    _check(lib().hstu_head_workspace_size(ctypes.byref(args), ctypes.byref(n)), "hstu_head_workspace_size")
    return n.value


def hstu_head_forward(args: hstu_head_args, stream: int):
    _check(lib().hstu_head_forward(ctypes.byref(args), stream or None), "hstu_head_forward")


class Batcher:
    """Owning wrapper of an hstu_batcher (host only)."""

    def __init__(self, max_batch: int = 8, max_delay_us: int = 0, max_tokens: int = 0):
        d = hstu_batcher_desc(max_batch, max_delay_us, max_tokens)
        h = c_vp()
        _check(lib().hstu_batcher_create(ctypes.byref(d), ctypes.byref(h)), "hstu_batcher_create")
        self.h, self.max_batch = h.value, max_batch
        self._ids = np.zeros(max_batch, np.int64)

    def __del__(self):
        if getattr(self, "h", None):
            lib().hstu_batcher_destroy(self.h)
            self.h = None

    def submit(self, request_id: int, user: int, n_new: int, arrival_us: int):
        _check(lib().hstu_batcher_submit(self.h, int(request_id), int(user), int(n_new), int(arrival_us)),
               "hstu_batcher_submit")

    def next(self, now_us: int):
        """(released request ids, wait_us)."""
        n, wait = c_i32(0), c_i64(0)
        _check(lib().hstu_batcher_next(self.h, int(now_us), _ptr(self._ids, c_i64), len(self._ids),
                                       ctypes.byref(n), ctypes.byref(wait)), "hstu_batcher_next")
        return [int(i) for i in self._ids[:n.value]], wait.value

    def pending(self) -> int:
        n = c_i32(0)
        _check(lib().hstu_batcher_pending(self.h, ctypes.byref(n)), "hstu_batcher_pending")
        return n.value


def hstu_timing_enable(enable, split_attention: bool = False):
    """enable: time every launch; split_attention: also run the attention of
    requests planned from now on over users with and without a cached prefix
    as two grids, timed apart."""
    mode = (2 if split_attention else 1) if enable else 0
    _check(lib().hstu_timing_enable(mode), "hstu_timing_enable")


def hstu_timing_read(kernel: str):
    """(launches, total milliseconds) of `kernel` since the last read."""
    n = c_i32(0)
    ms = ctypes.c_double(0.0)
    _check(lib().hstu_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)), "hstu_timing_read")
    return n.value, ms.value


def header_symbols(header_path: Optional[str] = None) -> Sequence[str]:
    """Function names declared in include/hstu.h."""
    import re
    if header_path is None:
        header_path = os.path.join(os.path.dirname(PKG), "include", "hstu.h")
    text = open(header_path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def hstu_ceiling_mfma(blocks: int, iters: int, out: int, stream: int):
    _check(lib().hstu_ceiling_mfma(blocks, iters, out, stream), "hstu_ceiling_mfma")


def hstu_ceiling_read(src: int, nbytes: int, out: int, stream: int):
    _check(lib().hstu_ceiling_read(src, nbytes, out, stream), "hstu_ceiling_read")


def hstu_ceiling_copy(src: int, dst: int, nbytes: int, stream: int):
    _check(lib().hstu_ceiling_copy(src, dst, nbytes, stream), "hstu_ceiling_copy")


ATTN_STAMP_DTYPE = np.dtype([("start", "<u8"), ("setup_done", "<u8"), ("loop_done", "<u8"), ("end", "<u8"),
                             ("hw_id", "<u4"), ("xcc_id", "<u4"), ("slot", "<i4"), ("tiles", "<i4")])


def hstu_attn_stamps(d_stamps: int, capacity: int):
    """Registers (capacity > 0) or clears the attention phase-record buffer."""
    _check(lib().hstu_attn_stamps(d_stamps or None, capacity), "hstu_attn_stamps")
