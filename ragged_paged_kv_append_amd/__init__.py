"""Ragged paged attention with KV append for AMD Instinct MI355X (gfx950).

Thin Python binding of ``librpa.so`` (the C ABI declared in ``include/rpa.h``).
It only marshals arguments: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.  If the library is not
built, every call raises ``RpaError``; there is no fallback.

Functions carry the C names (``rpa_plan_create``, ``rpa_plan_upload``,
``rpa_kv_append``, ``rpa_batch_attention``, ``rpa_merge_state``, ...).  The
``Plan`` class bundles a plan with its device workspace for convenience.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librpa.so")

RPA_OK = 0
RPA_ERR_INVALID_ARG = -1
RPA_ERR_UNSUPPORTED = -2
RPA_ERR_WORKSPACE_TOO_SMALL = -3
RPA_ERR_PAGE_OOB = -4
RPA_ERR_DUPLICATE_WRITE_PAGE = -5
RPA_ERR_HIP = -6
RPA_ERR_NOT_UPLOADED = -7
RPA_ERR_HOST_ALLOC = -8
RPA_ERR_INTERNAL = -9

RPA_DTYPE_F32 = 0
RPA_DTYPE_BF16 = 1

# Kernel classes reported by the plan's "items" table.
KC_GENERIC, KC_DECODE, KC_PREFILL, KC_MLA = 0, 1, 2, 3

EXPORTED_SYMBOLS = (
    "rpa_plan_create", "rpa_plan_create_tree", "rpa_plan_create_split", "rpa_plan_workspace_size",
    "rpa_plan_upload", "rpa_kv_append", "rpa_batch_attention", "rpa_batch_attention_noalloc",
    "rpa_split_attention", "rpa_merge_state",
    "rpa_page_copy",
    "rpa_plan_destroy",
    "rpa_status_string",
    "rpa_last_error_message", "rpa_abi_version", "rpa_plan_debug_dump", "rpa_profile_enable",
    "rpa_profile_read", "rpa_profile_reset", "rpa_profile_select",
)


class RpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class rpa_attn_config(ctypes.Structure):
    _fields_ = [("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


class rpa_batch_desc(ctypes.Structure):
    _fields_ = [("batch_size", ctypes.c_int32), ("qo_indptr", ctypes.POINTER(ctypes.c_int32)),
                ("kv_len", ctypes.POINTER(ctypes.c_int32)),
                ("kv_page_indptr", ctypes.POINTER(ctypes.c_int32)),
                ("kv_page_indices", ctypes.POINTER(ctypes.c_int32)),
                ("num_pages", ctypes.c_int32)]


class rpa_cache_strides(ctypes.Structure):
    _fields_ = [("page_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded librpa.so (raises RpaError if it has not been built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RpaError(RPA_ERR_UNSUPPORTED,
                       f"HIP library not built: {LIB_PATH} is missing "
                       "(run python -m ragged_paged_kv_append_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    L.rpa_plan_create.argtypes = [P(rpa_attn_config), P(rpa_batch_desc), i32, P(vp)]
    L.rpa_plan_create_tree.argtypes = [P(rpa_attn_config), P(rpa_batch_desc),
                                       P(ctypes.c_int32), P(ctypes.c_uint32), i32, P(vp)]
    L.rpa_plan_create_split.argtypes = [P(rpa_attn_config), P(rpa_batch_desc), i32, P(vp)]
    L.rpa_plan_workspace_size.argtypes = [vp, P(sz)]
    L.rpa_plan_upload.argtypes = [vp, vp, sz, vp]
    L.rpa_kv_append.argtypes = [vp, vp, vp, vp, vp, P(rpa_cache_strides), P(rpa_cache_strides), vp]
    L.rpa_batch_attention.argtypes = [vp, vp, vp, vp, P(rpa_cache_strides),
                                      P(rpa_cache_strides), vp, vp, vp]
    L.rpa_batch_attention_noalloc.argtypes = [vp, vp, vp, vp, P(rpa_cache_strides),
                                              P(rpa_cache_strides), vp, vp, vp]
    L.rpa_split_attention.argtypes = [vp, vp, vp, vp, vp, vp, P(rpa_cache_strides),
                                      P(rpa_cache_strides), vp, vp, vp]
    L.rpa_merge_state.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, vp]
    L.rpa_page_copy.argtypes = [vp, P(rpa_cache_strides), i32, i32, vp, vp,
                                P(rpa_cache_strides), i32, i32, vp, i32, i32, i32, i32, i32, i32,
                                i32, vp]
    L.rpa_plan_destroy.argtypes = [vp]
    L.rpa_plan_destroy.restype = None
    L.rpa_status_string.argtypes = [i32]
    L.rpa_status_string.restype = ctypes.c_char_p
    L.rpa_last_error_message.argtypes = []
    L.rpa_last_error_message.restype = ctypes.c_char_p
    L.rpa_abi_version.argtypes = []
    L.rpa_abi_version.restype = i32
    L.rpa_plan_debug_dump.argtypes = [vp, ctypes.c_char_p, P(i32), i64, P(i64)]
    L.rpa_profile_enable.argtypes = [i32]
    L.rpa_profile_read.argtypes = [ctypes.c_char_p, P(ctypes.c_double), P(i64)]
    L.rpa_profile_reset.argtypes = []
    L.rpa_profile_select.argtypes = [ctypes.c_char_p]
    for name in ("rpa_plan_create", "rpa_plan_create_tree", "rpa_plan_create_split",
                 "rpa_plan_workspace_size", "rpa_plan_upload", "rpa_kv_append",
                 "rpa_batch_attention", "rpa_batch_attention_noalloc", "rpa_split_attention",
                 "rpa_merge_state",
                 "rpa_page_copy", "rpa_plan_debug_dump", "rpa_profile_enable",
                 "rpa_profile_read", "rpa_profile_reset", "rpa_profile_select"):
        getattr(L, name).restype = i32
    _lib_handle = L
    return L


def _check(status: int):
    if status != RPA_OK:
        L = lib()
        msg = L.rpa_last_error_message().decode()
        name = L.rpa_status_string(status).decode()
        raise RpaError(status, f"{name}: {msg}")


def _ptr(x) -> Optional[int]:
    """Device/host address of a tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def make_config(num_qo_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size, dtype, causal=True,
                sm_scale=None) -> rpa_attn_config:
    if isinstance(dtype, str):
        dtype = {"bf16": RPA_DTYPE_BF16, "f32": RPA_DTYPE_F32}[dtype]
    if sm_scale is None:
        sm_scale = head_dim_qk ** -0.5
    return rpa_attn_config(num_qo_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size, dtype,
                           1 if causal else 0, float(sm_scale))


def strides_of(pool) -> rpa_cache_strides:
    """Strides (elements) of a 4-D pool tensor [pages, heads, page_size, dim]."""
    st = pool.stride()
    if st[3] != 1:
        raise RpaError(RPA_ERR_INVALID_ARG, "pool's last dimension must be contiguous")
    return rpa_cache_strides(st[0], st[1], st[2])


# ----------------------------------------------------------------------------
# C-named entry points
# ----------------------------------------------------------------------------


class _PlanHandle:
    def __init__(self, handle: int, arrays):
        self.handle = handle
        self._arrays = arrays

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                lib().rpa_plan_destroy(h)
            except Exception:
                pass
            self.handle = None


def rpa_plan_create(cfg: rpa_attn_config, qo_indptr, kv_len, kv_page_indptr, kv_page_indices,
                    num_pages: int, num_cus: int = 0) -> _PlanHandle:
    """Host-only planning (no device work).  Returns a plan handle."""
    L = lib()
    arrays = [_i32(qo_indptr), _i32(kv_len), _i32(kv_page_indptr), _i32(kv_page_indices)]
    batch = rpa_batch_desc(len(arrays[1]), _i32p(arrays[0]), _i32p(arrays[1]), _i32p(arrays[2]),
                           _i32p(arrays[3]), int(num_pages))
    out = ctypes.c_void_p()
    _check(L.rpa_plan_create(ctypes.byref(cfg), ctypes.byref(batch), int(num_cus),
                             ctypes.byref(out)))
    return _PlanHandle(out.value, arrays)


def rpa_plan_create_tree(cfg: rpa_attn_config, qo_indptr, kv_len, kv_page_indptr,
                         kv_page_indices, num_pages: int, tree_indptr, tree_words,
                         num_cus: int = 0) -> _PlanHandle:
    """rpa_plan_create with per-request tree masks among the new tokens."""
    L = lib()
    arrays = [_i32(qo_indptr), _i32(kv_len), _i32(kv_page_indptr), _i32(kv_page_indices)]
    ti = _i32(tree_indptr)
    tw = np.ascontiguousarray(np.asarray(tree_words, dtype=np.uint32))
    if tw.size == 0:
        tw = np.zeros(1, dtype=np.uint32)
    batch = rpa_batch_desc(len(arrays[1]), _i32p(arrays[0]), _i32p(arrays[1]), _i32p(arrays[2]),
                           _i32p(arrays[3]), int(num_pages))
    out = ctypes.c_void_p()
    _check(L.rpa_plan_create_tree(ctypes.byref(cfg), ctypes.byref(batch), _i32p(ti),
                                  tw.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                  int(num_cus), ctypes.byref(out)))
    return _PlanHandle(out.value, arrays + [ti, tw])


def rpa_plan_create_split(cfg: rpa_attn_config, qo_indptr, kv_len, kv_page_indptr,
                          kv_page_indices, num_pages: int, num_cus: int = 0) -> _PlanHandle:
    """Host-only planning of a causal step's split execution."""
    L = lib()
    arrays = [_i32(qo_indptr), _i32(kv_len), _i32(kv_page_indptr), _i32(kv_page_indices)]
    batch = rpa_batch_desc(len(arrays[1]), _i32p(arrays[0]), _i32p(arrays[1]), _i32p(arrays[2]),
                           _i32p(arrays[3]), int(num_pages))
    out = ctypes.c_void_p()
    _check(L.rpa_plan_create_split(ctypes.byref(cfg), ctypes.byref(batch), int(num_cus),
                                   ctypes.byref(out)))
    return _PlanHandle(out.value, arrays)


def tree_mask_words(masks) -> tuple[np.ndarray, np.ndarray]:
    """Pack per-request boolean masks ([n_r, n_r] arrays, or None for no mask)
    into (tree_indptr, tree_words) for rpa_plan_create_tree: row t of a
    request is ceil(n_r/32) words, bit u set iff new token t sees new token u."""
    indptr = [0]
    words = []
    for m in masks:
        if m is None:
            indptr.append(indptr[-1])
            continue
        m = np.asarray(m, dtype=bool)
        n = m.shape[0]
        wpr = (n + 31) // 32
        for t in range(n):
            row = [0] * wpr
            for u in np.nonzero(m[t])[0]:
                row[int(u) // 32] |= 1 << (int(u) % 32)
            words.extend(row)
        indptr.append(indptr[-1] + n * wpr)
    return np.array(indptr, dtype=np.int32), np.array(words, dtype=np.uint32)


def rpa_plan_workspace_size(plan: _PlanHandle) -> int:
    n = ctypes.c_size_t()
    _check(lib().rpa_plan_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def rpa_plan_upload(plan: _PlanHandle, workspace, nbytes: int, stream=None):
    _check(lib().rpa_plan_upload(plan.handle, _ptr(workspace), int(nbytes), _stream(stream)))


def rpa_kv_append(plan: _PlanHandle, k_new, v_new, k_cache, v_cache, ks: rpa_cache_strides,
                  vs: Optional[rpa_cache_strides], stream=None):
    _check(lib().rpa_kv_append(plan.handle, _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                               _ptr(v_cache), ctypes.byref(ks),
                               None if vs is None else ctypes.byref(vs), _stream(stream)))


def rpa_batch_attention(plan: _PlanHandle, q, k_cache, v_cache, ks: rpa_cache_strides,
                        vs: Optional[rpa_cache_strides], o, lse=None, stream=None):
    _check(lib().rpa_batch_attention(plan.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     ctypes.byref(ks), None if vs is None else ctypes.byref(vs),
                                     _ptr(o), _ptr(lse), _stream(stream)))


def rpa_split_attention(plan: _PlanHandle, q, k_new, v_new, k_cache, v_cache,
                        ks: rpa_cache_strides, vs: rpa_cache_strides, o, lse=None, stream=None):
    _check(lib().rpa_split_attention(plan.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(k_cache), _ptr(v_cache), ctypes.byref(ks),
                                     ctypes.byref(vs), _ptr(o), _ptr(lse), _stream(stream)))


def rpa_batch_attention_noalloc(plan: _PlanHandle, q, k_cache, v_cache, ks: rpa_cache_strides,
                                vs: Optional[rpa_cache_strides], o, lse=None, stream=None):
    """rpa_batch_attention with the plan's metadata and partials in the
    library's static device scratch (no workspace, no allocation)."""
    _check(lib().rpa_batch_attention_noalloc(plan.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             ctypes.byref(ks),
                                             None if vs is None else ctypes.byref(vs), _ptr(o),
                                             _ptr(lse), _stream(stream)))


def rpa_merge_state(o_a, lse_a, o_b, lse_b, o, lse, rows: int, heads: int, dim: int, dtype: int,
                    stream=None):
    _check(lib().rpa_merge_state(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o),
                                 _ptr(lse), int(rows), int(heads), int(dim), int(dtype),
                                 _stream(stream)))


def rpa_page_copy(src, src_strides: rpa_cache_strides, src_pool_pages: int, src_pool_heads: int,
                  src_pages, dst, dst_strides: rpa_cache_strides, dst_pool_pages: int,
                  dst_pool_heads: int, dst_pages, num_pages: int, src_head0: int, dst_head0: int,
                  num_heads: int, page_size: int, dim: int, dtype: int, stream=None):
    """Raw copy of head ranges of pages (page id arrays are device tensors or None)."""
    _check(lib().rpa_page_copy(_ptr(src), ctypes.byref(src_strides), int(src_pool_pages),
                               int(src_pool_heads), _ptr(src_pages), _ptr(dst),
                               ctypes.byref(dst_strides), int(dst_pool_pages),
                               int(dst_pool_heads), _ptr(dst_pages), int(num_pages),
                               int(src_head0), int(dst_head0), int(num_heads), int(page_size),
                               int(dim), int(dtype), _stream(stream)))


def copy_pages(src, dst, src_pages=None, dst_pages=None, src_head0=0, dst_head0=0,
               num_heads=None, stream=None):
    """Copy head ranges of pages between two 4-D views [pages, heads, slots, dim]
    (any strides, e.g. an HND pool, or an NHD buffer permuted to that order).
    Page id lists are device int32 tensors (or None for 0, 1, ...); pairs with
    an id outside either view's page count are skipped by the kernel."""
    import torch
    _require(src.dim() == 4 and dst.dim() == 4, "src and dst must be 4-D [pages, heads, slots, dim]")
    _require(src.dtype == dst.dtype and src.dtype in (torch.bfloat16, torch.float32),
             "src and dst must share a dtype (bfloat16 or float32)")
    _require(src.shape[2] == dst.shape[2] and src.shape[3] == dst.shape[3],
             "src and dst must have the same page size and row length")
    _require(src.is_cuda and dst.is_cuda and src.device == dst.device,
             "src and dst must be on the same GPU")
    for ids, name in ((src_pages, "src_pages"), (dst_pages, "dst_pages")):
        if ids is not None:
            _require(ids.dtype == torch.int32 and ids.dim() == 1 and ids.is_contiguous()
                     and ids.device == src.device, f"{name} must be a contiguous int32 vector "
                     "on the pools' GPU")
    n = int(src_pages.numel()) if src_pages is not None else (
        int(dst_pages.numel()) if dst_pages is not None else int(src.shape[0]))
    if src_pages is not None and dst_pages is not None:
        _require(src_pages.numel() == dst_pages.numel(), "page lists differ in length")
    heads = int(num_heads if num_heads is not None else src.shape[1] - src_head0)
    dtype = RPA_DTYPE_BF16 if src.dtype == torch.bfloat16 else RPA_DTYPE_F32
    rpa_page_copy(src, strides_of(src), int(src.shape[0]), int(src.shape[1]), src_pages, dst,
                  strides_of(dst), int(dst.shape[0]), int(dst.shape[1]), dst_pages, n, src_head0,
                  dst_head0, heads, int(src.shape[2]), int(src.shape[3]), dtype, stream)


def rpa_plan_destroy(plan: _PlanHandle):
    if plan.handle:
        lib().rpa_plan_destroy(plan.handle)
        plan.handle = None


def rpa_status_string(status: int) -> str:
    return lib().rpa_status_string(int(status)).decode()


def rpa_last_error_message() -> str:
    return lib().rpa_last_error_message().decode()


def rpa_abi_version() -> int:
    return int(lib().rpa_abi_version())


def rpa_plan_debug_dump(plan: _PlanHandle, name: str) -> np.ndarray:
    L = lib()
    n = ctypes.c_int64()
    _check(L.rpa_plan_debug_dump(plan.handle, name.encode(), None, 0, ctypes.byref(n)))
    out = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(L.rpa_plan_debug_dump(plan.handle, name.encode(), _i32p(out), n.value,
                                 ctypes.byref(n)))
    return out[:n.value]


def rpa_profile_enable(on: bool = True):
    _check(lib().rpa_profile_enable(1 if on else 0))


def rpa_profile_read(kernel: str) -> tuple[float, int]:
    """(total milliseconds, launches) of one kernel since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().rpa_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def rpa_profile_reset():
    _check(lib().rpa_profile_reset())


def rpa_profile_select(kernels=None):
    """Times only the named kernels (a list of names, or None for all)."""
    _check(lib().rpa_profile_select(",".join(kernels).encode() if kernels else None))


# ----------------------------------------------------------------------------
# Host-side tensor checks (the C ABI sees raw addresses only, so a tensor of
# the wrong dtype, shape or size would become an out-of-bounds device access)
# ----------------------------------------------------------------------------


def _require(cond: bool, msg: str):
    if not cond:
        raise RpaError(RPA_ERR_INVALID_ARG, f"RPA_ERR_INVALID_ARG: {msg}")


def _torch_dtype(cfg: rpa_attn_config):
    import torch
    return torch.bfloat16 if cfg.dtype == RPA_DTYPE_BF16 else torch.float32


def _check_rows(name, t, shape, dtype, device=None):
    """A contiguous tensor of exactly `shape` and `dtype` (on `device` if given)."""
    _require(t is not None, f"{name} is required")
    _require(t.dtype == dtype, f"{name} has dtype {t.dtype}, the plan needs {dtype}")
    _require(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, "
             f"the plan needs {tuple(shape)}")
    _require(t.is_contiguous(), f"{name} must be contiguous")
    if device is not None:
        _require(t.device == device, f"{name} is on {t.device}, not {device}")


def _check_pool(name, pool, cfg: rpa_attn_config, num_pages: int, row_len: int, device=None):
    """A 4-D pool view [pages >= num_pages, H_kv, page_size, >= row_len] of the
    plan's dtype with a contiguous last dimension."""
    _require(pool is not None, f"{name} is required")
    _require(pool.dtype == _torch_dtype(cfg), f"{name} has dtype {pool.dtype}, "
             f"the plan needs {_torch_dtype(cfg)}")
    _require(pool.dim() == 4, f"{name} must be 4-D [pages, heads, page_size, dim]")
    _require(pool.shape[0] >= num_pages, f"{name} holds {pool.shape[0]} pages, the plan's page "
             f"ids reach {num_pages}")
    _require(pool.shape[1] == cfg.num_kv_heads and pool.shape[2] == cfg.page_size,
             f"{name} has {pool.shape[1]} heads of {pool.shape[2]} slots, the plan needs "
             f"{cfg.num_kv_heads} of {cfg.page_size}")
    _require(pool.shape[3] >= row_len, f"{name} rows hold {pool.shape[3]} elements, "
             f"the plan needs {row_len}")
    _require(pool.stride(3) == 1, f"{name}'s last dimension must be contiguous")
    if device is not None:
        _require(pool.device == device, f"{name} is on {pool.device}, not {device}")


def check_append_args(cfg: rpa_attn_config, total_q: int, num_pages: int, k_new, v_new, k_cache,
                      v_cache):
    """Raises RpaError(INVALID_ARG) unless the tensors fit the plan's append."""
    latent = cfg.head_dim_qk == 576
    dt = _torch_dtype(cfg)
    _check_rows("k_new", k_new, (total_q, cfg.num_kv_heads, cfg.head_dim_qk), dt)
    _check_pool("k_cache", k_cache, cfg, num_pages, cfg.head_dim_qk)
    if latent:
        _require(v_new is None, "the shared latent cache takes no v_new")
        _require(v_cache is None or v_cache is k_cache, "the shared latent cache takes no "
                 "v_cache (or v_cache = k_cache)")
    else:
        _check_rows("v_new", v_new, (total_q, cfg.num_kv_heads, cfg.head_dim_v), dt)
        _check_pool("v_cache", v_cache, cfg, num_pages, cfg.head_dim_v)
    dev = k_new.device
    _require(dev.type == "cuda", f"k_new is on {dev}, not a GPU")
    for name, t in (("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t is not None:
            _require(t.device == dev, f"{name} is on {t.device}, not {dev}")


def check_attention_args(cfg: rpa_attn_config, total_q: int, num_pages: int, q, k_cache,
                         v_cache, o, lse):
    """Raises RpaError(INVALID_ARG) unless the tensors fit the plan's attention."""
    import torch
    latent = cfg.head_dim_qk == 576
    dt = _torch_dtype(cfg)
    _check_rows("q", q, (total_q, cfg.num_qo_heads, cfg.head_dim_qk), dt)
    _check_rows("o", o, (total_q, cfg.num_qo_heads, cfg.head_dim_v), dt)
    if lse is not None:
        _check_rows("lse", lse, (total_q, cfg.num_qo_heads), torch.float32)
    _check_pool("k_cache", k_cache, cfg, num_pages, cfg.head_dim_qk)
    if latent:
        _require(v_cache is None or v_cache is k_cache, "the shared latent cache takes no "
                 "v_cache (or v_cache = k_cache)")
    else:
        _check_pool("v_cache", v_cache, cfg, num_pages, cfg.head_dim_v)
    dev = q.device
    _require(dev.type == "cuda", f"q is on {dev}, not a GPU")
    for name, t in (("o", o), ("lse", lse), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t is not None:
            _require(t.device == dev, f"{name} is on {t.device}, not {dev}")


# ----------------------------------------------------------------------------
# Convenience wrapper
# ----------------------------------------------------------------------------


class Plan:
    """A plan plus its device workspace (a torch uint8 tensor on ``device``)."""

    def __init__(self, cfg: rpa_attn_config, qo_indptr, kv_len, kv_page_indptr, kv_page_indices,
                 num_pages: int, device="cuda", num_cus: int = 0, stream=None, tree_masks=None):
        """tree_masks: optional list with one [n_r, n_r] boolean array (or None)
        per request; see rpa_plan_create_tree."""
        import torch
        self.cfg = cfg
        if tree_masks is None:
            self.handle = rpa_plan_create(cfg, qo_indptr, kv_len, kv_page_indptr,
                                          kv_page_indices, num_pages, num_cus)
        else:
            ti, tw = tree_mask_words(tree_masks)
            self.handle = rpa_plan_create_tree(cfg, qo_indptr, kv_len, kv_page_indptr,
                                               kv_page_indices, num_pages, ti, tw, num_cus)
        self.total_q = int(np.asarray(qo_indptr)[-1]) if len(qo_indptr) else 0
        self.num_pages = int(num_pages)
        self.ws_bytes = rpa_plan_workspace_size(self.handle)
        self.workspace = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256
        rpa_plan_upload(self.handle, self.ws_ptr, self.ws_bytes, stream)

    @property
    def shared_latent(self) -> bool:
        return self.cfg.head_dim_qk == 576

    def append(self, k_new, v_new, k_cache, v_cache=None, stream=None):
        check_append_args(self.cfg, self.total_q, self.num_pages, k_new, v_new, k_cache, v_cache)
        ks = strides_of(k_cache)
        vs = None if v_cache is None else strides_of(v_cache)
        rpa_kv_append(self.handle, k_new, v_new, k_cache, v_cache, ks, vs, stream)

    def attention(self, q, k_cache, v_cache=None, o=None, lse=None, with_lse=True, stream=None):
        import torch
        if o is None:
            o = torch.empty((self.total_q, self.cfg.num_qo_heads, self.cfg.head_dim_v),
                            dtype=q.dtype, device=q.device)
        if lse is None and with_lse:
            lse = torch.empty((self.total_q, self.cfg.num_qo_heads), dtype=torch.float32,
                              device=q.device)
        check_attention_args(self.cfg, self.total_q, self.num_pages, q, k_cache, v_cache, o, lse)
        ks = strides_of(k_cache)
        vs = None if v_cache is None else strides_of(v_cache)
        rpa_batch_attention(self.handle, q, k_cache, v_cache, ks, vs, o, lse, stream)
        return o, lse

    def debug(self, name: str) -> np.ndarray:
        return rpa_plan_debug_dump(self.handle, name)


def merge_state(o_a, lse_a, o_b, lse_b, stream=None):
    """Merge two attention states [rows, heads, dim] (torch tensors on the GPU)."""
    import torch
    _require(o_a.dim() == 3, "o_a must be [rows, heads, dim]")
    rows, heads, dim = o_a.shape
    _require(o_a.dtype in (torch.bfloat16, torch.float32), "o dtype must be bfloat16 or float32")
    _check_rows("o_a", o_a, (rows, heads, dim), o_a.dtype, o_a.device)
    _check_rows("o_b", o_b, (rows, heads, dim), o_a.dtype, o_a.device)
    _check_rows("lse_a", lse_a, (rows, heads), torch.float32, o_a.device)
    _check_rows("lse_b", lse_b, (rows, heads), torch.float32, o_a.device)
    _require(o_a.is_cuda, "merge_state runs on the GPU")
    o = torch.empty_like(o_a)
    lse = torch.empty_like(lse_a)
    dtype = RPA_DTYPE_BF16 if o_a.dtype == torch.bfloat16 else RPA_DTYPE_F32
    rpa_merge_state(o_a, lse_a, o_b, lse_b, o, lse, rows, heads, dim, dtype, stream)
    return o, lse


class SplitChunkAttention:
    """Split execution of a causal step's attention ("Chunked prefill",
    section "correctness"): the new tokens of each request attend

      (a) to the request's c_r = kv_len - qo_len cached keys in the pages,
          every new token seeing all of them, and
      (b) causally to the step's own keys and values, read from the k_new /
          v_new buffers (token-major [total_q, num_kv_heads, d]),

    and the two states are merged, all inside rpa_split_attention (one
    launch per kernel class and part, then one merge, whatever the batch
    size).  The result equals the attention over the pages after
    rpa_kv_append, and the append may run before, after or beside it.  Not
    for the shared-latent form.  This class only holds the plan and its
    workspace and marshals the call.
    """

    def __init__(self, cfg: rpa_attn_config, qo_indptr, kv_len, kv_page_indptr, kv_page_indices,
                 num_pages: int, device="cuda", num_cus: int = 0, stream=None):
        import torch
        self.cfg = cfg
        self.handle = rpa_plan_create_split(cfg, qo_indptr, kv_len, kv_page_indptr,
                                            kv_page_indices, num_pages, num_cus)
        self.total_q = int(np.asarray(qo_indptr)[-1]) if len(qo_indptr) else 0
        self.num_pages = int(num_pages)
        self.ws_bytes = rpa_plan_workspace_size(self.handle)
        self.workspace = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        self.ws_ptr = (self.workspace.data_ptr() + 255) // 256 * 256
        rpa_plan_upload(self.handle, self.ws_ptr, self.ws_bytes, stream)

    def append(self, k_new, v_new, k_cache, v_cache, stream=None):
        check_append_args(self.cfg, self.total_q, self.num_pages, k_new, v_new, k_cache, v_cache)
        rpa_kv_append(self.handle, k_new, v_new, k_cache, v_cache, strides_of(k_cache),
                      strides_of(v_cache), stream)

    def run(self, q, k_new, v_new, k_cache, v_cache, o=None, lse=None, stream=None):
        """o, lse of the step (o in q's dtype, lse float32, natural log)."""
        import torch
        H, d_v = self.cfg.num_qo_heads, self.cfg.head_dim_v
        if o is None:
            o = torch.empty((self.total_q, H, d_v), dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty((self.total_q, H), dtype=torch.float32, device=q.device)
        check_attention_args(self.cfg, self.total_q, self.num_pages, q, k_cache, v_cache, o, lse)
        cfg = self.cfg
        _check_rows("k_new", k_new, (self.total_q, cfg.num_kv_heads, cfg.head_dim_qk), q.dtype,
                    q.device)
        _check_rows("v_new", v_new, (self.total_q, cfg.num_kv_heads, cfg.head_dim_v), q.dtype,
                    q.device)
        rpa_split_attention(self.handle, q, k_new, v_new, k_cache, v_cache, strides_of(k_cache),
                            strides_of(v_cache), o, lse, stream)
        return o, lse

    def debug(self, name: str) -> np.ndarray:
        return rpa_plan_debug_dump(self.handle, name)
