"""ctypes binding of libpa (include/pa.h), with the same names as the C entry points.

Argument marshalling only: every step of attention runs in libpa's HIP kernels.  If the
library is not built, loading fails with an error; there is no fallback path.
"""

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint64,
                    c_uint8, c_void_p)

import numpy as np

# The built library in the package; PA_LIBRARY may name another build of it (the CPU
# tests load a host-sanitized build that way).
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARG = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_WORKSPACE_TOO_SMALL = 3
PA_ERR_HIP = 4

PA_DTYPE_BF16 = 0
PA_DTYPE_FP32 = 1
PA_DTYPE_FP8_E4M3FN = 2
PA_DTYPE_NVFP4 = 3

_STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED",
                 3: "PA_ERR_WORKSPACE_TOO_SMALL", 4: "PA_ERR_HIP"}


class PaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class pa_kv_cache(Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("kv_dtype", c_int32), ("num_pages", c_int32),
                ("num_kv_heads", c_int32), ("page_size", c_int32), ("head_dim_qk", c_int32),
                ("head_dim_vo", c_int32), ("k_stride_page", c_int64), ("k_stride_head", c_int64),
                ("k_stride_token", c_int64), ("v_stride_page", c_int64),
                ("v_stride_head", c_int64), ("v_stride_token", c_int64), ("k_scale", c_float),
                ("v_scale", c_float), ("k_sf", c_void_p), ("v_sf", c_void_p),
                ("k_sf_stride_page", c_int64), ("k_sf_stride_head", c_int64),
                ("k_sf_stride_token", c_int64), ("v_sf_stride_page", c_int64),
                ("v_sf_stride_head", c_int64), ("v_sf_stride_token", c_int64)]


class pa_page_table(Structure):
    _fields_ = [("kv_indptr", c_void_p), ("kv_indices", c_void_p),
                ("kv_last_page_len", c_void_p), ("batch", c_int32)]


class pa_attn_params(Structure):
    _fields_ = [("num_qo_heads", c_int32), ("sm_scale", c_float), ("window", c_int32),
                ("causal", c_int32), ("q_dtype", c_int32), ("out_dtype", c_int32)]


class pa_plan(Structure):
    _fields_ = [("kind", c_int32), ("batch", c_int32), ("num_qo_heads", c_int32),
                ("num_kv_heads", c_int32), ("page_size", c_int32), ("head_dim_qk", c_int32),
                ("head_dim_vo", c_int32), ("kv_dtype", c_int32), ("window", c_int32),
                ("causal", c_int32), ("num_items", c_int32), ("num_slots", c_int32),
                ("num_merges", c_int32), ("block_tokens", c_int32), ("chunk_blocks", c_int32),
                ("num_splits", c_int32), ("tile_rows", c_int32), ("total_q", c_int32),
                ("max_kv_len", c_int32), ("num_workers", c_int32),
                ("deferred_partials", c_int32), ("short_tiles", c_int32),
                ("grouped_partials", c_int32), ("staged_pages", c_int32),
                ("plan_bytes", c_int64),
                ("items_offset", c_int64), ("merges_offset", c_int64),
                ("workers_offset", c_int64),
                ("partial_o_offset", c_int64), ("partial_lse_offset", c_int64),
                ("workspace_bytes", c_int64), ("staged_offset", c_int64)]


# Every symbol include/pa.h declares, with (restype, argtypes).
_P = c_void_p
_I32P = POINTER(c_int32)
SIGNATURES = {
    "pa_kv_cache_hnd": (c_int32, [_P, c_int32, c_int32, c_int32, c_int32, c_int32, c_float,
                                  c_float, POINTER(pa_kv_cache)]),
    "pa_kv_cache_separate": (c_int32, [_P, _P, c_int32, c_int32, c_int32, c_int32, c_int32,
                                       c_int32, c_float, c_float, POINTER(pa_kv_cache)]),
    "pa_kv_cache_nvfp4_hnd": (c_int32, [_P, _P, c_int32, c_int32, c_int32, c_int32, c_float,
                                        c_float, POINTER(pa_kv_cache)]),
    "pa_kv_cache_nvfp4_separate": (c_int32, [_P, _P, _P, _P, c_int32, c_int32, c_int32, c_int32,
                                             c_int32, c_float, c_float, POINTER(pa_kv_cache)]),
    "pa_validate_page_table_host": (c_int32, [_I32P, _I32P, _I32P, c_int32, c_int32, c_int32]),
    "pa_decode_plan": (c_int32, [POINTER(pa_attn_params), POINTER(pa_kv_cache), _I32P, _I32P,
                                 c_int32, c_int32, _P, c_size_t, POINTER(pa_plan)]),
    "pa_prefill_plan": (c_int32, [POINTER(pa_attn_params), POINTER(pa_kv_cache), _I32P, _I32P,
                                  _I32P, c_int32, _P, c_size_t, POINTER(pa_plan)]),
    "pa_plan_upload": (c_int32, [POINTER(pa_plan), _P, _P, c_size_t, _P]),
    "pa_paged_decode": (c_int32, [POINTER(pa_plan), _P, POINTER(pa_kv_cache),
                                  POINTER(pa_page_table), POINTER(pa_attn_params), _P, _P, _P,
                                  c_size_t, _P]),
    "pa_paged_decode_partial": (c_int32, [POINTER(pa_plan), _P, POINTER(pa_kv_cache),
                                          POINTER(pa_page_table), POINTER(pa_attn_params), _P,
                                          _P, _P, c_size_t, _P]),
    "pa_paged_decode_merge": (c_int32, [POINTER(pa_plan), _P, POINTER(pa_kv_cache),
                                        POINTER(pa_page_table), POINTER(pa_attn_params), _P, _P,
                                        _P, c_size_t, _P]),
    "pa_paged_decode_static": (c_int32, [POINTER(pa_plan), _P, _P, POINTER(pa_kv_cache),
                                         POINTER(pa_page_table), POINTER(pa_attn_params), _P,
                                         _P, _P]),
    "pa_paged_prefill": (c_int32, [POINTER(pa_plan), _P, _P, POINTER(pa_kv_cache),
                                   POINTER(pa_page_table), POINTER(pa_attn_params), _P, _P, _P,
                                   c_size_t, _P]),
    "pa_debug_gather_kv": (c_int32, [POINTER(pa_kv_cache), POINTER(pa_page_table), c_int32,
                                     c_int32, c_int32, _P, _P, _P]),
    "pa_debug_fp8_to_f32": (c_int32, [_P, _P, c_int32, _P]),
    "pa_last_error": (c_char_p, []),
    "pa_launch_count": (c_uint64, []),
    "pa_debug_launch_count": (c_uint64, []),
    "pa_version": (c_char_p, []),
}

_lib = None


def lib():
    """The loaded libpa; raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_attention_hd512_amd.build` (or "
                               "__graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status):
    if status != PA_OK:
        raise PaError(status, pa_last_error())


def _i32(arr):
    if arr is None:
        return None, None
    a = np.ascontiguousarray(arr, dtype=np.int32)
    return a, a.ctypes.data_as(_I32P)


def pa_last_error():
    return lib().pa_last_error().decode()


def pa_launch_count():
    return int(lib().pa_launch_count())


def pa_debug_launch_count():
    return int(lib().pa_debug_launch_count())


def pa_version():
    return lib().pa_version().decode()


def pa_kv_cache_hnd(base, kv_dtype, num_pages, num_kv_heads, page_size, head_dim, k_scale=1.0,
                    v_scale=1.0):
    c = pa_kv_cache()
    _check(lib().pa_kv_cache_hnd(base, kv_dtype, num_pages, num_kv_heads, page_size, head_dim,
                                 k_scale, v_scale, ctypes.byref(c)))
    return c


def pa_kv_cache_separate(k, v, kv_dtype, num_pages, num_kv_heads, page_size, head_dim_qk,
                         head_dim_vo, k_scale=1.0, v_scale=1.0):
    c = pa_kv_cache()
    _check(lib().pa_kv_cache_separate(k, v, kv_dtype, num_pages, num_kv_heads, page_size,
                                      head_dim_qk, head_dim_vo, k_scale, v_scale,
                                      ctypes.byref(c)))
    return c


def pa_kv_cache_nvfp4_hnd(data, sf, num_pages, num_kv_heads, page_size, head_dim, k_scale=1.0,
                          v_scale=1.0):
    c = pa_kv_cache()
    _check(lib().pa_kv_cache_nvfp4_hnd(data, sf, num_pages, num_kv_heads, page_size, head_dim,
                                       k_scale, v_scale, ctypes.byref(c)))
    return c


def pa_kv_cache_nvfp4_separate(k, v, k_sf, v_sf, num_pages, num_kv_heads, page_size,
                               head_dim_qk, head_dim_vo, k_scale=1.0, v_scale=1.0):
    c = pa_kv_cache()
    _check(lib().pa_kv_cache_nvfp4_separate(k, v, k_sf, v_sf, num_pages, num_kv_heads,
                                            page_size, head_dim_qk, head_dim_vo, k_scale,
                                            v_scale, ctypes.byref(c)))
    return c


def pa_validate_page_table_host(kv_indptr, kv_indices, kv_last_page_len, num_pages, page_size):
    ip, ipp = _i32(kv_indptr)
    ix, ixp = _i32(kv_indices)
    la, lap = _i32(kv_last_page_len)
    _check(lib().pa_validate_page_table_host(ipp, ixp, lap, len(ip) - 1, num_pages, page_size))


def pa_decode_plan(params, cache, kv_indptr_host, kv_last_page_len_host, num_splits):
    """Returns (plan, plan_buf) where plan_buf is the host work list (numpy uint8)."""
    ip, ipp = _i32(kv_indptr_host)
    la, lap = _i32(kv_last_page_len_host)
    batch = len(ip) - 1
    plan = pa_plan()
    _check(lib().pa_decode_plan(ctypes.byref(params), ctypes.byref(cache), ipp, lap, batch,
                                num_splits, None, 0, ctypes.byref(plan)))
    buf = np.zeros(max(1, plan.plan_bytes), dtype=np.uint8)
    _check(lib().pa_decode_plan(ctypes.byref(params), ctypes.byref(cache), ipp, lap, batch,
                                num_splits, buf.ctypes.data_as(c_void_p), buf.nbytes,
                                ctypes.byref(plan)))
    return plan, buf


def pa_prefill_plan(params, cache, qo_indptr_host, kv_indptr_host, kv_last_page_len_host):
    qp, qpp = _i32(qo_indptr_host)
    ip, ipp = _i32(kv_indptr_host)
    la, lap = _i32(kv_last_page_len_host)
    batch = len(ip) - 1
    plan = pa_plan()
    _check(lib().pa_prefill_plan(ctypes.byref(params), ctypes.byref(cache), qpp, ipp, lap,
                                 batch, None, 0, ctypes.byref(plan)))
    buf = np.zeros(max(1, plan.plan_bytes), dtype=np.uint8)
    _check(lib().pa_prefill_plan(ctypes.byref(params), ctypes.byref(cache), qpp, ipp, lap,
                                 batch, buf.ctypes.data_as(c_void_p), buf.nbytes,
                                 ctypes.byref(plan)))
    return plan, buf


def pa_plan_upload(plan, plan_buf, workspace, workspace_bytes, stream=None):
    _check(lib().pa_plan_upload(ctypes.byref(plan), plan_buf.ctypes.data_as(c_void_p), workspace,
                                workspace_bytes, stream))


def pa_paged_decode(plan, q, cache, table, params, out, lse, workspace, workspace_bytes,
                    stream=None):
    _check(lib().pa_paged_decode(ctypes.byref(plan), q, ctypes.byref(cache), ctypes.byref(table),
                                 ctypes.byref(params), out, lse, workspace, workspace_bytes,
                                 stream))


def pa_paged_decode_static(plan, plan_buf, q, cache, table, params, out, lse, stream=None):
    """pa_paged_decode with the library's own workspace; plan_buf is the host plan buffer."""
    _check(lib().pa_paged_decode_static(ctypes.byref(plan), plan_buf.ctypes.data_as(c_void_p),
                                        q, ctypes.byref(cache), ctypes.byref(table),
                                        ctypes.byref(params), out, lse, stream))


def pa_paged_decode_partial(plan, q, cache, table, params, out, lse, workspace,
                            workspace_bytes, stream=None):
    _check(lib().pa_paged_decode_partial(ctypes.byref(plan), q, ctypes.byref(cache),
                                         ctypes.byref(table), ctypes.byref(params), out, lse,
                                         workspace, workspace_bytes, stream))


def pa_paged_decode_merge(plan, q, cache, table, params, out, lse, workspace, workspace_bytes,
                          stream=None):
    _check(lib().pa_paged_decode_merge(ctypes.byref(plan), q, ctypes.byref(cache),
                                       ctypes.byref(table), ctypes.byref(params), out, lse,
                                       workspace, workspace_bytes, stream))


def pa_paged_prefill(plan, q, qo_indptr, cache, table, params, out, lse, workspace,
                     workspace_bytes, stream=None):
    _check(lib().pa_paged_prefill(ctypes.byref(plan), q, qo_indptr, ctypes.byref(cache),
                                  ctypes.byref(table), ctypes.byref(params), out, lse, workspace,
                                  workspace_bytes, stream))


def pa_debug_gather_kv(cache, table, request, kv_len, kv_head, k_out, v_out, stream=None):
    _check(lib().pa_debug_gather_kv(ctypes.byref(cache), ctypes.byref(table), request, kv_len,
                                    kv_head, k_out, v_out, stream))


def pa_debug_fp8_to_f32(codes, out, n, stream=None):
    _check(lib().pa_debug_fp8_to_f32(codes, out, n, stream))


# ----------------------------------------------------------------------------- torch helpers
# PyTorch supplies device memory and the stream; these classes only marshal pointers.

def _torch():
    import torch
    return torch


def kv_dtype_code(kv_dtype):
    return {"bf16": PA_DTYPE_BF16, "fp8": PA_DTYPE_FP8_E4M3FN, "nvfp4": PA_DTYPE_NVFP4}[kv_dtype]


def out_dtype_code(out_dtype):
    return {"bf16": PA_DTYPE_BF16, "fp32": PA_DTYPE_FP32}[out_dtype]


def cache_from_pools(k_pool, v_pool, kv_dtype, k_scale=1.0, v_scale=1.0, k_sf=None, v_sf=None):
    """pa_kv_cache for two [num_pages, Hkv, P, D] views (halves of a combined cache or
    separate pools), taking strides from the tensors.  NVFP4 pools are uint8
    [num_pages, Hkv, P, D/2] with block-scale views k_sf / v_sf [num_pages, Hkv, P, D/16]."""
    fp4 = kv_dtype == "nvfp4"
    if fp4 != (k_sf is not None and v_sf is not None):
        raise ValueError("block scales k_sf and v_sf go with kv_dtype 'nvfp4' and only with it")
    for t in (k_pool, v_pool) + ((k_sf, v_sf) if fp4 else ()):
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("pools must be [num_pages, num_kv_heads, page_size, head_dim] views "
                             "with a unit head_dim stride")
    per_unit = 2 if fp4 else 1  # elements per stored unit
    c = pa_kv_cache()
    c.k, c.v = k_pool.data_ptr(), v_pool.data_ptr()
    c.kv_dtype = kv_dtype_code(kv_dtype)
    c.num_pages, c.num_kv_heads, c.page_size = k_pool.shape[:3]
    c.head_dim_qk = k_pool.shape[3] * per_unit
    c.head_dim_vo = v_pool.shape[3] * per_unit
    c.k_stride_page, c.k_stride_head, c.k_stride_token = k_pool.stride()[:3]
    c.v_stride_page, c.v_stride_head, c.v_stride_token = v_pool.stride()[:3]
    c.k_scale, c.v_scale = k_scale, v_scale
    if fp4:
        if (k_sf.shape[3] * 16 != c.head_dim_qk or v_sf.shape[3] * 16 != c.head_dim_vo
                or tuple(k_sf.shape[:3]) != tuple(k_pool.shape[:3])
                or tuple(v_sf.shape[:3]) != tuple(v_pool.shape[:3])):
            raise ValueError("block scales must be [num_pages, num_kv_heads, page_size, D/16]")
        c.k_sf, c.v_sf = k_sf.data_ptr(), v_sf.data_ptr()
        c.k_sf_stride_page, c.k_sf_stride_head, c.k_sf_stride_token = k_sf.stride()[:3]
        c.v_sf_stride_page, c.v_sf_stride_head, c.v_sf_stride_token = v_sf.stride()[:3]
    return c


def current_stream_handle():
    torch = _torch()
    return c_void_p(torch.cuda.current_stream().cuda_stream)


class PagedDecode:
    """Plans a decode batch once, uploads the plan, and runs decode steps."""

    def __init__(self, k_pool, v_pool, kv_indptr, kv_indices, kv_last_page_len, num_qo_heads,
                 *, kv_dtype="bf16", k_scale=1.0, v_scale=1.0, sm_scale=None, window=0,
                 num_splits=0, out_dtype="bf16", k_sf=None, v_sf=None):
        torch = _torch()
        dev = k_pool.device
        self.cache = cache_from_pools(k_pool, v_pool, kv_dtype, k_scale, v_scale, k_sf, v_sf)
        self._keep = (k_pool, v_pool, k_sf, v_sf)
        self.params = pa_attn_params(num_qo_heads, sm_scale if sm_scale is not None
                                     else 1.0 / float(self.cache.head_dim_qk) ** 0.5,
                                     window, 1, PA_DTYPE_BF16, out_dtype_code(out_dtype))
        self.out_dtype = out_dtype
        self.indptr_d = torch.as_tensor(np.asarray(kv_indptr, np.int32)).to(dev)
        self.indices_d = torch.as_tensor(np.asarray(kv_indices, np.int32)).to(dev)
        self.last_d = torch.as_tensor(np.asarray(kv_last_page_len, np.int32)).to(dev)
        self.batch = len(kv_indptr) - 1
        self.table = pa_page_table(self.indptr_d.data_ptr(), self.indices_d.data_ptr(),
                                   self.last_d.data_ptr(), self.batch)
        self.plan, self.plan_buf = pa_decode_plan(self.params, self.cache, kv_indptr,
                                                  kv_last_page_len, num_splits)
        self.workspace = torch.empty(max(256, self.plan.workspace_bytes), dtype=torch.uint8,
                                     device=dev)
        pa_plan_upload(self.plan, self.plan_buf, self.workspace.data_ptr(),
                       self.workspace.numel(), current_stream_handle())
        torch.cuda.current_stream().synchronize()  # the host plan buffer may now change

    def run(self, q, out=None, lse=None, with_lse=True):
        torch = _torch()
        hq, dvo = self.params.num_qo_heads, self.cache.head_dim_vo
        if q.dtype != torch.bfloat16 or not q.is_contiguous() or tuple(q.shape) != (
                self.batch, hq, self.cache.head_dim_qk):
            raise ValueError("q must be a contiguous bf16 [batch, num_qo_heads, head_dim_qk]")
        odt = torch.float32 if self.out_dtype == "fp32" else torch.bfloat16
        if out is None:
            out = torch.empty((self.batch, hq, dvo), dtype=odt, device=q.device)
        if lse is None and with_lse:
            lse = torch.empty((self.batch, hq), dtype=torch.float32, device=q.device)
        pa_paged_decode(self.plan, q.data_ptr(), self.cache, self.table, self.params,
                        out.data_ptr(), lse.data_ptr() if lse is not None else None,
                        self.workspace.data_ptr(), self.workspace.numel(),
                        current_stream_handle())
        return out, lse


class PagedPrefill:
    """Plans a prefill batch once, uploads the plan, and runs prefills."""

    def __init__(self, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                 num_qo_heads, *, kv_dtype="bf16", k_scale=1.0, v_scale=1.0, sm_scale=None,
                 window=0, causal=True, out_dtype="bf16", k_sf=None, v_sf=None):
        torch = _torch()
        dev = k_pool.device
        self.cache = cache_from_pools(k_pool, v_pool, kv_dtype, k_scale, v_scale, k_sf, v_sf)
        self._keep = (k_pool, v_pool, k_sf, v_sf)
        self.params = pa_attn_params(num_qo_heads, sm_scale if sm_scale is not None
                                     else 1.0 / float(self.cache.head_dim_qk) ** 0.5,
                                     window, 1 if causal else 0, PA_DTYPE_BF16,
                                     out_dtype_code(out_dtype))
        self.out_dtype = out_dtype
        self.qo_indptr_d = torch.as_tensor(np.asarray(qo_indptr, np.int32)).to(dev)
        self.indptr_d = torch.as_tensor(np.asarray(kv_indptr, np.int32)).to(dev)
        self.indices_d = torch.as_tensor(np.asarray(kv_indices, np.int32)).to(dev)
        self.last_d = torch.as_tensor(np.asarray(kv_last_page_len, np.int32)).to(dev)
        self.batch = len(kv_indptr) - 1
        self.total_q = int(qo_indptr[-1])
        self.table = pa_page_table(self.indptr_d.data_ptr(), self.indices_d.data_ptr(),
                                   self.last_d.data_ptr(), self.batch)
        self.plan, self.plan_buf = pa_prefill_plan(self.params, self.cache, qo_indptr, kv_indptr,
                                                   kv_last_page_len)
        self.workspace = torch.empty(max(256, self.plan.workspace_bytes), dtype=torch.uint8,
                                     device=dev)
        pa_plan_upload(self.plan, self.plan_buf, self.workspace.data_ptr(),
                       self.workspace.numel(), current_stream_handle())
        torch.cuda.current_stream().synchronize()

    def run(self, q, out=None, lse=None, with_lse=True):
        torch = _torch()
        hq, dvo = self.params.num_qo_heads, self.cache.head_dim_vo
        if q.dtype != torch.bfloat16 or not q.is_contiguous() or tuple(q.shape) != (
                self.total_q, hq, self.cache.head_dim_qk):
            raise ValueError("q must be a contiguous bf16 [total_q, num_qo_heads, head_dim_qk]")
        odt = torch.float32 if self.out_dtype == "fp32" else torch.bfloat16
        if out is None:
            out = torch.empty((self.total_q, hq, dvo), dtype=odt, device=q.device)
        if lse is None and with_lse:
            lse = torch.empty((self.total_q, hq), dtype=torch.float32, device=q.device)
        pa_paged_prefill(self.plan, q.data_ptr(), self.qo_indptr_d.data_ptr(), self.cache,
                         self.table, self.params, out.data_ptr(),
                         lse.data_ptr() if lse is not None else None, self.workspace.data_ptr(),
                         self.workspace.numel(), current_stream_handle())
        return out, lse


def decode_segments(plan, plan_buf):
    """Raw segment records of a decode plan as a [num_items, 8] int32 array (b, kv_head,
    t_begin, t_end, slot, page_base, more_begin, more_count): the head segment of each wave
    in launch order, then the waves' further segments.  Bits 0-15 of a head's more_count
    count the wave's further segments; bits 16-23 of a wave's last segment give the size of
    its group of combined results (0: none) and bits 24-31 the group's first wave within
    the workgroup."""
    off = plan.items_offset
    return plan_buf[off:off + 32 * plan.num_items].view(np.int32).reshape(-1, 8)


def decode_waves(plan, plan_buf):
    """Segments of a decode plan per wave, in launch order: a list of [k, 5] int32 arrays
    of (b, kv_head, t_begin, t_end, slot)."""
    segs = decode_segments(plan, plan_buf)
    waves = []
    for w in range(plan.num_workers):
        more_begin, more_count = int(segs[w, 6]), int(segs[w, 7]) & 0xFFFF
        rows = [segs[w]] + [segs[more_begin + k] for k in range(more_count)]
        waves.append(np.stack(rows)[:, :5])
    return waves


def decode_groups(plan, plan_buf):
    """Per wave in launch order, (size, first wave within the workgroup) of the group whose
    results its last segment joins, or (0, 0)."""
    segs = decode_segments(plan, plan_buf)
    out = []
    for w in range(plan.num_workers):
        n_more = int(segs[w, 7]) & 0xFFFF
        last = segs[w] if n_more == 0 else segs[int(segs[w, 6]) + n_more - 1]
        bits = int(last[7]) & 0xFFFFFFFF
        out.append(((bits >> 16) & 0xFF, bits >> 24))
    return out


def decode_merges(plan, plan_buf):
    """Merge entries of a decode plan as a [num_merges, 4] int32 array
    (b, kv_head, slot_begin, num_slots)."""
    off = plan.merges_offset
    return plan_buf[off:off + 16 * plan.num_merges].view(np.int32).reshape(-1, 4)


def prefill_items(plan, plan_buf):
    """Items of a prefill plan as a [num_items, 9] int32 array (b, row_begin, row_end,
    kv_begin, kv_end, q_begin, kv_len, q_len, slot); slot -1 writes the output directly."""
    off = plan.items_offset
    return plan_buf[off:off + 48 * plan.num_items].view(np.int32).reshape(-1, 12)[:, :9]


def prefill_merges(plan, plan_buf):
    """Merge entries of a prefill plan (split tiles) as a [num_merges, 6] int32 array
    (b, row_begin, row_end, q_begin, slot_begin, num_slots)."""
    off = plan.merges_offset
    return plan_buf[off:off + 32 * plan.num_merges].view(np.int32).reshape(-1, 8)[:, :6]
