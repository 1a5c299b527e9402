"""Thin ctypes binding of libsdpa.so (the C-ABI in include/sdpa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  Tensors are torch tensors on the GPU (torch is used for device
memory and streams); pointers, element strides and the current HIP stream are
handed to the C entry points of the same names.  Outputs the caller does not
pass are allocated here with torch as a convenience; the library itself never
allocates.

The library must have been built (``python -m scaled_dot_product_19_amd.build``
or ``__graft_entry__.build()``); if it is missing, every call raises -- there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

SDPA_OK = 0
SDPA_ERR_NULL = 1
SDPA_ERR_SHAPE = 2
SDPA_ERR_UNSUPPORTED = 3
SDPA_ERR_WORKSPACE = 4
SDPA_ERR_LSE_LAYOUT = 5
SDPA_ERR_HIP = 6

SDPA_BF16 = 0
SDPA_FP32 = 1
SDPA_FP8_E4M3 = 2

LSE_NONE = 0
LSE_PACKED = 1
LSE_PADDED = 2
LSE_HEAD_MAJOR = 3

# every symbol include/sdpa.h declares
EXPORTS = ("sdpa_prefill_thd", "sdpa_prefill_thd_ex", "sdpa_prefill_thd_fp8",
           "sdpa_decode_workspace_bytes", "sdpa_decode_path", "sdpa_decode_paged", "sdpa_decode_paged_fp8",
           "sdpa_decode_paged_ex", "sdpa_decode_paged_noalloc", "sdpa_splitkv_combine", "sdpa_status_string",
           "sdpa_last_error_detail", "sdpa_version")


class SdpaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("sdpa status %d (%s): %s" % (status, _status_name(status), detail))
        self.status = status
        self.detail = detail


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libsdpa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libsdpa.so is not built at %s; run "
                           "`python -m scaled_dot_product_19_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                          ctypes.c_size_t)
    lib.sdpa_prefill_thd.restype = ctypes.c_int
    lib.sdpa_prefill_thd.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, I64, I64, P, P,
                                     I32, I32, I32, I32, I32, I32, I32, F, I32, P, I32, I32,
                                     I32, P]
    lib.sdpa_prefill_thd_ex.restype = ctypes.c_int
    lib.sdpa_prefill_thd_ex.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, I64, I64, P, P,
                                        I32, I32, I32, I32, I32, I32, I32, F, I32, I32, P, P, I32,
                                        I32, I32, I32, P]
    lib.sdpa_prefill_thd_fp8.restype = ctypes.c_int
    lib.sdpa_prefill_thd_fp8.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, I64, I64, P,
                                         P, I32, I32, I32, I32, I32, I32, I32, F, I32, I32, P, P,
                                         I32, I32, I32, P, P, P, P]
    lib.sdpa_decode_workspace_bytes.restype = SZ
    lib.sdpa_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.sdpa_decode_path.restype = ctypes.c_int
    lib.sdpa_decode_path.argtypes = [I32, I32, I32, I32, I32, I32, I32, I64, I64, I32, I32]
    lib.sdpa_decode_paged.restype = ctypes.c_int
    lib.sdpa_decode_paged.argtypes = [P, P, I64, I64, I64, P, I64, I64, I64, P, P, I32, P, I32,
                                      I32, I32, I32, I32, I32, I32, I32, F, I32, I32, P, SZ, P,
                                      P, I32, P]
    lib.sdpa_decode_paged_fp8.restype = ctypes.c_int
    lib.sdpa_decode_paged_fp8.argtypes = [P, P, I64, I64, I64, P, I64, I64, I64, P, P, I32, P,
                                          I32, I32, I32, I32, I32, I32, I32, I32, F, I32, I32, P,
                                          SZ, P, P, P, P, P, P]
    lib.sdpa_decode_paged_ex.restype = ctypes.c_int
    lib.sdpa_decode_paged_ex.argtypes = [P, P, I64, I64, I64, P, I64, I64, I64, P, P, I32, P,
                                         I32, I32, I32, I32, I32, I32, I32, I32, F, I32, I32, P,
                                         I32, I32, P, SZ, P, P, P, P, P, I32, P]
    lib.sdpa_decode_paged_noalloc.restype = ctypes.c_int
    lib.sdpa_decode_paged_noalloc.argtypes = [P, P, I64, I64, I64, P, I64, I64, I64, P, P, I32,
                                              P, I32, I32, I32, I32, I32, I32, I32, I32, F, I32,
                                              I32, P, P, I32, P]
    lib.sdpa_splitkv_combine.restype = ctypes.c_int
    lib.sdpa_splitkv_combine.argtypes = [P, P, I32, I64, I32, P, P, I32, P]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_last_error_detail.restype = ctypes.c_char_p
    lib.sdpa_last_error_detail.argtypes = []
    lib.sdpa_version.restype = ctypes.c_int
    lib.sdpa_version.argtypes = []
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load().sdpa_status_string(status).decode()
    except Exception:
        return "?"


def _check(rc: int):
    if rc != SDPA_OK:
        raise SdpaError(rc, load().sdpa_last_error_detail().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SDPA_BF16
    if t.dtype == torch.float32:
        return SDPA_FP32
    raise TypeError("Q/K/V must be bfloat16 or float32, got %s" % t.dtype)


def version() -> int:
    return int(load().sdpa_version())


def decode_workspace_bytes(batch: int, s_q: int, h_q: int, d_v: int, num_splits: int) -> int:
    return int(load().sdpa_decode_workspace_bytes(batch, s_q, h_q, d_v, num_splits))


PATH_NAMES = {1: "few_row", 2: "row_groups", 3: "prefill", 4: "prefill_folded", 5: "wide",
              6: "general"}


def decode_path(batch: int, s_q: int, h_q: int, h_kv: int, d_qk: int, d_v: int, page_size: int,
                k_st: int, v_st: int, num_splits: int, fp8: bool = False) -> str:
    """Name of the kernel sdpa_decode_paged (fp8: sdpa_decode_paged_fp8) runs for these
    extents, or "" when the call is declined (host-only, no GPU call)."""
    p = int(load().sdpa_decode_path(batch, s_q, h_q, h_kv, d_qk, d_v, page_size, k_st, v_st,
                                    num_splits, SDPA_FP8_E4M3 if fp8 else SDPA_BF16))
    return PATH_NAMES.get(p, "")


def prefill_thd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                cu_seqlens_kv: torch.Tensor, max_seqlen_q: int, max_seqlen_kv: int,
                scale: float, causal: bool = True, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, lse_layout: int = LSE_PACKED,
                lse_s_max: int = 0, stream=None):
    """sdpa_prefill_thd.  q [Tq, Hq, Dqk], k [Tk, Hkv, Dqk], v [Tk, Hkv, Dv] on the GPU.

    Returns (out [Tq, Hq, Dv], lse) where lse is [Tq, Hq] (packed), [B, lse_s_max, Hq]
    (padded) or None.
    """
    lib = load()
    batch = int(cu_seqlens_q.numel()) - 1
    hq, dqk = int(q.shape[1]), int(q.shape[2])
    hkv, dv = int(k.shape[1]), int(v.shape[2])
    if out is None:
        out = torch.empty((q.shape[0], hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and lse_layout == LSE_PACKED:
        lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    elif lse is None and lse_layout == LSE_PADDED:
        lse = torch.empty((batch, lse_s_max, hq), dtype=torch.float32, device=q.device)
    rc = lib.sdpa_prefill_thd(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1), _ptr(v),
        v.stride(0), v.stride(1), _ptr(out), out.stride(0), out.stride(1), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_kv), batch, int(max_seqlen_q), int(max_seqlen_kv), hq, hkv, dqk, dv,
        float(scale), int(bool(causal)), _ptr(lse) if lse_layout != LSE_NONE else None,
        int(lse_layout), int(lse_s_max), _dtype_code(q), _stream(stream))
    _check(rc)
    return out, (lse if lse_layout != LSE_NONE else None)


def prefill_thd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                   cu_seqlens_kv: torch.Tensor, max_seqlen_q: int, max_seqlen_kv: int,
                   scale: float, causal: bool = True, window_left: int = 0,
                   sinks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, lse_layout: int = LSE_PACKED,
                   lse_s_max: int = 0, stats_log2: bool = False, stream=None):
    """sdpa_prefill_thd_ex: sdpa_prefill_thd plus a left sliding window, per-head
    sinks (fp32 [Hq]) and base-2 Stats.  lse is [Tq, Hq] (packed), [B, lse_s_max, Hq]
    (padded), [Hq, lse_s_max] (head-major; lse_s_max defaults to Tq) or None.
    """
    lib = load()
    batch = int(cu_seqlens_q.numel()) - 1
    hq, dqk = int(q.shape[1]), int(q.shape[2])
    hkv, dv = int(k.shape[1]), int(v.shape[2])
    if out is None:
        out = torch.empty((q.shape[0], hq, dv), dtype=q.dtype, device=q.device)
    if lse_layout == LSE_HEAD_MAJOR and lse_s_max == 0:
        lse_s_max = int(q.shape[0])
    if lse is None and lse_layout == LSE_PACKED:
        lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    elif lse is None and lse_layout == LSE_PADDED:
        lse = torch.empty((batch, lse_s_max, hq), dtype=torch.float32, device=q.device)
    elif lse is None and lse_layout == LSE_HEAD_MAJOR:
        lse = torch.empty((hq, lse_s_max), dtype=torch.float32, device=q.device)
    rc = lib.sdpa_prefill_thd_ex(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1), _ptr(v),
        v.stride(0), v.stride(1), _ptr(out), out.stride(0), out.stride(1), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_kv), batch, int(max_seqlen_q), int(max_seqlen_kv), hq, hkv, dqk, dv,
        float(scale), int(bool(causal)), int(window_left), _ptr(sinks),
        _ptr(lse) if lse_layout != LSE_NONE else None, int(lse_layout), int(lse_s_max),
        int(bool(stats_log2)), _dtype_code(q), _stream(stream))
    _check(rc)
    return out, (lse if lse_layout != LSE_NONE else None)


def prefill_thd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_kv: torch.Tensor, max_seqlen_q: int, max_seqlen_kv: int,
                    scale: float, descale_q: torch.Tensor, descale_k: torch.Tensor,
                    descale_v: torch.Tensor, causal: bool = True, window_left: int = 0,
                    sinks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, lse_layout: int = LSE_PACKED,
                    lse_s_max: int = 0, stats_log2: bool = False, stream=None):
    """sdpa_prefill_thd_fp8: q [Tq, Hq, D], k/v [Tk, Hkv, D] uint8 E4M3 codes; descales are
    one-element fp32 device tensors.  Returns (out [Tq, Hq, D] bf16, lse as prefill_thd_ex)."""
    lib = load()
    for t in (q, k, v):
        if t.dtype != torch.uint8:
            raise TypeError("FP8 prefill takes uint8 E4M3 codes, got %s" % t.dtype)
    for t in (descale_q, descale_k, descale_v):
        if t.dtype != torch.float32 or t.numel() != 1:
            raise TypeError("descales are one-element float32 tensors")
    batch = int(cu_seqlens_q.numel()) - 1
    hq, dqk = int(q.shape[1]), int(q.shape[2])
    hkv, dv = int(k.shape[1]), int(v.shape[2])
    if out is None:
        out = torch.empty((q.shape[0], hq, dv), dtype=torch.bfloat16, device=q.device)
    if lse_layout == LSE_HEAD_MAJOR and lse_s_max == 0:
        lse_s_max = int(q.shape[0])
    if lse is None and lse_layout == LSE_PACKED:
        lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    elif lse is None and lse_layout == LSE_PADDED:
        lse = torch.empty((batch, lse_s_max, hq), dtype=torch.float32, device=q.device)
    elif lse is None and lse_layout == LSE_HEAD_MAJOR:
        lse = torch.empty((hq, lse_s_max), dtype=torch.float32, device=q.device)
    rc = lib.sdpa_prefill_thd_fp8(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.stride(1), _ptr(v),
        v.stride(0), v.stride(1), _ptr(out), out.stride(0), out.stride(1), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_kv), batch, int(max_seqlen_q), int(max_seqlen_kv), hq, hkv, dqk, dv,
        float(scale), int(bool(causal)), int(window_left), _ptr(sinks),
        _ptr(lse) if lse_layout != LSE_NONE else None, int(lse_layout), int(lse_s_max),
        int(bool(stats_log2)), _ptr(descale_q), _ptr(descale_k), _ptr(descale_v),
        _stream(stream))
    _check(rc)
    return out, (lse if lse_layout != LSE_NONE else None)


def decode_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 page_table_k: torch.Tensor, page_table_v: torch.Tensor,
                 seq_lens: torch.Tensor, max_seqlen_kv: int, scale: float, causal: bool = True,
                 num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 want_lse: bool = True, stream=None):
    """sdpa_decode_paged.  q [B, s_q, Hq, Dqk]; pools [P, page, Hkv, D*] (any strides with a
    contiguous last axis); page tables int32 [B, table_stride]; seq_lens int32 [B].

    Returns (out [B, s_q, Hq, Dv], lse [B, s_q, Hq] or None).
    """
    lib = load()
    B, s_q, hq, dqk = (int(x) for x in q.shape)
    page, hkv, dv = int(k_pool.shape[1]), int(k_pool.shape[2]), int(v_pool.shape[3])
    if out is None:
        out = torch.empty((B, s_q, hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, hq), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, s_q, hq, dv, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.sdpa_decode_paged(
        _ptr(q), _ptr(k_pool), k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(v_pool), v_pool.stride(0), v_pool.stride(1), v_pool.stride(2), _ptr(page_table_k),
        _ptr(page_table_v), int(page_table_k.shape[1]), _ptr(seq_lens), int(max_seqlen_kv), B,
        s_q, hq, hkv, dqk, dv, page, float(scale), int(bool(causal)), int(num_splits),
        _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _dtype_code(q), _stream(stream))
    _check(rc)
    return out, lse


def decode_paged_ex(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                    page_table_k: torch.Tensor, page_table_v: torch.Tensor,
                    seq_lens: torch.Tensor, max_seqlen_kv: int, scale: float,
                    causal: bool = True, window_left: int = 0,
                    sinks: Optional[torch.Tensor] = None, stats_log2: bool = False,
                    num_splits: int = 1, descale: Optional[tuple] = None,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """sdpa_decode_paged_ex.  bf16 q / pools, or uint8 E4M3 codes with descale =
    (descale_q, descale_k, descale_v) one-element fp32 device tensors; sinks fp32 [Hq].

    Returns (out [B, s_q, Hq, Dv] bf16, lse [B, s_q, Hq] or None).
    """
    lib = load()
    fp8 = q.dtype == torch.uint8
    if fp8 and (descale is None or len(descale) != 3):
        raise TypeError("E4M3 codes need descale = (descale_q, descale_k, descale_v)")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.dim() != 1):
        raise TypeError("sinks are a float32 [Hq] tensor")
    B, s_q, hq, dqk = (int(x) for x in q.shape)
    page, hkv, dv = int(k_pool.shape[1]), int(k_pool.shape[2]), int(v_pool.shape[3])
    if out is None:
        out = torch.empty((B, s_q, hq, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, hq), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, s_q, hq, dv, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dq, dk, dvs = (None, None, None) if descale is None else descale
    rc = lib.sdpa_decode_paged_ex(
        _ptr(q), _ptr(k_pool), k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(v_pool), v_pool.stride(0), v_pool.stride(1), v_pool.stride(2), _ptr(page_table_k),
        _ptr(page_table_v), int(page_table_k.shape[1]), _ptr(seq_lens), int(max_seqlen_kv), B,
        s_q, hq, hkv, dqk, dv, page, float(scale), int(bool(causal)), int(window_left),
        _ptr(sinks), int(bool(stats_log2)), int(num_splits), _ptr(workspace), ws_bytes,
        _ptr(dq), _ptr(dk), _ptr(dvs), _ptr(out), _ptr(lse),
        SDPA_FP8_E4M3 if fp8 else _dtype_code(q), _stream(stream))
    _check(rc)
    return out, lse


def decode_paged_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                         page_table_k: torch.Tensor, page_table_v: torch.Tensor,
                         seq_lens: torch.Tensor, max_seqlen_kv: int, scale: float,
                         out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                         causal: bool = True, num_splits: int = 1, stream=None):
    """sdpa_decode_paged_noalloc: sdpa_decode_paged with the split partials in the
    library-owned device array (no workspace argument; the caller passes out and lse).

    Returns (out, lse).
    """
    lib = load()
    B, s_q, hq, dqk = (int(x) for x in q.shape)
    page, hkv, dv = int(k_pool.shape[1]), int(k_pool.shape[2]), int(v_pool.shape[3])
    rc = lib.sdpa_decode_paged_noalloc(
        _ptr(q), _ptr(k_pool), k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(v_pool), v_pool.stride(0), v_pool.stride(1), v_pool.stride(2), _ptr(page_table_k),
        _ptr(page_table_v), int(page_table_k.shape[1]), _ptr(seq_lens), int(max_seqlen_kv), B,
        s_q, hq, hkv, dqk, dv, page, float(scale), int(bool(causal)), int(num_splits),
        _ptr(out), _ptr(lse), _dtype_code(q), _stream(stream))
    _check(rc)
    return out, lse


def decode_paged_fp8(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                     page_table_k: torch.Tensor, page_table_v: torch.Tensor,
                     seq_lens: torch.Tensor, max_seqlen_kv: int, scale: float,
                     descale_q: torch.Tensor, descale_k: torch.Tensor, descale_v: torch.Tensor,
                     causal: bool = True, num_splits: int = 1,
                     workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """sdpa_decode_paged_fp8.  q [B, s_q, Hq, D] and pools [P, page, Hkv, D] hold uint8 E4M3
    codes; descale_q/k/v are one-element fp32 device tensors.

    Returns (out [B, s_q, Hq, D] bf16, lse [B, s_q, Hq] or None).
    """
    lib = load()
    for t in (q, k_pool, v_pool):
        if t.dtype != torch.uint8:
            raise TypeError("FP8 decode takes uint8 E4M3 codes, got %s" % t.dtype)
    for t in (descale_q, descale_k, descale_v):
        if t.dtype != torch.float32 or t.numel() != 1:
            raise TypeError("descales are one-element float32 tensors")
    B, s_q, hq, dqk = (int(x) for x in q.shape)
    page, hkv, dv = int(k_pool.shape[1]), int(k_pool.shape[2]), int(v_pool.shape[3])
    if out is None:
        out = torch.empty((B, s_q, hq, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, hq), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, s_q, hq, dv, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.sdpa_decode_paged_fp8(
        _ptr(q), _ptr(k_pool), k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(v_pool), v_pool.stride(0), v_pool.stride(1), v_pool.stride(2), _ptr(page_table_k),
        _ptr(page_table_v), int(page_table_k.shape[1]), _ptr(seq_lens), int(max_seqlen_kv), B,
        s_q, hq, hkv, dqk, dv, page, float(scale), int(bool(causal)), int(num_splits),
        _ptr(workspace), ws_bytes, _ptr(descale_q), _ptr(descale_k), _ptr(descale_v), _ptr(out),
        _ptr(lse), _stream(stream))
    _check(rc)
    return out, lse


def splitkv_combine(o_part: torch.Tensor, lse_part: torch.Tensor,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.bfloat16, want_lse: bool = True,
                    stream=None):
    """sdpa_splitkv_combine.  o_part fp32 [S, rows, Dv], lse_part fp32 [S, rows]."""
    lib = load()
    S, rows, dv = (int(x) for x in o_part.shape)
    if out is None:
        out = torch.empty((rows, dv), dtype=out_dtype, device=o_part.device)
    if lse is None and want_lse:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device)
    rc = lib.sdpa_splitkv_combine(_ptr(o_part), _ptr(lse_part), S, rows, dv, _ptr(out), _ptr(lse),
                                  _dtype_code(out), _stream(stream))
    _check(rc)
    return out, lse
