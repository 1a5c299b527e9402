"""ctypes front of the fp64 CPU oracle (``sdpa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke entry point and the benchmark's
CPU-baseline leg use this module; the HIP library and its Python binding never
import it.  It shares no code with the GPU path.

Arrays are numpy.  bf16 inputs are passed as their raw ``uint16`` bit
patterns, fp32 inputs as ``float32``, FP8 E4M3 inputs as their ``uint8``
codes (with per-tensor descales); the C side widens them exactly to double.
Outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdpa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
F32 = 1
E4M3 = 2

_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc with IEEE semantics: no fast-math, no FMA contraction."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared",
           "-fPIC", "-o", tmp, src, "-lpthread", "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


def _load(path: str | None = None):
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_prefill_thd.restype = ctypes.c_int
    lib.oracle_prefill_thd.argtypes = [
        ctypes.c_int, P, I64, I64, P, I64, I64, P, I64, I64, P, P, I32, I32, I32, I32, I32,
        D, I32, I32, P, I64, P, P, P, P, P, I32]
    lib.oracle_prefill_thd_scaled.restype = ctypes.c_int
    lib.oracle_prefill_thd_scaled.argtypes = [
        ctypes.c_int, P, I64, I64, P, I64, I64, P, I64, I64, P, P, I32, I32, I32, I32, I32,
        D, I32, I32, P, D, D, D, I64, P, P, P, P, P, I32]
    lib.oracle_decode_paged.restype = ctypes.c_int
    lib.oracle_decode_paged.argtypes = [
        ctypes.c_int, P, P, I64, I64, I64, P, I64, I64, I64, P, P, I32, P, I32, I32, I32,
        I32, I32, I32, I32, D, I32, I32, I64, P, P, P, P, P, I32]
    lib.oracle_decode_paged_scaled.restype = ctypes.c_int
    lib.oracle_decode_paged_scaled.argtypes = [
        ctypes.c_int, P, P, I64, I64, I64, P, I64, I64, I64, P, P, I32, P, I32, I32, I32,
        I32, I32, I32, I32, D, I32, I32, I32, P, D, D, D, I64, P, P, P, P, P, I32]
    lib.oracle_e4m3_value.restype = D
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [P, P, I32, I64, I32, P, P]
    lib.oracle_nproc.restype = ctypes.c_int
    lib.oracle_nproc.argtypes = []
    _lib = lib
    return lib


class variant:
    """Context manager that points this module at another build of the oracle.

    Used only by the mutation tests, which compile copies of the oracle with a
    planted mistake and check that the pins reject them.
    """

    def __init__(self, lib_path: str):
        self.lib_path = lib_path
        self.saved = None

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = None
        _load(self.lib_path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def nproc() -> int:
    return int(_load().oracle_nproc())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError("oracle inputs are uint16 (bf16 bits), float32 or uint8 (E4M3 codes), "
                    "got %s" % a.dtype)


def e4m3_value(code: int) -> float:
    """The value of one OCP E4M3 code (0..255), by the format's definition."""
    return float(_load().oracle_e4m3_value(int(code)))


def _strides(a: np.ndarray):
    return [s // a.itemsize for s in a.strides]


def prefill_thd(q, k, v, cu_q, cu_kv, scale, causal, hq=None, hkv=None, sel_tok=None,
                sel_head=None, want_probs=False, nthreads=0, window=0, sinks=None, descale=None):
    """Packed THD prefill by definition.

    E4M3 inputs (uint8 codes) need descale = (descale_q, descale_k, descale_v): each
    code stands for its descale times its E4M3 value (per-tensor FP8).

    window > 0: left sliding window W (a row sees keys diag - W + 1 .. diag of its
    bottom-right diagonal position diag); sinks: Hq per-head sink logits (same units as
    scale * q.k) that join the softmax denominator and carry no value.

    q [Tq, Hq, Dqk], k [Tk, Hkv, Dqk], v [Tk, Hkv, Dv]; last axis contiguous,
    any token/head strides.  cu_q/cu_kv int32 [B+1].
    Returns (o, lse[, probs]): all rows -> o [Tq, Hq, Dv], lse [Tq, Hq];
    with sel_tok/sel_head -> o [n, Dv], lse [n].
    """
    lib = _load()
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    for a in (q, k, v):
        assert a.ndim == 3 and a.strides[2] == a.itemsize, "last axis must be contiguous"
    tq, hq_, dqk = q.shape
    _, hkv_, _ = k.shape
    dv = v.shape[2]
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    cu_kv = np.ascontiguousarray(cu_kv, dtype=np.int32)
    batch = len(cu_q) - 1
    if sel_tok is None:
        n_sel = -1
        o = np.zeros((tq * hq_, dv), np.float64)
        lse = np.zeros(tq * hq_, np.float64)
        st = sh = None
    else:
        st = np.ascontiguousarray(sel_tok, dtype=np.int64)
        sh = np.ascontiguousarray(sel_head, dtype=np.int32)
        n_sel = len(st)
        o = np.zeros((n_sel, dv), np.float64)
        lse = np.zeros(n_sel, np.float64)
    max_lk = max(1, int((cu_kv[1:] - cu_kv[:-1]).max()) if batch > 0 else 1)
    probs = None
    if want_probs:
        probs = np.zeros((o.shape[0], max_lk), np.float64)
    qs, ks, vs = _strides(q), _strides(k), _strides(v)
    sk = None
    if sinks is not None:
        sk = np.ascontiguousarray(sinks, dtype=np.float64)
        assert sk.shape == (hq_,)
    if dt == E4M3:
        assert descale is not None and len(descale) == 3, "E4M3 inputs need their descales"
        dsc = [float(x) for x in descale]
    else:
        assert descale is None, "descales apply to E4M3 inputs only"
        dsc = [1.0, 1.0, 1.0]
    rc = lib.oracle_prefill_thd_scaled(dt, _ptr(q), qs[0], qs[1], _ptr(k), ks[0], ks[1],
                                       _ptr(v), vs[0], vs[1], _ptr(cu_q), _ptr(cu_kv), batch,
                                       hq_, hkv_, dqk, dv, float(scale), int(bool(causal)),
                                       int(window), _ptr(sk), dsc[0], dsc[1], dsc[2], n_sel,
                                       _ptr(st), _ptr(sh), _ptr(o), _ptr(lse), _ptr(probs),
                                       int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill_thd rejected its arguments (rc=%d)" % rc)
    if sel_tok is None:
        o = o.reshape(tq, hq_, dv)
        lse = lse.reshape(tq, hq_)
    if want_probs:
        return o, lse, probs
    return o, lse


def decode_paged(q, k_pool, v_pool, pt_k, pt_v, seq_lens, page_size, scale, causal,
                 num_splits=1, sel_rows=None, want_partials=False, nthreads=0, descale=None,
                 window=0, sinks=None):
    """Paged decode by definition (num_splits > 1: per-chunk partials + LSE merge).

    window > 0: left sliding window W (token t at position L - sq + t sees keys
    L - sq + t - W + 1 ..); sinks: Hq per-head sink logits (same units as scale * q.k)
    that join the softmax denominator once (in the merge when split) and carry no value.

    E4M3 inputs (uint8 codes) need descale = (descale_q, descale_k, descale_v): each
    code stands for its descale times its E4M3 value (per-tensor FP8).

    q [B, sq, Hq, Dqk] contiguous; pools [P, page, Hkv, D] with contiguous last
    axis; page tables int32 [B, table_stride]; seq_lens int32 [B].
    Returns (o [B, sq, Hq, Dv], lse [B, sq, Hq]) for all rows, or (o [n, Dv],
    lse [n]) for sel_rows (row = (b*sq + t)*Hq + h).  want_partials adds
    (o_part [S, rows, Dv], lse_part [S, rows]).
    """
    lib = _load()
    dt = _dtype_code(q)
    assert _dtype_code(k_pool) == dt and _dtype_code(v_pool) == dt
    q = np.ascontiguousarray(q)
    B, sq, hq, dqk = q.shape
    hkv = k_pool.shape[2]
    dv = v_pool.shape[3]
    for a in (k_pool, v_pool):
        assert a.ndim == 4 and a.strides[3] == a.itemsize
    pt_k = np.ascontiguousarray(pt_k, dtype=np.int32)
    pt_v = np.ascontiguousarray(pt_v, dtype=np.int32)
    assert pt_k.shape == pt_v.shape
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    rows = B * sq * hq
    if sel_rows is None:
        n_sel, sr = -1, None
        o = np.zeros((rows, dv), np.float64)
        lse = np.zeros(rows, np.float64)
    else:
        sr = np.ascontiguousarray(sel_rows, dtype=np.int64)
        n_sel = len(sr)
        o = np.zeros((n_sel, dv), np.float64)
        lse = np.zeros(n_sel, np.float64)
    S = max(1, int(num_splits))
    o_part = lse_part = None
    if want_partials:
        assert sel_rows is None
        o_part = np.zeros((S, rows, dv), np.float64)
        lse_part = np.zeros((S, rows), np.float64)
    ks, vs = _strides(k_pool), _strides(v_pool)
    if dt == E4M3:
        assert descale is not None and len(descale) == 3, "E4M3 inputs need their descales"
        dsc = [float(x) for x in descale]
    else:
        assert descale is None, "descales apply to E4M3 inputs only"
        dsc = [1.0, 1.0, 1.0]
    sk = None
    if sinks is not None:
        sk = np.ascontiguousarray(sinks, dtype=np.float64)
        assert sk.shape == (hq,)
    rc = lib.oracle_decode_paged_scaled(
        dt, _ptr(q), _ptr(k_pool), ks[0], ks[1], ks[2], _ptr(v_pool), vs[0], vs[1], vs[2],
        _ptr(pt_k), _ptr(pt_v), pt_k.shape[1], _ptr(seq_lens), B, sq, hq, hkv, dqk, dv,
        int(page_size), float(scale), int(bool(causal)), int(num_splits), int(window), _ptr(sk),
        dsc[0], dsc[1], dsc[2], n_sel, _ptr(sr), _ptr(o), _ptr(lse), _ptr(o_part),
        _ptr(lse_part), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode_paged rejected its arguments (rc=%d)" % rc)
    if sel_rows is None:
        o = o.reshape(B, sq, hq, dv)
        lse = lse.reshape(B, sq, hq)
    if want_partials:
        return o, lse, o_part, lse_part
    return o, lse


def combine(o_part, lse_part):
    """LSE merge of split partials by definition: o_part [S, rows, Dv], lse_part [S, rows]."""
    lib = _load()
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    S, rows, dv = o_part.shape
    o = np.zeros((rows, dv), np.float64)
    lse = np.zeros(rows, np.float64)
    lib.oracle_combine(_ptr(o_part), _ptr(lse_part), S, rows, dv, _ptr(o), _ptr(lse))
    return o, lse
