"""Seeded synthetic inputs for the SDPA forward path.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path's tests/benchmark and the fp64 oracle
consume what it produces.

Every workload is drawn on the CPU from ``torch.Generator().manual_seed(seed)``
in a fixed order -- lengths, Q, K (or the K pool), V (or the V pool), the K page
permutation, the V page permutation -- with values N(0, 1) in fp32, then rounded
to bf16 (round-to-nearest-even) unless the workload is fp32.

Shapes follow the packed THD layout (token, head, dim; dim innermost) and the
paged pool layout (page, token-in-page, head, dim) of the serving path the
cuDNN Frontend release notes describe (v1.30.0 Release Notes, "New: the
FlashInfer serving path runs on FROST"; v1.31.0 Release Notes, "SDPA: paged KV,
split-KV, and engine selection").
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

CHUNK_ELEMS = 1 << 26  # draw big tensors in pieces to bound host memory


def _randn(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """N(0,1) fp32 draws, rounded to ``dtype``; drawn piecewise along dim 0."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=dtype)
    if out.numel() == 0:
        return out
    row = max(1, out.numel() // max(1, shape[0]))
    step = max(1, CHUNK_ELEMS // row)
    for s in range(0, shape[0], step):
        e = min(shape[0], s + step)
        out[s:e] = torch.randn((e - s,) + shape[1:], generator=g, dtype=torch.float32).to(dtype)
    return out


@dataclass
class ThdCase:
    """Packed THD ragged prefill problem (Q/K/V on the host)."""
    q: torch.Tensor            # [Tq, Hq, Dqk]
    k: torch.Tensor            # [Tk, Hkv, Dqk]
    v: torch.Tensor            # [Tk, Hkv, Dv]
    cu_q: torch.Tensor         # int32 [B+1]
    cu_kv: torch.Tensor        # int32 [B+1]
    lengths_q: List[int]
    lengths_kv: List[int]
    hq: int
    hkv: int
    scale: float
    causal: bool = True
    name: str = ""
    # per-tensor FP8: q / k / v hold uint8 E4M3 codes standing for descale * value
    descale: Optional[Tuple[float, float, float]] = None

    @property
    def batch(self) -> int:
        return len(self.lengths_q)

    @property
    def max_q(self) -> int:
        return max(self.lengths_q) if self.lengths_q else 0

    @property
    def max_kv(self) -> int:
        return max(self.lengths_kv) if self.lengths_kv else 0


@dataclass
class PagedCase:
    """Paged-KV decode problem (Q and the pools on the host)."""
    q: torch.Tensor            # [B, sq, Hq, Dqk]
    k_pool: torch.Tensor       # [P, page, Hkv, Dqk]
    v_pool: torch.Tensor       # [P, page, Hkv, Dv]
    pt_k: torch.Tensor         # int32 [B, table_stride]
    pt_v: torch.Tensor         # int32 [B, table_stride]
    seq_lens: torch.Tensor     # int32 [B]
    page_size: int
    hq: int
    hkv: int
    scale: float
    causal: bool
    num_splits: int
    name: str = ""
    # per-tensor FP8: q / k_pool / v_pool hold uint8 E4M3 codes standing for
    # descale * value; (descale_q, descale_k, descale_v), fp32-representable
    descale: Optional[Tuple[float, float, float]] = None

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def sq(self) -> int:
        return int(self.q.shape[1])

    @property
    def max_kv(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.numel() else 0


def thd_case(seed: int, hq: int, hkv: int, d_qk: int, d_v: Optional[int] = None,
             lengths: Optional[List[int]] = None, batch: int = 0, lo: int = 0, hi: int = 0,
             lengths_kv: Optional[List[int]] = None, dtype: torch.dtype = torch.bfloat16,
             causal: bool = True, scale: Optional[float] = None, name: str = "") -> ThdCase:
    """Ragged THD problem.  Lengths are given, or drawn uniform in [lo, hi]."""
    d_v = d_qk if d_v is None else d_v
    g = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    lengths = [int(x) for x in lengths]
    lengths_kv = lengths if lengths_kv is None else [int(x) for x in lengths_kv]
    tq, tk = sum(lengths), sum(lengths_kv)
    q = _randn(g, (tq, hq, d_qk), dtype)
    k = _randn(g, (tk, hkv, d_qk), dtype)
    v = _randn(g, (tk, hkv, d_v), dtype)
    cu_q = torch.tensor([0] + list(_cumsum(lengths)), dtype=torch.int32)
    cu_kv = torch.tensor([0] + list(_cumsum(lengths_kv)), dtype=torch.int32)
    sc = 1.0 / math.sqrt(d_qk) if scale is None else float(scale)
    return ThdCase(q, k, v, cu_q, cu_kv, lengths, lengths_kv, hq, hkv, sc, causal, name)


def _cumsum(xs):
    acc = 0
    for x in xs:
        acc += x
        yield acc


def paged_case(seed: int, batch: int, sq: int, hq: int, hkv: int, d_qk: int, d_v: int,
               page_size: int, lo: int = 0, hi: int = 0, lengths: Optional[List[int]] = None,
               num_splits: int = 1, causal: bool = True, scale: Optional[float] = None,
               dtype: torch.dtype = torch.bfloat16, poison: bool = False,
               name: str = "") -> PagedCase:
    """Paged decode problem with one shared K pool and one shared V pool.

    The pools hold exactly sum_b ceil(L_b / page) pages, filled N(0,1) in pool
    order.  Logical page p of sequence b (global index gi, sequences in order)
    lives at perm_k[gi] in the K pool and perm_v[gi] in the V pool: two
    independent random permutations.  Table stride = ceil(max L / page).

    poison=True appends one NaN page to each pool, points every unused table
    entry at it, and fills the slots past each sequence's end in its last
    page with NaN (the capacity-tail hazard).  Otherwise unused entries are 0.
    """
    g = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    lengths = [int(x) for x in lengths]
    batch = len(lengths)
    q = _randn(g, (batch, sq, hq, d_qk), dtype)
    pages_b = [(L + page_size - 1) // page_size for L in lengths]
    n_pages = sum(pages_b)
    extra = 1 if poison else 0
    k_pool = _randn(g, (n_pages + extra, page_size, hkv, d_qk), dtype)
    v_pool = _randn(g, (n_pages + extra, page_size, hkv, d_v), dtype)
    perm_k = torch.randperm(n_pages, generator=g) if n_pages else torch.zeros(0, dtype=torch.long)
    perm_v = torch.randperm(n_pages, generator=g) if n_pages else torch.zeros(0, dtype=torch.long)
    table_stride = max(1, max(pages_b) if pages_b else 1)
    fill = n_pages if poison else 0
    pt_k = torch.full((batch, table_stride), fill, dtype=torch.int32)
    pt_v = torch.full((batch, table_stride), fill, dtype=torch.int32)
    gi = 0
    for b, npg in enumerate(pages_b):
        pt_k[b, :npg] = perm_k[gi:gi + npg].to(torch.int32)
        pt_v[b, :npg] = perm_v[gi:gi + npg].to(torch.int32)
        gi += npg
    if poison:
        nan = float("nan")
        k_pool[n_pages] = nan
        v_pool[n_pages] = nan
        for b, L in enumerate(lengths):
            tail = L % page_size
            if tail and pages_b[b]:
                last = pages_b[b] - 1
                k_pool[int(pt_k[b, last]), tail:] = nan
                v_pool[int(pt_v[b, last]), tail:] = nan
    sc = 1.0 / math.sqrt(d_qk) if scale is None else float(scale)
    seq_lens = torch.tensor(lengths, dtype=torch.int32)
    return PagedCase(q, k_pool, v_pool, pt_k, pt_v, seq_lens, page_size, hq, hkv, sc, causal,
                     num_splits, name)



def sink_logits(seed: int, hq: int, special: bool = True) -> torch.Tensor:
    """fp32 [hq] attention-sink logits, N(0.5, 2^2) (the range of learned per-head
    sinks).  special=True makes head 0 -inf (no sink) and head 1 +12 (a sink that
    outweighs most rows' keys)."""
    g = torch.Generator().manual_seed(seed)
    s = torch.randn(hq, generator=g, dtype=torch.float32) * 2.0 + 0.5
    if special and hq > 0:
        s[0] = float("-inf")
    if special and hq > 1:
        s[1] = 12.0
    return s


E4M3_MAX = 448.0  # largest finite OCP E4M3 value


def quantize_e4m3(x: torch.Tensor) -> Tuple[torch.Tensor, float]:
    """Per-tensor FP8 of an fp32 tensor: descale = amax / 448 (rounded to fp32; NaNs
    ignored), codes = x / descale rounded to E4M3 (torch's float8_e4m3fn cast, RNE), as
    uint8.  NaN entries become the NaN code."""
    finite = x[torch.isfinite(x)]
    amax = float(finite.abs().max()) if finite.numel() else 1.0
    descale = float(torch.tensor(max(amax, 1e-30) / E4M3_MAX, dtype=torch.float32))
    codes = (x / descale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, descale


def fp8_thd_case(seed: int, hq: int, hkv: int, d: int, lengths: Optional[List[int]] = None,
                 batch: int = 0, lo: int = 0, hi: int = 0,
                 lengths_kv: Optional[List[int]] = None, causal: bool = True,
                 scale: Optional[float] = None, name: str = "") -> ThdCase:
    """THD prefill problem in per-tensor FP8 E4M3: the fp32 problem thd_case draws for the
    same arguments, Q, K and V each quantized on its own (quantize_e4m3)."""
    case = thd_case(seed, hq=hq, hkv=hkv, d_qk=d, lengths=lengths, batch=batch, lo=lo, hi=hi,
                    lengths_kv=lengths_kv, dtype=torch.float32, causal=causal, scale=scale,
                    name=name)
    q8, dq = quantize_e4m3(case.q)
    k8, dk = quantize_e4m3(case.k)
    v8, dv = quantize_e4m3(case.v)
    return dataclasses.replace(case, q=q8, k=k8, v=v8, descale=(dq, dk, dv))


def fp8_paged_case(seed: int, batch: int, sq: int, hq: int, hkv: int, d: int, page_size: int,
                   lo: int = 0, hi: int = 0, lengths: Optional[List[int]] = None,
                   num_splits: int = 1, causal: bool = True, scale: Optional[float] = None,
                   poison: bool = False, name: str = "",
                   d_v: Optional[int] = None) -> PagedCase:
    """Paged decode problem in per-tensor FP8 E4M3: the fp32 problem paged_case draws for
    the same arguments (d_v defaults to d), each of Q, the K pool and the V pool quantized
    on its own (quantize_e4m3).  Poisoned slots hold the NaN code."""
    pc = paged_case(seed, batch, sq, hq, hkv, d, d if d_v is None else d_v, page_size,
                    lo=lo, hi=hi, lengths=lengths,
                    num_splits=num_splits, causal=causal, scale=scale, dtype=torch.float32,
                    poison=poison, name=name)
    q8, dq = quantize_e4m3(pc.q)
    k8, dk = quantize_e4m3(pc.k_pool)
    v8, dv = quantize_e4m3(pc.v_pool)
    return dataclasses.replace(pc, q=q8, k_pool=k8, v_pool=v8, descale=(dq, dk, dv))

# ---- the five workloads -----------------------------------------------------

SEED_BASE = 1000      # seed 1000 + k for workload k
SEED_ALT = 1100       # a second parity seed, 1100 + k


def tiny_fp32(seed: int = SEED_BASE + 1) -> ThdCase:
    """Tiny dense causal fp32 THD: seqlens {5, 17}, 2 Q heads / 1 KV head, D=64."""
    return thd_case(seed, hq=2, hkv=1, d_qk=64, lengths=[5, 17], dtype=torch.float32,
                    name="thd_fp32_tiny_5_17_h2x1_d64")


def thd_prefill_d128(seed: int = SEED_BASE + 2, batch: int = 8, lo: int = 128,
                     hi: int = 4096) -> ThdCase:
    """Packed THD ragged causal prefill bf16: 8 sequences U[128, 4096], 32/8 heads, D=128."""
    return thd_case(seed, hq=32, hkv=8, d_qk=128, batch=batch, lo=lo, hi=hi,
                    name="thd_prefill_bf16_b%d_%d-%d_h32x8_d128" % (batch, lo, hi))


def paged_decode_d128(seed: int = SEED_BASE + 3, batch: int = 64, lo: int = 512,
                      hi: int = 32768, poison: bool = False) -> PagedCase:
    """Paged decode bf16: batch 64, 1 token, 32/8 heads, D=128, page 64, L U[512, 32768], 8 splits."""
    return paged_case(seed, batch=batch, sq=1, hq=32, hkv=8, d_qk=128, d_v=128, page_size=64,
                      lo=lo, hi=hi, num_splits=8, causal=True, poison=poison,
                      name="paged_decode_bf16_b%d_h32x8_d128_p64_%d-%d_s8" % (batch, lo, hi))


def paged_decode_d128_fp8(seed: int = SEED_BASE + 3, batch: int = 64, lo: int = 512,
                          hi: int = 32768, poison: bool = False) -> PagedCase:
    """The paged decode workload in per-tensor FP8 E4M3: the same draws as paged_decode_d128
    (before bf16 rounding), Q / K pool / V pool each quantized with its own descale."""
    return fp8_paged_case(seed, batch=batch, sq=1, hq=32, hkv=8, d=128, page_size=64, lo=lo,
                          hi=hi, num_splits=8, causal=True, poison=poison,
                          name="paged_decode_fp8_b%d_h32x8_d128_p64_%d-%d_s8" % (batch, lo, hi))


def dense_prefill_d256(seed: int = SEED_BASE + 4, seqlen: int = 8192) -> ThdCase:
    """Dense causal prefill bf16 D=256: batch 2 x 8192, 24 Q / 2 KV heads (GQA 12)."""
    return thd_case(seed, hq=24, hkv=2, d_qk=256, lengths=[seqlen, seqlen],
                    name="dense_prefill_bf16_2x%d_h24x2_d256" % seqlen)


def ragged_prefill_d256(seed: int = SEED_BASE + 4, lengths=(8192, 3000)) -> ThdCase:
    """The ragged variant of the D=256 workload: seqlens {8192, 3000}, padded LSE."""
    return thd_case(seed, hq=24, hkv=2, d_qk=256, lengths=list(lengths),
                    name="ragged_prefill_bf16_%s_h24x2_d256" % "_".join(map(str, lengths)))


def mla_decode(seed: int = SEED_BASE + 5, batch: int = 32, lo: int = 4096, hi: int = 16384,
               poison: bool = False) -> PagedCase:
    """Absorbed-MLA-shaped paged decode bf16: Dqk 576, Dv 512, 128/1 heads, 2 query tokens."""
    return paged_case(seed, batch=batch, sq=2, hq=128, hkv=1, d_qk=576, d_v=512, page_size=64,
                      lo=lo, hi=hi, num_splits=16, causal=True, poison=poison,
                      name="mla_decode_bf16_b%d_sq2_h128x1_d576-512_p64_%d-%d_s16"
                      % (batch, lo, hi))


def window_prefill_d64(seed: int = SEED_BASE + 9, batch: int = 8, lo: int = 128,
                      hi: int = 4096) -> ThdCase:
    """THD ragged causal prefill bf16 with the shape of sliding-window layers that carry
    sinks: 8 sequences U[128, 4096], 64/8 heads, D=64 (run with a 128-key window)."""
    return thd_case(seed, hq=64, hkv=8, d_qk=64, batch=batch, lo=lo, hi=hi,
                    name="thd_prefill_bf16_b%d_%d-%d_h64x8_d64" % (batch, lo, hi))


def chunked_prefill_paged(seed: int = SEED_BASE + 6, batch: int = 2, chunk: int = 1024,
                          lo: int = 32768, hi: int = 65536, num_splits: int = 4,
                          poison: bool = False) -> PagedCase:
    """Chunked prefill over the paged cache bf16: 1024-token query chunks against caches of
    U[32768, 65536] tokens (the chunk is the cache's last tokens), 32/8 heads, D=128, page 64,
    bottom-right causal, 4 splits."""
    return paged_case(seed, batch=batch, sq=chunk, hq=32, hkv=8, d_qk=128, d_v=128, page_size=64,
                      lo=lo, hi=hi, num_splits=num_splits, causal=True, poison=poison,
                      name="chunked_prefill_paged_bf16_b%d_c%d_h32x8_d128_p64_%d-%d_s%d"
                      % (batch, chunk, lo, hi, num_splits))


def context_chunk(chunk: int, cache: int, seed: int = SEED_BASE + 10, batch: int = 2,
                  num_splits: int = 0, poison: bool = False) -> PagedCase:
    """The context phase of serving: a query chunk of `chunk` tokens at the end of each of
    `batch` caches of exactly `cache` tokens, 32/8 heads, D=128, page 64, bottom-right causal
    (512- and 1024-token chunks against 64k and 128k caches).  Splits default to enough
    (chunk, head-group, split) work items to cover the CUs twice: 4 for 512-token chunks,
    2 for 1024."""
    splits = num_splits or max(1, 2048 // chunk)
    return paged_case(seed + chunk + cache, batch=batch, sq=chunk, hq=32, hkv=8, d_qk=128,
                      d_v=128, page_size=64, lengths=[cache] * batch, num_splits=splits,
                      causal=True, poison=poison,
                      name="context_chunk_bf16_b%d_c%d_h32x8_d128_p64_%d_s%d"
                      % (batch, chunk, cache, splits))


def mtp_decode_d128(seed: int = SEED_BASE + 7, batch: int = 4, cache: int = 131072,
                    q_tokens: int = 4, num_splits: int = 32) -> PagedCase:
    """Multi-token decode bf16 against 128k caches: batch 4, q_tokens (1 + MTP) query tokens
    at the end of each cache, 32/8 heads, D=128, page 64, 32 splits."""
    return paged_case(seed, batch=batch, sq=q_tokens, hq=32, hkv=8, d_qk=128, d_v=128,
                      page_size=64, lengths=[cache] * batch, num_splits=num_splits, causal=True,
                      name="mtp_decode_bf16_b%d_q%d_h32x8_d128_p64_%d_s%d"
                      % (batch, q_tokens, cache, num_splits))


def mla_decode_fp8(seed: int = SEED_BASE + 5, batch: int = 32, lo: int = 4096,
                   hi: int = 16384) -> PagedCase:
    """The MLA-shaped decode in per-tensor FP8 E4M3: the same draws as mla_decode (before
    bf16 rounding), Q / K pool / V pool each quantized with its own descale."""
    return fp8_paged_case(seed, batch=batch, sq=2, hq=128, hkv=1, d=576, page_size=64, lo=lo,
                          hi=hi, num_splits=16, causal=True, d_v=512,
                          name="mla_decode_fp8_b%d_sq2_h128x1_d576-512_p64_%d-%d_s16"
                          % (batch, lo, hi))


def mla_decode_aliased(seed: int = SEED_BASE + 8, batch: int = 32, lo: int = 4096,
                       hi: int = 16384) -> PagedCase:
    """The MLA-shaped decode over an absorbed-MLA cache: one 576-wide pool and one page table,
    V = the first 512 columns of each K row (a strided view of the K pool)."""
    pc = paged_case(seed, batch=batch, sq=2, hq=128, hkv=1, d_qk=576, d_v=576, page_size=64,
                    lo=lo, hi=hi, num_splits=16, causal=True,
                    name="mla_decode_aliased_bf16_b%d_sq2_h128x1_d576-512_p64_%d-%d_s16"
                    % (batch, lo, hi))
    return dataclasses.replace(pc, v_pool=pc.k_pool[..., :512], pt_v=pc.pt_k)


def thd_with_capacity(case: ThdCase, extra_rows: int, fill: float = float("nan")):
    """Copies of Q/K/V with ``extra_rows`` unwritten capacity rows appended (NaN by default)."""
    def pad(t):
        tail = torch.full((extra_rows,) + tuple(t.shape[1:]), fill, dtype=t.dtype)
        return torch.cat([t, tail], 0)
    return pad(case.q), pad(case.k), pad(case.v)


def bf16_bits(t: torch.Tensor):
    """Raw uint16 bit patterns of a bf16 tensor, as numpy (no copy if contiguous)."""
    import numpy as np
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def host_array(t: torch.Tensor):
    """numpy view of a host tensor in the oracle's input format (uint16 bf16 bits or float32)."""
    if t.dtype == torch.bfloat16:
        import numpy as np
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()  # float32, or uint8 E4M3 codes
