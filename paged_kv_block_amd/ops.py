"""Thin torch-facing binding of libpkb.so.

Argument marshalling only: tensors become device pointers and strides, host
metadata becomes int32 arrays, and every step of the attention path runs in the
library's HIP kernels.  Function names follow the C ABI (include/pkb.h); the
convenience functions at the bottom mirror the keyword signatures of the
FlashInfer pages they implement.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

from . import _lib as C
from ._lib import Bad, BsaPlan, BsaStaticArgs, PrefillPlan, PrefillStaticArgs, check, lib

_DTYPE = {torch.bfloat16: C.PKB_BF16, torch.float32: C.PKB_FP32}
_MASK = {"dense": C.PKB_MASK_DENSE, "causal": C.PKB_MASK_CAUSAL}


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def num_cus(device=None) -> int:
    return torch.cuda.get_device_properties(device or torch.cuda.current_device()).multi_processor_count


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _host_i32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu")
        if x.dtype != torch.int32:
            x = x.to(torch.int32)
        return np.ascontiguousarray(x.numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _hp(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _scale(x) -> float:
    """Softmax scale for the C ABI: None becomes NaN, the library's sentinel for
    the default 1/sqrt(D); any given value is passed through unchanged (the
    library rejects values that are not finite and positive)."""
    return math.nan if x is None else float(x)


def _mask(mask_type: str) -> int:
    try:
        return _MASK[mask_type]
    except KeyError:
        raise ValueError(f"mask_type must be 'dense' or 'causal', not {mask_type!r}") from None


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev_i32(t: torch.Tensor, name: str):
    _need(isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.int32 and t.is_contiguous(),
          f"{name} must be a contiguous int32 CUDA tensor")


def split_kv_cache(paged_kv_cache: Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]):
    """(k_ptr, v_ptr, page_stride, head_stride, P, Hkv, ps, D, dtype) from either
    a combined [P, 2, Hkv, ps, D] cache or a (K, V) tuple of [P, Hkv, ps, D]."""
    if isinstance(paged_kv_cache, (tuple, list)):
        k, v = paged_kv_cache
        _need(k.shape == v.shape and k.dim() == 4, "K and V pools must both be [P, Hkv, ps, D]")
        _need(k.stride() == v.stride() and k.stride(3) == 1 and k.stride(2) == k.shape[3],
              "K/V pools need token stride D and unit element stride")
        P, Hkv, ps, D = k.shape
        return k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), P, Hkv, ps, D, k.dtype, k.device
    c = paged_kv_cache
    _need(c.dim() == 5 and c.shape[1] == 2, "combined cache must be [P, 2, Hkv, ps, D]")
    _need(c.stride(4) == 1 and c.stride(3) == c.shape[4], "combined cache needs contiguous rows")
    P, _, Hkv, ps, D = c.shape
    return (c.data_ptr(), c[:, 1].data_ptr(), c.stride(0), c.stride(2), P, Hkv, ps, D, c.dtype,
            c.device)


# =============================================================================
# Block-sparse
# =============================================================================

def bsa_plan(B, Sq, Hq, Hkv, D, num_pages, page_size, q_block_size, kv_block_size,
             max_seq_len_kv, mask_type=C.PKB_MASK_DENSE, window_left=-1,
             qkv_dtype=C.PKB_BF16, out_dtype=C.PKB_BF16, num_cus_=None) -> BsaPlan:
    a = BsaStaticArgs(B, Sq, Hq, Hkv, D, num_pages, page_size, q_block_size, kv_block_size,
                      max_seq_len_kv, mask_type, window_left, qkv_dtype, out_dtype,
                      num_cus_ if num_cus_ is not None else num_cus())
    plan = BsaPlan()
    check(lib().bsa_plan(ctypes.byref(a), ctypes.byref(plan)), "bsa_plan")
    return plan


def bsa_validate(plan: BsaPlan, paged_kv_indptr, paged_kv_indices, block_indptr, block_indices,
                 seq_lens_kv, raise_on_error=True):
    """Host validation of live metadata (copies device tensors to the host)."""
    ip, ix = _host_i32(paged_kv_indptr), _host_i32(paged_kv_indices)
    bip, bix = _host_i32(block_indptr), _host_i32(block_indices)
    sl = _host_i32(seq_lens_kv)
    bad = Bad()
    st = lib().bsa_validate(ctypes.byref(plan), _hp(ip), _hp(ix), ix.size, _hp(bip), _hp(bix),
                            bix.size, _hp(sl), ctypes.byref(bad))
    if raise_on_error:
        check(st, "bsa_validate", bad)
    return st, bad.field, bad.index


def bsa_run(plan: BsaPlan, q, k_ptr, v_ptr, kv_page_stride, kv_head_stride, paged_kv_indptr,
            paged_kv_indices, block_indptr, block_indices, seq_lens_kv, kv_valid_bits, sm_scale,
            out, lse=None, stream=None):
    """Trusted launch (no host reads of live metadata)."""
    st = lib().bsa_run(ctypes.byref(plan), _ptr(q), k_ptr, v_ptr, kv_page_stride, kv_head_stride,
                       _ptr(paged_kv_indptr), _ptr(paged_kv_indices), _ptr(block_indptr),
                       _ptr(block_indices), _ptr(seq_lens_kv), _ptr(kv_valid_bits),
                       _scale(sm_scale), _ptr(out), _ptr(lse),
                       stream if stream is not None else _stream(q.device))
    check(st, "bsa_run")


class BlockSparsePagedWrapper:
    """Plan once from static capacities (outside any graph capture), then call
    ``run`` with live tensors any number of times (capturable: ``run`` only
    enqueues kernels)."""

    def __init__(self, B, Sq, Hq, Hkv, D, num_pages, page_size, q_block_size, kv_block_size,
                 max_seq_len_kv, mask_type="dense", window_left=-1, out_dtype=torch.bfloat16,
                 device=None):
        self.plan = bsa_plan(B, Sq, Hq, Hkv, D, num_pages, page_size, q_block_size,
                             kv_block_size, max_seq_len_kv,
                             _mask(mask_type), window_left, C.PKB_BF16, _DTYPE[out_dtype],
                             num_cus(device))
        self.out_dtype = out_dtype

    def run(self, q, paged_kv_cache, paged_kv_indptr, paged_kv_indices, block_indptr,
            block_indices, seq_lens_kv, kv_valid_bits=None, sm_scale=None, out=None, lse=None):
        kp, vp, ps_, hs_, P, Hkv, ps, D, dt, dev = split_kv_cache(paged_kv_cache)
        pl = self.plan
        _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous(),
              "q must be a contiguous bf16 CUDA tensor")
        _need(tuple(q.shape) == (pl.a.B, pl.a.Sq, pl.a.Hq, pl.a.D), "q shape does not match the plan")
        _need(dt == torch.bfloat16 and (P, Hkv, ps, D) == (pl.a.num_pages, pl.a.Hkv, pl.a.page_size, pl.a.D),
              "KV cache does not match the plan")
        for t, n in ((paged_kv_indptr, "paged_kv_indptr"), (paged_kv_indices, "paged_kv_indices"),
                     (block_indptr, "block_indptr"), (block_indices, "block_indices"),
                     (seq_lens_kv, "seq_lens_kv")):
            _dev_i32(t, n)
        _need(tuple(block_indptr.shape) == (pl.a.B, pl.a.Hkv, pl.num_q_blocks + 1),
              "block_indptr must be [B, Hkv, ceil(Sq/q_block_size)+1]")
        if kv_valid_bits is not None:
            _need(kv_valid_bits.is_cuda and kv_valid_bits.dtype in (torch.int32, torch.uint32)
                  and tuple(kv_valid_bits.shape) == (pl.a.B, pl.valid_words)
                  and kv_valid_bits.is_contiguous(),
                  "kv_valid_bits must be uint32 [B, ceil(max_seq_len_kv/32)]")
        if out is None:
            out = torch.empty(q.shape, dtype=self.out_dtype, device=q.device)
        _need(out.is_contiguous() and out.shape == q.shape and out.dtype == self.out_dtype,
              "out must be contiguous with q's shape and the planned dtype")
        if lse is not None:
            _need(lse.dtype == torch.float32 and lse.is_contiguous()
                  and lse.numel() == pl.a.B * pl.a.Sq * pl.a.Hq, "lse must be fp32 [B*Sq, Hq]")
        bsa_run(pl, q, kp, vp, ps_, hs_, paged_kv_indptr, paged_kv_indices, block_indptr,
                block_indices, seq_lens_kv, kv_valid_bits, sm_scale, out, lse)
        return out


def block_sparse_attention_with_paged_kv_cache(
        q, paged_kv_cache, paged_kv_indptr, paged_kv_indices, block_indptr, block_indices,
        q_block_size, kv_block_size, *, max_seq_len_kv, seq_lens_kv, kv_valid_bits=None,
        mask_type="dense", sm_scale=None, out=None, window_left=-1, lse=None):
    """Validate live metadata on the host, plan from capacities, run.

    Mirrors the page "block_sparse_attention_with_paged_kv_cache" (plus an
    optional ``lse`` output and ``window_left``); not capturable because of the
    synchronous validation.
    """
    _, _, _, _, P, Hkv, ps, D, _, dev = split_kv_cache(paged_kv_cache)
    B, Sq, Hq, _ = q.shape
    out_dtype = out.dtype if out is not None else q.dtype
    w = BlockSparsePagedWrapper(B, Sq, Hq, Hkv, D, P, ps, q_block_size, kv_block_size,
                                max_seq_len_kv, mask_type, window_left, out_dtype, dev)
    bsa_validate(w.plan, paged_kv_indptr, paged_kv_indices, block_indptr, block_indices,
                 seq_lens_kv)
    return w.run(q, paged_kv_cache, paged_kv_indptr, paged_kv_indices, block_indptr,
                 block_indices, seq_lens_kv, kv_valid_bits, sm_scale, out, lse)


# =============================================================================
# Prefill
# =============================================================================

def _prefill_args(B, Hq, Hkv, D, num_pages, page_size, total_q, width, mask_type, window_left,
                  out_dtype, ncu):
    return PrefillStaticArgs(B, Hq, Hkv, D, num_pages, page_size, total_q, width,
                             _mask(mask_type), window_left, C.PKB_BF16, _DTYPE[out_dtype], ncu)


def paged_prefill_validate(args: PrefillStaticArgs, qo_indptr, seq_lens_kv, block_tables,
                           raise_on_error=True):
    qo, sl, bt = _host_i32(qo_indptr), _host_i32(seq_lens_kv), _host_i32(block_tables)
    bad = Bad()
    st = lib().paged_prefill_validate(ctypes.byref(args), _hp(qo), _hp(sl), _hp(bt),
                                      bt.shape[1] if bt.ndim == 2 else args.block_table_width,
                                      ctypes.byref(bad))
    if raise_on_error:
        check(st, "paged_prefill_validate", bad)
    return st, bad.field, bad.index


def paged_prefill_plan(args: PrefillStaticArgs, qo_indptr, seq_lens_kv):
    """Host plan: returns (plan, worklist int32 numpy [n_work, 2])."""
    qo, sl = _host_i32(qo_indptr), _host_i32(seq_lens_kv)
    plan = PrefillPlan()
    n = ctypes.c_int64(0)
    st = lib().paged_prefill_plan(ctypes.byref(args), _hp(qo), _hp(sl), ctypes.byref(plan), None,
                                  0, ctypes.byref(n))
    if st != C.PKB_ERR_WORKSPACE or n.value == 0:
        check(st, "paged_prefill_plan")
    wl = np.zeros((max(n.value, 1), 2), dtype=np.int32)
    check(lib().paged_prefill_plan(ctypes.byref(args), _hp(qo), _hp(sl), ctypes.byref(plan),
                                   _hp(wl), n.value, ctypes.byref(n)), "paged_prefill_plan")
    return plan, wl[:n.value]


def paged_prefill_plan_capacity(args: PrefillStaticArgs, max_qlen):
    """Capacity plan (reads no request metadata): (plan, worklist int32 [n_work, 2])."""
    plan = PrefillPlan()
    n = ctypes.c_int64(0)
    st = lib().paged_prefill_plan_capacity(ctypes.byref(args), int(max_qlen), ctypes.byref(plan),
                                           None, 0, ctypes.byref(n))
    if st != C.PKB_ERR_WORKSPACE:
        check(st, "paged_prefill_plan_capacity")
    wl = np.zeros((n.value, 2), dtype=np.int32)
    check(lib().paged_prefill_plan_capacity(ctypes.byref(args), int(max_qlen), ctypes.byref(plan),
                                            _hp(wl), n.value, ctypes.byref(n)),
          "paged_prefill_plan_capacity")
    return plan, wl


def paged_prefill_run(plan: PrefillPlan, worklist_d, q, k_cache, v_cache, qo_indptr,
                      block_tables, seq_lens_kv, sm_scale=None, output_scale=1.0, out=None,
                      lse=None, stream=None):
    st = lib().paged_prefill_run(ctypes.byref(plan), _ptr(worklist_d), _ptr(q), _ptr(k_cache),
                                 _ptr(v_cache), k_cache.stride(0), k_cache.stride(1),
                                 _ptr(qo_indptr), _ptr(block_tables), block_tables.stride(0),
                                 _ptr(seq_lens_kv), _scale(sm_scale), float(output_scale),
                                 _ptr(out), _ptr(lse),
                                 stream if stream is not None else _stream(q.device))
    check(st, "paged_prefill_run")


class BatchPrefillPagedWrapper:
    """Plan from host copies of qo_indptr / seq_lens (exact bounds), then ``run``
    binds the device tensors (capturable)."""

    def __init__(self, qo_indptr, seq_lens_kv, Hq, Hkv, D, num_pages, page_size,
                 block_table_width, mask_type="dense", window_left=-1, out_dtype=torch.bfloat16,
                 device=None, validate_tables=None):
        qo = _host_i32(qo_indptr)
        B = qo.size - 1
        self.args = _prefill_args(B, Hq, Hkv, D, num_pages, page_size, int(qo[-1]),
                                  block_table_width, mask_type, window_left, out_dtype,
                                  num_cus(device))
        if validate_tables is not None:
            paged_prefill_validate(self.args, qo, seq_lens_kv, validate_tables)
        self.plan, wl = paged_prefill_plan(self.args, qo, seq_lens_kv)
        dev = device if device is not None else torch.device("cuda")
        self.worklist = torch.from_numpy(wl.copy()).to(dev)
        self.out_dtype = out_dtype

    @classmethod
    def for_capacity(cls, B, max_qlen, total_q, Hq, Hkv, D, num_pages, page_size,
                     block_table_width, mask_type="dense", window_left=-1,
                     out_dtype=torch.bfloat16, device=None):
        """Plan from static bounds only, for a ``run`` captured once in a graph and
        replayed while qo_indptr / seq_lens / block_tables change (every qlen at
        most max_qlen, qo_indptr[B] at most total_q)."""
        self = cls.__new__(cls)
        self.args = _prefill_args(B, Hq, Hkv, D, num_pages, page_size, total_q,
                                  block_table_width, mask_type, window_left, out_dtype,
                                  num_cus(device))
        self.plan, wl = paged_prefill_plan_capacity(self.args, max_qlen)
        dev = device if device is not None else torch.device("cuda")
        self.worklist = torch.from_numpy(wl.copy()).to(dev)
        self.out_dtype = out_dtype
        return self

    def run(self, q, k_cache, v_cache, qo_indptr, block_tables, seq_lens_kv, sm_scale=None,
            output_scale=1.0, out=None, lse=None):
        a = self.args
        _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous()
              and tuple(q.shape) == (a.total_q, a.Hq, a.D), "q must be bf16 [total_q, Hq, D]")
        for t in (k_cache, v_cache):
            _need(t.dtype == torch.bfloat16 and tuple(t.shape) == (a.num_pages, a.Hkv, a.page_size, a.D)
                  and t.stride(3) == 1 and t.stride(2) == a.D, "K/V pools must be HND [P, Hkv, ps, D]")
        _need(k_cache.stride() == v_cache.stride(), "K and V pools must share strides")
        for t, n in ((qo_indptr, "qo_indptr"), (seq_lens_kv, "seq_lens_kv")):
            _dev_i32(t, n)
        _need(block_tables.is_cuda and block_tables.dtype == torch.int32 and block_tables.dim() == 2
              and block_tables.stride(1) == 1 and block_tables.shape[1] >= a.block_table_width,
              "block_tables must be int32 [B, C] with unit column stride")
        if out is None:
            out = torch.empty(q.shape, dtype=self.out_dtype, device=q.device)
        _need(out.is_contiguous() and out.shape == q.shape and out.dtype == self.out_dtype,
              "out must be contiguous [total_q, Hq, D] of the planned dtype")
        if lse is not None:
            _need(lse.dtype == torch.float32 and lse.numel() == a.total_q * a.Hq and lse.is_contiguous(),
                  "lse must be fp32 [total_q, Hq]")
        paged_prefill_run(self.plan, self.worklist, q, k_cache, v_cache, qo_indptr, block_tables,
                          seq_lens_kv, sm_scale, output_scale, out, lse)
        return out


def batch_prefill_with_paged_kv_cache(q, k_cache, v_cache, qo_indptr, block_tables, seq_lens_kv,
                                      *, page_size=32, kv_layout="HND", mask_type="dense",
                                      window_left=-1, sm_scale=None, output_scale=1.0,
                                      out_dtype=None, out=None, lse=None):
    """Mirrors the page "batch_prefill_with_paged_kv_cache": reads request
    metadata on the host for exact plan bounds (not capturable)."""
    _need(kv_layout == "HND", "only the HND layout is supported")
    _need(k_cache.shape[2] == page_size, "page_size does not match the K/V pools")
    od = out_dtype or (out.dtype if out is not None else q.dtype)
    w = BatchPrefillPagedWrapper(qo_indptr, seq_lens_kv, q.shape[1], k_cache.shape[1], q.shape[2],
                                 k_cache.shape[0], page_size, block_tables.shape[1], mask_type,
                                 window_left, od, q.device, validate_tables=block_tables)
    return w.run(q, k_cache, v_cache, qo_indptr, block_tables, seq_lens_kv, sm_scale,
                 output_scale, out, lse)


# =============================================================================
# Decode
# =============================================================================

def paged_decode_workspace_size(B, Hq, Hkv, D, max_seq_len, page_size, num_cus_=None):
    nb = ctypes.c_size_t(0)
    S = ctypes.c_int32(0)
    sl = ctypes.c_int32(0)
    check(lib().paged_decode_workspace_size(B, Hq, Hkv, D, max_seq_len, page_size,
                                            num_cus_ if num_cus_ is not None else num_cus(),
                                            ctypes.byref(nb), ctypes.byref(S), ctypes.byref(sl)),
          "paged_decode_workspace_size")
    return nb.value, S.value, sl.value


def paged_decode_validate(B, num_pages, page_size, max_seq_len, paged_kv_indptr, paged_kv_indices,
                          seq_lens, raise_on_error=True):
    ip, ix, sl = _host_i32(paged_kv_indptr), _host_i32(paged_kv_indices), _host_i32(seq_lens)
    bad = Bad()
    st = lib().paged_decode_validate(B, num_pages, page_size, max_seq_len, _hp(ip), _hp(ix),
                                     ix.size, _hp(sl), ctypes.byref(bad))
    if raise_on_error:
        check(st, "paged_decode_validate", bad)
    return st, bad.field, bad.index


def paged_decode_run(query, kv_cache, paged_kv_indptr, paged_kv_indices, seq_lens, max_seq_len,
                     workspace, *, mask_type="dense", window_left=-1, bmm1_scale=None,
                     bmm2_scale=1.0, out=None, lse=None, num_cus_=None, stream=None):
    kp, vp, pst, hst, P, Hkv, ps, D, dt, dev = split_kv_cache(kv_cache)
    B, Hq, Dq = query.shape
    _need(Dq == D and dt == torch.bfloat16 and query.dtype == torch.bfloat16 and query.is_contiguous(),
          "query must be contiguous bf16 [B, Hq, D] matching the cache")
    for t, n in ((paged_kv_indptr, "paged_kv_indptr"), (paged_kv_indices, "paged_kv_indices"),
                 (seq_lens, "seq_lens")):
        _dev_i32(t, n)
    if out is None:
        out = torch.empty_like(query)
    _need(out.is_contiguous() and out.shape == query.shape and out.dtype in _DTYPE,
          "out must be contiguous [B, Hq, D] bf16 or fp32")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.numel() == B * Hq and lse.is_contiguous(),
              "lse must be fp32 [B, Hq]")
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().paged_decode_run(_ptr(query), kp, vp, pst, hst, _ptr(paged_kv_indptr),
                                _ptr(paged_kv_indices), _ptr(seq_lens), B, Hq, Hkv, D, P, ps,
                                int(max_seq_len),
                                _mask(mask_type), int(window_left), _scale(bmm1_scale),
                                float(bmm2_scale),
                                _DTYPE[out.dtype], _ptr(out), _ptr(lse), ws_ptr, ws_bytes,
                                num_cus_ if num_cus_ is not None else num_cus(query.device),
                                stream if stream is not None else _stream(query.device))
    check(st, "paged_decode_run")
    return out


def paged_decode_run_noalloc(query, kv_cache, paged_kv_indptr, paged_kv_indices, seq_lens,
                             max_seq_len, *, mask_type="dense", window_left=-1, bmm1_scale=None,
                             bmm2_scale=1.0, out=None, lse=None, num_cus_=None, stream=None):
    """paged_decode_run without a caller workspace: split partials go to the
    library's fixed per-device scratch (PKB_DECODE_SCRATCH_BYTES).  Calls that
    overlap on one GPU race on that scratch."""
    kp, vp, pst, hst, P, Hkv, ps, D, dt, dev = split_kv_cache(kv_cache)
    B, Hq, Dq = query.shape
    _need(Dq == D and dt == torch.bfloat16 and query.dtype == torch.bfloat16 and query.is_contiguous(),
          "query must be contiguous bf16 [B, Hq, D] matching the cache")
    for t, n in ((paged_kv_indptr, "paged_kv_indptr"), (paged_kv_indices, "paged_kv_indices"),
                 (seq_lens, "seq_lens")):
        _dev_i32(t, n)
    _need(out is not None and out.is_contiguous() and out.shape == query.shape
          and out.dtype in _DTYPE, "out must be a contiguous [B, Hq, D] bf16 or fp32 tensor")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.numel() == B * Hq and lse.is_contiguous(),
              "lse must be fp32 [B, Hq]")
    st = lib().paged_decode_run_noalloc(_ptr(query), kp, vp, pst, hst, _ptr(paged_kv_indptr),
                                        _ptr(paged_kv_indices), _ptr(seq_lens), B, Hq, Hkv, D, P,
                                        ps, int(max_seq_len), _mask(mask_type), int(window_left),
                                        _scale(bmm1_scale), float(bmm2_scale), _DTYPE[out.dtype],
                                        _ptr(out), _ptr(lse),
                                        num_cus_ if num_cus_ is not None else num_cus(query.device),
                                        stream if stream is not None else _stream(query.device))
    check(st, "paged_decode_run_noalloc")
    return out


def batch_decode_with_paged_kv_cache(query, kv_cache, workspace_buffer, paged_kv_indptr,
                                     paged_kv_indices, seq_lens, max_seq_len, *, bmm1_scale=None,
                                     bmm2_scale=1.0, out=None, out_dtype=None, mask_type="dense",
                                     window_left=-1, kv_layout="HND", lse=None):
    """Mirrors the page "prims_ts_batch_decode_with_kv_cache" for seq_len_q = 1.
    No host read of device metadata; ``workspace_buffer`` is caller scratch of at
    least ``paged_decode_workspace_size(...)`` bytes."""
    _need(kv_layout == "HND", "only the HND layout is supported")
    if out is None:
        out = torch.empty(query.shape, dtype=out_dtype or query.dtype, device=query.device)
    return paged_decode_run(query, kv_cache, paged_kv_indptr, paged_kv_indices, seq_lens,
                            max_seq_len, workspace_buffer, mask_type=mask_type,
                            window_left=window_left, bmm1_scale=bmm1_scale,
                            bmm2_scale=bmm2_scale, out=out, lse=lse)


# =============================================================================
# Multi-token decode (fixed seq_len_q or packed qo_indptr)
# =============================================================================

def paged_decode_q_workspace_size(B, max_q, Hq, Hkv, D, max_seq_len, page_size, num_cus_=None):
    nb = ctypes.c_size_t(0)
    S = ctypes.c_int32(0)
    sl = ctypes.c_int32(0)
    check(lib().paged_decode_q_workspace_size(B, max_q, Hq, Hkv, D, max_seq_len, page_size,
                                              num_cus_ if num_cus_ is not None else num_cus(),
                                              ctypes.byref(nb), ctypes.byref(S),
                                              ctypes.byref(sl)),
          "paged_decode_q_workspace_size")
    return nb.value, S.value, sl.value


def paged_decode_q_validate(B, num_pages, page_size, max_seq_len, paged_kv_indptr,
                            paged_kv_indices, seq_lens, *, qo_indptr=None, total_q=0,
                            seq_len_q=0, max_seq_len_q=0, mask_type="causal",
                            raise_on_error=True):
    ip, ix, sl = _host_i32(paged_kv_indptr), _host_i32(paged_kv_indices), _host_i32(seq_lens)
    qo = None if qo_indptr is None else _host_i32(qo_indptr)
    bad = Bad()
    st = lib().paged_decode_q_validate(B, num_pages, page_size, max_seq_len, _hp(ip), _hp(ix),
                                       ix.size, _hp(sl), _hp(qo), int(total_q), int(seq_len_q),
                                       int(max_seq_len_q), _mask(mask_type), ctypes.byref(bad))
    if raise_on_error:
        check(st, "paged_decode_q_validate", bad)
    return st, bad.field, bad.index


def paged_decode_q_run(query, kv_cache, paged_kv_indptr, paged_kv_indices, seq_lens, max_seq_len,
                       workspace, *, qo_indptr=None, max_seq_len_q=0, mask_type="causal",
                       window_left=-1, bmm1_scale=None, bmm2_scale=1.0, out=None, lse=None,
                       num_cus_=None, stream=None):
    """query [B, Sq, Hq, D] (fixed) or [total_q, Hq, D] with device ``qo_indptr``."""
    kp, vp, pst, hst, P, Hkv, ps, D, dt, dev = split_kv_cache(kv_cache)
    _need(query.dtype == torch.bfloat16 and dt == torch.bfloat16 and query.is_contiguous(),
          "query must be contiguous bf16 matching the cache")
    if qo_indptr is None:
        _need(query.dim() == 4 and query.shape[3] == D, "query must be [B, Sq, Hq, D]")
        B, Sq, Hq = query.shape[0], query.shape[1], query.shape[2]
        tokens = B * Sq
    else:
        _need(query.dim() == 3 and query.shape[2] == D, "query must be [total_q, Hq, D]")
        _dev_i32(qo_indptr, "qo_indptr")
        B, Sq, Hq = qo_indptr.numel() - 1, 0, query.shape[1]
        tokens = query.shape[0]
        _need(max_seq_len_q >= 1, "max_seq_len_q is required with qo_indptr")
    for t, n in ((paged_kv_indptr, "paged_kv_indptr"), (paged_kv_indices, "paged_kv_indices"),
                 (seq_lens, "seq_lens")):
        _dev_i32(t, n)
    if out is None:
        out = torch.empty_like(query)
    _need(out.is_contiguous() and out.shape == query.shape and out.dtype in _DTYPE,
          "out must be contiguous bf16 or fp32 in the query's layout")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.numel() == tokens * Hq and lse.is_contiguous(),
              "lse must be fp32 [tokens, Hq]")
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().paged_decode_q_run(_ptr(query), kp, vp, pst, hst, _ptr(paged_kv_indptr),
                                  _ptr(paged_kv_indices), _ptr(seq_lens), _ptr(qo_indptr), B,
                                  int(Sq), int(max_seq_len_q), Hq, Hkv, D, P, ps,
                                  int(max_seq_len), _mask(mask_type), int(window_left),
                                  _scale(bmm1_scale), float(bmm2_scale),
                                  _DTYPE[out.dtype], _ptr(out), _ptr(lse), ws_ptr, ws_bytes,
                                  num_cus_ if num_cus_ is not None else num_cus(query.device),
                                  stream if stream is not None else _stream(query.device))
    check(st, "paged_decode_q_run")
    return out


# =============================================================================
# Sage
# =============================================================================

def bsa_sage_validate(q2k_block_index, capacity, block_sparse_num, block_sizes, q2k_block_nums,
                      uniform_block_count, B, H, Sq, Sk, raise_on_error=True):
    idx = _host_i32(q2k_block_index)
    bs = None if block_sizes is None else _host_i32(block_sizes)
    nm = None if q2k_block_nums is None else _host_i32(q2k_block_nums)
    bad = Bad()
    st = lib().bsa_sage_validate(_hp(idx), capacity, block_sparse_num, _hp(bs),
                                 0 if bs is None else bs.ndim, _hp(nm), int(uniform_block_count),
                                 B, H, Sq, Sk, ctypes.byref(bad))
    if raise_on_error:
        check(st, "bsa_sage_validate", bad)
    return st, bad.field, bad.index


def bsa_sage_run(q_int8, k_int8, v_fp8, q_scale, k_scale, v_scale, q2k_block_index,
                 block_sparse_num, block_sizes=None, q2k_block_nums=None, softmax_scale=None, *,
                 out, uniform_block_count=False, contiguous_block_indices=False,
                 mask_type="dense", lse=None, stream=None):
    B, H, Sq, D = q_int8.shape
    Sk = k_int8.shape[2]
    _need(D == 128 and k_int8.shape[3] == 128, "head dim must be 128")
    _need(q_int8.dtype == torch.int8 and k_int8.dtype == torch.int8, "q/k must be int8")
    _need(v_fp8.dtype in (torch.float8_e4m3fn, torch.uint8)
          and tuple(v_fp8.shape) == (B, H, 128, -(-Sk // 64) * 64), "v must be e4m3 HDS")
    _need(tuple(q_scale.shape) == (B, H, -(-Sq // 128) * 4), "q_scale shape")
    _need(tuple(k_scale.shape) == (B, H, -(-Sk // 64)) and tuple(v_scale.shape) == (B, H, 128),
          "k_scale / v_scale shape")
    cap = q2k_block_index.shape[-1]
    _need(tuple(q2k_block_index.shape) == (B, H, -(-Sq // 64), cap), "q2k_block_index shape")
    for t in (q_int8, k_int8, v_fp8, q_scale, k_scale, v_scale, q2k_block_index, out):
        _need(t.is_cuda and t.is_contiguous(), "all Sage tensors must be contiguous CUDA tensors")
    _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (B, H, Sq, 128), "out must be bf16 BHSD")
    if lse is not None:
        _need(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
              and lse.numel() == B * H * Sq, "lse must be fp32 [B, H, Sq]")
    rank = 0 if block_sizes is None else block_sizes.dim()
    st = lib().bsa_sage_run(_ptr(q_int8), _ptr(k_int8), _ptr(v_fp8), _ptr(q_scale), _ptr(k_scale),
                            _ptr(v_scale), _ptr(q2k_block_index), cap, int(block_sparse_num),
                            _ptr(block_sizes), rank, _ptr(q2k_block_nums),
                            int(bool(uniform_block_count)), int(bool(contiguous_block_indices)),
                            B, H, Sq, Sk, _scale(softmax_scale), _mask(mask_type),
                            _ptr(out), _ptr(lse),
                            stream if stream is not None else _stream(q_int8.device))
    check(st, "bsa_sage_run")
    return out


def bsa_attn_blk64_sage_fwd(q_int8, k_int8, v_fp8, q_scale, k_scale, v_scale, q2k_block_index,
                            block_sparse_num, block_sizes=None, q2k_block_nums=None,
                            softmax_scale=None, *, out=None, uniform_block_count=False,
                            contiguous_block_indices=False, validate=False, mask_type="dense",
                            lse=None):
    """Mirrors the page "bsa_attn_sm120_blk64_sage_fwd" (caller-owned ``out``;
    allocated here when omitted).  ``mask_type="causal"`` and ``lse`` are
    additions beyond the page."""
    B, H, Sq, _ = q_int8.shape
    Sk = k_int8.shape[2]
    if validate:
        bsa_sage_validate(q2k_block_index, q2k_block_index.shape[-1], block_sparse_num,
                          block_sizes, q2k_block_nums, uniform_block_count, B, H, Sq, Sk)
    if out is None:
        out = torch.empty(B, H, Sq, 128, dtype=torch.bfloat16, device=q_int8.device)
    return bsa_sage_run(q_int8, k_int8, v_fp8, q_scale, k_scale, v_scale, q2k_block_index,
                        block_sparse_num, block_sizes, q2k_block_nums, softmax_scale, out=out,
                        uniform_block_count=uniform_block_count,
                        contiguous_block_indices=contiguous_block_indices, mask_type=mask_type,
                        lse=lse)


# =============================================================================
# Packed-query token-granular sparse attention
# =============================================================================

def qsa_validate(lo, hi, blk_base, tok_base, block_first, block_last, raise_on_error=True):
    """Host check of the packed partition (copies device tensors to the host)."""
    a = [_host_i32(x) for x in (lo, hi, blk_base, tok_base, block_first, block_last)]
    bad = Bad()
    st = lib().qsa_validate(a[0].size, a[4].size, *[_hp(x) for x in a], ctypes.byref(bad))
    if raise_on_error:
        check(st, "qsa_validate", bad)
    return st, bad.field, bad.index


def qsa_run(q, k, v, sel_blocks, lo, hi, blk_base, tok_base, scale=0.0625, block_size=4, *,
            out=None, out_fp32=None, lse=None, stream=None):
    """Trusted launch; any of out (bf16), out_fp32, lse [Hq, T] may be given."""
    T, Hq, D = q.shape
    _need(q.dtype == torch.bfloat16 and k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16,
          "q, k, v must be bf16")
    _need(k.dim() == 3 and k.shape == v.shape and k.shape[0] == T and k.shape[2] == D,
          "k, v must be [T, Hkv, D]")
    _need(sel_blocks.dtype == torch.uint8 and sel_blocks.dim() == 2 and sel_blocks.shape[0] == T,
          "sel_blocks must be uint8 [T, NB]")
    for t in (q, k, v, sel_blocks):
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous CUDA tensors")
    for t, n in ((lo, "lo"), (hi, "hi"), (blk_base, "blk_base"), (tok_base, "tok_base")):
        _dev_i32(t, n)
        _need(t.numel() == T, f"{n} must be [T]")
    if out is not None:
        _need(out.dtype == torch.bfloat16 and out.shape == q.shape and out.is_contiguous(),
              "out must be bf16 [T, Hq, D]")
    if out_fp32 is not None:
        _need(out_fp32.dtype == torch.float32 and out_fp32.shape == q.shape
              and out_fp32.is_contiguous(), "out_fp32 must be fp32 [T, Hq, D]")
    if lse is not None:
        _need(lse.dtype == torch.float32 and tuple(lse.shape) == (Hq, T) and lse.is_contiguous(),
              "lse must be fp32 [Hq, T]")
    st = lib().qsa_run(_ptr(q), _ptr(k), _ptr(v), _ptr(sel_blocks), _ptr(lo), _ptr(hi),
                       _ptr(blk_base), _ptr(tok_base), T, sel_blocks.shape[1], Hq, k.shape[1], D,
                       float(scale), int(block_size), _ptr(out), _ptr(out_fp32), _ptr(lse),
                       stream if stream is not None else _stream(q.device))
    check(st, "qsa_run")


def qsa_forward(q, k, v, sel_blocks, lo, hi, blk_base, tok_base, block_first, block_last,
                scale=0.0625, block_size=4, validate=False):
    """Mirrors the page "qsa_forward": returns (out bf16, out_fp32, lse [Hq, T]).
    ``validate`` checks the packed partition on the host first (a device->host
    copy; leave it off inside graph capture)."""
    if validate:
        qsa_validate(lo, hi, blk_base, tok_base, block_first, block_last)
    T, Hq, D = q.shape
    out = torch.empty_like(q)
    out_fp32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(Hq, T, dtype=torch.float32, device=q.device)
    qsa_run(q, k, v, sel_blocks, lo, hi, blk_base, tok_base, scale, block_size, out=out,
            out_fp32=out_fp32, lse=lse)
    return out, out_fp32, lse
