"""Helpers shared by the GPU parity tests: move generated cases to the device,
run them through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_block_amd as P
from oracle import attention as A

# Correctness bar: bf16 outputs, fp32 outputs / LSE (absolute error).
TOL_BF16 = 2e-2
TOL_F32 = 2e-3
TOL_LSE = 2e-3

DEV = "cuda"


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def dev_bits(words):
    if words is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV)


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_close(got, want, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    fin = np.isfinite(want)
    bad_fin = ~np.isfinite(got[fin])
    assert not bad_fin.any(), f"{what}: non-finite GPU values where the oracle is finite"
    assert np.array_equal(got[~fin], want[~fin]), f"{what}: -inf / special values differ"
    if fin.any():
        err = np.max(np.abs(got[fin] - want[fin]))
        assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"
        return float(err)
    return 0.0


def run_bsa(case, out_dtype=torch.bfloat16, combined=False, k=None, v=None, indices=None,
            with_lse=True):
    """Run a BsaCase through block_sparse_attention_with_paged_kv_cache."""
    k = case.k if k is None else k
    v = case.v if v is None else v
    if combined:
        cache = torch.stack([k, v], dim=1).to(DEV)
    else:
        cache = (k.to(DEV), v.to(DEV))
    q = case.q.to(DEV)
    B, Sq, Hq, D = q.shape
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    lse = torch.empty(B * Sq, Hq, dtype=torch.float32, device=DEV) if with_lse else None
    P.block_sparse_attention_with_paged_kv_cache(
        q, cache, dev_i32(case.kv_indptr), dev_i32(case.kv_indices if indices is None else indices),
        dev_i32(case.block_indptr), dev_i32(case.block_indices), case.q_block_size,
        case.kv_block_size, max_seq_len_kv=case.max_seq_len_kv, seq_lens_kv=dev_i32(case.seq_lens),
        kv_valid_bits=dev_bits(case.valid_bits), mask_type=case.mask, sm_scale=case.sm_scale,
        out=out, window_left=case.window_left, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_bsa(case, tokens=None):
    return A.bsa_reference(case.q, case.k, case.v, case.kv_indptr, case.kv_indices,
                           case.block_indptr, case.block_indices, case.q_block_size,
                           case.kv_block_size, case.seq_lens, valid_bits=case.valid_bits,
                           mask=case.mask, window_left=case.window_left, sm_scale=case.sm_scale,
                           tokens=tokens)


def run_prefill(case, out_dtype=torch.bfloat16, with_lse=True):
    q = case.q.to(DEV)
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=DEV) if with_lse else None
    P.batch_prefill_with_paged_kv_cache(
        q, case.k.to(DEV), case.v.to(DEV), dev_i32(case.qo_indptr), dev_i32(case.block_tables),
        dev_i32(case.seq_lens), page_size=case.k.shape[2], mask_type=case.mask,
        window_left=case.window_left, sm_scale=case.sm_scale, output_scale=case.output_scale,
        out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_prefill(case, rows=None):
    return A.prefill_reference(case.q, case.k, case.v, case.qo_indptr, case.block_tables,
                               case.seq_lens, mask=case.mask, window_left=case.window_left,
                               sm_scale=case.sm_scale, output_scale=case.output_scale, rows=rows)


def run_decode(case, out_dtype=torch.bfloat16, combined=False, num_cus=None):
    q = case.q.to(DEV)
    B, Hq, D = q.shape
    ncu = num_cus if num_cus is not None else P.num_cus()
    nbytes, S, split_len = P.paged_decode_workspace_size(B, Hq, case.k.shape[1], D,
                                                         case.max_seq_len, case.k.shape[2], ncu)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    cache = torch.stack([case.k, case.v], dim=1).to(DEV) if combined else \
        (case.k.to(DEV), case.v.to(DEV))
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    P.paged_decode_run(q, cache, dev_i32(case.kv_indptr), dev_i32(case.kv_indices),
                       dev_i32(case.seq_lens), case.max_seq_len, ws, mask_type=case.mask,
                       window_left=case.window_left, bmm1_scale=case.bmm1_scale,
                       bmm2_scale=case.bmm2_scale, out=out, lse=lse, num_cus_=ncu)
    torch.cuda.synchronize()
    return out, lse, S


def oracle_decode(case, requests=None):
    return A.decode_reference(case.q, case.k, case.v, case.kv_indptr, case.kv_indices,
                              case.seq_lens, mask=case.mask, window_left=case.window_left,
                              bmm1_scale=case.bmm1_scale, bmm2_scale=case.bmm2_scale,
                              requests=requests)


def run_decode_q(case, out_dtype=torch.bfloat16, num_cus=None):
    """Multi-token decode of a DecodeQCase through paged_decode_q_run."""
    q = case.q.to(DEV)
    Hq, D = q.shape[-2], q.shape[-1]
    B = len(case.seq_lens)
    ncu = num_cus if num_cus is not None else P.num_cus()
    nbytes, S, _ = P.paged_decode_q_workspace_size(B, case.seq_len_q, Hq, case.k.shape[1], D,
                                                   case.max_seq_len, case.k.shape[2], ncu)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    qo = None if case.qo_indptr is None else dev_i32(case.qo_indptr)
    P.paged_decode_q_run(q, (case.k.to(DEV), case.v.to(DEV)), dev_i32(case.kv_indptr),
                         dev_i32(case.kv_indices), dev_i32(case.seq_lens), case.max_seq_len, ws,
                         qo_indptr=qo, max_seq_len_q=case.seq_len_q, mask_type=case.mask,
                         window_left=case.window_left, out=out, lse=lse, num_cus_=ncu)
    torch.cuda.synchronize()
    return out, lse, S


def oracle_decode_q(case):
    return A.decode_q_reference(case.q, case.k, case.v, case.kv_indptr, case.kv_indices,
                                case.seq_lens, qo_indptr=case.qo_indptr, mask=case.mask,
                                window_left=case.window_left)
