"""Page pools past 4 GiB.  The live pages of a small case are placed at the top
of a pool larger than 4 GiB (their IDs shifted by the same amount) and every
path must return bit-identical output and LSE: the kernels address the pool
with 64-bit offsets.  (The small-pool results are checked against the oracle
by the other tests.)"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from gen import workloads as W
from tests.gpu_util import dev_i32, run_bsa, run_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"
POOL_BYTES = 9 << 29          # 4.5 GiB per pool


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _shifted_pool(small: torch.Tensor, shift: int) -> torch.Tensor:
    big = torch.zeros((shift + small.shape[0],) + tuple(small.shape[1:]), dtype=small.dtype,
                      device=DEV)
    big[shift:] = small.to(DEV)
    return big


def _shift_for(pool: torch.Tensor) -> int:
    page_bytes = pool[0].numel() * pool.element_size()
    return -(-POOL_BYTES // page_bytes)


def _done(*ts):
    del ts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_bsa_large_pool():
    case = W.tiny_bsa("causal")
    out, lse = run_bsa(case)
    shift = _shift_for(case.k)
    _say("bsa large pool: shift", shift)
    bk, bv = _shifted_pool(case.k, shift), _shifted_pool(case.v, shift)
    out2, lse2 = run_bsa(case, k=bk, v=bv, indices=np.asarray(case.kv_indices) + shift)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _done(bk, bv)


def test_prefill_large_pool():
    case = W.make_prefill(710, 2, [70, 150], [300, 40], 8, 2, 128, 32, mask="causal")
    out, lse = run_prefill(case)
    shift = _shift_for(case.k)
    _say("prefill large pool: shift", shift)
    bt = np.asarray(case.block_tables)
    big = dataclasses.replace(case, k=_shifted_pool(case.k, shift), v=_shifted_pool(case.v, shift),
                              block_tables=np.where(bt >= 0, bt + shift, bt).astype(np.int32))
    out2, lse2 = run_prefill(big)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _done(big.k, big.v)


def test_decode_large_pool():
    case = W.make_decode(720, 3, 32, 8, 128, [2000, 333, 4097], 16)
    B, Hq, D = case.q.shape
    Hkv, ps = case.k.shape[1], case.k.shape[2]
    nbytes, S, _ = P.paged_decode_workspace_size(B, Hq, Hkv, D, case.max_seq_len, ps)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    q = case.q.to(DEV)

    def run(k, v, shift):
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        P.paged_decode_run(q, (k, v), dev_i32(case.kv_indptr),
                           dev_i32(np.asarray(case.kv_indices) + shift), dev_i32(case.seq_lens),
                           case.max_seq_len, ws, out=out, lse=lse)
        torch.cuda.synchronize()
        return out, lse

    out, lse = run(case.k.to(DEV), case.v.to(DEV), 0)
    shift = _shift_for(case.k)
    _say("decode large pool: shift", shift)
    bk, bv = _shifted_pool(case.k, shift), _shifted_pool(case.v, shift)
    out2, lse2 = run(bk, bv, shift)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _done(bk, bv)
