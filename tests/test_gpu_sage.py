"""GPU parity of the Sage-style quantized block-sparse kernel against the fp64
oracle run on the dequantised inputs (bar: 5e-2 absolute, bf16 output)."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from gen import workloads as W
from oracle import attention as A
from tests.gpu_util import assert_close, f64

pytestmark = pytest.mark.gpu
TOL_SAGE = 5e-2
DEV = "cuda"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_sage(case, uniform=None, scalar_only=False):
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)  # noqa: E731
    q, k = case.q_int8.to(DEV), case.k_int8.to(DEV)
    v = case.v_fp8.to(DEV)
    B, H, Sq, _ = q.shape
    out = torch.empty(B, H, Sq, 128, dtype=torch.bfloat16, device=DEV)
    nums = None if scalar_only else case.q2k_block_nums
    P.bsa_attn_blk64_sage_fwd(q, k, v, case.q_scale.to(DEV), case.k_scale.to(DEV),
                              case.v_scale.to(DEV), t(case.q2k_block_index),
                              case.block_sparse_num, t(case.block_sizes), t(nums),
                              case.softmax_scale, out=out,
                              uniform_block_count=case.uniform_block_count if uniform is None else uniform,
                              validate=True)
    torch.cuda.synchronize()
    return out


def oracle(case, rows=None, uniform=None, scalar_only=False):
    return A.sage_reference(case.q_int8, case.k_int8, case.v_fp8.view(torch.uint8).numpy(),
                            case.q_scale, case.k_scale, case.v_scale, case.q2k_block_index,
                            case.block_sparse_num, case.block_sizes,
                            None if scalar_only else case.q2k_block_nums,
                            case.uniform_block_count if uniform is None else uniform,
                            case.softmax_scale, Sk=case.Sk, rows=rows)


@pytest.mark.parametrize("rank", [1, 2, 3])
def test_sage_small(rank):
    case = W.sage_small(15 + rank, block_sizes_rank=rank)
    _say("sage_small rank", rank)
    out = run_sage(case)
    ref = oracle(case)
    assert_close(f64(out), ref, TOL_SAGE, "sage out")
    nums = case.q2k_block_nums
    for b, h, r in zip(*np.nonzero(nums == 0)):
        assert torch.all(out[b, h, r * 64:(r + 1) * 64] == 0)


def test_sage_scalar_count_and_uniform():
    case = W.sage_small(21, block_sizes_rank=1)
    out = run_sage(case, scalar_only=True)
    assert_close(f64(out), oracle(case, scalar_only=True), TOL_SAGE, "scalar count")
    out_u = run_sage(case, uniform=True)                 # per-row counts ignored
    assert_close(f64(out_u), oracle(case, uniform=True), TOL_SAGE, "uniform flag")
    assert torch.equal(out, out_u)


def test_sage_no_block_sizes_and_full_selection():
    case = W.make_sage(22, 1, 2, 300, 260, cap=5, nsel=5, per_row_counts=False,
                       block_sizes_rank=0)
    out = run_sage(case)
    assert_close(f64(out), oracle(case), TOL_SAGE, "all blocks")


def test_sage_long_sampled():
    case = W.sage_long()
    _say("sage_long: generated")
    out = run_sage(case)
    rng = np.random.default_rng(9)
    rows = [(int(b), int(h), int(r)) for b, h, r in
            zip(rng.integers(0, 2, 6), rng.integers(0, 16, 6), rng.integers(0, 256, 6))]
    rows += [(0, 0, 0), (1, 15, 255)]
    ref = oracle(case, rows=rows)
    got = f64(out)
    for b, h, r in rows:
        assert_close(got[b, h, r * 64:(r + 1) * 64], ref[b, h, r * 64:(r + 1) * 64], TOL_SAGE,
                     f"sage long ({b},{h},{r})")
    assert torch.isfinite(out.float()).all()
