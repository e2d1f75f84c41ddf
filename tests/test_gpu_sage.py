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


def test_sage_long_full():
    """Full-size Sage workload (the benchmark's launch): every query block of
    every (request, head) against the oracle, one request at a time."""
    case = W.sage_long()
    _say("sage_long: generated")
    out = run_sage(case)
    assert torch.isfinite(out.float()).all()
    got = f64(out)
    for b in range(2):
        rows = [(b, h, r) for h in range(16) for r in range(256)]
        ref = oracle(case, rows=rows)
        _say("sage_long: oracle request", b)
        assert_close(got[b], ref[b], TOL_SAGE, f"sage long (request {b})")


# ----------------------------------------------------------------------------- additions

def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _run_ext(case, index=None, mask="dense", contiguous=False, uniform=None):
    q, k, v = case.q_int8.to(DEV), case.k_int8.to(DEV), case.v_fp8.to(DEV)
    B, H, Sq, _ = q.shape
    out = torch.empty(B, H, Sq, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, Sq, dtype=torch.float32, device=DEV)
    idx = case.q2k_block_index if index is None else index
    P.bsa_sage_run(q, k, v, case.q_scale.to(DEV), case.k_scale.to(DEV), case.v_scale.to(DEV),
                   _dev(idx), case.block_sparse_num, _dev(case.block_sizes),
                   _dev(case.q2k_block_nums), case.softmax_scale, out=out,
                   uniform_block_count=case.uniform_block_count if uniform is None else uniform,
                   contiguous_block_indices=contiguous, mask_type=mask, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _oracle_ext(case, mask="dense", uniform=None):
    return A.sage_reference(case.q_int8, case.k_int8, case.v_fp8.view(torch.uint8).numpy(),
                            case.q_scale, case.k_scale, case.v_scale, case.q2k_block_index,
                            case.block_sparse_num, case.block_sizes, case.q2k_block_nums,
                            case.uniform_block_count if uniform is None else uniform,
                            case.softmax_scale, Sk=case.Sk, mask=mask, with_lse=True)


@pytest.mark.parametrize("mask", ["dense", "causal"])
@pytest.mark.parametrize("rank", [1, 3])
def test_sage_mask_and_lse(mask, rank):
    case = W.sage_small(40 + rank, block_sizes_rank=rank)
    _say("sage mask/lse", mask, rank)
    out, lse = _run_ext(case, mask=mask)
    ref_o, ref_l = _oracle_ext(case, mask=mask)
    assert_close(f64(out), ref_o, TOL_SAGE, f"out {mask}")
    assert_close(f64(lse), ref_l, 2e-3, f"lse {mask}")


@pytest.mark.parametrize("Sq,Sk", [(100, 300), (200, 130)])
def test_sage_causal_rectangular(Sq, Sk):
    """Bottom-right causal alignment with Sq != Sk (every block selected); with
    Sq > Sk the first Sq - Sk rows admit nothing (zeros, LSE -inf)."""
    nkb = -(-Sk // 64)
    case = W.make_sage(44, 1, 2, Sq, Sk, cap=nkb, nsel=nkb, per_row_counts=False,
                       block_sizes_rank=1)
    _say("sage causal", Sq, Sk)
    out, lse = _run_ext(case, mask="causal")
    ref_o, ref_l = _oracle_ext(case, mask="causal")
    assert_close(f64(out), ref_o, TOL_SAGE, "out")
    assert_close(f64(lse), ref_l, 2e-3, "lse")


def test_sage_contiguous_fast_path():
    """uniform_block_count + contiguous_block_indices: rows select runs
    start .. start + n - 1; only the first index is read, so entries after it
    may hold anything."""
    case = W.make_sage(45, 2, 3, 700, 900, cap=6, nsel=4, per_row_counts=True,
                       uniform=True, block_sizes_rank=2)
    nkb = -(-900 // 64)
    rng = np.random.default_rng(45)
    idx = np.full(case.q2k_block_index.shape, -7, dtype=np.int32)
    starts = rng.integers(0, nkb - 4 + 1, size=idx.shape[:3])
    for t in range(4):
        idx[..., t] = starts + t
    case.q2k_block_index = idx
    _say("sage contiguous")
    out_c, lse_c = _run_ext(case, contiguous=True)
    ref_o, ref_l = _oracle_ext(case)
    assert_close(f64(out_c), ref_o, TOL_SAGE, "contiguous out")
    assert_close(f64(lse_c), ref_l, 2e-3, "contiguous lse")
    # the same selections read index by index give the same result bit for bit
    out_i, lse_i = _run_ext(case, contiguous=False)
    assert torch.equal(out_c, out_i) and torch.equal(lse_c, lse_i)
    # garbage after the first index does not matter on the fast path
    junk = idx.copy()
    junk[..., 1:] = rng.integers(-100, 100, size=junk[..., 1:].shape)
    out_j, _ = _run_ext(case, index=junk, contiguous=True)
    assert torch.equal(out_c, out_j)


def test_sage_growing_scores():
    """Every row visits its blocks in order and each block's keys are scaled
    12% above the previous one's, so the running row max keeps rising through
    the walk: some rises stay inside the kernel's rescale slack and others pass
    it (the running output is then rescaled).  Output and LSE stay on the bar."""
    nkb = 16
    case = W.make_sage(46, 1, 2, 128, 64 * nkb, cap=nkb, nsel=nkb, per_row_counts=False,
                       block_sizes_rank=0)
    case.q2k_block_index[:] = np.arange(nkb, dtype=np.int32)
    grow = torch.tensor([1.12 ** blk for blk in range(nkb)], dtype=torch.float32)
    case.k_scale = (case.k_scale * grow).contiguous()
    case.softmax_scale = 0.3
    _say("sage growing scores")
    out, lse = _run_ext(case)
    ref_o, ref_l = _oracle_ext(case)
    assert_close(f64(out), ref_o, TOL_SAGE, "out")
    assert_close(f64(lse), ref_l, 2e-3, "lse")
