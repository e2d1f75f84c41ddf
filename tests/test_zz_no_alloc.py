"""The allocation-free decode entry point (paged_decode_run_noalloc) against
paged_decode_run with a caller workspace: same kernels and split policy, so the
outputs must be identical, and both within the oracle's bars.  Two calls in a
row share the library's per-device scratch, the second with a smaller batch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from gen import workloads as W
from tests.gpu_util import (TOL_BF16, TOL_LSE, assert_close, dev_i32, f64, oracle_decode,
                            run_decode)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _noalloc(case, num_cus, out_dtype=torch.bfloat16):
    """One call through the C ABI (ctypes), no workspace argument."""
    q = case.q.to("cuda")
    B, Hq, D = q.shape
    k, v = case.k.to("cuda"), case.v.to("cuda")
    Hkv, ps = k.shape[1], k.shape[2]
    ip, ix, sl = dev_i32(case.kv_indptr), dev_i32(case.kv_indices), dev_i32(case.seq_lens)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    st = P.lib().paged_decode_run_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), ip.data_ptr(),
        ix.data_ptr(), sl.data_ptr(), B, Hq, Hkv, D, k.shape[0], ps, case.max_seq_len,
        1 if case.mask == "causal" else 0, case.window_left, float("nan"), case.bmm2_scale,
        0 if out_dtype == torch.bfloat16 else 1, out.data_ptr(), lse.data_ptr(), num_cus,
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, P.lib().pkb_status_string(st)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # seed, B, Hq, Hkv, D, seq_lens, page_size, mask, window, num_cus
    (900, 4, 32, 8, 128, [3000, 1000, 5000, 77], 16, "causal", -1, 256),   # split partials
    (901, 2, 32, 8, 128, [700, 300], 16, "causal", -1, 256),               # smaller, again split
    (902, 3, 16, 2, 256, [129, 4097, 2], 32, "causal", 64, 256),          # D = 256 partials
    (903, 6, 32, 8, 128, [1, 31, 200, 33, 127, 1000], 16, "dense", -1, 4),  # single pass: no scratch
]


def test_noalloc_decode_equals_workspace_decode():
    for seed, B, Hq, Hkv, D, sl, ps, mask, w, ncu in CASES:
        _say("noalloc decode", seed, B, Hq, Hkv, D, sl, ps, mask, w, ncu)
        nbytes, S, _ = P.paged_decode_workspace_size(B, Hq, Hkv, D, max(sl), ps, ncu)
        assert nbytes <= P._lib.PKB_DECODE_SCRATCH_BYTES
        assert (S > 1) == (seed != 903)
        case = W.make_decode(seed, B, Hq, Hkv, D, sl, ps, mask=mask, window_left=w,
                             extra_pages=2, bmm2_scale=1.1)
        ref_o, ref_l, S_ref = run_decode(case, num_cus=ncu)
        got_o, got_l = _noalloc(case, ncu)
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l)
        want_o, want_l = oracle_decode(case)
        assert_close(f64(got_o), want_o, TOL_BF16, "out")
        assert_close(f64(got_l), want_l, TOL_LSE, "lse")


def test_noalloc_decode_rejects_oversized_partials():
    # 300 requests x 32 heads x 8 splits x 260 floats exceed the 32 MiB scratch;
    # the call returns before anything is enqueued (no pointer is used).
    nbytes, S, _ = P.paged_decode_workspace_size(300, 32, 8, 256, 8192, 16, 256)
    assert nbytes > P._lib.PKB_DECODE_SCRATCH_BYTES
    d = ctypes.c_void_p(256)
    st = P.lib().paged_decode_run_noalloc(d, d, d, 8 * 16 * 256, 16 * 256, d, d, d, 300, 32, 8,
                                          256, 1000, 16, 8192, 0, -1, float("nan"), 1.0, 0, d,
                                          None, 256, None)
    assert st == P._lib.PKB_ERR_WORKSPACE
