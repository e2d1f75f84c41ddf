"""GPU parity for page sizes that are not a multiple of 8.

The block-sparse and decode pages constrain block sizes only, so a pool may
use any page size; an 8-token chunk then spans pages and the kernels translate
each K/V row on its own.  Each case checks bf16 and fp32 outputs and the LSE
against the fp64 oracle (bars as in the other parity tests), over small
batches that span several 64-key tiles and query tiles with ragged tails, on
every kernel path: block-sparse at 1, 2 and 4 waves, contiguous and
small-block walks, D = 128 and 256; the split-KV and single-pass decode
kernels; multi-token decode in both of its kernels.
"""
import sys

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from gen import workloads as W
from tests.gpu_util import (TOL_BF16, TOL_F32, TOL_LSE, assert_close, f64, oracle_bsa,
                            oracle_decode, oracle_decode_q, run_bsa, run_decode, run_decode_q)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


BSA_RAGGED = [
    # B, Sq, Hq, Hkv, D, seq_lens, ps, qbs, kvbs, mask, w, bits_p, extra
    (2, 64, 4, 1, 128, [200, 333], 1, 16, 32, "causal", -1, 0.95, {}),      # 2 waves, small blocks
    (2, 70, 8, 2, 128, [70, 190], 3, 8, 8, "dense", -1, None, {}),          # 1 wave
    (1, 100, 4, 4, 128, [300], 5, 8, 16, "causal", 37, 0.9, {}),            # MHA, window
    (2, 96, 16, 2, 128, [500, 260], 12, 16, 128, "dense", -1, 0.8, {"allow_empty": True}),
    (1, 130, 32, 8, 128, [700], 20, 64, 64, "causal", -1, 0.99, {}),        # 4 waves, 2 tiles/row
    (2, 40, 2, 1, 256, [90, 123], 7, 4, 32, "causal", 20, 0.9, {}),
    (1, 33, 8, 2, 256, [180], 17, 16, 192, "dense", -1, None, {}),
    (3, 50, 8, 1, 128, [0, 55, 129], 6, 4, 64, "causal", -1, None,
     {"out_of_range": 1, "max_seq_len_kv": 400}),
    (2, 64, 32, 8, 256, [64, 500], 2, 32, 64, "causal", -1, 0.9, {}),        # D=256, 4 waves
]


@pytest.mark.parametrize("i", range(len(BSA_RAGGED)))
def test_bsa_ragged_page_size(i):
    B, Sq, Hq, Hkv, D, sl, ps, qbs, kvbs, mask, w, bits_p, extra = BSA_RAGGED[i]
    _say("bsa ragged page size", BSA_RAGGED[i])
    case = W.make_bsa(900 + i, B, Sq, Hq, Hkv, D, sl, ps, qbs, kvbs, mask=mask, window_left=w,
                      bits_p=bits_p, extra_pages=3, **extra)
    assert case.k.shape[2] == ps
    out, lse = run_bsa(case)
    ref_o, ref_l = oracle_bsa(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _ = run_bsa(case, out_dtype=torch.float32, with_lse=False)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")
    out_c, lse_c = run_bsa(case, combined=True)
    assert torch.equal(out_c, out) and torch.equal(lse_c, lse)


DECODE_RAGGED = [
    # B, Hq, Hkv, D, seq_lens, ps, mask, w, num_cus, single pass
    (4, 32, 8, 128, [1, 63, 64, 1000], 1, "dense", -1, 256, False),
    (3, 8, 8, 128, [4097, 5, 300], 5, "causal", 100, 256, False),
    (2, 16, 2, 256, [777, 2049], 12, "dense", -1, 256, False),
    (5, 4, 1, 128, [129, 1, 2000, 64, 65], 3, "causal", 0, 8, False),
    (6, 32, 8, 128, [1, 31, 32, 33, 127, 1000], 1, "dense", -1, 4, True),
    (5, 16, 2, 256, [4097, 5, 300, 2049, 64], 20, "causal", 100, 3, True),
    (7, 4, 1, 128, [129, 1, 2000, 64, 65, 700, 3], 7, "causal", 0, 2, True),
    (4, 16, 1, 128, [333, 1024, 8, 5000], 33, "dense", -1, 2, True),          # G = 16
]


@pytest.mark.parametrize("i", range(len(DECODE_RAGGED)))
def test_decode_ragged_page_size(i):
    B, Hq, Hkv, D, sl, ps, mask, w, ncu, single = DECODE_RAGGED[i]
    _say("decode ragged page size", DECODE_RAGGED[i])
    case = W.make_decode(930 + i, B, Hq, Hkv, D, sl, ps, mask=mask, window_left=w, extra_pages=2,
                         bmm2_scale=1.25)
    assert case.k.shape[2] == ps
    out, lse, S = run_decode(case, num_cus=ncu)
    assert (S == 1) if single else (S > 1)
    ref_o, ref_l = oracle_decode(case)
    assert_close(f64(out), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, lse32, _ = run_decode(case, out_dtype=torch.float32, num_cus=ncu)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")
    assert_close(f64(lse32), ref_l, TOL_LSE, "lse (fp32 run)")
    out_c, lse_c, _ = run_decode(case, combined=True, num_cus=ncu)
    assert torch.equal(out_c, out) and torch.equal(lse_c, lse)


DECODE_Q_RAGGED = [
    # B, Hq, Hkv, D, seq_lens, ps, SQ (fixed) or qlens (packed), mask, w, num_cus
    (2, 32, 2, 128, [300, 5000], 5, [8, 3], "causal", -1, 64),         # > 16 rows: split mode
    (3, 16, 4, 256, [5, 129, 700], 12, [5, 1, 4], "causal", 0, 16),     # > 16 rows, qlen == L
    (4, 32, 8, 128, [9, 3000, 4, 700], 1, [1, 4, 2, 3], "causal", 40, 256),   # <= 16 rows
    (4, 8, 2, 128, [77, 1, 300, 4100], 3, 1, "dense", -1, 3),           # single pass
    (5, 16, 4, 256, [16, 2049, 90, 5, 64], 9, 4, "causal", -1, 4),      # single pass
]


@pytest.mark.parametrize("i", range(len(DECODE_Q_RAGGED)))
def test_decode_q_ragged_page_size(i):
    B, Hq, Hkv, D, sl, ps, sq, mask, w, ncu = DECODE_Q_RAGGED[i]
    _say("decode_q ragged page size", DECODE_Q_RAGGED[i])
    fixed = isinstance(sq, int)
    case = W.make_decode_q(960 + i, B, Hq, Hkv, D, sl, ps, seq_len_q=sq if fixed else None,
                           qlens=None if fixed else sq, mask=mask, window_left=w, extra_pages=2)
    assert case.k.shape[2] == ps
    out, lse, S = run_decode_q(case, num_cus=ncu)
    ref_o, ref_l = oracle_decode_q(case)
    assert_close(f64(out), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _, _ = run_decode_q(case, out_dtype=torch.float32, num_cus=ncu)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")


def test_batch_decode_page_size_1_sampled():
    """The batch decode workload (B=64, lengths U{512..8192}) stored one token
    per page: sampled requests against the oracle, all outputs finite."""
    case = W.batch_decode(page_size=1)
    _say("batch_decode page_size=1: generated", int(case.seq_lens.sum()))
    out, lse, S = run_decode(case)
    reqs = [0, 5, 40, 63] + [int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens))]
    ref_o, ref_l = oracle_decode(case, requests=reqs)
    assert_close(f64(out[reqs]), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse[reqs]), ref_l, TOL_LSE, "lse")
    assert torch.isfinite(out.float()).all()
