"""GPU parity of the packed-query token-granular sparse attention kernel against
the fp64 oracle.  Bars: bf16 out 2e-2, fp32 out and LSE 2e-3 (absolute); the
bf16 output is the rounding of the fp32 one."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from gen import workloads as W
from oracle import attention as A
from tests.gpu_util import DEV, TOL_BF16, TOL_F32, TOL_LSE, assert_close, dev_i32, f64

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_qsa(case):
    sel = torch.from_numpy(case.sel_blocks).to(DEV)
    P.qsa_validate(case.lo, case.hi, case.blk_base, case.tok_base, case.block_first,
                   case.block_last)
    out, out32, lse = P.qsa_forward(case.q.to(DEV), case.k.to(DEV), case.v.to(DEV), sel,
                                    dev_i32(case.lo), dev_i32(case.hi), dev_i32(case.blk_base),
                                    dev_i32(case.tok_base), dev_i32(case.block_first),
                                    dev_i32(case.block_last), scale=case.scale)
    torch.cuda.synchronize()
    return out, out32, lse


def oracle(case, tokens=None):
    return A.qsa_reference(case.q, case.k, case.v, case.sel_blocks, case.lo, case.hi,
                           case.block_first, case.block_last, case.scale, tokens=tokens)


QSA_SWEEP = [
    # seq_lens, Hq, Hkv, D, kwargs
    ([7, 100, 33], 12, 1, 256, dict(p_sel=0.3, mode="causal")),
    ([64, 1, 130], 12, 1, 256, dict(p_sel=0.5, mode="dense", empty_rows=3, junk_bits=0.05)),
    ([300], 24, 2, 256, dict(p_sel=0.2, mode="causal", window=37)),
    ([50, 77], 8, 1, 128, dict(p_sel=0.4, mode="causal", force_diag=False)),
    ([129, 3, 64], 16, 4, 128, dict(n_sel=5, mode="dense")),
    ([500], 12, 1, 256, dict(p_sel=1.0, mode="causal")),       # every block: causal attention
    ([40, 40], 12, 1, 256, dict(p_sel=0.0, mode="causal", force_diag=False)),   # all rows empty
    # block counts that are multiples of 16: one 16-byte bitmap load per lane
    ([64, 64], 12, 1, 256, dict(p_sel=0.5, mode="causal")),
    ([256, 128], 8, 1, 128, dict(p_sel=0.3, mode="causal", window=90)),
    ([1024, 960], 12, 1, 256, dict(n_sel=40, mode="dense", junk_bits=0.05)),
    ([4864], 12, 1, 256, dict(n_sel=48, mode="causal")),      # 1216 blocks: two candidate chunks
]


@pytest.mark.parametrize("i", range(len(QSA_SWEEP)))
def test_qsa_sweep(i):
    lens, Hq, Hkv, D, kw = QSA_SWEEP[i]
    _say("qsa_sweep", QSA_SWEEP[i])
    case = W.make_qsa(800 + i, lens, Hq=Hq, Hkv=Hkv, D=D, **kw)
    out, out32, lse = run_qsa(case)
    ref_o, ref_l = oracle(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(out32), ref_o, TOL_F32, "out_fp32")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    assert torch.equal(out, out32.to(torch.bfloat16))


def test_qsa_long_full():
    """Full-size packed-query workload (4 x 4096 tokens): every token's outputs
    and LSE."""
    case = W.qsa_long()
    _say("qsa_long: generated", case.q.shape[0], "tokens")
    out, out32, lse = run_qsa(case)
    ref_o, ref_l = oracle(case)
    assert_close(f64(out32), ref_o, TOL_F32, "out_fp32")
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
