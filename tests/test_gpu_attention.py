"""GPU parity of the bf16 attention kernels against the fp64 oracle.

Small cases span several 64-key tiles and query tiles with ragged tails; the
named workloads run at full size and are checked on every row (long-context
prefill: sampled rows).  Bars: bf16
out 2e-2, fp32 out 2e-3, LSE 2e-3 (absolute).
"""
import sys

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from gen import workloads as W
from tests.gpu_util import (TOL_BF16, TOL_F32, TOL_LSE, assert_close, f64, oracle_bsa,
                            oracle_decode, oracle_decode_q, oracle_prefill, run_bsa, run_decode,
                            run_decode_q, run_prefill)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- block-sparse

@pytest.mark.parametrize("mask", ["dense", "causal"])
def test_tiny_bsa(mask):
    case = W.tiny_bsa(mask)
    _say("tiny_bsa", mask)
    out, lse = run_bsa(case)
    ref_o, ref_l = oracle_bsa(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, lse32 = run_bsa(case, out_dtype=torch.float32)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")
    # the bf16 output agrees with the fp32 one to the bf16 bar
    assert (out.float() - out32).abs().max().item() <= TOL_BF16


BSA_SWEEP = [
    # B, Sq, Hq, Hkv, D, seq_lens, ps, qbs, kvbs, mask, w, bits_p, extra
    (2, 64, 4, 1, 128, [200, 333], 16, 16, 32, "causal", -1, 0.95, {}),
    (2, 70, 8, 2, 128, [70, 190], 16, 8, 8, "dense", -1, None, {}),
    (1, 100, 4, 4, 128, [300], 32, 8, 16, "causal", 37, 0.9, {}),
    (3, 50, 8, 1, 128, [0, 55, 129], 8, 4, 64, "causal", -1, None, {"out_of_range": 1, "max_seq_len_kv": 400}),
    (2, 96, 16, 2, 128, [500, 260], 64, 16, 128, "dense", -1, 0.8, {"allow_empty": True}),
    (1, 130, 32, 8, 128, [700], 64, 64, 64, "causal", -1, 0.99, {}),
    (2, 40, 2, 1, 256, [90, 123], 16, 4, 32, "causal", 20, 0.9, {}),
    (1, 33, 8, 2, 256, [180], 32, 16, 192, "dense", -1, None, {}),
    (2, 20, 1, 1, 128, [64, 8], 8, 8, 8, "dense", -1, 0.5, {"allow_empty": True}),
]


@pytest.mark.parametrize("i", range(len(BSA_SWEEP)))
def test_bsa_sweep(i):
    B, Sq, Hq, Hkv, D, sl, ps, qbs, kvbs, mask, w, bits_p, extra = BSA_SWEEP[i]
    _say("bsa_sweep", BSA_SWEEP[i])
    case = W.make_bsa(300 + i, B, Sq, Hq, Hkv, D, sl, ps, qbs, kvbs, mask=mask, window_left=w,
                      bits_p=bits_p, extra_pages=3, **extra)
    out, lse = run_bsa(case)
    ref_o, ref_l = oracle_bsa(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _ = run_bsa(case, out_dtype=torch.float32, with_lse=False)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")


def test_bsa_empty_rows_exact():
    case = W.make_bsa(41, 2, 32, 4, 1, 128, [100, 90], 16, 16, 32, mask="dense", p_sel=0.0,
                      allow_empty=True)
    case.block_indptr[:] = 0        # no row selects anything
    case.block_indices = np.zeros(0, dtype=np.int32)
    out, lse = run_bsa(case)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_bsa_poison_unused_memory():
    """NaN in unreferenced pages and in slots past the live length changes nothing."""
    case = W.make_bsa(42, 2, 48, 8, 2, 128, [77, 150], 16, 16, 32, mask="causal", bits_p=0.9,
                      extra_pages=9)
    ref, ref_l = run_bsa(case)
    last = []
    for b in range(2):
        L = int(case.seq_lens[b])
        pg = case.kv_indices[case.kv_indptr[b] + (L - 1) // 16]
        last.append((int(pg), L % 16 if L % 16 else 16))
    used = []
    for b in range(2):
        n = -(-int(case.seq_lens[b]) // 16)
        used += list(case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b] + n])
    k2, v2 = W.poison_unused_pages(case.k, case.v, used, last)
    out, lse = run_bsa(case, k=k2, v=v2)
    assert torch.equal(out, ref) and torch.equal(lse, ref_l)


def test_bsa_page_permutation_and_combined_cache_bit_identical():
    case = W.make_bsa(43, 2, 64, 8, 2, 128, [210, 95], 16, 16, 32, mask="causal", bits_p=0.9,
                      extra_pages=6)
    ref, ref_l = run_bsa(case)
    perm = np.random.default_rng(0).permutation(case.k.shape[0])
    k2 = torch.empty_like(case.k); v2 = torch.empty_like(case.v)
    k2[torch.from_numpy(perm)] = case.k
    v2[torch.from_numpy(perm)] = case.v
    out, lse = run_bsa(case, k=k2, v=v2, indices=perm[case.kv_indices].astype(np.int32))
    assert torch.equal(out, ref) and torch.equal(lse, ref_l)
    out_c, lse_c = run_bsa(case, combined=True)
    assert torch.equal(out_c, ref) and torch.equal(lse_c, ref_l)


def test_bsa_all_blocks_equals_prefill():
    B, Sq, Hq, Hkv, D = 2, 96, 8, 2, 128
    case = W.make_bsa(44, B, Sq, Hq, Hkv, D, [96, 250], 32, 32, 64, mask="causal", p_sel=1.0)
    out, lse = run_bsa(case, out_dtype=torch.float32)
    table = np.full((B, 8), -1, dtype=np.int32)
    for b in range(B):
        ids = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]]
        table[b, :len(ids)] = ids
    pc = W.PrefillCase(case.q.reshape(B * Sq, Hq, D), case.k, case.v,
                       np.array([0, Sq, 2 * Sq], dtype=np.int32), table, case.seq_lens, "causal")
    out_p, lse_p = run_prefill(pc, out_dtype=torch.float32)
    assert (out.reshape(B * Sq, Hq, D) - out_p).abs().max().item() <= 1e-5
    assert (lse - lse_p).abs().max().item() <= 1e-5


def test_long_bsa_full():
    """Full-size long-context block-sparse workload (the launch the benchmark
    times): every output row and LSE of all 4 requests against the oracle, one
    request at a time."""
    case = W.long_bsa()
    _say("long_bsa: generated")
    out, lse = run_bsa(case)
    assert torch.isfinite(out.float()).all()
    for b in range(4):
        toks = [(b, i) for i in range(8192)]
        ref_o, ref_l = oracle_bsa(case, tokens=toks)
        _say("long_bsa: oracle request", b)
        assert_close(f64(out[b]), ref_o, TOL_BF16, f"out (request {b})")
        assert_close(f64(lse[b * 8192:(b + 1) * 8192]), ref_l, TOL_LSE, f"lse (request {b})")


# ----------------------------------------------------------------------------- prefill

PREFILL_SWEEP = [
    # B, qlens, prefixes, Hq, Hkv, D, ps, mask, w
    (3, [5, 130, 64], [0, 70, 300], 8, 2, 128, 16, "causal", -1),
    (2, [200, 33], [100, 0], 32, 8, 128, 32, "causal", 50),
    (2, [40, 77], [10, 20], 4, 4, 128, 64, "dense", -1),
    (2, [129, 7], [257, 1], 8, 1, 256, 128, "causal", -1),
    (1, [300], [0], 4, 2, 256, 32, "causal", 0),
]


@pytest.mark.parametrize("i", range(len(PREFILL_SWEEP)))
def test_prefill_sweep(i):
    B, ql, pf, Hq, Hkv, D, ps, mask, w = PREFILL_SWEEP[i]
    _say("prefill_sweep", PREFILL_SWEEP[i])
    case = W.make_prefill(400 + i, B, ql, pf, Hq, Hkv, D, ps, mask=mask, window_left=w,
                          extra_pages=2, output_scale=0.75)
    out, lse = run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _ = run_prefill(case, out_dtype=torch.float32, with_lse=False)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")


def test_prefill_growing_scores():
    """Key magnitudes grow along each request (row t scaled by 1 + t/50), so
    the running row max keeps rising: rises past the kernel's rescale slack
    rescale the running output, smaller ones keep the old reference."""
    case = W.make_prefill(470, 2, [64, 200], [900, 300], 8, 2, 128, 16, mask="causal",
                          extra_pages=2)
    ps = case.k.shape[2]
    k = case.k.float()
    for b, L in enumerate(case.seq_lens):
        for t in range(int(L)):
            k[int(case.block_tables[b, t // ps]), :, t % ps, :] *= 1.0 + t / 50.0
    case.k = k.to(torch.bfloat16)
    _say("prefill growing scores")
    out, lse = run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _ = run_prefill(case, out_dtype=torch.float32, with_lse=False)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")


@pytest.mark.parametrize("D", [128, 256])
def test_prefill_score_spikes(D):
    """Keys of the first 64 tokens scaled by 3 (a high early reference) and a
    random 5% of the later ones by 4 (scores far past it): within one launch
    some waves keep their reference for a tile, others find a lane whose
    probabilities would pass the rescale slack and take the row max."""
    case = W.make_prefill(480 + D, 2, [128, 300], [700, 500], 8, 2, D, 16, mask="causal",
                          extra_pages=2)
    ps = case.k.shape[2]
    k = case.k.float()
    rng = np.random.default_rng(D)
    for b, L in enumerate(case.seq_lens):
        for t in range(int(L)):
            f = 3.0 if t < 64 else (4.0 if rng.random() < 0.05 else 1.0)
            k[int(case.block_tables[b, t // ps]), :, t % ps, :] *= f
    case.k = k.to(torch.bfloat16)
    _say("prefill score spikes", D)
    out, lse = run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _ = run_prefill(case, out_dtype=torch.float32, with_lse=False)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")


@pytest.mark.parametrize("D,w", [(128, -1), (128, 1024), (256, -1)])
def test_batch_prefill_full(D, w):
    """Full-size batch prefill (the benchmark's shapes): every output row and LSE."""
    case = W.batch_prefill(3, D=D, window_left=w)
    _say("batch_prefill", D, w, int(case.qo_indptr[-1]))
    out, lse = run_prefill(case)
    ref_o, ref_l = oracle_prefill(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")


@pytest.mark.parametrize("D,w", [(128, -1), (128, 4096), (256, -1)])
def test_prefill_long_context_sampled(D, w):
    """Two requests with 64k- and 40k-token prefixes (about a thousand KV tiles
    per work item), causal; sampled rows against the oracle."""
    case = W.make_prefill(610 + D + max(w, 0), 2, [1024, 700], [65536, 40000], 32, 8, D, 32,
                          window_left=w)
    _say("prefill long context", D, w)
    out, lse = run_prefill(case)
    T = int(case.qo_indptr[-1])
    rows = [0, 1, 511, 1023, 1024, 1400, T - 1]
    ref_o, ref_l = oracle_prefill(case, rows=rows)
    assert_close(f64(out[rows]), ref_o, TOL_BF16, "out")
    assert_close(f64(lse[rows]), ref_l, TOL_LSE, "lse")
    assert torch.isfinite(out.float()).all()


# ----------------------------------------------------------------------------- decode

DECODE_SWEEP = [
    # B, Hq, Hkv, D, seq_lens, ps, mask, w, num_cus
    (4, 32, 8, 128, [1, 63, 64, 1000], 16, "dense", -1, 256),
    (3, 8, 8, 128, [4097, 5, 300], 16, "causal", 100, 256),
    (2, 16, 2, 256, [777, 2049], 32, "dense", -1, 256),
    (5, 4, 1, 128, [129, 1, 2000, 64, 65], 8, "causal", 0, 8),
    (2, 64, 1, 128, [333, 1024], 16, "dense", -1, 256),
]


def test_decode_growing_scores():
    """Key magnitudes grow along each request (row t scaled by 1 + t/100), so
    every split's running max keeps rising and its output is rescaled often;
    the merge then combines splits whose maxima differ widely."""
    case = W.make_decode(560, 3, 16, 4, 128, [3000, 700, 1500], 16, extra_pages=2)
    ps = case.k.shape[2]
    k = case.k.float()
    for b, L in enumerate(case.seq_lens):
        pages = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]]
        for t in range(int(L)):
            k[int(pages[t // ps]), :, t % ps, :] *= 1.0 + t / 100.0
    case.k = k.to(torch.bfloat16)
    _say("decode growing scores")
    out, lse, S = run_decode(case, num_cus=16)
    assert S > 1
    ref_o, ref_l = oracle_decode(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")


@pytest.mark.parametrize("i", range(len(DECODE_SWEEP)))
def test_decode_sweep(i):
    B, Hq, Hkv, D, sl, ps, mask, w, ncu = DECODE_SWEEP[i]
    _say("decode_sweep", DECODE_SWEEP[i])
    case = W.make_decode(500 + i, B, Hq, Hkv, D, sl, ps, mask=mask, window_left=w, extra_pages=2,
                         bmm2_scale=1.25)
    out, lse, S = run_decode(case, num_cus=ncu)
    ref_o, ref_l = oracle_decode(case)
    assert_close(f64(out), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _, _ = run_decode(case, out_dtype=torch.float32, num_cus=ncu)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")
    out_c, lse_c, _ = run_decode(case, combined=True, num_cus=ncu)
    assert torch.equal(out_c, out) and torch.equal(lse_c, lse)


# Wide batches run the single-pass kernel (whole (request, KV head) items
# split over the waves of a workgroup, merged in LDS).  A small num_cus makes
# small batches wide: several rounds of the snake deal per workgroup.
COOP_SWEEP = [
    # B, Hq, Hkv, D, seq_lens, ps, mask, w, num_cus
    (6, 32, 8, 128, [1, 31, 32, 33, 127, 1000], 16, "dense", -1, 4),
    (5, 16, 2, 256, [4097, 5, 300, 2049, 64], 32, "causal", 100, 3),
    (7, 4, 1, 128, [129, 1, 2000, 64, 65, 700, 3], 8, "causal", 0, 2),
    (4, 16, 1, 128, [333, 1024, 8, 5000], 16, "dense", -1, 2),       # G = 16
    (9, 8, 8, 128, [100] * 9, 16, "dense", -1, 4),                    # MHA, equal lengths
    (3, 32, 8, 256, [2, 130, 4096], 16, "causal", 1000, 12),
]


@pytest.mark.parametrize("i", range(len(COOP_SWEEP)))
def test_decode_single_pass_sweep(i):
    B, Hq, Hkv, D, sl, ps, mask, w, ncu = COOP_SWEEP[i]
    _say("decode single-pass sweep", COOP_SWEEP[i])
    assert P.paged_decode_workspace_size(B, Hq, Hkv, D, max(sl), ps, ncu)[:2] == (0, 1)
    case = W.make_decode(530 + i, B, Hq, Hkv, D, sl, ps, mask=mask, window_left=w, extra_pages=2,
                         bmm2_scale=0.8)
    out, lse, S = run_decode(case, num_cus=ncu)
    assert S == 1
    ref_o, ref_l = oracle_decode(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, lse32, _ = run_decode(case, out_dtype=torch.float32, num_cus=ncu)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")
    assert_close(f64(lse32), ref_l, TOL_LSE, "lse (fp32 run)")
    out_c, lse_c, _ = run_decode(case, combined=True, num_cus=ncu)
    assert torch.equal(out_c, out) and torch.equal(lse_c, lse)


def test_decode_single_pass_growing_scores():
    """Key magnitudes grow along each request, so the waves that share an item
    end with very different running maxima; their LDS merge must weight them
    by those maxima."""
    case = W.make_decode(561, 3, 16, 4, 128, [3000, 700, 1500], 16, extra_pages=2)
    ps = case.k.shape[2]
    k = case.k.float()
    for b, L in enumerate(case.seq_lens):
        pages = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]]
        for t in range(int(L)):
            k[int(pages[t // ps]), :, t % ps, :] *= 1.0 + t / 100.0
    case.k = k.to(torch.bfloat16)
    _say("decode single-pass growing scores")
    out, lse, S = run_decode(case, num_cus=2)
    assert S == 1
    ref_o, ref_l = oracle_decode(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")


@pytest.mark.parametrize("mask,w", [("dense", -1), ("causal", 50000)])
def test_decode_long_requests_many_splits(mask, w):
    """Requests of 131,072 and 100,000 tokens: the split policy cuts them into
    about a thousand chunks, so the merge combines that many partials per row."""
    case = W.make_decode(590, 2, 32, 8, 128, [131072, 100000], 16, mask=mask, window_left=w)
    _say("decode long requests", mask, w)
    out, lse, S = run_decode(case)
    assert S > 256
    ref_o, ref_l = oracle_decode(case)
    assert_close(f64(out), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _, _ = run_decode(case, out_dtype=torch.float32)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")


def test_batch_decode_full():
    """The headline batch decode workload: every request's output and LSE."""
    case = W.batch_decode()
    _say("batch_decode: generated", int(case.seq_lens.sum()))
    out, lse, S = run_decode(case)
    ref_o, ref_l = oracle_decode(case)
    assert_close(f64(out), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")


# ----------------------------------------------------------------------------- multi-token decode

DECODE_Q_SWEEP = [
    # B, Hq, Hkv, D, seq_lens, ps, SQ (fixed) or qlens (packed), mask, w, num_cus
    (4, 32, 8, 128, [4, 63, 1000, 3000], 16, 4, "causal", -1, 256),
    (2, 8, 1, 256, [40, 64], 16, 3, "dense", -1, 256),            # one split
    (4, 32, 8, 128, [10, 500, 2, 4097], 16, [1, 5, 2, 7], "causal", 50, 256),
    (2, 32, 2, 128, [300, 5000], 32, [8, 3], "causal", -1, 64),   # 2 row tiles
    (2, 64, 1, 128, [200, 77], 16, [3, 1], "dense", -1, 256),     # G=64
    (3, 16, 4, 256, [5, 129, 700], 8, [5, 1, 4], "causal", 0, 16),  # qlen == L
    # rows of a KV head fit 16 columns (tokens x group <= 16): the dedicated kernel
    (4, 32, 8, 128, [9, 3000, 4, 700], 16, [1, 4, 2, 3], "causal", 40, 256),
    (3, 16, 8, 128, [16, 2049, 90], 16, [8, 3, 1], "causal", -1, 64),
    (2, 4, 4, 128, [16, 1500], 16, [16, 9], "causal", 5, 256),        # MHA, qlen == L
    (2, 32, 8, 256, [333, 4097], 32, 2, "dense", -1, 256),
    (3, 8, 2, 128, [40, 64, 50], 16, 4, "causal", -1, 256),            # one split
]


# single-pass kernel (tokens x group <= 16 and a wide batch for the given num_cus)
DECODE_Q_COOP_SWEEP = [
    (4, 32, 8, 128, [9, 3000, 4, 700], 16, [1, 4, 2, 3], "causal", 40, 8),
    (5, 16, 4, 256, [16, 2049, 90, 5, 64], 16, 4, "causal", -1, 4),
    (3, 4, 4, 128, [16, 1500, 40], 16, [16, 9, 1], "causal", 5, 2),     # MHA, qlen == L
    (4, 8, 2, 128, [77, 1, 300, 4100], 16, 1, "dense", -1, 3),
]


@pytest.mark.parametrize("i", range(len(DECODE_Q_COOP_SWEEP)))
def test_decode_q_single_pass_sweep(i):
    B, Hq, Hkv, D, sl, ps, sq, mask, w, ncu = DECODE_Q_COOP_SWEEP[i]
    _say("decode_q single-pass sweep", DECODE_Q_COOP_SWEEP[i])
    fixed = isinstance(sq, int)
    case = W.make_decode_q(740 + i, B, Hq, Hkv, D, sl, ps, seq_len_q=sq if fixed else None,
                           qlens=None if fixed else sq, mask=mask, window_left=w, extra_pages=2)
    out, lse, S = run_decode_q(case, num_cus=ncu)
    assert S == 1
    ref_o, ref_l = oracle_decode_q(case)
    assert_close(f64(out), ref_o, TOL_BF16, "out")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _, _ = run_decode_q(case, out_dtype=torch.float32, num_cus=ncu)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")


def test_batch_decode_q_full():
    """The multi-token decode workload the benchmark times (B=64, 4 query tokens
    per request, causal): every output row and LSE."""
    case = W.batch_decode_q()
    _say("batch_decode_q: generated", int(case.seq_lens.sum()))
    out, lse, S = run_decode_q(case)
    ref_o, ref_l = oracle_decode_q(case)
    assert_close(f64(out), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")


@pytest.mark.parametrize("i", range(len(DECODE_Q_SWEEP)))
def test_decode_q_sweep(i):
    B, Hq, Hkv, D, sl, ps, sq, mask, w, ncu = DECODE_Q_SWEEP[i]
    _say("decode_q_sweep", DECODE_Q_SWEEP[i])
    fixed = isinstance(sq, int)
    case = W.make_decode_q(700 + i, B, Hq, Hkv, D, sl, ps, seq_len_q=sq if fixed else None,
                           qlens=None if fixed else sq, mask=mask, window_left=w, extra_pages=2)
    out, lse, S = run_decode_q(case, num_cus=ncu)
    ref_o, ref_l = oracle_decode_q(case)
    assert_close(f64(out), ref_o, TOL_BF16, f"out (splits={S})")
    assert_close(f64(lse), ref_l, TOL_LSE, "lse")
    out32, _, _ = run_decode_q(case, out_dtype=torch.float32, num_cus=ncu)
    assert_close(f64(out32), ref_o, TOL_F32, "out fp32")
