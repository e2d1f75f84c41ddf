"""Graph capture of the planned run calls.

Each path is planned from static capacities, its ``run`` is captured once in a
HIP graph (torch.cuda.CUDAGraph), and the graph is replayed while the live
metadata (lengths, page IDs, sparse selections, query offsets) and the Q / K / V
contents change between replays within the plan's bounds.  Eager work (the
copies that stage the next case and an eager run) and device synchronisation
sit between replays.  Every replay must equal an eager run of the same call on
the same buffers bit for bit, and the oracle to the usual bars.
"""
import sys

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from gen import workloads as W
from oracle import attention as A
from tests.gpu_util import (DEV, TOL_BF16, TOL_LSE, assert_close, dev_i32, f64, oracle_bsa,
                            oracle_decode, oracle_decode_q)

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _stage(dst, src):
    """Copy a CPU tensor / numpy array into the leading rows of a device buffer."""
    if isinstance(src, np.ndarray):
        src = torch.from_numpy(np.ascontiguousarray(src))
    src = src.reshape(-1, *dst.shape[1:]) if dst.dim() > 1 else src.reshape(-1)
    dst[:src.shape[0]].copy_(src.to(dst.dtype) if src.dtype != dst.dtype else src)


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                     # warm-up launch outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _pool(cases, attr):
    return max(getattr(c, attr).shape[0] for c in cases)


# ----------------------------------------------------------------------------- block-sparse

def test_graph_bsa_replays_with_changing_metadata():
    B, Sq, Hq, Hkv, D, ps, qbs, kvbs, maxlen = 2, 96, 8, 2, 128, 16, 16, 32, 400
    cases = [W.make_bsa(900 + r, B, Sq, Hq, Hkv, D, L, ps, qbs, kvbs, mask="causal",
                        bits_p=0.9, max_seq_len_kv=maxlen, extra_pages=r)
             for r, L in enumerate([[200, 333], [400, 96], [97, 250], [320, 400]])]
    Pcap = _pool(cases, "k")
    k = torch.zeros(Pcap, Hkv, ps, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    q = torch.empty(B, Sq, Hq, D, dtype=torch.bfloat16, device=DEV)
    ip = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    ix = torch.zeros(max(c.kv_indices.size for c in cases), dtype=torch.int32, device=DEV)
    bip = torch.empty(B, Hkv, Sq // qbs + 1, dtype=torch.int32, device=DEV)
    bix = torch.zeros(max(c.block_indices.size for c in cases), dtype=torch.int32, device=DEV)
    sl = torch.empty(B, dtype=torch.int32, device=DEV)
    bits = torch.empty(B, -(-maxlen // 32), dtype=torch.int32, device=DEV)
    out = torch.empty(B, Sq, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B * Sq, Hq, dtype=torch.float32, device=DEV)
    w = P.BlockSparsePagedWrapper(B, Sq, Hq, Hkv, D, Pcap, ps, qbs, kvbs, maxlen, "causal")

    def stage(c):
        for dst, src in ((q, c.q), (k, c.k), (v, c.v), (ip, c.kv_indptr), (ix, c.kv_indices),
                         (bip, c.block_indptr), (bix, c.block_indices), (sl, c.seq_lens),
                         (bits, c.valid_bits.view(np.int32))):
            _stage(dst, src)

    def run(o=out, l=lse):
        w.run(q, (k, v), ip, ix, bip, bix, sl, kv_valid_bits=bits, out=o, lse=l)

    stage(cases[0])
    g = _capture(run)
    for r in range(REPLAYS):
        c = cases[r % len(cases)]
        _say("bsa graph replay", r, c.seq_lens.tolist())
        stage(c)
        g.replay()
        torch.cuda.synchronize()
        go, gl = out.clone(), lse.clone()
        eo, el = torch.empty_like(out), torch.empty_like(lse)
        run(eo, el)
        torch.cuda.synchronize()
        assert torch.equal(go, eo) and torch.equal(gl, el), f"replay {r} differs from eager"
        ref_o, ref_l = oracle_bsa(c)
        assert_close(f64(go), ref_o, TOL_BF16, f"out replay {r}")
        assert_close(f64(gl), ref_l, TOL_LSE, f"lse replay {r}")


# ----------------------------------------------------------------------------- prefill

def test_graph_prefill_capacity_plan_replays():
    B, Hq, Hkv, D, ps, max_qlen, total_cap, width = 3, 16, 4, 128, 32, 300, 600, 40
    shapes = [([300, 17, 200], [0, 500, 64]), ([1, 1, 1], [900, 0, 5]),
              ([150, 299, 90], [1000, 3, 0]), ([64, 64, 64], [64, 64, 64])]
    cases = [W.make_prefill(950 + r, B, ql, pf, Hq, Hkv, D, ps, extra_pages=r)
             for r, (ql, pf) in enumerate(shapes)]
    Pcap = _pool(cases, "k")
    k = torch.zeros(Pcap, Hkv, ps, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    q = torch.zeros(total_cap, Hq, D, dtype=torch.bfloat16, device=DEV)
    qo = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    bt = torch.full((B, width), -1, dtype=torch.int32, device=DEV)
    sl = torch.empty(B, dtype=torch.int32, device=DEV)
    out = torch.zeros(total_cap, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(total_cap, Hq, dtype=torch.float32, device=DEV)
    w = P.BatchPrefillPagedWrapper.for_capacity(B, max_qlen, total_cap, Hq, Hkv, D, Pcap, ps,
                                                width, mask_type="causal")

    def stage(c):
        assert c.block_tables.shape[1] <= width
        bt.fill_(-1)
        bt[:, :c.block_tables.shape[1]].copy_(torch.from_numpy(c.block_tables))
        for dst, src in ((q, c.q), (k, c.k), (v, c.v), (qo, c.qo_indptr), (sl, c.seq_lens)):
            _stage(dst, src)

    def run(o=out, l=lse):
        w.run(q, k, v, qo, bt, sl, out=o, lse=l)

    stage(cases[0])
    g = _capture(run)
    for r in range(REPLAYS):
        c = cases[r % len(cases)]
        n = int(c.qo_indptr[-1])
        _say("prefill graph replay", r, np.diff(c.qo_indptr).tolist(), c.seq_lens.tolist())
        stage(c)
        g.replay()
        torch.cuda.synchronize()
        go, gl = out[:n].clone(), lse[:n].clone()
        eo, el = torch.empty_like(out), torch.empty_like(lse)
        run(eo, el)
        torch.cuda.synchronize()
        assert torch.equal(go, eo[:n]) and torch.equal(gl, el[:n]), f"replay {r} differs from eager"
        ref_o, ref_l = A.prefill_reference(c.q, c.k, c.v, c.qo_indptr, c.block_tables,
                                           c.seq_lens, mask="causal")
        assert_close(f64(go), ref_o, TOL_BF16, f"out replay {r}")
        assert_close(f64(gl), ref_l, TOL_LSE, f"lse replay {r}")


# ----------------------------------------------------------------------------- decode

@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 2)])
def test_graph_decode_replays(Hq, Hkv):
    B, D, ps, maxlen = 4, 128, 16, 3000
    lens = [[1, 3000, 70, 900], [2999, 5, 1200, 64], [640, 641, 1, 2048], [3000, 3000, 3000, 3000]]
    cases = [W.make_decode(960 + r, B, Hq, Hkv, D, L, ps, extra_pages=r, max_seq_len=maxlen)
             for r, L in enumerate(lens)]
    Pcap = _pool(cases, "k")
    k = torch.zeros(Pcap, Hkv, ps, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    ip = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    ix = torch.zeros(max(c.kv_indices.size for c in cases), dtype=torch.int32, device=DEV)
    sl = torch.empty(B, dtype=torch.int32, device=DEV)
    nbytes, S, _ = P.paged_decode_workspace_size(B, Hq, Hkv, D, maxlen, ps)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)

    def stage(c):
        for dst, src in ((q, c.q), (k, c.k), (v, c.v), (ip, c.kv_indptr), (ix, c.kv_indices),
                         (sl, c.seq_lens)):
            _stage(dst, src)

    def run(o=out, l=lse):
        P.paged_decode_run(q, (k, v), ip, ix, sl, maxlen, ws, out=o, lse=l)

    stage(cases[0])
    g = _capture(run)
    for r in range(REPLAYS):
        c = cases[r % len(cases)]
        _say("decode graph replay", Hq, Hkv, r, c.seq_lens.tolist(), "splits", S)
        stage(c)
        g.replay()
        torch.cuda.synchronize()
        go, gl = out.clone(), lse.clone()
        eo, el = torch.empty_like(out), torch.empty_like(lse)
        run(eo, el)
        torch.cuda.synchronize()
        assert torch.equal(go, eo) and torch.equal(gl, el), f"replay {r} differs from eager"
        ref_o, ref_l = oracle_decode(c)
        assert_close(f64(go), ref_o, TOL_BF16, f"out replay {r}")
        assert_close(f64(gl), ref_l, TOL_LSE, f"lse replay {r}")


# Single-pass decode (a wide batch for the given num_cus) and the allocation-free
# entry point (its split partials in the library's fixed scratch) under capture.
@pytest.mark.parametrize("entry,ncu", [("run", 4), ("noalloc", 4), ("noalloc", 256)])
def test_graph_decode_single_pass_and_noalloc_replays(entry, ncu):
    B, Hq, Hkv, D, ps, maxlen = 6, 32, 8, 128, 16, 3000
    lens = [[1, 3000, 70, 900, 33, 2048], [2999, 5, 1200, 64, 640, 1],
            [640, 641, 1, 2048, 3000, 17], [3000] * 6]
    cases = [W.make_decode(990 + r, B, Hq, Hkv, D, L, ps, extra_pages=r, max_seq_len=maxlen)
             for r, L in enumerate(lens)]
    _, S, _ = P.paged_decode_workspace_size(B, Hq, Hkv, D, maxlen, ps, ncu)
    assert (S == 1) == (ncu == 4)
    Pcap = _pool(cases, "k")
    k = torch.zeros(Pcap, Hkv, ps, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    ip = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    ix = torch.zeros(max(c.kv_indices.size for c in cases), dtype=torch.int32, device=DEV)
    sl = torch.empty(B, dtype=torch.int32, device=DEV)
    nbytes, _, _ = P.paged_decode_workspace_size(B, Hq, Hkv, D, maxlen, ps, ncu)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)

    def stage(c):
        for dst, src in ((q, c.q), (k, c.k), (v, c.v), (ip, c.kv_indptr), (ix, c.kv_indices),
                         (sl, c.seq_lens)):
            _stage(dst, src)

    def run(o=out, l=lse):
        if entry == "run":
            P.paged_decode_run(q, (k, v), ip, ix, sl, maxlen, ws, out=o, lse=l, num_cus_=ncu)
        else:
            P.paged_decode_run_noalloc(q, (k, v), ip, ix, sl, maxlen, out=o, lse=l, num_cus_=ncu)

    stage(cases[0])
    g = _capture(run)
    for r in range(REPLAYS):
        c = cases[r % len(cases)]
        _say("decode graph replay", entry, ncu, r, c.seq_lens.tolist(), "splits", S)
        stage(c)
        g.replay()
        torch.cuda.synchronize()
        go, gl = out.clone(), lse.clone()
        eo, el = torch.empty_like(out), torch.empty_like(lse)
        run(eo, el)
        torch.cuda.synchronize()
        assert torch.equal(go, eo) and torch.equal(gl, el), f"replay {r} differs from eager"
        ref_o, ref_l = oracle_decode(c)
        assert_close(f64(go), ref_o, TOL_BF16, f"out replay {r}")
        assert_close(f64(gl), ref_l, TOL_LSE, f"lse replay {r}")


@pytest.mark.parametrize("max_q", [6, 4])     # 6 x 4 heads: general kernel; 4 x 4: decode kernel
def test_graph_decode_q_packed_replays(max_q):
    B, Hq, Hkv, D, ps, maxlen, total_cap = 3, 32, 8, 128, 16, 2000, 18
    shapes = [([6, 1, 3], [6, 2000, 40]), ([1, 1, 1], [1, 1, 1]), ([5, 6, 6], [1999, 64, 700]),
              ([2, 4, 1], [100, 1000, 2000])]
    shapes = [([min(q, max_q) for q in ql], L) for ql, L in shapes]
    cases = [W.make_decode_q(970 + r, B, Hq, Hkv, D, L, ps, qlens=ql, mask="causal",
                             extra_pages=r) for r, (ql, L) in enumerate(shapes)]
    for c in cases:
        c.seq_len_q, c.max_seq_len = max_q, maxlen
    Pcap = _pool(cases, "k")
    k = torch.zeros(Pcap, Hkv, ps, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    q = torch.zeros(total_cap, Hq, D, dtype=torch.bfloat16, device=DEV)
    qo = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    ip = torch.empty(B + 1, dtype=torch.int32, device=DEV)
    ix = torch.zeros(max(c.kv_indices.size for c in cases), dtype=torch.int32, device=DEV)
    sl = torch.empty(B, dtype=torch.int32, device=DEV)
    nbytes, S, _ = P.paged_decode_q_workspace_size(B, max_q, Hq, Hkv, D, maxlen, ps)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.zeros(total_cap, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(total_cap, Hq, dtype=torch.float32, device=DEV)

    def stage(c):
        for dst, src in ((q, c.q), (k, c.k), (v, c.v), (qo, c.qo_indptr), (ip, c.kv_indptr),
                         (ix, c.kv_indices), (sl, c.seq_lens)):
            _stage(dst, src)

    def run(o=out, l=lse):
        P.paged_decode_q_run(q, (k, v), ip, ix, sl, maxlen, ws, qo_indptr=qo,
                             max_seq_len_q=max_q, mask_type="causal", out=o, lse=l)

    stage(cases[0])
    g = _capture(run)
    for r in range(REPLAYS):
        c = cases[r % len(cases)]
        n = int(c.qo_indptr[-1])
        _say("decode_q graph replay", r, np.diff(c.qo_indptr).tolist(), "splits", S)
        stage(c)
        g.replay()
        torch.cuda.synchronize()
        go, gl = out[:n].clone(), lse[:n].clone()
        eo, el = torch.empty_like(out), torch.empty_like(lse)
        run(eo, el)
        torch.cuda.synchronize()
        assert torch.equal(go, eo[:n]) and torch.equal(gl, el[:n]), f"replay {r} differs from eager"
        ref_o, ref_l = oracle_decode_q(c)
        assert_close(f64(go), ref_o, TOL_BF16, f"out replay {r}")
        assert_close(f64(gl), ref_l, TOL_LSE, f"lse replay {r}")


# ----------------------------------------------------------------------------- sage

def test_graph_sage_replays_with_changing_selection():
    cases = [W.sage_small(980 + r, block_sizes_rank=3) for r in range(REPLAYS)]
    c0 = cases[0]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)  # noqa: E731
    names = ("q_int8", "k_int8", "v_fp8", "q_scale", "k_scale", "v_scale")
    bufs = {n: getattr(c0, n).to(DEV).clone() for n in names}
    idx, nums, bsz = t(c0.q2k_block_index), t(c0.q2k_block_nums), t(c0.block_sizes)
    B, H, Sq, _ = c0.q_int8.shape
    out = torch.empty(B, H, Sq, 128, dtype=torch.bfloat16, device=DEV)

    def run(o=out):
        P.bsa_sage_run(bufs["q_int8"], bufs["k_int8"], bufs["v_fp8"], bufs["q_scale"],
                       bufs["k_scale"], bufs["v_scale"], idx, c0.block_sparse_num, bsz, nums,
                       c0.softmax_scale, out=o)

    g = _capture(run)
    for r in range(REPLAYS):
        c = cases[r]
        _say("sage graph replay", r)
        for n in names:
            bufs[n].copy_(getattr(c, n).to(DEV))
        for dst, src in ((idx, c.q2k_block_index), (nums, c.q2k_block_nums), (bsz, c.block_sizes)):
            dst.copy_(t(src))
        g.replay()
        torch.cuda.synchronize()
        go = out.clone()
        eo = torch.empty_like(out)
        run(eo)
        torch.cuda.synchronize()
        assert torch.equal(go, eo), f"replay {r} differs from eager"
        ref = A.sage_reference(c.q_int8, c.k_int8, c.v_fp8.view(torch.uint8).numpy(), c.q_scale,
                               c.k_scale, c.v_scale, c.q2k_block_index, c.block_sparse_num,
                               c.block_sizes, c.q2k_block_nums, c.uniform_block_count,
                               c.softmax_scale, Sk=c.Sk)
        assert_close(f64(go), ref, 5e-2, f"sage replay {r}")
