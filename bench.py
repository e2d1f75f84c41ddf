#!/usr/bin/env python3
"""Benchmark of the paged / block-sparse attention path on one MI355X.

Headline (the single JSON line's ``value``): batch paged decode, KV-read GB/s --
B=64 requests, Hq=32 / Hkv=8, D=128, seq_lens ~ U{512..8192}, 16-token pages
with randomly permuted CSR page IDs, bf16.  One step = one decode call over the
whole batch (at this batch width a single kernel; narrower batches add a small
merge kernel after the split-KV kernel).

Secondary entries (same JSON line, ``secondary``): long-context block-sparse
attention (B=4, S=8192, Hq=32/Hkv=8, 16 blocks of 64 per BSR row, causal, 1%
invalid bits), packed causal prefill (B=8, qlen ~ U{256..2048} + prefix
~ U{0..2048}), the Sage-style int8/fp8 block-sparse case (B=2, H=16, S=16384,
64 of 256 blocks per query block) and the tiny block-sparse case -- each as
TFLOP/s (TOP/s) over the admitted (query, key) pairs only (4*D operations per
admitted pair and query head).

Timing: inputs are generated (seeded), copied to HBM and planned before the
timed region; W warm-up launches, then K launches bracketed by device
synchronisation, each launch also bracketed by HIP events on the stream it is
enqueued on (torch's current stream).  ``cpu_baseline`` times the fp64 oracle
on a bounded sample of the headline workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
INT8_PEAK_TOPS = 5000.0        # dense int8 / fp8 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------- HBM traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def _sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernels, workload):
    """HBM bytes per launch of the named kernels on one workload, from the counter
    runs recorded in profiles/hbm_traffic.md (FETCH_SIZE and WRITE_SIZE per
    dispatch, each scaled by what the same counter reads for a plain copy of
    known size).  None when a kernel has no record for the workload or its
    source changed since the record was taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    recs = {}
    for ln in lines:
        if not ln.startswith("traffic-record:"):
            continue
        f = dict(kv.split("=", 1) for kv in ln.split()[1:])
        recs[(f["kernel"], f["workload"])] = f
    total = 0
    for k in kernels:
        r = recs.get((k, workload))
        if r is None or _sha256([os.path.join(ROOT, x) for x in r["source"].split(",")]) != r["sha256"]:
            return None
        total += int(r["bytes_per_launch"])
    return total


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


WARMUP_MIN_S = 0.2   # untimed warmup keeps going until this much wall time has passed


def time_launches(fn, steps, warmup):
    """Run fn() at least `warmup` times, and on until WARMUP_MIN_S of untimed
    work has run (the engine clock ramps up over the first tens of ms of
    sustained load; timed right after a few calls, a kernel reads up to 10%
    slow).  Then time `steps` back-to-back calls between two events (the step
    time: nothing else is enqueued between the launches), then `steps` more
    calls each bracketed by its own events (the mean launch duration).
    Returns (total_ms / steps, mean per-launch ms)."""
    t_start = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t_start < WARMUP_MIN_S:
        for _ in range(max(1, warmup)):
            fn()
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return t0.elapsed_time(t1) / steps, float(np.mean(per))


# ---------------------------------------------------------------------------- work counts

def bsa_admitted_pairs(case, use_bits=True):
    """Admitted (query token, key) pairs summed over query heads."""
    B, Sq, Hq, Hkv, D, P, ps = case.dims
    G = Hq // Hkv
    qbs, kvbs = case.q_block_size, case.kv_block_size
    causal = case.mask == "causal"
    w = case.window_left
    total = 0
    for b in range(B):
        L = int(case.seq_lens[b])
        valid = np.ones(L, dtype=np.int64)
        if use_bits and case.valid_bits is not None:
            words = case.valid_bits[b].astype(np.uint64)
            j = np.arange(L)
            valid = ((words[j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)).astype(np.int64)
        C = np.concatenate([[0], np.cumsum(valid)])
        for g in range(Hkv):
            for r in range(case.block_indptr.shape[2] - 1):
                lo_, hi_ = case.block_indptr[b, g, r], case.block_indptr[b, g, r + 1]
                blk = np.unique(case.block_indices[lo_:hi_]).astype(np.int64)
                if blk.size == 0:
                    continue
                i = np.arange(r * qbs, min((r + 1) * qbs, Sq))
                p = L - Sq + i
                a0 = np.clip(blk * kvbs, 0, L)[None, :]
                a1 = np.clip(blk * kvbs + kvbs, 0, L)[None, :]
                hi = np.minimum(a1, (p + 1)[:, None]) if causal else a1
                lo = np.maximum(a0, (p - w)[:, None]) if w >= 0 else a0
                hi = np.clip(hi, 0, L)
                lo = np.clip(lo, 0, L)
                total += int(np.sum(np.where(hi > lo, C[hi] - C[lo], 0)))
    return total * G


def prefill_admitted_pairs(case):
    Hq = case.q.shape[1]
    total = 0
    for b in range(len(case.seq_lens)):
        L = int(case.seq_lens[b])
        qlen = int(case.qo_indptr[b + 1] - case.qo_indptr[b])
        p = L - qlen + np.arange(qlen)
        hi = np.minimum(L, p + 1) if case.mask == "causal" else np.full(qlen, L)
        lo = np.maximum(0, p - case.window_left) if case.window_left >= 0 else np.zeros(qlen, int)
        total += int(np.sum(np.maximum(hi - lo, 0)))
    return total * Hq


# ---------------------------------------------------------------------------- workloads

def bench_decode(steps, warmup, W, P):
    log("decode: generating inputs")
    case = W.batch_decode()
    B, Hq, D = case.q.shape
    Hkv, ps = case.k.shape[1], case.k.shape[2]
    q = case.q.cuda()
    k = case.k.cuda()
    v = case.v.cuda()
    ip, ix, sl = dev_i32(case.kv_indptr), dev_i32(case.kv_indices), dev_i32(case.seq_lens)
    nbytes, S, split_len = P.paged_decode_workspace_size(B, Hq, Hkv, D, case.max_seq_len, ps)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    P.paged_decode_validate(B, k.shape[0], ps, case.max_seq_len, case.kv_indptr,
                            case.kv_indices, case.seq_lens)

    def step():
        P.paged_decode_run(q, (k, v), ip, ix, sl, case.max_seq_len, ws, out=out, lse=lse)

    ms_step, ms_launch = time_launches(step, steps, warmup)
    kv_bytes = int(case.seq_lens.astype(np.int64).sum()) * Hkv * D * 2 * 2
    gbs = kv_bytes / (ms_step * 1e-3) / 1e9
    ach = kv_bytes / (ms_launch * 1e-3) / 1e9
    cfg = {"workload": "batch paged decode B=64 Hq=32 Hkv=8 D=128 seq_lens~U[512,8192] "
                       "page_size=16 bf16 (seed 2)",
           "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "page_size": ps,
           "sum_seq_len": int(case.seq_lens.sum()), "num_splits": S, "split_len": split_len,
           "kv_bytes_per_step": kv_bytes}
    kern = ["decode_coop_kernel<128>"] if S == 1 else ["decode_kernel<128>", "decode_merge_kernel<128>"]
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kern, "decode"),
            "kernel": " + ".join(kern) + " (one step)",
            "per_unit": "4096 B of K+V per live token (Hkv=8, D=128, bf16)"}
    return case, gbs, ms_step, cfg, roof


def bench_decode_q(steps, warmup, W, P, SQ=4):
    log(f"decode_q: generating inputs (SQ={SQ})")
    case = W.batch_decode_q(SQ=SQ)
    B, _, Hq, D = case.q.shape
    Hkv, ps = case.k.shape[1], case.k.shape[2]
    q = case.q.cuda()
    k = case.k.cuda()
    v = case.v.cuda()
    ip, ix, sl = dev_i32(case.kv_indptr), dev_i32(case.kv_indices), dev_i32(case.seq_lens)
    nbytes, S, split_len = P.paged_decode_q_workspace_size(B, SQ, Hq, Hkv, D, case.max_seq_len, ps)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(B, SQ, Hq, dtype=torch.float32, device="cuda")
    P.paged_decode_q_validate(B, k.shape[0], ps, case.max_seq_len, case.kv_indptr,
                              case.kv_indices, case.seq_lens, seq_len_q=SQ)

    def step():
        P.paged_decode_q_run(q, (k, v), ip, ix, sl, case.max_seq_len, ws, mask_type="causal",
                             out=out, lse=lse)

    ms_step, ms_launch = time_launches(step, steps, warmup)
    kv_bytes = int(case.seq_lens.astype(np.int64).sum()) * Hkv * D * 2 * 2
    kern = ["decode_coop_kernel<128>"] if S == 1 else ["decode_kernel<128>", "decode_merge_kernel<128>"]
    return {"workload": f"multi-token paged decode B=64 SQ={SQ} Hq=32 Hkv=8 D=128 causal "
                        "seq_lens~U[512,8192] page_size=16 bf16 (seed 2)",
            "metric": "decode KV-read GB/s", "value": round(kv_bytes / (ms_step * 1e-3) / 1e9, 1),
            "unit": "GB/s", "ms_per_step": round(ms_step, 4), "num_splits": S,
            "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "achieved": round(kv_bytes / (ms_launch * 1e-3) / 1e9, 1),
                         "frac": round(kv_bytes / (ms_launch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(kern, "decode_q"),
                         "kernel": " + ".join(kern) + " (16 query rows per KV head: 4 tokens x "
                                   "4 heads)"}}


def bench_bsa_long(steps, warmup, W, P):
    log("long block-sparse: generating inputs")
    case = W.long_bsa()
    B, Sq, Hq, Hkv, D, Pn, ps = case.dims
    q = case.q.cuda()
    k, v = case.k.cuda(), case.v.cuda()
    ip, ix = dev_i32(case.kv_indptr), dev_i32(case.kv_indices)
    bip, bix, sl = dev_i32(case.block_indptr), dev_i32(case.block_indices), dev_i32(case.seq_lens)
    bits = torch.from_numpy(case.valid_bits.view(np.int32)).cuda()
    wr = P.BlockSparsePagedWrapper(B, Sq, Hq, Hkv, D, Pn, ps, 64, 64, Sq, "causal")
    P.bsa_validate(wr.plan, case.kv_indptr, case.kv_indices, case.block_indptr,
                   case.block_indices, case.seq_lens)
    out = torch.empty_like(q)
    lse = torch.empty(B * Sq, Hq, dtype=torch.float32, device="cuda")

    def step():
        wr.run(q, (k, v), ip, ix, bip, bix, sl, bits, None, out, lse)

    ms_step, ms_launch = time_launches(step, steps, warmup)
    pairs = bsa_admitted_pairs(case)
    flops = 4.0 * D * pairs
    tf = flops / (ms_step * 1e-3) / 1e12
    ach = flops / (ms_launch * 1e-3) / 1e12
    return {"workload": "long block-sparse paged attention B=4 S=8192 Hq=32 Hkv=8 D=128 "
                        "page=64 q/kv block 64, 16 blocks/row, causal, 1% invalid bits",
            "metric": "block-sparse paged attn TFLOP/s (admitted pairs)", "value": round(tf, 2),
            "unit": "TFLOP/s", "ms_per_step": round(ms_step, 4), "admitted_pairs": pairs,
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(["attn_fwd_kernel<128,%d,bsa>" % wr.plan.waves], "bsa"),
                         "kernel": "attn_fwd_kernel<128,%d,bsa>" % wr.plan.waves}}


def bench_prefill(steps, warmup, W, P, D=128, window_left=-1):
    log(f"prefill D={D} w={window_left}: generating inputs")
    case = W.batch_prefill(3, D=D, window_left=window_left)
    q = case.q.cuda()
    k, v = case.k.cuda(), case.v.cuda()
    qo, bt, sl = dev_i32(case.qo_indptr), dev_i32(case.block_tables), dev_i32(case.seq_lens)
    wr = P.BatchPrefillPagedWrapper(case.qo_indptr, case.seq_lens, q.shape[1], k.shape[1], D,
                                    k.shape[0], k.shape[2], case.block_tables.shape[1], "causal",
                                    window_left, validate_tables=case.block_tables)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")

    def step():
        wr.run(q, k, v, qo, bt, sl, None, 1.0, out, lse)

    ms_step, ms_launch = time_launches(step, steps, warmup)
    pairs = prefill_admitted_pairs(case)
    flops = 4.0 * D * pairs
    tf = flops / (ms_step * 1e-3) / 1e12
    ach = flops / (ms_launch * 1e-3) / 1e12
    return {"workload": f"batch paged prefill B=8 causal window_left={window_left} Hq=32 "
                        f"Hkv=8 D={D} page=32 total_q={int(case.qo_indptr[-1])}",
            "metric": "paged prefill TFLOP/s (admitted pairs)", "value": round(tf, 2),
            "unit": "TFLOP/s", "ms_per_step": round(ms_step, 4), "admitted_pairs": pairs,
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(
                             ["attn_fwd_kernel<%d,%d,prefill>" % (D, wr.plan.waves)],
                             "prefill_d%d_w%d" % (D, window_left)),
                         "kernel": "attn_fwd_kernel<%d,%d,prefill>" % (D, wr.plan.waves)}}


def bench_bsa_tiny(steps, warmup, W, P):
    case = W.tiny_bsa("causal")
    B, Sq, Hq, Hkv, D, Pn, ps = case.dims
    q = case.q.cuda()
    k, v = case.k.cuda(), case.v.cuda()
    args = [dev_i32(x) for x in (case.kv_indptr, case.kv_indices, case.block_indptr,
                                 case.block_indices, case.seq_lens)]
    bits = torch.from_numpy(case.valid_bits.view(np.int32)).cuda()
    wr = P.BlockSparsePagedWrapper(B, Sq, Hq, Hkv, D, Pn, ps, 16, 32, 333, "causal")
    out = torch.empty_like(q)

    def step():
        wr.run(q, (k, v), *args, bits, case.sm_scale, out)

    ms_step, ms_launch = time_launches(step, steps, warmup)
    pairs = bsa_admitted_pairs(case)
    tf = 4.0 * D * pairs / (ms_step * 1e-3) / 1e12
    return {"workload": "tiny block-sparse B=2 Sq=64 Hq=4 Hkv=1 D=128 causal (latency-bound)",
            "metric": "block-sparse paged attn TFLOP/s (admitted pairs)", "value": round(tf, 4),
            "unit": "TFLOP/s", "ms_per_step": round(ms_step, 4), "admitted_pairs": pairs,
            "us_per_launch": round(ms_launch * 1e3, 2)}


def sage_admitted_pairs(case):
    """(query, key) pairs over selected blocks' valid tokens, summed over heads."""
    B, H, Sq, _ = case.q_int8.shape
    nqb = -(-Sq // 64)
    idx = case.q2k_block_index
    nums = case.q2k_block_nums
    total = 0
    for b in range(B):
        for h in range(H):
            for r in range(nqb):
                n = int(nums[b, h, r]) if (nums is not None and not case.uniform_block_count) \
                    else case.block_sparse_num
                rows = min(64, Sq - 64 * r)
                for beta in idx[b, h, r, :n]:
                    bs = 64
                    if case.block_sizes is not None:
                        bsz = case.block_sizes
                        bs = int(bsz[beta] if bsz.ndim == 1 else (bsz[b, beta] if bsz.ndim == 2
                                                                   else bsz[b, h, beta]))
                    total += rows * max(0, min(bs, case.Sk - 64 * int(beta)))
    return total


def bench_sage(steps, warmup, W, P):
    log("sage: generating inputs")
    case = W.sage_long()
    q, k, v = case.q_int8.cuda(), case.k_int8.cuda(), case.v_fp8.cuda()
    qs, ks, vs = case.q_scale.cuda(), case.k_scale.cuda(), case.v_scale.cuda()
    idx = dev_i32(case.q2k_block_index)
    bsz = dev_i32(case.block_sizes)
    nums = dev_i32(case.q2k_block_nums)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")

    def step():
        P.bsa_sage_run(q, k, v, qs, ks, vs, idx, case.block_sparse_num, bsz, nums, None, out=out)

    ms_step, ms_launch = time_launches(step, steps, warmup)
    pairs = sage_admitted_pairs(case)
    ops = 4.0 * 128 * pairs
    tops = ops / (ms_step * 1e-3) / 1e12
    ach = ops / (ms_launch * 1e-3) / 1e12
    return {"workload": "Sage block-sparse B=2 H=16 Sq=Sk=16384 D=128 int8 Q/K fp8 V, "
                        "64 of 256 blocks per query block, last block partial",
            "metric": "Sage block-sparse TOP/s (admitted pairs, int8 QK + fp8 PV)",
            "value": round(tops, 2), "unit": "TOP/s", "ms_per_step": round(ms_step, 4),
            "admitted_pairs": pairs,
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(ach / INT8_PEAK_TOPS, 4),
                         "frac_of_bf16_peak": round(ach / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(["sage_kernel"], "sage"), "kernel": "sage_kernel"}}


def bench_qsa(steps, warmup, W, P):
    log("qsa: generating inputs")
    case = W.qsa_long()
    T, Hq, D = case.q.shape
    Hkv = case.k.shape[1]
    q, k, v = case.q.cuda(), case.k.cuda(), case.v.cuda()
    sel = torch.from_numpy(case.sel_blocks).cuda()
    lo, hi, bb, tb = (dev_i32(x) for x in (case.lo, case.hi, case.blk_base, case.tok_base))
    P.qsa_validate(case.lo, case.hi, case.blk_base, case.tok_base, case.block_first,
                   case.block_last)
    out = torch.empty_like(q)
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(Hq, T, dtype=torch.float32, device="cuda")

    def step():
        P.qsa_run(q, k, v, sel, lo, hi, bb, tb, case.scale, out=out, out_fp32=out32, lse=lse)

    ms_step, ms_launch = time_launches(step, steps, warmup)
    # admitted (token, key) pairs: the selected blocks' tokens inside [lo, hi]
    bf, bl = case.block_first.astype(np.int64), case.block_last.astype(np.int64)
    pairs = 0
    for t in range(T):
        nb = np.nonzero(case.sel_blocks[t])[0]
        a = np.maximum(bf[nb], case.lo[t])
        b = np.minimum(bl[nb], case.hi[t])
        pairs += int(np.maximum(b - a + 1, 0).sum())
    flops = 4.0 * D * pairs * Hq
    gathered = pairs * Hkv * D * 2 * 2          # K + V rows read per (token, KV head)
    tf = flops / (ms_step * 1e-3) / 1e12
    ach = flops / (ms_launch * 1e-3) / 1e12
    return {"workload": f"packed token-granular sparse attention T={T} (4x4096 causal) Hq={Hq} "
                        f"Hkv={Hkv} D={D} 4-token blocks, <=64 selected blocks per token",
            "metric": "QSA TFLOP/s (admitted pairs)", "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms_step, 4), "admitted_pairs": pairs,
            "gathered_kv_GBps": round(gathered / (ms_launch * 1e-3) / 1e9, 1),
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(["qsa_kernel<256>"], "qsa"),
                         "kernel": "qsa_kernel<256>"}}


def bench_copy():
    """A plain 1 GiB device-to-device copy, three times: the calibration run
    for the FETCH_SIZE / WRITE_SIZE counters (what they read for known bytes)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"workload": "device copy", "bytes_per_copy": n, "copies": 3}


def cpu_baseline_decode(case, budget_s=15.0):
    """fp64 oracle on the first requests of the decode batch until ~budget_s."""
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    done, nbytes = [], 0
    Hkv, D = case.k.shape[1], case.k.shape[3]
    t0 = time.perf_counter()
    for b in range(len(case.seq_lens)):
        A.decode_reference(case.q, case.k, case.v, case.kv_indptr, case.kv_indices,
                           case.seq_lens, requests=[b])
        done.append(b)
        nbytes += int(case.seq_lens[b]) * Hkv * D * 2 * 2
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle over requests {done[0]}..{done[-1]} "
                      f"({len(done)} of 64, {nbytes} live K+V bytes) in {dt:.1f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps before each timed region (at least this many, and "
                         "on until 0.2 s of untimed work has run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=["decode", "decode_q", "bsa", "prefill", "prefill_w1024", "prefill256", "tiny",
                                       "sage", "qsa", "copy"], default=None,
                    help="run one workload only (for profiling; copy = counter calibration)")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU component "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    from gen import workloads as W
    import paged_kv_block_amd as P

    if a.only and a.only != "decode":
        fn = {"bsa": lambda: bench_bsa_long(a.steps, a.warmup, W, P),
              "prefill": lambda: bench_prefill(a.steps, a.warmup, W, P),
              "prefill_w1024": lambda: bench_prefill(a.steps, a.warmup, W, P, window_left=1024),
              "prefill256": lambda: bench_prefill(a.steps, a.warmup, W, P, D=256),
              "tiny": lambda: bench_bsa_tiny(a.steps, a.warmup, W, P),
              "sage": lambda: bench_sage(a.steps, a.warmup, W, P),
              "decode_q": lambda: bench_decode_q(a.steps, a.warmup, W, P),
              "qsa": lambda: bench_qsa(a.steps, a.warmup, W, P),
              "copy": bench_copy}[a.only]
        print(json.dumps(fn()), flush=True)
        return 0

    case, gbs, ms_step, cfg, roof = bench_decode(a.steps, a.warmup, W, P)
    log(f"decode: {gbs:.1f} GB/s, {ms_step * 1e3:.1f} us/step")
    secondary = []
    if not a.no_secondary and a.only is None:
        for fn in (lambda: bench_bsa_long(a.steps, a.warmup, W, P),
                   lambda: bench_prefill(a.steps, a.warmup, W, P),
                   lambda: bench_prefill(a.steps, a.warmup, W, P, window_left=1024),
                   lambda: bench_prefill(a.steps, a.warmup, W, P, D=256),
                   lambda: bench_sage(a.steps, a.warmup, W, P),
                   lambda: bench_decode_q(a.steps, a.warmup, W, P),
                   lambda: bench_qsa(a.steps, a.warmup, W, P),
                   lambda: bench_bsa_tiny(a.steps, a.warmup, W, P)):
            r = fn()
            log(f"{r['workload']}: {r['value']} {r['unit']}")
            secondary.append(r)
            torch.cuda.empty_cache()
    cpu = None
    if not a.no_cpu_baseline:
        log("cpu baseline: timing the oracle")
        cpu = cpu_baseline_decode(case)
    line = {"metric": "decode KV-read GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16)",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu, "secondary": secondary}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
