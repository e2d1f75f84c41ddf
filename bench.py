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
~ U{0..2048}; D=128, window 1024, D=256), the Sage-style int8/fp8 block-sparse
case (B=2, H=16, S=16384, 64 of 256 blocks per query block), multi-token
decode, packed-query token-granular sparse attention and the tiny block-sparse
case -- attention as TFLOP/s (TOP/s) over the admitted (query, key) pairs only
(4*D operations per pair and query head).

Timing: inputs are generated (seeded; their SHA-256 is reported), copied to
HBM and planned before the timed region; W warm-up launches (and on until
0.2 s of untimed work has run), then K launches between two HIP events (the
step time), then K launches each bracketed by its own events on the stream
they are enqueued on (the mean launch duration, ``roofline.achieved``).

Roofline denominators: MI355X's published peaks, and the ceilings measured on
the same device by libpkb_peaks.so (``peaks``; ``frac_measured``).
``cpu_baseline`` times the fp64 oracle on bounded samples of the decode and
long block-sparse workloads, in worker processes over every host core.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

# The CPU-baseline workers are spawned processes that re-import this file as
# "__mp_main__": they run NumPy only and never load torch (or its HIP runtime).
if __name__ != "__mp_main__":
    import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
INT8_PEAK_TOPS = 5000.0        # dense int8 / fp8 MFMA

PEAKS = {}                     # ceilings measured on this device (measure_peaks)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------- HBM traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def _sha256(paths):
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


def input_sha256(*xs):
    """SHA-256 over the bytes of the generated inputs (CPU tensors / arrays), in
    argument order: identifies the exact synthetic draw a figure was taken on."""
    h = hashlib.sha256()
    for x in xs:
        if x is None:
            continue
        if isinstance(x, torch.Tensor):
            x = x.detach().contiguous().view(torch.uint8).numpy()
        h.update(np.ascontiguousarray(x).view(np.uint8).data)
    return h.hexdigest()


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


def roofline(bound, achieved, unit, peak, measured_key, traffic, kernel, **extra):
    """Roofline entry: the published peak, and the ceiling measured on this
    device (``PEAKS[measured_key]``) when the peaks were taken."""
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4) if peak else None, "traffic": traffic}
    pm = PEAKS.get(measured_key) if measured_key else None
    if pm:
        r["peak_measured"] = round(pm, 1)
        r["frac_measured"] = round(achieved / pm, 4)
    r["kernel"] = kernel
    r.update(extra)
    return r


# ---------------------------------------------------------------------------- on-device peaks

def _peaks_lib():
    path = os.path.join(ROOT, "paged_kv_block_amd", "libpkb_peaks.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with paged_kv_block_amd/build.py")
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.pkb_peak_hbm_read.argtypes = [vp, i64, vp, i32, i32, vp]
    L.pkb_peak_hbm_gather.argtypes = [vp, i64, i64, vp, i32, i32, ctypes.POINTER(i64), vp]
    L.pkb_peak_l2_gather.argtypes = [vp, i64, i64, vp, i32, ctypes.POINTER(i64), vp]
    L.pkb_peak_mfma.argtypes = [i32, i32, vp, i32, vp]
    L.pkb_peak_issue.argtypes = [i32, i32, i32, vp, i32, vp]
    L.pkb_peak_coexec.argtypes = [i32, i32, i32, vp, i32, vp]
    for f in (L.pkb_peak_hbm_read, L.pkb_peak_hbm_gather, L.pkb_peak_l2_gather, L.pkb_peak_mfma,
              L.pkb_peak_issue, L.pkb_peak_coexec):
        f.restype = ctypes.c_int
    return L


def _best_ms(fn, n=10):
    """Shortest of n launches, each between its own events, after >= 0.2 s of
    untimed launches (clock ramp)."""
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < WARMUP_MIN_S:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return min(a.elapsed_time(b) for a, b in evs)


def measure_peaks(P):
    """Ceilings of this device from hand-written probe kernels: an HBM streaming
    read of 4 GiB and a gather of random 4 KiB slabs (decode's access shape),
    each with plain and with non-temporal loads, a
    gather of random 512-byte rows from a 2 MiB L2-resident buffer (the
    packed-query kernel's), dense MFMA loops at two waves per SIMD, and the
    instruction-issue and MFMA / VALU co-execution probes."""
    L = _peaks_lib()
    st = torch.cuda.current_stream().cuda_stream
    ncu = P.num_cus()
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    nbytes = 4 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = {}

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed (HIP error {-rc})")

    # each ceiling is the best over 4, 8, 16 and 32 waves per CU; the HBM ones
    # also over plain and non-temporal loads (both are reported)
    got = ctypes.c_int64(0)
    for nt, tag in ((0, "plain"), (1, "nt")):
        best = 0.0
        for mult in (1, 2, 4, 8):
            ms = _best_ms(lambda: ok(L.pkb_peak_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(),
                                                         ncu * mult, nt, st), "hbm read"))
            best = max(best, nbytes / (ms * 1e-3) / 1e9)
        out[f"hbm_read_{tag}_GBps"] = best
        best = 0.0
        for mult in (1, 2, 4, 8):
            ms = _best_ms(lambda: ok(L.pkb_peak_hbm_gather(buf.data_ptr(), nbytes, 1 << 20, sink.data_ptr(),
                                                           ncu * mult, nt, ctypes.byref(got), st),
                                     "hbm gather"))
            best = max(best, got.value / (ms * 1e-3) / 1e9)
        out[f"hbm_gather_4k_{tag}_GBps"] = best
    out["hbm_read_GBps"] = max(out["hbm_read_plain_GBps"], out["hbm_read_nt_GBps"])
    out["hbm_gather_4k_GBps"] = max(out["hbm_gather_4k_plain_GBps"], out["hbm_gather_4k_nt_GBps"])
    small = 2 << 20
    best = 0.0
    for mult in (1, 2, 4, 8):
        ms = _best_ms(lambda: ok(L.pkb_peak_l2_gather(buf.data_ptr(), small, 1 << 24, sink.data_ptr(),
                                                      ncu * mult, ctypes.byref(got), st), "l2 gather"))
        best = max(best, got.value / (ms * 1e-3) / 1e9)
    out["l2_gather_512_GBps"] = best
    del buf
    torch.cuda.empty_cache()
    grid, iters = ncu * 2, 4096
    for kind, key, per in ((0, "mfma_bf16_TFLOPs", 32768), (1, "mfma_i8_TOPs", 65536),
                           (2, "mfma_f8_TOPs", 131072)):
        ms = _best_ms(lambda: ok(L.pkb_peak_mfma(kind, iters, sink.data_ptr(), grid, st), "mfma"))
        out[key] = grid * 4 * iters * 8 * per / (ms * 1e-3) / 1e12
    # Sage runs equal int8 (QK^T) and fp8 (PV) operation counts: its ceiling is
    # the harmonic mean of the two.
    out["mfma_i8_f8_half_TOPs"] = 2.0 / (1.0 / out["mfma_i8_TOPs"] + 1.0 / out["mfma_f8_TOPs"])
    res = {k: round(v, 1) for k, v in out.items()}
    # Issue rates (SIMD cycles per wave instruction at the 2.4 GHz the MFMA loop
    # runs at) with one and two waves per SIMD, and MFMA / VALU co-execution.
    clk = 2.4e9
    iters = 20000
    for kind, key in ((0, "fma"), (1, "exp"), (2, "add_and_salu")):
        for waves in (4, 8):
            ms = _best_ms(lambda: ok(L.pkb_peak_issue(kind, iters, waves, sink.data_ptr(), ncu, st),
                                     "issue"))
            res[f"issue_{key}_cycles_{waves // 4}wave"] = round(
                ms * 1e-3 * clk / (iters * 8 * (waves // 4)), 2)
    t = {}
    for mode in (0, 1, 2):
        t[mode] = _best_ms(lambda: ok(L.pkb_peak_coexec(mode, 10000, 40000, sink.data_ptr(), ncu, st),
                                      "coexec"))
    res["coexec_mfma_ms"], res["coexec_valu_ms"], res["coexec_both_ms"] = (
        round(t[0], 4), round(t[1], 4), round(t[2], 4))
    return res


# ---------------------------------------------------------------------------- work counts

def bsa_admitted_pairs(case, use_bits=True):
    """Admitted (query token, key) pairs summed over query heads.  use_bits=False
    leaves validity-bit zeros in (the selected-and-causal count)."""
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


def bsa_block_area_pairs(case):
    """Selected blocks x query tokens of the row x keys of the block (no mask):
    the work a dense-per-block kernel would do."""
    B, Sq, Hq, Hkv, D, P, ps = case.dims
    G = Hq // Hkv
    qbs, kvbs = case.q_block_size, case.kv_block_size
    total = 0
    for b in range(B):
        L = int(case.seq_lens[b])
        for g in range(Hkv):
            for r in range(case.block_indptr.shape[2] - 1):
                blk = np.unique(case.block_indices[case.block_indptr[b, g, r]:case.block_indptr[b, g, r + 1]])
                rows = min((r + 1) * qbs, Sq) - r * qbs
                keys = np.clip(blk.astype(np.int64) * kvbs + kvbs, 0, L) - np.clip(blk.astype(np.int64) * kvbs, 0, L)
                total += rows * int(keys.sum())
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

def bench_decode(steps, warmup, W, P, page_size=16):
    log("decode: generating inputs")
    case = W.batch_decode(page_size=page_size)
    sha = input_sha256(case.q, case.k, case.v, case.kv_indptr, case.kv_indices, case.seq_lens)
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
                       f"page_size={ps} bf16 (seed 2)",
           "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "page_size": ps,
           "sum_seq_len": int(case.seq_lens.sum()), "num_splits": S, "split_len": split_len,
           "kv_bytes_per_step": kv_bytes, "input_sha256": sha}
    kern = ["decode_coop_kernel<128>"] if S == 1 else ["decode_kernel<128>", "decode_merge_kernel<128>"]
    gather = PEAKS.get("hbm_gather_4k_GBps")
    roof = roofline("hbm", ach, "GB/s", HBM_PEAK_GBS, "hbm_read_GBps",
                    measured_traffic(kern, "decode" if ps == 16 else f"decode_ps{ps}"),
                    " + ".join(kern) + " (one step)",
                    per_unit="4096 B of K+V per live token (Hkv=8, D=128, bf16)")
    if gather:
        roof["frac_of_measured_4k_gather"] = round(ach / gather, 4)
    del q, k, v, ws
    torch.cuda.empty_cache()
    return case, gbs, ms_step, cfg, roof


def bench_decode_q(steps, warmup, W, P, SQ=4):
    log(f"decode_q: generating inputs (SQ={SQ})")
    case = W.batch_decode_q(SQ=SQ)
    sha = input_sha256(case.q, case.k, case.v, case.kv_indptr, case.kv_indices, case.seq_lens)
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
            "input_sha256": sha,
            "roofline": roofline("hbm", kv_bytes / (ms_launch * 1e-3) / 1e9, "GB/s", HBM_PEAK_GBS,
                                 "hbm_read_GBps", measured_traffic(kern, "decode_q"),
                                 " + ".join(kern) + " (16 query rows per KV head: 4 tokens x "
                                 "4 heads)")}


def bench_bsa_long(steps, warmup, W, P, cpu=False):
    log("long block-sparse: generating inputs")
    case = W.long_bsa()
    sha = input_sha256(case.q, case.k, case.v, case.kv_indptr, case.kv_indices, case.block_indptr,
                       case.block_indices, case.seq_lens, case.valid_bits)
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
    del q, k, v, out, lse
    torch.cuda.empty_cache()
    pairs = bsa_admitted_pairs(case, use_bits=False)       # selected blocks, causal, < L
    pairs_bits = bsa_admitted_pairs(case, use_bits=True)   # ... and validity bit set
    area = bsa_block_area_pairs(case)
    flops = 4.0 * D * pairs
    tf = flops / (ms_step * 1e-3) / 1e12
    ach = flops / (ms_launch * 1e-3) / 1e12
    kname = "attn_fwd_kernel<128,%d,bsa>" % wr.plan.waves
    r = {"workload": "long block-sparse paged attention B=4 S=8192 Hq=32 Hkv=8 D=128 "
                     "page=64 q/kv block 64, 16 blocks/row, causal, 1% invalid bits (seed 4)",
         "metric": "block-sparse paged attn TFLOP/s (selected blocks)", "value": round(tf, 2),
         "unit": "TFLOP/s", "ms_per_step": round(ms_step, 4),
         "work": {"admitted_pairs": pairs, "admitted_pairs_valid_bits": pairs_bits,
                  "block_area_pairs": area,
                  "counted": "4*D flops per pair of a selected block that passes causal and j < L "
                             "(validity-bit zeros not subtracted)"},
         "input_sha256": sha,
         "roofline": roofline("mfma", ach, "TFLOP/s", BF16_PEAK_TFLOPS, "mfma_bf16_TFLOPs",
                              measured_traffic([kname], "bsa"), kname)}
    if cpu:
        r["cpu_baseline"] = cpu_baseline_bsa(case)
    return r


def bench_prefill(steps, warmup, W, P, D=128, window_left=-1):
    log(f"prefill D={D} w={window_left}: generating inputs")
    case = W.batch_prefill(3, D=D, window_left=window_left)
    sha = input_sha256(case.q, case.k, case.v, case.qo_indptr, case.block_tables, case.seq_lens)
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
    kname = "attn_fwd_kernel<%d,%d,prefill>" % (D, wr.plan.waves)
    return {"workload": f"batch paged prefill B=8 causal window_left={window_left} Hq=32 "
                        f"Hkv=8 D={D} page=32 total_q={int(case.qo_indptr[-1])} (seed 3)",
            "metric": "paged prefill TFLOP/s (admitted pairs)", "value": round(tf, 2),
            "unit": "TFLOP/s", "ms_per_step": round(ms_step, 4), "admitted_pairs": pairs,
            "input_sha256": sha,
            "roofline": roofline("mfma", ach, "TFLOP/s", BF16_PEAK_TFLOPS, "mfma_bf16_TFLOPs",
                                 measured_traffic([kname], "prefill_d%d_w%d" % (D, window_left)),
                                 kname)}


def bench_bsa_tiny(steps, warmup, W, P):
    case = W.tiny_bsa("causal")
    sha = input_sha256(case.q, case.k, case.v, case.kv_indptr, case.kv_indices, case.block_indptr,
                       case.block_indices, case.seq_lens, case.valid_bits)
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
    return {"workload": "tiny block-sparse B=2 Sq=64 Hq=4 Hkv=1 D=128 causal (latency-bound, seed 1)",
            "metric": "block-sparse paged attn TFLOP/s (admitted pairs)", "value": round(tf, 4),
            "unit": "TFLOP/s", "ms_per_step": round(ms_step, 4), "admitted_pairs": pairs,
            "us_per_launch": round(ms_launch * 1e3, 2), "input_sha256": sha}


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
    sha = input_sha256(case.q_int8, case.k_int8, case.v_fp8, case.q_scale, case.k_scale,
                       case.v_scale, case.q2k_block_index, case.q2k_block_nums, case.block_sizes)
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
    roof = roofline("mfma", ach, "TOP/s", INT8_PEAK_TOPS, "mfma_i8_f8_half_TOPs",
                    measured_traffic(["sage_kernel"], "sage"), "sage_kernel",
                    frac_of_bf16_peak=round(ach / BF16_PEAK_TFLOPS, 4))
    if PEAKS.get("mfma_bf16_TFLOPs"):
        roof["frac_of_measured_bf16_peak"] = round(ach / PEAKS["mfma_bf16_TFLOPs"], 4)
    return {"workload": "Sage block-sparse B=2 H=16 Sq=Sk=16384 D=128 int8 Q/K fp8 V, "
                        "64 of 256 blocks per query block, last block partial (seed 5)",
            "metric": "Sage block-sparse TOP/s (admitted pairs, int8 QK + fp8 PV)",
            "value": round(tops, 2), "unit": "TOP/s", "ms_per_step": round(ms_step, 4),
            "admitted_pairs": pairs, "input_sha256": sha, "roofline": roof}


def bench_qsa(steps, warmup, W, P):
    log("qsa: generating inputs")
    case = W.qsa_long()
    sha = input_sha256(case.q, case.k, case.v, case.sel_blocks, case.lo, case.hi, case.blk_base,
                       case.tok_base)
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
    ach_tf = flops / (ms_launch * 1e-3) / 1e12
    ach_gb = gathered / (ms_launch * 1e-3) / 1e9
    l2 = PEAKS.get("l2_gather_512_GBps")
    # Bound: gathering one K and one V row of D bf16 per admitted key from L2;
    # no published figure exists for that rate, so the measured ceiling is the peak.
    roof = roofline("l2_gather", ach_gb, "GB/s", l2, "l2_gather_512_GBps",
                    measured_traffic(["qsa_kernel<256>"], "qsa"), "qsa_kernel<256>",
                    per_unit=f"{Hkv * D * 2 * 2} B of K+V rows gathered per admitted key",
                    mfma_achieved_TFLOPs=round(ach_tf, 2),
                    mfma_frac=round(ach_tf / BF16_PEAK_TFLOPS, 4))
    return {"workload": f"packed token-granular sparse attention T={T} (4x4096 causal) Hq={Hq} "
                        f"Hkv={Hkv} D={D} 4-token blocks, <=64 selected blocks per token (seed 7)",
            "metric": "QSA TFLOP/s (admitted pairs)", "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms_step, 4), "admitted_pairs": pairs,
            "gathered_kv_GBps": round(gathered / (ms_step * 1e-3) / 1e9, 1),
            "input_sha256": sha, "roofline": roof}


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


# ---------------------------------------------------------------------------- CPU oracle baseline
#
# The fp64 oracle runs in worker processes, one per host core (one BLAS thread
# each).  The inputs sit in shared memory; each task takes one request's pages
# (decode) or one BSR row's query tokens and its request's pages for one KV
# head (block-sparse), and runs the oracle on exactly that data.

_SHM = {}


def _shm_put(name, arr):
    from multiprocessing import shared_memory
    arr = np.ascontiguousarray(arr)
    shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
    np.ndarray(arr.shape, arr.dtype, buffer=shm.buf)[...] = arr
    _SHM[name] = shm
    return (shm.name, arr.shape, arr.dtype.str)


def _shm_view(desc):
    from multiprocessing import shared_memory
    name, shape, dt = desc
    shm = shared_memory.SharedMemory(name=name)
    _SHM[name] = shm                       # keep the mapping alive in the worker
    return np.ndarray(shape, np.dtype(dt), buffer=shm.buf)


_W = {}


def _worker_init(descs):
    for k, d in descs.items():
        _W[k] = _shm_view(d)


def _worker_ready(_):
    from oracle import attention  # noqa: F401  (import before the timed region)
    return os.getpid()


def _bf16_bits_to_f32(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32)


def _decode_task(b):
    from oracle import attention as A
    ip, ix, sl = _W["indptr"], _W["indices"], _W["seq_lens"]
    pages = ix[ip[b]:ip[b + 1]]
    n = len(pages)
    kb = _bf16_bits_to_f32(_W["k"][pages])
    vb = _bf16_bits_to_f32(_W["v"][pages])
    qb = _bf16_bits_to_f32(_W["q"][b:b + 1])
    A.decode_reference(qb, kb, vb, np.array([0, n]), np.arange(n), sl[b:b + 1])
    return b


def _bsa_task(t):
    from oracle import attention as A
    b, g, r = t
    ip, ix = _W["indptr"], _W["indices"]
    bip, bix, sl, bits = _W["block_indptr"], _W["block_indices"], _W["seq_lens"], _W["bits"]
    q = _W["q"]
    Sq, G, qbs = q.shape[1], q.shape[2] // _W["k"].shape[1], 64
    pages = ix[ip[b]:ip[b + 1]]
    n = len(pages)
    kb = _bf16_bits_to_f32(_W["k"][pages, g:g + 1])
    vb = _bf16_bits_to_f32(_W["v"][pages, g:g + 1])
    rows = np.arange(r * qbs, min((r + 1) * qbs, Sq))
    qm = np.zeros((1, Sq, G, q.shape[3]), np.float32)
    qm[0, rows] = _bf16_bits_to_f32(q[b, rows, g * G:(g + 1) * G])
    sel = bix[bip[b, g, r]:bip[b, g, r + 1]]
    nqb = bip.shape[2] - 1
    bipm = np.where(np.arange(nqb + 1) <= r, 0, len(sel)).astype(np.int64).reshape(1, 1, nqb + 1)
    A.bsa_reference(qm, kb, vb, np.array([0, n]), np.arange(n), bipm, sel, qbs, 64,
                    sl[b:b + 1], valid_bits=bits[b:b + 1], mask="causal",
                    tokens=[(0, int(i)) for i in rows])
    return t


def _cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{cfg.get('name')} {cfg.get('version')}"
    except Exception:  # pragma: no cover
        pass
    return model, blas


def _run_pool(descs, fn, tasks):
    """Wall time of fn over tasks in worker processes (one per host core, one
    BLAS thread each), started and warmed before the clock starts."""
    import multiprocessing as mp
    if any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ):
        # Worker processes would inherit the profiler's preloaded tool, which
        # attaches to the GPU in every child: never run the pool under it.
        raise RuntimeError("the CPU baseline does not run under a profiler "
                           "(pass --no-cpu-baseline)")
    cores = len(os.sched_getaffinity(0))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS", "HIP_VISIBLE_DEVICES",
                                            "ROCR_VISIBLE_DEVICES", "CUDA_VISIBLE_DEVICES")}
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    for k in ("HIP_VISIBLE_DEVICES", "ROCR_VISIBLE_DEVICES", "CUDA_VISIBLE_DEVICES"):
        os.environ[k] = ""          # the workers never touch a GPU
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(cores, initializer=_worker_init, initargs=(descs,)) as pool:
            pool.map(_worker_ready, range(cores), chunksize=1)
            t0 = time.perf_counter()
            pool.map(fn, tasks, chunksize=1)
            dt = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return dt, cores


def _shm_release():
    for shm in _SHM.values():
        try:
            shm.close()
            shm.unlink()
        except FileNotFoundError:
            pass
    _SHM.clear()


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def cpu_baseline_decode(case, passes=4):
    """The fp64 oracle over the whole decode batch (64 requests), `passes`
    times (one pass is only a few core-seconds)."""
    try:
        descs = {"q": _shm_put("q", _u16(case.q)), "k": _shm_put("k", _u16(case.k)),
                 "v": _shm_put("v", _u16(case.v)), "indptr": _shm_put("ip", case.kv_indptr),
                 "indices": _shm_put("ix", case.kv_indices),
                 "seq_lens": _shm_put("sl", case.seq_lens)}
        B = len(case.seq_lens)
        order = sorted(range(B), key=lambda b: -int(case.seq_lens[b]))   # longest first
        dt, cores = _run_pool(descs, _decode_task, [b for b in order for _ in range(passes)])
    finally:
        _shm_release()
    Hkv, D = case.k.shape[1], case.k.shape[3]
    nbytes = int(case.seq_lens.astype(np.int64).sum()) * Hkv * D * 2 * 2
    model, blas = _cpu_info()
    return {"value": round(passes * nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle, {passes} passes over all {B} requests of the decode "
                      f"batch ({nbytes} live K+V bytes per pass) in {dt:.2f} s wall, {cores} "
                      "worker processes with one BLAS thread each",
            "cpu_model": model, "blas": blas}


def cpu_baseline_bsa(case, heads_per_row=2):
    """The fp64 oracle over a sample of the long block-sparse work: every BSR
    row of every request, `heads_per_row` of its KV heads (rotating)."""
    B, Sq, Hq, Hkv, D, Pn, ps = case.dims
    nqb = case.block_indptr.shape[2] - 1
    tasks = [(b, (b * 3 + r + k * Hkv // heads_per_row) % Hkv, r) for b in range(B)
             for r in range(nqb) for k in range(heads_per_row)]
    G = Hq // Hkv
    pairs = 0
    for b, g, r in tasks:     # selected-and-causal pairs of the row (the GPU headline's count)
        L = int(case.seq_lens[b])
        blk = np.unique(case.block_indices[case.block_indptr[b, g, r]:case.block_indptr[b, g, r + 1]])
        p = L - Sq + np.arange(r * 64, min(r * 64 + 64, Sq))
        a0 = np.clip(blk.astype(np.int64) * 64, 0, L)[None, :]
        a1 = np.clip(blk.astype(np.int64) * 64 + 64, 0, L)[None, :]
        hi = np.minimum(a1, (p + 1)[:, None])
        pairs += int(np.maximum(hi - a0, 0).sum()) * G
    try:
        descs = {"q": _shm_put("q", _u16(case.q)), "k": _shm_put("k", _u16(case.k)),
                 "v": _shm_put("v", _u16(case.v)), "indptr": _shm_put("ip", case.kv_indptr),
                 "indices": _shm_put("ix", case.kv_indices),
                 "block_indptr": _shm_put("bip", case.block_indptr),
                 "block_indices": _shm_put("bix", case.block_indices),
                 "seq_lens": _shm_put("sl", case.seq_lens), "bits": _shm_put("bits", case.valid_bits)}
        dt, cores = _run_pool(descs, _bsa_task, tasks)
    finally:
        _shm_release()
    model, blas = _cpu_info()
    flops = 4.0 * D * pairs
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle over {len(tasks)} of {B * Hkv * nqb} (request, KV head, "
                      f"BSR row) units (every row, {heads_per_row} of {Hkv} KV heads each; {pairs} "
                      f"admitted pairs) in {dt:.2f} s wall, {cores} worker processes with one BLAS "
                      "thread each",
            "cpu_model": model, "blas": blas}


# ---------------------------------------------------------------------------- trace summaries

def trace_summary(path, last):
    """Markdown table of a rocprofv3 kernel trace (kernel_trace.csv): per
    kernel, the dispatch count and mean duration over all dispatches and over
    the last `last` dispatches (bench's timed launches, after its warmup)."""
    import csv
    durs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            durs.setdefault(row["Kernel_Name"], []).append((int(row["Start_Timestamp"]), d))
    lines = ["| kernel | dispatches | mean, all (us) | timed dispatches | mean, timed (us) | min (us) |",
             "|---|---|---|---|---|---|"]
    for name, xs in sorted(durs.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        xs.sort()
        ds = [d for _, d in xs]
        tail = ds[-last:] if len(ds) > last else ds
        lines.append(f"| `{name}` | {len(ds)} | {np.mean(ds):.2f} | {len(tail)} | "
                     f"{np.mean(tail):.2f} | {min(tail):.2f} |")
    return "\n".join(lines)


def pmc_summary(path, last, num_cus=256, xcds=8):
    """Markdown table of a rocprofv3 counter collection (counter_collection.csv):
    per kernel, each counter's mean over its last `last` dispatches, and the
    derived figures.  GRBM_GUI_ACTIVE counts every XCD's cycles (their sum), so
    the kernel's clock is GRBM_GUI_ACTIVE / xcds / duration, and the share of
    SIMD cycles the matrix pipe is busy is
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / xcds * num_cus * 4)."""
    import csv
    vals, durs = {}, {}
    with open(path) as f:
        for row in csv.DictReader(f):
            k, did = row["Kernel_Name"], int(row["Dispatch_Id"])
            vals.setdefault(k, {}).setdefault(row["Counter_Name"], {})[did] = float(row["Counter_Value"])
            durs.setdefault(k, {})[did] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
    out = []
    for k, cs in vals.items():
        if k.startswith("__amd_rocclr") or "at::native" in k:
            continue
        ids = sorted(durs[k])[-last:]
        mean = {c: float(np.mean([v[i] for i in ids if i in v])) for c, v in cs.items()}
        dur = float(np.mean([durs[k][i] for i in ids]))
        out.append(f"**`{k}`** -- {len(ids)} dispatches, mean duration {dur:.2f} us")
        out.append("")
        out.append("| counter | mean per dispatch |")
        out.append("|---|---|")
        for c in sorted(mean):
            out.append(f"| {c} | {mean[c]:,.0f} |")
        gui = mean.get("GRBM_GUI_ACTIVE")
        derived = []
        if gui:
            cyc = gui / xcds
            derived.append(("clock (GHz)", f"{cyc / (dur * 1e3):.3f}"))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                derived.append(("matrix pipe busy (share of SIMD cycles)",
                                f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * num_cus * 4):.4f}"))
            for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS",
                      "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                      "SQ_WAVE_CYCLES", "SQ_LDS_IDX_ACTIVE"):
                if c in mean:
                    derived.append((f"{c} / (SIMD cycles)", f"{mean[c] / (cyc * num_cus * 4):.4f}"))
        mf = mean.get("SQ_INSTS_MFMA")
        if mf:
            if "SQ_INSTS_VALU" in mean:
                derived.append(("non-MFMA VALU instructions per MFMA",
                                f"{(mean['SQ_INSTS_VALU'] - mf) / mf:.2f}"))
            for c in ("SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_SMEM"):
                if c in mean:
                    derived.append((f"{c} per MFMA", f"{mean[c] / mf:.2f}"))
        for c, per in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 512), ("SQ_INSTS_VALU_MFMA_MOPS_I8", 512),
                       ("SQ_INSTS_VALU_MFMA_MOPS_F8", 512)):
            if mean.get(c):
                derived.append((f"{c} x {per} (matrix ops executed)", f"{mean[c] * per:.4e}"))
        if derived:
            out.append("")
            out.append("| derived | value |")
            out.append("|---|---|")
            out += [f"| {a} | {b} |" for a, b in derived]
        out.append("")
    return "\n".join(out)


# Kernel short names and the sources each one is built from (a traffic record
# is valid only while these files are unchanged).
_KERNEL_SOURCES = {
    "attn_fwd_kernel": "paged_kv_block_amd/csrc/attn_fwd_kernel.h",
    "decode_coop_kernel": "paged_kv_block_amd/csrc/decode_fwd.hip",
    "decode_kernel": "paged_kv_block_amd/csrc/decode_fwd.hip",
    "decode_merge_kernel": "paged_kv_block_amd/csrc/decode_fwd.hip",
    "sage_kernel": "paged_kv_block_amd/csrc/sage_fwd.hip",
    "qsa_kernel": "paged_kv_block_amd/csrc/qsa_fwd.hip",
}
_COMMON_SOURCES = ["paged_kv_block_amd/csrc/device_common.h",
                   "paged_kv_block_amd/csrc/pkb_internal.h", "paged_kv_block_amd/csrc/policy.h"]
_TRAFFIC_WORKLOADS = {"decode": "decode", "decode_q": "decode_q", "bsa": "bsa",
                      "prefill": "prefill_d128_w-1", "prefill_w1024": "prefill_d128_w1024",
                      "prefill256": "prefill_d256_w-1", "sage": "sage", "qsa": "qsa"}


def _short_kernel(name):
    """'void pkb::attn_fwd_kernel<128, 4, 0, false, true>(...)' -> 'attn_fwd_kernel<128,4,bsa>'."""
    import re
    m = re.search(r"pkb::(\w+)(?:<([^>]*)>)?\(", name)
    if not m:
        return None
    base, targs = m.group(1), [t.strip() for t in (m.group(2) or "").split(",") if t.strip()]
    if base == "attn_fwd_kernel":
        return f"attn_fwd_kernel<{targs[0]},{targs[1]},{['bsa', 'prefill', 'decode'][int(targs[2])]}>"
    if base in ("decode_coop_kernel", "decode_kernel", "decode_merge_kernel", "qsa_kernel"):
        return f"{base}<{targs[0]}>"
    return base


def _counter_means(path, last):
    import csv
    vals, durs = {}, {}
    with open(path) as f:
        for row in csv.DictReader(f):
            k = row["Kernel_Name"]
            vals.setdefault(k, {}).setdefault(row["Counter_Name"], {})[int(row["Dispatch_Id"])] = \
                float(row["Counter_Value"])
    out = {}
    for k, cs in vals.items():
        for c, v in cs.items():
            ids = sorted(v)[-last:]
            out.setdefault(k, {})[c] = float(np.mean([v[i] for i in ids]))
    return out


def traffic_summary(directory, last=4):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs, one counter per run, in
    <directory>/tf_<workload>_<COUNTER>/p_counter_collection.csv.  Each counter (KiB per
    dispatch) is scaled by what it reads for the plain 1 GiB device copy (tf_copy_*: three
    __amd_rocclr_copyBuffer launches of 1,048,576 KiB).  Prints the table rows and the
    machine-readable records that measured_traffic() reads."""
    def load(w, c):
        return _counter_means(os.path.join(directory, f"tf_{w}_{c}", "p_counter_collection.csv"), last)
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = [v[c] for k, v in load("copy", c).items() if k.startswith("__amd_rocclr_copyBuffer")]
        cal[c] = (1 << 20) / copy[0]
    rows = ["| calibration (1 GiB = 1,048,576 KiB copied) | counter reads (KiB) | scale factor |",
            "|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        rows.append(f"| {c} | {(1 << 20) / cal[c]:,.1f} | {cal[c]:.4f} |")
    rows += ["", "| workload | kernel | FETCH_SIZE KiB / dispatch | WRITE_SIZE KiB / dispatch | "
                 "bytes per launch |", "|---|---|---|---|---|"]
    recs = []
    for w, wname in _TRAFFIC_WORKLOADS.items():
        fe, wr = load(w, "FETCH_SIZE"), load(w, "WRITE_SIZE")
        for k in fe:
            short = _short_kernel(k)
            if short is None or k not in wr:
                continue
            f_kib, w_kib = fe[k]["FETCH_SIZE"], wr[k]["WRITE_SIZE"]
            nbytes = int(round((f_kib * cal["FETCH_SIZE"] + w_kib * cal["WRITE_SIZE"]) * 1024))
            src = [_KERNEL_SOURCES[short.split("<")[0]]] + _COMMON_SOURCES
            rows.append(f"| {wname} | `{short}` | {f_kib:,.0f} | {w_kib:,.0f} | {nbytes:,} |")
            recs.append(f"traffic-record: kernel={short} workload={wname} source={','.join(src)} "
                        f"sha256={_sha256([os.path.join(ROOT, x) for x in src])} "
                        f"fetch_kib={f_kib:.1f} write_kib={w_kib:.1f} "
                        f"fetch_scale={cal['FETCH_SIZE']:.4f} write_scale={cal['WRITE_SIZE']:.4f} "
                        f"bytes_per_launch={nbytes}")
    return "\n".join(rows + [""] + recs)


# ---------------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps before each timed region (at least this many, and "
                         "on until 0.2 s of untimed work has run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--only", choices=["decode", "decode_q", "bsa", "prefill", "prefill_w1024",
                                       "prefill256", "tiny", "sage", "qsa", "copy", "peaks"],
                    default=None,
                    help="run one workload only (for profiling; copy = counter calibration, "
                         "peaks = the on-device ceilings)")
    ap.add_argument("--decode-page-size", type=int, default=16,
                    help="page size of the decode batch (with --only decode; the headline "
                         "uses 16)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV", default=None,
                    help="print a markdown summary of a rocprofv3 kernel trace and exit (mean "
                         "over the last 2*steps dispatches of each kernel: the timed ones)")
    ap.add_argument("--pmc-summary", metavar="COUNTER_COLLECTION_CSV", default=None,
                    help="print a markdown summary of a rocprofv3 counter collection and exit "
                         "(means over the last 2*steps dispatches of each kernel)")
    ap.add_argument("--traffic-summary", metavar="DIR", default=None,
                    help="print HBM traffic rows and records from FETCH_SIZE / WRITE_SIZE "
                         "runs under DIR (tf_<workload>_<counter>/) and exit")
    a = ap.parse_args(argv)
    if a.traffic_summary:
        print(traffic_summary(a.traffic_summary))
        return 0
    if a.trace_summary:
        print(trace_summary(a.trace_summary, 2 * a.steps))
        return 0
    if a.pmc_summary:
        print(pmc_summary(a.pmc_summary, 2 * a.steps))
        return 0
    if a.decode_page_size != 16 and a.only != "decode":
        print("--decode-page-size applies to --only decode", file=sys.stderr)
        return 2
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

    if a.only == "peaks" or (a.only is None and not a.no_peaks):
        log("peaks: measuring on-device ceilings")
        PEAKS.update(measure_peaks(P))
        log(f"peaks: {PEAKS}")
        if a.only == "peaks":
            print(json.dumps({"peaks": PEAKS}), flush=True)
            return 0

    if a.only:
        if a.only == "decode":
            case, gbs, ms_step, cfg, roof = bench_decode(a.steps, a.warmup, W, P,
                                                         a.decode_page_size)
            print(json.dumps({"metric": "decode KV-read GB/s", "value": round(gbs, 1),
                              "unit": "GB/s", "ms_per_step": round(ms_step, 4), "config": cfg,
                              "roofline": roof}), flush=True)
            return 0
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
        for fn in (lambda: bench_bsa_long(a.steps, a.warmup, W, P, cpu=not a.no_cpu_baseline),
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
        log("cpu baseline: timing the oracle on the decode batch")
        cpu = cpu_baseline_decode(case)
    line = {"metric": "decode KV-read GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16)",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu,
            "peaks": PEAKS or None, "secondary": secondary}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
