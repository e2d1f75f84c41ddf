"""Host metadata rules and launch policies, restated in Python -- TEST INFRASTRUCTURE.

The C library (``libpkb.so``) implements the same rules in C++; the two share no
code.  Tests compare them bit for bit (status, failing field and index, plan
fields, prefill work list, decode split policy).

Metadata contracts come from the FlashInfer pages:
  * "prims_ts_batch_decode_with_kv_cache" (description): CSR page IDs -- indptr
    starts at 0, increases strictly, ends at numel; each request owns
    ceil(seq_len/page_size) entries; every live page ID indexes the cache;
    sequence lengths positive and <= max_seq_len <= 2,147,483,520.
  * "block_sparse_attention_with_paged_kv_cache" (Parameters): BSR row offsets
    [B, Hkv, ceil(Sq/q_block_size)+1]; kv_block_size in {8, 16, 32} or a
    multiple of 64; (q_block_size * Hq/Hkv) % 8 == 0; the convenience path
    validates live page and sparse metadata before the trusted run.
  * "batch_prefill_with_paged_kv_cache": page_size in {16, 32, 64, 128}, D in
    {128, 256}, packed qo_indptr, row-strided block tables.
  * "bsa_attn_sm120_blk64_sage_fwd": block_sparse_num in [0, capacity],
    per-row counts, block_sizes of rank 1-3.

Readings where the pages are silent (offsets are absolute into the flat index
array; duplicate block IDs in a row are rejected; kv_indptr increases strictly
as on the decode page) are the ones the library documents in its header.  The
block-sparse and decode pages constrain only block sizes, so any page size of
at least 1 is accepted there; the prefill page lists its four.
"""
from __future__ import annotations

import numpy as np

PKB_OK = 0
PKB_ERR_ARG = -1
PKB_ERR_SHAPE = -2
PKB_ERR_DTYPE = -3
PKB_ERR_UNSUPPORTED = -4
PKB_ERR_METADATA = -5
PKB_ERR_WORKSPACE = -6

F_NONE, F_KV_INDPTR, F_KV_INDICES, F_SEQ_LENS = 0, 1, 2, 3
F_BLOCK_INDPTR, F_BLOCK_INDICES, F_QO_INDPTR, F_BLOCK_TABLES = 4, 5, 6, 7
F_Q2K_INDEX, F_Q2K_NUMS, F_BLOCK_SIZES = 8, 9, 10
F_LO, F_HI, F_BLK_BASE, F_TOK_BASE, F_BLOCK_FIRST, F_BLOCK_LAST = 11, 12, 13, 14, 15, 16

BF16, FP32 = 0, 1
DENSE, CAUSAL = 0, 1
MAX_SEQ_LEN = 2 ** 31 - 128      # 2,147,483,520
KV_TILE = 64                     # KV tokens per kernel tile (split granularity)


def cdiv(a, b):
    return -(-int(a) // int(b))


OK = (PKB_OK, F_NONE, -1)


def _bad(field, index):
    return (PKB_ERR_METADATA, field, int(index))


def _check_csr(B, P, ps, indptr, indices, seq_lens):
    """kv_indptr rules, then per-request sufficiency and live page IDs.

    Returns None when fine, else the failure triple.
    """
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    if indptr[0] != 0:
        return _bad(F_KV_INDPTR, 0)
    for b in range(1, B + 1):
        if indptr[b] <= indptr[b - 1]:
            return _bad(F_KV_INDPTR, b)
    if indptr[B] != indices.size:
        return _bad(F_KV_INDPTR, B)
    return None


def _check_pages(B, P, ps, indptr, indices, seq_lens):
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    for b in range(B):
        need = cdiv(int(seq_lens[b]), ps)
        if need > indptr[b + 1] - indptr[b]:
            return _bad(F_KV_INDPTR, b + 1)
        for j in range(int(indptr[b]), int(indptr[b]) + need):
            if not (0 <= indices[j] < P):
                return _bad(F_KV_INDICES, j)
    return None


# ----------------------------------------------------------------------------
# Block-sparse
# ----------------------------------------------------------------------------

def bsa_plan(B, Sq, Hq, Hkv, D, num_pages, page_size, q_block_size, kv_block_size,
             max_seq_len_kv, mask_type, window_left, qkv_dtype, out_dtype, num_cus):
    """Returns (status, plan dict)."""
    if min(B, Sq, Hq, Hkv, num_pages, q_block_size, num_cus) < 1 or page_size < 1:
        return PKB_ERR_ARG, None
    if Hq % Hkv:
        return PKB_ERR_SHAPE, None
    if qkv_dtype != BF16 or out_dtype not in (BF16, FP32):
        return PKB_ERR_DTYPE, None
    if D not in (128, 256):
        return PKB_ERR_UNSUPPORTED, None
    G = Hq // Hkv
    if (q_block_size * G) % 8:
        return PKB_ERR_ARG, None
    if not (kv_block_size in (8, 16, 32) or (kv_block_size > 0 and kv_block_size % 64 == 0)):
        return PKB_ERR_ARG, None
    if not (1 <= max_seq_len_kv <= MAX_SEQ_LEN):
        return PKB_ERR_ARG, None
    if mask_type not in (DENSE, CAUSAL) or window_left < -1:
        return PKB_ERR_ARG, None
    if window_left >= 0 and mask_type != CAUSAL:
        return PKB_ERR_ARG, None
    rows = q_block_size * G
    waves = 1 if rows <= 32 else (2 if rows <= 64 else 4)
    tile_m = 32 * waves
    nqb = cdiv(Sq, q_block_size)
    tpb = cdiv(rows, tile_m)
    plan = dict(group=G, rows_per_brow=rows, num_q_blocks=nqb,
                num_kv_blocks=cdiv(max_seq_len_kv, kv_block_size),
                valid_words=cdiv(max_seq_len_kv, 32), waves=waves, tile_m=tile_m,
                tiles_per_brow=tpb, grid_x=nqb * tpb, grid_y=Hkv, grid_z=B,
                kernel_id=kernel_id(D, waves, out_dtype))
    return PKB_OK, plan


def kernel_id(D, waves, out_dtype):
    return (1 if D == 256 else 0) * 100 + waves * 10 + (1 if out_dtype == FP32 else 0)


def bsa_validate(plan_args, kv_indptr, kv_indices, block_indptr, block_indices, seq_lens):
    """plan_args: dict with B, Hkv, num_pages, page_size, max_seq_len_kv,
    num_q_blocks, num_kv_blocks.  Returns (status, field, index)."""
    a = plan_args
    B, Hkv, P, ps = a["B"], a["Hkv"], a["num_pages"], a["page_size"]
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    r = _check_csr(B, P, ps, kv_indptr, kv_indices, seq_lens)
    if r:
        return r
    for b in range(B):
        if not (0 <= seq_lens[b] <= a["max_seq_len_kv"]):
            return _bad(F_SEQ_LENS, b)
    r = _check_pages(B, P, ps, kv_indptr, kv_indices, seq_lens)
    if r:
        return r
    bip = np.asarray(block_indptr, dtype=np.int64).reshape(B, Hkv, a["num_q_blocks"] + 1)
    bid = np.asarray(block_indices, dtype=np.int64)
    n = bid.size
    nq1 = a["num_q_blocks"] + 1
    for b in range(B):
        for h in range(Hkv):
            for r_ in range(nq1):
                f = (b * Hkv + h) * nq1 + r_
                v = bip[b, h, r_]
                if not (0 <= v <= n):
                    return _bad(F_BLOCK_INDPTR, f)
                if r_ > 0 and v < bip[b, h, r_ - 1]:
                    return _bad(F_BLOCK_INDPTR, f)
    for b in range(B):
        for h in range(Hkv):
            for r_ in range(a["num_q_blocks"]):
                seen = set()
                for k in range(int(bip[b, h, r_]), int(bip[b, h, r_ + 1])):
                    x = int(bid[k])
                    if not (0 <= x < a["num_kv_blocks"]) or x in seen:
                        return _bad(F_BLOCK_INDICES, k)
                    seen.add(x)
    return OK


# ----------------------------------------------------------------------------
# Prefill
# ----------------------------------------------------------------------------

def prefill_check_static(B, Hq, Hkv, D, num_pages, page_size, total_q, width, mask_type,
                         window_left, qkv_dtype, out_dtype, num_cus):
    if min(B, Hq, Hkv, num_pages, total_q, width, num_cus) < 1:
        return PKB_ERR_ARG
    if Hq % Hkv:
        return PKB_ERR_SHAPE
    if qkv_dtype != BF16 or out_dtype not in (BF16, FP32):
        return PKB_ERR_DTYPE
    if D not in (128, 256) or page_size not in (16, 32, 64, 128):
        return PKB_ERR_UNSUPPORTED
    if mask_type not in (DENSE, CAUSAL) or window_left < -1:
        return PKB_ERR_ARG
    if window_left >= 0 and mask_type != CAUSAL:
        return PKB_ERR_ARG
    return PKB_OK


def prefill_validate(args, qo_indptr, seq_lens, block_tables, row_stride):
    B, P, ps, C = args["B"], args["num_pages"], args["page_size"], args["block_table_width"]
    qo = np.asarray(qo_indptr, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    tab = np.asarray(block_tables, dtype=np.int64).ravel()
    if qo[0] != 0:
        return _bad(F_QO_INDPTR, 0)
    for b in range(1, B + 1):
        if qo[b] <= qo[b - 1]:
            return _bad(F_QO_INDPTR, b)
    if qo[B] != args["total_q"]:
        return _bad(F_QO_INDPTR, B)
    for b in range(B):
        L = seq_lens[b]
        if L < 0 or (args["mask_type"] == CAUSAL and qo[b + 1] - qo[b] > L):
            return _bad(F_SEQ_LENS, b)
    for b in range(B):
        need = cdiv(int(seq_lens[b]), ps)
        if need > C:
            return _bad(F_SEQ_LENS, b)
        for j in range(need):
            x = tab[b * row_stride + j]
            if not (0 <= x < P):
                return _bad(F_BLOCK_TABLES, b * row_stride + j)
    return OK


def prefill_waves(args):
    return 4


def prefill_tile_span(row0, tile_m, G, qlen, L, causal, window_left):
    """Visited KV positions [lo, hi) of one work tile (lo rounded down to 8)."""
    i0 = row0 // G
    i1 = (min(qlen * G, row0 + tile_m) - 1) // G
    p0 = L - qlen + i0
    p1 = L - qlen + i1
    hi = min(L, p1 + 1) if causal else L
    lo = max(0, p0 - window_left) if window_left >= 0 else 0
    lo = (lo // 8) * 8
    return lo, hi


def prefill_plan(args, qo_indptr, seq_lens):
    """Returns (status, plan dict, worklist [n, 2] int32)."""
    st = prefill_check_static(**{k: args[k] for k in (
        "B", "Hq", "Hkv", "D", "num_pages", "page_size", "total_q", "width", "mask_type",
        "window_left", "qkv_dtype", "out_dtype", "num_cus")})
    if st != PKB_OK:
        return st, None, None
    B, Hq, Hkv = args["B"], args["Hq"], args["Hkv"]
    G = Hq // Hkv
    waves = prefill_waves(args)
    tile_m = 32 * waves
    causal = args["mask_type"] == CAUSAL
    w = args["window_left"]
    qo = np.asarray(qo_indptr, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    items = []
    for b in range(B):
        qlen = int(qo[b + 1] - qo[b])
        L = int(seq_lens[b])
        for row0 in range(0, qlen * G, tile_m):
            lo, hi = prefill_tile_span(row0, tile_m, G, qlen, L, causal, w)
            items.append((max(0, hi - lo), b, row0))
    items.sort(key=lambda t: (-t[0], t[1], t[2]))
    wl = np.array([[b, r] for _, b, r in items], dtype=np.int32).reshape(-1, 2)
    plan = dict(group=G, waves=waves, tile_m=tile_m, n_work=len(items),
                grid_x=len(items), grid_y=Hkv, kernel_id=kernel_id(args["D"], waves,
                                                                 args["out_dtype"]),
                kv_tokens=int(sum(t[0] for t in items)))
    return PKB_OK, plan, wl


def prefill_plan_capacity(args, max_qlen):
    """Capacity work list for graph capture: every request may own up to
    max_qlen rows; tile indices from last to first, requests in order within
    one.  Returns (status, plan dict, worklist [n, 2] int32)."""
    st = prefill_check_static(**{k: args[k] for k in (
        "B", "Hq", "Hkv", "D", "num_pages", "page_size", "total_q", "width", "mask_type",
        "window_left", "qkv_dtype", "out_dtype", "num_cus")})
    if st != PKB_OK:
        return st, None, None
    if not (1 <= max_qlen <= args["total_q"]):
        return PKB_ERR_ARG, None, None
    B, Hq, Hkv = args["B"], args["Hq"], args["Hkv"]
    G = Hq // Hkv
    waves = prefill_waves(args)
    tile_m = 32 * waves
    T = cdiv(max_qlen * G, tile_m)
    wl = np.array([[b, t * tile_m] for t in range(T - 1, -1, -1) for b in range(B)],
                  dtype=np.int32).reshape(-1, 2)
    plan = dict(group=G, waves=waves, tile_m=tile_m, n_work=len(wl), grid_x=len(wl),
                grid_y=Hkv, kernel_id=kernel_id(args["D"], waves, args["out_dtype"]),
                kv_tokens=0)
    return PKB_OK, plan, wl


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------

def decode_policy(B, Hq, Hkv, D, max_seq_len, page_size, num_cus, per_wave=8, max_q=1):
    """Chunk (split) policy from the static maximum length.  A wide batch -- at
    most 16 query rows per KV head (max_q * Hq/Hkv), at most 256 requests and
    B*Hkv >= 2*num_cus -- runs in one pass: one chunk of max_seq_len tokens, no
    workspace.  Otherwise the chunk length CH starts at 1024 tokens (doubled
    while a request would need > 4096 chunks), then halves down to 64 until
    B*Hkv*ceil(max_seq_len/CH) >= per_wave items per persistent wave (4 waves
    per CU).  Returns (status, bytes, chunks, CH)."""
    if min(B, Hq, Hkv, num_cus) < 1 or page_size < 1:
        return PKB_ERR_ARG, 0, 0, 0
    if Hq % Hkv:
        return PKB_ERR_SHAPE, 0, 0, 0
    if D not in (128, 256):
        return PKB_ERR_UNSUPPORTED, 0, 0, 0
    if not (1 <= max_seq_len <= MAX_SEQ_LEN):
        return PKB_ERR_ARG, 0, 0, 0
    if max_q * (Hq // Hkv) <= 16 and B <= 256 and B * Hkv >= 2 * num_cus:
        return PKB_OK, 0, 1, max_seq_len
    CH = 1024
    while cdiv(max_seq_len, CH) > 4096:
        CH *= 2
    waves = 4 * num_cus
    while CH > 64 and B * Hkv * cdiv(max_seq_len, CH) < per_wave * waves:
        CH //= 2
    S = cdiv(max_seq_len, CH)
    split_len = CH
    nbytes = 0 if S == 1 else B * Hq * S * (D + 4) * 4   # fp32 partials (O, m, l, pad)
    return PKB_OK, nbytes, S, split_len


def decode_validate(B, P, ps, max_seq_len, kv_indptr, kv_indices, seq_lens):
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    r = _check_csr(B, P, ps, kv_indptr, kv_indices, seq_lens)
    if r:
        return r
    for b in range(B):
        if not (1 <= seq_lens[b] <= max_seq_len):
            return _bad(F_SEQ_LENS, b)
    r = _check_pages(B, P, ps, kv_indptr, kv_indices, seq_lens)
    if r:
        return r
    return OK


def decode_q_policy(B, max_q, Hq, Hkv, D, max_seq_len, page_size, num_cus):
    """Multi-token decode: the same chunk policy, aiming at 4 items per wave
    when max_q > 1; partials [B, max_q, Hq, S, D+4]."""
    if max_q < 1:
        return PKB_ERR_ARG, 0, 0, 0
    st, nbytes, S, CH = decode_policy(B, Hq, Hkv, D, max_seq_len, page_size, num_cus,
                                      4 if max_q > 1 else 8, max_q)
    if st != PKB_OK:
        return st, 0, 0, 0
    return PKB_OK, nbytes * max_q, S, CH


def decode_q_validate(B, P, ps, max_seq_len, kv_indptr, kv_indices, seq_lens, qo_indptr,
                      total_q, seq_len_q, max_seq_len_q, causal):
    """Decode page, description: the packed-offset contract (start at zero,
    strictly increasing, every delta at most max_seq_len_q, end at the query
    row count) and, for causal, every query length no greater than seq_len."""
    if qo_indptr is not None:
        if max_seq_len_q < 1 or total_q < 1:
            return PKB_ERR_ARG, F_NONE, -1
    elif seq_len_q < 1:
        return PKB_ERR_ARG, F_NONE, -1
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    r = _check_csr(B, P, ps, kv_indptr, kv_indices, seq_lens)
    if r:
        return r
    for b in range(B):
        if not (1 <= seq_lens[b] <= max_seq_len):
            return _bad(F_SEQ_LENS, b)
    if qo_indptr is not None:
        qo = np.asarray(qo_indptr, dtype=np.int64)
        if qo[0] != 0:
            return _bad(F_QO_INDPTR, 0)
        for b in range(B):
            d = qo[b + 1] - qo[b]
            if d < 1 or d > max_seq_len_q:
                return _bad(F_QO_INDPTR, b + 1)
        if qo[B] != total_q:
            return _bad(F_QO_INDPTR, B)
    if causal:
        for b in range(B):
            qlen = (qo_indptr[b + 1] - qo_indptr[b]) if qo_indptr is not None else seq_len_q
            if qlen > seq_lens[b]:
                return _bad(F_SEQ_LENS, b)
    r = _check_pages(B, P, ps, kv_indptr, kv_indices, seq_lens)
    if r:
        return r
    return OK


# ----------------------------------------------------------------------------
# Sage
# ----------------------------------------------------------------------------

def sage_validate(index, capacity, block_sparse_num, block_sizes, nums, uniform, B, H, Sq, Sk):
    if not (0 <= block_sparse_num <= capacity):
        return (PKB_ERR_ARG, F_NONE, -1)
    nqb = cdiv(Sq, 64)
    nkb = cdiv(Sk, 64)
    idx = np.asarray(index, dtype=np.int64).reshape(B, H, nqb, capacity)
    use_nums = nums is not None and not uniform
    if use_nums:
        nm = np.asarray(nums, dtype=np.int64).reshape(B, H, nqb)
        for f, x in enumerate(nm.ravel()):
            if not (0 <= x <= capacity):
                return _bad(F_Q2K_NUMS, f)
    for b in range(B):
        for h in range(H):
            for r in range(nqb):
                n = int(nm[b, h, r]) if use_nums else block_sparse_num
                seen = set()
                for k in range(n):
                    x = int(idx[b, h, r, k])
                    if not (0 <= x < nkb) or x in seen:
                        return _bad(F_Q2K_INDEX, ((b * H + h) * nqb + r) * capacity + k)
                    seen.add(x)
    if block_sizes is not None:
        for f, x in enumerate(np.asarray(block_sizes, dtype=np.int64).ravel()):
            if not (0 <= x <= 64):
                return _bad(F_BLOCK_SIZES, f)
    return OK


# ----------------------------------------------------------------------------
# QSA
# ----------------------------------------------------------------------------

def qsa_validate(lo, hi, blk_base, tok_base, block_first, block_last):
    """Page "qsa_forward", Notes: the metadata must describe one consistent packed
    partition.  Sequences are the runs of tokens sharing tok_base (starting at
    their own index); a sequence of length L at s0 owns blocks blk_base ..
    blk_base + ceil(L/4) - 1 inside [0, NB), block m spanning s0 + 4m ..
    min(s0 + 4m + 3, s0 + L - 1) (block_size 4, numbering restarting per
    sequence); lo/hi lie inside the sequence unless lo > hi (an empty row)."""
    lo, hi, bb, tb = (np.asarray(x, np.int64) for x in (lo, hi, blk_base, tok_base))
    bf, bl = np.asarray(block_first, np.int64), np.asarray(block_last, np.int64)
    T, NB = lo.size, bf.size
    if T < 1 or NB < 1:
        return PKB_ERR_ARG, F_NONE, -1
    seq_end = np.zeros(T, np.int64)
    t = 0
    while t < T:
        if tb[t] != t:
            return _bad(F_TOK_BASE, t)
        e = t + 1
        while e < T and tb[e] == t:
            e += 1
        if e < T and tb[e] != e:
            return _bad(F_TOK_BASE, e)
        nblk = cdiv(e - t, 4)
        for u in range(t, e):
            if bb[u] != bb[t] or bb[t] < 0 or bb[t] + nblk > NB:
                return _bad(F_BLK_BASE, u)
            seq_end[u] = e - 1
        t = e
    t = 0
    while t < T:
        e = int(seq_end[t]) + 1
        for m in range(cdiv(e - t, 4)):
            nb = int(bb[t]) + m
            if bf[nb] != t + 4 * m:
                return _bad(F_BLOCK_FIRST, nb)
            if bl[nb] != min(t + 4 * m + 3, e - 1):
                return _bad(F_BLOCK_LAST, nb)
        t = e
    for t in range(T):
        if lo[t] > hi[t]:
            continue
        if lo[t] < tb[t] or lo[t] > seq_end[t]:
            return _bad(F_LO, t)
        if hi[t] > seq_end[t]:
            return _bad(F_HI, t)
    return OK
