"""Loop-only attention for tiny inputs -- TEST INFRASTRUCTURE.

A second, independent statement of the same definition as ``attention.py``
(FlashInfer pages "block_sparse_attention_with_paged_kv_cache",
"batch_prefill_with_paged_kv_cache", "prims_ts_batch_decode_with_kv_cache"),
written with plain Python loops over (request, query, head, key) and
``math.fsum`` so that it shares no vectorised code with the main oracle.  Use
only on inputs with a few thousand (query, key) pairs.
"""
from __future__ import annotations

import math


def _lst(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        if x.is_floating_point():
            x = x.to(torch.float64)
        return x.tolist()
    if hasattr(x, "tolist"):
        return x.tolist()
    return x


def _row_softmax(qvec, keys, vals, scale, out_scale):
    """keys/vals: lists of D-vectors for the admitted keys, in any order."""
    D = len(qvec)
    if not keys:
        return [0.0] * D, -math.inf
    s = [scale * math.fsum(qvec[d] * kk[d] for d in range(D)) for kk in keys]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    tot = math.fsum(e)
    lse = mx + math.log(tot)
    out = [out_scale * math.fsum(e[t] * vals[t][d] for t in range(len(keys))) / tot
           for d in range(D)]
    return out, lse


def _bit(words, b, j):
    if words is None:
        return True
    w = int(words[b][j // 32]) & 0xFFFFFFFF
    return ((w >> (j % 32)) & 1) == 1


def bsa_bruteforce(q, k, v, kv_indptr, kv_indices, block_indptr, block_indices, qbs, kvbs,
                   seq_lens, valid_bits=None, mask="dense", window_left=-1, sm_scale=None):
    q, k, v = _lst(q), _lst(k), _lst(v)
    kv_indptr, kv_indices = _lst(kv_indptr), _lst(kv_indices)
    block_indptr, block_indices = _lst(block_indptr), _lst(block_indices)
    seq_lens = _lst(seq_lens)
    words = _lst(valid_bits) if valid_bits is not None else None
    B, Sq, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, ps = len(k[0]), len(k[0][0])
    grp = Hq // Hkv
    scale = sm_scale if sm_scale else 1.0 / math.sqrt(D)
    out = [[[None] * Hq for _ in range(Sq)] for _ in range(B)]
    lse = [[None] * Hq for _ in range(B * Sq)]
    for b in range(B):
        L = seq_lens[b]
        for i in range(Sq):
            pos = L - Sq + i
            r = i // qbs
            for h in range(Hq):
                g = h // grp
                blocks = set(block_indices[block_indptr[b][g][r]:block_indptr[b][g][r + 1]])
                keys, vals = [], []
                for j in range(L):
                    if (j // kvbs) not in blocks:
                        continue
                    if not _bit(words, b, j):
                        continue
                    if mask == "causal" and j > pos:
                        continue
                    if window_left >= 0 and j < pos - window_left:
                        continue
                    page = kv_indices[kv_indptr[b] + j // ps]
                    keys.append(k[page][g][j % ps])
                    vals.append(v[page][g][j % ps])
                o, s = _row_softmax(q[b][i][h], keys, vals, scale, 1.0)
                out[b][i][h] = o
                lse[b * Sq + i][h] = s
    return out, lse


def prefill_bruteforce(q, k, v, qo_indptr, block_tables, seq_lens, mask="causal",
                       window_left=-1, sm_scale=None, output_scale=1.0):
    q, k, v = _lst(q), _lst(k), _lst(v)
    qo, table, seq_lens = _lst(qo_indptr), _lst(block_tables), _lst(seq_lens)
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, ps = len(k[0]), len(k[0][0])
    grp = Hq // Hkv
    scale = sm_scale if sm_scale else 1.0 / math.sqrt(D)
    out = [None] * T
    lse = [None] * T
    for b in range(len(seq_lens)):
        L = seq_lens[b]
        qlen = qo[b + 1] - qo[b]
        for i in range(qlen):
            row = qo[b] + i
            pos = L - qlen + i
            out[row] = [None] * Hq
            lse[row] = [None] * Hq
            for h in range(Hq):
                g = h // grp
                keys, vals = [], []
                for j in range(L):
                    if mask == "causal" and j > pos:
                        continue
                    if window_left >= 0 and j < pos - window_left:
                        continue
                    page = table[b][j // ps]
                    keys.append(k[page][g][j % ps])
                    vals.append(v[page][g][j % ps])
                out[row][h], lse[row][h] = _row_softmax(q[row][h], keys, vals, scale,
                                                        output_scale)
    return out, lse


def decode_bruteforce(q, k, v, kv_indptr, kv_indices, seq_lens, mask="dense",
                      window_left=-1, bmm1_scale=None, bmm2_scale=1.0):
    q, k, v = _lst(q), _lst(k), _lst(v)
    kv_indptr, kv_indices, seq_lens = _lst(kv_indptr), _lst(kv_indices), _lst(seq_lens)
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, ps = len(k[0]), len(k[0][0])
    grp = Hq // Hkv
    scale = bmm1_scale if bmm1_scale else 1.0 / math.sqrt(D)
    out = [[None] * Hq for _ in range(B)]
    lse = [[None] * Hq for _ in range(B)]
    for b in range(B):
        L = seq_lens[b]
        pos = L - 1
        for h in range(Hq):
            g = h // grp
            keys, vals = [], []
            for j in range(L):
                if mask == "causal" and j > pos:
                    continue
                if window_left >= 0 and j < pos - window_left:
                    continue
                page = kv_indices[kv_indptr[b] + j // ps]
                keys.append(k[page][g][j % ps])
                vals.append(v[page][g][j % ps])
            out[b][h], lse[b][h] = _row_softmax(q[b][h], keys, vals, scale, bmm2_scale)
    return out, lse


def decode_q_bruteforce(q, k, v, kv_indptr, kv_indices, seq_lens, qo_indptr,
                        mask="causal", window_left=-1, bmm1_scale=None, bmm2_scale=1.0):
    """Packed multi-token decode, q [total_q, Hq, D], one loop per admitted key."""
    q, k, v = _lst(q), _lst(k), _lst(v)
    kv_indptr, kv_indices = _lst(kv_indptr), _lst(kv_indices)
    seq_lens, qo = _lst(seq_lens), _lst(qo_indptr)
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, ps = len(k[0]), len(k[0][0])
    grp = Hq // Hkv
    scale = bmm1_scale if bmm1_scale else 1.0 / math.sqrt(D)
    out = [None] * T
    lse = [None] * T
    for b in range(len(seq_lens)):
        L = seq_lens[b]
        qlen = qo[b + 1] - qo[b]
        for i in range(qlen):
            row = qo[b] + i
            pos = L - qlen + i
            out[row] = [None] * Hq
            lse[row] = [None] * Hq
            for h in range(Hq):
                g = h // grp
                keys, vals = [], []
                for j in range(L):
                    if mask == "causal" and j > pos:
                        continue
                    if window_left >= 0 and j < pos - window_left:
                        continue
                    page = kv_indices[kv_indptr[b] + j // ps]
                    keys.append(k[page][g][j % ps])
                    vals.append(v[page][g][j % ps])
                out[row][h], lse[row][h] = _row_softmax(q[row][h], keys, vals, scale,
                                                        bmm2_scale)
    return out, lse


def qsa_bruteforce(q, k, v, sel_blocks, lo, hi, block_first, block_last, scale):
    """Page "qsa_forward": loops over (token, head, block, key) -- tiny inputs only.
    Returns (out [T][Hq][D], lse [Hq][T])."""
    q, k, v = _lst(q), _lst(k), _lst(v)
    sel, lo, hi = _lst(sel_blocks), _lst(lo), _lst(hi)
    bf, bl = _lst(block_first), _lst(block_last)
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    out = [[None] * Hq for _ in range(T)]
    lse = [[None] * T for _ in range(Hq)]
    for t in range(T):
        keys = set()
        for nb in range(len(bf)):
            if sel[t][nb]:
                for j in range(bf[nb], bl[nb] + 1):
                    if lo[t] <= j <= hi[t]:
                        keys.add(j)
        keys = sorted(keys)
        for h in range(Hq):
            g = h // G
            o, s = _row_softmax(q[t][h], [k[j][g] for j in keys], [v[j][g] for j in keys],
                                scale, 1.0)
            out[t][h] = o
            lse[h][t] = s
    return out, lse
