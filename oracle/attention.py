"""Plain fp64 definition of scaled-dot-product attention over a paged KV cache.

TEST INFRASTRUCTURE: only tests, ``__graft_entry__.smoke()`` and the bench's
cpu_baseline leg may call this module.  It shares no code with the HIP path.

The fast kernels (tiling, online softmax, split-KV) reach exactly this result up
to rounding order, so the oracle is the definition written out, per request b,
query row i and query head h (sources: the FlashInfer pages
"block_sparse_attention_with_paged_kv_cache", "batch_prefill_with_paged_kv_cache",
"prims_ts_batch_decode_with_kv_cache", "qsa_forward" (Returns / Notes) and
"bsa_attn_sm120_blk64_sage_fwd"):

  * kv head g = h // (Hq/Hkv): consecutive query heads share one KV head.
  * L = seq_lens[b]; query position p = L - qlen + i (bottom-right alignment).
  * key j (0 <= j < L) lives at page page(b, j), slot j % page_size, where the
    page comes from the CSR IDs (paged_kv_indices[paged_kv_indptr[b] + j//ps])
    or the row-strided table (block_tables[b, j//ps]).
  * key j is admitted when it is in a selected KV block of the query's BSR row
    (block-sparse only), its validity bit is set (LSB-first words), it passes the
    causal test j <= p (causal only), and the left window j >= p - w (w >= 0).
  * s_j = scale * <q, k_j>;  LSE = log sum_{admitted} exp(s_j) (natural log);
    out = output_scale * sum_{admitted} exp(s_j - LSE) v_j.
  * no admitted key: out = 0 exactly and LSE = -inf.

All inputs are NumPy arrays; floating inputs are converted to float64 exactly.
"""
from __future__ import annotations

import math
from collections import defaultdict

import numpy as np

from .fp8 import e4m3_decode


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # a torch tensor
        x = x.detach().to("cpu")
        import torch  # local: the oracle itself only needs NumPy
        if x.dtype in (torch.bfloat16, torch.float16, torch.float32):
            x = x.to(torch.float64)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x).astype(np.int64)


def attend(qrows: np.ndarray, keys: np.ndarray, vals: np.ndarray, admitted: np.ndarray,
           scale: float, out_scale: float = 1.0):
    """Softmax attention of ``qrows`` [n, D] over ``keys``/``vals`` [m, D].

    ``admitted`` [n, m] bool says which keys each row may see.  Returns
    out [n, D] and the natural-log LSE [n]; rows with no admitted key get an
    exact zero output and LSE = -inf.
    """
    n, D = qrows.shape
    out = np.zeros((n, vals.shape[1] if vals.ndim == 2 else D), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if keys.shape[0] == 0 or n == 0:
        return out, lse
    s = (qrows @ keys.T) * scale
    has = admitted.any(axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        s = np.where(admitted, s, -np.inf)
        m = np.where(has, s.max(axis=1), 0.0)
        w = np.where(admitted, np.exp(s - m[:, None]), 0.0)
    l = w.sum(axis=1)
    if has.any():
        out[has] = out_scale * (w[has] @ vals) / l[has, None]
        lse[has] = m[has] + np.log(l[has])
    return out, lse


def gather_csr(pool: np.ndarray, indptr, indices, b: int, L: int) -> np.ndarray:
    """Tokens 0..L-1 of request b from an HND pool [P, Hkv, ps, D] -> [L, Hkv, D]."""
    ps = pool.shape[2]
    j = np.arange(L)
    pages = np.asarray(indices)[int(indptr[b]) + j // ps]
    return pool[pages, :, j % ps, :]


def gather_table(pool: np.ndarray, table, b: int, L: int) -> np.ndarray:
    ps = pool.shape[2]
    j = np.arange(L)
    pages = np.asarray(table)[b, j // ps]
    return pool[pages, :, j % ps, :]


def bit_valid(valid_bits, b: int, j: np.ndarray) -> np.ndarray:
    """Bit (j mod 32) of word valid_bits[b, j // 32]; None means all valid."""
    if valid_bits is None:
        return np.ones(j.shape, dtype=bool)
    words = np.asarray(valid_bits).view(np.uint32) if np.asarray(valid_bits).dtype != np.uint32 \
        else np.asarray(valid_bits)
    w = words[b, j // 32].astype(np.uint64)
    return ((w >> (j % 32).astype(np.uint64)) & np.uint64(1)).astype(bool)


def position_mask(p: np.ndarray, j: np.ndarray, causal: bool, window_left: int) -> np.ndarray:
    """[len(p), len(j)] causal / left-window admission for query positions p."""
    ok = np.ones((p.shape[0], j.shape[0]), dtype=bool)
    if causal:
        ok &= j[None, :] <= p[:, None]
    if window_left >= 0:
        ok &= j[None, :] >= (p[:, None] - window_left)
    return ok


def _default_scale(scale, D):
    return (1.0 / math.sqrt(D)) if (scale is None or scale <= 0) else float(scale)


# ----------------------------------------------------------------------------
# Block-sparse attention over a paged cache (fixed-Q layout)
# ----------------------------------------------------------------------------

def bsa_reference(q, k, v, kv_indptr, kv_indices, block_indptr, block_indices,
                  q_block_size, kv_block_size, seq_lens, valid_bits=None,
                  mask="dense", window_left=-1, sm_scale=None, tokens=None):
    """Block-sparse paged attention.

    q [B, Sq, Hq, D]; k, v [P, Hkv, ps, D] (a combined [P, 2, ...] cache is
    passed as its two halves); block_indptr [B, Hkv, ceil(Sq/qbs)+1] holds
    absolute offsets into the flat block_indices.  Query row i belongs to BSR
    row i // q_block_size; logical KV block beta covers tokens
    [beta*kvbs, (beta+1)*kvbs) clipped to [0, L).

    tokens: optional list of (b, i) query tokens to evaluate.  Returns
    (out, lse): out [B, Sq, Hq, D] and lse [B*Sq, Hq] for all tokens, or
    [n, Hq, D] and [n, Hq] in the order of ``tokens``.
    """
    q = _f64(q); k = _f64(k); v = _f64(v)
    kv_indptr = _i64(kv_indptr); kv_indices = _i64(kv_indices)
    block_indptr = _i64(block_indptr); block_indices = _i64(block_indices)
    seq_lens = _i64(seq_lens)
    B, Sq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(sm_scale, D)
    causal = (mask == "causal")
    full = tokens is None
    if full:
        tokens = [(b, i) for b in range(B) for i in range(Sq)]
    out = np.zeros((len(tokens), Hq, D))
    lse = np.full((len(tokens), Hq), -np.inf)
    groups = defaultdict(list)
    for n, (b, i) in enumerate(tokens):
        groups[(int(b), int(i) // q_block_size)].append((n, int(i)))
    cache = {}
    for (b, r), items in sorted(groups.items()):
        L = int(seq_lens[b])
        if b not in cache:
            cache = {b: (gather_csr(k, kv_indptr, kv_indices, b, L),
                         gather_csr(v, kv_indptr, kv_indices, b, L))}
        Kb, Vb = cache[b]
        ns = np.array([n for n, _ in items])
        its = np.array([i for _, i in items])
        p = L - Sq + its
        for g in range(Hkv):
            lo, hi = block_indptr[b, g, r], block_indptr[b, g, r + 1]
            sel = np.unique(block_indices[lo:hi])
            if sel.size:
                j = (sel[:, None] * kv_block_size + np.arange(kv_block_size)[None, :]).ravel()
                j = np.unique(j[j < L])
            else:
                j = np.zeros(0, dtype=np.int64)
            adm = position_mask(p, j, causal, window_left) & bit_valid(valid_bits, b, j)[None, :]
            qr = q[b, its, g * G:(g + 1) * G, :].reshape(-1, D)
            o, s = attend(qr, Kb[j, g, :], Vb[j, g, :], np.repeat(adm, G, axis=0), scale)
            out[ns, g * G:(g + 1) * G, :] = o.reshape(len(its), G, D)
            lse[ns, g * G:(g + 1) * G] = s.reshape(len(its), G)
    if full:
        return out.reshape(B, Sq, Hq, D), lse.reshape(B * Sq, Hq)
    return out, lse


# ----------------------------------------------------------------------------
# Packed-Q paged prefill (row-strided block tables)
# ----------------------------------------------------------------------------

def prefill_reference(q, k, v, qo_indptr, block_tables, seq_lens, mask="causal",
                      window_left=-1, sm_scale=None, output_scale=1.0, rows=None,
                      chunk=512):
    """Packed-Q attention: q [total_q, Hq, D]; request b owns rows
    qo_indptr[b]:qo_indptr[b+1]; its pages are block_tables[b, :].

    rows: optional list of packed row indices to evaluate.  Returns (out, lse)
    with out [total_q, Hq, D] / lse [total_q, Hq], or [n, ...] for ``rows``.
    """
    q = _f64(q); k = _f64(k); v = _f64(v)
    qo = _i64(qo_indptr); table = _i64(block_tables); seq_lens = _i64(seq_lens)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(sm_scale, D)
    causal = (mask == "causal")
    full = rows is None
    if full:
        rows = list(range(T))
    rows = np.asarray(rows, dtype=np.int64)
    req = np.searchsorted(qo, rows, side="right") - 1
    out = np.zeros((len(rows), Hq, D))
    lse = np.full((len(rows), Hq), -np.inf)
    for b in np.unique(req):
        b = int(b)
        L = int(seq_lens[b])
        qlen = int(qo[b + 1] - qo[b])
        Kb = gather_table(k, table, b, L)
        Vb = gather_table(v, table, b, L)
        sel = np.nonzero(req == b)[0]
        j = np.arange(L)
        for c0 in range(0, len(sel), chunk):
            ns = sel[c0:c0 + chunk]
            its = rows[ns] - qo[b]
            p = L - qlen + its
            adm = position_mask(p, j, causal, window_left)
            for g in range(Hkv):
                qr = q[rows[ns], g * G:(g + 1) * G, :].reshape(-1, D)
                o, s = attend(qr, Kb[:, g, :], Vb[:, g, :], np.repeat(adm, G, axis=0),
                              scale, output_scale)
                out[ns, g * G:(g + 1) * G, :] = o.reshape(len(ns), G, D)
                lse[ns, g * G:(g + 1) * G] = s.reshape(len(ns), G)
    return out, lse


# ----------------------------------------------------------------------------
# Single-token paged decode (CSR page IDs)
# ----------------------------------------------------------------------------

def decode_reference(q, k, v, kv_indptr, kv_indices, seq_lens, mask="dense",
                     window_left=-1, bmm1_scale=None, bmm2_scale=1.0, requests=None):
    """Decode: q [B, Hq, D], one query token per request at position L-1.

    bmm1_scale is the softmax scale (default 1/sqrt(D)); bmm2_scale multiplies
    the normalised output.  Returns out [B, Hq, D], lse [B, Hq] (or the rows of
    ``requests``).
    """
    q = _f64(q); k = _f64(k); v = _f64(v)
    kv_indptr = _i64(kv_indptr); kv_indices = _i64(kv_indices); seq_lens = _i64(seq_lens)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = _default_scale(bmm1_scale, D)
    causal = (mask == "causal")
    reqs = list(range(B)) if requests is None else [int(x) for x in requests]
    out = np.zeros((len(reqs), Hq, D))
    lse = np.full((len(reqs), Hq), -np.inf)
    for n, b in enumerate(reqs):
        L = int(seq_lens[b])
        Kb = gather_csr(k, kv_indptr, kv_indices, b, L)
        Vb = gather_csr(v, kv_indptr, kv_indices, b, L)
        j = np.arange(L)
        adm = position_mask(np.array([L - 1]), j, causal, window_left)
        for g in range(Hkv):
            o, s = attend(q[b, g * G:(g + 1) * G, :], Kb[:, g, :], Vb[:, g, :],
                          np.repeat(adm, G, axis=0), scale, bmm2_scale)
            out[n, g * G:(g + 1) * G] = o
            lse[n, g * G:(g + 1) * G] = s
    return out, lse


def decode_q_reference(q, k, v, kv_indptr, kv_indices, seq_lens, qo_indptr=None,
                       mask="causal", window_left=-1, bmm1_scale=None, bmm2_scale=1.0):
    """Multi-token decode over CSR pages ("prims_ts_batch_decode_with_kv_cache",
    description: seq_len_q > 1 uses token-major [B, SQ, Hq, D]; with qo_indptr,
    packed [total_q, Hq, D] where request b owns rows qo_indptr[b]:qo_indptr[b+1]).
    Query i of request b sits at position L - qlen + i.  Returns (out, lse) in the
    query's layout ([..., Hq, D] and [..., Hq])."""
    q = _f64(q); k = _f64(k); v = _f64(v)
    kv_indptr = _i64(kv_indptr); kv_indices = _i64(kv_indices); seq_lens = _i64(seq_lens)
    B = len(seq_lens)
    Hkv = k.shape[1]
    D = q.shape[-1]
    Hq = q.shape[-2]
    G = Hq // Hkv
    scale = _default_scale(bmm1_scale, D)
    causal = (mask == "causal")
    if qo_indptr is None:
        SQ = q.shape[1]
        qo = np.arange(B + 1, dtype=np.int64) * SQ
        qp = q.reshape(B * SQ, Hq, D)
    else:
        qo = _i64(qo_indptr)
        qp = q
    out = np.zeros(qp.shape)
    lse = np.full(qp.shape[:2], -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        qlen = int(qo[b + 1] - qo[b])
        Kb = gather_csr(k, kv_indptr, kv_indices, b, L)
        Vb = gather_csr(v, kv_indptr, kv_indices, b, L)
        p = L - qlen + np.arange(qlen)
        adm = position_mask(p, np.arange(L), causal, window_left)
        for g in range(Hkv):
            qr = qp[qo[b]:qo[b + 1], g * G:(g + 1) * G, :].reshape(-1, D)
            o, s = attend(qr, Kb[:, g, :], Vb[:, g, :], np.repeat(adm, G, axis=0), scale,
                          bmm2_scale)
            out[qo[b]:qo[b + 1], g * G:(g + 1) * G] = o.reshape(qlen, G, D)
            lse[qo[b]:qo[b + 1], g * G:(g + 1) * G] = s.reshape(qlen, G)
    if qo_indptr is None:
        return out.reshape(q.shape), lse.reshape(B, q.shape[1], Hq)
    return out, lse


# ----------------------------------------------------------------------------
# Sage-style prequantized block-sparse attention
# ----------------------------------------------------------------------------

def sage_dequantize(q_int8, k_int8, v_fp8_codes, q_scale, k_scale, v_scale, Sk=None):
    """Exact dequantisation (page "bsa_attn_sm120_blk64_sage_fwd", Parameters):

    Q~[b,h,i,:] = q_int8[b,h,i,:] * q_scale[b,h,i//32]   (ceil(Sq/128)*4 scales)
    K~[b,h,j,:] = k_int8[b,h,j,:] * k_scale[b,h,j//64]
    V~[b,h,j,d] = e4m3(v_fp8[b,h,d,j]) * v_scale[b,h,d]  (HDS storage)
    """
    qi = _i64(q_int8).astype(np.float64)
    ki = _i64(k_int8).astype(np.float64)
    Sq = qi.shape[2]
    Sk = ki.shape[2] if Sk is None else Sk
    qs = _f64(q_scale); ks = _f64(k_scale); vs = _f64(v_scale)
    Qd = qi * qs[:, :, np.arange(Sq) // 32][..., None]
    Kd = ki * ks[:, :, np.arange(Sk) // 64][..., None]
    codes = np.asarray(v_fp8_codes)
    Vd = e4m3_decode(codes[..., :Sk]).transpose(0, 1, 3, 2) * vs[:, :, None, :]
    return Qd, Kd, Vd


def sage_block_size(block_sizes, b, h, beta):
    if block_sizes is None:
        return 64
    bs = np.asarray(block_sizes)
    if bs.ndim == 1:
        return int(bs[beta])
    if bs.ndim == 2:
        return int(bs[b, beta])
    return int(bs[b, h, beta])


def sage_reference(q_int8, k_int8, v_fp8_codes, q_scale, k_scale, v_scale,
                   q2k_block_index, block_sparse_num, block_sizes=None,
                   q2k_block_nums=None, uniform_block_count=False, softmax_scale=None,
                   Sk=None, rows=None, mask="dense", with_lse=False):
    """Sage block-sparse attention on the dequantised inputs (MHA, D=128,
    64-token blocks).

    Query block r = i // 64 uses n = q2k_block_nums[b,h,r] when counts are given
    and ``uniform_block_count`` is false, else ``block_sparse_num``; it selects
    blocks q2k_block_index[b,h,r,:n].  Block beta admits its first
    block_sizes[..beta] tokens, clipped to Sk.  With mask="causal" (the
    token-level causal rule of the block-sparse page, bottom-right aligned:
    query i sits at position Sk - Sq + i) a selected token j is admitted only
    when j <= Sk - Sq + i.  rows: optional list of (b, h, r) query blocks.
    Returns out [B, H, Sq, 128] (NaN outside ``rows``) and, with ``with_lse``,
    the natural-log LSE [B, H, Sq] of the scaled scores (-inf for empty rows).
    """
    Qd, Kd, Vd = sage_dequantize(q_int8, k_int8, v_fp8_codes, q_scale, k_scale, v_scale, Sk)
    B, H, Sq, D = Qd.shape
    Sk = Kd.shape[2]
    scale = _default_scale(softmax_scale, D)
    index = _i64(q2k_block_index)
    nums = None if q2k_block_nums is None else _i64(q2k_block_nums)
    nqb = -(-Sq // 64)
    if rows is None:
        rows = [(b, h, r) for b in range(B) for h in range(H) for r in range(nqb)]
        out = np.zeros((B, H, Sq, D))
        lse = np.full((B, H, Sq), -np.inf)
    else:
        out = np.full((B, H, Sq, D), np.nan)
        lse = np.full((B, H, Sq), np.nan)
    for b, h, r in rows:
        n = int(nums[b, h, r]) if (nums is not None and not uniform_block_count) \
            else int(block_sparse_num)
        toks = []
        for beta in np.unique(index[b, h, r, :n]):
            bs = sage_block_size(block_sizes, b, h, int(beta))
            t = np.arange(int(beta) * 64, int(beta) * 64 + bs)
            toks.append(t[t < Sk])
        j = np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)
        i0, i1 = r * 64, min(r * 64 + 64, Sq)
        p = Sk - Sq + np.arange(i0, i1)
        adm = position_mask(p, j, mask == "causal", -1)
        o, s = attend(Qd[b, h, i0:i1], Kd[b, h, j], Vd[b, h, j], adm, scale)
        out[b, h, i0:i1] = o
        lse[b, h, i0:i1] = s
    return (out, lse) if with_lse else out


# ----------------------------------------------------------------------------
# Packed-query token-granular sparse attention (QSA)
# ----------------------------------------------------------------------------

def qsa_reference(q, k, v, sel_blocks, lo, hi, block_first, block_last, scale=None,
                  tokens=None):
    """Page "qsa_forward" (Parameters, Returns, Notes): query token t attends to
    the key tokens j of every global block nb it selects (sel_blocks[t, nb] != 0,
    block nb spanning block_first[nb] .. block_last[nb] inclusive) that also lie
    in [lo[t], hi[t]] (inclusive); nothing else is added (no implicit causal
    tail).  K/V are the packed token arrays [T, Hkv, D]; query head h reads KV
    head h // (Hq / Hkv).  Empty rows: out 0, LSE -inf.  Returns out [T, Hq, D]
    and lse [Hq, T] (the page's layout).  ``tokens``: optional subset of query
    tokens (others NaN)."""
    q = _f64(q); k = _f64(k); v = _f64(v)
    sel = np.asarray(sel_blocks)
    lo = _i64(lo); hi = _i64(hi)
    bf = _i64(block_first); bl = _i64(block_last)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = _default_scale(scale, D)
    fill = 0.0 if tokens is None else np.nan
    out = np.full((T, Hq, D), fill)
    lse = np.full((Hq, T), -np.inf if tokens is None else np.nan)
    for t in (range(T) if tokens is None else tokens):
        spans = [np.arange(bf[nb], bl[nb] + 1) for nb in np.nonzero(sel[t])[0]]
        j = np.unique(np.concatenate(spans)) if spans else np.zeros(0, np.int64)
        j = j[(j >= lo[t]) & (j <= hi[t])]
        for g in range(Hkv):
            o, s = attend(q[t, g * G:(g + 1) * G], k[j, g], v[j, g],
                          np.ones((G, j.size), bool), sc)
            out[t, g * G:(g + 1) * G] = o
            lse[g * G:(g + 1) * G, t] = s
    return out, lse
