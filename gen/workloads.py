"""Seeded synthetic inputs for paged / block-sparse attention.

This module only *builds inputs*: random tensors, page tables, sparse block
lists and validity bitmaps.  It holds none of the attention arithmetic, so both
the fp64 oracle (``oracle/``) and the HIP path (``paged_kv_block_amd``) can use
it without sharing code with each other.

Every generator draws from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order.  Floating-point tensors are drawn as N(0, 1) float32 and rounded to
bfloat16 (round-to-nearest-even, via a CPU ``torch`` cast).  Integer metadata is
int32, bitmaps are uint32.  All tensors are returned on the CPU; callers copy
them to the device.

Workload shapes follow the problem statements of the FlashInfer pages
"block_sparse_attention_with_paged_kv_cache" (Parameters: q, paged_kv_cache,
paged_kv_indptr/indices, block_indptr/indices, kv_valid_bits),
"batch_prefill_with_paged_kv_cache" (Parameters: qo_indptr, block_tables, HND
pools), "prims_ts_batch_decode_with_kv_cache" (CSR page IDs, seq_lens) and
"bsa_attn_sm120_blk64_sage_fwd" (int8 Q/K, fp8 E4M3 HDS V, scales,
q2k_block_index/nums, block_sizes).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

INV_SQRT = lambda d: 1.0 / math.sqrt(d)  # noqa: E731  (default softmax scale 1/sqrt(D))


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def randn_bf16(rng: np.random.Generator, shape) -> torch.Tensor:
    """N(0,1) float32 draws rounded to bfloat16 (RNE), as a CPU tensor."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def _i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32)))


# ----------------------------------------------------------------------------
# Page tables
# ----------------------------------------------------------------------------

def csr_page_table(rng, seq_lens, page_size, extra_pages=0, slack=None):
    """CSR page IDs: request b owns ceil(L_b/ps) (+ slack[b]) entries.

    Physical IDs are a random permutation of a pool of
    ``sum(entries) + extra_pages`` pages, so IDs are not identity ordered.
    Returns (indptr[B+1], indices[n], num_pages).
    """
    need = [max(1, -(-int(L) // page_size)) for L in seq_lens]
    if slack is not None:
        need = [n + int(s) for n, s in zip(need, slack)]
    total = int(sum(need))
    num_pages = total + int(extra_pages)
    perm = rng.permutation(num_pages)
    indptr = np.zeros(len(need) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(need)
    indices = perm[:total].astype(np.int32)
    return indptr, indices, num_pages


def strided_block_table(rng, seq_lens, page_size, extra_pages=0, width=None):
    """Row-strided page table [B, C] (padded with -1), from a permuted pool."""
    need = [max(1, -(-int(L) // page_size)) for L in seq_lens]
    total = int(sum(need))
    num_pages = total + int(extra_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    C = int(width if width is not None else max(need))
    table = np.full((len(need), C), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, num_pages


def random_bits(rng, B, max_len, p_one):
    """uint32 bitmap [B, ceil(max_len/32)]; each bit is 1 with probability p_one."""
    W = -(-int(max_len) // 32)
    bits = rng.random(size=(B, W, 32)) < p_one
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    words = (bits.astype(np.uint64) * weights).sum(axis=2).astype(np.uint32)
    return words


def bits_tensor(words: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).view(torch.int32)


# ----------------------------------------------------------------------------
# Case containers
# ----------------------------------------------------------------------------

@dataclass
class BsaCase:
    """Fixed-Q paged block-sparse attention inputs (CPU tensors)."""
    q: torch.Tensor                 # [B, Sq, Hq, D] bf16
    k: torch.Tensor                 # [P, Hkv, ps, D] bf16
    v: torch.Tensor                 # [P, Hkv, ps, D] bf16
    kv_indptr: np.ndarray           # [B+1] int32
    kv_indices: np.ndarray          # [n] int32
    block_indptr: np.ndarray        # [B, Hkv, NQB+1] int32 (absolute offsets)
    block_indices: np.ndarray       # [nnz] int32 logical KV block IDs
    seq_lens: np.ndarray            # [B] int32
    q_block_size: int
    kv_block_size: int
    max_seq_len_kv: int
    valid_bits: Optional[np.ndarray] = None   # [B, ceil(max_len/32)] uint32
    mask: str = "dense"
    window_left: int = -1
    sm_scale: Optional[float] = None
    name: str = ""

    @property
    def dims(self):
        B, Sq, Hq, D = self.q.shape
        P, Hkv, ps, _ = self.k.shape
        return B, Sq, Hq, Hkv, D, P, ps


@dataclass
class PrefillCase:
    q: torch.Tensor                 # [total_q, Hq, D] bf16
    k: torch.Tensor                 # [P, Hkv, ps, D]
    v: torch.Tensor
    qo_indptr: np.ndarray           # [B+1]
    block_tables: np.ndarray        # [B, C] (-1 padded)
    seq_lens: np.ndarray            # [B]
    mask: str = "causal"
    window_left: int = -1
    sm_scale: Optional[float] = None
    output_scale: float = 1.0
    name: str = ""


@dataclass
class DecodeCase:
    q: torch.Tensor                 # [B, Hq, D]
    k: torch.Tensor                 # [P, Hkv, ps, D]
    v: torch.Tensor
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    seq_lens: np.ndarray
    max_seq_len: int
    mask: str = "dense"
    window_left: int = -1
    bmm1_scale: Optional[float] = None
    bmm2_scale: float = 1.0
    name: str = ""


@dataclass
class SageCase:
    q_int8: torch.Tensor            # [B, H, Sq, 128] int8
    k_int8: torch.Tensor            # [B, H, Sk, 128] int8
    v_fp8: torch.Tensor             # [B, H, 128, ceil(Sk/64)*64] float8_e4m3fn (HDS)
    q_scale: torch.Tensor           # [B, H, ceil(Sq/128)*4] fp32
    k_scale: torch.Tensor           # [B, H, ceil(Sk/64)] fp32
    v_scale: torch.Tensor           # [B, H, 128] fp32
    q2k_block_index: np.ndarray     # [B, H, ceil(Sq/64), cap] int32
    block_sparse_num: int
    block_sizes: Optional[np.ndarray] = None   # [nkb] | [B,nkb] | [B,H,nkb]
    q2k_block_nums: Optional[np.ndarray] = None  # [B, H, ceil(Sq/64)]
    uniform_block_count: bool = False
    softmax_scale: Optional[float] = None
    Sk: int = 0
    name: str = ""


@dataclass
class QsaCase:
    """Packed-query token-granular sparse attention inputs (non-paged K/V)."""
    q: torch.Tensor                 # [T, Hq, D] bf16
    k: torch.Tensor                 # [T, Hkv, D] bf16
    v: torch.Tensor                 # [T, Hkv, D] bf16
    sel_blocks: np.ndarray          # [T, NB] uint8, nonzero selects a global block
    lo: np.ndarray                  # [T] int32 inclusive key bounds
    hi: np.ndarray                  # [T] int32
    blk_base: np.ndarray            # [T] int32 first global block of the token's sequence
    tok_base: np.ndarray            # [T] int32 first global token of the token's sequence
    block_first: np.ndarray         # [NB] int32 inclusive token span of each block
    block_last: np.ndarray          # [NB] int32
    seq_lens: np.ndarray            # [n_seq] packed sequence lengths
    scale: float = 0.0625
    name: str = ""


# ----------------------------------------------------------------------------
# Block-sparse selections
# ----------------------------------------------------------------------------

def bsr_bernoulli(rng, B, Hkv, Sq, qbs, kvbs, seq_lens, p=0.5, always_last=True,
                  max_seq_len_kv=None, out_of_range=0, allow_empty=False):
    """Each BSR row selects each in-range KV block with probability p.

    The last in-range block is always included (``always_last``).  ``out_of_range``
    extra block IDs in [ceil(L/kvbs), ceil(max_len/kvbs)) may be appended to test
    that blocks past the live length contribute nothing.  Offsets are absolute
    into one flat ``block_indices`` array.
    """
    NQB = -(-Sq // qbs)
    maxlen = max_seq_len_kv or int(max(seq_lens))
    nblk_cap = -(-maxlen // kvbs)
    indptr = np.zeros((B, Hkv, NQB + 1), dtype=np.int32)
    flat = []
    off = 0
    for b in range(B):
        nb = -(-int(seq_lens[b]) // kvbs)
        for h in range(Hkv):
            indptr[b, h, 0] = off
            for r in range(NQB):
                sel = [beta for beta in range(max(nb - 1, 0)) if rng.random() < p]
                if always_last and nb > 0:
                    sel.append(nb - 1)
                if allow_empty and rng.random() < 0.15:
                    sel = []
                extra = [int(x) for x in rng.integers(nb, nblk_cap, size=out_of_range)] \
                    if (out_of_range and nb < nblk_cap) else []
                sel = sorted(set(sel) | set(extra))
                flat.extend(sel)
                off += len(sel)
                indptr[b, h, r + 1] = off
    return indptr, np.asarray(flat, dtype=np.int32)


def bsr_causal_topk(rng, B, Hkv, NQB, nsel=16):
    """Row r selects min(nsel, r+1) causal-admissible blocks (qbs == kvbs).

    For r >= nsel-1 the set is {0, r} plus nsel-2 distinct blocks drawn from
    {1..r-1}; for smaller r it is all of {0..r}.  Sorted, drawn independently per
    (b, kv head, row).
    """
    indptr = np.zeros((B, Hkv, NQB + 1), dtype=np.int32)
    flat = []
    off = 0
    for b in range(B):
        for h in range(Hkv):
            indptr[b, h, 0] = off
            for r in range(NQB):
                if r + 1 <= nsel:
                    sel = list(range(r + 1))
                else:
                    mid = rng.choice(np.arange(1, r), size=nsel - 2, replace=False)
                    sel = sorted([0, r] + [int(x) for x in mid])
                flat.extend(sel)
                off += len(sel)
                indptr[b, h, r + 1] = off
    return indptr, np.asarray(flat, dtype=np.int32)


# ----------------------------------------------------------------------------
# Generic builders (used by parity sweeps)
# ----------------------------------------------------------------------------

def make_bsa(seed, B, Sq, Hq, Hkv, D, seq_lens, page_size, qbs, kvbs, mask="dense",
             window_left=-1, bits_p=None, p_sel=0.5, extra_pages=0,
             max_seq_len_kv=None, out_of_range=0, allow_empty=False,
             sm_scale=None, name=""):
    rng = _rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    maxlen = int(max_seq_len_kv or max(int(seq_lens.max()), 1))
    q = randn_bf16(rng, (B, Sq, Hq, D))
    indptr, indices, P = csr_page_table(rng, seq_lens, page_size, extra_pages)
    k = randn_bf16(rng, (P, Hkv, page_size, D))
    v = randn_bf16(rng, (P, Hkv, page_size, D))
    bip, bid = bsr_bernoulli(rng, B, Hkv, Sq, qbs, kvbs, seq_lens, p=p_sel,
                             max_seq_len_kv=maxlen, out_of_range=out_of_range,
                             allow_empty=allow_empty)
    bits = random_bits(rng, B, maxlen, bits_p) if bits_p is not None else None
    return BsaCase(q, k, v, indptr, indices, bip, bid, seq_lens, qbs, kvbs, maxlen,
                   bits, mask, window_left, sm_scale, name)


def make_prefill(seed, B, qlens, prefixes, Hq, Hkv, D, page_size, mask="causal",
                 window_left=-1, extra_pages=0, sm_scale=None, output_scale=1.0,
                 name=""):
    rng = _rng(seed)
    qlens = np.asarray(qlens, dtype=np.int64)
    seq_lens = (qlens + np.asarray(prefixes, dtype=np.int64)).astype(np.int32)
    qo = np.zeros(B + 1, dtype=np.int32)
    qo[1:] = np.cumsum(qlens)
    q = randn_bf16(rng, (int(qo[-1]), Hq, D))
    table, P = strided_block_table(rng, seq_lens, page_size, extra_pages)
    k = randn_bf16(rng, (P, Hkv, page_size, D))
    v = randn_bf16(rng, (P, Hkv, page_size, D))
    return PrefillCase(q, k, v, qo, table, seq_lens, mask, window_left, sm_scale,
                       output_scale, name)


def make_decode(seed, B, Hq, Hkv, D, seq_lens, page_size, mask="dense", window_left=-1,
                extra_pages=0, max_seq_len=None, bmm1_scale=None, bmm2_scale=1.0,
                name=""):
    rng = _rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q = randn_bf16(rng, (B, Hq, D))
    indptr, indices, P = csr_page_table(rng, seq_lens, page_size, extra_pages)
    k = randn_bf16(rng, (P, Hkv, page_size, D))
    v = randn_bf16(rng, (P, Hkv, page_size, D))
    return DecodeCase(q, k, v, indptr, indices, seq_lens,
                      int(max_seq_len or seq_lens.max()), mask, window_left,
                      bmm1_scale, bmm2_scale, name)


@dataclass
class DecodeQCase:
    """Multi-token (fixed SQ or packed) decode inputs with CSR page IDs."""
    q: torch.Tensor                 # [B, SQ, Hq, D] (fixed) or [total_q, Hq, D] (packed)
    k: torch.Tensor                 # [P, Hkv, ps, D]
    v: torch.Tensor
    kv_indptr: np.ndarray           # [B+1] int32
    kv_indices: np.ndarray          # int32
    seq_lens: np.ndarray            # [B] int32
    qo_indptr: np.ndarray | None    # [B+1] int32 (packed) or None (fixed SQ)
    seq_len_q: int                  # SQ (fixed) or max_seq_len_q (packed)
    max_seq_len: int
    mask: str
    window_left: int
    name: str = ""


def make_decode_q(seed, B, Hq, Hkv, D, seq_lens, page_size, seq_len_q=None, qlens=None,
                  mask="causal", window_left=-1, extra_pages=0, name=""):
    """Fixed SQ (qlens None) or packed per-request query lengths `qlens`."""
    rng = _rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if qlens is None:
        q = randn_bf16(rng, (B, seq_len_q, Hq, D))
        qo = None
        sq = int(seq_len_q)
    else:
        qlens = np.asarray(qlens, dtype=np.int32)
        qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        q = randn_bf16(rng, (int(qo[-1]), Hq, D))
        sq = int(seq_len_q or qlens.max())
    indptr, indices, P = csr_page_table(rng, seq_lens, page_size, extra_pages)
    k = randn_bf16(rng, (P, Hkv, page_size, D))
    v = randn_bf16(rng, (P, Hkv, page_size, D))
    return DecodeQCase(q, k, v, indptr, indices, seq_lens, qo, sq, int(seq_lens.max()), mask,
                       window_left, name)


def qsa_partition(seq_lens, block_size=4):
    """Packed partition: per token its sequence's first token and first global
    block; per global block its inclusive token span.  Blocks are numbered
    globally, restarting at each sequence boundary (a sequence of length L owns
    ceil(L/4) blocks, the last one possibly partial)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    T = int(seq_lens.sum())
    tok_base = np.zeros(T, dtype=np.int32)
    blk_base = np.zeros(T, dtype=np.int32)
    first, last = [], []
    t0 = nb0 = 0
    for L in seq_lens:
        L = int(L)
        tok_base[t0:t0 + L] = t0
        blk_base[t0:t0 + L] = nb0
        for m in range(-(-L // block_size)):
            first.append(t0 + block_size * m)
            last.append(min(t0 + block_size * m + block_size - 1, t0 + L - 1))
        nb0 += -(-L // block_size)
        t0 += L
    return tok_base, blk_base, np.asarray(first, np.int32), np.asarray(last, np.int32)


def make_qsa(seed, seq_lens, Hq=12, Hkv=1, D=256, p_sel=0.3, mode="causal", window=-1,
             force_diag=True, n_sel=None, empty_rows=0, junk_bits=0.0, name=""):
    """Token-granular selections over packed sequences.

    Each token selects blocks of its own sequence: with probability ``p_sel``
    each, or (``n_sel``) a random set of up to n_sel of the blocks its bounds
    reach; ``force_diag`` adds the block holding the token itself.  Bounds:
    causal lo = sequence start (or t - window), hi = t; dense lo/hi = the whole
    sequence.  ``empty_rows`` tokens get lo > hi; ``junk_bits`` sets random bits
    on blocks outside the token's bounds (they must not matter)."""
    rng = _rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    tok_base, blk_base, bfirst, blast = qsa_partition(seq_lens)
    T, NB = int(seq_lens.sum()), bfirst.size
    q = randn_bf16(rng, (T, Hq, D))
    k = randn_bf16(rng, (T, Hkv, D))
    v = randn_bf16(rng, (T, Hkv, D))
    lo = np.zeros(T, np.int32)
    hi = np.zeros(T, np.int32)
    sel = np.zeros((T, NB), np.uint8)
    for t in range(T):
        s0 = int(tok_base[t])
        send = s0 + int(seq_lens[np.searchsorted(np.cumsum(seq_lens), t, side="right")]) - 1
        if mode == "causal":
            lo[t] = s0 if window < 0 else max(s0, t - window)
            hi[t] = t
        else:
            lo[t], hi[t] = s0, send
        b0 = int(blk_base[t])
        nb_lo = b0 + (int(lo[t]) - s0) // 4
        nb_hi = b0 + (int(hi[t]) - s0) // 4
        cand = np.arange(nb_lo, nb_hi + 1)
        if n_sel is None:
            pick = cand[rng.random(cand.size) < p_sel]
        else:
            pick = rng.permutation(cand)[:n_sel]
        sel[t, pick] = 1
        if force_diag:
            sel[t, b0 + (t - s0) // 4] = 1
        if junk_bits > 0:
            other = np.ones(NB, bool)
            other[cand] = False
            sel[t, other & (rng.random(NB) < junk_bits)] = 1
    if empty_rows:
        for t in rng.choice(T, size=empty_rows, replace=False):
            lo[t], hi[t] = hi[t] + 1, hi[t]
    return QsaCase(q, k, v, sel, lo, hi, blk_base, tok_base, bfirst, blast,
                   seq_lens.astype(np.int32), 1.0 / math.sqrt(D), name)


# ----------------------------------------------------------------------------
# The five named workloads
# ----------------------------------------------------------------------------

def tiny_bsa(mask="dense", seed=1):
    """B=2, Sq=64, Hq=4, Hkv=1, D=128; L=[200,333]; 48-page pool of 16 tokens;
    q_block 16, kv_block 32; BSR p=0.5 plus the last in-range block; 5% zero
    validity bits; sm_scale = 1/sqrt(128)."""
    rng = _rng(seed)
    B, Sq, Hq, Hkv, D, ps = 2, 64, 4, 1, 128, 16
    seq_lens = np.array([200, 333], dtype=np.int32)
    q = randn_bf16(rng, (B, Sq, Hq, D))
    k = randn_bf16(rng, (48, Hkv, ps, D))
    v = randn_bf16(rng, (48, Hkv, ps, D))
    perm = rng.permutation(48).astype(np.int32)
    indptr = np.array([0, 13, 34], dtype=np.int32)
    indices = perm[:34].copy()
    bip, bid = bsr_bernoulli(rng, B, Hkv, Sq, 16, 32, seq_lens, p=0.5)
    bits = random_bits(rng, B, 333, 0.95)
    return BsaCase(q, k, v, indptr, indices, bip, bid, seq_lens, 16, 32, 333, bits,
                   mask, -1, INV_SQRT(128), f"tiny_bsa_{mask}")


def batch_decode(seed=2, B=64, Hq=32, Hkv=8, D=128, lo=512, hi=8192, page_size=16):
    """B=64 single-token decode, Hq=32/Hkv=8, D=128, L ~ U{512..8192}, 16-token
    pages with CSR IDs from a random permutation, dense mask."""
    rng = _rng(seed)
    seq_lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    q = randn_bf16(rng, (B, Hq, D))
    indptr, indices, P = csr_page_table(rng, seq_lens, page_size)
    k = randn_bf16(rng, (P, Hkv, page_size, D))
    v = randn_bf16(rng, (P, Hkv, page_size, D))
    return DecodeCase(q, k, v, indptr, indices, seq_lens, int(seq_lens.max()),
                      "dense", -1, None, 1.0, "batch_decode")


def batch_decode_q(seed=2, B=64, SQ=4, Hq=32, Hkv=8, D=128, lo=512, hi=8192, page_size=16):
    """Multi-token decode (speculative verification): the batch_decode recipe with
    SQ query tokens per request at the last SQ positions, causal mask."""
    rng = _rng(seed)
    seq_lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    q = randn_bf16(rng, (B, SQ, Hq, D))
    indptr, indices, P = csr_page_table(rng, seq_lens, page_size)
    k = randn_bf16(rng, (P, Hkv, page_size, D))
    v = randn_bf16(rng, (P, Hkv, page_size, D))
    return DecodeQCase(q, k, v, indptr, indices, seq_lens, None, SQ, int(seq_lens.max()),
                       "causal", -1, f"batch_decode_q{SQ}")


def batch_prefill(seed=3, D=128, window_left=-1, B=8, Hq=32, Hkv=8, page_size=32,
                  qlo=256, qhi=2048, plo=0, phi=2048):
    """B=8 packed causal prefill, qlen ~ U{256..2048}, KV = qlen + U{0..2048}
    prefix, Hq=32/Hkv=8, 32-token HND pages, row-strided block tables."""
    rng = _rng(seed)
    qlens = rng.integers(qlo, qhi + 1, size=B)
    prefixes = rng.integers(plo, phi + 1, size=B)
    seq_lens = (qlens + prefixes).astype(np.int32)
    qo = np.zeros(B + 1, dtype=np.int32)
    qo[1:] = np.cumsum(qlens)
    q = randn_bf16(rng, (int(qo[-1]), Hq, D))
    table, P = strided_block_table(rng, seq_lens, page_size)
    k = randn_bf16(rng, (P, Hkv, page_size, D))
    v = randn_bf16(rng, (P, Hkv, page_size, D))
    return PrefillCase(q, k, v, qo, table, seq_lens, "causal", window_left, None, 1.0,
                       f"batch_prefill_d{D}_w{window_left}")


def long_bsa(seed=4, B=4, S=8192, Hq=32, Hkv=8, D=128, blk=64, nsel=16, p_zero=0.01):
    """B=4, Sq=Skv=8192, Hq=32/Hkv=8, D=128, 64-token pages and blocks; each BSR
    row keeps block 0, the diagonal and 14 other causal-admissible blocks;
    causal mask; 1% zero validity bits."""
    rng = _rng(seed)
    seq_lens = np.full(B, S, dtype=np.int32)
    q = randn_bf16(rng, (B, S, Hq, D))
    npg = S // blk
    P = B * npg
    perm = rng.permutation(P).astype(np.int32)
    indptr = (np.arange(B + 1) * npg).astype(np.int32)
    k = randn_bf16(rng, (P, Hkv, blk, D))
    v = randn_bf16(rng, (P, Hkv, blk, D))
    bip, bid = bsr_causal_topk(rng, B, Hkv, S // blk, nsel)
    bits = random_bits(rng, B, S, 1.0 - p_zero)
    return BsaCase(q, k, v, indptr, perm, bip, bid, seq_lens, blk, blk, S, bits,
                   "causal", -1, None, f"long_bsa_s{S}")


# ----------------------------------------------------------------------------
# Sage-style quantized inputs
# ----------------------------------------------------------------------------

def quantize_int8_rows(x: torch.Tensor, rows_per_scale: int):
    """Symmetric int8 per group of ``rows_per_scale`` rows along dim -2.

    scale = amax/127 (1 when amax == 0); q = clamp(RNE(x/scale), -127, 127).
    Input construction only: the attention path consumes the quantized tensors.
    Returns (int8 [..., S, D], fp32 scales [..., ceil(S/rows)]).
    """
    *lead, S, D = x.shape
    G = -(-S // rows_per_scale)
    pad = G * rows_per_scale - S
    xf = x.float()
    if pad:
        xf = torch.cat([xf, xf.new_zeros(*lead, pad, D)], dim=-2)
    xg = xf.reshape(*lead, G, rows_per_scale, D)
    amax = xg.abs().amax(dim=(-1, -2))
    scale = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax))
    qv = torch.clamp(torch.round(xg / scale[..., None, None]), -127, 127).to(torch.int8)
    return qv.reshape(*lead, G * rows_per_scale, D)[..., :S, :].contiguous(), scale.contiguous()


def make_sage(seed, B, H, Sq, Sk, cap, nsel=None, per_row_counts=True, count_lo=None,
              uniform=False, block_sizes_rank=1, last_partial=True, name=""):
    """Prequantized Sage inputs: Q/K int8 (Q scale per 32 rows, K per 64 rows),
    V fp8 E4M3 in HDS layout with per-channel scales; random non-contiguous
    unsorted block selections of ``nsel`` (or per-row U{count_lo..cap}) blocks."""
    rng = _rng(seed)
    D = 128
    nqb = -(-Sq // 64)
    nkb = -(-Sk // 64)
    qf = randn_bf16(rng, (B, H, Sq, D))
    kf = randn_bf16(rng, (B, H, Sk, D))
    vf = randn_bf16(rng, (B, H, Sk, D))
    q8, qs = quantize_int8_rows(qf, 32)
    k8, ks = quantize_int8_rows(kf, 64)
    # q_scale storage is ceil(Sq/128)*4 entries (one per 32 rows, padded).
    qs_full = torch.ones(B, H, -(-Sq // 128) * 4, dtype=torch.float32)
    qs_full[..., :qs.shape[-1]] = qs
    vamax = vf.float().abs().amax(dim=2)                       # [B,H,D]
    vscale = torch.where(vamax > 0, vamax / 448.0, torch.ones_like(vamax))
    v8 = (vf.float() / vscale[:, :, None, :]).to(torch.float8_e4m3fn)  # [B,H,Sk,D]
    v_hds = torch.zeros(B, H, D, nkb * 64, dtype=torch.float8_e4m3fn)
    v_hds[..., :Sk] = v8.transpose(-1, -2)
    cap = int(cap)
    index = np.zeros((B, H, nqb, cap), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for r in range(nqb):
                index[b, h, r] = rng.permutation(nkb)[:cap] if cap <= nkb else \
                    rng.integers(0, nkb, size=cap)
    bsn = int(nsel if nsel is not None else cap)
    nums = None
    if per_row_counts:
        if count_lo is None:
            nums = np.full((B, H, nqb), bsn, dtype=np.int32)
        else:
            nums = rng.integers(count_lo, cap + 1, size=(B, H, nqb)).astype(np.int32)
    if block_sizes_rank == 0:
        bsz = None
    else:
        shape = {1: (nkb,), 2: (B, nkb), 3: (B, H, nkb)}[block_sizes_rank]
        bsz = np.full(shape, 64, dtype=np.int32)
        if last_partial:
            bsz[..., -1] = rng.integers(1, 64, size=bsz[..., -1].shape)
        if block_sizes_rank > 1:
            # a few interior blocks with fewer valid tokens as well
            m = rng.random(size=bsz.shape) < 0.1
            bsz = np.where(m, rng.integers(0, 65, size=bsz.shape), bsz).astype(np.int32)
    return SageCase(q8, k8, v_hds.contiguous(), qs_full.contiguous(), ks, vscale.contiguous(),
                    index, bsn, bsz, nums, uniform, None, Sk, name)


def qsa_long(seed=7, n_seq=4, seq_len=4096, n_sel=64):
    """Token-granular sparse attention at the page's geometry: 4 packed causal
    sequences of 4096 tokens, Hq=12 / Hkv=1, D=256, 4-token blocks; every token
    selects up to 64 random blocks of its causal range plus its own block."""
    return make_qsa(seed, [seq_len] * n_seq, Hq=12, Hkv=1, D=256, mode="causal",
                    n_sel=n_sel, name=f"qsa_{n_seq}x{seq_len}_sel{n_sel}")


def sage_long(seed=5):
    """B=2, H=16, Sq=Sk=16384, D=128, 64-token blocks, each Q block selects 25%
    (64 of 256) KV blocks at random (non-contiguous), per-row counts supplied,
    final KV block partial."""
    return make_sage(seed, 2, 16, 16384, 16384, cap=64, nsel=64, per_row_counts=True,
                     block_sizes_rank=1, last_partial=True, name="sage_s16384")


def sage_small(seed=15, block_sizes_rank=2):
    """Parity companion: Sq=Sk=1000 (partial storage), per-row counts
    U{0..cap} including zero rows, rank-2/3 block_sizes."""
    return make_sage(seed, 2, 3, 1000, 1000, cap=8, nsel=5, per_row_counts=True,
                     count_lo=0, block_sizes_rank=block_sizes_rank, last_partial=True,
                     name=f"sage_small_r{block_sizes_rank}")


# ----------------------------------------------------------------------------
# Poisoning helpers (unused memory holds NaN)
# ----------------------------------------------------------------------------

def poison_unused_pages(k: torch.Tensor, v: torch.Tensor, used_pages, seq_lens_pages):
    """Return copies of k/v where every page not in ``used_pages`` is NaN and
    every slot at or past the live length in a request's last page is NaN.

    ``seq_lens_pages``: list of (page_id, first_dead_slot) for each request's
    last page.
    """
    k = k.clone()
    v = v.clone()
    used = np.zeros(k.shape[0], dtype=bool)
    used[np.asarray(used_pages, dtype=np.int64)] = True
    dead = torch.from_numpy(~used)
    k[dead] = float("nan")
    v[dead] = float("nan")
    for pg, s0 in seq_lens_pages:
        if s0 < k.shape[2]:
            k[pg, :, s0:] = float("nan")
            v[pg, :, s0:] = float("nan")
    return k, v
