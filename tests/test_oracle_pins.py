"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: an independent loop-only implementation on tiny inputs;
* a library routine: torch's scaled_dot_product_attention in fp64 with an
  explicit boolean mask (GQA by repeat_interleave of the KV heads);
* hand-derived closed forms (tests/golden/closed_form_cases.json);
* invariants the pages fix: page-ID permutation, empty rows, window rules,
  all-blocks-selected == dense, constant V, LSE identities, split merging.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import attention as A
from oracle import bruteforce as BF
from oracle.fp8 import e4m3_decode, e4m3_value

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def f64(t):
    return t.to(torch.float64).numpy()


def cmp(a, b, tol=1e-10):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    if fin.any():
        assert np.max(np.abs(a[fin] - b[fin])) <= tol


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

BSA_TINY = [
    dict(B=2, Sq=6, Hq=4, Hkv=2, D=8, seq_lens=[21, 34], page_size=4, qbs=2, kvbs=8,
         mask="dense", bits_p=None),
    dict(B=2, Sq=6, Hq=4, Hkv=2, D=8, seq_lens=[21, 34], page_size=4, qbs=2, kvbs=8,
         mask="causal", bits_p=0.8),
    dict(B=1, Sq=5, Hq=2, Hkv=1, D=4, seq_lens=[30], page_size=8, qbs=3, kvbs=5,
         mask="causal", window_left=4, bits_p=0.7),
    dict(B=3, Sq=4, Hq=3, Hkv=3, D=4, seq_lens=[3, 17, 9], page_size=2, qbs=4, kvbs=4,
         mask="dense", bits_p=0.6, allow_empty=True),
    dict(B=2, Sq=7, Hq=6, Hkv=2, D=4, seq_lens=[0, 12], page_size=4, qbs=2, kvbs=3,
         mask="causal", bits_p=None, out_of_range=2, max_seq_len_kv=20),
]


@pytest.mark.parametrize("cfg", range(len(BSA_TINY)))
def test_bsa_oracle_matches_bruteforce(cfg):
    c = dict(BSA_TINY[cfg])
    w = c.pop("window_left", -1)
    case = W.make_bsa(100 + cfg, window_left=w, **c)
    args = (f64(case.q), f64(case.k), f64(case.v), case.kv_indptr, case.kv_indices,
            case.block_indptr, case.block_indices, case.q_block_size, case.kv_block_size,
            case.seq_lens)
    kw = dict(valid_bits=case.valid_bits, mask=case.mask, window_left=case.window_left,
              sm_scale=0.37)
    o, l = A.bsa_reference(*args, **kw)
    ob, lb = BF.bsa_bruteforce(*args, **kw)
    cmp(o, ob)
    cmp(l, lb)
    # the token-subset interface gives the same rows
    toks = [(b, i) for b in range(case.q.shape[0]) for i in range(case.q.shape[1])][::3]
    o2, l2 = A.bsa_reference(*args, tokens=toks, **kw)
    cmp(o2, np.stack([o[b, i] for b, i in toks]))
    cmp(l2, np.stack([l[b * case.q.shape[1] + i] for b, i in toks]))


@pytest.mark.parametrize("mask,w", [("causal", -1), ("causal", 3), ("dense", -1)])
def test_prefill_oracle_matches_bruteforce(mask, w):
    case = W.make_prefill(7, 3, [3, 5, 1], [4, 0, 9], 4, 2, 8, 4, mask=mask, window_left=w)
    args = (f64(case.q), f64(case.k), f64(case.v), case.qo_indptr, case.block_tables,
            case.seq_lens)
    o, l = A.prefill_reference(*args, mask=mask, window_left=w, sm_scale=0.5,
                               output_scale=1.5)
    ob, lb = BF.prefill_bruteforce(*args, mask=mask, window_left=w, sm_scale=0.5,
                                   output_scale=1.5)
    cmp(o, ob)
    cmp(l, lb)


@pytest.mark.parametrize("mask,w", [("dense", -1), ("causal", 5)])
def test_decode_oracle_matches_bruteforce(mask, w):
    case = W.make_decode(8, 3, 4, 2, 8, [1, 13, 30], 4, mask=mask, window_left=w)
    args = (f64(case.q), f64(case.k), f64(case.v), case.kv_indptr, case.kv_indices,
            case.seq_lens)
    o, l = A.decode_reference(*args, mask=mask, window_left=w, bmm1_scale=0.3,
                              bmm2_scale=0.5)
    ob, lb = BF.decode_bruteforce(*args, mask=mask, window_left=w, bmm1_scale=0.3,
                                  bmm2_scale=0.5)
    cmp(o, ob)
    cmp(l, lb)


# ---------------------------------------------------------------------------
# library routine: torch SDPA (fp64, explicit mask)
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, allowed, scale):
    """q [Hq, n, D], k/v [Hq, m, D] (already GQA-expanded), allowed [n, m]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(allowed), scale=scale).numpy()


def test_bsa_all_blocks_matches_torch_sdpa():
    """All blocks selected, no bitmap, causal: equals SDPA with the bottom-right
    causal mask over the gathered (de-paged) keys; GQA via repeat_interleave."""
    B, Sq, Hq, Hkv, D, ps, kvbs = 2, 24, 6, 2, 16, 8, 16
    case = W.make_bsa(11, B, Sq, Hq, Hkv, D, [40, 57], ps, 8, kvbs, mask="causal", p_sel=1.0)
    o, l = A.bsa_reference(f64(case.q), f64(case.k), f64(case.v), case.kv_indptr,
                           case.kv_indices, case.block_indptr, case.block_indices, 8, kvbs,
                           case.seq_lens, mask="causal")
    kf, vf, qf = f64(case.k), f64(case.v), f64(case.q)
    for b in range(B):
        L = int(case.seq_lens[b])
        j = np.arange(L)
        pages = case.kv_indices[case.kv_indptr[b] + j // ps]
        K = np.repeat(kf[pages, :, j % ps, :].transpose(1, 0, 2), Hq // Hkv, axis=0)
        V = np.repeat(vf[pages, :, j % ps, :].transpose(1, 0, 2), Hq // Hkv, axis=0)
        p = L - Sq + np.arange(Sq)
        allowed = j[None, :] <= p[:, None]
        ref = _sdpa(qf[b].transpose(1, 0, 2).copy(), K.copy(), V.copy(), allowed,
                    1 / math.sqrt(D))
        cmp(o[b].transpose(1, 0, 2), ref, 1e-12)


def test_prefill_window_matches_torch_sdpa():
    case = W.make_prefill(12, 2, [9, 14], [6, 2], 4, 2, 16, 16, mask="causal", window_left=5)
    o, _ = A.prefill_reference(f64(case.q), f64(case.k), f64(case.v), case.qo_indptr,
                               case.block_tables, case.seq_lens, mask="causal", window_left=5)
    kf, vf, qf = f64(case.k), f64(case.v), f64(case.q)
    for b in range(2):
        L = int(case.seq_lens[b]); qlen = int(case.qo_indptr[b + 1] - case.qo_indptr[b])
        j = np.arange(L)
        pages = case.block_tables[b, j // 16]
        K = np.repeat(kf[pages, :, j % 16, :].transpose(1, 0, 2), 2, axis=0)
        V = np.repeat(vf[pages, :, j % 16, :].transpose(1, 0, 2), 2, axis=0)
        p = L - qlen + np.arange(qlen)
        allowed = (j[None, :] <= p[:, None]) & (j[None, :] >= p[:, None] - 5)
        rows = slice(case.qo_indptr[b], case.qo_indptr[b + 1])
        ref = _sdpa(qf[rows].transpose(1, 0, 2).copy(), K.copy(), V.copy(), allowed, 0.25)
        cmp(o[rows].transpose(1, 0, 2), ref, 1e-12)


# ---------------------------------------------------------------------------
# hand-derived closed forms
# ---------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_two_keys():
    g = _golden()["two_keys"]
    o, l = A.attend(np.array([g["q"]]), np.array(g["k"]), np.array(g["v"]),
                    np.ones((1, 2), bool), g["sm_scale"])
    cmp(o[0], g["out"], 1e-12)
    assert abs(l[0] - g["lse"]) < 1e-12


def _pool_from_values(page_ids, ps, vals):
    """Build a [P,1,ps,D] pool whose logical token t holds vals[t]."""
    D = len(vals[0])
    P = max(page_ids) + 1
    pool = np.full((P, 1, ps, D), np.nan)
    for t, val in enumerate(vals):
        pool[page_ids[t // ps], 0, t % ps] = val
    return pool


def test_golden_bsa_causal_bits():
    g = _golden()["bsa_causal_bits"]
    L, ps = g["L"], g["page_size"]
    vals = [[t, 2 * t] for t in range(L)]
    v = _pool_from_values(g["page_ids"], ps, vals)
    k = np.where(np.isnan(v), np.nan, 0.3)          # any finite keys: q = 0
    q = np.zeros((1, 2, 1, 2))
    bits = np.array([[g["valid_word0"]]], dtype=np.uint32)
    o, l = A.bsa_reference(q, k, v, [0, len(g["page_ids"])], g["page_ids"],
                           np.array(g["block_indptr"]).reshape(1, 1, 3), g["block_indices"],
                           1, g["kv_block_size"], [L], valid_bits=bits, mask="causal")
    cmp(o[0, :, 0, :], g["out"], 1e-12)
    cmp(l[:, 0], g["lse"], 1e-12)
    ob, lb = BF.bsa_bruteforce(q, k, v, [0, 5], g["page_ids"],
                               np.array(g["block_indptr"]).reshape(1, 1, 3),
                               g["block_indices"], 1, g["kv_block_size"], [L],
                               valid_bits=bits, mask="causal", sm_scale=1.0)
    cmp(np.array(ob)[0, :, 0, :], g["out"], 1e-12)


def test_golden_prefill_bottom_right():
    g = _golden()["prefill_bottom_right"]
    vals = [[t, -t] for t in range(g["L"])]
    v = _pool_from_values(g["page_ids"], g["page_size"], vals)
    k = np.where(np.isnan(v), np.nan, -1.0)
    q = np.zeros((g["qlen"], 1, 2))
    o, l = A.prefill_reference(q, k, v, [0, g["qlen"]], np.array([g["page_ids"]]),
                               [g["L"]], mask="causal")
    cmp(o[:, 0, :], g["out"], 1e-12)
    cmp(l[:, 0], g["lse"], 1e-12)


def test_golden_decode_window():
    g = _golden()["decode_window"]
    vals = [[t, 1.0] for t in range(g["L"])]
    v = _pool_from_values(g["page_ids"], g["page_size"], vals)
    k = np.where(np.isnan(v), np.nan, 2.0)
    o, l = A.decode_reference(np.zeros((1, 1, 2)), k, v, [0, 3], g["page_ids"], [g["L"]],
                              mask="causal", window_left=g["window_left"])
    cmp(o[0, 0], g["out"], 1e-12)
    assert abs(l[0, 0] - g["lse"]) < 1e-12


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_page_permutation_invariance():
    case = W.make_bsa(21, 2, 16, 4, 2, 8, [45, 60], 8, 4, 16, mask="causal", bits_p=0.9,
                      extra_pages=5)
    base = A.bsa_reference(f64(case.q), f64(case.k), f64(case.v), case.kv_indptr,
                           case.kv_indices, case.block_indptr, case.block_indices, 4, 16,
                           case.seq_lens, valid_bits=case.valid_bits, mask="causal")
    rng = np.random.default_rng(0)
    P = case.k.shape[0]
    perm = rng.permutation(P)               # new physical slot of old page p
    k2 = np.empty_like(f64(case.k)); v2 = np.empty_like(f64(case.v))
    k2[perm] = f64(case.k); v2[perm] = f64(case.v)
    idx2 = perm[case.kv_indices]
    moved = A.bsa_reference(f64(case.q), k2, v2, case.kv_indptr, idx2, case.block_indptr,
                            case.block_indices, 4, 16, case.seq_lens,
                            valid_bits=case.valid_bits, mask="causal")
    cmp(moved[0], base[0], 0.0)
    cmp(moved[1], base[1], 0.0)


def test_all_blocks_equals_prefill_and_decode():
    """BSA with every block selected == packed prefill over the same pages, and a
    one-token BSA == decode."""
    B, Sq, Hq, Hkv, D, ps = 2, 8, 4, 2, 8, 8
    case = W.make_bsa(22, B, Sq, Hq, Hkv, D, [30, 19], ps, 8, 8, mask="causal", p_sel=1.0)
    o, l = A.bsa_reference(f64(case.q), f64(case.k), f64(case.v), case.kv_indptr,
                           case.kv_indices, case.block_indptr, case.block_indices, 8, 8,
                           case.seq_lens, mask="causal")
    table = np.full((B, 8), -1, dtype=np.int32)
    for b in range(B):
        n = case.kv_indptr[b + 1] - case.kv_indptr[b]
        table[b, :n] = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]]
    qo = np.array([0, Sq, 2 * Sq])
    op, lp = A.prefill_reference(f64(case.q).reshape(B * Sq, Hq, D), f64(case.k), f64(case.v),
                                 qo, table, case.seq_lens, mask="causal")
    cmp(o.reshape(B * Sq, Hq, D), op, 1e-13)
    cmp(l, lp, 1e-13)
    # last query token of each request == decode at p = L-1
    od, ld = A.decode_reference(f64(case.q)[:, -1], f64(case.k), f64(case.v), case.kv_indptr,
                                case.kv_indices, case.seq_lens, mask="causal")
    cmp(o[:, -1], od, 1e-13)


def test_empty_rows_exact_zero_and_neg_inf():
    case = W.make_bsa(23, 1, 4, 2, 1, 8, [20], 4, 2, 4, mask="dense")
    bip = np.array([[[0, 0, 0]]], dtype=np.int32)      # no blocks in either row
    o, l = A.bsa_reference(f64(case.q), f64(case.k), f64(case.v), case.kv_indptr,
                           case.kv_indices, bip, np.zeros(0, np.int32), 2, 4, case.seq_lens)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))
    # selected blocks but every token masked by the bitmap -> same
    case = W.make_bsa(24, 1, 4, 2, 1, 8, [20], 4, 2, 4, mask="dense", p_sel=1.0)
    bits = np.zeros((1, 1), dtype=np.uint32)
    o, l = A.bsa_reference(f64(case.q), f64(case.k), f64(case.v), case.kv_indptr,
                           case.kv_indices, case.block_indptr, case.block_indices, 2, 4,
                           case.seq_lens, valid_bits=bits)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


def test_window_zero_gives_current_value_and_wide_window_is_off():
    case = W.make_prefill(25, 2, [5, 3], [7, 0], 4, 2, 8, 4, mask="causal", window_left=0)
    args = (f64(case.q), f64(case.k), f64(case.v), case.qo_indptr, case.block_tables,
            case.seq_lens)
    o, l = A.prefill_reference(*args, mask="causal", window_left=0, output_scale=2.0)
    kf, vf = f64(case.k), f64(case.v)
    for b in range(2):
        L = int(case.seq_lens[b]); qlen = int(case.qo_indptr[b + 1] - case.qo_indptr[b])
        for i in range(qlen):
            p = L - qlen + i
            page = case.block_tables[b, p // 4]
            for h in range(4):
                assert np.array_equal(o[case.qo_indptr[b] + i, h], 2.0 * vf[page, h // 2, p % 4])
    o1, l1 = A.prefill_reference(*args, mask="causal", window_left=100)
    o2, l2 = A.prefill_reference(*args, mask="causal", window_left=-1)
    cmp(o1, o2, 0.0)
    cmp(l1, l2, 0.0)


def test_constant_v_gives_constant_output():
    case = W.make_bsa(26, 2, 8, 4, 2, 8, [33, 50], 8, 4, 8, mask="causal", bits_p=0.8)
    v = np.full(f64(case.v).shape, 0.625)
    o, l = A.bsa_reference(f64(case.q), f64(case.k), v, case.kv_indptr, case.kv_indices,
                           case.block_indptr, case.block_indices, 4, 8, case.seq_lens,
                           valid_bits=case.valid_bits, mask="causal")
    fin = np.isfinite(l)
    assert np.allclose(o.reshape(-1, 4, 8)[fin], 0.625, atol=1e-14, rtol=0)
    assert np.all(o.reshape(-1, 4, 8)[~fin] == 0.0)


def test_key_shift_moves_lse_only():
    """Adding one vector c to every key shifts row scores by scale*<q,c>: out is
    unchanged and LSE moves by exactly that amount."""
    case = W.make_decode(27, 2, 4, 2, 8, [19, 40], 4)
    c = np.linspace(-1, 1, 8)
    kf = f64(case.k)
    o1, l1 = A.decode_reference(f64(case.q), kf, f64(case.v), case.kv_indptr, case.kv_indices,
                                case.seq_lens)
    o2, l2 = A.decode_reference(f64(case.q), kf + c, f64(case.v), case.kv_indptr,
                                case.kv_indices, case.seq_lens)
    shift = (f64(case.q) @ c) / math.sqrt(8)
    cmp(o2, o1, 1e-12)
    cmp(l2, l1 + shift, 1e-12)


def test_lse_normalises_weights():
    case = W.make_decode(28, 2, 2, 1, 8, [23, 9], 4)
    qf, kf = f64(case.q), f64(case.k)
    _, lse = A.decode_reference(qf, kf, f64(case.v), case.kv_indptr, case.kv_indices,
                                case.seq_lens)
    for b in range(2):
        L = int(case.seq_lens[b]); j = np.arange(L)
        K = kf[case.kv_indices[case.kv_indptr[b] + j // 4], 0, j % 4, :]
        for h in range(2):
            s = (K @ qf[b, h]) / math.sqrt(8)
            assert abs(math.fsum(np.exp(s - lse[b, h])) - 1.0) < 1e-12


def test_split_merge_invariance():
    """Partials over any partition of [0, L) merged by LSE weights equal the
    unsplit result (the split-KV decode identity)."""
    case = W.make_decode(29, 1, 2, 1, 8, [37], 4)
    qf, kf, vf = f64(case.q), f64(case.k), f64(case.v)
    L = 37
    j = np.arange(L)
    pages = case.kv_indices[j // 4]
    K, V = kf[pages, 0, j % 4], vf[pages, 0, j % 4]
    full_o, full_l = A.attend(qf[0], K, V, np.ones((2, L), bool), 1 / math.sqrt(8))
    cuts = [0, 5, 6, 20, 37]
    parts = [A.attend(qf[0], K[a:b], V[a:b], np.ones((2, b - a), bool), 1 / math.sqrt(8))
             for a, b in zip(cuts[:-1], cuts[1:])]
    lses = np.stack([p[1] for p in parts])
    tot = np.logaddexp.reduce(lses, axis=0)
    merged = sum(np.exp(p[1] - tot)[:, None] * p[0] for p in parts)
    cmp(tot, full_l, 1e-12)
    cmp(merged, full_o, 1e-12)


def test_combined_cache_equals_tuple():
    case = W.make_decode(30, 2, 4, 2, 8, [17, 25], 8)
    comb = torch.stack([case.k, case.v], dim=1)        # [P, 2, Hkv, ps, D]
    o1, l1 = A.decode_reference(f64(case.q), f64(case.k), f64(case.v), case.kv_indptr,
                                case.kv_indices, case.seq_lens)
    o2, l2 = A.decode_reference(f64(case.q), f64(comb[:, 0]), f64(comb[:, 1]),
                                case.kv_indptr, case.kv_indices, case.seq_lens)
    cmp(o1, o2, 0.0)


# ---------------------------------------------------------------------------
# Sage pins
# ---------------------------------------------------------------------------

def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert e4m3_value(0x7E) == 448.0 and e4m3_value(0x01) == 2.0 ** -9


def test_sage_all_blocks_equals_dense_sdpa():
    case = W.make_sage(31, 1, 2, 150, 150, cap=3, nsel=3, per_row_counts=False,
                       block_sizes_rank=0)
    nkb = 3
    idx = np.tile(np.arange(nkb, dtype=np.int32)[::-1], (1, 2, 3, 1))
    out = A.sage_reference(case.q_int8, case.k_int8, case.v_fp8.view(torch.uint8).numpy(),
                           case.q_scale, case.k_scale, case.v_scale, idx, 3, Sk=150)
    Qd, Kd, Vd = A.sage_dequantize(case.q_int8, case.k_int8,
                                   case.v_fp8.view(torch.uint8).numpy(), case.q_scale,
                                   case.k_scale, case.v_scale, 150)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qd), torch.from_numpy(Kd), torch.from_numpy(Vd),
        scale=1 / math.sqrt(128)).numpy()
    cmp(out, ref, 1e-12)


@pytest.mark.parametrize("Sq,Sk", [(150, 150), (100, 180)])
def test_sage_causal_all_blocks_equals_masked_sdpa(Sq, Sk):
    """Causal Sage with every block selected is dense SDPA with the bottom-right
    causal mask on the dequantised tensors (torch fp64, explicit boolean mask),
    and its LSE normalises the softmax weights of the admitted keys."""
    case = W.make_sage(33, 1, 2, Sq, Sk, cap=3, nsel=3, per_row_counts=False,
                       block_sizes_rank=0)
    nkb = -(-Sk // 64)
    idx = np.tile(np.arange(nkb, dtype=np.int32), (1, 2, -(-Sq // 64), 1))
    codes = case.v_fp8.view(torch.uint8).numpy()
    out, lse = A.sage_reference(case.q_int8, case.k_int8, codes, case.q_scale, case.k_scale,
                                case.v_scale, idx, nkb, Sk=Sk, mask="causal", with_lse=True)
    Qd, Kd, Vd = A.sage_dequantize(case.q_int8, case.k_int8, codes, case.q_scale,
                                   case.k_scale, case.v_scale, Sk)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    m = torch.from_numpy(j <= Sk - Sq + i)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qd), torch.from_numpy(Kd), torch.from_numpy(Vd), attn_mask=m,
        scale=1 / math.sqrt(128)).numpy()
    cmp(out, ref, 1e-12)
    s = np.einsum("bhid,bhjd->bhij", Qd, Kd) / math.sqrt(128)
    w = np.where(m.numpy()[None, None], np.exp(s - lse[..., None]), 0.0)
    cmp(w.sum(-1), np.ones_like(lse), 1e-12)
    # the first query of a square problem sees key 0 only: out = V[0], LSE = s[0, 0]
    if Sq == Sk:
        cmp(out[:, :, 0], Vd[:, :, 0], 1e-12)
        cmp(lse[:, :, 0], s[:, :, 0, 0], 1e-12)


def test_sage_dense_lse_matches_logsumexp_of_selected_keys():
    """Dense Sage LSE of one query block equals scipy's logsumexp over exactly the
    selected keys (block order permuted, one partial block)."""
    from scipy.special import logsumexp
    case = W.sage_small(34, block_sizes_rank=1)
    codes = case.v_fp8.view(torch.uint8).numpy()
    out, lse = A.sage_reference(case.q_int8, case.k_int8, codes, case.q_scale, case.k_scale,
                                case.v_scale, case.q2k_block_index, case.block_sparse_num,
                                case.block_sizes, case.q2k_block_nums, False, None, Sk=case.Sk,
                                with_lse=True)
    Qd, Kd, _ = A.sage_dequantize(case.q_int8, case.k_int8, codes, case.q_scale, case.k_scale,
                                  case.v_scale, case.Sk)
    for b, h, r in [(0, 0, 0), (1, 2, 15), (0, 1, 7)]:
        n = int(case.q2k_block_nums[b, h, r])
        toks = [t for beta in case.q2k_block_index[b, h, r, :n]
                for t in range(beta * 64, beta * 64 + int(case.block_sizes[beta])) if t < case.Sk]
        for i in range(r * 64, min(r * 64 + 64, 1000), 13):
            if not toks:
                assert lse[b, h, i] == -np.inf
                continue
            sc = np.array([Qd[b, h, i] @ Kd[b, h, t] for t in toks]) / math.sqrt(128)
            cmp(lse[b, h, i], logsumexp(sc), 1e-12)


def test_sage_dequant_groups():
    """One q scale per 32 rows (ceil(Sq/128)*4 entries) and one k scale per 64
    rows: a constructed case with distinct per-group scales."""
    B, H, S = 1, 1, 130
    q8 = torch.ones(B, H, S, 128, dtype=torch.int8)
    k8 = torch.ones(B, H, S, 128, dtype=torch.int8)
    qs = torch.arange(1, 2 * 4 + 1, dtype=torch.float32).reshape(1, 1, 8)   # ceil(130/128)*4
    ks = torch.tensor([[[10.0, 20.0, 30.0]]])
    v = torch.zeros(B, H, 128, 192, dtype=torch.uint8)
    vs = torch.ones(1, 1, 128)
    Qd, Kd, _ = A.sage_dequantize(q8, k8, v.numpy(), qs, ks, vs, S)
    assert Qd[0, 0, 31, 0] == 1 and Qd[0, 0, 32, 0] == 2 and Qd[0, 0, 129, 0] == 5
    assert Kd[0, 0, 63, 0] == 10 and Kd[0, 0, 64, 0] == 20 and Kd[0, 0, 128, 0] == 30


def test_sage_zero_count_rows_and_partial_blocks():
    case = W.sage_small(32, block_sizes_rank=3)
    codes = case.v_fp8.view(torch.uint8).numpy()
    out = A.sage_reference(case.q_int8, case.k_int8, codes, case.q_scale, case.k_scale,
                           case.v_scale, case.q2k_block_index, case.block_sparse_num,
                           case.block_sizes, case.q2k_block_nums, False, None, Sk=case.Sk)
    nums = case.q2k_block_nums
    for b, h, r in zip(*np.nonzero(nums == 0)):
        assert np.all(out[b, h, r * 64:(r + 1) * 64] == 0.0)
    # brute force one row through the loop-only softmax
    Qd, Kd, Vd = A.sage_dequantize(case.q_int8, case.k_int8, codes, case.q_scale,
                                   case.k_scale, case.v_scale, case.Sk)
    b, h, r = 1, 2, 3
    n = int(nums[b, h, r])
    toks = []
    for beta in case.q2k_block_index[b, h, r, :n]:
        bs = int(case.block_sizes[b, h, beta])
        toks += [t for t in range(beta * 64, beta * 64 + bs) if t < case.Sk]
    i = r * 64 + 5
    ob, _ = BF._row_softmax(list(Qd[b, h, i]), [list(Kd[b, h, t]) for t in toks],
                            [list(Vd[b, h, t]) for t in toks], 1 / math.sqrt(128), 1.0)
    cmp(out[b, h, i], ob, 1e-12)


# ---------------------------------------------------------------- multi-token decode

def _csr_to_table(case):
    ps = case.k.shape[2]
    npg = [-(-int(L) // ps) for L in case.seq_lens]
    tab = np.full((len(npg), max(npg)), -1, dtype=np.int64)
    for b, n in enumerate(npg):
        tab[b, :n] = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b] + n]
    return tab


@pytest.mark.parametrize("mask,w", [("causal", -1), ("causal", 2), ("dense", -1)])
def test_decode_q_oracle_matches_bruteforce(mask, w):
    case = W.make_decode_q(21, 3, 4, 2, 8, [5, 12, 9], 4, qlens=[2, 4, 1], mask=mask,
                           window_left=w)
    args = (f64(case.q), f64(case.k), f64(case.v), case.kv_indptr, case.kv_indices,
            case.seq_lens, case.qo_indptr)
    o, l = A.decode_q_reference(*args, mask=mask, window_left=w, bmm1_scale=0.4,
                                bmm2_scale=1.5)
    ob, lb = BF.decode_q_bruteforce(*args, mask=mask, window_left=w, bmm1_scale=0.4,
                                    bmm2_scale=1.5)
    cmp(o, ob)
    cmp(l, lb)


@pytest.mark.parametrize("mask,w", [("dense", -1), ("causal", 7)])
def test_decode_q_single_token_is_decode(mask, w):
    """SQ = 1 reduces to single-token decode at position L - 1."""
    case = W.make_decode_q(22, 3, 8, 2, 16, [1, 17, 40], 8, seq_len_q=1, mask=mask,
                           window_left=w)
    args = (f64(case.q), f64(case.k), f64(case.v), case.kv_indptr, case.kv_indices,
            case.seq_lens)
    o, l = A.decode_q_reference(*args, mask=mask, window_left=w)
    od, ld = A.decode_reference(f64(case.q)[:, 0], *args[1:], mask=mask, window_left=w)
    cmp(o[:, 0], od)
    cmp(l[:, 0], ld)


def test_decode_q_matches_prefill_on_the_same_pages():
    """Packed multi-token decode over CSR pages = packed prefill over the same
    pages written as a block table (both bottom-right aligned)."""
    case = W.make_decode_q(23, 4, 6, 3, 16, [9, 33, 20, 5], 8, qlens=[3, 8, 1, 5],
                           mask="causal", window_left=4)
    o, l = A.decode_q_reference(f64(case.q), f64(case.k), f64(case.v), case.kv_indptr,
                                case.kv_indices, case.seq_lens, case.qo_indptr,
                                mask="causal", window_left=4)
    op, lp = A.prefill_reference(f64(case.q), f64(case.k), f64(case.v), case.qo_indptr,
                                 _csr_to_table(case), case.seq_lens, mask="causal",
                                 window_left=4)
    cmp(o, op)
    cmp(l, lp)


def test_decode_q_fixed_layout_is_packed_layout():
    """[B, SQ, Hq, D] is the packed layout with qo_indptr = b * SQ."""
    case = W.make_decode_q(24, 3, 4, 1, 8, [6, 10, 4], 4, seq_len_q=4, mask="causal")
    args = (f64(case.k), f64(case.v), case.kv_indptr, case.kv_indices, case.seq_lens)
    o, l = A.decode_q_reference(f64(case.q), *args)
    qo = np.arange(4) * 4
    op, lp = A.decode_q_reference(f64(case.q).reshape(12, 4, 8), *args, qo_indptr=qo)
    cmp(o.reshape(12, 4, 8), op)
    cmp(l.reshape(12, 4), lp)


# ----------------------------------------------------------------------------- QSA

@pytest.mark.parametrize("mode", ["causal", "dense"])
def test_qsa_matches_bruteforce(mode):
    case = W.make_qsa(50, [7, 10, 5], Hq=4, Hkv=2, D=16, p_sel=0.4, mode=mode, empty_rows=2,
                      junk_bits=0.2)
    out, lse = A.qsa_reference(case.q, case.k, case.v, case.sel_blocks, case.lo, case.hi,
                               case.block_first, case.block_last, case.scale)
    bo, bl = BF.qsa_bruteforce(case.q, case.k, case.v, case.sel_blocks, case.lo, case.hi,
                               case.block_first, case.block_last, case.scale)
    cmp(out, np.array(bo), 1e-12)
    cmp(lse, np.array(bl), 1e-12)
    empty = case.lo > case.hi
    assert empty.sum() == 2
    assert np.all(out[empty] == 0.0) and np.all(lse[:, empty] == -np.inf)


def test_qsa_all_blocks_causal_equals_per_sequence_sdpa():
    """Every block selected with lo = sequence start, hi = t is causal attention
    inside each packed sequence (torch fp64 SDPA, GQA by repeat_interleave)."""
    lens = [37, 64, 9]
    case = W.make_qsa(51, lens, Hq=6, Hkv=2, D=32, p_sel=1.0, mode="causal")
    out, lse = A.qsa_reference(case.q, case.k, case.v, case.sel_blocks, case.lo, case.hi,
                               case.block_first, case.block_last, case.scale)
    t0 = 0
    for L in lens:
        qs = case.q[t0:t0 + L].to(torch.float64).transpose(0, 1)
        ks = case.k[t0:t0 + L].to(torch.float64).transpose(0, 1).repeat_interleave(3, 0)
        vs = case.v[t0:t0 + L].to(torch.float64).transpose(0, 1).repeat_interleave(3, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=True,
                                                               scale=case.scale)
        cmp(out[t0:t0 + L], ref.transpose(0, 1).numpy(), 1e-12)
        s = (qs @ ks.transpose(1, 2)) * case.scale
        s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), -math.inf)
        cmp(lse[:, t0:t0 + L], torch.logsumexp(s, -1).numpy(), 1e-12)
        t0 += L


def test_qsa_single_key_rows_and_out_of_bound_bits():
    """Selecting only the token's own block with lo = hi = t leaves one key: out =
    v[t], LSE = scale*<q, k_t>.  Bits set on blocks outside [lo, hi] change
    nothing."""
    case = W.make_qsa(52, [13, 6], Hq=2, Hkv=1, D=16, p_sel=0.0, mode="causal")
    lo = np.arange(19, dtype=np.int32)
    out, lse = A.qsa_reference(case.q, case.k, case.v, case.sel_blocks, lo, lo,
                               case.block_first, case.block_last, case.scale)
    qf, kf, vf = (x.to(torch.float64).numpy() for x in (case.q, case.k, case.v))
    cmp(out, np.repeat(vf, 2, axis=1), 1e-12)
    cmp(lse, (np.einsum("thd,td->ht", qf, kf[:, 0]) * case.scale), 1e-12)
    junk = case.sel_blocks.copy()
    junk[:, :] = 1
    out2, lse2 = A.qsa_reference(case.q, case.k, case.v, junk, lo, lo, case.block_first,
                                 case.block_last, case.scale)
    cmp(out2, out, 0.0)
    cmp(lse2, lse, 0.0)


def test_qsa_partition_spans():
    """Block numbering restarts per sequence: a sequence of length L owns
    ceil(L/4) consecutive global blocks of 4 tokens, the last one partial."""
    from gen.workloads import qsa_partition
    tb, bb, bf, bl = qsa_partition([7, 4, 1])
    assert tb.tolist() == [0] * 7 + [7] * 4 + [11]
    assert bb.tolist() == [0] * 7 + [2] * 4 + [3]
    assert bf.tolist() == [0, 4, 7, 11] and bl.tolist() == [3, 6, 10, 11]


# ---------------------------------------------------------------------------
# row-subset selectors (the full-size GPU tests compare sampled rows through
# them): each equals the matching slice of the full result
# ---------------------------------------------------------------------------

def test_prefill_rows_selector_is_slice_of_full():
    case = W.make_prefill(31, 3, [37, 5, 70], [10, 0, 33], 4, 2, 16, 16, mask="causal",
                          window_left=20)
    args = (case.q, case.k, case.v, case.qo_indptr, case.block_tables, case.seq_lens)
    o, l = A.prefill_reference(*args, mask="causal", window_left=20)
    rows = [111, 0, 36, 37, 41, 42, 75, 3]        # unsorted, request boundaries
    os_, ls_ = A.prefill_reference(*args, mask="causal", window_left=20, rows=rows)
    cmp(os_, o[rows], 1e-12)
    cmp(ls_, l[rows], 1e-12)
    # rows past a chunk boundary of the selector's batching
    o2, l2 = A.prefill_reference(*args, mask="causal", window_left=20, rows=list(range(112)),
                                 chunk=7)
    cmp(o2, o, 1e-12)
    cmp(l2, l, 1e-12)


def test_decode_requests_selector_is_slice_of_full():
    case = W.make_decode(32, 5, 8, 2, 16, [40, 1, 77, 16, 5], 8, mask="causal", window_left=9)
    args = (case.q, case.k, case.v, case.kv_indptr, case.kv_indices, case.seq_lens)
    o, l = A.decode_reference(*args, mask="causal", window_left=9, bmm2_scale=0.7)
    reqs = [4, 0, 2, 2]
    os_, ls_ = A.decode_reference(*args, mask="causal", window_left=9, bmm2_scale=0.7,
                                  requests=reqs)
    cmp(os_, o[reqs], 1e-12)
    cmp(ls_, l[reqs], 1e-12)


def test_sage_rows_selector_is_slice_of_full():
    case = W.make_sage(33, 2, 2, 200, 300, 4, count_lo=0, block_sizes_rank=3)
    codes = case.v_fp8.view(torch.uint8).numpy()
    args = (case.q_int8, case.k_int8, codes, case.q_scale, case.k_scale, case.v_scale,
            case.q2k_block_index, case.block_sparse_num, case.block_sizes, case.q2k_block_nums)
    for mask in ("dense", "causal"):
        o, l = A.sage_reference(*args, Sk=case.Sk, mask=mask, with_lse=True)
        rows = [(1, 0, 3), (0, 1, 0), (1, 1, 2)]
        os_, ls_ = A.sage_reference(*args, Sk=case.Sk, mask=mask, with_lse=True, rows=rows)
        for b, h, r in rows:
            sl = slice(64 * r, min(64 * r + 64, 200))
            cmp(os_[b, h, sl], o[b, h, sl], 1e-12)
            cmp(ls_[b, h, sl], l[b, h, sl], 1e-12)
        # everything outside the selected rows is left unset
        keep = np.zeros((2, 2, 200), bool)
        for b, h, r in rows:
            keep[b, h, 64 * r:64 * r + 64] = True
        assert np.isnan(os_[~keep]).all() and np.isnan(ls_[~keep]).all()


def test_qsa_tokens_selector_is_slice_of_full():
    case = W.make_qsa(34, [9, 14, 7], Hq=4, Hkv=2, D=16, p_sel=0.4, empty_rows=2)
    args = (case.q, case.k, case.v, case.sel_blocks, case.lo, case.hi, case.block_first,
            case.block_last, case.scale)
    o, l = A.qsa_reference(*args)
    toks = [29, 0, 13, 9, 8]
    os_, ls_ = A.qsa_reference(*args, tokens=toks)
    cmp(os_[toks], o[toks], 1e-12)
    cmp(ls_[:, toks], l[:, toks], 1e-12)
    rest = np.setdiff1d(np.arange(30), toks)
    assert np.isnan(os_[rest]).all() and np.isnan(ls_[:, rest]).all()


def test_sage_uniform_count_ignores_per_row_counts():
    """Sage page (Parameters): with uniform_block_count set every row uses
    block_sparse_num and the per-row counts are ignored -- the same result as
    passing no counts at all, and different from honouring the counts."""
    case = W.make_sage(35, 1, 2, 130, 400, 5, nsel=3, count_lo=0, block_sizes_rank=1)
    codes = case.v_fp8.view(torch.uint8).numpy()
    base = (case.q_int8, case.k_int8, codes, case.q_scale, case.k_scale, case.v_scale,
            case.q2k_block_index, 3, case.block_sizes)
    assert (case.q2k_block_nums != 3).any()
    o_uni = A.sage_reference(*base, case.q2k_block_nums, uniform_block_count=True, Sk=case.Sk)
    o_none = A.sage_reference(*base, None, Sk=case.Sk)
    o_rows = A.sage_reference(*base, case.q2k_block_nums, uniform_block_count=False, Sk=case.Sk)
    cmp(o_uni, o_none, 0.0)
    differ = [(0, h, r) for h in range(2) for r in range(3) if case.q2k_block_nums[0, h, r] != 3]
    assert any(not np.allclose(o_uni[0, h, 64 * r:64 * r + 64], o_rows[0, h, 64 * r:64 * r + 64])
               for _, h, r in differ)
