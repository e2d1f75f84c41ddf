"""CPU tests of the C ABI: exports, static checks, plans and host validation.

No kernel runs here.  Plan fields, validation status + first bad index, the
prefill work list and the decode split policy must match the Python statement
of the same rules (oracle/metadata.py) bit for bit.
"""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import paged_kv_block_amd as P
from paged_kv_block_amd import _lib as C
from gen import workloads as W
from oracle import metadata as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions(header="pkb.h"):
    txt = open(os.path.join(ROOT, "include", header)).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(C.EXPORTS)
    L = P.lib()
    for n in names:
        assert hasattr(L, n)


def test_peaks_library_exports_its_header():
    """libpkb_peaks.so (the on-device ceilings the benchmark measures) exports
    every function include/pkb_peaks.h declares."""
    names = header_functions("pkb_peaks.h")
    assert names == ["pkb_peak_coexec", "pkb_peak_hbm_gather", "pkb_peak_hbm_read",
                     "pkb_peak_issue", "pkb_peak_l2_gather", "pkb_peak_mfma"]
    lib = os.path.join(ROOT, "paged_kv_block_amd", "libpkb_peaks.so")
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    assert set(names) <= exported


def test_status_strings_and_version():
    L = P.lib()
    assert L.pkb_abi_version() == 3
    for st in range(0, -8, -1):
        assert L.pkb_status_string(st).decode() not in ("", "unknown status")
    assert M.MAX_SEQ_LEN == 2147483520 == C.PKB_MAX_SEQ_LEN   # 2^31 - 128


def _c_bsa_plan(args):
    a = C.BsaStaticArgs(*[args[k] for k in (
        "B", "Sq", "Hq", "Hkv", "D", "num_pages", "page_size", "q_block_size", "kv_block_size",
        "max_seq_len_kv", "mask_type", "window_left", "qkv_dtype", "out_dtype", "num_cus")])
    plan = C.BsaPlan()
    st = P.lib().bsa_plan(ctypes.byref(a), ctypes.byref(plan))
    return st, plan


def _rand_static(rng):
    """Mostly valid static arguments, each field occasionally out of contract."""
    def pick(good, bad):
        return int(rng.choice(bad)) if rng.random() < 0.06 else int(rng.choice(good))
    Hkv = pick([1, 2, 8], [3])
    return dict(B=pick([1, 2, 4], [0]), Sq=pick([1, 17, 64, 300], [0]),
                Hq=Hkv * pick([1, 2, 4, 8], [1]) if rng.random() > 0.05 else 3,
                Hkv=Hkv, D=pick([128, 256], [64]), num_pages=pick([1, 99], [0]),
                page_size=pick([8, 16, 64, 128], [4, 24, 0]),
                q_block_size=pick([8, 16, 64, 65, 128], [0, 1, 3]),
                kv_block_size=pick([8, 16, 32, 64, 128, 192], [0, 24, 48, 96]),
                max_seq_len_kv=pick([1, 500, M.MAX_SEQ_LEN], [0, M.MAX_SEQ_LEN + 1]),
                mask_type=pick([0, 1], [2]), window_left=pick([-1, -1, 0, 7], [-2]),
                qkv_dtype=pick([0], [1]), out_dtype=pick([0, 1], [2]),
                num_cus=pick([80, 256], [0]))


def test_bsa_plan_matches_spec():
    rng = np.random.default_rng(0)
    n_ok = 0
    for _ in range(3000):
        a = _rand_static(rng)
        st_py, plan_py = M.bsa_plan(**a)
        st_c, plan_c = _c_bsa_plan(a)
        assert st_c == st_py, (a, st_c, st_py)
        if st_c == 0:
            n_ok += 1
            for k, v in plan_py.items():
                assert getattr(plan_c, k) == v, (k, a)
    assert n_ok > 500


def _bsa_args_from_case(case, num_cus=256):
    B, Sq, Hq, Hkv, D, Pn, ps = case.dims
    return dict(B=B, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, num_pages=Pn, page_size=ps,
                q_block_size=case.q_block_size, kv_block_size=case.kv_block_size,
                max_seq_len_kv=case.max_seq_len_kv, mask_type=1 if case.mask == "causal" else 0,
                window_left=case.window_left, qkv_dtype=0, out_dtype=0, num_cus=num_cus)


def _c_bsa_validate(plan, ip, ix, bip, bix, sl):
    bad = C.Bad()
    ip, ix, bip, bix, sl = (np.ascontiguousarray(x, dtype=np.int32) for x in (ip, ix, bip, bix, sl))
    st = P.lib().bsa_validate(ctypes.byref(plan), ip.ctypes.data, ix.ctypes.data, ix.size,
                              bip.ctypes.data, bix.ctypes.data, bix.size, sl.ctypes.data,
                              ctypes.byref(bad))
    return (st, bad.field, bad.index) if st == M.PKB_ERR_METADATA else (st, 0, -1)


def _mutations(rng, case):
    """Yield (ip, ix, bip, bix, sl) with one random corruption each."""
    base = [case.kv_indptr.copy(), case.kv_indices.copy(), case.block_indptr.copy(),
            case.block_indices.copy(), case.seq_lens.copy()]
    yield [x.copy() for x in base]
    for _ in range(60):
        ip, ix, bip, bix, sl = [x.copy() for x in base]
        kind = rng.integers(0, 9)
        if kind == 0 and ix.size:
            ix[rng.integers(0, ix.size)] = rng.choice([-1, case.k.shape[0], 10 ** 6])
        elif kind == 1:
            ip[rng.integers(0, ip.size)] += int(rng.choice([-3, -1, 1, 5]))
        elif kind == 2:
            sl[rng.integers(0, sl.size)] = rng.choice([-1, case.max_seq_len_kv + 1,
                                                       case.max_seq_len_kv])
        elif kind == 3 and bix.size:
            bix[rng.integers(0, bix.size)] = rng.choice([-1, 10 ** 5])
        elif kind == 4 and bix.size > 1:
            i = rng.integers(1, bix.size)
            bix[i] = bix[i - 1]                       # duplicate within a row (often)
        elif kind == 5:
            f = bip.reshape(-1)
            f[rng.integers(0, f.size)] += int(rng.choice([-2, 1, 3]))
        elif kind == 6:
            sl[rng.integers(0, sl.size)] += 40         # may need more pages than owned
        elif kind == 7:
            f = bip.reshape(-1)
            f[-1] = bix.size + 1
        else:
            ip[0] = 1
        yield ip, ix, bip, bix, sl


@pytest.mark.parametrize("seed", range(6))
def test_bsa_validate_matches_spec(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    case = W.make_bsa(200 + seed, B, int(rng.integers(4, 40)), 4, 2, 128,
                      [int(x) for x in rng.integers(1, 90, size=B)], 8, 4,
                      int(rng.choice([8, 16, 64])), mask="causal", p_sel=0.6,
                      max_seq_len_kv=120)
    a = _bsa_args_from_case(case)
    st, plan = _c_bsa_plan(a)
    assert st == 0
    spec_args = dict(a, num_q_blocks=plan.num_q_blocks, num_kv_blocks=plan.num_kv_blocks)
    n_bad = 0
    for ip, ix, bip, bix, sl in _mutations(rng, case):
        want = M.bsa_validate(spec_args, ip, ix, bip, bix, sl)
        got = _c_bsa_validate(plan, ip, ix, bip, bix, sl)
        assert got == want, (got, want)
        n_bad += want[0] != 0
    assert n_bad > 20


def test_bsa_validate_accepts_generated_workloads():
    for case in (W.tiny_bsa("dense"), W.tiny_bsa("causal")):
        a = _bsa_args_from_case(case)
        st, plan = _c_bsa_plan(a)
        assert st == 0
        got = _c_bsa_validate(plan, case.kv_indptr, case.kv_indices, case.block_indptr,
                              case.block_indices, case.seq_lens)
        assert got == (0, 0, -1)


def test_window_requires_causal_and_static_rules():
    base = dict(B=1, Sq=16, Hq=4, Hkv=1, D=128, num_pages=4, page_size=16, q_block_size=16,
                kv_block_size=32, max_seq_len_kv=64, mask_type=0, window_left=-1, qkv_dtype=0,
                out_dtype=0, num_cus=256)
    assert _c_bsa_plan(base)[0] == 0
    assert _c_bsa_plan(dict(base, window_left=3))[0] == M.PKB_ERR_ARG     # needs causal
    assert _c_bsa_plan(dict(base, window_left=3, mask_type=1))[0] == 0
    assert _c_bsa_plan(dict(base, kv_block_size=48))[0] == M.PKB_ERR_ARG
    assert _c_bsa_plan(dict(base, kv_block_size=192))[0] == 0
    assert _c_bsa_plan(dict(base, q_block_size=1, Hq=4, Hkv=2))[0] == M.PKB_ERR_ARG  # 1*2 % 8
    assert _c_bsa_plan(dict(base, q_block_size=4, Hq=4, Hkv=2))[0] == 0              # 4*2 % 8
    assert _c_bsa_plan(dict(base, max_seq_len_kv=M.MAX_SEQ_LEN))[0] == 0
    assert _c_bsa_plan(dict(base, max_seq_len_kv=M.MAX_SEQ_LEN + 1))[0] == M.PKB_ERR_ARG
    assert _c_bsa_plan(dict(base, D=64))[0] == M.PKB_ERR_UNSUPPORTED
    assert _c_bsa_plan(dict(base, Hq=3, Hkv=2))[0] == M.PKB_ERR_SHAPE


def test_small_page_quotient_rule():
    """The attention kernel finds a row's page inside a chunk from the slot x
    of the chunk's first token plus the row (x < page_size + 7): for page sizes
    below 8 as (x * ceil(2^32 / page_size)) >> 32, else as x >= page_size.
    Both equal x // page_size over every operand they receive."""
    for ps in range(1, 8):
        magic = ((1 << 32) + ps - 1) // ps
        assert all((x * magic) >> 32 == x // ps for x in range(ps + 7))
    for ps in list(range(8, 600)) + [4095, 65536, 1 << 20]:
        assert all(int(x >= ps) == x // ps for x in range(ps + 7))


def test_nonzero_byte_rule():
    """The packed-query kernel marks the nonzero bytes of a 32-bit word as
    bit 7 of (((x & 0x7F7F7F7F) + 0x7F7F7F7F) | x) & 0x80808080 and gathers
    them with one multiply; over every zero / nonzero byte pattern (nonzero
    bytes drawn from 1..255, 0x7F, 0x80 and 0xFF) that equals byte != 0."""
    rng = np.random.default_rng(3)

    def rule(x):
        t = (((x & 0x7F7F7F7F) + 0x7F7F7F7F) | x) & 0x80808080
        return ((((t >> 7) * 0x00204081) & 0xFFFFFFFF) >> 21) & 0xF

    for pattern in range(16):
        for _ in range(200):
            bs = [int(rng.choice([1, 0x7F, 0x80, 0xFF, rng.integers(1, 256)])) if pattern >> i & 1 else 0
                  for i in range(4)]
            x = bs[0] | bs[1] << 8 | bs[2] << 16 | bs[3] << 24
            assert rule(x) == pattern, (hex(x), pattern)


def test_any_page_size_for_block_sparse_and_decode():
    """The block-sparse and decode pages constrain block sizes only, so every
    page size >= 1 plans (prefill keeps its page's four sizes)."""
    base = dict(B=1, Sq=16, Hq=4, Hkv=1, D=128, num_pages=4, page_size=16, q_block_size=16,
                kv_block_size=32, max_seq_len_kv=64, mask_type=0, window_left=-1, qkv_dtype=0,
                out_dtype=0, num_cus=256)
    for ps in (1, 2, 3, 5, 7, 12, 17, 20, 24, 100):
        assert _c_bsa_plan(dict(base, page_size=ps))[0] == 0, ps
        assert P.paged_decode_workspace_size(4, 32, 8, 128, 1000, ps, 256)[1] >= 1
        assert P.paged_decode_q_workspace_size(4, 3, 32, 8, 128, 1000, ps, 256)[1] >= 1
    assert _c_bsa_plan(dict(base, page_size=0))[0] == M.PKB_ERR_ARG
    with pytest.raises(P.PkbError):
        P.paged_decode_workspace_size(4, 32, 8, 128, 1000, 0, 256)
    for ps in (8, 24, 48):
        st = C.lib().paged_prefill_validate(
            ctypes.byref(C.PrefillStaticArgs(1, 4, 1, 128, 4, ps, 16, 4, 1, -1, 0, 0, 256)),
            None, None, None, 0, ctypes.byref(C.Bad()))
        assert st == M.PKB_ERR_UNSUPPORTED, ps


# ----------------------------------------------------------------------------- prefill

def _prefill_args(B, total_q, width, mask_type=1, window_left=-1, page_size=32, D=128, Hq=32,
                  Hkv=8, num_pages=1000):
    return dict(B=B, Hq=Hq, Hkv=Hkv, D=D, num_pages=num_pages, page_size=page_size,
                total_q=total_q, width=width, mask_type=mask_type, window_left=window_left,
                qkv_dtype=0, out_dtype=0, num_cus=256)


def _c_prefill(args, qo, sl):
    a = C.PrefillStaticArgs(args["B"], args["Hq"], args["Hkv"], args["D"], args["num_pages"],
                            args["page_size"], args["total_q"], args["width"], args["mask_type"],
                            args["window_left"], args["qkv_dtype"], args["out_dtype"],
                            args["num_cus"])
    return P.paged_prefill_plan(a, qo, sl)


@pytest.mark.parametrize("mask,w", [(1, -1), (1, 1024), (0, -1), (1, 0)])
def test_prefill_worklist_matches_spec(mask, w):
    for D in (128, 256):
        case = W.batch_prefill(3, D=D, window_left=w)
        args = _prefill_args(8, int(case.qo_indptr[-1]), case.block_tables.shape[1], mask, w, D=D,
                             num_pages=case.k.shape[0])
        st, plan_py, wl_py = M.prefill_plan(args, case.qo_indptr, case.seq_lens)
        assert st == 0
        plan_c, wl_c = _c_prefill(args, case.qo_indptr, case.seq_lens)
        assert np.array_equal(wl_c, wl_py)
        for k, v in plan_py.items():
            assert getattr(plan_c, k) == v, k


@pytest.mark.parametrize("D,mq", [(128, 1), (128, 300), (256, 2048), (128, 65)])
def test_prefill_capacity_plan_matches_spec(D, mq):
    args = _prefill_args(5, 4000, 64, 1, -1, D=D, num_pages=100)
    st, plan_py, wl_py = M.prefill_plan_capacity(args, mq)
    assert st == 0
    a = C.PrefillStaticArgs(*[args[k] for k in ("B", "Hq", "Hkv", "D", "num_pages", "page_size",
                                                "total_q", "width", "mask_type", "window_left",
                                                "qkv_dtype", "out_dtype", "num_cus")])
    plan_c, wl_c = P.paged_prefill_plan_capacity(a, mq)
    assert np.array_equal(wl_c, wl_py)
    for k, v in plan_py.items():
        assert getattr(plan_c, k) == v, k
    # every (request, tile) that any qlen <= mq can need appears exactly once
    G, tm = plan_py["group"], plan_py["tile_m"]
    need = {(b, r) for b in range(5) for r in range(0, mq * G, tm)}
    assert sorted(map(tuple, wl_py.tolist())) == sorted(need)
    for bad_q in (0, 4001):
        assert M.prefill_plan_capacity(args, bad_q)[0] == M.PKB_ERR_ARG
        with pytest.raises(P.PkbError):
            P.paged_prefill_plan_capacity(a, bad_q)


def _c_prefill_validate(args, qo, sl, bt):
    a = C.PrefillStaticArgs(args["B"], args["Hq"], args["Hkv"], args["D"], args["num_pages"],
                            args["page_size"], args["total_q"], args["width"], args["mask_type"],
                            args["window_left"], args["qkv_dtype"], args["out_dtype"],
                            args["num_cus"])
    st, f, i = P.paged_prefill_validate(a, qo, sl, bt, raise_on_error=False)
    return (st, f, i) if st == M.PKB_ERR_METADATA else (st, 0, -1)


def test_prefill_validate_matches_spec():
    rng = np.random.default_rng(5)
    case = W.make_prefill(9, 3, [5, 17, 9], [3, 0, 40], 8, 2, 128, 16)
    args = _prefill_args(3, int(case.qo_indptr[-1]), case.block_tables.shape[1], Hq=8, Hkv=2,
                         page_size=16, num_pages=case.k.shape[0])
    args_spec = dict(args, block_table_width=args["width"])
    n_bad = 0
    for t in range(150):
        qo, sl, bt = case.qo_indptr.copy(), case.seq_lens.copy(), case.block_tables.copy()
        k = t % 6
        if t == 0:
            pass
        elif k == 0:
            qo[rng.integers(0, qo.size)] += int(rng.choice([-2, 1]))
        elif k == 1:
            sl[rng.integers(0, sl.size)] = int(rng.choice([-1, 0, 2, 80]))
        elif k == 2:
            bt[rng.integers(0, bt.shape[0]), rng.integers(0, bt.shape[1])] = int(rng.choice([-1, 10 ** 4]))
        elif k == 3:
            sl[rng.integers(0, sl.size)] += 16 * bt.shape[1]
        elif k == 4:
            qo[-1] += 1
        else:
            bt[:, 0] = -5
        want = M.prefill_validate(args_spec, qo, sl, bt, bt.shape[1])
        got = _c_prefill_validate(args, qo, sl, bt)
        assert got == want, (t, got, want)
        n_bad += want[0] != 0
    assert n_bad > 60


# ----------------------------------------------------------------------------- decode

def test_decode_policy_matches_spec():
    rng = np.random.default_rng(1)
    for _ in range(2000):
        B = int(rng.integers(1, 300)); Hkv = int(rng.choice([1, 2, 8])); Hq = Hkv * int(rng.choice([1, 4, 8]))
        D = int(rng.choice([128, 256, 64])); msl = int(rng.choice([1, 63, 64, 65, 4096, 8192, 131072, M.MAX_SEQ_LEN]))
        ps = int(rng.choice([8, 16, 12])); cus = int(rng.choice([80, 256]))
        st, nbytes, S, sl = M.decode_policy(B, Hq, Hkv, D, msl, ps, cus)
        if st != 0:
            nb = ctypes.c_size_t(); s = ctypes.c_int32(); l = ctypes.c_int32()
            assert P.lib().paged_decode_workspace_size(B, Hq, Hkv, D, msl, ps, cus, ctypes.byref(nb),
                                                       ctypes.byref(s), ctypes.byref(l)) == st
            continue
        if S > 65535:
            continue
        got = P.paged_decode_workspace_size(B, Hq, Hkv, D, msl, ps, cus)
        assert got == (nbytes, S, sl)
        assert S * sl >= msl and (sl % 64 == 0 or (S == 1 and sl == msl and nbytes == 0))


def test_decode_policy_single_pass_cases():
    """Wide batches run in one pass (no workspace); the batch-decode workload
    (B=64, Hq=32, Hkv=8 on 256 CUs) is one, and so is its 4-token variant.
    Narrow batches, more than 256 requests or more than 16 query rows per KV
    head keep the chunked policy."""
    assert M.decode_policy(64, 32, 8, 128, 8192, 16, 256) == (0, 0, 1, 8192)
    assert P.paged_decode_workspace_size(64, 32, 8, 128, 8192, 16, 256) == (0, 1, 8192)
    assert M.decode_q_policy(64, 4, 32, 8, 128, 8192, 16, 256) == (0, 0, 1, 8192)
    assert M.decode_policy(63, 32, 8, 128, 8192, 16, 256)[2] > 1      # 504 < 512 items
    assert M.decode_policy(257, 32, 8, 128, 8192, 16, 256)[2] > 1     # too many to order in LDS
    assert M.decode_q_policy(64, 5, 32, 8, 128, 8192, 16, 256)[2] > 1  # 20 query rows per KV head


def test_decode_validate_matches_spec():
    rng = np.random.default_rng(2)
    case = W.make_decode(10, 4, 8, 2, 128, [5, 40, 1, 77], 16, extra_pages=3)
    n_bad = 0
    for t in range(200):
        ip, ix, sl = case.kv_indptr.copy(), case.kv_indices.copy(), case.seq_lens.copy()
        k = t % 5
        if t == 0:
            pass
        elif k == 0:
            ix[rng.integers(0, ix.size)] = int(rng.choice([-1, case.k.shape[0]]))
        elif k == 1:
            ip[rng.integers(0, ip.size)] += int(rng.choice([-1, 1, 2]))
        elif k == 2:
            sl[rng.integers(0, sl.size)] = int(rng.choice([0, -3, 78, 200]))
        elif k == 3:
            sl[rng.integers(0, sl.size)] += 17
        else:
            ip[0] = -1
        want = M.decode_validate(4, case.k.shape[0], 16, 100, ip, ix, sl)
        st, f, i = P.paged_decode_validate(4, case.k.shape[0], 16, 100, ip, ix, sl,
                                           raise_on_error=False)
        got = (st, f, i) if st == M.PKB_ERR_METADATA else (st, 0, -1)
        assert got == want, (t, got, want)
        n_bad += want[0] != 0
    assert n_bad > 80


def test_decode_q_policy_matches_spec():
    rng = np.random.default_rng(4)
    for _ in range(1000):
        B = int(rng.integers(1, 300)); Hkv = int(rng.choice([1, 2, 8])); Hq = Hkv * int(rng.choice([1, 4, 16]))
        D = int(rng.choice([128, 256, 64])); msl = int(rng.choice([1, 64, 65, 8192, M.MAX_SEQ_LEN]))
        ps = int(rng.choice([8, 16, 12])); cus = int(rng.choice([80, 256]))
        mq = int(rng.choice([0, 1, 2, 7, 64]))
        want = M.decode_q_policy(B, mq, Hq, Hkv, D, msl, ps, cus)
        nb = ctypes.c_size_t(); s = ctypes.c_int32(); l = ctypes.c_int32()
        st = P.lib().paged_decode_q_workspace_size(B, mq, Hq, Hkv, D, msl, ps, cus, ctypes.byref(nb),
                                                   ctypes.byref(s), ctypes.byref(l))
        assert st == want[0]
        if st == 0:
            assert (nb.value, s.value, l.value) == want[1:]


def test_decode_q_validate_matches_spec():
    rng = np.random.default_rng(5)
    case = W.make_decode_q(11, 4, 8, 2, 128, [5, 40, 3, 77], 16, qlens=[2, 6, 3, 1],
                           extra_pages=3)
    n_bad = 0
    for t in range(300):
        ip, ix, sl = case.kv_indptr.copy(), case.kv_indices.copy(), case.seq_lens.copy()
        qo = case.qo_indptr.copy()
        total, sq, msq, causal = int(qo[-1]), 0, 6, bool(rng.random() < 0.7)
        packed = t % 7 != 6
        k = t % 8
        if t < 2:
            pass
        elif k == 0:
            ix[rng.integers(0, ix.size)] = int(rng.choice([-1, case.k.shape[0]]))
        elif k == 1:
            ip[rng.integers(0, ip.size)] += int(rng.choice([-1, 1, 2]))
        elif k == 2:
            sl[rng.integers(0, sl.size)] = int(rng.choice([0, -3, 78, 200, 2]))
        elif k == 3:
            qo[rng.integers(0, qo.size)] += int(rng.choice([-1, 1, 3]))
        elif k == 4:
            msq = int(rng.choice([0, 3, 5]))
        elif k == 5:
            total = int(rng.choice([0, total - 1, total + 1]))
        else:
            sq = int(rng.choice([0, 1, 3, 4, 6]))
        if not packed:
            sq = sq or 2
        want = M.decode_q_validate(4, case.k.shape[0], 16, 100, ip, ix, sl,
                                   qo if packed else None, total, sq, msq, causal)
        st, f, i = P.paged_decode_q_validate(4, case.k.shape[0], 16, 100, ip, ix, sl,
                                             qo_indptr=qo if packed else None, total_q=total,
                                             seq_len_q=sq, max_seq_len_q=msq,
                                             mask_type="causal" if causal else "dense",
                                             raise_on_error=False)
        got = (st, f, i) if st == M.PKB_ERR_METADATA else (st, 0, -1)
        assert got == want, (t, packed, causal, got, want)
        n_bad += want[0] != 0
    assert n_bad > 100


# ----------------------------------------------------------------------------- sage

def test_sage_validate_matches_spec():
    rng = np.random.default_rng(3)
    for t in range(120):
        B, H, Sq, Sk, cap = 2, 3, int(rng.integers(1, 300)), int(rng.integers(1, 400)), int(rng.integers(0, 6))
        nqb, nkb = -(-Sq // 64), -(-Sk // 64)
        idx = rng.integers(-1, nkb + 1, size=(B, H, nqb, max(cap, 1)))[..., :cap].astype(np.int32)
        if rng.random() < 0.5:
            for b in range(B):
                for h in range(H):
                    for r in range(nqb):
                        k = min(cap, nkb)
                        idx[b, h, r, :k] = rng.permutation(nkb)[:k]
        nums = rng.integers(-1, cap + 2, size=(B, H, nqb)).astype(np.int32) if rng.random() < 0.6 else None
        if nums is not None and rng.random() < 0.5:
            nums = np.clip(nums, 0, min(cap, nkb)).astype(np.int32)
        bsn = int(rng.integers(-1, cap + 2))
        rank = int(rng.integers(0, 4))
        bs = None if rank == 0 else rng.integers(-1, 66, size=[(nkb,), (B, nkb), (B, H, nkb)][rank - 1]).astype(np.int32)
        uniform = bool(rng.random() < 0.3)
        want = M.sage_validate(idx, cap, bsn, bs, nums, uniform, B, H, Sq, Sk)
        st, f, i = P.bsa_sage_validate(idx, cap, bsn, bs, nums, uniform, B, H, Sq, Sk,
                                       raise_on_error=False)
        got = (st, f, i) if st == M.PKB_ERR_METADATA else (st, 0, -1)
        assert got == want, (t, got, want)


def test_sage_run_static_errors():
    # Rejected before any device work: the dummy pointers are never dereferenced.
    L = P.lib()
    d = ctypes.c_void_p(256)

    def run(B=1, H=1, Sq=64, Sk=64, q=d, mask=M.DENSE, scale=math.nan):
        return L.bsa_sage_run(q, d, d, d, d, d, d, 1, 1, None, 0, None, 0, 0,
                              B, H, Sq, Sk, scale, mask, d, None, None)
    assert run(q=None) == M.PKB_ERR_ARG
    assert run(Sk=0) == M.PKB_ERR_ARG
    assert run(mask=7) == M.PKB_ERR_ARG
    # the page asks for a positive scale; NaN is the default's sentinel
    for bad in (0.0, -0.5, math.inf, -math.inf):
        assert run(scale=bad) == M.PKB_ERR_ARG, bad
    # V^T offsets inside one head are 32-bit: Sk up to 2^25
    assert run(Sk=(1 << 25) + 1) == M.PKB_ERR_UNSUPPORTED


# ----------------------------------------------------------------------------- QSA

def test_qsa_run_static_errors():
    # Rejected before any device work: the dummy pointers are never dereferenced.
    L = P.lib()
    d = ctypes.c_void_p(256)

    def run(T=64, NB=16, Hq=12, Hkv=1, D=256, scale=0.0625, bs=4, q=d):
        return L.qsa_run(q, d, d, d, d, d, d, d, T, NB, Hq, Hkv, D, scale, bs, d, None, None, None)
    assert run(q=None) == M.PKB_ERR_ARG
    assert run(T=0) == M.PKB_ERR_ARG
    assert run(bs=8) == M.PKB_ERR_UNSUPPORTED
    assert run(Hq=24) == M.PKB_ERR_UNSUPPORTED          # 24 query heads per KV head
    assert run(scale=float("inf")) == M.PKB_ERR_ARG
    # K / V rows are addressed with 32-bit byte offsets: each pool at most 4 GiB
    assert run(T=(1 << 23) + 1, Hkv=1, D=256) == M.PKB_ERR_UNSUPPORTED


def test_qsa_validate_matches_spec():
    rng = np.random.default_rng(6)
    case = W.make_qsa(60, [9, 1, 14, 4, 7], Hq=2, Hkv=1, D=16, p_sel=0.3, empty_rows=2)
    base = [case.lo, case.hi, case.blk_base, case.tok_base, case.block_first, case.block_last]
    n_bad = 0
    for t in range(400):
        a = [x.copy() for x in base]
        k = t % 7
        if t < 3:
            pass
        else:
            which = int(rng.integers(0, 6))
            arr = a[which]
            i = int(rng.integers(0, arr.size))
            arr[i] += int(rng.choice([-5, -1, 1, 2, 40]))
            if k == 6:      # a second, independent change
                arr2 = a[int(rng.integers(0, 6))]
                arr2[int(rng.integers(0, arr2.size))] = int(rng.integers(-2, 40))
        want = M.qsa_validate(*a)
        st, f, i = P.qsa_validate(*a, raise_on_error=False)
        got = (st, f, i) if st == M.PKB_ERR_METADATA else (st, 0, -1)
        assert got == want, (t, got, want)
        n_bad += want[0] != 0
    assert n_bad > 150
    assert M.qsa_validate(*base) == M.OK


# ----------------------------------------------------------------------------- scales

def test_runs_reject_bad_softmax_scales():
    """A softmax scale that is zero, negative or not finite is rejected before
    anything is launched (NaN alone selects the default 1/sqrt(D)); the dummy
    device pointers are never dereferenced.  Only rejections are exercised
    here: an accepted scale would launch a kernel."""
    L = P.lib()
    d = ctypes.c_void_p(256)
    bsa = P.bsa_plan(1, 64, 4, 1, 128, 8, 16, 16, 64, 128, M.CAUSAL, num_cus_=256)
    pre_args = P.ops._prefill_args(1, 4, 1, 128, 8, 16, 64, 8, "causal", -1, torch.bfloat16, 256)
    pre, _ = P.paged_prefill_plan(pre_args, [0, 64], [100])
    for bad in (0.0, -1.0, math.inf, -math.inf):
        assert L.bsa_run(ctypes.byref(bsa), d, d, d, 8 * 16 * 128, 16 * 128, d, d, d, d, d, None,
                         bad, d, None, None) == M.PKB_ERR_ARG, bad
        assert L.paged_prefill_run(ctypes.byref(pre), d, d, d, d, 16 * 128, 16 * 128, d, d, 8, d,
                                   bad, 1.0, d, None, None) == M.PKB_ERR_ARG, bad
        assert L.paged_decode_run(d, d, d, 8 * 16 * 128, 16 * 128, d, d, d, 4, 32, 8, 128, 64, 16,
                                  512, M.DENSE, -1, bad, 1.0, 0, d, None, d, 1 << 30, 256,
                                  None) == M.PKB_ERR_ARG, bad
        assert L.paged_decode_q_run(d, d, d, 8 * 16 * 128, 16 * 128, d, d, d, None, 4, 2, 0, 32, 8,
                                    128, 64, 16, 512, M.CAUSAL, -1, bad, 1.0, 0, d, None, d,
                                    1 << 30, 256, None) == M.PKB_ERR_ARG, bad


def test_binding_rejects_unknown_mask_strings():
    """Mask names are looked up strictly: a misspelt name is an error, never a
    silent dense mask."""
    with pytest.raises(ValueError):
        P.BlockSparsePagedWrapper(1, 64, 4, 1, 128, 8, 16, 16, 64, 128, "Causal")
    with pytest.raises(ValueError):
        P.ops._prefill_args(1, 4, 1, 128, 8, 16, 64, 8, "causal ", -1, torch.bfloat16, 256)


def test_noalloc_decode_rejects_oversized_partials_before_launch():
    """The allocation-free decode checks its partials against the fixed scratch
    (PKB_DECODE_SCRATCH_BYTES) before any device work; the dummy pointers are
    never dereferenced."""
    nbytes, S, _ = P.paged_decode_workspace_size(300, 32, 8, 256, 8192, 16, 256)
    assert S > 1 and nbytes > C.PKB_DECODE_SCRATCH_BYTES == 32 << 20
    d = ctypes.c_void_p(256)
    st = P.lib().paged_decode_run_noalloc(d, d, d, 8 * 16 * 256, 16 * 256, d, d, d, 300, 32, 8,
                                          256, 1000, 16, 8192, M.DENSE, -1, math.nan, 1.0, 0, d,
                                          None, 256, None)
    assert st == C.PKB_ERR_WORKSPACE
