"""ctypes view of libpkb.so (the C ABI declared in include/pkb.h).

Loading fails loudly when the library has not been built: there is no fallback
implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PKB_LIBRARY", os.path.join(HERE, "libpkb.so"))

PKB_OK = 0
PKB_ERR_ARG = -1
PKB_ERR_SHAPE = -2
PKB_ERR_DTYPE = -3
PKB_ERR_UNSUPPORTED = -4
PKB_ERR_METADATA = -5
PKB_ERR_WORKSPACE = -6
PKB_ERR_HIP = -7

PKB_BF16, PKB_FP32, PKB_I8, PKB_FP8E4M3 = 0, 1, 2, 3
PKB_MASK_DENSE, PKB_MASK_CAUSAL = 0, 1
PKB_MAX_SEQ_LEN = 2147483520
PKB_DECODE_SCRATCH_BYTES = 32 << 20

FIELD_NAMES = {0: "none", 1: "paged_kv_indptr", 2: "paged_kv_indices", 3: "seq_lens",
               4: "block_indptr", 5: "block_indices", 6: "qo_indptr", 7: "block_tables",
               8: "q2k_block_index", 9: "q2k_block_nums", 10: "block_sizes", 11: "lo",
               12: "hi", 13: "blk_base", 14: "tok_base", 15: "block_first", 16: "block_last"}


class BsaStaticArgs(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "B", "Sq", "Hq", "Hkv", "D", "num_pages", "page_size", "q_block_size",
        "kv_block_size", "max_seq_len_kv", "mask_type", "window_left", "qkv_dtype",
        "out_dtype", "num_cus")]


class BsaPlan(ctypes.Structure):
    _fields_ = [("a", BsaStaticArgs)] + [(n, c_int32) for n in (
        "group", "rows_per_brow", "num_q_blocks", "num_kv_blocks", "valid_words", "waves",
        "tile_m", "tiles_per_brow", "grid_x", "grid_y", "grid_z", "kernel_id")]


class PrefillStaticArgs(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "B", "Hq", "Hkv", "D", "num_pages", "page_size", "total_q", "block_table_width",
        "mask_type", "window_left", "qkv_dtype", "out_dtype", "num_cus")]


class PrefillPlan(ctypes.Structure):
    _fields_ = [("a", PrefillStaticArgs)] + [(n, c_int32) for n in (
        "group", "waves", "tile_m", "n_work", "grid_x", "grid_y", "kernel_id")] + \
        [("kv_tokens", c_int64)]


class Bad(ctypes.Structure):
    _fields_ = [("field", c_int32), ("index", c_int64)]


I32P = POINTER(c_int32)

_SIGS = {
    "pkb_status_string": (ctypes.c_char_p, [c_int]),
    "pkb_abi_version": (c_int, []),
    "pkb_last_hip_error": (ctypes.c_char_p, []),
    "bsa_plan": (c_int, [POINTER(BsaStaticArgs), POINTER(BsaPlan)]),
    "bsa_validate": (c_int, [POINTER(BsaPlan), c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                             c_int64, c_void_p, POINTER(Bad)]),
    "bsa_run": (c_int, [POINTER(BsaPlan), c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                        c_void_p, c_void_p, c_void_p]),
    "paged_prefill_validate": (c_int, [POINTER(PrefillStaticArgs), c_void_p, c_void_p, c_void_p,
                                       c_int64, POINTER(Bad)]),
    "paged_prefill_plan": (c_int, [POINTER(PrefillStaticArgs), c_void_p, c_void_p,
                                   POINTER(PrefillPlan), c_void_p, c_int64, POINTER(c_int64)]),
    "paged_prefill_plan_capacity": (c_int, [POINTER(PrefillStaticArgs), c_int32,
                                            POINTER(PrefillPlan), c_void_p, c_int64,
                                            POINTER(c_int64)]),
    "paged_prefill_run": (c_int, [POINTER(PrefillPlan), c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int64, c_int64, c_void_p, c_void_p, c_int64, c_void_p,
                                  c_float, c_float, c_void_p, c_void_p, c_void_p]),
    "paged_decode_workspace_size": (c_int, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                            c_int32, POINTER(c_size_t), POINTER(c_int32),
                                            POINTER(c_int32)]),
    "paged_decode_validate": (c_int, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                      c_int64, c_void_p, POINTER(Bad)]),
    "paged_decode_run": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p,
                                 c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                 c_int32, c_int32, c_int32, c_int32, c_float, c_float, c_int32,
                                 c_void_p, c_void_p, c_void_p, c_size_t, c_int32, c_void_p]),
    "paged_decode_run_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                         c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                         c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                         c_float, c_float, c_int32, c_void_p, c_void_p, c_int32,
                                         c_void_p]),
    "paged_decode_q_workspace_size": (c_int, [c_int32, c_int32, c_int32, c_int32, c_int32,
                                              c_int32, c_int32, c_int32, POINTER(c_size_t),
                                              POINTER(c_int32), POINTER(c_int32)]),
    "paged_decode_q_validate": (c_int, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                        c_int64, c_void_p, c_void_p, c_int64, c_int32, c_int32,
                                        c_int32, POINTER(Bad)]),
    "paged_decode_q_run": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                   c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                   c_int32, c_float, c_float, c_int32, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_int32, c_void_p]),
    "qsa_validate": (c_int, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, POINTER(Bad)]),
    "qsa_run": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                        c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_float, c_int32,
                        c_void_p, c_void_p, c_void_p, c_void_p]),
    "bsa_sage_validate": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p,
                                  c_int32, c_int32, c_int32, c_int32, c_int32, POINTER(Bad)]),
    "bsa_sage_run": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_int32,
                             c_int32, c_int32, c_int32, c_int32, c_int32, c_float, c_int32,
                             c_void_p, c_void_p, c_void_p]),
}

EXPORTS = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libpkb.so is missing (no fallback path)."""
    global _lib
    if _lib is None:
        # torch brings its own HIP runtime (same soname as the system one).  Load
        # it first so libpkb binds to that copy: two HIP runtimes in one process
        # do not share devices, streams or allocations.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libpkb.so not found at {LIB_PATH}: build it with "
                "`python -m paged_kv_block_amd.build` (there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class PkbError(RuntimeError):
    def __init__(self, status: int, what: str = "", bad: Bad | None = None):
        msg = f"{what}: {lib().pkb_status_string(status).decode()} (status {status})"
        if status == PKB_ERR_HIP:
            msg += f" [{lib().pkb_last_hip_error().decode()}]"
        if bad is not None and bad.field:
            msg += f"; first violation in {FIELD_NAMES.get(bad.field, bad.field)}[{bad.index}]"
        super().__init__(msg)
        self.status = status
        self.field = bad.field if bad is not None else 0
        self.index = bad.index if bad is not None else -1


def check(status: int, what: str, bad: Bad | None = None):
    if status != PKB_OK:
        raise PkbError(status, what, bad)
