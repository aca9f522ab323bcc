"""ctypes mirror of include/tg.h and the loader of ``libtg.so``.

The shared library must have been built (``python -m
non_uniform_paged_amd.build``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

# TG_LIB_PATH names another build of the same library (the sanitizer build
# of the CPU tests); by default the in-tree libtg.so is loaded.
LIB_PATH = os.environ.get("TG_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtg.so")

TG_OK = 0
TG_EINVAL = -1
TG_ENOMEM = -2
TG_EOVERFLOW = -3
TG_EDEVICE = -4
TG_EUNSUPPORTED = -5
STATUS_NAMES = {0: "TG_OK", -1: "TG_EINVAL", -2: "TG_ENOMEM", -3: "TG_EOVERFLOW",
                -4: "TG_EDEVICE", -5: "TG_EUNSUPPORTED"}

TG_TIER_I8 = 0
TG_TIER_BF16 = 1
TG_GROUP_WIDTH = 32
TG_BENCH_READ_BLOCKS = 4096
TG_MAX_CLUSTERS = 16
TG_NOALLOC_SCRATCH_BYTES = 32 << 20
TG_Q_F32 = 0
TG_Q_BF16 = 1

P32 = POINTER(c_int32)
P64 = POINTER(c_int64)


class BudgetTable(ctypes.Structure):
    _fields_ = [("n_kv_heads", c_int32), ("head_rank", P32), ("ratio_hi_ppm", c_int32),
                ("ratio_lo_ppm", c_int32), ("n_clusters", c_int32), ("recent_ppm", c_int32),
                ("quant_block", c_int32)]


class Reservation(ctypes.Structure):
    _fields_ = [("B", c_int32), ("n_kv_heads", c_int32), ("n_clusters", c_int32),
                ("budget", P32), ("length", P32), ("n_i8", P32), ("n_bf", P32),
                ("cluster_of_head", P32), ("slot_in_cluster", P32), ("cluster_size", P32),
                ("recent_ppm", c_int32), ("quant_block", c_int32)]


class ShareDesc(ctypes.Structure):
    _fields_ = [("n_nodes", P32), ("node_ids", P32), ("n_node_table", c_int32), ("node_len", P32)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("chunk_bf", c_int32), ("chunk_i8", c_int32), ("lpt", c_int32), ("group_size", c_int32),
                ("gen_tokens", c_int32), ("chunk_group", c_int32)]


class TableSizes(ctypes.Structure):
    _fields_ = [("stride", (c_int32 * 2) * TG_MAX_CLUSTERS), ("n_items", c_int32),
                ("n_gitems", c_int32), ("n_slots", c_int32),
                ("pages_needed", (c_int64 * 2) * TG_MAX_CLUSTERS)]


class Tables(ctypes.Structure):
    _fields_ = [("bt", (P32 * 2) * TG_MAX_CLUSTERS), ("stride", (c_int32 * 2) * TG_MAX_CLUSTERS),
                ("len", P32), ("work", P32), ("n_items", c_int32), ("part_off", P32),
                ("released", P32), ("gitems", P32), ("n_gitems", c_int32), ("ring", P32), ("B", c_int32)]


class Cache(ctypes.Structure):
    _fields_ = [("B", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("page_size", c_int32), ("quant_block", c_int32), ("n_clusters", c_int32),
                ("pool", (c_void_p * 2) * TG_MAX_CLUSTERS),
                ("page_bytes", (c_int64 * 2) * TG_MAX_CLUSTERS),
                ("n_pages", (c_int64 * 2) * TG_MAX_CLUSTERS),
                ("bt", (c_void_p * 2) * TG_MAX_CLUSTERS),
                ("stride", (c_int32 * 2) * TG_MAX_CLUSTERS),
                ("cluster_of_head", c_void_p), ("slot_in_cluster", c_void_p), ("len", c_void_p),
                ("n_fixed", c_void_p), ("ring", c_void_p), ("bf_base", c_void_p), ("recent_ppm", c_int32),
                ("old_bits", c_int32),
                ("head_major", (c_int32 * 2) * TG_MAX_CLUSTERS)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("n_q_heads", c_int32), ("q_dtype", c_int32), ("q", c_void_p), ("work", c_void_p),
                ("n_items", c_int32), ("part_off", c_void_p), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t), ("out", c_void_p), ("sm_scale", c_float),
                ("gitems", c_void_p), ("n_gitems", c_int32), ("n_slots", c_int32)]


# name -> (restype, argtypes); the full exported surface of include/tg.h
SIGNATURES = {
    "tg_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "tg_reserve": (ctypes.c_int, [POINTER(BudgetTable), c_int32, P32, P32, P32, POINTER(Reservation)]),
    "tg_pool_create": (ctypes.c_int, [c_int32, P32, c_int32, c_int32, c_int32, c_int32, P64, P64,
                                      POINTER(c_void_p)]),
    "tg_pool_destroy": (None, [c_void_p]),
    "tg_pool_page_bytes": (c_int64, [c_void_p, c_int32, c_int32]),
    "tg_pool_capacity": (c_int64, [c_void_p, c_int32, c_int32]),
    "tg_pool_free_pages": (c_int64, [c_void_p, c_int32, c_int32]),
    "tg_pool_refcount": (c_int32, [c_void_p, c_int32, c_int32, c_int64]),
    "tg_size_tables": (ctypes.c_int, [POINTER(Reservation), c_int32, c_int32, POINTER(ShareDesc),
                                      POINTER(PlanOpts), POINTER(TableSizes)]),
    "tg_build_tables": (ctypes.c_int, [c_void_p, POINTER(Reservation), POINTER(ShareDesc),
                                       POINTER(PlanOpts), POINTER(Tables)]),
    "tg_release": (ctypes.c_int, [c_void_p, POINTER(Tables), c_int32]),
    "tg_check_tables": (ctypes.c_int, [c_void_p, POINTER(Reservation), POINTER(Tables), ctypes.c_char_p,
                                       c_size_t]),
    "tg_write_kv": (ctypes.c_int, [POINTER(Cache), c_void_p, c_void_p, c_void_p, c_void_p]),
    "tg_decode_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "tg_decode_attn": (ctypes.c_int, [POINTER(Cache), POINTER(DecodeArgs), c_void_p]),
    "tg_decode_split": (ctypes.c_int, [POINTER(Cache), POINTER(DecodeArgs), c_void_p]),
    "tg_decode_attn_noalloc": (ctypes.c_int, [POINTER(Cache), POINTER(DecodeArgs), c_void_p]),
    "tg_merge_partials": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                         c_void_p, c_void_p]),
    "tg_decode_split_timed": (ctypes.c_int, [POINTER(Cache), POINTER(DecodeArgs), c_void_p, c_void_p, c_void_p]),
    "tg_bench_read": (ctypes.c_int, [c_void_p, c_size_t, c_void_p, c_void_p, c_void_p, c_void_p]),
    "tg_bench_streams": (ctypes.c_int, [c_void_p, c_size_t, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p]),
    "tg_append_kv": (ctypes.c_int, [POINTER(Cache), c_void_p, c_void_p, c_void_p]),
    "tg_stream_staging_bytes": (c_size_t, [POINTER(Cache), POINTER(Tables)]),
    "tg_decode_streamed": (ctypes.c_int, [POINTER(Cache), POINTER(Tables), POINTER(DecodeArgs), P32, c_void_p,
                                          c_size_t, c_void_p]),
    "tg_stream_order": (ctypes.c_int, [POINTER(Tables), c_int32, P32, P32]),
    "tg_zip_bound": (c_size_t, [c_int64]),
    "tg_zip_workspace_bytes": (c_size_t, [c_int64]),
    "tg_zip_encode": (ctypes.c_int, [c_void_p, c_int64, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]),
    "tg_zip_decode": (ctypes.c_int, [c_void_p, c_int64, c_void_p, c_void_p]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """Load ``libtg.so`` once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m non_uniform_paged_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class TGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {self.name} ({lib().tg_strerror(status).decode()})")


def check(status: int, where: str) -> None:
    if status != TG_OK:
        raise TGError(status, where)
