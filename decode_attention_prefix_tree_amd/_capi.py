"""ctypes declarations of libchunkattn.so (include/chunkattn.h).

Loading fails loudly when the library is missing: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libchunkattn.so")
HEADER = os.path.join(ROOT, "include", "chunkattn.h")

CA_OK = 0
CA_CREATE_UNSHARED = 1
CA_CREATE_NO_CHUNK_FIRST = 2
CA_OPT_CF_CHUNKS_PER_TASK = 1
CA_OPT_SF_CHUNKS_PER_TASK = 2
CA_OPT_FUSED_MERGE = 3
CA_OPT_MERGE_POLL_LIMIT = 4
CA_OPT_FAIL_DEVICE_OPS = 5
CA_OPT_PREBUILD_PLAN = 6
CA_OPT_ROW_APPENDS = 7
CA_OPT_FAIL_AFTER_DEVICE_OPS = 8
CA_NOALLOC_SCRATCH_BYTES = 16 << 20
CA_PHASE_CHUNK_FIRST = 1
CA_PHASE_SEQUENCE_FIRST = 2
CA_PHASE_MERGE = 3
CA_PHASE_PARTIALS = 4

ERROR_NAMES = {
    -1: "invalid_arg", -2: "unsupported", -3: "no_capacity", -4: "dup_seq", -5: "unknown_seq",
    -6: "empty", -7: "workspace", -8: "hip", -9: "no_pool", -10: "state", -11: "internal",
}


class CaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code
        self.name = ERROR_NAMES.get(code, str(code))


class ca_stats_t(ctypes.Structure):
    _fields_ = [
        ("live_sequences", ctypes.c_int64),
        ("chunks", ctypes.c_int64),
        ("shared_chunks", ctypes.c_int64),
        ("unique_tokens", ctypes.c_int64),
        ("attended_tokens", ctypes.c_int64),
        ("capacity_slots", ctypes.c_int64),
        ("free_slots", ctypes.c_int64),
        ("table_rebuilds", ctypes.c_int64),
        ("last_rebuild_ms", ctypes.c_double),
        ("cf_tasks", ctypes.c_int64),
        ("cf_units", ctypes.c_int64),
        ("sf_tasks", ctypes.c_int64),
        ("partials", ctypes.c_int64),
        ("cf_chunk_reads", ctypes.c_int64),
        ("sf_chunk_reads", ctypes.c_int64),
        ("unique_kv_bytes", ctypes.c_int64),
        ("attended_kv_bytes", ctypes.c_int64),
        ("shared_tokens", ctypes.c_int64),
        ("private_tokens", ctypes.c_int64),
        ("fill_refreshes", ctypes.c_int64),
        ("table_uploads", ctypes.c_int64),
        ("patched_appends", ctypes.c_int64),
        ("cf_chunks_per_task", ctypes.c_int64),
        ("one_launch_step", ctypes.c_int64),
        ("sf_chunks_per_task", ctypes.c_int64),
        ("prebuilt_plans", ctypes.c_int64),
        ("row_chunks", ctypes.c_int64),
    ]


_c = ctypes
_SIGS = {
    "ca_slot_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int]),
    "ca_create": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.POINTER(_c.c_void_p)]),
    "ca_create_ex": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.POINTER(_c.c_void_p)]),
    "ca_destroy": (None, [_c.c_void_p]),
    "ca_attach_pool": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64]),
    "ca_workspace_bytes": (_c.c_int, [_c.c_void_p, _c.POINTER(_c.c_size_t)]),
    "ca_attach_workspace": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t]),
    "ca_staging_bytes": (_c.c_int, [_c.c_void_p, _c.POINTER(_c.c_size_t)]),
    "ca_attach_staging": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t]),
    "ca_set_option": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int]),
    "ca_insert": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.POINTER(_c.c_int32), _c.c_int32, _c.c_void_p,
                             _c.c_void_p, _c.c_void_p, _c.POINTER(_c.c_int32)]),
    "ca_append": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.POINTER(_c.c_int32), _c.c_int32, _c.c_void_p,
                             _c.c_void_p, _c.c_void_p]),
    "ca_append_batch": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.POINTER(_c.c_int64), _c.POINTER(_c.c_int32),
                                   _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "ca_remove": (_c.c_int, [_c.c_void_p, _c.c_int64]),
    "ca_attend": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "ca_attend_noalloc": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    # tokens as an address: the binding passes the array's data pointer
    "ca_decode_step": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                  _c.c_void_p, _c.c_void_p]),
    "ca_prepare": (_c.c_int, [_c.c_void_p, _c.c_void_p]),
    "ca_attend_phase": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "ca_list_sequences": (_c.c_int, [_c.c_void_p, _c.POINTER(_c.c_int64), _c.c_int]),
    "ca_export_table": (_c.c_int, [_c.c_void_p, _c.POINTER(_c.c_int32), _c.c_int, _c.POINTER(_c.c_int64),
                                   _c.c_int, _c.POINTER(_c.c_int), _c.POINTER(_c.c_int)]),
    "ca_export_plan": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.POINTER(_c.c_size_t)]),
    "ca_stats": (_c.c_int, [_c.c_void_p, _c.POINTER(ca_stats_t)]),
    "ca_last_error": (_c.c_char_p, [_c.c_void_p]),
}

_lib = None


def header_symbols() -> list:
    """Function names declared in include/chunkattn.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*\s]+?)\b(ca_\w+)\s*\(", text, re.M)))


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decode_attention_prefix_tree_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(ctx, rc: int) -> int:
    if rc < 0:
        msg = load().ca_last_error(ctx)
        raise CaError(rc, msg.decode() if msg else "")
    return rc
