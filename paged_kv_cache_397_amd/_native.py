"""ctypes loader of libpagedkv.so with the signatures of include/pagedkv.h.

Only marshalling lives here.  If the library has not been built the import of
any op fails with a clear error: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

# Always the in-package build: no environment variable can point the binding at
# another copy of the library.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

c_i32, c_i64, c_sz, c_f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
c_vp = ctypes.c_void_p
c_u32 = ctypes.c_uint32
P_i32, P_i64 = ctypes.POINTER(c_i32), ctypes.POINTER(c_i64)

STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_OOM",
                4: "PA_ERR_STATE", 5: "PA_ERR_HIP", 6: "PA_ERR_TOO_LARGE"}
(PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_OOM, PA_ERR_STATE, PA_ERR_HIP,
 PA_ERR_TOO_LARGE) = range(7)
# PA_DECODE_NOALLOC_SCRATCH_BYTES: size of the static buffer behind pa_paged_attn_decode_noalloc
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({_status_string(status)})")


class SchedPlan(ctypes.Structure):
    """pa_sched_plan: counts and pointers into the scheduler's arrays."""
    _fields_ = [("step", c_i64),
                ("num_finished", c_i32), ("num_arrived", c_i32), ("num_admitted", c_i32),
                ("num_preempted", c_i32), ("num_prefill", c_i32), ("num_decode", c_i32),
                ("num_decode_cows", c_i32), ("num_swapped_in", c_i32), ("num_swapped_out", c_i32),
                ("num_prefill_tokens", c_i64),
                ("finished", P_i64), ("arrived", P_i64), ("admitted", P_i64),
                ("admitted_cached", P_i32), ("preempted", P_i64),
                ("prefill_rid", P_i64), ("prefill_start", P_i32), ("prefill_count", P_i32),
                ("prefill_slots", P_i64),
                ("decode_rid", P_i64), ("decode_pos", P_i64), ("decode_slot", P_i64),
                ("decode_cow", P_i32),
                ("swapped_in", P_i64), ("swapped_in_pairs", P_i32), ("swap_in", P_i32),
                ("swapped_out", P_i64), ("swapped_out_pairs", P_i32), ("swap_out", P_i32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", c_i32), ("block_size", c_i32), ("num_kv_heads", c_i32),
                ("head_dim", c_i32), ("dtype", c_i32)]


P_desc = ctypes.POINTER(CacheDesc)

# name -> (restype, argtypes); one entry per function declared in include/pagedkv.h
SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [c_i32]),
    "pa_abi_version": (c_i32, []),
    "pa_cache_bytes": (c_sz, [P_desc]),
    "pa_reshape_and_cache": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "pa_copy_blocks": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_i32, c_vp]),
    "pa_update_block_tables": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_i32, c_vp]),
    "pa_append_tokens": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_i32,
                                 c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp]),
    "pa_decode_workspace_bytes": (c_sz, [P_desc, c_i32, c_i32]),
    "pa_decode_default_units": (c_i32, []),
    "pa_paged_attn_decode": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                     c_i32, c_f32, c_i32, c_vp, c_sz, c_u32, c_vp]),
    "pa_paged_attn_decode_partial": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                             c_i32, c_i32, c_f32, c_i32, c_vp, c_sz, c_u32, c_vp]),
    "pa_decode_step_workspace_bytes": (c_sz, [P_desc, c_i32, c_i32, c_i32]),
    "pa_decode_step": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                               c_vp, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp, c_sz, c_u32, c_vp]),
    "pa_paged_attn_decode_noalloc": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                             c_i32, c_i32, c_f32, c_i32, c_u32, c_vp]),
    "pa_paged_attn_decode_merge": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                           c_i32, c_i32, c_f32, c_i32, c_vp, c_sz, c_u32, c_vp]),
    "pa_paged_attn_prefill": (c_i32, [P_desc, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                      c_i32, c_i32, c_i32, c_i32, c_f32, c_vp]),
    "pa_alloc_create": (c_i32, [c_i32, c_i32, c_vp, ctypes.POINTER(c_vp)]),
    "pa_alloc_destroy": (None, [c_vp]),
    "pa_alloc_num_free": (c_i32, [c_vp]),
    "pa_alloc_num_seqs": (c_i32, [c_vp]),
    "pa_alloc_refcount": (c_i32, [c_vp, c_i32]),
    "pa_alloc_free_list": (c_i32, [c_vp, c_vp, c_i32, P_i32]),
    "pa_seq_add": (c_i32, [c_vp, c_i64, c_i32]),
    "pa_seq_append": (c_i32, [c_vp, c_i64, P_i64, P_i32, P_i32]),
    "pa_seq_append_batch": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, P_i32]),
    "pa_seq_fork": (c_i32, [c_vp, c_i64, c_i64]),
    "pa_seq_free": (c_i32, [c_vp, c_i64]),
    "pa_seq_slots": (c_i32, [c_vp, c_i64, c_i32, c_i32, c_vp]),
    "pa_seq_info": (c_i32, [c_vp, c_i64, P_i32, P_i32]),
    "pa_seq_block_table": (c_i32, [c_vp, c_i64, c_vp, c_i32]),
    "pa_batch_metadata": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_vp]),
    "pa_seq_add_prefix": (c_i32, [c_vp, c_i64, c_vp, c_i32, P_i32]),
    "pa_seq_register_blocks": (c_i32, [c_vp, c_i64, c_vp, c_i32]),
    "pa_alloc_prefix_stats": (c_i32, [c_vp, P_i64, P_i64, P_i32]),
    "pa_alloc_block_cached": (c_i32, [c_vp, c_i32, ctypes.POINTER(ctypes.c_uint64)]),
    "pa_swap_blocks": (c_i32, [P_desc, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_i32, c_vp]),
    "pa_alloc_set_host_pool": (c_i32, [c_vp, c_i32]),
    "pa_alloc_num_free_host": (c_i32, [c_vp]),
    "pa_alloc_host_free_list": (c_i32, [c_vp, c_vp, c_i32, P_i32]),
    "pa_seq_host_blocks": (c_i32, [c_vp, c_i64, c_vp, c_i32]),
    "pa_seq_is_swapped": (c_i32, [c_vp, c_i64]),
    "pa_seq_swap_out": (c_i32, [c_vp, c_i64, c_vp, c_i32, P_i32]),
    "pa_seq_swap_in": (c_i32, [c_vp, c_i64, c_vp, c_i32, P_i32]),
    "pa_sched_create": (c_i32, [c_i32, c_i32, c_vp, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)]),
    "pa_sched_destroy": (None, [c_vp]),
    "pa_sched_allocator": (c_vp, [c_vp]),
    "pa_sched_add_requests": (c_i32, [c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "pa_sched_push_tokens": (c_i32, [c_vp, c_vp, c_vp, c_i32]),
    "pa_sched_step": (c_i32, [c_vp, ctypes.POINTER(SchedPlan)]),
    "pa_sched_running": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32]),
    "pa_sched_waiting": (c_i32, [c_vp, c_vp, c_i32]),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m paged_kv_cache_397_amd.build` (there is no CPU fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _status_string(status: int) -> str:
    try:
        return lib().pa_status_string(status).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def check(status: int, what: str) -> None:
    if status != PA_OK:
        raise PagedKVError(status, what)
