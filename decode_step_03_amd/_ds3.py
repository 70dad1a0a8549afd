"""ctypes binding of libds3.so: the C ABI declared in include/ds3.h, function for function, same names.

Argument marshalling only. Every step of the decode path runs in the library's HIP kernels; nothing here computes.
If the library is missing, loading fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char, c_double, c_float, c_int32, c_int64, c_uint32, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libds3.so")

DS3_ABI_VERSION = 5

# ds3_status
DS3_OK = 0
DS3_E_INVALID = 1
DS3_E_UNSUPPORTED = 2
DS3_E_UNBOUND = 3
DS3_E_NOT_LOADED = 4
DS3_E_NEEDS_RESET = 5
DS3_E_KERNEL_CHECK = 6
DS3_E_TIMEOUT = 7
DS3_E_DEVICE_LOST = 8
DS3_E_POISONED = 9
STATUS_NAMES = {0: "DS3_OK", 1: "DS3_E_INVALID", 2: "DS3_E_UNSUPPORTED", 3: "DS3_E_UNBOUND", 4: "DS3_E_NOT_LOADED",
                5: "DS3_E_NEEDS_RESET", 6: "DS3_E_KERNEL_CHECK", 7: "DS3_E_TIMEOUT", 8: "DS3_E_DEVICE_LOST",
                9: "DS3_E_POISONED"}

DS3_F32, DS3_BF16 = 0, 1
DS3_KV_CONTIGUOUS, DS3_KV_PAGED = 0, 1
DS3_GRAPH, DS3_EAGER = 0, 1
DS3_PLAN_AUTO, DS3_PLAN_PER_OP, DS3_PLAN_FUSED = 0, 1, 2
DS3_TRACE_OFF, DS3_TRACE_BARRIERS, DS3_TRACE_PHASES = 0, 1, 2
DS3_MAX_CHAIN = 1024
DS3_SWEEP_FULL, DS3_SWEEP_VISIBLE = 0, 1
DS3_MAX_PREFILL = 8192
DS3_MAX_LOGPROBS = 8
DS3_NOALLOC_MAX_BYTES = 8 << 20   # the fixed device array of ds3_write_kv_noalloc
DS3_BUF_WEIGHTS, DS3_BUF_KV, DS3_BUF_WORK, DS3_BUF_LOGITS, DS3_NUM_BUFFERS = 0, 1, 2, 3, 4
DS3_INJECT_KERNEL_CHECK, DS3_INJECT_TIMEOUT_NEXT, DS3_INJECT_BARRIER_TIMEOUT = 1, 2, 3

ROLES = {"embed": 0, "attn_norm": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5, "ffn_norm": 6, "w_gate": 7, "w_up": 8,
         "w_down": 9, "final_norm": 10, "lm_head": 11}


class ds3_sampling(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("top_p", c_float), ("min_p", c_float), ("repetition_penalty", c_float),
                ("presence_penalty", c_float), ("frequency_penalty", c_float), ("top_k", c_int32),
                ("n_logprobs", c_int32), ("seed", c_uint64)]


class ds3_config(ctypes.Structure):
    _fields_ = [("abi_version", c_uint32), ("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn_dim", c_int32), ("vocab", c_int32),
                ("rms_eps", c_float), ("rope_theta", c_double), ("rows", c_int32), ("cap", c_int32),
                ("kv_layout", c_int32), ("page_size", c_int32), ("pool_pages", c_int32), ("weight_dtype", c_int32),
                ("kv_dtype", c_int32), ("exec_mode", c_int32), ("timeout_ms", c_uint32), ("kernel_plan", c_int32),
                ("trace", c_int32), ("prefill_rows", c_int32)]


class ds3_buffer_req(ctypes.Structure):
    _fields_ = [("id", c_int32), ("name", c_char * 32), ("bytes", c_uint64), ("align", c_uint32)]


class ds3_weight_src(ctypes.Structure):
    _fields_ = [("role", c_int32), ("layer", c_int32), ("dtype", c_int32), ("rows", c_int64), ("cols", c_int64),
                ("data", c_void_p)]


class ds3_stats(ctypes.Structure):
    _fields_ = [("steps", c_uint64), ("replays", c_uint64), ("captures", c_uint64), ("kernels_per_step", c_int32),
                ("state", c_int32), ("last_host_us", c_double), ("last_gpu_us", c_double),
                ("attn_splits", c_int32), ("kernel_plan", c_int32),
                ("last_submit_us", c_double), ("prefill_tokens", c_uint64), ("last_prefill_gpu_us", c_double)]


class ds3_kernel_time(ctypes.Structure):
    _fields_ = [("name", c_char * 40), ("launches", c_int32), ("total_us", c_double), ("bytes", c_double)]


# (name, restype, argtypes) for every function of include/ds3.h
SIGNATURES = [
    ("ds3_query_buffers", c_int32, [POINTER(ds3_config), POINTER(ds3_buffer_req), POINTER(c_int32)]),
    ("ds3_create", c_int32, [POINTER(ds3_config), POINTER(c_void_p), c_int32, c_void_p, POINTER(c_void_p)]),
    ("ds3_load_weights", c_int32, [c_void_p, POINTER(ds3_weight_src), c_int32]),
    ("ds3_set_slot_map", c_int32, [c_void_p, c_void_p]),
    ("ds3_step", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, POINTER(c_uint32)]),
    ("ds3_step_greedy", c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    ("ds3_set_kv_sweep", c_int32, [c_void_p, c_int32]),
    ("ds3_prefill", c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, POINTER(c_uint32)]),
    ("ds3_set_sampling", c_int32, [c_void_p, c_int32, c_void_p]),
    ("ds3_set_history", c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_void_p]),
    ("ds3_step_sample", c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    ("ds3_reset_state", c_int32, [c_void_p]),
    ("ds3_write_kv", c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    ("ds3_read_kv", c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    ("ds3_write_kv_noalloc", c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    ("ds3_stats_get", c_int32, [c_void_p, POINTER(ds3_stats)]),
    ("ds3_profile_kernels", c_int32, [c_void_p, c_int32, POINTER(ds3_kernel_time), POINTER(c_int32)]),
    ("ds3_phase_trace", c_int32, [c_void_p, POINTER(c_uint64), POINTER(c_int32)]),
    ("ds3_debug_inject", c_int32, [c_void_p, c_int32]),
    ("ds3_probe_read", c_int32, [c_void_p, ctypes.c_uint64, c_void_p, c_void_p]),
    ("ds3_last_error", ctypes.c_char_p, [c_void_p]),
    ("ds3_destroy", None, [c_void_p]),
]

_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libds3.so (built in-tree by decode_step_03_amd.build). Raises if it is missing: no fallback exists."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build the HIP library first (python -m decode_step_03_amd.build)")
    lib = ctypes.CDLL(p)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class DS3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def _check(st: int, handle=None) -> None:
    if st != DS3_OK:
        msg = load_library().ds3_last_error(handle)
        raise DS3Error(st, msg.decode() if msg else "")


# ---- thin wrappers, same names as the C ABI --------------------------------------------------------------


def ds3_query_buffers(cfg: ds3_config) -> list:
    lib = load_library()
    reqs = (ds3_buffer_req * DS3_NUM_BUFFERS)()
    n = c_int32(DS3_NUM_BUFFERS)
    _check(lib.ds3_query_buffers(ctypes.byref(cfg), reqs, ctypes.byref(n)))
    return list(reqs)[: n.value]


def ds3_create(cfg: ds3_config, dev_ptrs, stream_handle: int | None) -> int:
    lib = load_library()
    arr = (c_void_p * len(dev_ptrs))(*dev_ptrs)
    out = c_void_p()
    _check(lib.ds3_create(ctypes.byref(cfg), arr, len(dev_ptrs), c_void_p(stream_handle or 0), ctypes.byref(out)))
    return out.value


def ds3_load_weights(h: int, srcs) -> None:
    arr = (ds3_weight_src * len(srcs))(*srcs)
    _check(load_library().ds3_load_weights(h, arr, len(srcs)), h)


def ds3_set_slot_map(h: int, ptr: int) -> None:
    _check(load_library().ds3_set_slot_map(h, ptr), h)


def ds3_step(h: int, tokens_ptr: int, pos_ptr: int, write_map_ptr: int | None, logits_ptr: int | None) -> int:
    flags = c_uint32(0)
    _check(load_library().ds3_step(h, tokens_ptr, pos_ptr, write_map_ptr, logits_ptr, ctypes.byref(flags)), h)
    return flags.value


def ds3_step_greedy(h: int, tokens_ptr: int, pos_ptr: int, n_steps: int, ids_ptr: int, flags_ptr: int | None) -> None:
    _check(load_library().ds3_step_greedy(h, tokens_ptr, pos_ptr, n_steps, ids_ptr, flags_ptr), h)


def ds3_prefill(h: int, row: int, tokens_ptr: int, pos0: int, n: int, logits_ptr: int | None) -> int:
    flags = c_uint32(0)
    _check(load_library().ds3_prefill(h, row, tokens_ptr, pos0, n, logits_ptr, ctypes.byref(flags)), h)
    return flags.value


def ds3_set_sampling(h: int, row: int, params: "ds3_sampling") -> None:
    _check(load_library().ds3_set_sampling(h, row, ctypes.byref(params)), h)


def ds3_set_history(h: int, row: int, tokens_ptr: int | None, n: int, bias_ptr: int | None) -> None:
    _check(load_library().ds3_set_history(h, row, tokens_ptr, n, bias_ptr), h)


def ds3_step_sample(h: int, tokens_ptr: int, pos_ptr: int, n_steps: int, ids_ptr: int, flags_ptr: int | None,
                    lp_ptr: int | None, lp_ids_ptr: int | None) -> None:
    _check(load_library().ds3_step_sample(h, tokens_ptr, pos_ptr, n_steps, ids_ptr, flags_ptr, lp_ptr, lp_ids_ptr), h)


def ds3_set_kv_sweep(h: int, mode: int) -> None:
    _check(load_library().ds3_set_kv_sweep(h, mode), h)


def ds3_reset_state(h: int) -> None:
    _check(load_library().ds3_reset_state(h), h)


def ds3_write_kv(h: int, layer: int, row: int, pos0: int, n: int, k_ptr: int, v_ptr: int) -> None:
    _check(load_library().ds3_write_kv(h, layer, row, pos0, n, k_ptr, v_ptr), h)


def ds3_read_kv(h: int, layer: int, row: int, pos0: int, n: int, k_ptr: int, v_ptr: int) -> None:
    _check(load_library().ds3_read_kv(h, layer, row, pos0, n, k_ptr, v_ptr), h)


def ds3_write_kv_noalloc(h: int, layer: int, row: int, pos0: int, n: int, k_ptr: int, v_ptr: int) -> None:
    _check(load_library().ds3_write_kv_noalloc(h, layer, row, pos0, n, k_ptr, v_ptr), h)


def ds3_stats_get(h: int) -> ds3_stats:
    s = ds3_stats()
    _check(load_library().ds3_stats_get(h, ctypes.byref(s)), h)
    return s


def ds3_profile_kernels(h: int, iters: int) -> list:
    out = (ds3_kernel_time * 16)()
    n = c_int32(16)
    _check(load_library().ds3_profile_kernels(h, iters, out, ctypes.byref(n)), h)
    return list(out)[: n.value]


def ds3_phase_trace(h: int, n: int):
    out = (c_uint64 * n)()
    k = c_int32(n)
    _check(load_library().ds3_phase_trace(h, out, ctypes.byref(k)), h)
    return list(out)[: k.value]


def ds3_probe_read(buf_ptr: int, nbytes: int, sink_ptr: int, stream_ptr: int) -> None:
    """One streaming read of `nbytes` of device memory (measurement only; see include/ds3.h)."""
    _check(load_library().ds3_probe_read(buf_ptr, nbytes, sink_ptr, stream_ptr), None)


def ds3_debug_inject(h: int, kind: int) -> None:
    _check(load_library().ds3_debug_inject(h, kind), h)


def ds3_last_error(h: int | None) -> str:
    m = load_library().ds3_last_error(h)
    return m.decode() if m else ""


def ds3_destroy(h: int) -> None:
    load_library().ds3_destroy(h)
