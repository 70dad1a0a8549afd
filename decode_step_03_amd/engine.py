"""Python face of libds3.so: allocate the device buffers with PyTorch, hand them to the library, marshal calls.

PyTorch provides device memory and a stream here and nothing else; every computation of the step runs inside the
library's HIP kernels. The executor contract follows the poot documentation's "Execution" page, section
"Per backend" (load_weights, step, reset_state, stats, unload).
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _ds3 as C


def make_config(*, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps, rope_theta, rows,
                cap, kv_layout="contiguous", page_size=0, pool_pages=0, weight_dtype="bf16", kv_dtype="bf16",
                exec_mode="graph", timeout_ms=0, kernel_plan="auto", trace="off", prefill_rows=0) -> C.ds3_config:
    dt = {"f32": C.DS3_F32, "bf16": C.DS3_BF16}
    return C.ds3_config(
        C.DS3_ABI_VERSION, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps, rope_theta,
        rows, cap, C.DS3_KV_PAGED if kv_layout == "paged" else C.DS3_KV_CONTIGUOUS, page_size, pool_pages,
        dt[weight_dtype], dt[kv_dtype], C.DS3_EAGER if exec_mode == "eager" else C.DS3_GRAPH, timeout_ms,
        {"auto": C.DS3_PLAN_AUTO, "per_op": C.DS3_PLAN_PER_OP, "fused": C.DS3_PLAN_FUSED}[kernel_plan],
        {"off": C.DS3_TRACE_OFF, "barriers": C.DS3_TRACE_BARRIERS, "phases": C.DS3_TRACE_PHASES}[trace],
        prefill_rows)


class Engine:
    """One decode-step engine on one GPU: fixed rows, capacity and KV layout; weights loaded once."""

    def __init__(self, cfg: C.ds3_config, device: str = "cuda:0"):
        import torch
        self.cfg = cfg
        self.rows, self.vocab = cfg.rows, cfg.vocab
        self.device = torch.device(device)
        self._torch = torch
        reqs = C.ds3_query_buffers(cfg)
        with torch.cuda.device(self.device):
            self.buffers = [torch.empty(max(int(r.bytes), 256), dtype=torch.uint8, device=self.device) for r in reqs]
            self.stream = torch.cuda.Stream(self.device)
            torch.cuda.synchronize(self.device)
            self.handle = C.ds3_create(cfg, [b.data_ptr() for b in self.buffers], self.stream.cuda_stream)
        self.logits_device = self.buffers[C.DS3_BUF_LOGITS][: 4 * self.rows * self.vocab].view(torch.float32).view(
            self.rows, self.vocab)
        self._logits_host = torch.empty((self.rows, self.vocab), dtype=torch.float32, pin_memory=True)
        self._tok = np.zeros(self.rows, np.int32)
        self._pos = np.zeros(self.rows, np.int32)
        self._wm = np.zeros(self.rows, np.int32)

    # -- contract ------------------------------------------------------------------------------------------

    def load_weights(self, layers: list, glob: dict) -> None:
        """Bind weights by role: `layers[l][role]` and `glob[role]` are numpy arrays (bf16 words or float32)."""
        dtype = self.cfg.weight_dtype
        srcs, keep = [], []

        def add(role, layer, arr):
            a = np.ascontiguousarray(arr)
            keep.append(a)
            rows, cols = (1, a.shape[0]) if a.ndim == 1 else a.shape
            srcs.append(C.ds3_weight_src(C.ROLES[role], layer, dtype, rows, cols, a.ctypes.data))

        for li, L in enumerate(layers):
            for role, arr in L.items():
                add(role, li, arr)
        for role, arr in glob.items():
            add(role, -1, arr)
        C.ds3_load_weights(self.handle, srcs)

    def set_slot_map(self, slot_map: np.ndarray) -> None:
        a = np.ascontiguousarray(slot_map, dtype=np.int32)
        C.ds3_set_slot_map(self.handle, a.ctypes.data)

    def step(self, tokens, pos, write_map=None, copy_logits: bool = True):
        """One decode step. Returns (logits float32 [rows, vocab] numpy view of pinned memory or None, flags)."""
        self._tok[:] = tokens
        self._pos[:] = pos
        wm = None
        if write_map is not None:
            self._wm[:] = write_map
            wm = self._wm.ctypes.data
        out = self._logits_host.data_ptr() if copy_logits else None
        flags = C.ds3_step(self.handle, self._tok.ctypes.data, self._pos.ctypes.data, wm, out)
        return (self._logits_host.numpy() if copy_logits else None), flags

    def step_greedy(self, tokens, pos, n_steps: int):
        """n_steps chained steps with the greedy pick on the device and one host wait. Returns (ids int32
        [n_steps, rows], flags uint32 [n_steps]); step 0 takes `tokens` at `pos`, step i the previous pick at pos + i."""
        self._tok[:] = tokens
        self._pos[:] = pos
        ids = np.empty((n_steps, self.cfg.rows), np.int32)
        flags = np.empty(n_steps, np.uint32)
        C.ds3_step_greedy(self.handle, self._tok.ctypes.data, self._pos.ctypes.data, n_steps, ids.ctypes.data,
                          flags.ctypes.data)
        return ids, flags

    def prefill(self, row: int, tokens, pos0: int):
        """Prefill: tokens (int32 [n]) of row `row` at positions pos0 .. pos0 + n - 1, prefill_rows per launch.
        Returns (logits float32 [vocab] of the last token, flags)."""
        toks = np.ascontiguousarray(np.asarray(tokens, np.int32))
        out = np.empty(self.cfg.vocab, np.float32)
        flags = C.ds3_prefill(self.handle, row, toks.ctypes.data, pos0, toks.size, out.ctypes.data)
        return out, flags

    def set_sampling(self, row: int, *, temperature=0.0, top_k=0, top_p=1.0, min_p=0.0, repetition_penalty=1.0,
                     presence_penalty=0.0, frequency_penalty=0.0, n_logprobs=0, seed=0) -> None:
        C.ds3_set_sampling(self.handle, row, C.ds3_sampling(temperature, top_p, min_p, repetition_penalty,
                                                            presence_penalty, frequency_penalty, top_k, n_logprobs,
                                                            seed))

    def set_history(self, row: int, tokens=(), bias=None) -> None:
        toks = np.ascontiguousarray(np.asarray(tokens, np.int32))
        b = None if bias is None else np.ascontiguousarray(np.asarray(bias, np.float32))
        C.ds3_set_history(self.handle, row, toks.ctypes.data if toks.size else None, toks.size,
                          None if b is None else b.ctypes.data)

    def step_sample(self, tokens, pos, n_steps: int):
        """n_steps chained steps, each row's token drawn by the sampling suffix. Returns (ids [n, rows], flags [n],
        logprobs [n, rows, 1 + 8] (drawn token's, then top n), logprob ids [n, rows, 8])."""
        self._tok[:] = tokens
        self._pos[:] = pos
        R = self.cfg.rows
        ids = np.empty((n_steps, R), np.int32)
        flags = np.empty(n_steps, np.uint32)
        lp = np.empty((n_steps, R, 1 + C.DS3_MAX_LOGPROBS), np.float32)
        lpi = np.empty((n_steps, R, C.DS3_MAX_LOGPROBS), np.int32)
        C.ds3_step_sample(self.handle, self._tok.ctypes.data, self._pos.ctypes.data, n_steps, ids.ctypes.data,
                          flags.ctypes.data, lp.ctypes.data, lpi.ctypes.data)
        return ids, flags, lp, lpi

    def set_kv_sweep(self, mode: str) -> None:
        """"full" (the method: every position of [cap] is loaded) or "visible" (chunks wholly after pos are skipped;
        outputs bit-identical)."""
        C.ds3_set_kv_sweep(self.handle, {"full": C.DS3_SWEEP_FULL, "visible": C.DS3_SWEEP_VISIBLE}[mode])

    def reset_state(self) -> None:
        C.ds3_reset_state(self.handle)

    def write_kv(self, layer: int, row: int, pos0: int, k: np.ndarray, v: np.ndarray) -> None:
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        C.ds3_write_kv(self.handle, layer, row, pos0, k.shape[1], k.ctypes.data, v.ctypes.data)

    def write_kv_noalloc(self, layer: int, row: int, pos0: int, k: np.ndarray, v: np.ndarray) -> None:
        """As write_kv, staged through the library's fixed device array (no allocation; see include/ds3.h)."""
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        C.ds3_write_kv_noalloc(self.handle, layer, row, pos0, k.shape[1], k.ctypes.data, v.ctypes.data)

    def read_kv(self, layer: int, row: int, pos0: int, n: int):
        dt = np.uint16 if self.cfg.kv_dtype == C.DS3_BF16 else np.float32
        shape = (self.cfg.n_kv_heads, n, self.cfg.head_dim)
        k, v = np.empty(shape, dt), np.empty(shape, dt)
        C.ds3_read_kv(self.handle, layer, row, pos0, n, k.ctypes.data, v.ctypes.data)
        return k, v

    def stats(self) -> dict:
        s = C.ds3_stats_get(self.handle)
        d = {f: getattr(s, f) for f, _ in s._fields_}
        d["kernel_plan"] = {C.DS3_PLAN_PER_OP: "per_op", C.DS3_PLAN_FUSED: "fused"}.get(d["kernel_plan"], "?")
        return d

    def profile_kernels(self, iters: int = 5) -> list:
        return [{"name": k.name.decode(), "launches": k.launches, "us_per_step": k.total_us, "bytes_per_step": k.bytes}
                for k in C.ds3_profile_kernels(self.handle, iters)]

    def phase_trace(self, sub_phases: bool = False):
        """Fused plan: [barriers, blocks, 2] arrival / release clock ticks (100 MHz) of the last step; with
        sub_phases also [barriers, blocks, 8] sub-phase ticks (zero unless created with trace="phases"). Needs an
        engine created with trace="barriers" or "phases"."""
        nb = 5 * self.cfg.n_layers
        n = nb * 256 * 2
        a = np.array(C.ds3_phase_trace(self.handle, 5 * n if sub_phases else n), dtype=np.uint64)
        bar = a[:n].reshape(nb, 256, 2)
        return (bar, a[n:].reshape(nb, 256, 8)) if sub_phases else bar

    def debug_inject(self, kind: int) -> None:
        C.ds3_debug_inject(self.handle, kind)

    def last_error(self) -> str:
        return C.ds3_last_error(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            C.ds3_destroy(self.handle)
            self.handle = None
            self.buffers = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
