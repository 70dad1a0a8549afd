"""Shared helpers of the GPU parity tests: build an engine and an oracle model from the same seeded inputs.

Inputs come only from `synth` (seeded draws); expected values come only from `oracle`. The two sides share no
arithmetic.
"""
from __future__ import annotations

import functools
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

# Tolerances stated for the decode step: logits max-abs 1e-4 with fp32 weights, 2e-2 with bf16 weights (fp32
# accumulate); greedy ids must match wherever the oracle's top-2 margin exceeds 5e-2.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
GREEDY_MARGIN = 5e-2


def log(*a):
    print("[ds3-test]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def weights(model: synth.ModelShape, gains: str = "ones") -> synth.WeightSet:
    """The seeded weights of `model`, drawn once per test session (the 8B shape's 16 GB serve every test of it)."""
    t0 = time.time()
    ws = synth.make_weights(model, gains=gains)
    log(f"weights of {model.name} ({model.n_layers} layers) drawn in {time.time() - t0:.1f}s")
    return ws


def logits_tol(w: synth.Workload) -> float:
    return TOL_F32 if w.model.weight_dtype == "f32" else TOL_BF16


def engine_config(w: synth.Workload, exec_mode="graph", timeout_ms=0, rows=None, cap=None, kernel_plan="auto",
                  trace="off", prefill_rows=0):
    from decode_step_03_amd import make_config
    m = w.model
    return make_config(n_layers=m.n_layers, d_model=m.d_model, n_q_heads=m.n_q_heads, n_kv_heads=m.n_kv_heads,
                       head_dim=m.head_dim, ffn_dim=m.ffn_dim, vocab=m.vocab, rms_eps=m.rms_eps,
                       rope_theta=m.rope_theta, rows=rows or w.rows, cap=cap or w.cap, kv_layout=w.kv_layout,
                       page_size=w.page_size, pool_pages=w.pool_pages, weight_dtype=m.weight_dtype,
                       kv_dtype=w.kv_dtype, exec_mode=exec_mode, timeout_ms=timeout_ms, kernel_plan=kernel_plan,
                       trace=trace, prefill_rows=prefill_rows)


def make_engine(w: synth.Workload, ws: synth.WeightSet, exec_mode="graph", timeout_ms=0, kernel_plan="auto",
                trace="off", prefill_rows=0):
    from decode_step_03_amd import Engine
    eng = Engine(engine_config(w, exec_mode, timeout_ms, kernel_plan=kernel_plan, trace=trace,
                               prefill_rows=prefill_rows))
    eng.load_weights(ws.layers, ws.glob)
    return eng


def kv_value_tol(oracle_vals: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Per-element K/V state tolerance: 1e-4 for float32 state; for bf16 state max(2e-2, one bf16 ulp)."""
    if kv_dtype == "f32":
        return np.full(oracle_vals.shape, TOL_F32)
    mag = np.abs(oracle_vals)
    ulp = np.where(mag > 0, np.ldexp(1.0, np.frexp(mag)[1] - 8), 0.0)
    return np.maximum(TOL_BF16, ulp)


def kv_to_f64(a: np.ndarray) -> np.ndarray:
    return oracle.widen(a)


class Lockstep:
    """Runs the engine and the oracle side by side, teacher-forced by the oracle's greedy token."""

    def __init__(self, w: synth.Workload, ws: synth.WeightSet, engine, n_alloc=None):
        """n_alloc: positions the oracle's cache holds per row (an int for every row, or one per row); the
        capacity when None."""
        self.w, self.ws, self.engine = w, ws, engine
        self.model = oracle.OracleModel.from_weightset(ws)
        per_row = [n_alloc or w.cap] * w.rows if not hasattr(n_alloc, "__len__") else list(n_alloc)
        self.caches = [oracle.RowCache(self.model, int(n), w.kv_dtype) for n in per_row]
        self.max_err = 0.0
        self.greedy_checked = 0
        self.greedy_flips_inside_margin = 0

    def prefill_random_kv(self, n_pos_per_row, seed=0):
        """K/V contents ~ N(0,1) (stored in the KV dtype) at positions [0, n) of every row and layer, both sides.
        The draws run on a thread pool (a window of jobs at a time); the engine and the oracle take them in order."""
        jobs = [(li, r, int(n)) for r, n in enumerate(n_pos_per_row) if n > 0 for li in range(self.w.model.n_layers)]

        def gen(job):
            li, r, n = job
            return li, r, synth.kv_prefill(self.w, li, r, "k", n, seed), synth.kv_prefill(self.w, li, r, "v", n, seed)

        t0 = time.time()
        window = 32
        with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
            for lo in range(0, len(jobs), window):
                for li, r, K, V in ex.map(gen, jobs[lo:lo + window]):
                    self.engine.write_kv(li, r, 0, K, V)
                    self.caches[r].set(li, 0, K, V)
        if len(jobs) > 64:
            log(f"K/V pre-filled for {len(jobs)} (layer, row) pairs in {time.time() - t0:.1f}s")

    def step(self, tokens, pos, write_map=None, check=True):
        t0 = time.time()
        got, flags = self.engine.step(tokens, pos, write_map)
        got = got.copy()
        t1 = time.time()
        ref = oracle.decode_rows(self.model, self.caches, [int(t) for t in tokens], [int(p) for p in pos])
        t2 = time.time()
        if check:
            self.check_logits(got, ref, flags)
        return got, ref, (t1 - t0, t2 - t1)

    def check_logits(self, got, ref, flags):
        assert np.all(np.isfinite(ref)), "oracle logits not finite"
        assert flags == 0 and np.all(np.isfinite(got)), "non-finite GPU logits where the oracle is finite"
        err = float(np.max(np.abs(got.astype(np.float64) - ref)))
        self.max_err = max(self.max_err, err)
        tol = logits_tol(self.w)
        assert err <= tol, f"logits max-abs error {err:.3e} > {tol:.1e}"
        for r in range(ref.shape[0]):
            gi, m = oracle.greedy(ref[r])
            if m > GREEDY_MARGIN:
                assert int(np.argmax(got[r])) == gi, f"greedy id differs with oracle margin {m:.3f}"
                self.greedy_checked += 1
            elif int(np.argmax(got[r])) != gi:
                self.greedy_flips_inside_margin += 1

    def check_kv(self, layer, row, pos0, n):
        k, v = self.engine.read_kv(layer, row, pos0, n)
        for got, ref in ((k, self.caches[row].K[layer][:, pos0:pos0 + n]), (v, self.caches[row].V[layer][:, pos0:pos0 + n])):
            g = kv_to_f64(got)
            rf = ref.astype(np.float64)
            tol = kv_value_tol(rf, self.w.kv_dtype)
            bad = np.abs(g - rf) > tol
            assert not np.any(bad), f"KV state differs: max {np.max(np.abs(g - rf)):.3e}"
            assert np.all(np.isfinite(g))
