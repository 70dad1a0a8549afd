"""The visible K/V sweep (ds3_set_kv_sweep VISIBLE): chunks wholly after pos are neither loaded nor computed. A
hidden position contributes nothing under the mask, so every output must be bit-identical to the full sweep of
the method, on every attention kernel: the vector one (fp32 K/V), the matrix-core one (bf16, contiguous and
paged) and the fused step kernel. Switching is a slot word: one capture serves both modes.
"""
from dataclasses import replace

import numpy as np
import pytest

import bench
import synth
from decode_step_03_amd import DS3Error, _ds3 as C
from tests.ds3_testlib import Lockstep, log, make_engine

pytestmark = pytest.mark.gpu


def _workload(name):
    if name == "tiny-fp32":
        return synth.workload("tiny-fp32")
    if name == "8b-fused":
        base = synth.workload("llama8b-bf16-cap8192")
        return replace(synth.small_variant(base, n_layers=2, vocab=4096), name="llama8b-2l-sweep")
    if name == "8b-fused-cap16384":   # two chunks per split, the second loaded in the attention phase
        base = synth.workload("llama8b-bf16-cap8192")
        return replace(synth.small_variant(base, n_layers=2, vocab=4096, cap=16384), name="llama8b-2l-sweep-16k")
    if name == "8b-r8":
        base = synth.workload("llama8b-bf16-r8-cap32768")
        return replace(synth.small_variant(base, n_layers=1, vocab=4096, cap=8192), name="llama8b-r8-sweep")
    if name == "8b-r16-paged":
        base = synth.workload("llama8b-bf16-r16-paged")
        return replace(synth.small_variant(base, n_layers=1, vocab=4096), name="llama8b-r16-paged-sweep")
    raise KeyError(name)


@pytest.mark.parametrize("name", ["tiny-fp32", "8b-fused", "8b-fused-cap16384", "8b-r8", "8b-r16-paged"])
def test_visible_sweep_is_bit_identical(name):
    w = _workload(name)
    ws = synth.make_weights(w.model)
    full = make_engine(w, ws)
    vis = make_engine(w, ws)
    try:
        sp = np.minimum(synth.start_positions(w), w.cap - 8).astype(np.int32)
        tok = synth.start_tokens(w)
        for e in (full, vis):
            bench.prefill(e, w, sp)
        vis.set_kv_sweep("visible")
        t = tok.copy()
        for i in range(3):
            a, fa = full.step(t, sp + i)
            b, fb = vis.step(t, sp + i)
            assert fa == fb == 0
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"step {i}: logits differ"
            t = a.argmax(axis=1).astype(np.int32)
        ia, _ = full.step_greedy(t, sp + 3, 4)
        ib, _ = vis.step_greedy(t, sp + 3, 4)
        assert np.array_equal(ia, ib)
        vis.set_kv_sweep("full")   # and back, on the same capture
        a, _ = full.step(ia[-1], sp + 7)
        b, _ = vis.step(ib[-1], sp + 7)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert vis.stats()["captures"] == 1
        log(name, "plan", full.stats()["kernel_plan"], "positions", sp.tolist()[:4])
        with pytest.raises(DS3Error) as ei:
            C.ds3_set_kv_sweep(vis.handle, 7)
        assert ei.value.status == C.DS3_E_INVALID
    finally:
        full.close()
        vis.close()


@pytest.mark.parametrize("name", ["8b-fused", "8b-r8", "8b-r16-paged"])
def test_visible_sweep_follows_oracle(name):
    """The visible sweep against the oracle itself (not only against the GPU's full sweep): teacher-forced steps of
    the fused, matrix-core contiguous and paged engines with the sweep set to VISIBLE, every logit within the
    tolerance, greedy ids outside the margin, and this step's K/V in the cache."""
    w = _workload(name)
    ws = synth.make_weights(w.model)
    eng = make_engine(w, ws)
    try:
        eng.set_kv_sweep("visible")
        sp = np.minimum(synth.start_positions(w), 1500).astype(np.int32)
        n = 3
        ls = Lockstep(w, ws, eng, n_alloc=[int(p) + n for p in sp])
        if w.kv_layout == "paged":
            eng.set_slot_map(synth.page_table(w))
        ls.prefill_random_kv([int(p) for p in sp])
        t = synth.start_tokens(w)
        for i in range(n):
            _, ref, _ = ls.step(t, sp + i)
            t = ref.argmax(axis=1).astype(np.int32)
        for r in range(w.rows):
            ls.check_kv(0, r, int(sp[r]), n)
        log(name, "plan", eng.stats()["kernel_plan"], "visible-sweep max err", ls.max_err)
    finally:
        eng.close()
