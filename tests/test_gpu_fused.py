"""The fused step kernel (the whole batch-1 step as one persistent launch with grid barriers) against the oracle,
against the per-operation kernels, and under the properties the method fixes: replay equals eager bit for bit,
a capture serves every position, K/V garbage after the position cannot leak, and a grid barrier that outlasts its
limit ends the step with a kernel-check error instead of a hang.
"""
from dataclasses import replace

import numpy as np
import pytest

import synth
from decode_step_03_amd import DS3Error, _ds3 as C
from tests.ds3_testlib import TOL_BF16, Lockstep, log, make_engine

pytestmark = pytest.mark.gpu


def _case(n_layers=1, cap=8192, vocab=4096, gains="random"):
    base = synth.workload("llama8b-bf16-cap8192")
    w = replace(synth.small_variant(base, n_layers=n_layers, vocab=vocab, cap=cap), name=f"llama8b-{n_layers}l-cap{cap}")
    ws = synth.make_weights(w.model, gains=gains)
    return w, ws


@pytest.mark.parametrize("cap", [8192, 4096, 16384, 12288])
def test_fused_matches_oracle_and_per_op(cap):
    """8B-shaped layers (2 of them), one row: the fused kernel (one 256- or 128-position chunk per split at caps 8192
    and 4096; two 256-position and three 128-position chunks per split at 16384 and 12288, the later ones loaded in
    the attention phase) and the per-operation kernels both within 2e-2 of the oracle on every logit, positions
    spread over the capacity and across the chunk boundaries."""
    w, ws = _case(n_layers=2, cap=cap)
    f = make_engine(w, ws, kernel_plan="fused")
    o = make_engine(w, ws, kernel_plan="per_op")
    try:
        assert f.stats()["kernel_plan"] == "fused" and o.stats()["kernel_plan"] == "per_op"
        lf, lo = Lockstep(w, ws, f), Lockstep(w, ws, o)
        pre = cap // 4
        for ls in (lf, lo):
            ls.prefill_random_kv([pre])
        tok = np.array([123], np.int32)
        for p in (pre, pre + 1, pre + 2, cap - 1, 0, 255, 256, cap // 2 - 1, cap // 2, 8192 % cap + 1):
            a, ref, _ = lf.step(tok, np.array([p], np.int32))
            b, _, _ = lo.step(tok, np.array([p], np.int32))
            d = float(np.max(np.abs(a.astype(np.float64) - b)))
            assert d <= TOL_BF16, f"fused and per-op logits differ by {d:.3e} at pos {p}"
            for li in range(w.model.n_layers):
                lf.check_kv(li, 0, p, 1)
            tok = np.array([int(np.argmax(ref[0]))], np.int32)
        log(w.name, "fused max err", f"{lf.max_err:.3e}", "per-op max err", f"{lo.max_err:.3e}")
    finally:
        f.close()
        o.close()


def test_fused_replay_equals_eager_and_serves_every_position():
    """Capture at one position, replay at others: bit-identical to launching the fused kernel eagerly."""
    w, ws = _case(n_layers=1)
    g = make_engine(w, ws, "graph", kernel_plan="fused")
    e = make_engine(w, ws, "eager", kernel_plan="fused")
    try:
        for eng in (g, e):
            Lockstep(w, ws, eng).prefill_random_kv([3000])
        for p, t in [(3000, 5), (3001, 17), (4095, 9), (0, 1), (8191, 2047), (256, 3)]:
            a, _ = g.step([t], [p])
            a = a.copy()
            b, _ = e.step([t], [p])
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay differs from eager at pos {p}"
        st = g.stats()
        assert st["captures"] == 1 and st["replays"] == 6 and st["kernels_per_step"] == 1   # (greedy pick included)
    finally:
        g.close()
        e.close()


@pytest.mark.parametrize("cap,pos", [(8192, 300), (16384, 300), (16384, 9000)])
def test_fused_garbage_after_position_does_not_leak(cap, pos):
    """K/V after pos (huge values, NaN, +-inf) leave the fused kernel's logits bit-identical, whether the garbage
    sits in the chunks staged during the gate/up phase or in those loaded during the attention phase."""
    w, ws = _case(n_layers=1, cap=cap)
    eng = make_engine(w, ws, kernel_plan="fused")
    try:
        ls = Lockstep(w, ws, eng)
        ls.prefill_random_kv([pos])
        clean, _ = eng.step([7], [pos])
        clean = clean.copy()
        rng = np.random.default_rng(1)
        n = 2000
        nkv, hd = w.model.n_kv_heads, w.model.head_dim
        huge = synth.f32_to_bf16_words((rng.standard_normal((nkv, n, hd)) * 1e4).astype(np.float32))
        specials = np.array([0x7fc0, 0x7f80, 0xff80], np.uint16)      # NaN, +inf, -inf
        weird = rng.choice(specials, (nkv, n, hd))
        for garbage in (huge, weird):
            eng.write_kv(0, 0, pos + 1, garbage, garbage)
            eng.write_kv(0, 0, w.cap - n, garbage, garbage)
            ls.prefill_random_kv([pos])
            got, flags = eng.step([7], [pos])
            assert flags == 0
            assert np.array_equal(got.view(np.uint32), clean.view(np.uint32))
    finally:
        eng.close()


def test_fused_barrier_timeout_needs_reset():
    """A grid-barrier wait limit of one tick (forced from the host): the step ends with DS3_E_KERNEL_CHECK, the
    engine needs a reset, and after the reset the fused kernel is back in parity with the oracle."""
    w, ws = _case(n_layers=1)
    eng = make_engine(w, ws, kernel_plan="fused")
    try:
        ls = Lockstep(w, ws, eng)
        ls.prefill_random_kv([100])
        ls.step(np.array([3], np.int32), np.array([100], np.int32))
        eng.debug_inject(C.DS3_INJECT_BARRIER_TIMEOUT)
        with pytest.raises(DS3Error) as ei:
            eng.step([3], [101])
        assert ei.value.status == C.DS3_E_KERNEL_CHECK
        with pytest.raises(DS3Error) as ei:
            eng.step([3], [101])
        assert ei.value.status == C.DS3_E_NEEDS_RESET
        eng.reset_state()
        ls2 = Lockstep(w, ws, eng)
        ls2.prefill_random_kv([100])
        for p in (100, 101, 102):
            ls2.step(np.array([3], np.int32), np.array([p], np.int32))
    finally:
        eng.close()


def test_fused_profile_reports_phases_and_restores_state():
    """Profiling the fused plan: one kernel per step, and a positive share for each phase kind."""
    w, ws = _case(n_layers=2)
    eng = make_engine(w, ws, kernel_plan="fused")
    try:
        ls = Lockstep(w, ws, eng)
        ls.prefill_random_kv([500])
        tok = np.array([9], np.int32)
        _, ref, _ = ls.step(tok, np.array([500], np.int32))
        kinds = {k["name"]: k for k in eng.profile_kernels(3)}
        assert kinds["decode_step_fused"]["launches"] == 1 and kinds["decode_step_fused"]["us_per_step"] > 0
        for name in ("qkv_rope_kvwrite", "attention_splitk", "o_proj_residual", "gateup_swiglu",
                     "down_proj_residual"):
            assert kinds[name]["launches"] == w.model.n_layers and kinds[name]["us_per_step"] > 0, kinds[name]
        assert kinds["lm_head"]["launches"] == 1 and kinds["lm_head"]["us_per_step"] > 0
        ls.check_kv(1, 0, 500, 1)
        tok = np.array([int(np.argmax(ref[0]))], np.int32)
        ls.step(tok, np.array([501], np.int32))
    finally:
        eng.close()


def test_fused_phase_trace_records_barriers_and_leaves_results_alone():
    """A traced engine (the separately compiled, traced step kernel) gives the untraced engine's logits bit for
    bit; its barrier trace has, for every block and barrier, arrival <= release, releases in barrier order, every
    block released only after the last block arrived (after the QKV phase: the last block of its kv-head group);
    its GEMV sub-phase clocks are in order. An
    untraced engine refuses the trace."""
    w, ws = _case(n_layers=2)
    plain = make_engine(w, ws, kernel_plan="fused")
    traced = make_engine(w, ws, kernel_plan="fused", trace="phases")
    try:
        for eng in (plain, traced):
            ls = Lockstep(w, ws, eng)
            ls.prefill_random_kv([700])
        tok = np.array([5], np.int32)
        for p in (700, 701):
            a, _ = plain.step(tok, np.array([p], np.int32))
            b, _ = traced.step(tok, np.array([p], np.int32))
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"traced logits differ at pos {p}"
            tok = np.array([int(np.argmax(a[0]))], np.int32)
        bar, sub = traced.phase_trace(sub_phases=True)
        nb = 5 * w.model.n_layers
        assert bar.shape == (nb, 256, 2) and sub.shape == (nb, 256, 8)
        arr, rel = bar[..., 0].astype(np.int64), bar[..., 1].astype(np.int64)
        assert (arr > 0).all() and (arr <= rel).all()
        assert (np.diff(rel, axis=0) >= 0).all(), "releases out of barrier order"
        grid = [i for i in range(nb) if i % 5 != 0]   # the QKV phase closes with a wait of each kv-head group
        assert (rel[grid].min(axis=1) >= arr[grid].max(axis=1)).all(), "a block was released before every block arrived"
        qa = arr[0::5].reshape(w.model.n_layers, 8, 32)
        qr = rel[0::5].reshape(w.model.n_layers, 8, 32)
        assert (qr.min(axis=2) >= qa.max(axis=2)).all(), "a group's attention began before its QKV blocks arrived"
        for ph in (0, 2, 3, 4):   # GEMV phases: start, first batch consumed, batches done, block done
            st = sub[ph::5, :, :4].astype(np.int64)
            assert (st > 0).all() and (np.diff(st, axis=2) >= 0).all()
        with pytest.raises(DS3Error) as ei:
            plain.phase_trace()
        assert ei.value.status == C.DS3_E_UNSUPPORTED
    finally:
        plain.close()
        traced.close()
