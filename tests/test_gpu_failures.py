"""Failure handling of the C ABI on the GPU: typed errors, needs-reset after a failed in-kernel check, poisoning
after a timeout ("Execution" page, section "Failure handling"). Every condition is forced from the host; no kernel
faults or hangs.
"""
from dataclasses import replace

import numpy as np
import pytest

import synth
from decode_step_03_amd import DS3Error, _ds3 as C
from tests.ds3_testlib import make_engine

pytestmark = pytest.mark.gpu


def _engine(**kw):
    w = synth.workload("tiny-fp32")
    ws = synth.make_weights(w.model)
    return w, ws, make_engine(w, ws, **kw)


def test_invalid_arguments_leave_engine_usable():
    w, ws, eng = _engine()
    try:
        for tok, pos in [([w.model.vocab], [0]), ([-1], [0]), ([0], [w.cap]), ([0], [-5])]:
            with pytest.raises(DS3Error) as ei:
                eng.step(tok, pos)
            assert ei.value.status == C.DS3_E_INVALID
        eng.step([1], [0])      # still usable
        assert eng.stats()["state"] == 0
    finally:
        eng.close()


def test_kernel_check_needs_reset():
    w, ws, eng = _engine()
    try:
        eng.step([1], [0])
        eng.debug_inject(C.DS3_INJECT_KERNEL_CHECK)
        with pytest.raises(DS3Error) as ei:
            eng.step([2], [1])
        assert ei.value.status == C.DS3_E_KERNEL_CHECK
        with pytest.raises(DS3Error) as ei:
            eng.step([2], [1])
        assert ei.value.status == C.DS3_E_NEEDS_RESET
        eng.reset_state()
        eng.step([2], [0])
    finally:
        eng.close()


def test_timeout_poisons_engine():
    w, ws, eng = _engine()
    try:
        eng.step([1], [0])
        eng.debug_inject(C.DS3_INJECT_TIMEOUT_NEXT)
        with pytest.raises(DS3Error) as ei:
            eng.step([2], [1])
        assert ei.value.status == C.DS3_E_TIMEOUT
        for call in (lambda: eng.step([2], [1]), eng.reset_state, lambda: eng.read_kv(0, 0, 0, 1)):
            with pytest.raises(DS3Error) as ei:
                call()
            assert ei.value.status == C.DS3_E_POISONED
    finally:
        eng.close()


def test_unbound_and_bad_weights():
    from decode_step_03_amd import Engine
    from tests.ds3_testlib import engine_config
    w = synth.workload("tiny-fp32")
    ws = synth.make_weights(w.model)
    eng = Engine(engine_config(w))
    try:
        layers = [dict(L) for L in ws.layers]
        del layers[1]["w_up"]
        with pytest.raises(DS3Error) as ei:
            eng.load_weights(layers, ws.glob)
        assert ei.value.status == C.DS3_E_UNBOUND and "UP" in ei.value.message
        with pytest.raises(DS3Error) as ei:
            eng.step([0], [0])
        assert ei.value.status == C.DS3_E_NOT_LOADED
        layers = [dict(L) for L in ws.layers]
        layers[0]["wq"] = layers[0]["wq"][:-1]
        with pytest.raises(DS3Error) as ei:
            eng.load_weights(layers, ws.glob)
        assert ei.value.status == C.DS3_E_INVALID
        eng.load_weights(ws.layers, ws.glob)
        eng.step([0], [0])
    finally:
        eng.close()


def test_unsupported_config_is_refused_with_field():
    w = replace(synth.workload("tiny-fp32"), name="x")
    from tests.ds3_testlib import engine_config
    cfg = engine_config(w)
    cfg.head_dim = 80
    with pytest.raises(DS3Error) as ei:
        C.ds3_query_buffers(cfg)
    assert ei.value.status == C.DS3_E_UNSUPPORTED and "head_dim" in ei.value.message


def test_paged_step_needs_the_page_table_and_a_consistent_write_map():
    """A paged step reads every position through the page table: without one, every step is refused, also with an
    explicit write map; an explicit write map must be the page-table slot of pos. Nothing runs on the device."""
    base = synth.workload("llama8b-bf16-r16-paged")
    w = replace(synth.small_variant(base, n_layers=1, vocab=1024, cap=256, pool_pages=40), rows=2, name="paged-guard")
    ws = synth.make_weights(w.model)
    eng = make_engine(w, ws)
    try:
        tok, pos = np.array([1, 2], np.int32), np.array([5, 17], np.int32)
        for wm in (None, np.array([5, 17], np.int32)):
            with pytest.raises(DS3Error) as ei:
                eng.step(tok, pos, wm)
            assert ei.value.status == C.DS3_E_INVALID and "slot map" in ei.value.message
        table = np.arange(32, dtype=np.int32)[::-1].copy().reshape(2, 16)
        eng.set_slot_map(table)
        good = np.array([table[0, 0] * 16 + 5, table[1, 1] * 16 + 1], np.int32)
        with pytest.raises(DS3Error) as ei:
            eng.step(tok, pos, good + 1)
        assert ei.value.status == C.DS3_E_INVALID and "write_map" in ei.value.message
        eng.step(tok, pos, good)
        eng.step(tok, pos + 1)
        assert eng.stats()["state"] == 0
    finally:
        eng.close()
