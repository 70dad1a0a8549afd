"""The on-device greedy pick and chained steps (ds3_step_greedy): n steps per host wait, each step's token the
previous step's pick. The picks must equal the host's argmax of the same engine's logits bit for bit (both take
the first index of the largest float32 logit), follow the oracle's greedy tokens wherever its top-2 margin is
wide, and leave the K/V state and the slots as the same steps taken one by one would.
"""
from dataclasses import replace

import numpy as np
import pytest

import bench
import oracle
import synth
from decode_step_03_amd import DS3Error, _ds3 as C
from tests.ds3_testlib import GREEDY_MARGIN, Lockstep, log, make_engine

pytestmark = pytest.mark.gpu


def _workload(name):
    if name == "tiny-fp32":
        w = synth.workload("tiny-fp32")
    elif name == "8b-fused":
        base = synth.workload("llama8b-bf16-cap8192")
        w = replace(synth.small_variant(base, n_layers=2, vocab=4096), name="llama8b-2l-greedy")
    elif name == "8b-r16-paged":
        base = synth.workload("llama8b-bf16-r16-paged")
        w = replace(synth.small_variant(base, n_layers=1, vocab=4096), name="llama8b-r16-paged-1l-greedy")
    else:
        raise KeyError(name)
    return w, synth.make_weights(w.model)


def _setup(w, ws, eng):
    sp = synth.start_positions(w)
    bench.prefill(eng, w, sp)
    return sp, synth.start_tokens(w)


@pytest.mark.parametrize("name", ["tiny-fp32", "8b-fused", "8b-r16-paged"])
def test_chained_picks_equal_host_argmax(name):
    """ds3_step_greedy(n) on one engine against n ds3_step calls plus host argmax on a second engine with the same
    state: identical ids at every step, no non-finite flag; then both continue with a host-driven step and give
    bit-identical logits (the chain left the same K/V state)."""
    w, ws = _workload(name)
    n = 6
    a = make_engine(w, ws)
    b = make_engine(w, ws)
    try:
        sp, tok = _setup(w, ws, a)
        _setup(w, ws, b)
        ids, flags = a.step_greedy(tok, sp, n)
        assert ids.shape == (n, w.rows) and flags.shape == (n,)
        assert not flags.any()
        t = tok.copy()
        for i in range(n):
            lg, fl = b.step(t, sp + i)
            host = lg.argmax(axis=1).astype(np.int32)
            assert fl == 0
            assert np.array_equal(ids[i], host), f"step {i}: device picks {ids[i]} != host argmax {host}"
            t = host
        la, _ = a.step(t, sp + n)
        lb, _ = b.step(t, sp + n)
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
        st = a.stats()
        log(name, "plan", st["kernel_plan"], "kernels/step", st["kernels_per_step"])
    finally:
        a.close()
        b.close()


def test_chained_picks_follow_oracle_and_kv():
    """The fused plan's chain against the oracle: at every step the oracle's logits at the device's token and
    position; the device pick equals the oracle's greedy id wherever the oracle's top-2 margin exceeds the margin
    rule's; the K/V written by the chain matches the oracle's."""
    w, ws = _workload("8b-fused")
    eng = make_engine(w, ws)
    try:
        ls = Lockstep(w, ws, eng)
        p0 = 900
        ls.prefill_random_kv([p0])
        tok = 17
        n = 5
        ids, flags = eng.step_greedy([tok], [p0], n)
        assert not flags.any()
        checked = 0
        for i in range(n):
            ref = oracle.decode_step(ls.model, ls.caches[0], tok, p0 + i)
            gi, m = oracle.greedy(ref)
            if m > GREEDY_MARGIN:
                assert int(ids[i, 0]) == gi, f"step {i}: pick {ids[i, 0]} != oracle {gi} (margin {m:.3f})"
                checked += 1
            tok = int(ids[i, 0])
        for li in range(w.model.n_layers):
            ls.check_kv(li, 0, p0, n)
        log("greedy checked", checked, "of", n)
    finally:
        eng.close()


def test_chain_refuses_bad_lengths():
    w, ws = _workload("tiny-fp32")
    eng = make_engine(w, ws)
    try:
        sp, tok = _setup(w, ws, eng)
        for n in (0, C.DS3_MAX_CHAIN + 1):
            with pytest.raises(DS3Error) as ei:
                eng.step_greedy(tok, sp, n)
            assert ei.value.status == C.DS3_E_INVALID
        with pytest.raises(DS3Error) as ei:   # would pass the capacity
            eng.step_greedy(tok, np.full(w.rows, w.cap - 2, np.int32), 3)
        assert ei.value.status == C.DS3_E_INVALID
        ids, _ = eng.step_greedy(tok, sp, 1)   # still usable
        assert ids.shape == (1, w.rows)
    finally:
        eng.close()
