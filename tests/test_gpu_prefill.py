"""Multi-token prefill (ds3_prefill): a prompt of one row goes prefill_rows tokens per launch sequence, every token
of a chunk an activation row of the same K/V row. Against the oracle fed the same tokens one decode step at a
time (a prefill is steps at consecutive absolute positions): the last token's logits within
the stated tolerance and its greedy id outside the margin, the K/V of every prompt position, and decoding after
the prefill staying in parity. Chunks of 16 tokens run the projections on the matrix cores with one 16-row
activation tile, chunks of 17..64 with four (a 40-token chunk pads 24 rows), chunks of up to 4 on the GEMV kernels;
the last chunk may be partial, and a chunk may sweep the whole capacity or only the visible positions.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from decode_step_03_amd import DS3Error, _ds3 as C
from tests.ds3_testlib import GREEDY_MARGIN, Lockstep, log, logits_tol, make_engine

pytestmark = pytest.mark.gpu


def _check_last(w, got, ref):
    tol = logits_tol(w)
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    assert err <= tol, f"last-token logits max-abs error {err:.3e} > {tol:.1e}"
    gi, m = oracle.greedy(ref)
    if m > GREEDY_MARGIN:
        assert int(np.argmax(got)) == gi
    return err


@pytest.mark.parametrize("case", ["1b-mfma16", "1b-mfma64", "1b-mfma64-visible", "1b-mfma40", "tiny-gemv3",
                                  "1b-paged16", "8b-paged64"])
def test_prefill_matches_oracle_then_decodes(case):
    sweep = "visible" if case.endswith("visible") else "full"
    if case.startswith("1b-mfma"):
        base = synth.workload("llama1b-bf16")
        w = replace(synth.small_variant(base, n_layers=2, vocab=4096), name="llama1b-2l-prefill")
        T, row, pos0, n = {"1b-mfma16": (16, 0, 0, 40), "1b-mfma64": (64, 0, 0, 150),
                           "1b-mfma64-visible": (64, 0, 0, 150), "1b-mfma40": (40, 0, 30, 90)}[case]
    elif case == "tiny-gemv3":
        w = synth.workload("tiny-fp32")
        T, row, pos0, n = 3, 0, 5, 20
    else:
        base = synth.workload("llama8b-bf16-r16-paged")
        w = replace(synth.small_variant(base, n_layers=1, vocab=4096, rows=2, cap=1024, pool_pages=256),
                    name="llama8b-r2-paged-prefill")
        T, row, pos0, n = (16, 1, 100, 37) if case == "1b-paged16" else (64, 1, 100, 100)
    ws = synth.make_weights(w.model)
    eng = make_engine(w, ws, prefill_rows=T)
    try:
        eng.set_kv_sweep(sweep)
        ls = Lockstep(w, ws, eng)
        if w.kv_layout == "paged":
            eng.set_slot_map(synth.page_table(w))
        if pos0:
            ls.prefill_random_kv([pos0 if r == row else 0 for r in range(w.rows)])
        toks = np.random.default_rng(7).integers(0, w.model.vocab, size=n).astype(np.int32)
        got, flags = eng.prefill(row, toks, pos0)
        assert flags == 0
        ref = None
        for i in range(n):
            ref = oracle.decode_step(ls.model, ls.caches[row], int(toks[i]), pos0 + i)
        err = _check_last(w, got, ref)
        for li in range(w.model.n_layers):
            ls.check_kv(li, row, pos0, n)
        st = eng.stats()
        assert st["prefill_tokens"] == n and st["last_prefill_gpu_us"] > 0
        log(case, "last-token err", err, "prefill us", st["last_prefill_gpu_us"])
        # decoding continues from the prefill (rows other than `row` stay where they were)
        if w.rows == 1:
            tok = np.array([int(np.argmax(ref))], np.int32)
            for i in range(3):
                _, r2, _ = ls.step(tok, np.array([pos0 + n + i], np.int32))
                tok = np.array([int(np.argmax(r2[0]))], np.int32)
    finally:
        eng.close()


def test_prefill_refusals():
    w = synth.workload("tiny-fp32")
    ws = synth.make_weights(w.model)
    eng = make_engine(w, ws)
    try:
        with pytest.raises(DS3Error) as ei:
            eng.prefill(0, [1, 2, 3], 0)
        assert ei.value.status == C.DS3_E_UNSUPPORTED
    finally:
        eng.close()
    eng = make_engine(w, ws, prefill_rows=4)
    try:
        for row, toks, pos0 in ((1, [1], 0), (0, [w.model.vocab], 0), (0, [1, 2], w.cap - 1)):
            with pytest.raises(DS3Error) as ei:
                eng.prefill(row, toks, pos0)
            assert ei.value.status == C.DS3_E_INVALID
        logits, flags = eng.prefill(0, [1, 2, 3, 4, 5], 0)   # still usable
        assert logits.shape == (w.model.vocab,) and flags == 0
    finally:
        eng.close()
