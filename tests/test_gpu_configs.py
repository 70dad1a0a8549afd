"""Parity at the workloads' own sizes, all layers, against the CPU oracle, through the C ABI and in the launch
configuration bench.py times (HIP-graph replay, the engine's own kernel plan and split plan):

* the 1B-shaped decoder (16 layers, vocab 32000, cap 4096): the 512-token random prompt through ds3_prefill in
  64-token chunks (matrix-core projections, four activation tiles), checked against a causal forward of the whole
  prompt (last-token
  logits, the K/V of every prompt position at the first and last layer), then greedy decode steps on the fused
  step kernel, teacher-forced by the oracle's pick;
* the 8B-shaped decoder with 8 rows of contiguous K/V at cap 32768 and seeded start positions in [1024, 32000];
* the 8B-shaped decoder with 16 rows of paged K/V (16-token pages, a 16384-page pool, logical cap 16384, the
  seeded page permutation) and seeded start positions in [512, 16000].

Each decode step is checked in full: every logit within the bf16-weight tolerance, the greedy id equal wherever
the oracle's top-2 margin exceeds it, and the K/V each row wrote at its position (first and last layer) within the
bf16 state tolerance. The last step of each case runs with the visible K/V sweep, which must still match the oracle.
"""
import time

import numpy as np
import pytest

import oracle
import synth
from tests.ds3_testlib import Lockstep, log, make_engine, weights

pytestmark = pytest.mark.gpu


def _release():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _decode(ls, eng, tok, pos, steps, visible_from):
    w = ls.w
    last = w.model.n_layers - 1
    for i in range(steps):
        if i == visible_from:
            eng.set_kv_sweep("visible")
        got, ref, (tg, to) = ls.step(tok, pos)
        for r in range(w.rows):
            for li in (0, last):
                ls.check_kv(li, r, int(pos[r]), 1)
        log(f"{w.name} step {i} ({'visible' if i >= visible_from else 'full'} sweep): GPU {tg * 1e3:.1f} ms, "
            f"oracle {to:.1f} s, max err so far {ls.max_err:.3e}, greedy checked {ls.greedy_checked}")
        tok = ref.argmax(axis=1).astype(np.int32)
        pos = pos + 1
    return tok, pos


def test_llama1b_prompt_prefill_then_greedy_full_depth():
    w = synth.workload("llama1b-bf16")
    ws = weights(w.model)
    eng = make_engine(w, ws, prefill_rows=64)
    try:
        n = w.prefill_len
        ls = Lockstep(w, ws, eng, n_alloc=n + 16)
        prompt = synth.prefill_tokens(w)[0]
        t0 = time.time()
        got, flags = eng.prefill(0, prompt, 0)
        t1 = time.time()
        ref = oracle.causal_forward(ls.model, prompt, w.kv_dtype, cache=ls.caches[0])
        log(f"prompt of {n}: GPU prefill {1e3 * (t1 - t0):.1f} ms, oracle causal forward {time.time() - t1:.1f} s")
        ls.check_logits(got[None, :].copy(), ref[-1:], flags)
        for li in (0, w.model.n_layers - 1):
            ls.check_kv(li, 0, 0, n)
        st = eng.stats()
        assert st["kernel_plan"] == "fused" and st["prefill_tokens"] == n
        tok = np.array([int(np.argmax(ref[-1]))], np.int32)
        _decode(ls, eng, tok, np.array([n], np.int32), steps=8, visible_from=6)
        assert eng.stats()["captures"] == 3   # the decode graph and the prefill graphs (with and without the head)
    finally:
        eng.close()
        _release()


@pytest.mark.parametrize("name", ["llama8b-bf16-r8-cap32768", "llama8b-bf16-r16-paged"])
def test_llama8b_batched_full_size(name):
    w = synth.workload(name)
    ws = weights(w.model)
    eng = make_engine(w, ws)
    try:
        if w.kv_layout == "paged":
            eng.set_slot_map(synth.page_table(w))
        sp = synth.start_positions(w)
        ls = Lockstep(w, ws, eng, n_alloc=sp + 4)
        ls.prefill_random_kv(sp)
        st = eng.stats()
        log(f"{name}: rows {w.rows}, cap {w.cap}, splits {st['attn_splits']}, positions {sp.tolist()}")
        _decode(ls, eng, synth.start_tokens(w), sp.copy(), steps=3, visible_from=2)
        assert eng.stats()["captures"] == 1
    finally:
        eng.close()
        _release()
