"""The sampling suffix (ds3_step_sample): penalties and bias from the device-kept token history, greedy or a
temperature draw with top-k / top-p / min-p, SplitMix64 draws, logprobs. Against the sampling oracle applied to the
same engine state's logits (a second engine, same tokens): a greedy pick is the oracle's exactly; a drawn token
lies in the oracle's kept set and its inverse-CDF interval holds the oracle's u (the device cuts on 2^-40 fixed
point weights, the oracle in float64, so a boundary case may differ by rounding only); logprobs agree; the
history grows by every drawn token; a seed replays the same tokens.
"""
from dataclasses import replace

import numpy as np
import pytest

import bench
import synth
from decode_step_03_amd import DS3Error, _ds3 as C
from oracle import sampler as S
from tests.ds3_testlib import log, make_engine, weights

pytestmark = pytest.mark.gpu

PARAMS = [   # one row each: (temperature, top_k, top_p, min_p, rep, presence, frequency, n_logprobs)
    (0.0, 0, 1.0, 0.0, 1.3, 0.2, 0.1, 4),
    (0.9, 0, 1.0, 0.0, 1.0, 0.0, 0.0, 8),
    (1.2, 20, 0.9, 0.0, 1.1, 0.0, 0.05, 3),
    (0.7, 0, 0.8, 0.05, 1.0, 0.3, 0.0, 0),
    (1.0, 50, 1.0, 0.1, 1.0, 0.0, 0.0, 2),      # top-k alone (the set gathered into LDS), with min-p
    (0.8, 1500, 0.7, 0.0, 1.0, 0.0, 0.0, 0),    # top-k above the gathered-set limit: the whole-vocabulary path
    (0.8, 40, 0.95, 0.02, 1.1, 0.0, 0.0, 5),    # the parameters bench.py times
    (1.0, 5000, 0.98, 0.0, 1.0, 0.1, 0.0, 1),   # a large top-k with top-p
    (0.9, 100, 0.9, 0.0, 1.0, 0.0, 0.0, 6),     # a candidate-path top-k above one wave's lanes, logprobs from it
    (1.0, 3, 1.0, 0.0, 1.0, 0.0, 0.1, 8),       # more logprobs than top-k: the segments' own top-n lists
]


def _workload(name):
    if name == "tiny-fp32":
        return synth.workload("tiny-fp32")
    if name == "8b-fused":
        base = synth.workload("llama8b-bf16-cap8192")
        return replace(synth.small_variant(base, n_layers=1, vocab=4096), name="llama8b-1l-sample")
    if name == "8b-fullvocab":   # the full 128,256-token vocabulary the benchmark samples from
        base = synth.workload("llama8b-bf16-cap8192")
        return replace(synth.small_variant(base, n_layers=1), name="llama8b-1l-sample-v128256")
    if name == "8b-r8":
        base = synth.workload("llama8b-bf16-r8-cap32768")
        return replace(synth.small_variant(base, n_layers=1, vocab=4096, cap=4096), name="llama8b-r8-sample")
    raise KeyError(name)


def _set(eng, w, rng, shift=0):
    hist, bias, prm = [], [], []
    for r in range(w.rows):
        t, k, p, mp, rep, pres, freq, nl = PARAMS[(r + shift) % len(PARAMS)]
        seed = 1000 + 17 * r
        eng.set_sampling(r, temperature=t, top_k=k, top_p=p, min_p=mp, repetition_penalty=rep,
                         presence_penalty=pres, frequency_penalty=freq, n_logprobs=nl, seed=seed)
        h = rng.integers(0, w.model.vocab, size=30).astype(np.int32)
        b = np.zeros(w.model.vocab, np.float32)
        b[rng.integers(0, w.model.vocab, size=10)] = rng.normal(0, 2, size=10).astype(np.float32)
        eng.set_history(r, h, b)
        hist.append(np.bincount(h, minlength=w.model.vocab).astype(np.int64))
        bias.append(b)
        prm.append((t, k, p, mp, rep, pres, freq, nl, seed))
    return hist, bias, prm


@pytest.mark.parametrize("name,shift", [("tiny-fp32", 1), ("tiny-fp32", 2), ("8b-fused", 0), ("8b-fused", 2),
                                        ("8b-fused", 3), ("8b-fused", 4), ("8b-fused", 5), ("8b-r8", 0),
                                        ("8b-fullvocab", 6), ("8b-fullvocab", 7), ("8b-fullvocab", 5),
                                        ("8b-fullvocab", 8), ("8b-fullvocab", 9)])
def test_sampler_follows_oracle(name, shift):
    w = _workload(name)
    ws = weights(w.model)
    a = make_engine(w, ws)
    b = make_engine(w, ws)
    try:
        sp = np.minimum(synth.start_positions(w), w.cap - 16).astype(np.int32)
        tok = synth.start_tokens(w)
        for e in (a, b):
            bench.prefill(e, w, sp)
        hist, bias, prm = _set(a, w, np.random.default_rng(3), shift)
        n = 6
        ids, flags, lp, lpi = a.step_sample(tok, sp, n)
        assert not flags.any()
        t = tok.copy()
        drawn = checked = 0
        for i in range(n):
            lg, fl = b.step(t, sp + i)
            assert fl == 0
            for r in range(w.rows):
                T, k, p, mp, rep, pres, freq, nl, seed = prm[r]
                z = S.adjust(lg[r], hist[r], bias[r], rep, pres, freq)
                got = int(ids[i, r])
                if T == 0.0:
                    srt = np.sort(z)
                    if srt[-1] - srt[-2] > 1e-5:
                        assert got == int(np.argmax(z)), f"step {i} row {r}: greedy {got} != {int(np.argmax(z))}"
                        checked += 1
                else:
                    kept, wts = S.keep_set(z, T, k, p, mp)
                    u = S.uniform(seed, i)
                    run = np.concatenate([[0.0], np.cumsum(wts)]) / np.sum(wts)
                    if got in kept:
                        j = int(np.nonzero(kept == got)[0][0])
                        assert run[j] - 1e-4 <= u <= run[j + 1] + 1e-4, f"step {i} row {r}: u {u} outside [{run[j]}, {run[j + 1]}]"
                        checked += 1
                    else:
                        # only a token on a cut boundary may differ from the oracle's kept set (the device cuts on
                        # fixed-point weights): its score is within 1e-4 of the last kept one, and u falls in its
                        # inverse-CDF interval once it is added to the kept set
                        s = z / T
                        order = np.lexsort((np.arange(s.size), -s))
                        rank = int(np.nonzero(order == got)[0][0])
                        assert abs(s[got] - s[order[min(rank, len(kept)) - 1]]) < 1e-4, f"step {i} row {r}: {got} not kept"
                        k2 = np.sort(np.append(kept, got))
                        w2 = np.exp(s[k2] - np.max(s[k2]))
                        run2 = np.concatenate([[0.0], np.cumsum(w2)]) / np.sum(w2)
                        j = int(np.nonzero(k2 == got)[0][0])
                        assert run2[j] - 1e-4 <= u <= run2[j + 1] + 1e-4, f"step {i} row {r}: u {u} outside the cut token's interval"
                    drawn += 1
                if nl > 0:
                    top, lps, lt = S.logprobs(z, T, nl, got)
                    assert abs(lp[i, r, 0] - lt) < 2e-3
                    assert np.max(np.abs(lp[i, r, 1:1 + nl] - lps)) < 2e-3
                    gaps = np.abs(np.diff(np.sort(z / (T if T > 0 else 1.0))[::-1][:nl + 1]))
                    if np.all(gaps > 1e-4):
                        assert list(lpi[i, r, :nl]) == list(top)
                hist[r][got] += 1
            t = ids[i].copy()
        log(name, "params", shift, "draws", drawn, "checked", checked)
    finally:
        a.close()
        b.close()


def test_sampler_seed_replays_and_greedy_matches_greedy_chain():
    w = _workload("tiny-fp32")
    ws = synth.make_weights(w.model)
    eng = make_engine(w, ws)
    try:
        sp = synth.start_positions(w)
        tok = synth.start_tokens(w)
        bench.prefill(eng, w, sp)
        eng.set_sampling(0, temperature=1.0, top_p=0.95, seed=42)
        i1, _, _, _ = eng.step_sample(tok, sp, 5)
        eng.reset_state()
        eng.set_history(0)
        eng.set_sampling(0, temperature=1.0, top_p=0.95, seed=42)   # restarts the row's draw count
        i2, _, _, _ = eng.step_sample(tok, sp, 5)
        assert np.array_equal(i1, i2)
        eng.reset_state()
        eng.set_history(0)
        eng.set_sampling(0)   # greedy, no penalties
        g1, _, _, _ = eng.step_sample(tok, sp, 5)
        eng.reset_state()
        g2, _ = eng.step_greedy(tok, sp, 5)
        assert np.array_equal(g1, g2)
        for bad in (dict(temperature=-1.0), dict(top_p=0.0), dict(min_p=1.0), dict(repetition_penalty=0.0),
                    dict(top_k=-1), dict(n_logprobs=C.DS3_MAX_LOGPROBS + 1)):
            with pytest.raises(DS3Error) as ei:
                eng.set_sampling(0, **bad)
            assert ei.value.status == C.DS3_E_INVALID
    finally:
        eng.close()
