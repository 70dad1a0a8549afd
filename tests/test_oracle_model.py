"""Pins of the oracle's whole step.

* Positions are absolute and a prefill is just steps at consecutive positions, so step-by-step decode must equal a
  causal forward over the whole prefix, evaluated by an independent entry point with a full [T, T] mask and no
  cache.
* A one-layer toy decoder evaluated with plain Python loops (no numpy) must give the same logits: this pins the
  order of the pre-norm residual pair, which weight feeds which product, and the head.
* The cache holds exactly the rounded k and v of each position.
* Rows of a step are independent: the several-row step equals the one-row step of each row, and the K/V a causal
  forward forms for a prefix equal what the step-by-step decode writes into the cache.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import ModelShape, make_weights


def _tiny_model(kv_heads=2, dtype="f32", layers=2, gains="random"):
    shape = ModelShape("pin-tiny", layers, 32, 4, kv_heads, 8, 48, 64, 1e-5, 1e4, dtype)
    ws = make_weights(shape, seed=3, std=0.2, gains=gains)
    return oracle.OracleModel.from_weightset(ws)


@pytest.mark.parametrize("kv_dtype,wdtype,kvh", [("f32", "f32", 2), ("bf16", "bf16", 1), ("f32", "f32", 4)])
def test_step_by_step_equals_causal_forward(kv_dtype, wdtype, kvh):
    model = _tiny_model(kv_heads=kvh, dtype=wdtype)
    tokens = np.random.default_rng(0).integers(0, model.vocab, size=12)
    ref = oracle.causal_forward(model, tokens, kv_dtype)
    cache = oracle.RowCache(model, 16, kv_dtype)
    for p, t in enumerate(tokens):
        got = oracle.decode_step(model, cache, int(t), p)
        np.testing.assert_allclose(got, ref[p], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("kv_dtype,wdtype", [("f32", "f32"), ("bf16", "bf16")])
def test_rows_step_equals_each_row_alone(kv_dtype, wdtype):
    """Three rows at different positions with different histories: decode_rows gives each row the logits and the
    cache entries that decode_step gives it alone (the rows only share the weight passes)."""
    model = _tiny_model(kv_heads=2, dtype=wdtype)
    rng = np.random.default_rng(4)
    positions = [0, 5, 13]
    tokens = rng.integers(0, model.vocab, size=3)
    a = [oracle.RowCache(model, 16, kv_dtype) for _ in positions]
    b = [oracle.RowCache(model, 16, kv_dtype) for _ in positions]
    for r, p in enumerate(positions):
        for li in range(model.n_layers):
            K = oracle.round_to_kv(rng.standard_normal((2, p, 8)), kv_dtype).astype(np.float32)
            V = oracle.round_to_kv(rng.standard_normal((2, p, 8)), kv_dtype).astype(np.float32)
            a[r].set(li, 0, K, V)
            b[r].set(li, 0, K, V)
    got = oracle.decode_rows(model, a, tokens, positions)
    for r, p in enumerate(positions):
        ref = oracle.decode_step(model, b[r], int(tokens[r]), p)
        np.testing.assert_allclose(got[r], ref, rtol=1e-11, atol=1e-12)
        for li in range(model.n_layers):
            np.testing.assert_array_equal(a[r].K[li], b[r].K[li])
            np.testing.assert_array_equal(a[r].V[li], b[r].V[li])


@pytest.mark.parametrize("kv_dtype,wdtype", [("f32", "f32"), ("bf16", "bf16")])
def test_causal_forward_cache_equals_step_by_step_cache(kv_dtype, wdtype):
    """The K/V a causal forward returns for a prefix are the ones T decode steps write, up to one unit in the last
    place of the KV dtype (the two evaluate the same float64 products in a different order before rounding)."""
    model = _tiny_model(kv_heads=2, dtype=wdtype)
    tokens = np.random.default_rng(6).integers(0, model.vocab, size=11)
    c1 = oracle.RowCache(model, 16, kv_dtype)
    c2 = oracle.RowCache(model, 16, kv_dtype)
    oracle.causal_forward(model, tokens, kv_dtype, cache=c1)
    for p, t in enumerate(tokens):
        oracle.decode_step(model, c2, int(t), p)
    ulp_bits = 8 if kv_dtype == "bf16" else 24
    for li in range(model.n_layers):
        for A, B in ((c1.K[li], c2.K[li]), (c1.V[li], c2.V[li])):
            a, b = A.astype(np.float64), B.astype(np.float64)
            assert np.any(a[:, :11] != 0)
            np.testing.assert_array_equal(a[:, 11:], 0.0)
            ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(b), 1e-30))[1] - ulp_bits)
            assert np.all(np.abs(a - b) <= ulp)


def test_cache_holds_rounded_k_and_v():
    model = _tiny_model(kv_heads=2, dtype="bf16")
    cache = oracle.RowCache(model, 8, "bf16")
    trace = {}
    oracle.decode_step(model, cache, 5, 0, trace=trace)
    for li in range(model.n_layers):
        k = cache.K[li][:, 0].astype(np.float64)
        assert np.array_equal(oracle.round_to_bf16(k), k)          # every stored value is a bf16 value
        assert np.any(k != 0)


def _py_rmsnorm(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gi for v, gi in zip(x, g)]


def _py_mv(W, h):
    return [sum(W[i][j] * h[j] for j in range(len(h))) for i in range(len(W))]


def _py_rope(v, p, base):
    hd = len(v)
    half = hd // 2
    out = list(v)
    for i in range(half):
        t = p * base ** (-2.0 * i / hd)
        a, b = v[i], v[i + half]
        out[i] = a * math.cos(t) - b * math.sin(t)
        out[i + half] = a * math.sin(t) + b * math.cos(t)
    return out


def test_toy_decoder_brute_force_python_loops():
    """Whole step of a 1-layer toy decoder (d=4, 2 q heads sharing 1 kv head of width 2) in plain Python."""
    shape = ModelShape("pin-toy", 1, 4, 2, 1, 2, 3, 5, 1e-5, 10.0, "f32")
    ws = make_weights(shape, seed=11, std=0.5, gains="random")
    model = oracle.OracleModel.from_weightset(ws)
    L = {k: v.astype(np.float64).tolist() for k, v in ws.layers[0].items()}
    G = {k: v.astype(np.float64).tolist() for k, v in ws.glob.items()}
    eps, base = shape.rms_eps, shape.rope_theta

    Kc, Vc = [], []
    cache = oracle.RowCache(model, 4, "f32")
    for p, tok in enumerate([3, 0, 4]):
        x = list(G["embed"][tok])
        h = _py_rmsnorm(x, L["attn_norm"], eps)
        q = _py_mv(L["wq"], h)
        k = _py_rope(_py_mv(L["wk"], h), p, base)
        v = _py_mv(L["wv"], h)
        qh = [_py_rope(q[0:2], p, base), _py_rope(q[2:4], p, base)]
        Kc.append([float(np.float32(t)) for t in k])
        Vc.append([float(np.float32(t)) for t in v])
        o = []
        for hh in range(2):
            s = [sum(qh[hh][i] * Kc[j][i] for i in range(2)) / math.sqrt(2) for j in range(p + 1)]
            m = max(s)
            e = [math.exp(t - m) for t in s]
            tot = sum(e)
            o += [sum(e[j] / tot * Vc[j][i] for j in range(p + 1)) for i in range(2)]
        x = [a + b for a, b in zip(x, _py_mv(L["wo"], o))]
        h2 = _py_rmsnorm(x, L["ffn_norm"], eps)
        gt, up = _py_mv(L["w_gate"], h2), _py_mv(L["w_up"], h2)
        a = [g / (1 + math.exp(-g)) * u for g, u in zip(gt, up)]
        x = [xa + xb for xa, xb in zip(x, _py_mv(L["w_down"], a))]
        ref = _py_mv(G["lm_head"], _py_rmsnorm(x, G["final_norm"], eps))
        got = oracle.decode_step(model, cache, tok, p)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_positions_need_not_be_consecutive():
    """Absolute positions: given cache contents for 0..p-1, a step at p only reads those and writes p."""
    model = _tiny_model()
    rng = np.random.default_rng(21)
    cache = oracle.RowCache(model, 32, "f32")
    for li in range(model.n_layers):
        cache.set(li, 0, rng.standard_normal((2, 20, 8)).astype(np.float32),
                  rng.standard_normal((2, 20, 8)).astype(np.float32))
    a = oracle.decode_step(model, cache, 7, 20)
    # garbage beyond p is never read
    cache2 = oracle.RowCache(model, 32, "f32")
    for li in range(model.n_layers):
        cache2.K[li][:] = cache.K[li]
        cache2.V[li][:] = cache.V[li]
        cache2.K[li][:, 21:] = np.nan
        cache2.V[li][:, 21:] = np.inf
    b = oracle.decode_step(model, cache2, 7, 20)
    np.testing.assert_array_equal(a, b)


def test_synth_streams_are_deterministic_and_independent():
    shape = ModelShape("pin-tiny", 2, 32, 4, 2, 8, 48, 64, 1e-5, 1e4, "bf16")
    a = make_weights(shape, seed=0)
    b = make_weights(shape, seed=0)
    c = make_weights(shape, seed=1)
    assert np.array_equal(a.layers[1]["wq"], b.layers[1]["wq"])
    assert not np.array_equal(a.layers[1]["wq"], c.layers[1]["wq"])
    assert not np.array_equal(a.layers[0]["wq"][:8], a.layers[1]["wq"][:8])
    assert a.layers[0]["wq"].dtype == np.uint16
    w = synth.workload("llama8b-bf16-r16-paged")
    pt = synth.page_table(w)
    assert pt.shape == (16, 1024) and len(np.unique(pt)) == pt.size and pt.max() < w.pool_pages
