"""Pins of the oracle's components against facts fixed outside the oracle itself.

Each test checks a closed form, an invariant, a brute-force evaluation with Python loops on a tiny input, or a
special case that reduces to a library routine (torch's bf16 conversion, numpy's float32 cast and matmul,
complex multiplication). A plausible slip in the oracle (a dropped term, a wrong sign, index or pairing, a
transposed operand) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle


# ------------------------------------------------------------------------------------------------- storage


def test_round_to_bf16_matches_library_conversion():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-20),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e20),
    ])
    # exact ties: 8 significant bits plus exactly one half unit in the last place
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(2 + 2 ** -7), 1.5 + 2 ** -8, 3 * 2 ** -9 * (1 + 2 ** -8)],
                    dtype=np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_to_bf16_ties_to_even():
    assert oracle.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0                   # tie, even is 1.0
    assert oracle.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6      # tie, even is up
    assert oracle.round_to_bf16(np.array([1 + 2 ** -8 + 2 ** -30]))[0] == 1 + 2 ** -7
    assert oracle.round_to_bf16(np.array([0.0]))[0] == 0.0


def test_round_to_kv_f32_is_float32_cast():
    v = np.random.default_rng(2).standard_normal(1000) * 10
    np.testing.assert_array_equal(oracle.round_to_kv(v, "f32"), v.astype(np.float32).astype(np.float64))


def test_widen_bf16_words_exact():
    x = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16)
    words = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.widen(words), x.to(torch.float64).numpy())


# ------------------------------------------------------------------------------------------------- RMSNorm


@pytest.mark.parametrize("c", [1e-3, 0.5, 1.0, 7.0, -3.0])
@pytest.mark.parametrize("d", [1, 4, 256])
def test_rmsnorm_constant_vector_closed_form(c, d):
    eps = 1e-5
    g = np.linspace(0.5, 1.5, d)
    y = oracle.rmsnorm(np.full(d, c), g, eps)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * g, rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    x = np.random.default_rng(3).standard_normal(512) * 5
    g = np.ones(512)
    y1 = oracle.rmsnorm(x, g, 0.0)
    y2 = oracle.rmsnorm(x * 37.0, g, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    assert abs(np.mean(y1 * y1) - 1.0) < 1e-12
    # with eps the mean square is ms/(ms+eps)
    eps = 0.25
    ms = np.mean(x * x)
    y3 = oracle.rmsnorm(x, g, eps)
    assert abs(np.mean(y3 * y3) - ms / (ms + eps)) < 1e-12


def test_rmsnorm_gain_is_elementwise():
    x = np.random.default_rng(4).standard_normal(64)
    g = np.random.default_rng(5).standard_normal(64)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 1e-5), oracle.rmsnorm(x, np.ones(64), 1e-5) * g, rtol=1e-14)


# ------------------------------------------------------------------------------------------------- RoPE


def test_rope_identity_at_position_zero():
    v = np.random.default_rng(6).standard_normal((3, 64))
    np.testing.assert_array_equal(oracle.apply_rope(v, 0, 1e4), v)


def test_rope_equals_complex_multiplication():
    # half-split pairing: z_i = v_i + 1j * v_{i+hd/2}, rotated by exp(1j * p * base^(-2i/hd))
    rng = np.random.default_rng(7)
    for hd, base, p in [(64, 1e4, 17), (128, 5e5, 31999), (8, 100.0, 3)]:
        v = rng.standard_normal((4, hd))
        half = hd // 2
        z = v[:, :half] + 1j * v[:, half:]
        freq = np.array([base ** (-2.0 * i / hd) for i in range(half)])
        zr = z * np.exp(1j * p * freq)
        ref = np.concatenate([zr.real, zr.imag], axis=-1)
        np.testing.assert_allclose(oracle.apply_rope(v, p, base), ref, rtol=1e-12, atol=1e-12)


def test_rope_frequency_convention_closed_form():
    # hd = 4, base = 100: pair 0 turns by p rad, pair 1 by p * 100^(-1/2) = p / 10 rad.
    e0 = np.array([1.0, 0.0, 0.0, 0.0])
    e1 = np.array([0.0, 1.0, 0.0, 0.0])
    np.testing.assert_allclose(oracle.apply_rope(e0, 2, 100.0), [math.cos(2), 0, math.sin(2), 0], atol=1e-15)
    np.testing.assert_allclose(oracle.apply_rope(e1, 10, 100.0), [0, math.cos(1), 0, math.sin(1)], atol=1e-15)
    # the second element of a pair turns the same way: (0, 1) -> (-sin t, cos t)
    e2 = np.array([0.0, 0.0, 1.0, 0.0])
    np.testing.assert_allclose(oracle.apply_rope(e2, 2, 100.0), [-math.sin(2), 0, math.cos(2), 0], atol=1e-15)


def test_rope_preserves_pair_norms_and_composes():
    rng = np.random.default_rng(8)
    v = rng.standard_normal(128)
    r = oracle.apply_rope(v, 1234, 5e5)
    np.testing.assert_allclose(r[:64] ** 2 + r[64:] ** 2, v[:64] ** 2 + v[64:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(oracle.apply_rope(oracle.apply_rope(v, 100, 5e5), 23, 5e5),
                               oracle.apply_rope(v, 123, 5e5), rtol=1e-10, atol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = oracle.apply_rope(q, 50, 1e4) @ oracle.apply_rope(k, 20, 1e4)
    b = oracle.apply_rope(q, 1030, 1e4) @ oracle.apply_rope(k, 1000, 1e4)
    assert abs(a - b) < 1e-10


# ------------------------------------------------------------------------------------------------- softmax / attention


def _softmax_loops(s):
    m = max(s)
    e = [math.exp(v - m) for v in s]
    t = sum(e)
    return [v / t for v in e]


def test_softmax_brute_force_and_invariants():
    rng = np.random.default_rng(10)
    for n in [1, 2, 7]:
        s = rng.standard_normal(n) * 4
        np.testing.assert_allclose(oracle.softmax(s), _softmax_loops(list(s)), rtol=1e-14)
        np.testing.assert_allclose(oracle.softmax(s + 123.0), oracle.softmax(s), rtol=1e-12)
        assert abs(oracle.softmax(s).sum() - 1) < 1e-14
    # large scores do not overflow
    assert np.all(np.isfinite(oracle.softmax(np.array([1000.0, 999.0, -1000.0]))))


def _attend_loops(q, K, V):
    nq, hd = len(q), len(q[0])
    nkv, n = len(K), len(K[0])
    rep = nq // nkv
    out = []
    for h in range(nq):
        g = h // rep
        s = [sum(q[h][i] * K[g][j][i] for i in range(hd)) / math.sqrt(hd) for j in range(n)]
        w = _softmax_loops(s)
        out.append([sum(w[j] * V[g][j][i] for j in range(n)) for i in range(hd)])
    return out


@pytest.mark.parametrize("nq,nkv,hd,n", [(1, 1, 4, 1), (2, 1, 8, 5), (4, 2, 4, 7), (3, 3, 2, 3)])
def test_attention_brute_force(nq, nkv, hd, n):
    rng = np.random.default_rng(nq * 100 + nkv * 10 + n)
    q = rng.standard_normal((nq, hd))
    K = rng.standard_normal((nkv, n, hd))
    V = rng.standard_normal((nkv, n, hd))
    ref = _attend_loops(q.tolist(), K.tolist(), V.tolist())
    np.testing.assert_allclose(oracle.attend_prefix(q, K, V), ref, rtol=1e-12, atol=1e-14)


def test_attention_single_position_returns_value_row_exactly():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((8, 16)) * 100
    K = rng.standard_normal((2, 1, 16))
    V = rng.standard_normal((2, 1, 16))
    out = oracle.attend_prefix(q, K, V)
    for h in range(8):
        np.testing.assert_array_equal(out[h], V[h // 4, 0])


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(12)
    nq, nkv, hd, n = 8, 2, 16, 9
    q = rng.standard_normal((nq, hd))
    K = rng.standard_normal((nkv, n, hd))
    V = rng.standard_normal((nkv, n, hd))
    Kr, Vr = np.repeat(K, nq // nkv, axis=0), np.repeat(V, nq // nkv, axis=0)   # head h gets group h // 4
    np.testing.assert_allclose(oracle.attend_prefix(q, K, V), oracle.attend_prefix(q, Kr, Vr), rtol=1e-14)


@pytest.mark.parametrize("p", [0, 1, 37, 127])
def test_masked_cap_sweep_equals_prefix_attention(p):
    rng = np.random.default_rng(13 + p)
    nq, nkv, hd, cap = 4, 2, 8, 128
    q = rng.standard_normal((nq, hd))
    K = rng.standard_normal((nkv, cap, hd))
    V = rng.standard_normal((nkv, cap, hd))
    np.testing.assert_allclose(oracle.masked_cap_attend(q, K, V, p),
                               oracle.attend_prefix(q, K[:, :p + 1], V[:, :p + 1]), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("p", [0, 5, 62])
def test_masked_cap_sweep_ignores_garbage_after_position(p):
    rng = np.random.default_rng(14 + p)
    nq, nkv, hd, cap = 4, 4, 8, 64
    q = rng.standard_normal((nq, hd))
    K = rng.standard_normal((nkv, cap, hd))
    V = rng.standard_normal((nkv, cap, hd))
    clean = oracle.masked_cap_attend(q, K, V, p)
    Kg, Vg = K.copy(), V.copy()
    Kg[:, p + 1:] = rng.standard_normal(Kg[:, p + 1:].shape) * 100.0
    Vg[:, p + 1:] = rng.standard_normal(Vg[:, p + 1:].shape) * 100.0
    np.testing.assert_array_equal(oracle.masked_cap_attend(q, Kg, Vg, p), clean)
    specials = np.array([np.nan, np.inf, -np.inf])
    Kg[:, p + 1:] = rng.choice(specials, Kg[:, p + 1:].shape)
    Vg[:, p + 1:] = rng.choice(specials, Vg[:, p + 1:].shape)
    with np.errstate(invalid="ignore"):
        np.testing.assert_array_equal(oracle.masked_cap_attend(q, Kg, Vg, p), clean)


# ------------------------------------------------------------------------------------------------- SwiGLU / matvec


def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    z = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, atol=1e-14)        # z*sig(z) - (-z)*sig(-z)
    np.testing.assert_allclose(oracle.silu(np.array([40.0])), [40.0], rtol=1e-15)
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matvec_matches_float64_matmul(dtype):
    rng = np.random.default_rng(15)
    W32 = rng.standard_normal((1000, 700)).astype(np.float32)
    if dtype == "bf16":
        W = torch.from_numpy(W32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        Wf = torch.from_numpy(W32).to(torch.bfloat16).to(torch.float64).numpy()
    else:
        W, Wf = W32, W32.astype(np.float64)
    h = rng.standard_normal(700)
    np.testing.assert_allclose(oracle.matvec(W, h), Wf @ h, rtol=1e-12, atol=1e-12)
    # threaded row blocks give the same bits as one thread
    big = np.tile(W, (3, 3))
    hb = np.tile(h, 3)
    t = oracle.threads()
    try:
        oracle.set_threads(1)
        a = oracle.matvec(big, hb)
        oracle.set_threads(4)
        b = oracle.matvec(big, hb)
    finally:
        oracle.set_threads(t)
    np.testing.assert_array_equal(a, b)


def test_greedy_ties_to_lowest_index_and_margin():
    i, m = oracle.greedy(np.array([0.5, 2.0, 2.0, -1.0]))
    assert i == 1 and m == 0.0
    i, m = oracle.greedy(np.array([0.5, 2.0, 1.25, -1.0]))
    assert i == 1 and m == 0.75
