"""CPU oracle of the constant-shape transformer decode step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this package: only the tests,
the smoke check of the graft entry point and the benchmark's CPU-baseline leg use it. It shares no code with the
HIP path (no kernels, headers, tables or helpers) and imports nothing from it.

What it computes, and where that comes from (pages of the poot documentation):

* "Execution", section "A constant-shape decode graph": each step writes the new K/V at the current position and
  attention hides every position after it. The fixed capacity, the mask and the slot buffers exist only so that
  one recorded dispatch sequence serves every position; they do not change the result. So the oracle computes
  the plain definition: for a token at absolute position p, the last-token logits of a pre-norm decoder run
  causally over positions 0..p, attending over exactly those p+1 cached positions -- no capacity, no mask
  arithmetic, no slot buffers.
* "Models, Registry and the Driver", section "Shared components": a decoder embeds the tokens, runs
  x += mixer(norm(x)); x += ffn(norm(x)) per layer, then applies the final norm and the head. The components it
  names (norms, rotary embeddings, linear projections, attention, gated feed-forward) are given no formulas on the
  pages; the readings taken for them are the standard Llama-style ones, listed per function below.
* "Models, Registry and the Driver", section "The Model": positions are absolute, and a prefill of n tokens is n
  steps at consecutive positions; `causal_forward` evaluates a whole prefix at once to pin that equivalence.

Precision: everything is evaluated in float64. Stored inputs are widened exactly (bf16 words or float32). The one
rounding that belongs to the method's state is kept: the K/V cache holds values in the workload's KV dtype
(float32, or bf16 with round-to-nearest-even), so k and v are rounded when written, as the cache stores them.

Parity pins for every function here live in tests/test_oracle_*.py (closed forms, invariants, brute force and
library special cases); no value in them comes from the HIP path.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "widen", "round_to_bf16", "round_to_kv", "rmsnorm", "rope_inv_freq", "apply_rope", "softmax",
    "attend_prefix", "masked_cap_attend", "silu", "matvec", "OracleModel", "RowCache", "decode_step",
    "decode_rows", "causal_forward", "greedy",
]

_MATVEC_ROWS = 256          # weight rows widened at a time (keeps the float64 copy cache-sized)
_threads = max(1, min(16, os.cpu_count() or 1))
_pool: ThreadPoolExecutor | None = None


def set_threads(n: int) -> None:
    """Number of host threads used for the row blocks of a matrix-vector product."""
    global _threads, _pool
    _threads = max(1, int(n))
    if _pool is not None:
        _pool.shutdown()
        _pool = None


def threads() -> int:
    return _threads


# ------------------------------------------------------------------------------------------------------------
# storage formats


def widen(a: np.ndarray) -> np.ndarray:
    """Stored values -> float64, exactly. bf16 words (uint16) carry the upper 16 bits of a float32."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits), ties to even; returned as float64.

    bf16 keeps float32's exponent range and 8 significant bits. Writing v = m * 2**e with 0.5 <= |m| < 1, the
    nearest value with 8 significant bits is rint(m * 2**8) * 2**(e - 8), and numpy's rint rounds halves to
    even. Normal range only (|v| >= 2**-126), which every value here is in; zero maps to zero.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_to_kv(v: np.ndarray, kv_dtype: str) -> np.ndarray:
    """The value the K/V cache holds for v: float32 or bf16 storage."""
    if kv_dtype == "bf16":
        return round_to_bf16(v)
    if kv_dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


# ------------------------------------------------------------------------------------------------------------
# components


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g (eps inside the root)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * widen(g)


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """Rotary frequencies base^(-2i/hd), i = 0 .. hd/2 - 1 (no frequency scaling)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def apply_rope(v: np.ndarray, p: int, base: float) -> np.ndarray:
    """Rotate every head of v ([..., hd]) to absolute position p.

    Pairing is half-split: element i pairs with element i + hd/2. The pair (a, b) turns by angle
    p * base^(-2i/hd): (a cos t - b sin t, a sin t + b cos t).
    """
    v = np.asarray(v, dtype=np.float64)
    hd = v.shape[-1]
    half = hd // 2
    t = float(p) * rope_inv_freq(hd, base)
    c, s = np.cos(t), np.sin(t)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_prefix(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Attention of one token over the cached positions it can see.

    q: [nq, hd]; K, V: [nkv, n, hd] holding exactly the visible positions 0..p (n = p + 1).
    Query head h reads kv head h // (nq / nkv) (contiguous groups). Scores are q.k / sqrt(hd).
    Returns [nq, hd]. (Each kv head is widened to float64 once and serves its group of query heads.)
    """
    nq, hd = q.shape
    nkv = K.shape[0]
    rep = nq // nkv
    out = np.empty((nq, hd), dtype=np.float64)
    for g in range(nkv):
        Kg = np.asarray(K[g], dtype=np.float64)
        Vg = np.asarray(V[g], dtype=np.float64)
        for h in range(g * rep, (g + 1) * rep):
            w = softmax(Kg @ q[h] / math.sqrt(hd))
            out[h] = w @ Vg
    return out


def masked_cap_attend(q: np.ndarray, K_cap: np.ndarray, V_cap: np.ndarray, p: int) -> np.ndarray:
    """The method's arrangement of the same attention: sweep a fixed [cap] buffer and hide j > p.

    The mask is an iota over [cap] compared with p. Hidden positions are removed by selection, never by an
    additive bias or a multiply by zero, so whatever the buffer holds after p (garbage, inf, NaN) cannot reach
    the result. Used only to pin that the sweep equals `attend_prefix`.
    """
    nq, hd = q.shape
    nkv, cap, _ = K_cap.shape
    rep = nq // nkv
    visible = np.arange(cap) <= p
    out = np.empty((nq, hd), dtype=np.float64)
    for h in range(nq):
        g = h // rep
        Kg = np.where(visible[:, None], np.asarray(K_cap[g], dtype=np.float64), 0.0)
        Vg = np.where(visible[:, None], np.asarray(V_cap[g], dtype=np.float64), 0.0)
        s = np.where(visible, Kg @ q[h] / math.sqrt(hd), -np.inf)
        m = np.max(s)
        e = np.where(visible, np.exp(s - m), 0.0)
        out[h] = (e / np.sum(e)) @ Vg
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU: z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def matvec(W: np.ndarray, h: np.ndarray) -> np.ndarray:
    """W @ h in float64 for a stored [out, in] matrix; rows are widened a block at a time.

    h is one input vector [in] or several independent ones as the columns of [in, R] (result [out, R]): the same
    products, one weight pass for all of them.
    """
    global _pool
    h = np.asarray(h, dtype=np.float64)
    n = W.shape[0]
    if n * W.shape[1] <= (1 << 20) or _threads == 1:
        return np.concatenate([widen(W[lo:lo + _MATVEC_ROWS]) @ h for lo in range(0, n, _MATVEC_ROWS)])
    if _pool is None:
        _pool = ThreadPoolExecutor(_threads)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        parts = list(_pool.map(lambda lo: widen(W[lo:lo + _MATVEC_ROWS]) @ h, range(0, n, _MATVEC_ROWS)))
    return np.concatenate(parts)


# ------------------------------------------------------------------------------------------------------------
# model and state


class OracleModel:
    """A decoder's shape and stored weights (as drawn: bf16 words or float32; matrices [out, in])."""

    def __init__(self, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps, rope_theta,
                 layers, glob):
        self.n_layers, self.d_model = n_layers, d_model
        self.n_q_heads, self.n_kv_heads, self.head_dim = n_q_heads, n_kv_heads, head_dim
        self.ffn_dim, self.vocab = ffn_dim, vocab
        self.rms_eps, self.rope_theta = float(rms_eps), float(rope_theta)
        self.layers, self.glob = layers, glob

    @classmethod
    def from_weightset(cls, ws) -> "OracleModel":
        m = ws.model
        return cls(m.n_layers, m.d_model, m.n_q_heads, m.n_kv_heads, m.head_dim, m.ffn_dim, m.vocab, m.rms_eps,
                   m.rope_theta, ws.layers, ws.glob)


class RowCache:
    """The carried K/V state of one sequence: per layer [nkv, n_alloc, hd], values already in the KV dtype.

    Held as float32 (every bf16 and float32 value is exact in it). Only positions a step may see are read.
    """

    def __init__(self, model: OracleModel, n_alloc: int, kv_dtype: str):
        self.kv_dtype = kv_dtype
        shape = (model.n_kv_heads, n_alloc, model.head_dim)
        self.K = [np.zeros(shape, np.float32) for _ in range(model.n_layers)]
        self.V = [np.zeros(shape, np.float32) for _ in range(model.n_layers)]

    def set(self, layer: int, pos0: int, K: np.ndarray, V: np.ndarray) -> None:
        """Place given K/V contents ([nkv, n, hd], stored values) at positions pos0 .. pos0 + n - 1."""
        n = K.shape[1]
        self.K[layer][:, pos0:pos0 + n] = widen(K).astype(np.float32)
        self.V[layer][:, pos0:pos0 + n] = widen(V).astype(np.float32)


def decode_step(model: OracleModel, cache: RowCache, token: int, p: int, *, trace: dict | None = None) -> np.ndarray:
    """One decode step of one row: token at absolute position p -> logits [vocab] (float64).

    Writes this position's k and v into `cache` (rounded to the KV dtype) and attends over positions 0..p.
    When `trace` is a dict it receives intermediate values per layer (for kernel-level comparisons).
    """
    nq, nkv, hd = model.n_q_heads, model.n_kv_heads, model.head_dim
    eps = model.rms_eps
    x = widen(model.glob["embed"][token])
    for li, L in enumerate(model.layers):
        h = rmsnorm(x, L["attn_norm"], eps)
        q = apply_rope(matvec(L["wq"], h).reshape(nq, hd), p, model.rope_theta)
        k = apply_rope(matvec(L["wk"], h).reshape(nkv, hd), p, model.rope_theta)
        v = matvec(L["wv"], h).reshape(nkv, hd)
        cache.K[li][:, p] = round_to_kv(k, cache.kv_dtype)
        cache.V[li][:, p] = round_to_kv(v, cache.kv_dtype)
        o = attend_prefix(q, cache.K[li][:, :p + 1], cache.V[li][:, :p + 1])
        x = x + matvec(L["wo"], o.reshape(-1))
        h2 = rmsnorm(x, L["ffn_norm"], eps)
        a = silu(matvec(L["w_gate"], h2)) * matvec(L["w_up"], h2)
        x = x + matvec(L["w_down"], a)
        if trace is not None:
            trace.setdefault("q", []).append(q)
            trace.setdefault("attn", []).append(o)
            trace.setdefault("x", []).append(x.copy())
    return matvec(model.glob["lm_head"], rmsnorm(x, model.glob["final_norm"], eps))


def decode_rows(model: OracleModel, caches, tokens, positions) -> np.ndarray:
    """One decode step of several independent rows: row r takes tokens[r] at absolute position positions[r] with
    its own cache caches[r]. Returns logits [rows, vocab] (float64).

    Each row computes exactly what `decode_step` computes for it alone; the only difference is that every weight
    matrix is multiplied with the rows' activations as the columns of one matrix (one weight pass per step).
    """
    nq, nkv, hd = model.n_q_heads, model.n_kv_heads, model.head_dim
    eps = model.rms_eps
    R = len(tokens)
    X = np.stack([widen(model.glob["embed"][int(t)]) for t in tokens])                # [R, d]
    for li, L in enumerate(model.layers):
        H = rmsnorm(X, L["attn_norm"], eps)
        Qa, Ka, Va = matvec(L["wq"], H.T).T, matvec(L["wk"], H.T).T, matvec(L["wv"], H.T).T
        O = np.empty((R, nq * hd))
        for r in range(R):
            p = int(positions[r])
            q = apply_rope(Qa[r].reshape(nq, hd), p, model.rope_theta)
            k = apply_rope(Ka[r].reshape(nkv, hd), p, model.rope_theta)
            c = caches[r]
            c.K[li][:, p] = round_to_kv(k, c.kv_dtype)
            c.V[li][:, p] = round_to_kv(Va[r].reshape(nkv, hd), c.kv_dtype)
            O[r] = attend_prefix(q, c.K[li][:, :p + 1], c.V[li][:, :p + 1]).reshape(-1)
        X = X + matvec(L["wo"], O.T).T
        H2 = rmsnorm(X, L["ffn_norm"], eps)
        A = silu(matvec(L["w_gate"], H2.T)) * matvec(L["w_up"], H2.T)
        X = X + matvec(L["w_down"], A).T
    return matvec(model.glob["lm_head"], rmsnorm(X, model.glob["final_norm"], eps).T).T


def causal_forward(model: OracleModel, tokens, kv_dtype: str, cache: "RowCache | None" = None) -> np.ndarray:
    """All positions of a prefix at once: logits [T, vocab] for tokens at positions 0..T-1.

    No cache is read: each layer forms K and V for the whole prefix (rounded to the KV dtype, as the cache would
    hold them) and applies a full [T, T] causal mask (key j visible to query i iff j <= i). When `cache` is given
    it receives those K and V at positions 0..T-1 of every layer (what T decode steps would have written).
    """
    tokens = np.asarray(tokens)
    T = len(tokens)
    nq, nkv, hd = model.n_q_heads, model.n_kv_heads, model.head_dim
    rep = nq // nkv
    eps = model.rms_eps
    X = np.stack([widen(model.glob["embed"][t]) for t in tokens])                  # [T, d]
    causal = np.tril(np.ones((T, T), dtype=bool))
    for li, L in enumerate(model.layers):
        H = rmsnorm(X, L["attn_norm"], eps)
        QH, KH = H @ widen(L["wq"]).T, H @ widen(L["wk"]).T                        # [T, nq hd], [T, nkv hd]
        Q = np.stack([apply_rope(QH[i].reshape(nq, hd), i, model.rope_theta) for i in range(T)])
        Kx = np.stack([apply_rope(KH[i].reshape(nkv, hd), i, model.rope_theta) for i in range(T)])
        Vx = (H @ widen(L["wv"]).T).reshape(T, nkv, hd)
        Kx, Vx = round_to_kv(Kx, kv_dtype), round_to_kv(Vx, kv_dtype)
        if cache is not None:
            cache.K[li][:, :T] = Kx.transpose(1, 0, 2)
            cache.V[li][:, :T] = Vx.transpose(1, 0, 2)
        O = np.empty((T, nq, hd))
        for hh in range(nq):
            g = hh // rep
            S = (Q[:, hh, :] @ Kx[:, g, :].T) / math.sqrt(hd)                    # [T, T]
            S = np.where(causal, S, -np.inf)
            O[:, hh, :] = softmax(S) @ Vx[:, g, :]
        X = X + O.reshape(T, nq * hd) @ widen(L["wo"]).T
        H2 = rmsnorm(X, L["ffn_norm"], eps)
        A = silu(H2 @ widen(L["w_gate"]).T) * (H2 @ widen(L["w_up"]).T)
        X = X + A @ widen(L["w_down"]).T
    return rmsnorm(X, model.glob["final_norm"], eps) @ widen(model.glob["lm_head"]).T


def greedy(logits: np.ndarray) -> tuple[int, float]:
    """Greedy pick: (argmax with ties to the lowest index, top-1 minus top-2 margin)."""
    logits = np.asarray(logits)
    i = int(np.argmax(logits))
    top2 = np.partition(logits, -2)[-2:]
    return i, float(top2[1] - top2[0])
