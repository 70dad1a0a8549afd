"""Seeded synthetic workloads for the transformer decode step.

This module only *draws* data: model shapes, weights, pre-filled K/V contents, tokens, start positions and
page maps. It holds none of the step's arithmetic (no norm, projection, rotation, attention or activation), so
both the CPU oracle's tests and the GPU path's tests and benchmark can take their inputs from here without
sharing any of the method.

Every tensor is drawn from its own independent stream, keyed by (seed, model, purpose, layer, row, chunk), so any
tensor can be regenerated on its own and the values do not depend on thread count or call order.

Storage rounding: bf16 tensors are drawn in float32 and rounded once, round-to-nearest-even, to bf16 words
(numpy uint16). fp32 tensors are returned as float32.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "workload", "small_variant",
    "WeightSet", "make_weights", "kv_prefill", "start_tokens", "prefill_tokens",
    "start_positions", "page_table", "f32_to_bf16_words", "bf16_words_to_f32",
]

_CHUNK = 1 << 22  # elements per independent stream chunk


@dataclass(frozen=True)
class ModelShape:
    """Shape of a Llama-style pre-norm decoder (no biases, untied embedding and head)."""
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float
    rope_theta: float
    weight_dtype: str  # "f32" | "bf16"

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def n_params(self) -> int:
        d, hd, F = self.d_model, self.head_dim, self.ffn_dim
        per_layer = d * self.qkv_rows + self.n_q_heads * hd * d + 3 * d * F + 2 * d
        return self.n_layers * per_layer + 2 * self.vocab * d + d


@dataclass(frozen=True)
class Workload:
    """One decode workload: a model, a batch of rows, a KV capacity and layout, and a step schedule."""
    name: str
    model: ModelShape
    rows: int
    cap: int
    kv_layout: str          # "contiguous" | "paged"
    kv_dtype: str           # "f32" | "bf16"
    steps: int              # decode steps per row
    start: str              # "token_at_0" | "prefill_tokens" | "random_kv"
    prefill_len: int = 0    # tokens fed before the timed steps ("prefill_tokens") or pre-filled KV length
    pos_lo: int = 0         # per-row start position range (inclusive) for "random_kv" with rows > 1
    pos_hi: int = 0
    page_size: int = 0
    pool_pages: int = 0

    @property
    def pages_per_row(self) -> int:
        return self.cap // self.page_size if self.kv_layout == "paged" else 0


_TINY = ModelShape("tiny", 2, 256, 4, 4, 64, 688, 1024, 1e-5, 1e4, "f32")
_L1B = ModelShape("llama1b", 16, 2048, 32, 8, 64, 8192, 32000, 1e-5, 1e4, "bf16")
_L8B = ModelShape("llama8b", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 5e5, "bf16")

WORKLOADS = {
    # tiny fp32 decoder, 64 greedy steps from position 0
    "tiny-fp32": Workload("tiny-fp32", _TINY, 1, 128, "contiguous", "f32", 64, "token_at_0"),
    # 1B-shaped bf16 decoder: 512 random prompt tokens, then 256 greedy steps
    "llama1b-bf16": Workload("llama1b-bf16", _L1B, 1, 4096, "contiguous", "bf16", 256, "prefill_tokens",
                             prefill_len=512),
    # 8B-shaped bf16 decoder, batch 1, cap 8192, KV pre-filled with N(0,1) up to 2048, 512 steps
    "llama8b-bf16-cap8192": Workload("llama8b-bf16-cap8192", _L8B, 1, 8192, "contiguous", "bf16", 512,
                                     "random_kv", prefill_len=2048),
    # 8B-shaped, 8 rows, contiguous cap 32768, per-row start position ~ U[1024, 32000], 128 steps
    "llama8b-bf16-r8-cap32768": Workload("llama8b-bf16-r8-cap32768", _L8B, 8, 32768, "contiguous", "bf16", 128,
                                         "random_kv", pos_lo=1024, pos_hi=32000),
    # 8B-shaped, 16 rows, paged KV (16-token pages, 16384-page pool), logical cap 16384, pos ~ U[512, 16000]
    "llama8b-bf16-r16-paged": Workload("llama8b-bf16-r16-paged", _L8B, 16, 16384, "paged", "bf16", 128,
                                       "random_kv", pos_lo=512, pos_hi=16000, page_size=16, pool_pages=16384),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def small_variant(w: Workload, *, n_layers: int | None = None, vocab: int | None = None, cap: int | None = None,
                  rows: int | None = None, pool_pages: int | None = None, name_suffix: str = "-small") -> Workload:
    """Same per-layer shapes, fewer layers / smaller vocab / cap, for parity cases the oracle finishes quickly."""
    m = w.model
    m2 = replace(m, n_layers=n_layers or m.n_layers, vocab=vocab or m.vocab)
    w2 = replace(w, name=w.name + name_suffix, model=m2, cap=cap or w.cap, rows=rows or w.rows,
                 pool_pages=pool_pages if pool_pages is not None else w.pool_pages)
    return w2


# ----------------------------------------------------------------------------------------------------------
# streams


def _key(*parts) -> list[int]:
    out = []
    for p in parts:
        if isinstance(p, str):
            out.append(zlib.crc32(p.encode()))
        else:
            out.append(int(p) & 0xFFFFFFFF)
    return out


def _gen(*parts) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence(_key(*parts))))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_words(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return the 16-bit words."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_words_to_f32(w: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 words to float32."""
    return (np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_tensor(shape, std: float, dtype: str, key: tuple, pool: ThreadPoolExecutor | None) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(ci: int):
        lo = ci * _CHUNK
        hi = min(n, lo + _CHUNK)
        v = _gen(*key, ci).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if dtype == "bf16":
            out[lo:hi] = f32_to_bf16_words(v)
        else:
            out[lo:hi] = v

    nch = (n + _CHUNK - 1) // _CHUNK
    if pool is None or nch == 1:
        for ci in range(nch):
            fill(ci)
    else:
        list(pool.map(fill, range(nch)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------------------------------------
# weights


ROLES_PER_LAYER = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
ROLES_GLOBAL = ("embed", "final_norm", "lm_head")


@dataclass
class WeightSet:
    """Weights of one model as stored: bf16 words (uint16) or float32, matrices [out, in] row-major."""
    model: ModelShape
    layers: list            # list of dict role -> array
    glob: dict              # role -> array
    dtype: str

    def shape_of(self, role: str) -> tuple:
        m = self.model
        d, hd, F = m.d_model, m.head_dim, m.ffn_dim
        return {
            "attn_norm": (d,), "ffn_norm": (d,), "final_norm": (d,),
            "wq": (m.n_q_heads * hd, d), "wk": (m.n_kv_heads * hd, d), "wv": (m.n_kv_heads * hd, d),
            "wo": (d, m.n_q_heads * hd), "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F),
            "embed": (m.vocab, d), "lm_head": (m.vocab, d),
        }[role]


def make_weights(model: ModelShape, seed: int = 0, *, std: float = 0.02, gains: str = "ones",
                 gain_std: float = 0.1) -> WeightSet:
    """Draw every weight of `model`: matrices ~ N(0, std^2); RMSNorm gains = 1 ("ones") or 1 + N(0, gain_std^2)."""
    ws = WeightSet(model, [], {}, model.weight_dtype)
    dt = model.weight_dtype
    import torch
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)      # the chunk workers already use every core
    try:
        _draw_weights(ws, model, seed, std, gains, gain_std, dt)
    finally:
        torch.set_num_threads(torch_threads)
    return ws


def _draw_weights(ws, model, seed, std, gains, gain_std, dt):
    with ThreadPoolExecutor(_threads()) as pool:
        def gain(role, layer):
            if gains == "ones":
                g = np.ones(model.d_model, np.float32)
            else:
                g = 1.0 + _normal_tensor((model.d_model,), gain_std, "f32", (seed, model.name, role, layer), None)
                g = g.astype(np.float32)
            return f32_to_bf16_words(g) if dt == "bf16" else g

        for li in range(model.n_layers):
            layer = {}
            for role in ROLES_PER_LAYER:
                if role.endswith("norm"):
                    layer[role] = gain(role, li)
                else:
                    layer[role] = _normal_tensor(ws.shape_of(role), std, dt, (seed, model.name, role, li), pool)
            ws.layers.append(layer)
        ws.glob["embed"] = _normal_tensor(ws.shape_of("embed"), std, dt, (seed, model.name, "embed", -1), pool)
        ws.glob["lm_head"] = _normal_tensor(ws.shape_of("lm_head"), std, dt, (seed, model.name, "lm_head", -1), pool)
        ws.glob["final_norm"] = gain("final_norm", -1)


# ----------------------------------------------------------------------------------------------------------
# per-step inputs and initial state


def start_tokens(w: Workload, seed: int = 0) -> np.ndarray:
    """One start token per row, uniform over the vocabulary."""
    return _gen(seed, w.name, "start_tokens").integers(0, w.model.vocab, size=w.rows).astype(np.int32)


def prefill_tokens(w: Workload, seed: int = 0) -> np.ndarray:
    """Uniform random prompt tokens [rows, prefill_len] for workloads that start with a token prefill."""
    return _gen(seed, w.name, "prefill_tokens").integers(0, w.model.vocab, size=(w.rows, w.prefill_len)).astype(
        np.int32)


def start_positions(w: Workload, seed: int = 0) -> np.ndarray:
    """Position of each row's first decode step."""
    if w.start == "token_at_0":
        return np.zeros(w.rows, np.int32)
    if w.start == "prefill_tokens":
        return np.full(w.rows, w.prefill_len, np.int32)
    if w.pos_hi > 0:
        return _gen(seed, w.name, "start_positions").integers(w.pos_lo, w.pos_hi + 1, size=w.rows).astype(np.int32)
    return np.full(w.rows, w.prefill_len, np.int32)


def kv_prefill(w: Workload, layer: int, row: int, which: str, n_pos: int, seed: int = 0,
               std: float = 1.0) -> np.ndarray:
    """K or V contents ~ N(0, std^2) for logical positions [0, n_pos) of one row and layer: [n_kv, n_pos, hd]."""
    m = w.model
    return _normal_tensor((m.n_kv_heads, n_pos, m.head_dim), std, w.kv_dtype,
                          (seed, m.name, "kv_prefill", which, layer, row), None)


def page_table(w: Workload, seed: int = 0) -> np.ndarray:
    """Paged layout: one random permutation of the pool's pages, cut into consecutive per-row chunks.

    Returns int32 [rows, cap // page_size]: logical page -> physical page. Rows own disjoint pages.
    """
    assert w.kv_layout == "paged"
    need = w.rows * w.pages_per_row
    if need > w.pool_pages:
        raise ValueError(f"pool of {w.pool_pages} pages cannot hold {w.rows} rows x {w.pages_per_row} pages")
    perm = _gen(seed, w.name, "page_table").permutation(w.pool_pages).astype(np.int32)
    return perm[:need].reshape(w.rows, w.pages_per_row)
