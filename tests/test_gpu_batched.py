"""GPU parity of the batched decode step (more than 4 rows: projections on the matrix cores) and of the paged
K/V layout, against the CPU oracle, through the C ABI.

Rows of one step are independent sequences: each row r is checked against the oracle run on that row alone, with
its own start position and its own K/V history. Paged K/V (the pool addressed through a per-row page table,
"ScatterUpdate through a WriteMap") must give bit-identical logits for any page table, since it only moves data.
"""
from dataclasses import replace

import numpy as np
import pytest

import synth
from tests.ds3_testlib import Lockstep, log, make_engine

pytestmark = pytest.mark.gpu


def _layers2(base_name, **kw):
    base = synth.workload(base_name)
    return synth.small_variant(base, n_layers=2, vocab=4096, **kw)


def _run(w, ws, start_pos, steps, slot_map=None):
    eng = make_engine(w, ws)
    try:
        if slot_map is not None:
            eng.set_slot_map(slot_map)
        ls = Lockstep(w, ws, eng)
        ls.prefill_random_kv(list(start_pos))
        tokens = synth.start_tokens(w)
        pos = np.array(start_pos, np.int32)
        outs = []
        for _ in range(steps):
            got, ref, _ = ls.step(tokens, pos)
            outs.append(got)
            tokens = ref.argmax(axis=1).astype(np.int32)
            for r in range(w.rows):
                ls.check_kv(w.model.n_layers - 1, r, int(pos[r]), 1)
            pos = pos + 1
        log(w.name, "rows", w.rows, "max logits err", f"{ls.max_err:.3e}", "greedy checked", ls.greedy_checked)
        return outs
    finally:
        eng.close()


def test_eight_rows_contiguous_mfma():
    """8 rows (the 8B-shaped layers, 2 layers): contiguous K/V, per-row start positions spread over the capacity."""
    w = replace(_layers2("llama8b-bf16-r8-cap32768", cap=4096), name="llama8b-2l-r8")
    ws = synth.make_weights(w.model, gains="random")
    _run(w, ws, [1, 100, 511, 1024, 2047, 3000, 4000, 4090], steps=4)


def test_five_rows_padded_tile():
    """5 rows: the matrix-core tile is padded from 5 to 16 activation rows; padding must never reach an output."""
    w = replace(_layers2("llama8b-bf16-r8-cap32768", cap=1024), rows=5, name="llama8b-2l-r5")
    ws = synth.make_weights(w.model, gains="random")
    _run(w, ws, [0, 7, 300, 513, 1000], steps=3)


@pytest.mark.parametrize("rows", [3, 4])
def test_three_and_four_rows_of_the_8b_shape(rows):
    """3 and 4 rows of the 8B-shaped layers: the vector path's activations (rows x 14336 floats) do not fit the LDS,
    so these steps run their projections on the matrix cores (padded tile), and must match the oracle."""
    w = replace(_layers2("llama8b-bf16-r8-cap32768", cap=2048), rows=rows, name=f"llama8b-2l-r{rows}")
    ws = synth.make_weights(w.model, gains="random")
    _run(w, ws, [0, 1000, 2040, 513][:rows], steps=3)


def test_sixteen_rows_paged_and_page_table_invariance():
    """16 rows over a paged pool (16-token pages): parity with the oracle, and bit-identical logits for two
    different page tables (identity and a random permutation of the pool)."""
    base = synth.workload("llama8b-bf16-r16-paged")
    w = replace(synth.small_variant(base, n_layers=2, vocab=4096, cap=1024, pool_pages=16 * 64 + 37),
                name="llama8b-2l-r16-paged")
    ws = synth.make_weights(w.model, gains="random")
    rng = np.random.default_rng(5)
    start = rng.integers(1, 1000, size=16)
    perm = synth.page_table(w)
    ident = np.arange(16 * 64, dtype=np.int32).reshape(16, 64)
    a = _run(w, ws, start, steps=3, slot_map=perm)
    b = _run(w, ws, start, steps=3, slot_map=ident)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), "page table changed the logits"


def test_paged_single_row_gemv_path():
    """Paged K/V with one row (vector path) and an explicit WriteMap per step."""
    base = synth.workload("llama8b-bf16-r16-paged")
    w = replace(synth.small_variant(base, n_layers=2, vocab=4096, cap=512, pool_pages=97), rows=1,
                name="llama8b-2l-paged-r1")
    ws = synth.make_weights(w.model, gains="random")
    table = np.random.default_rng(3).permutation(97)[:32].astype(np.int32).reshape(1, 32)
    eng = make_engine(w, ws)
    try:
        eng.set_slot_map(table)
        ls = Lockstep(w, ws, eng)
        ls.prefill_random_kv([200])
        tok = np.array([11], np.int32)
        for p in (200, 201, 511):
            wm = np.array([table[0, p // 16] * 16 + p % 16], np.int32)
            got, ref, _ = ls.step(tok, np.array([p], np.int32), write_map=wm)
            ls.check_kv(1, 0, p, 1)
            tok = ref.argmax(axis=1).astype(np.int32)
    finally:
        eng.close()


def test_narrow_shapes_ragged_stream_k():
    """A narrow bf16 model (d_model 384, q width 256, ffn 640, vocab 1152, 6 rows) puts every matrix-core kernel on
    its uneven paths: fewer blocks than CUs (12, 6, 30 and 15 blocks for the projections, 9 for the head), quads
    whose inputs span up to 5 blocks, d_model not a multiple of the prep kernels' 512 inputs, d_model != q width,
    and G = 2 heads per kv head."""
    m = synth.ModelShape("narrow", 2, 384, 4, 2, 64, 640, 1152, 1e-5, 1e4, "bf16")
    w = synth.Workload("narrow-bf16-r6", m, 6, 256, "contiguous", "bf16", 3, "random_kv")
    ws = synth.make_weights(w.model, gains="random")
    _run(w, ws, [0, 5, 64, 127, 200, 255 - 3], steps=3)
