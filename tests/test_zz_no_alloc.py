"""ds3_write_kv_noalloc (the K/V write for callers that cannot allocate) against ds3_write_kv: two engines of the
same configuration take the same K/V contents, one through each entry point, in two calls in a row (the second
smaller and elsewhere); the states read back and the logits of a decode step on them must be bit-identical. Sizes
beyond the fixed array are refused before anything is written."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from decode_step_03_amd import DS3Error, _ds3 as C
from tests.ds3_testlib import log, make_engine

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "tiny-fp32":
        return synth.workload("tiny-fp32"), None
    base = synth.workload("llama8b-bf16-r16-paged")
    w = replace(synth.small_variant(base, n_layers=2, vocab=1024, cap=4096, pool_pages=600), rows=2,
                name="noalloc-paged")
    return w, synth.page_table(w)


@pytest.mark.parametrize("name", ["tiny-fp32", "bf16-paged"])
def test_noalloc_write_kv_matches_write_kv(name):
    w, table = _case(name)
    ws = synth.make_weights(w.model)
    a, b = make_engine(w, ws), make_engine(w, ws)
    try:
        if table is not None:
            a.set_slot_map(table)
            b.set_slot_map(table)
        row = w.rows - 1
        calls = [(5, min(300, w.cap - 5)), (w.cap // 2, 37)]   # the second call smaller, elsewhere
        for li in range(w.model.n_layers):
            for ci, (pos0, n) in enumerate(calls):
                K = synth.kv_prefill(w, li, row, "k", n, seed=10 + ci)
                V = synth.kv_prefill(w, li, row, "v", n, seed=20 + ci)
                a.write_kv(li, row, pos0, K, V)
                b.write_kv_noalloc(li, row, pos0, K, V)
                ka, va = a.read_kv(li, row, 0, w.cap)
                kb, vb = b.read_kv(li, row, 0, w.cap)
                assert np.array_equal(ka, kb) and np.array_equal(va, vb), f"layer {li} call {ci}: states differ"
                assert np.array_equal(kb[:, pos0:pos0 + n], K) and np.array_equal(vb[:, pos0:pos0 + n], V)
        tok = np.arange(w.rows, dtype=np.int32) + 3
        pos = np.full(w.rows, w.cap // 2 + 37, np.int32)
        la, _ = a.step(tok, pos)
        la = la.copy()
        lb, _ = b.step(tok, pos)
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), "logits differ"
        # beyond the fixed array: refused, nothing written
        kvb = 2 if w.kv_dtype == "bf16" else 4
        n_big = C.DS3_NOALLOC_MAX_BYTES // (2 * w.model.n_kv_heads * w.model.head_dim * kvb) + 1
        if n_big <= w.cap:
            K = np.ones((w.model.n_kv_heads, n_big, w.model.head_dim), np.uint16 if kvb == 2 else np.float32)
            with pytest.raises(DS3Error) as ei:
                b.write_kv_noalloc(0, row, 0, K, K)
            assert ei.value.status == C.DS3_E_INVALID and "scratch" in ei.value.message
        log(name, "noalloc K/V writes identical; oversize refused" if n_big <= w.cap else "noalloc K/V writes identical")
    finally:
        a.close()
        b.close()
