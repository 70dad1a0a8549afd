"""The C-ABI library loads without a GPU and exports every function include/ds3.h declares.

No compute call is made here; argument and configuration checks that never touch a device are exercised.
"""
import ctypes
import os
import re

import pytest

import decode_step_03_amd as ds3
from decode_step_03_amd import _ds3 as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "ds3.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ds3_[a-z_]+)\s*\(", src)))


def test_header_declares_the_executor_contract():
    names = _declared_functions()
    for required in ("ds3_load_weights", "ds3_step", "ds3_reset_state", "ds3_stats_get", "ds3_destroy"):
        assert required in names


def test_library_exports_every_declared_function():
    lib = ds3.load_library()
    names = _declared_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # the Python binding wraps each of them under the same name
    assert sorted(n for n, _, _ in C.SIGNATURES) == names


def test_struct_layouts_match_the_header(tmp_path):
    """sizeof and field offsets of the ABI structs, as a C compiler lays them out from include/ds3.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"ds3_config": C.ds3_config, "ds3_weight_src": C.ds3_weight_src, "ds3_stats": C.ds3_stats,
               "ds3_buffer_req": C.ds3_buffer_req, "ds3_kernel_time": C.ds3_kernel_time}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ds3.h"', "int main(void) {"]
    for name, py in structs.items():
        lines.append(f'  printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for name, py in structs.items():
        assert int(out[name]) == ctypes.sizeof(py), name
        for f, _ in py._fields_:
            assert int(out[f"{name}.{f}"]) == getattr(py, f).offset, f"{name}.{f}"


def _cfg(**kw):
    base = dict(n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn_dim=14336, vocab=128256,
                rms_eps=1e-5, rope_theta=5e5, rows=1, cap=8192)
    base.update(kw)
    return ds3.make_config(**base)


def test_query_buffers_sizes():
    reqs = C.ds3_query_buffers(_cfg())
    by = {r.name.decode(): r.bytes for r in reqs}
    assert by["kv"] == 2 * 32 * 8 * 8192 * 128 * 2
    assert by["logits"] == 128256 * 4
    # packed weights hold every parameter (bf16) plus fp32 norm gains, with 256-byte alignment padding
    n_params = 32 * (4096 * 6144 + 4096 * 4096 + 3 * 4096 * 14336) + 2 * 128256 * 4096
    assert n_params * 2 < by["weights"] < n_params * 2 + 4 * 1024 * 1024
    paged = C.ds3_query_buffers(_cfg(rows=2, cap=16384, kv_layout="paged", page_size=16, pool_pages=16384))
    assert {r.name.decode(): r.bytes for r in paged}["kv"] == 2 * 32 * 16384 * 8 * 16 * 128 * 2


@pytest.mark.parametrize("field,value,word", [("head_dim", 96, "head_dim"), ("rows", 0, "rows"),
                                              ("n_kv_heads", 5, "n_q_heads"), ("vocab", 1001, "vocab"),
                                              ("d_model", 4092, "d_model")])
def test_unsupported_configs_name_the_field(field, value, word):
    cfg = _cfg()
    setattr(cfg, field, value)
    with pytest.raises(ds3.DS3Error) as ei:
        C.ds3_query_buffers(cfg)
    assert ei.value.status == C.DS3_E_UNSUPPORTED and word in ei.value.message


def test_create_rejects_bad_buffers_without_touching_a_device():
    with pytest.raises(ds3.DS3Error) as ei:
        C.ds3_create(_cfg(), [0, 0, 0, 0], None)
    assert ei.value.status == C.DS3_E_INVALID


def test_probe_read_rejects_bad_arguments_without_touching_a_device():
    """The streaming-read probe validates before any HIP call: null pointers and sizes that are not a positive
    multiple of 16 bytes are DS3_E_INVALID."""
    for buf, n, sink in [(0, 4096, 4096), (4096, 4096, 0), (4096, 17, 4096), (4096, 0, 4096)]:
        with pytest.raises(ds3.DS3Error) as ei:
            C.ds3_probe_read(buf, n, sink, None)
        assert ei.value.status == C.DS3_E_INVALID and "probe" in ei.value.message
