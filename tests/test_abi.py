"""The C ABI without a GPU: the library loads, exports every function
include/libblock.h declares, its struct layouts match the Python binding,
and configuration errors are reported before any device call."""
import ctypes as C
import os
import re
import subprocess

import pytest

from transformer_decoder_block_amd import binding as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libblock.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(blk_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    lib = L.load()
    names = declared_functions()
    assert "blk_create" in names and "blk_forward" in names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    fields = {
        "blk_config": [f for f, _ in L.blk_config._fields_],
        "blk_weights": [f for f, _ in L.blk_weights._fields_],
        "blk_taps": [f for f, _ in L.blk_taps._fields_],
        "blk_io": [f for f, _ in L.blk_io._fields_],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "libblock.h"',
             'int main(void) {']
    for s, fs in fields.items():
        lines.append(f'printf("{s} %zu\\n", sizeof({s}));')
        for f in fs:
            lines.append(f'printf("{s}.{f} %zu\\n", offsetof({s}, {f}));')
    lines.append("return 0; }")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True,
                                                 text=True, check=True).stdout.splitlines())
    for s, fs in fields.items():
        cls = getattr(L, s)
        assert int(got[s]) == C.sizeof(cls), s
        for f in fs:
            assert int(got[f"{s}.{f}"]) == getattr(cls, f).offset, (s, f)


def test_abi_version_and_status_names():
    assert L.blk_abi_version() == L.ABI_VERSION == 6
    for code, name in enumerate(["BLK_OK", "BLK_E_NULL", "BLK_E_CONFIG", "BLK_E_SHAPE",
                                 "BLK_E_ALIGN", "BLK_E_DTYPE", "BLK_E_OOM", "BLK_E_HIP"]):
        assert L.blk_status_str(code) == name


def good_config(**kw):
    c = L.blk_config(dtype=L.BLK_BF16, hidden=256, num_heads=4, num_kv_heads=2,
                     head_dim=64, mlp_kind=L.BLK_MLP_SWIGLU, intermediate=512,
                     rms_eps=1e-5, rope_theta=1e4, use_rope=1, max_batch=1, max_seq=16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


BAD = [
    dict(dtype=7), dict(hidden=100), dict(hidden=16384), dict(num_heads=5),
    dict(head_dim=96), dict(rms_eps=0.0), dict(sliding_window=-1),
    dict(head_gate_dim=3), dict(max_seq=0), dict(intermediate=12),
    dict(mlp_kind=9),
    dict(mlp_kind=L.BLK_MLP_MOE, num_experts=0, top_k=1, moe_intermediate=64),
    dict(mlp_kind=L.BLK_MLP_MOE, num_experts=300, top_k=1, moe_intermediate=64),
    dict(mlp_kind=L.BLK_MLP_MOE, num_experts=8, top_k=9, moe_intermediate=64),
    dict(mlp_kind=L.BLK_MLP_MOE, num_experts=8, top_k=2, moe_intermediate=60),
    dict(max_batch=4096, max_seq=65536),
]


@pytest.mark.parametrize("kw", BAD, ids=[str(b) for b in BAD])
def test_create_rejects_bad_config(kw):
    st, h = L.blk_create(good_config(**kw))
    assert st == L.BLK_E_CONFIG
    assert not h
    assert L.blk_last_error()


def test_create_rejects_null():
    lib = L.load()
    assert lib.blk_create(None, None) == L.BLK_E_NULL
    assert "NULL" in L.blk_last_error()
    assert lib.blk_forward(None, None, None, None, None) == L.BLK_E_NULL
    assert lib.blk_forward_layers(None, None, None, 1, None) == L.BLK_E_NULL
    assert lib.blk_profile_end(None, 0, None, None, None) == -1
    lib.blk_destroy(None)  # ignored


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """With no built library the binding raises instead of falling back to
    anything else."""
    from transformer_decoder_block_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libblock.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.load()
