"""The C-ABI library on the host (no GPU): it loads, exports every function
that include/ds_decode.h declares, and its pure-host queries agree with the
arena and cache formats."""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import synth
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ds_decode.h")


@pytest.fixture(scope="module")
def dsa():
    lib = os.path.join(ROOT, "decode_step_02_amd", "libds_decode.so")
    if not os.path.exists(lib):  # build.py by path: the package does not import without the library
        subprocess.run([sys.executable, os.path.join(ROOT, "decode_step_02_amd", "build.py")], check=True)
    import decode_step_02_amd
    return decode_step_02_amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_function_is_exported(dsa):
    names = declared_functions()
    assert len(names) >= 18
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (ds_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(dsa.exported_symbols())


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_layout_queries_match_the_arena_format(dsa, name):
    w = synth.WORKLOADS[name]
    cfg = dsa.ds_config.of(w.model)
    table, total = synth.tensor_table(w.model)
    assert dsa.ds_weights_bytes(cfg) == total
    assert dsa.ds_weights_count(cfg) == len(table)
    assert dsa.ds_weights_offsets(cfg) == [t[1] for t in table]
    m = w.model
    assert dsa.ds_kv_cache_bytes(cfg, w.batch, w.ctx) == 4 * m.n_layers * 2 * w.batch * m.n_kv_heads * w.ctx * m.head_dim
    assert dsa.ds_workspace_bytes(cfg, w.batch, w.ctx) > 0


def test_invalid_configs_are_rejected(dsa):
    base = synth.TINY
    bad = {
        "n_kv_heads": 3,       # 4 % 3 != 0
        "head_dim": 15,        # odd
        "dim": 0,
        "weight_dtype": 7,
        "head_dim_12": None,   # not a multiple of 8
    }
    import dataclasses
    for k, v in bad.items():
        shape = dataclasses.replace(base, head_dim=12) if v is None else dataclasses.replace(base, **{k: v})
        cfg = dsa.ds_config.of(shape)
        assert dsa.ds_weights_bytes(cfg) == 0, k
        assert dsa.ds_last_error() != ""
    # head sizes the attention kernels are not built for
    for hd in (8, 24, 48, 96, 512):
        cfg = dsa.ds_config.of(dataclasses.replace(base, head_dim=hd, dim=128, hidden_dim=192))
        assert dsa.ds_weights_bytes(cfg) == 0 and "head_dim" in dsa.ds_last_error(), hd
    for hd in (16, 32, 64, 128, 256):
        assert dsa.ds_weights_bytes(dsa.ds_config.of(dataclasses.replace(base, head_dim=hd, dim=128,
                                                                         hidden_dim=192))) > 0, hd
    # bf16 rows of 172 elements are not whole 16-byte chunks
    cfg = dsa.ds_config.of(dataclasses.replace(base, weight_dtype=synth.BF16))
    assert dsa.ds_weights_bytes(cfg) == 0 and "16-byte" in dsa.ds_last_error()
    with pytest.raises(dsa.DSError):
        dsa.ds_weights_offsets(dsa.ds_config.of(dataclasses.replace(base, n_kv_heads=3)))


@pytest.mark.parametrize("dt", ["q8", "q4"])
@pytest.mark.parametrize("name", ["llama135m_p5", "llama8b_p4096"])
def test_q8_layout_queries_match_the_arena_format(dsa, name, dt):
    """Block-quantised int8 / int4 matrices (DS_Q8, DS_Q4): the values (one
    byte, or half a byte each), then one fp32 scale per 32 values of a row
    from the next 256-byte boundary."""
    import dataclasses
    m = dataclasses.replace(synth.WORKLOADS[name].model, weight_dtype=synth.Q8 if dt == "q8" else synth.Q4)
    cfg = dsa.ds_config.of(m)
    table, total = synth.tensor_table(m)
    assert dsa.ds_weights_bytes(cfg) == total
    assert dsa.ds_weights_offsets(cfg) == [t[1] for t in table]
    V, d = m.vocab_size, m.dim
    vb = V * d if dt == "q8" else V * d // 2
    assert table[1][1] == ((vb + 255) // 256 * 256 + 4 * V * d // 32 + 255) // 256 * 256


def test_q8_needs_rows_of_whole_blocks(dsa):
    import dataclasses
    cfg = dsa.ds_config.of(dataclasses.replace(synth.TINY, weight_dtype=synth.Q8))  # hidden_dim 172
    assert dsa.ds_weights_bytes(cfg) == 0 and "multiples of 32" in dsa.ds_last_error()
    cfg = dsa.ds_config.of(dataclasses.replace(synth.TINY, weight_dtype=synth.Q8, hidden_dim=192))
    assert dsa.ds_weights_bytes(cfg) > 0
