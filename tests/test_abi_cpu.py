"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching a device."""
import ctypes

import numpy as np
import pytest

import looped_transformer_amd as tl
from tests.harness import ensure_built, make_config
import synth


@pytest.fixture(scope="module")
def L():
    ensure_built()
    return tl.lib()


def test_exports_every_header_symbol(L):
    names = tl.header_symbols()
    assert {"tl_load_weights", "tl_forward", "tl_decode_step", "tl_free", "tl_decode_run"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def _load(L, cfg, w=None):
    out = ctypes.c_void_p()
    return L.tl_load_weights(ctypes.byref(cfg) if cfg is not None else None,
                             ctypes.byref(w) if w is not None else None,
                             tl.ALLOC_FN(0), tl.DEALLOC_FN(0), None, None, ctypes.byref(out))


def test_null_arguments_rejected(L):
    assert _load(L, None) == tl.TL_E_ARG
    assert "NULL" in tl.tl_last_error()
    cfg = make_config(synth.SPECS[1])
    assert _load(L, cfg, None) == tl.TL_E_ARG
    assert L.tl_forward(None, 1, None, None, 1, None, None, 0, None, None, None, None, None) == tl.TL_E_ARG
    assert L.tl_decode_step(None, 1, None, None, None, None, None, None, None, None, None) == tl.TL_E_ARG
    assert L.tl_decode_step_noalloc(None, 1, None, None, None, None, None, None, None, None) == tl.TL_E_ARG
    assert L.tl_decode_run(None, 1, None, 1, None, None, None, None, None, 1, None) == tl.TL_E_ARG
    assert L.tl_decode_step_ee(None, 1, None, None, None, None, None, None, None, None, None) == tl.TL_E_ARG
    assert L.tl_append(None, 1, None, None, None, None, None, None, None, None, None) == tl.TL_E_ARG
    assert L.tl_lane_fork(None, 0, 1, 1, 0, None) == tl.TL_E_ARG
    assert L.tl_speculate(None, 1, None, 2, 8, 4, 8, None, None, None) == tl.TL_E_ARG
    assert L.tl_lane_release(None, 0) == tl.TL_E_ARG
    assert L.tl_timing_enable(None, 1) == tl.TL_E_ARG
    assert L.tl_timing_read(None, None, None) == tl.TL_E_ARG
    assert L.tl_timing_read_kernels(None, None, None) == tl.TL_E_ARG


def _weights_struct():
    blk = (tl.tl_block_weights * 2)()
    dummy = np.zeros(16, np.float32)
    for i in range(2):
        blk[i] = tl.tl_block_weights(*([dummy.ctypes.data] * 7))
    return tl.tl_weights(dummy.ctypes.data, dummy.ctypes.data, dummy.ctypes.data, blk), dummy


@pytest.mark.parametrize("field,value,status", [
    ("d_model", 65, tl.TL_E_ARG),              # d != H * dh
    ("n_loop", 0, tl.TL_E_ARG),
    ("max_L", 0, tl.TL_E_ARG),
    ("act_dtype", 7, tl.TL_E_UNSUPPORTED),
    ("boundary_dtype", tl.TL_DT_F16, tl.TL_E_UNSUPPORTED),
])
def test_config_validation(L, field, value, status):
    cfg = make_config(synth.SPECS[1])
    setattr(cfg, field, value)
    w, keep = _weights_struct()
    assert _load(L, cfg, w) == status
    assert tl.tl_last_error() != ""


def test_w4_constraints(L):
    spec = synth.SPECS[2]
    cfg = make_config(spec)
    cfg.ffn = 5632 + 64                       # not a multiple of 128
    w, keep = _weights_struct()
    assert _load(L, cfg, w) == tl.TL_E_UNSUPPORTED
    cfg = make_config(spec)
    cfg.act_dtype = cfg.boundary_dtype = tl.TL_DT_BF16   # INT4 needs fp16 operands
    assert _load(L, cfg, w) == tl.TL_E_UNSUPPORTED
    cfg = make_config(synth.SPECS[5])
    cfg.loop_fp16_body = 1                    # body cache only for INT4 loops
    assert _load(L, cfg, w) == tl.TL_E_ARG


_LOG_PROBE = """
import looped_transformer_amd as tl
L = tl.lib()
assert L.tl_forward(None, 1, None, None, 1, None, None, 0, None, None, None, None, None) == tl.TL_E_ARG
"""


@pytest.mark.parametrize("level,printed", [(None, False), ("0", False), ("1", True), ("2", True), ("7", True),
                                           ("x", True)])
def test_log_level(L, level, printed):
    """TL_LOG_LEVEL: errors reach stderr from level 1 (out-of-range values count as 1),
    nothing is printed when unset or 0."""
    import os
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("TL_LOG_LEVEL", None)
    if level is not None:
        env["TL_LOG_LEVEL"] = level
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _LOG_PROBE], cwd=root, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert ("[tl] error -1: NULL argument" in r.stderr) == printed, r.stderr
