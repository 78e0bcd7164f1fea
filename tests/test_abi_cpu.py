"""Host-only checks of the C ABI: the library loads, exports every declared symbol, and its
configuration validation returns the documented status codes without touching a GPU."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "hybrid_decode_replay_amd", "libreplayssm.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libreplayssm.so not built")


def test_every_declared_function_is_exported():
    from hybrid_decode_replay_amd import binding as rb
    names = rb.header_functions()
    assert len(names) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(LIB)
    for n in names:
        getattr(lib, n)


def test_abi_version_and_status_strings():
    from hybrid_decode_replay_amd import binding as rb
    assert rb.lib().replay_abi_version() == rb.ABI_VERSION
    for s in range(9):
        assert rb.lib().replay_status_str(s)
    assert rb.lib().replay_status_str(99) == b"unknown status"


def _cfg(**kw):
    from hybrid_decode_replay_amd import binding as rb
    base = dict(kind=rb.MAMBA2, batch=256, nheads=128, ngroups=8, head_dim=64, state_dim=128, buf_cap=16,
                io_dtype=rb.BF16)
    base.update(kw)
    return rb.make_config(**base)


def test_config_validation_codes():
    from hybrid_decode_replay_amd import binding as rb
    assert rb.config_check(_cfg()) == rb.OK
    cases = [
        (dict(batch=0), rb.ERR_SHAPE), (dict(ngroups=3), rb.ERR_SHAPE), (dict(head_dim=40), rb.ERR_SHAPE),
        (dict(head_dim=272), rb.ERR_SHAPE), (dict(state_dim=96), rb.ERR_SHAPE), (dict(buf_cap=0), rb.ERR_SHAPE),
        (dict(buf_cap=17), rb.ERR_SHAPE), (dict(io_dtype=rb.F16), rb.ERR_DTYPE), (dict(kind=7), rb.ERR_ARG),
        (dict(flags=0x80), rb.ERR_ARG), (dict(read_copy=rb.BF16), rb.ERR_DTYPE),
        (dict(flags=rb.FLAG_MX_SCALE_CEIL), rb.ERR_ARG),
        (dict(flags=rb.FLAG_MX_SCALE_CEIL, read_copy=rb.FP8_E4M3), rb.ERR_ARG),
    ]
    for kw, want in cases:
        assert rb.config_check(_cfg(**kw)) == want, kw
        assert rb.state_bytes(_cfg(**kw)) == 0
        assert rb.lib().replay_last_error()
    assert rb.config_check(_cfg(flags=rb.FLAG_MX_SCALE_CEIL, read_copy=rb.MXFP4)) == rb.OK
    bad = _cfg()
    bad.abi_version = 2
    assert rb.config_check(bad) == rb.ERR_ARG


def test_state_bytes_layout_matches_sizes():
    from hybrid_decode_replay_amd import binding as rb
    B, H, G, P, N, cap = 256, 128, 8, 64, 128, 16
    n = rb.state_bytes(_cfg())
    ckpt = B * H * P * N * 4
    bufs = 2 * (B * H * cap * P * 2 + B * G * cap * N * 2 + B * H * cap * 4)
    assert ckpt + bufs <= n <= ckpt + bufs + 16 * 256 + 2 * 3 * B * 4 + 256
    assert n % 256 == 0


def test_null_and_phase_free_errors():
    from hybrid_decode_replay_amd import binding as rb
    L = rb.lib()
    assert L.replay_decode_step(None, None, None, None) == rb.ERR_ARG
    assert L.replay_flush(None, None, None) == rb.ERR_ARG
    assert L.replay_spec_commit(None, None, None) == rb.ERR_ARG
    assert L.replay_state_free(None) == rb.ERR_ARG
    assert L.replay_state_phase(None) == -1
    cfg = _cfg()
    out = ctypes.c_void_p()
    assert L.replay_state_alloc(ctypes.byref(cfg), None, 0, None, ctypes.byref(out)) == rb.ERR_ARG
    assert L.replay_state_alloc(ctypes.byref(cfg), ctypes.c_void_p(0x1010), 1 << 40, None,
                                ctypes.byref(out)) == rb.ERR_ALIGN
    assert L.replay_state_alloc(ctypes.byref(cfg), ctypes.c_void_p(0x1000), 100, None,
                                ctypes.byref(out)) == rb.ERR_ALIGN
    assert L.replay_stream_copy(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 17, None) == rb.ERR_ALIGN
