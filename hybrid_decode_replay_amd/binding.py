"""ctypes binding of libreplayssm.so (include/replayssm.h): argument marshalling only.

Every step of the decode path runs in the HIP library; this module turns torch
tensors into device pointers and the current HIP stream into a handle, and
turns non-OK status codes into exceptions.  Importing it without the built
library raises immediately: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(_HERE, "libreplayssm.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "replayssm.h")

if not os.path.exists(LIBPATH):
    raise ImportError(f"{LIBPATH} is not built; build it first: python -m hybrid_decode_replay_amd.build (hipcc, gfx950)")

_lib = ctypes.CDLL(LIBPATH)

# ---- constants (mirrors of the header's enums) --------------------------
ABI_VERSION = 1
MAX_BUF = 16
OK, ERR_ARG, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_STATE, ERR_CAPACITY, ERR_UNSUPPORTED, ERR_HIP = range(9)
MAMBA2, GDN = 0, 1
NONE, F32, F16, BF16, FP8_E4M3, MXFP4 = range(6)
DEVERR_COMMIT_CLAMPED = 0x1
FLAG_VALU_FOLD = 0x1
FLAG_QUANTIZED_CKPT = 0x2
FLAG_STAGGER_FLUSH = 0x4
FLAG_MX_SCALE_CEIL = 0x8


class ReplayConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "kind", "batch", "nheads", "ngroups", "head_dim", "state_dim", "buf_cap",
        "ckpt_dtype", "read_copy", "io_dtype", "flags")] + [("scale", ctypes.c_float)]


class ReplayInputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "B", "C", "dt", "A", "D", "q", "k", "v", "alpha", "beta")]


class ReplayLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "total_bytes", "ckpt_off", "ckpt_bytes", "rcopy_off", "rcopy_bytes", "rscale_off", "rscale_bytes")] + [
        ("buf_off", ctypes.c_uint64 * 4), ("buf_bytes", ctypes.c_uint64 * 4)] + [
        (n, ctypes.c_uint64) for n in ("book_off", "book_bytes", "err_off")]


_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_CP, _IP, _LP = ctypes.POINTER(ReplayConfig), ctypes.POINTER(ReplayInputs), ctypes.POINTER(ReplayLayout)

_SIGS = {
    "replay_abi_version": ([], _i32),
    "replay_status_str": ([_i32], ctypes.c_char_p),
    "replay_last_error": ([], ctypes.c_char_p),
    "replay_config_check": ([_CP], _i32),
    "replay_state_bytes": ([_CP], _sz),
    "replay_state_alloc": ([_CP, _vp, _sz, _vp, ctypes.POINTER(_vp)], _i32),
    "replay_state_free": ([_vp], _i32),
    "replay_state_layout": ([_vp, _LP], _i32),
    "replay_state_phase": ([_vp], _i32),
    "replay_load_checkpoint": ([_vp, _vp, _vp], _i32),
    "replay_load_checkpoint_f32": ([_vp, _vp, _vp], _i32),
    "replay_load_slots": ([_vp, _i32, ctypes.POINTER(_i32), _vp, _vp], _i32),
    "replay_decode_step_masked": ([_vp, _IP, _vp, _vp, _vp], _i32),
    "replay_spec_append_masked": ([_vp, _i32, _IP, _vp, _vp, _vp], _i32),
    "replay_stack_load_f32": ([_vp, ctypes.POINTER(_vp), _vp], _i32),
    "replay_stack_load_slots": ([_vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_vp), _vp], _i32),
    "replay_stack_decode_layer_masked": ([_vp, _i32, _IP, _vp, _vp, _vp], _i32),
    "replay_stack_spec_layer_masked": ([_vp, _i32, _i32, _IP, _vp, _vp, _vp], _i32),
    "replay_read_checkpoint": ([_vp, _vp, _vp], _i32),
    "replay_read_copy": ([_vp, _vp, _vp, _vp], _i32),
    "replay_read_book": ([_vp, _vp, _vp, _vp], _i32),
    "replay_decode_step": ([_vp, _IP, _vp, _vp], _i32),
    "replay_flush": ([_vp, _IP, _vp], _i32),
    "replay_spec_append": ([_vp, _i32, _IP, _vp, _vp], _i32),
    "replay_spec_commit": ([_vp, _vp, _vp], _i32),
    "replay_spec_rollback": ([_vp, _vp], _i32),
    "replay_conv_decode_step": ([_CP, _vp, _IP, _vp, _vp], _i32),
    "replay_conv_spec_step": ([_CP, _vp, _vp, _i32, _IP, _vp, _vp], _i32),
    "replay_conv_spec_restore": ([_CP, _vp, _vp, _i32, _vp, _vp], _i32),
    "replay_stack_create": ([ctypes.POINTER(_vp), _i32, _vp, ctypes.POINTER(_vp)], _i32),
    "replay_stack_free": ([_vp], _i32),
    "replay_stack_load": ([_vp, ctypes.POINTER(_vp), _vp], _i32),
    "replay_stack_decode_layer": ([_vp, _i32, _IP, _vp, _vp], _i32),
    "replay_stack_spec_layer": ([_vp, _i32, _i32, _IP, _vp, _vp], _i32),
    "replay_stack_flush": ([_vp, ctypes.POINTER(_IP), _vp], _i32),
    "replay_stack_commit": ([_vp, _vp, _vp], _i32),
    "replay_stack_rollback": ([_vp, _vp], _i32),
    "replay_stack_read_book": ([_vp, _vp, _vp, _vp], _i32),
    "replay_stack_layers": ([_vp], _i32),
    "replay_stack_next_layer": ([_vp], _i32),
    "replay_stack_phase": ([_vp], _i32),
    "replay_standin_linear": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp], _i32),
    "replay_standin_attention": ([_vp, ctypes.c_int64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float,
                                  _vp], _i32),
    "replay_stream_copy": ([_vp, _vp, _sz, _vp], _i32),
    "replay_stream_read": ([_vp, _sz, _vp, _vp], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def header_functions(path: str = HEADER):
    """Names of the functions the public header declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(replay_[a-z0-9_]+)\s*\(", text)) - {"replay_state"})


class ReplayError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.replay_last_error().decode() or _lib.replay_status_str(status).decode()
        super().__init__(f"{where}: {_lib.replay_status_str(status).decode()} ({msg})")


def _check(status, where):
    if status != OK:
        raise ReplayError(status, where)


def lib():
    return _lib


def make_config(kind, batch, nheads, ngroups, head_dim, state_dim, buf_cap=16, io_dtype=F32,
                read_copy=NONE, ckpt_dtype=F32, flags=0, scale=1.0):
    return ReplayConfig(ABI_VERSION, kind, batch, nheads, ngroups, head_dim, state_dim, buf_cap,
                        ckpt_dtype, read_copy, io_dtype, flags, scale)


def config_check(cfg: ReplayConfig) -> int:
    return _lib.replay_config_check(ctypes.byref(cfg))


def state_bytes(cfg: ReplayConfig) -> int:
    return _lib.replay_state_bytes(ctypes.byref(cfg))


# ---- torch marshalling -----------------------------------------------------
def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _io_torch_dtype(io):
    torch = _torch()
    return torch.bfloat16 if io == BF16 else torch.float32


def ckpt_torch_dtype(cfg: ReplayConfig):
    """torch dtype of logical checkpoints and conventional-baseline states for `cfg`."""
    torch = _torch()
    return {F16: torch.float16, FP8_E4M3: torch.float8_e4m3fn}.get(cfg.ckpt_dtype, torch.float32)


def make_inputs(cfg: ReplayConfig, tensors: dict, params: dict | None = None) -> ReplayInputs:
    """Pack a dict of device tensors into ReplayInputs.

    Mamba-2 keys: x, Bm, Cm, dt (io dtype) and A, D (fp32, via `params` or `tensors`).
    GDN keys: q, k, v (io dtype), alpha, beta (fp32)."""
    torch = _torch()
    iot = _io_torch_dtype(cfg.io_dtype)
    p = dict(params or {})
    p.update(tensors)
    ri = ReplayInputs()
    if cfg.kind == MAMBA2:
        ri.x = _ptr(p.get("x"), iot, "x")
        ri.B = _ptr(p.get("Bm"), iot, "Bm")
        ri.C = _ptr(p.get("Cm"), iot, "Cm")
        ri.dt = _ptr(p.get("dt"), iot, "dt")
        ri.A = _ptr(p.get("A"), torch.float32, "A")
        ri.D = _ptr(p.get("D"), torch.float32, "D")
    else:
        ri.q = _ptr(p.get("q"), iot, "q")
        ri.k = _ptr(p.get("k"), iot, "k")
        ri.v = _ptr(p.get("v"), iot, "v")
        ri.alpha = _ptr(p.get("alpha"), torch.float32, "alpha")
        ri.beta = _ptr(p.get("beta"), torch.float32, "beta")
    return ri


def _load_call(st, S, what):
    """Load a whole-state checkpoint: fp32 through the library's own rounding, or already in
    the checkpoint dtype.  No dtype conversion happens here."""
    torch = _torch()
    if tuple(S.shape) != st.ckpt_shape:
        raise ValueError(f"checkpoint shape {tuple(S.shape)}, expected {st.ckpt_shape}")
    if S.dtype == torch.float32:
        _check(_lib.replay_load_checkpoint_f32(st.h, _ptr(S, name="S"), _stream()), what + "_f32")
    elif S.dtype == st.ckt:
        _check(_lib.replay_load_checkpoint(st.h, _ptr(S, name="S"), _stream()), what)
    else:
        raise TypeError(f"checkpoint dtype {S.dtype}: pass fp32 or {st.ckt}")
    st._keep = S


def _slot_array(slots, B):
    """Host int32 array of slot indices (the library validates range and distinctness)."""
    vals = [int(b) for b in slots]
    return (_i32 * len(vals))(*vals)


def _mask_ptr(active, B):
    torch = _torch()
    if tuple(active.shape) != (B,):
        raise ValueError(f"active mask has shape {tuple(active.shape)}, expected ({B},)")
    return _ptr(active, torch.uint8, "active")


class ReplayState:
    """A replayed SSM layer state (checkpoint + input buffer) in caller-owned device memory."""

    def __init__(self, cfg: ReplayConfig, device="cuda"):
        torch = _torch()
        _check(_lib.replay_config_check(ctypes.byref(cfg)), "config")
        self.cfg = cfg
        self.device = torch.device(device)
        n = _lib.replay_state_bytes(ctypes.byref(cfg))
        self.mem = torch.empty(n + 256, dtype=torch.uint8, device=self.device)
        base = self.mem.data_ptr()
        self._off = (-base) % 256
        h = ctypes.c_void_p()
        _check(_lib.replay_state_alloc(ctypes.byref(cfg), ctypes.c_void_p(base + self._off), n, _stream(),
                                       ctypes.byref(h)), "replay_state_alloc")
        self.h = h
        self.iot = _io_torch_dtype(cfg.io_dtype)
        self.ckt = ckpt_torch_dtype(cfg)

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and h.value:
            _lib.replay_state_free(h)
            self.h = None

    # -- shapes
    @property
    def ckpt_shape(self):
        c = self.cfg
        return (c.batch, c.nheads, c.head_dim, c.state_dim)

    def layout(self) -> ReplayLayout:
        L = ReplayLayout()
        _check(_lib.replay_state_layout(self.h, ctypes.byref(L)), "replay_state_layout")
        return L

    def phase(self) -> int:
        return _lib.replay_state_phase(self.h)

    # -- checkpoint I/O
    def load_checkpoint(self, S):
        """S: logical [B][H][rows][cols] device tensor, either fp32 (the library rounds it to
        the checkpoint dtype: replay_load_checkpoint_f32) or already in the checkpoint dtype."""
        _load_call(self, S, "replay_load_checkpoint")

    def load_slots(self, slots, S):
        """Per-sequence arrival: sequences `slots` (ints) take the fp32 checkpoints S [n][H][rows][cols]
        (device); every other sequence keeps its state (replay_load_slots)."""
        torch = _torch()
        arr = _slot_array(slots, self.cfg.batch)
        c = self.cfg
        if tuple(S.shape) != (len(arr), c.nheads, c.head_dim, c.state_dim):
            raise ValueError(f"S has shape {tuple(S.shape)}, expected {(len(arr), c.nheads, c.head_dim, c.state_dim)}")
        _check(_lib.replay_load_slots(self.h, len(arr), arr, _ptr(S, torch.float32, "S"), _stream()),
               "replay_load_slots")
        self._keep = S

    def read_checkpoint(self):
        torch = _torch()
        out = torch.empty(self.ckpt_shape, dtype=self.ckt, device=self.device)
        _check(_lib.replay_read_checkpoint(self.h, _ptr(out), _stream()), "replay_read_checkpoint")
        return out

    def read_copy(self):
        torch = _torch()
        c = self.cfg
        codes = torch.empty(self.ckpt_shape, dtype=torch.uint8, device=self.device)
        scales = None
        if c.read_copy == MXFP4:
            scales = torch.empty((c.batch, c.nheads, c.head_dim, c.state_dim // 32), dtype=torch.uint8,
                                 device=self.device)
        _check(_lib.replay_read_copy(self.h, _ptr(codes), _ptr(scales), _stream()), "replay_read_copy")
        return codes, scales

    def read_book(self):
        """(len, pend, fc, err) as device tensors."""
        torch = _torch()
        book = torch.empty((3, self.cfg.batch), dtype=torch.int32, device=self.device)
        err = torch.empty((1,), dtype=torch.int32, device=self.device)
        _check(_lib.replay_read_book(self.h, _ptr(book), _ptr(err), _stream()), "replay_read_book")
        return book[0], book[1], book[2], err

    # -- the decode path
    def decode(self, tokens: dict, params: dict | None = None, y=None, active=None):
        """One decode token; with `active` (device uint8 [B]) only the sequences it marks step
        (replay_decode_step_masked), and the rows of y of the others are left as they were."""
        torch = _torch()
        c = self.cfg
        if y is None:
            y = torch.zeros((1, c.batch, c.nheads, c.head_dim), dtype=self.iot, device=self.device)
        ri = make_inputs(c, tokens, params)
        if active is None:
            _check(_lib.replay_decode_step(self.h, ctypes.byref(ri), _ptr(y, self.iot, "y"), _stream()),
                   "replay_decode_step")
        else:
            _check(_lib.replay_decode_step_masked(self.h, ctypes.byref(ri), _mask_ptr(active, c.batch),
                                                  _ptr(y, self.iot, "y"), _stream()), "replay_decode_step_masked")
        return y

    def flush(self, params: dict | None = None):
        ri = make_inputs(self.cfg, {}, params)
        _check(_lib.replay_flush(self.h, ctypes.byref(ri), _stream()), "replay_flush")

    def spec_append(self, k: int, drafts: dict, params: dict | None = None, y=None, active=None):
        torch = _torch()
        c = self.cfg
        if y is None:
            y = torch.zeros((k, c.batch, c.nheads, c.head_dim), dtype=self.iot, device=self.device)
        ri = make_inputs(c, drafts, params)
        if active is None:
            _check(_lib.replay_spec_append(self.h, int(k), ctypes.byref(ri), _ptr(y, self.iot, "y"), _stream()),
                   "replay_spec_append")
        else:
            _check(_lib.replay_spec_append_masked(self.h, int(k), ctypes.byref(ri), _mask_ptr(active, c.batch),
                                                  _ptr(y, self.iot, "y"), _stream()), "replay_spec_append_masked")
        return y

    def commit(self, accepted):
        torch = _torch()
        _check(_lib.replay_spec_commit(self.h, _ptr(accepted, torch.int32, "accepted"), _stream()),
               "replay_spec_commit")

    def rollback(self):
        _check(_lib.replay_spec_rollback(self.h, _stream()), "replay_spec_rollback")


class ReplayStack:
    """The SSM layers of one model with one shared bookkeeping set (replay_stack_* in the
    C ABI).  `layers` are ReplayState objects with equal batch and buf_cap; they stay
    referenced here, so they outlive the stack handle."""

    def __init__(self, layers):
        self.layers = list(layers)
        arr = (_vp * len(self.layers))(*[st.h.value for st in self.layers])
        h = _vp()
        _check(_lib.replay_stack_create(arr, len(self.layers), _stream(), ctypes.byref(h)), "replay_stack_create")
        self.h = h

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and h.value:
            _lib.replay_stack_free(h)
            self.h = None

    def free(self):
        """Unbind the layers now (each must then be loaded before it steps on its own)."""
        self.__del__()

    def next_layer(self) -> int:
        return _lib.replay_stack_next_layer(self.h)

    def phase(self) -> int:
        return _lib.replay_stack_phase(self.h)

    def load(self, checkpoints):
        """checkpoints[l]: layer l's logical checkpoint, all fp32 (rounded by the library to each
        layer's checkpoint dtype: replay_stack_load_f32) or all in the layers' checkpoint dtypes."""
        torch = _torch()
        for st, S in zip(self.layers, checkpoints, strict=True):
            if tuple(S.shape) != st.ckpt_shape:
                raise ValueError(f"checkpoint shape {tuple(S.shape)}, expected {st.ckpt_shape}")
        f32 = all(S.dtype == torch.float32 for S in checkpoints)
        if not f32 and any(S.dtype != st.ckt for st, S in zip(self.layers, checkpoints)):
            raise TypeError("stack checkpoints must all be fp32 or all in their layers' checkpoint dtypes")
        arr = (_vp * len(checkpoints))(*[_ptr(S, name="S").value for S in checkpoints])
        if f32:
            _check(_lib.replay_stack_load_f32(self.h, arr, _stream()), "replay_stack_load_f32")
        else:
            _check(_lib.replay_stack_load(self.h, arr, _stream()), "replay_stack_load")
        self._keep = list(checkpoints)

    def load_slots(self, slots, checkpoints):
        """Per-sequence arrival in every layer: checkpoints[l] is layer l's fp32 [n][H][rows][cols]."""
        torch = _torch()
        arr = _slot_array(slots, self.layers[0].cfg.batch)
        for st, S in zip(self.layers, checkpoints, strict=True):
            c = st.cfg
            if tuple(S.shape) != (len(arr), c.nheads, c.head_dim, c.state_dim):
                raise ValueError("slot checkpoint shape mismatch")
        ptrs = (_vp * len(checkpoints))(*[_ptr(S, torch.float32, "S").value for S in checkpoints])
        _check(_lib.replay_stack_load_slots(self.h, len(arr), arr, ptrs, _stream()), "replay_stack_load_slots")
        self._keep = list(checkpoints)

    def decode_layer(self, layer: int, tokens: dict, params: dict | None = None, y=None, active=None):
        torch = _torch()
        st = self.layers[layer]
        c = st.cfg
        if y is None:
            y = torch.zeros((1, c.batch, c.nheads, c.head_dim), dtype=st.iot, device=st.device)
        ri = make_inputs(c, tokens, params)
        if active is None:
            _check(_lib.replay_stack_decode_layer(self.h, int(layer), ctypes.byref(ri), _ptr(y, st.iot, "y"),
                                                  _stream()), "replay_stack_decode_layer")
        else:
            _check(_lib.replay_stack_decode_layer_masked(self.h, int(layer), ctypes.byref(ri),
                                                         _mask_ptr(active, c.batch), _ptr(y, st.iot, "y"),
                                                         _stream()), "replay_stack_decode_layer_masked")
        return y

    def spec_layer(self, layer: int, k: int, drafts: dict, params: dict | None = None, y=None, active=None):
        torch = _torch()
        st = self.layers[layer]
        c = st.cfg
        if y is None:
            y = torch.zeros((k, c.batch, c.nheads, c.head_dim), dtype=st.iot, device=st.device)
        ri = make_inputs(c, drafts, params)
        if active is None:
            _check(_lib.replay_stack_spec_layer(self.h, int(layer), int(k), ctypes.byref(ri), _ptr(y, st.iot, "y"),
                                                _stream()), "replay_stack_spec_layer")
        else:
            _check(_lib.replay_stack_spec_layer_masked(self.h, int(layer), int(k), ctypes.byref(ri),
                                                       _mask_ptr(active, c.batch), _ptr(y, st.iot, "y"),
                                                       _stream()), "replay_stack_spec_layer_masked")
        return y

    def flush(self, params=None):
        """params[l]: layer l's parameter dict (Mamba-2 needs A) or None."""
        params = params or [None] * len(self.layers)
        ris = [make_inputs(st.cfg, {}, p) for st, p in zip(self.layers, params, strict=True)]
        arr = (_IP * len(ris))(*[ctypes.pointer(ri) for ri in ris])
        _check(_lib.replay_stack_flush(self.h, arr, _stream()), "replay_stack_flush")

    def commit(self, accepted):
        torch = _torch()
        _check(_lib.replay_stack_commit(self.h, _ptr(accepted, torch.int32, "accepted"), _stream()),
               "replay_stack_commit")

    def rollback(self):
        _check(_lib.replay_stack_rollback(self.h, _stream()), "replay_stack_rollback")

    def read_book(self):
        """(len, pend, fc, err) of the shared bookkeeping, as device tensors."""
        torch = _torch()
        B = self.layers[0].cfg.batch
        book = torch.empty((3, B), dtype=torch.int32, device=self.layers[0].device)
        err = torch.empty((1,), dtype=torch.int32, device=self.layers[0].device)
        _check(_lib.replay_stack_read_book(self.h, _ptr(book), _ptr(err), _stream()), "replay_stack_read_book")
        return book[0], book[1], book[2], err


# ---- conventional baselines -----------------------------------------------------
def conv_decode_step(cfg: ReplayConfig, S, tokens: dict, params: dict | None = None, y=None):
    torch = _torch()
    if y is None:
        y = torch.empty((1, cfg.batch, cfg.nheads, cfg.head_dim), dtype=_io_torch_dtype(cfg.io_dtype), device=S.device)
    ri = make_inputs(cfg, tokens, params)
    _check(_lib.replay_conv_decode_step(ctypes.byref(cfg), _ptr(S, ckpt_torch_dtype(cfg), "S"), ctypes.byref(ri),
                                        _ptr(y), _stream()), "replay_conv_decode_step")
    return y


def conv_spec_step(cfg: ReplayConfig, S, snaps, k: int, drafts: dict, params: dict | None = None, y=None):
    torch = _torch()
    if y is None:
        y = torch.empty((k, cfg.batch, cfg.nheads, cfg.head_dim), dtype=_io_torch_dtype(cfg.io_dtype), device=S.device)
    ri = make_inputs(cfg, drafts, params)
    ckt = ckpt_torch_dtype(cfg)
    _check(_lib.replay_conv_spec_step(ctypes.byref(cfg), _ptr(S, ckt, "S"), _ptr(snaps, ckt, "snaps"),
                                      int(k), ctypes.byref(ri), _ptr(y), _stream()), "replay_conv_spec_step")
    return y


def conv_spec_restore(cfg: ReplayConfig, S, snaps, k: int, accepted):
    torch = _torch()
    ckt = ckpt_torch_dtype(cfg)
    _check(_lib.replay_conv_spec_restore(ctypes.byref(cfg), _ptr(S, ckt, "S"),
                                         _ptr(snaps, ckt, "snaps"), int(k),
                                         _ptr(accepted, torch.int32, "accepted"), _stream()),
           "replay_conv_spec_restore")


# ---- stand-in non-SSM layers of a model step ---------------------------------------
def standin_linear(X, W, Y=None):
    """Y = X W^T in bf16 (X [M][K], W [N][K]) by replay_standin_linear."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N][K]")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    bf = torch.bfloat16
    _check(_lib.replay_standin_linear(_ptr(X, bf, "X"), _ptr(W, bf, "W"), _ptr(Y, bf, "Y"), M, K, N, _stream()),
           "replay_standin_linear")
    return Y


def standin_attention(q, K, V, scale, o=None):
    """Decode attention (replay_standin_attention): q [B][Hq*D] rows (any row stride), K and V
    [B][Hkv][L][D]; returns o [B][Hq][D]."""
    torch = _torch()
    B, Hkv, L, D = K.shape
    if q.dim() != 2 or q.stride(1) != 1:
        raise ValueError("q must be [B][row] with contiguous rows")
    Hq = q.shape[1] // D
    if o is None:
        o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=K.device)
    bf = torch.bfloat16
    if q.dtype != bf or not q.is_cuda:
        raise ValueError("q must be a bf16 device tensor")
    _check(_lib.replay_standin_attention(ctypes.c_void_p(q.data_ptr()), q.stride(0), _ptr(K, bf, "K"),
                                         _ptr(V, bf, "V"), _ptr(o, bf, "o"), B, Hq, Hkv, D, L, float(scale),
                                         _stream()), "replay_standin_attention")
    return o


def stream_copy(dst, src, nbytes: int):
    _check(_lib.replay_stream_copy(_ptr(dst), _ptr(src), int(nbytes), _stream()), "replay_stream_copy")


STREAM_TILE_BYTES = 32768


def stream_read_partials(nbytes: int) -> int:
    """Number of per-tile sums replay_stream_read writes for nbytes."""
    return max(1, -(-int(nbytes) // STREAM_TILE_BYTES))


def stream_read(src, nbytes: int, partials=None):
    """Read nbytes of src as fp32; returns the device tensor of per-32-KiB-tile sums."""
    import torch
    if partials is None:
        partials = torch.empty(stream_read_partials(nbytes), dtype=torch.float32, device=src.device)
    if partials.dtype != torch.float32 or partials.numel() < stream_read_partials(nbytes) or not partials.is_cuda:
        raise ValueError("partials: a device fp32 tensor of stream_read_partials(nbytes) entries")
    _check(_lib.replay_stream_read(_ptr(src), int(nbytes), _ptr(partials), _stream()), "replay_stream_read")
    return partials
