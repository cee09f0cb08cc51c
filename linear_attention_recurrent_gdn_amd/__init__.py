"""Python binding of liblq.so: windowed INT8 recurrent-state decode for Gated
DeltaNet and Kimi Delta Attention on MI355X (gfx950).

The functions carry the C ABI's names (``include/lq.h``) and only marshal
arguments: they check dtypes, devices, contiguity and sizes of torch tensors
(the kernels trust the sizes), turn them into device pointers, take the
current HIP stream, and raise ``LQError`` on a non-zero return code.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  PyTorch supplies device memory and streams only.
"""
from __future__ import annotations

import ctypes
import dataclasses
import functools
import os
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblq.so")

LQ_OK = 0
LQ_EINVAL = -1
LQ_EUNSUPPORTED = -2
LQ_EHIP = -3
LQ_ESCRATCH = -4
LQ_NOALLOC_MAX_UNITS = 262144
LQ_GATE_SCALAR = 0
LQ_GATE_CHANNEL = 1
LQ_CODE_INT8 = 0
LQ_CODE_E4M3 = 1
LQ_BUFFER_FP32 = 0
LQ_BUFFER_FP16 = 1
LQ_BUFFER_NFORM = 2
LQ_LOADS_AUTO = 0
LQ_LOADS_STREAM = 1
LQ_LOADS_CACHED = 2
LQ_DEV_WINDOW_OVERFLOW = 0x1
LQ_DEV_NONFINITE_INPUT = 0x2
LQ_DEV_BUFFER_SATURATED = 0x4

EXPORTS = ("lq_state_bytes", "lq_state_layout", "lq_state_init", "lq_prefill", "lq_decode_step",
           "lq_window_flush", "lq_dequant_state", "lq_fp32_decode_step", "lq_read_status",
           "lq_clear_status", "lq_window_flush_noalloc", "lq_strerror")


class LQError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {strerror(code)} (code {code})")


class _CConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_seq", "n_v_heads", "n_k_heads", "d_k", "d_v", "window", "n_comp", "gate_kind",
                 "code_format", "buffer_format", "flush_cus", "load_policy")]


_LAYOUT_FIELDS = ("total_bytes", "status", "fill", "codes", "sigma", "smooth", "comp_idx",
                  "comp_vec", "buf_k", "buf_v", "buf_beta", "buf_gate", "work")


class _CLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _LAYOUT_FIELDS]


@dataclasses.dataclass(frozen=True)
class Config:
    """Mirror of ``lq_config``."""
    n_seq: int
    n_v_heads: int
    n_k_heads: int
    d_k: int
    d_v: int
    window: int
    n_comp: int
    gate_kind: int = LQ_GATE_SCALAR
    code_format: int = LQ_CODE_INT8
    buffer_format: int = LQ_BUFFER_FP32
    flush_cus: int = 0
    load_policy: int = LQ_LOADS_AUTO

    @property
    def n_units(self) -> int:
        return self.n_seq * self.n_v_heads

    def c(self) -> _CConfig:
        return _CConfig(*(int(getattr(self, f)) for f, _ in _CConfig._fields_))


_lib = None


def load_library(path: Optional[str] = None):
    """Load liblq.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("LQ_LIB_PATH") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build it first (python -m linear_attention_recurrent_gdn_amd._build)")
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    CP = ctypes.POINTER(_CConfig)
    lib.lq_state_bytes.argtypes = [CP, ctypes.POINTER(ctypes.c_size_t)]
    lib.lq_state_layout.argtypes = [CP, ctypes.POINTER(_CLayout)]
    lib.lq_state_init.argtypes = [CP, P, P, P]
    lib.lq_decode_step.argtypes = [CP, P, P, P, P, P, P, P, P]
    lib.lq_prefill.argtypes = [CP, P, P, ctypes.c_int32, P, P, P, P, P, P, P]
    lib.lq_window_flush.argtypes = [CP, P, P, P]
    lib.lq_window_flush_noalloc.argtypes = [CP, P, P, P]
    lib.lq_dequant_state.argtypes = [CP, P, P, ctypes.c_int32, P]
    lib.lq_fp32_decode_step.argtypes = [CP, P, P, P, P, P, P, P, P]
    lib.lq_read_status.argtypes = [CP, P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.lq_clear_status.argtypes = [CP, P, P]
    for f in EXPORTS[:-1]:
        getattr(lib, f).restype = ctypes.c_int32
    lib.lq_strerror.argtypes = [ctypes.c_int32]
    lib.lq_strerror.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().lq_strerror(int(code)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != LQ_OK:
        raise LQError(fn, rc)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, name: str, dtype=None, numel: Optional[int] = None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):  # a raw device pointer: the caller vouches for it
        return ctypes.c_void_p(t)
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or a device pointer")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _sizes(cfg: Config) -> Dict[str, int]:
    g = cfg.d_k if cfg.gate_kind == LQ_GATE_CHANNEL else 1
    return {
        "qk": cfg.n_seq * cfg.n_k_heads * cfg.d_k,
        "v": cfg.n_units * cfg.d_v,
        "beta": cfg.n_units,
        "gate": cfg.n_units * g,
        "state": cfg.n_units * cfg.d_v * cfg.d_k,
    }


# ---------------------------------------------------------------------------
# entry points (names as in lq.h)
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=256)
def lq_state_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check("lq_state_bytes", load_library().lq_state_bytes(ctypes.byref(cfg.c()), ctypes.byref(n)))
    return n.value


def lq_state_layout(cfg: Config) -> Dict[str, int]:
    L = _CLayout()
    _check("lq_state_layout", load_library().lq_state_layout(ctypes.byref(cfg.c()), ctypes.byref(L)))
    return {f: getattr(L, f) for f in _LAYOUT_FIELDS}


def _state_ptr(cfg: Config, state):
    import torch

    if isinstance(state, torch.Tensor):
        if state.dtype != torch.uint8:
            raise ValueError("state: expected a uint8 tensor")
        if state.numel() < lq_state_bytes(cfg):
            raise ValueError(f"state: {state.numel()} bytes, need {lq_state_bytes(cfg)}")
    return _ptr(state, "state")


def lq_state_init(cfg: Config, state, S0=None, stream=None) -> None:
    import torch

    sz = _sizes(cfg)
    rc = load_library().lq_state_init(ctypes.byref(cfg.c()), _state_ptr(cfg, state),
                                      _ptr(S0, "S0", torch.float32, sz["state"], allow_none=True),
                                      _stream(stream))
    _check("lq_state_init", rc)


def lq_prefill(cfg: Config, state, S0, q, k, v, beta, gate, o=None, stream=None) -> None:
    """Prompt of T tokens (token-major tensors, leading dimension T) through the
    recurrence from S0 (or zero), outputs into o (or none), final state quantized."""
    import torch

    sz = _sizes(cfg)
    T = int(k.shape[0]) if k is not None else 0
    rc = load_library().lq_prefill(
        ctypes.byref(cfg.c()), _state_ptr(cfg, state),
        _ptr(S0, "S0", torch.float32, sz["state"], allow_none=True), T,
        _ptr(q, "q", torch.float32, T * sz["qk"], allow_none=T == 0),
        _ptr(k, "k", torch.float32, T * sz["qk"], allow_none=T == 0),
        _ptr(v, "v", torch.float32, T * sz["v"], allow_none=T == 0),
        _ptr(beta, "beta", torch.float32, T * sz["beta"], allow_none=T == 0),
        _ptr(gate, "gate", torch.float32, T * sz["gate"], allow_none=T == 0),
        _ptr(o, "o", torch.float32, T * sz["v"], allow_none=True), _stream(stream))
    _check("lq_prefill", rc)


def lq_decode_step(cfg: Config, state, q, k, v, beta, gate, o, stream=None) -> None:
    import torch

    sz, f = _sizes(cfg), torch.float32
    rc = load_library().lq_decode_step(
        ctypes.byref(cfg.c()), _state_ptr(cfg, state), _ptr(q, "q", f, sz["qk"]),
        _ptr(k, "k", f, sz["qk"]), _ptr(v, "v", f, sz["v"]), _ptr(beta, "beta", f, sz["beta"]),
        _ptr(gate, "gate", f, sz["gate"]), _ptr(o, "o", f, sz["v"]), _stream(stream))
    _check("lq_decode_step", rc)


def lq_window_flush(cfg: Config, state, force_mask=None, stream=None) -> None:
    import torch

    rc = load_library().lq_window_flush(
        ctypes.byref(cfg.c()), _state_ptr(cfg, state),
        _ptr(force_mask, "force_mask", torch.uint8, cfg.n_seq, allow_none=True), _stream(stream))
    _check("lq_window_flush", rc)


def lq_window_flush_noalloc(cfg: Config, state, force_mask=None, stream=None) -> None:
    import torch

    rc = load_library().lq_window_flush_noalloc(
        ctypes.byref(cfg.c()), _state_ptr(cfg, state),
        _ptr(force_mask, "force_mask", torch.uint8, cfg.n_seq, allow_none=True), _stream(stream))
    _check("lq_window_flush_noalloc", rc)


def lq_dequant_state(cfg: Config, state, S_out, include_buffer: bool = False, stream=None) -> None:
    import torch

    rc = load_library().lq_dequant_state(
        ctypes.byref(cfg.c()), _state_ptr(cfg, state),
        _ptr(S_out, "S_out", torch.float32, _sizes(cfg)["state"]), int(bool(include_buffer)),
        _stream(stream))
    _check("lq_dequant_state", rc)


def lq_fp32_decode_step(cfg: Config, S, q, k, v, beta, gate, o, stream=None) -> None:
    import torch

    sz, f = _sizes(cfg), torch.float32
    rc = load_library().lq_fp32_decode_step(
        ctypes.byref(cfg.c()), _ptr(S, "S", f, sz["state"]), _ptr(q, "q", f, sz["qk"]),
        _ptr(k, "k", f, sz["qk"]), _ptr(v, "v", f, sz["v"]), _ptr(beta, "beta", f, sz["beta"]),
        _ptr(gate, "gate", f, sz["gate"]), _ptr(o, "o", f, sz["v"]), _stream(stream))
    _check("lq_fp32_decode_step", rc)


def lq_read_status(cfg: Config, state, clear: bool = False, stream=None) -> int:
    """The blob's sticky device flags (synchronizes the stream); with
    ``clear`` they are then reset through lq_clear_status."""
    flags = ctypes.c_uint32(0)
    rc = load_library().lq_read_status(ctypes.byref(cfg.c()), _state_ptr(cfg, state),
                                       ctypes.byref(flags), _stream(stream))
    _check("lq_read_status", rc)
    if clear:
        lq_clear_status(cfg, state, stream)
    return flags.value


def lq_clear_status(cfg: Config, state, stream=None) -> None:
    rc = load_library().lq_clear_status(ctypes.byref(cfg.c()), _state_ptr(cfg, state), _stream(stream))
    _check("lq_clear_status", rc)


def lq_strerror(code: int) -> str:
    return strerror(code)


# ---------------------------------------------------------------------------
# conveniences for callers holding the blob in a torch tensor
# ---------------------------------------------------------------------------

def new_state(cfg: Config, device="cuda"):
    """A uint8 tensor of lq_state_bytes(cfg) bytes (torch allocations are 256-byte aligned)."""
    import torch

    t = torch.empty(lq_state_bytes(cfg), dtype=torch.uint8, device=device)
    if t.data_ptr() % 256:
        raise RuntimeError("state allocation is not 256-byte aligned")
    return t


def state_views(cfg: Config, state) -> Dict[str, "object"]:
    """Typed torch views of the blob's sections (for inspection and checkpoints)."""
    import torch

    L = lq_state_layout(cfg)
    U, D = cfg.n_units, max(cfg.d_k, cfg.d_v)
    W, nc = cfg.window, cfg.n_comp
    g = cfg.d_k if cfg.gate_kind == LQ_GATE_CHANNEL else 1
    bt = torch.float16 if cfg.buffer_format == LQ_BUFFER_FP16 else torch.float32

    def view(off, n, dtype, shape):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return state[off:off + nbytes].view(dtype).view(*shape)

    return {
        "status": view(L["status"], 1, torch.int32, (1,)),
        "fill": view(L["fill"], U, torch.int32, (U,)),
        "codes": view(L["codes"], U * cfg.d_v * cfg.d_k, torch.int8, (U, cfg.d_v, cfg.d_k)),
        "sigma": view(L["sigma"], U * cfg.d_v, torch.float32, (U, cfg.d_v)),
        "smooth": view(L["smooth"], U * cfg.d_k, torch.float32, (U, cfg.d_k)),
        "comp_idx": view(L["comp_idx"], U * nc, torch.int32, (U, nc)),
        "comp_vec": view(L["comp_vec"], U * nc * D, torch.float32, (U, nc, D)),
        "buf_k": view(L["buf_k"], cfg.n_seq * cfg.n_k_heads * W * cfg.d_k, bt,
                      (cfg.n_seq, cfg.n_k_heads, W, cfg.d_k)),
        "buf_v": view(L["buf_v"], U * W * cfg.d_v, bt, (U, W, cfg.d_v)),
        "buf_beta": view(L["buf_beta"], U * W, torch.float32, (U, W)),
        "buf_gate": view(L["buf_gate"], U * W * g, torch.float32, (U, W) if g == 1 else (U, W, g)),
        "work": view(L["work"], U + 1, torch.int32, (U + 1,)),
    }
