"""Plain FP64 CPU oracle for windowed INT8 recurrent-state decode (GDN / KDA).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; the GPU library and its Python
binding never import it, and it shares no source with them.

The arithmetic lives in ``lq_oracle.c`` (plain C, FP64, OpenMP over independent
units); this module only compiles it, loads it and marshals numpy arrays.  The
exact rational checks in ``exact.py`` pin it.

Every function follows the pages about arXiv 2609.38166 ("LeapQuant: Efficient
Linear Attention with Accurate Recurrent State Quantization"); the citations sit
next to each C function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GATE_SCALAR = 0  # GDN
GATE_CHANNEL = 1  # KDA

CC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
            "-ffp-contract=off"]


def build(force: bool = False) -> str:
    """Compile lq_oracle.c into liboracle.so (gcc, baseline x86-64, FP64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = os.environ.get("LQ_ORACLE_LIB")  # a deliberately broken copy, for mutation tests
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.orc_num_threads.restype = I
        lib.orc_set_num_threads.argtypes = [I]
        lib.orc_recurrence.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        lib.orc_qz.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        lib.orc_dequant.argtypes = [I, I, I, I, I, P, P, P, P, P, P]
        lib.orc_replay_output.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
        lib.orc_windowed_run.argtypes = [I, I, I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        lib.orc_fp16_round.argtypes = [ctypes.c_float]
        lib.orc_fp16_round.restype = ctypes.c_float
        lib.orc_fp16_round_array.argtypes = [ctypes.c_long, P, P]
        lib.orc_e4m3_value.argtypes = [I]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
        for f in ("orc_recurrence", "orc_qz", "orc_dequant", "orc_replay_output",
                  "orc_windowed_run", "orc_e4m3_encode"):
            getattr(lib, f).restype = I
        _lib = lib
        return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


def _gate_kind(gate, n_tok_units_shape, dk):
    return GATE_SCALAR if gate.shape == n_tok_units_shape else GATE_CHANNEL


def recurrence(S, q, k, v, beta, gate, want_outputs=True):
    """O1, the plain recurrence, on ``n_units`` independent units.

    S: [U, dv, dk] (copied; returned updated, fp64).  Token-major inputs:
    q, k [T, U, dk]; v [T, U, dv]; beta [T, U]; gate [T, U] (GDN) or [T, U, dk]
    (KDA).  Returns (S_T, o [T, U, dv] or None).
    """
    lib = _load()
    S = _f64(S).copy()
    U, dv, dk = S.shape
    k = _f32(k)
    T = k.shape[0]
    v, beta, gate = _f32(v), _f32(beta), _f32(gate)
    gk = _gate_kind(gate, (T, U), dk)
    qq = _f32(q) if (want_outputs and q is not None) else None
    o = np.zeros((T, U, dv), np.float64) if qq is not None else None
    rc = lib.orc_recurrence(U, dk, dv, T, gk, _p(S), _p(qq), _p(k), _p(v), _p(beta), _p(gate),
                            _p(o))
    assert rc == 0
    return S, o


FORMATS = {"int8": 0, "e4m3": 1}


def _fmt(fmt: str) -> int:
    if fmt not in FORMATS:
        raise ValueError(f"unknown code format {fmt!r}")
    return FORMATS[fmt]


def e4m3_value(code: int) -> float:
    """Value of one E4M3 byte (NaN for the two NaN codes)."""
    return _load().orc_e4m3_value(int(code) & 0xFF)


def e4m3_encode(x: float) -> int:
    """E4M3 byte of the nearest value to x (ties to the even mantissa, saturating at 448)."""
    return _load().orc_e4m3_encode(float(x))


def fp16_round(x) -> np.ndarray:
    """Each fp32 value as stored in a binary16 buffer (nearest, ties to even,
    saturating at 65504), returned as fp32."""
    x = _f32(x)
    out = np.empty_like(x)
    _load().orc_fp16_round_array(x.size, _p(x), _p(out))
    return out


def code_values(codes, fmt: str = "int8") -> np.ndarray:
    """fp64 values of an array of stored codes."""
    codes = np.asarray(codes, np.int8)
    if _fmt(fmt) == 0:
        return codes.astype(np.float64)
    table = np.array([e4m3_value(c) for c in range(256)])
    return table[codes.view(np.uint8)]


class Blob:
    """The stored low-bit state of ``U`` units, as the oracle holds it."""

    __slots__ = ("codes", "sigma", "smooth", "comp_idx", "comp_vec", "fmt")

    def __init__(self, codes, sigma, smooth, comp_idx, comp_vec, fmt="int8"):
        self.codes = np.ascontiguousarray(codes).view(np.int8)
        self.sigma = _f32(sigma)
        self.smooth = _f32(smooth)
        self.comp_idx = np.ascontiguousarray(comp_idx, np.int32)
        self.comp_vec = _f32(comp_vec)
        _fmt(fmt)
        self.fmt = fmt

    @property
    def n_comp(self):
        return self.comp_idx.shape[1]

    def take(self, units):
        return Blob(self.codes[units], self.sigma[units], self.smooth[units],
                    self.comp_idx[units], self.comp_vec[units], self.fmt)


def qz(S, n_c, smooth=True, force_sel=None, fmt="int8"):
    """Qz: compensators, smoothing and 8-bit codes (``fmt`` "int8" or "e4m3")
    of each unit's state.

    Returns (Blob, x_unrounded [U, dv, dk], scores [U, dv + dk]).
    """
    lib = _load()
    S = _f64(S)
    U, dv, dk = S.shape
    D = max(dk, dv)
    codes = np.zeros((U, dv, dk), np.int8)
    sigma = np.zeros((U, dv), np.float32)
    sm = np.zeros((U, dk), np.float32)
    ci = np.zeros((U, max(n_c, 0)), np.int32)
    cv = np.zeros((U, max(n_c, 0), D), np.float32)
    x = np.zeros((U, dv, dk), np.float64)
    sc = np.zeros((U, dv + dk), np.float64)
    fs = None if force_sel is None else np.ascontiguousarray(force_sel, np.int32)
    rc = lib.orc_qz(_fmt(fmt), U, dk, dv, n_c, 1 if smooth else 0, _p(S), _p(fs), _p(codes),
                    _p(sigma), _p(sm), _p(ci), _p(cv), _p(x), _p(sc))
    assert rc == 0
    return Blob(codes, sigma, sm, ci, cv, fmt), x, sc


def dequant(blob: Blob):
    """Window-start state Diag(sigma) Q Diag(s) + sum_c v_c k_c^T, fp64 [U, dv, dk]."""
    lib = _load()
    U, dv, dk = blob.codes.shape
    S = np.zeros((U, dv, dk), np.float64)
    rc = lib.orc_dequant(_fmt(blob.fmt), U, dk, dv, blob.n_comp, _p(blob.codes), _p(blob.sigma),
                         _p(blob.smooth), _p(blob.comp_idx), _p(blob.comp_vec), _p(S))
    assert rc == 0
    return S


def replay_output(blob: Blob, bk, bv, bb, bg, q):
    """O3: output from the stored state plus the buffered window (reverse replay).

    bk [U, n, dk], bv [U, n, dv], bb [U, n], bg [U, n] or [U, n, dk] hold the
    window's tokens 1..n in order, the current token last; q [U, dk].
    """
    lib = _load()
    U, dv, dk = blob.codes.shape
    bk, bv, bb, bg, q = _f32(bk), _f32(bv), _f32(bb), _f32(bg), _f32(q)
    n = bk.shape[1]
    gk = GATE_SCALAR if bg.shape == (U, n) else GATE_CHANNEL
    o = np.zeros((U, dv), np.float64)
    rc = lib.orc_replay_output(_fmt(blob.fmt), U, dk, dv, blob.n_comp, gk, n, _p(blob.codes), _p(blob.sigma),
                               _p(blob.smooth), _p(blob.comp_idx), _p(blob.comp_vec), _p(bk),
                               _p(bv), _p(bb), _p(bg), _p(q), _p(o))
    assert rc == 0
    return o


def windowed_run(S0, q, k, v, beta, gate, W, n_c, smooth=True, force_at=None, want_state=False,
                 fmt="int8", buffer="fp32"):
    """O2: the windowed scheme in its definitional form over T tokens.

    S0 [U, dv, dk] unquantized start state; token-major inputs as in
    ``recurrence``.  ``force_at[u]`` = token index after which unit u takes a
    forced partial flush (-1: none).  W=1, n_c=0, smooth=False gives the naive
    per-token quantization; ``fmt`` selects the code format ("int8" or "e4m3");
    ``buffer="fp16"`` rounds every token's k and v to binary16 as the window
    buffer stores them.
    Returns o [T, U, dv] (and the final state).
    """
    lib = _load()
    S0 = _f64(S0)
    U, dv, dk = S0.shape
    q, k, v, beta, gate = _f32(q), _f32(k), _f32(v), _f32(beta), _f32(gate)
    T = k.shape[0]
    gk = _gate_kind(gate, (T, U), dk)
    fa = None if force_at is None else np.ascontiguousarray(force_at, np.int32)
    o = np.zeros((T, U, dv), np.float64)
    Sout = np.zeros((U, dv, dk), np.float64) if want_state else None
    if buffer not in ("fp32", "fp16"):
        raise ValueError(f"unknown buffer format {buffer!r}")
    rc = lib.orc_windowed_run(_fmt(fmt), 1 if buffer == "fp16" else 0, U, dk, dv, T, gk, W, n_c, 1 if smooth else 0, _p(S0), _p(q),
                              _p(k), _p(v), _p(beta), _p(gate), _p(fa), _p(o), _p(Sout))
    assert rc == 0
    return (o, Sout) if want_state else o
