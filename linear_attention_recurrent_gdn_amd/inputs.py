"""Seeded synthetic inputs for the decode workloads (no method arithmetic here).

This module only draws random numbers and shapes them the way the workloads
are described: q and k are standard normal then L2-normalised per head, v is
standard normal (Student-t with 3 degrees of freedom for the KDA workload),
beta ~ U(0, 1) and the gate ~ U(lo, hi) per head (GDN) or per key channel
(KDA).  The recurrence that turns a prefill stream into a start state is *not*
here: the tests run the CPU oracle over ``prefill_tokens`` and the benchmark
runs the library's FP32-state kernel over them.

Seeding: every (workload seed, layer, phase, token, tensor) gets its own numpy
``Generator(PCG64(SeedSequence([...])))`` so any chunking of the token range
yields identical values.  Everything is fp32 in the library's layouts:

    q, k   [n_seq, n_k_heads, d]        v     [n_seq, n_v_heads, d]
    beta   [n_seq, n_v_heads]           gate  [n_seq, n_v_heads] (GDN)
                                              [n_seq, n_v_heads, d] (KDA)

The pages' own workloads are LLM evaluations on Qwen, Kimi and GLM models with
standard NLP benchmarks; neither the weights nor the benchmark data are used
here -- these inputs stand in for the decode shapes only.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

PHASE_PREFILL = 0
PHASE_DECODE = 1
_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "beta": 4, "gate": 5, "outlier": 6, "hidden": 7,
               "weights": 8}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    n_v_heads: int
    n_k_heads: int
    d: int
    gate: str  # "scalar" (GDN) or "channel" (KDA)
    window: int
    n_comp: int
    prefill: int
    decode: int
    gate_lo: float
    gate_hi: float
    seed: int
    v_dist: str = "normal"  # or "t3"
    outlier_rows: int = 0
    outlier_cols: int = 0
    outlier_factor: float = 1.0
    stagger: bool = False
    layers: int = 1
    projected: bool = False  # inputs come from random bf16 projections of a hidden state
    hidden: int = 0
    code_format: str = "int8"  # 8-bit code format of the stored state: "int8" or "e4m3"
    buffer_format: str = "fp32"  # window buffer: "fp32", "fp16" (k and v) or "nform" (chain-free, fp32)

    @property
    def n_units(self) -> int:
        return self.n_seq * self.n_v_heads

    @property
    def group(self) -> int:
        return self.n_v_heads // self.n_k_heads

    @property
    def gate_kind(self) -> int:
        return 0 if self.gate == "scalar" else 1

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five decode workloads (sizes, distributions, window, compensators).
WORKLOADS: Dict[str, Workload] = {
    "tiny_gdn": Workload("tiny_gdn", n_seq=1, n_v_heads=1, n_k_heads=1, d=64, gate="scalar",
                         window=64, n_comp=2, prefill=0, decode=256, gate_lo=0.90,
                         gate_hi=0.999, seed=0),
    "gdn_decode": Workload("gdn_decode", n_seq=64, n_v_heads=16, n_k_heads=16, d=128,
                           gate="scalar", window=64, n_comp=4, prefill=4096, decode=512,
                           gate_lo=0.9, gate_hi=1.0, seed=1, outlier_rows=4, outlier_cols=4,
                           outlier_factor=20.0),
    "kda_decode": Workload("kda_decode", n_seq=128, n_v_heads=32, n_k_heads=32, d=128,
                           gate="channel", window=128, n_comp=8, prefill=2048, decode=256,
                           gate_lo=0.85, gate_hi=1.0, seed=2, v_dist="t3"),
    "gdn_serving": Workload("gdn_serving", n_seq=512, n_v_heads=32, n_k_heads=32, d=128,
                            gate="scalar", window=64, n_comp=4, prefill=256, decode=128,
                            gate_lo=0.9, gate_hi=1.0, seed=3, stagger=True),
    "hybrid_stack": Workload("hybrid_stack", n_seq=256, n_v_heads=32, n_k_heads=16, d=128,
                             gate="scalar", window=64, n_comp=4, prefill=64, decode=64,
                             gate_lo=0.9, gate_hi=1.0, seed=4, layers=36, projected=True,
                             hidden=2048),
}


def _rng(wl: Workload, layer: int, phase: int, t: int, tensor: str,
         per_unit: bool = False) -> np.random.Generator:
    ss = np.random.SeedSequence([wl.seed, layer, phase, int(per_unit), t, _TENSOR_IDS[tensor]])
    return np.random.Generator(np.random.PCG64(ss))


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    n = np.sqrt((x64 * x64).sum(axis=-1, keepdims=True))
    return (x64 / n).astype(np.float32)


def token(wl: Workload, t: int, phase: int = PHASE_DECODE, layer: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of token ``t`` of ``phase`` for one layer (not for projected workloads)."""
    if wl.projected:
        raise ValueError("projected workloads draw inputs with projected_token()")
    S, H, KH, d = wl.n_seq, wl.n_v_heads, wl.n_k_heads, wl.d
    q = _l2_normalise(_rng(wl, layer, phase, t, "q").standard_normal((S, KH, d), np.float32))
    k = _l2_normalise(_rng(wl, layer, phase, t, "k").standard_normal((S, KH, d), np.float32))
    rv = _rng(wl, layer, phase, t, "v")
    if wl.v_dist == "t3":
        v = rv.standard_t(3, size=(S, H, d)).astype(np.float32)
    else:
        v = rv.standard_normal((S, H, d), np.float32)
    beta = _rng(wl, layer, phase, t, "beta").uniform(0.0, 1.0, (S, H)).astype(np.float32)
    gshape = (S, H) if wl.gate == "scalar" else (S, H, d)
    gate = _rng(wl, layer, phase, t, "gate").uniform(wl.gate_lo, wl.gate_hi, gshape).astype(
        np.float32)
    return {"q": q, "k": k, "v": v, "beta": beta, "gate": gate}


def tokens(wl: Workload, t0: int, n: int, phase: int = PHASE_DECODE, layer: int = 0):
    """Stack ``n`` tokens starting at ``t0``: each array gets a leading token axis."""
    toks = [token(wl, t, phase, layer) for t in range(t0, t0 + n)]
    return {key: np.stack([tk[key] for tk in toks]) for key in toks[0]} if toks else None


def unit_stream(wl: Workload, unit: int, n: int, phase: int = PHASE_PREFILL, layer: int = 0,
                with_queries: bool = False) -> Dict[str, np.ndarray]:
    """``n`` tokens of one unit: k [n, d], v [n, d], beta [n], gate [n] or [n, d]
    (and q [n, d] with ``with_queries``).

    Keyed per unit (q and k per (sequence, key head), so the value heads of
    one key head share them), so any subset of units can be generated on its
    own.  Prefill needs no queries (no outputs are read).
    """
    if wl.projected:
        raise ValueError("projected workloads draw inputs through projected_token()")
    d = wl.d
    s, h = divmod(unit, wl.n_v_heads)
    key_id = s * wl.n_k_heads + h // wl.group
    k = _l2_normalise(_rng(wl, layer, phase, key_id, "k", True).standard_normal((n, d), np.float32))
    rv = _rng(wl, layer, phase, unit, "v", True)
    v = (rv.standard_t(3, size=(n, d)).astype(np.float32) if wl.v_dist == "t3"
         else rv.standard_normal((n, d), np.float32))
    beta = _rng(wl, layer, phase, unit, "beta", True).uniform(0.0, 1.0, n).astype(np.float32)
    gshape = (n,) if wl.gate == "scalar" else (n, d)
    gate = _rng(wl, layer, phase, unit, "gate", True).uniform(wl.gate_lo, wl.gate_hi, gshape).astype(
        np.float32)
    out = {"k": k, "v": v, "beta": beta, "gate": gate}
    if with_queries:
        out["q"] = _l2_normalise(_rng(wl, layer, phase, key_id, "q", True).standard_normal((n, d), np.float32))
    return out


def prefill_stream(wl: Workload, unit: int, layer: int = 0) -> Dict[str, np.ndarray]:
    """The prefill tokens of one unit (see ``unit_stream``)."""
    return unit_stream(wl, unit, wl.prefill, PHASE_PREFILL, layer)


def prefill_streams(wl: Workload, units, layer: int = 0, n: Optional[int] = None,
                    phase: int = PHASE_PREFILL, with_queries: bool = False) -> Dict[str, np.ndarray]:
    """Token-major per-unit streams of several units: k [n, U', d], v [n, U', d], ..."""
    n = wl.prefill if n is None else n
    per = [unit_stream(wl, int(u), n, phase, layer, with_queries) for u in units]
    return {key: np.ascontiguousarray(np.stack([p[key] for p in per], axis=1)) for key in per[0]}


def surrogate_state(wl: Workload, units, layer: int = 0, scale: float = 0.5) -> np.ndarray:
    """Gaussian stand-in start states [n, d, d] for units whose outputs are not checked."""
    out = np.empty((len(units), wl.d, wl.d), np.float32)
    for i, u in enumerate(units):
        out[i] = _rng(wl, layer, PHASE_PREFILL, int(u), "hidden", True).standard_normal(
            (wl.d, wl.d), np.float32) * np.float32(scale)
    return out


def torch_token(wl: Workload, gen, device, phase_scale: float = 1.0):
    """One token of inputs drawn on the device with a torch Generator (same
    distributions as ``token``; used where numpy generation would dominate)."""
    import torch

    S, H, KH, d = wl.n_seq, wl.n_v_heads, wl.n_k_heads, wl.d
    f = torch.float32

    def nrm(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=f)
        return x / x.norm(dim=-1, keepdim=True)

    q, k = nrm((S, KH, d)), nrm((S, KH, d))
    if wl.v_dist == "t3":
        # Student-t(3) = N / sqrt(chi2_3 / 3)
        z = torch.randn((S, H, d), generator=gen, device=device, dtype=f)
        c = torch.randn((S, H, d, 3), generator=gen, device=device, dtype=f).pow(2).sum(-1)
        v = z / torch.sqrt(c / 3.0)
    else:
        v = torch.randn((S, H, d), generator=gen, device=device, dtype=f)
    beta = torch.rand((S, H), generator=gen, device=device, dtype=f)
    gshape = (S, H) if wl.gate == "scalar" else (S, H, d)
    gate = wl.gate_lo + (wl.gate_hi - wl.gate_lo) * torch.rand(gshape, generator=gen, device=device, dtype=f)
    return {"q": q, "k": k, "v": v, "beta": beta, "gate": gate}


def outlier_scale(wl: Workload, layer: int = 0):
    """Per-unit row and column multipliers for planting outlier lines.

    For each unit, ``outlier_rows`` random rows and ``outlier_cols`` random
    columns get the factor (entries on both get its square); the caller applies
    S <- Diag(r) S Diag(c).  Returns (r [U, d], c [U, d]) fp32 or None.
    """
    if wl.outlier_rows == 0 and wl.outlier_cols == 0:
        return None
    rng = _rng(wl, layer, PHASE_PREFILL, 0, "outlier")
    U, d = wl.n_units, wl.d
    r = np.ones((U, d), np.float32)
    c = np.ones((U, d), np.float32)
    for u in range(U):
        r[u, rng.choice(d, wl.outlier_rows, replace=False)] = wl.outlier_factor
        c[u, rng.choice(d, wl.outlier_cols, replace=False)] = wl.outlier_factor
    return r, c


def stagger_schedule(wl: Workload) -> Optional[np.ndarray]:
    """Warm-up step (0-based) after which each sequence takes a forced flush.

    Sequence s gets offset o_s = s mod W: a forced flush after warm-up token
    W - o_s - 1 leaves it o_s tokens into a window when the timed tokens start,
    so about 1/W of the sequences reach a window boundary at every step.
    Offset 0 is the natural boundary, so its entry is -1 (no forced flush).
    """
    if not wl.stagger:
        return None
    W = wl.window
    off = np.arange(wl.n_seq) % W
    return np.where(off == 0, -1, W - off - 1).astype(np.int32)


# ---------------------------------------------------------------------------
# Projected workload (hybrid stack): inputs from random bf16 projections
# ---------------------------------------------------------------------------

def projection_weights(wl: Workload, layer: int):
    """bf16 weights ~ N(0, 1/hidden) of one layer, as numpy float32 arrays.

    W_q, W_k: hidden -> n_k_heads*d;  W_v: hidden -> n_v_heads*d;
    w_alpha, w_beta: hidden -> n_v_heads.
    """
    rng = _rng(wl, layer, PHASE_PREFILL, 0, "weights")
    h, KH, H, d = wl.hidden, wl.n_k_heads, wl.n_v_heads, wl.d
    std = 1.0 / np.sqrt(h)
    mats = {}
    for name, n_out in (("wq", KH * d), ("wk", KH * d), ("wv", H * d), ("wa", H), ("wb", H)):
        mats[name] = (rng.standard_normal((n_out, h), np.float32) * np.float32(std))
    return mats


def hidden_state(wl: Workload, layer: int, t: int, phase: int = PHASE_DECODE) -> np.ndarray:
    """Hidden state ~ N(0, 1) [n_seq, hidden], fresh per token and per layer."""
    return _rng(wl, layer, phase, t, "hidden").standard_normal((wl.n_seq, wl.hidden), np.float32)


def projected_token(wl: Workload, weights, hidden, device=None) -> Dict[str, np.ndarray]:
    """q, k, v, beta, alpha of one token from a hidden state (bf16 matmuls in torch).

    q, k = L2-normalised per key head; v = W_v h; beta = sigmoid(w_beta . h);
    alpha = 0.9 + 0.1 sigmoid(w_alpha . h).  This is model-side input synthesis
    for the decode step, not part of the recurrent-state path.
    """
    import torch

    dev = torch.device(device) if device is not None else torch.device("cpu")
    hb = torch.as_tensor(hidden, device=dev).to(torch.bfloat16)

    def proj(name):
        w = weights[name]
        if not isinstance(w, torch.Tensor):
            w = torch.as_tensor(w, device=dev).to(torch.bfloat16)
        return (hb @ w.t().contiguous()).float()

    S, KH, H, d = wl.n_seq, wl.n_k_heads, wl.n_v_heads, wl.d
    q = proj("wq").view(S, KH, d)
    k = proj("wk").view(S, KH, d)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = proj("wv").view(S, H, d)
    beta = torch.sigmoid(proj("wb"))
    alpha = 0.9 + 0.1 * torch.sigmoid(proj("wa"))
    out = {"q": q, "k": k, "v": v, "beta": beta, "gate": alpha}
    return {key: val.contiguous().cpu().numpy().astype(np.float32) for key, val in out.items()}


def expand_keys(x: np.ndarray, group: int) -> np.ndarray:
    """[..., n_seq, n_k_heads, d] -> [..., n_seq, n_k_heads*group, d] (value head h uses key head h // group)."""
    return np.repeat(x, group, axis=-2)


def per_unit(x: np.ndarray, wl: Workload, kind: str) -> np.ndarray:
    """Flatten (n_seq, heads) into the unit axis u = s * n_v_heads + h.

    kind: "key" for q, k [..., n_seq, n_k_heads, d] (expanded so value head h
    sees key head h // group); "value" for v or a channel gate
    [..., n_seq, n_v_heads, d]; "head" for beta or a scalar gate
    [..., n_seq, n_v_heads].
    """
    if kind == "key":
        x = expand_keys(x, wl.group)
        kind = "value"
    if kind == "value":
        return x.reshape(*x.shape[:-3], wl.n_units, x.shape[-1])
    if kind == "head":
        return x.reshape(*x.shape[:-2], wl.n_units)
    raise ValueError(kind)


def tokens_per_unit(wl: Workload, toks: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Token-major inputs in the oracle's per-unit layout."""
    return {
        "q": per_unit(toks["q"], wl, "key"),
        "k": per_unit(toks["k"], wl, "key"),
        "v": per_unit(toks["v"], wl, "value"),
        "beta": per_unit(toks["beta"], wl, "head"),
        "gate": per_unit(toks["gate"], wl, "head" if wl.gate == "scalar" else "value"),
    }
