"""Teacher-forced comparison of the HIP path (through the C ABI) with the CPU
oracle on one workload.

Tolerances (the decode step's outputs are fp32; the oracle is fp64):
  * outputs: relative L2 error of each decode call's outputs <= 1e-4, both
    over all checked units together and for every checked unit on its own
    (the per-unit maximum is reported);
  * codes after each init / flush: identical, except neighbouring codes (1 LSB
    for INT8, one grid spacing for E4M3) where the oracle's unrounded value
    lies within 2^-10 of a spacing of their midpoint, in at most 0.01% of that
    call's codes;
  * compensator selection identical, unless the oracle's n_c-th and
    (n_c+1)-th line scores are within 1e-6 relative (then the GPU's choice is
    adopted and the oracle's quantizer re-run with it forced);
  * compensator vectors <= 1e-4 relative L2; scales and smoothing <= 1e-6 relative;
  * dequantized state (with and without the buffer) <= 1e-4 relative L2,
    over all checked units and per unit, against the oracle's dequantization
    of the GPU's own stored state.
After each init and flush the oracle adopts the GPU's stored state, so a
permitted code difference never compounds.

Start states: the oracle runs the workload's prefill for every checked unit
(fp64, rounded to fp32); units whose outputs are not checked (sampled runs at
full size) get a seeded Gaussian stand-in so every launch still has the full
shape.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

import linear_attention_recurrent_gdn_amd as lq
import oracle as orc
from linear_attention_recurrent_gdn_amd import inputs as I

TOL_OUT = 1e-4
TOL_STATE = 1e-4
TOL_COMP = 1e-4
TOL_SCALE = 1e-6
TIE_TAU = 2.0 ** -10
FLIP_BUDGET = 1e-4  # fraction of a call's codes
AMBIG = 1e-6


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a - b))


def unit_rel_l2(a, b) -> np.ndarray:
    """Relative L2 error of each unit (leading axis) on its own."""
    a = np.asarray(a, np.float64).reshape(len(a), -1)
    b = np.asarray(b, np.float64).reshape(len(b), -1)
    d = np.linalg.norm(a - b, axis=1)
    n = np.linalg.norm(b, axis=1)
    return np.where(n > 0, d / np.where(n > 0, n, 1.0), d)


def config_of(wl: I.Workload) -> lq.Config:
    fmt = {"int8": lq.LQ_CODE_INT8, "e4m3": lq.LQ_CODE_E4M3}[wl.code_format]
    buf = {"fp32": lq.LQ_BUFFER_FP32, "fp16": lq.LQ_BUFFER_FP16, "nform": lq.LQ_BUFFER_NFORM}[wl.buffer_format]
    return lq.Config(wl.n_seq, wl.n_v_heads, wl.n_k_heads, wl.d, wl.d, wl.window, wl.n_comp,
                     wl.gate_kind, fmt, buf)


@dataclasses.dataclass
class Report:
    name: str
    max_out_err: float = 0.0         # worst decode call, all checked units together
    max_unit_out_err: float = 0.0    # worst single unit in any decode call
    max_state_err: float = 0.0
    max_unit_state_err: float = 0.0
    flushes: int = 0
    codes_checked: int = 0
    code_flips: int = 0
    ambiguous_selections: int = 0
    decode_calls: int = 0


class TokenSource:
    """Decode and prefill inputs of one layer of a workload (numpy, library layouts)."""

    def __init__(self, wl: I.Workload, layer: int = 0, device="cuda"):
        self.wl, self.layer, self.device = wl, layer, device
        self.weights = I.projection_weights(wl, layer) if wl.projected else None
        if self.weights is not None:
            self.weights = {k: torch.as_tensor(v, device=device).to(torch.bfloat16)
                            for k, v in self.weights.items()}

    def token(self, t: int, phase: int = I.PHASE_DECODE):
        if self.wl.projected:
            h = I.hidden_state(self.wl, self.layer, t, phase)
            return I.projected_token(self.wl, self.weights, h, self.device)
        return I.token(self.wl, t, phase, self.layer)

    def prefill(self, units):
        """Token-major prefill inputs of ``units`` (k, v, beta, gate; per-unit layout)."""
        wl = self.wl
        if not wl.projected:
            return I.prefill_streams(wl, units, self.layer)
        toks = [I.tokens_per_unit(wl, {k: v[None] for k, v in self.token(t, I.PHASE_PREFILL).items()})
                for t in range(wl.prefill)]
        return {key: np.ascontiguousarray(np.concatenate([tk[key] for tk in toks])[:, units])
                for key in ("k", "v", "beta", "gate")}


def start_states(wl: I.Workload, checked: np.ndarray, layer: int = 0, src: "TokenSource" = None) -> np.ndarray:
    """fp32 [U, d, d]: oracle prefill for checked units, stand-ins elsewhere."""
    U, d = wl.n_units, wl.d
    S0 = np.zeros((U, d, d), np.float32)
    others = np.setdiff1d(np.arange(U), checked)
    if len(others):
        S0[others] = I.surrogate_state(wl, others, layer)
    if wl.prefill > 0 and len(checked):
        st = (src or TokenSource(wl, layer)).prefill(checked)
        S, _ = orc.recurrence(np.zeros((len(checked), d, d)), None, st["k"], st["v"], st["beta"],
                              st["gate"], want_outputs=False)
        S0[checked] = S.astype(np.float32)
    sc = I.outlier_scale(wl, layer)
    if sc is not None:
        r, c = sc
        S0 = (S0 * r[:, :, None] * c[:, None, :]).astype(np.float32)
    return S0


def blob_host(views, units, fmt: str = "int8") -> orc.Blob:
    idx = torch.as_tensor(np.asarray(units), device=views["codes"].device, dtype=torch.long)
    g = lambda key: views[key].index_select(0, idx).cpu().numpy()
    return orc.Blob(g("codes"), g("sigma"), g("smooth"), g("comp_idx"), g("comp_vec"), fmt)


_GRIDS = {}


def code_grid(fmt: str) -> np.ndarray:
    """The sorted finite code values of a format (INT8: -127..127)."""
    if fmt not in _GRIDS:
        v = orc.code_values(np.arange(256, dtype=np.uint8).view(np.int8), fmt)
        v = v[np.isfinite(v) & (v >= -448) & ((v >= -127) if fmt == "int8" else True)]
        _GRIDS[fmt] = np.unique(v)
    return _GRIDS[fmt]


def check_quantizer(S_ref: np.ndarray, gpu: orc.Blob, n_c: int, rep: Report, where: str):
    """Compare the GPU's quantizer output with the oracle's on the same fp64 state."""
    fmt = gpu.fmt
    ob, x, scores = orc.qz(S_ref, n_c, fmt=fmt)
    U = S_ref.shape[0]
    if n_c > 0:
        mism = np.where((ob.comp_idx != gpu.comp_idx).any(axis=1))[0]
        if len(mism):
            # near-ties in the line scores may go either way
            srt = -np.sort(-scores, axis=1)
            for u in mism:
                hi, lo = srt[u, n_c - 1], srt[u, n_c] if srt.shape[1] > n_c else 0.0
                assert hi - lo <= AMBIG * max(abs(hi), 1e-300), (
                    f"{where}: unit {u} compensator choice {gpu.comp_idx[u]} vs oracle "
                    f"{ob.comp_idx[u]} with a clear score gap ({hi} vs {lo})")
            rep.ambiguous_selections += len(mism)
            ob, x, scores = orc.qz(S_ref, n_c, force_sel=gpu.comp_idx, fmt=fmt)
    bad = np.argwhere(gpu.codes != ob.codes)
    if len(bad):
        vg = orc.code_values(gpu.codes, fmt)
        vo = orc.code_values(ob.codes, fmt)
    flips = 0
    for (u, i, j) in bad:
        # allowed: the two codes are neighbours on the code grid (1 LSB for INT8,
        # one spacing for E4M3) and x lies within TIE_TAU of a spacing of their
        # midpoint, where the FP64 rounding order of the two sides decides
        xv, a, b = x[u, i, j], vg[u, i, j], vo[u, i, j]
        step = abs(a - b)
        lo, hi = min(a, b), max(a, b)
        grid = code_grid(fmt)
        neighbours = step > 0 and not np.any((grid > lo) & (grid < hi))
        near_mid = abs(xv - (a + b) / 2) <= TIE_TAU * step
        assert neighbours and near_mid, (
            f"{where}: code mismatch at unit {u} ({i},{j}): gpu {gpu.codes[u, i, j]} oracle "
            f"{ob.codes[u, i, j]} x={xv!r}")
        flips += 1
    n_codes = gpu.codes.size
    assert flips <= FLIP_BUDGET * n_codes, f"{where}: {flips} tie flips in {n_codes} codes"
    rep.codes_checked += n_codes
    rep.code_flips += flips
    np.testing.assert_allclose(gpu.sigma, ob.sigma, rtol=TOL_SCALE, atol=0, err_msg=where)
    np.testing.assert_allclose(gpu.smooth, ob.smooth, rtol=TOL_SCALE, atol=0, err_msg=where)
    if n_c > 0:
        for u in range(U):
            e = rel_l2(gpu.comp_vec[u], ob.comp_vec[u])
            assert e <= TOL_COMP, f"{where}: compensator vectors of unit {u} differ ({e})"


def run(wl: I.Workload, n_tokens: Optional[int] = None, checked: Optional[Sequence[int]] = None,
        layer: int = 0, dequant_every: int = 0, device="cuda") -> Report:
    """Run ``n_tokens`` decode steps (plus flushes) on the GPU and the oracle."""
    cfg = config_of(wl)
    U, d, W, nc = wl.n_units, wl.d, wl.window, wl.n_comp
    n_tokens = wl.decode if n_tokens is None else n_tokens
    checked = np.arange(U) if checked is None else np.asarray(sorted(set(int(c) for c in checked)))
    rep = Report(wl.name)
    print(f"[parity] {wl.name}: units={U} checked={len(checked)} d={d} W={W} n_c={nc} "
          f"tokens={n_tokens}", flush=True)

    src = TokenSource(wl, layer, device)
    S0 = start_states(wl, checked, layer, src)
    state = lq.new_state(cfg, device)
    views = lq.state_views(cfg, state)
    lq.lq_state_init(cfg, state, torch.from_numpy(S0).to(device))
    torch.cuda.synchronize()
    gb = blob_host(views, checked, wl.code_format)
    check_quantizer(S0[checked].astype(np.float64), gb, nc, rep, "init")
    assert int(views["fill"].max()) == 0 and int(views["fill"].min()) == 0
    S_hat = orc.dequant(gb)  # teacher-forced window-start state of the checked units

    # forced partial flushes (staggered windows): host mirror of every unit's fill
    fill = np.zeros(U, np.int64)
    seq_of = np.arange(U) // wl.n_v_heads
    sched = I.stagger_schedule(wl)
    o_dev = torch.empty((wl.n_seq, wl.n_v_heads, d), dtype=torch.float32, device=device)
    S_out = torch.empty((U, d, d), dtype=torch.float32, device=device)
    chk_dev = torch.as_tensor(checked, device=device, dtype=torch.long)
    frozen = None
    for t in range(n_tokens):
        tk = src.token(t)
        dev = {k_: torch.from_numpy(v_).to(device) for k_, v_ in tk.items()}
        if frozen is None:
            frozen = {k_: views[k_].clone() for k_ in ("codes", "sigma", "smooth", "comp_idx", "comp_vec")}
        lq.lq_decode_step(cfg, state, dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], o_dev)
        o_chk = o_dev.view(U, d).index_select(0, chk_dev).cpu().numpy()
        pu = I.tokens_per_unit(wl, {k_: v_[None] for k_, v_ in tk.items()})
        if wl.buffer_format == "fp16":
            # the token enters the window as the binary16 buffer holds it
            pu["k"], pu["v"] = orc.fp16_round(pu["k"]), orc.fp16_round(pu["v"])
        # the appended entry holds exactly the (rounded) k and v (the chain-free
        # form keeps its own vector n in place of v: the outputs, the state it
        # dequantizes to and the boundary's codes check it)
        j_chk = fill[checked]
        if wl.buffer_format != "nform":
            bv_chk = views["buf_v"].index_select(0, chk_dev).float().cpu().numpy()
            assert np.array_equal(bv_chk[np.arange(len(checked)), j_chk], pu["v"][0][checked]), \
                f"{wl.name}: token {t}: buffered v differs from the appended token"
        kh_of = (checked % wl.n_v_heads) // wl.group
        bk_all = views["buf_k"]
        bk_chk = bk_all[torch.as_tensor(checked // wl.n_v_heads, device=device),
                        torch.as_tensor(kh_of, device=device),
                        torch.as_tensor(j_chk, device=device)].float().cpu().numpy()
        assert np.array_equal(bk_chk, pu["k"][0][checked]), \
            f"{wl.name}: token {t}: buffered k differs from the appended token"
        sel = lambda a: np.ascontiguousarray(a[:, checked])
        S_hat, o_ref = orc.recurrence(S_hat, sel(pu["q"]), sel(pu["k"]), sel(pu["v"]), sel(pu["beta"]),
                                      sel(pu["gate"]))
        err = rel_l2(o_chk, o_ref[0])
        assert err <= TOL_OUT, f"{wl.name}: decode token {t}: output rel-L2 {err}"
        per = unit_rel_l2(o_chk, o_ref[0])
        worst = int(np.argmax(per))
        assert per[worst] <= TOL_OUT, \
            f"{wl.name}: decode token {t}: unit {checked[worst]} output rel-L2 {per[worst]}"
        rep.max_out_err = max(rep.max_out_err, err)
        rep.max_unit_out_err = max(rep.max_unit_out_err, float(per[worst]))
        rep.decode_calls += 1
        fill += 1
        # the stored low-bit state is read-only inside a window
        for k_, v_ in frozen.items():
            assert torch.equal(views[k_], v_), f"{wl.name}: decode step {t} modified {k_}"

        if dequant_every and (t % dequant_every == dequant_every - 1):
            lq.lq_dequant_state(cfg, state, S_out, include_buffer=True)
            g1 = S_out.index_select(0, chk_dev).cpu().numpy()
            e1, p1 = rel_l2(g1, S_hat), unit_rel_l2(g1, S_hat).max()
            lq.lq_dequant_state(cfg, state, S_out, include_buffer=False)
            g0 = S_out.index_select(0, chk_dev).cpu().numpy()
            r0 = orc.dequant(blob_host(views, checked, wl.code_format))
            e0, p0 = rel_l2(g0, r0), unit_rel_l2(g0, r0).max()
            assert max(e0, e1) <= TOL_STATE, f"{wl.name}: dequantized state at token {t}: {e0}, {e1}"
            assert max(p0, p1) <= TOL_STATE, \
                f"{wl.name}: dequantized state at token {t}: worst unit {p0}, {p1}"
            rep.max_state_err = max(rep.max_state_err, e0, e1)
            rep.max_unit_state_err = max(rep.max_unit_state_err, float(p0), float(p1))

        force_seq = np.zeros(wl.n_seq, np.uint8)
        if sched is not None:
            force_seq[(sched == t)] = 1
        due = (fill >= W) | ((force_seq[seq_of] != 0) & (fill > 0))
        if due.any():
            fm = torch.from_numpy(force_seq).to(device) if force_seq.any() else None
            lq.lq_window_flush(cfg, state, fm)
            torch.cuda.synchronize()
            rep.flushes += 1
            fill[due] = 0
            assert torch.equal(views["fill"].cpu(), torch.from_numpy(fill.astype(np.int32))), \
                f"{wl.name}: fill after flush at token {t}"
            due_c = np.where(due[checked])[0]
            if len(due_c):
                gb = blob_host(views, checked[due_c], wl.code_format)
                check_quantizer(S_hat[due_c], gb, nc, rep, f"flush after token {t}")
                S_hat[due_c] = orc.dequant(gb)
            frozen = None
    flags = lq.lq_read_status(cfg, state)
    assert flags == 0, f"{wl.name}: device flags {flags:#x}"
    print(f"[parity] {wl.name}: ok max_out_err={rep.max_out_err:.3g} "
          f"max_unit_out_err={rep.max_unit_out_err:.3g} max_unit_state_err={rep.max_unit_state_err:.3g} "
          f"flushes={rep.flushes} "
          f"flips={rep.code_flips}/{rep.codes_checked} ambiguous={rep.ambiguous_selections}",
          flush=True)
    return rep
