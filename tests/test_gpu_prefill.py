"""GPU parity of lq_prefill: a prompt through the chunked recurrence on the
FP64 matrix cores, then the quantizer.

The arXiv abstract ("Abstract (arXiv)" section, mlsanity.com paper page): the
recurrent state compresses the context and is quantized once at a window's
end.  The reference is the oracle's plain recurrence O1 over the prompt (FP64)
followed by its quantizer Qz -- both pinned in the CPU tests, so this needs no
new oracle arithmetic.  Bars: the prompt's outputs within 1e-4 relative L2
(they come out of FP64 arithmetic, so about 1e-7 is expected), and the
quantized final state with the tie and ambiguity rules of tests/parity.py.
Ragged prompts (not a multiple of the 16-token chunk), one-token and empty
prompts, a zero start state, GQA, both gates and both head sizes.  Needs an
MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linear_attention_recurrent_gdn_amd as lq  # noqa: E402
import oracle as orc  # noqa: E402
from linear_attention_recurrent_gdn_amd import inputs as I  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

W = I.WORKLOADS


def small(base, **kw):
    return W[base].scaled(**kw)


CASES = {
    # name: (workload, prompt tokens, start state: "random" or None)
    "gdn_ragged": (small("gdn_decode", name="p_gdn", n_seq=2, n_v_heads=3, n_k_heads=3), 100, "random"),
    "kda_ragged": (small("kda_decode", name="p_kda", n_seq=1, n_v_heads=3, n_k_heads=3), 77, "random"),
    "gqa_d64_zero_start": (small("gdn_decode", name="p_gqa", n_seq=2, n_v_heads=4, n_k_heads=2, d=64,
                                 n_comp=3), 40, None),
    "kda_d64": (small("kda_decode", name="p_kda64", n_seq=2, n_v_heads=2, n_k_heads=2, d=64, n_comp=2), 33,
                "random"),
    "one_token": (small("gdn_decode", name="p_one", n_seq=1, n_v_heads=2, n_k_heads=2), 1, "random"),
    "two_chunks_exact": (small("kda_decode", name="p_two", n_seq=1, n_v_heads=2, n_k_heads=2), 32, None),
    "e4m3_fp16buf": (small("gdn_decode", name="p_e4m3", n_seq=1, n_v_heads=3, n_k_heads=3, code_format="e4m3",
                           buffer_format="fp16"), 50, "random"),
}


def host_prompt(wl, T):
    toks = I.tokens(wl, 0, T, I.PHASE_PREFILL)
    return toks, I.tokens_per_unit(wl, toks)


def start_state(wl, kind):
    if kind is None:
        return None
    return I.surrogate_state(wl, np.arange(wl.n_units)).astype(np.float32)


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_parity(name):
    wl, T, s0 = CASES[name]
    cfg = parity.config_of(wl)
    U, d = wl.n_units, wl.d
    dev = torch.device("cuda", 0)
    toks, pu = host_prompt(wl, T)
    S0 = start_state(wl, s0)
    state = lq.new_state(cfg, dev)
    x = {k_: torch.from_numpy(v_).to(dev) for k_, v_ in toks.items()}
    o = torch.full((T, wl.n_seq, wl.n_v_heads, d), float("nan"), device=dev)
    print(f"[prefill] {name}: units={U} d={d} T={T} gate={wl.gate} start={'random' if s0 else 'zero'}",
          flush=True)
    lq.lq_prefill(cfg, state, None if S0 is None else torch.from_numpy(S0).to(dev),
                  x["q"], x["k"], x["v"], x["beta"], x["gate"], o)
    torch.cuda.synchronize()
    assert lq.lq_read_status(cfg, state) == 0

    S_init = np.zeros((U, d, d)) if S0 is None else S0.astype(np.float64)
    S_T, o_ref = orc.recurrence(S_init, pu["q"], pu["k"], pu["v"], pu["beta"], pu["gate"])
    o_gpu = o.view(T, U, d).cpu().numpy()
    err = parity.rel_l2(o_gpu, o_ref)
    per_tok = max(parity.rel_l2(o_gpu[t], o_ref[t]) for t in range(T))
    print(f"[prefill] {name}: outputs rel-L2 {err:.3g}, worst token {per_tok:.3g}", flush=True)
    assert err <= parity.TOL_OUT and per_tok <= parity.TOL_OUT

    views = lq.state_views(cfg, state)
    assert int(views["fill"].abs().max()) == 0
    rep = parity.Report(name)
    parity.check_quantizer(S_T, parity.blob_host(views, np.arange(U), wl.code_format), wl.n_comp, rep,
                           f"{name}: prefill end")
    print(f"[prefill] {name}: codes {rep.codes_checked}, tie flips {rep.code_flips}", flush=True)


def test_empty_prompt_is_state_init():
    wl = small("kda_decode", name="p_empty", n_seq=2, n_v_heads=2, n_k_heads=2)
    cfg = parity.config_of(wl)
    dev = torch.device("cuda", 0)
    S0 = torch.from_numpy(start_state(wl, "random")).to(dev)
    a, b = lq.new_state(cfg, dev), lq.new_state(cfg, dev)
    a.zero_()
    b.zero_()
    lq.lq_state_init(cfg, a, S0)
    lq.lq_prefill(cfg, b, S0, None, None, None, None, None, None)
    torch.cuda.synchronize()
    va, vb = lq.state_views(cfg, a), lq.state_views(cfg, b)
    for key in ("codes", "sigma", "smooth", "comp_idx", "comp_vec", "fill", "status"):
        assert torch.equal(va[key], vb[key]), key


@pytest.mark.parametrize("name", ["gdn_decode", "kda_decode"])
def test_prefill_fullsize_sampled(name):
    """The workload's whole prefill at full size (every unit on the GPU, inputs
    drawn on the device), the final quantized state checked on sampled units,
    and the prompt's outputs on those units for the last 64 tokens."""
    wl = W[name]
    cfg = parity.config_of(wl)
    U, d, T = wl.n_units, wl.d, wl.prefill
    dev = torch.device("cuda", 0)
    gen = torch.Generator(dev).manual_seed(77 + wl.seed)
    toks = [I.torch_token(wl, gen, dev) for _ in range(T)]
    x = {k_: torch.stack([tk[k_] for tk in toks]).contiguous() for k_ in toks[0]}
    del toks
    S0 = torch.randn((U, d, d), generator=gen, device=dev) * 0.3
    state = lq.new_state(cfg, dev)
    tail = 64
    o = torch.empty((T, wl.n_seq, wl.n_v_heads, d), device=dev) if T * U * d * 4 <= (1 << 32) else None
    print(f"[prefill] {name} full size: units={U} T={T} outputs={'yes' if o is not None else 'no'}", flush=True)
    lq.lq_prefill(cfg, state, S0, x["q"], x["k"], x["v"], x["beta"], x["gate"], o)
    torch.cuda.synchronize()
    assert lq.lq_read_status(cfg, state) == 0

    rng = np.random.default_rng(5)
    units = np.unique(np.concatenate([[0, U - 1, wl.n_v_heads], rng.choice(U, 12, replace=False)]))
    s_of, h_of = units // wl.n_v_heads, units % wl.n_v_heads
    kh_of = h_of // wl.group
    sel_key = lambda t: t[:, torch.as_tensor(s_of, device=dev), torch.as_tensor(kh_of, device=dev)].cpu().numpy()
    sel_val = lambda t: t[:, torch.as_tensor(s_of, device=dev), torch.as_tensor(h_of, device=dev)].cpu().numpy()
    pu = {"q": sel_key(x["q"]), "k": sel_key(x["k"]), "v": sel_val(x["v"]), "beta": sel_val(x["beta"]),
          "gate": sel_val(x["gate"])}
    S_T, o_ref = orc.recurrence(S0[torch.as_tensor(units, device=dev)].cpu().numpy().astype(np.float64),
                                pu["q"], pu["k"], pu["v"], pu["beta"], pu["gate"])
    if o is not None:
        o_gpu = o.view(T, U, d)[T - tail:, torch.as_tensor(units, device=dev)].cpu().numpy()
        err = parity.rel_l2(o_gpu, o_ref[T - tail:])
        print(f"[prefill] {name}: last {tail} tokens, outputs rel-L2 {err:.3g}", flush=True)
        assert err <= parity.TOL_OUT
    views = lq.state_views(cfg, state)
    rep = parity.Report(name)
    parity.check_quantizer(S_T, parity.blob_host(views, units), wl.n_comp, rep, f"{name}: prefill end")
    print(f"[prefill] {name}: codes {rep.codes_checked}, tie flips {rep.code_flips}", flush=True)
