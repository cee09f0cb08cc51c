"""Quality of the windowed 8-bit path (INT8 and E4M3 codes) against the FP64 recurrence, next to the
naive per-token quantization ablation and the FP32-state kernel.

The bedrocknews.com review of arXiv 2609.38166: naive per-token quantization of
the state collapses quality, while quantizing once per window with the outliers
kept in high precision stays close to the FP32 baseline; the arXiv abstract
("Abstract (arXiv)", mlsanity.com paper page) calls the result comparable to
FP32.  The pages give no numbers, so this is a report with two sanity gates:
the windowed path must beat the naive ablation, and the FP32 kernel must track
the FP64 recurrence to fp32 accuracy.

Per workload (all units of a reduced batch, the full token count):
  reference   O1, the plain recurrence in FP64 from the unquantized start state;
  leapquant   the library free-running (init, decode steps, window flushes);
  naive       the oracle's windowed form with W = 1, no compensators, no smoothing;
  fp32        the library's FP32-state kernel.
Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linear_attention_recurrent_gdn_amd as lq  # noqa: E402
import oracle as orc  # noqa: E402
from linear_attention_recurrent_gdn_amd import inputs as I  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_gdn": dict(),
    "gdn_decode": dict(n_seq=2),
    "kda_decode": dict(n_seq=1),
    "gdn_serving": dict(n_seq=1, stagger=False),
}


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("variant", ["int8", "e4m3", "int8+fp16"])
@pytest.mark.parametrize("name", list(CASES))
def test_quality_report(name, variant):
    fmt, _, buf = variant.partition("+")
    buf = buf or "fp32"
    wl = I.WORKLOADS[name].scaled(code_format=fmt, buffer_format=buf, **CASES[name])
    cfg = parity.config_of(wl)
    U, d, W, T = wl.n_units, wl.d, wl.window, wl.decode
    S0 = parity.start_states(wl, np.arange(U))
    toks = [I.token(wl, t) for t in range(T)]
    pu = [I.tokens_per_unit(wl, {k: v[None] for k, v in tk.items()}) for tk in toks]
    st = {key: np.ascontiguousarray(np.concatenate([p[key] for p in pu])) for key in pu[0]}

    _, o_ref = orc.recurrence(S0.astype(np.float64), st["q"], st["k"], st["v"], st["beta"], st["gate"])
    o_naive = orc.windowed_run(S0, st["q"], st["k"], st["v"], st["beta"], st["gate"], 1, 0, smooth=False)
    o_o2 = orc.windowed_run(S0, st["q"], st["k"], st["v"], st["beta"], st["gate"], W, wl.n_comp, fmt=fmt,
                            buffer=buf)

    dev = torch.device("cuda", 0)
    state = lq.new_state(cfg, dev)
    lq.lq_state_init(cfg, state, torch.from_numpy(S0).to(dev))
    S = torch.from_numpy(S0).to(dev)
    o = torch.empty((wl.n_seq, wl.n_v_heads, d), device=dev)
    o32 = torch.empty_like(o)
    o_lq, o_fp32 = np.zeros((T, U, d)), np.zeros((T, U, d))
    for t in range(T):
        x = {k: torch.from_numpy(v).to(dev) for k, v in toks[t].items()}
        lq.lq_decode_step(cfg, state, x["q"], x["k"], x["v"], x["beta"], x["gate"], o)
        lq.lq_fp32_decode_step(cfg, S, x["q"], x["k"], x["v"], x["beta"], x["gate"], o32)
        if (t + 1) % W == 0:
            lq.lq_window_flush(cfg, state, None)
        o_lq[t] = o.view(U, d).cpu().numpy()
        o_fp32[t] = o32.view(U, d).cpu().numpy()
    assert lq.lq_read_status(cfg, state) == 0

    e = {"leapquant": rel(o_lq, o_ref), "naive_per_token": rel(o_naive, o_ref), "fp32_kernel": rel(o_fp32, o_ref),
         "oracle_windowed": rel(o_o2, o_ref), "leapquant_vs_oracle_windowed": rel(o_lq, o_o2)}
    last = {"leapquant": rel(o_lq[-1], o_ref[-1]), "naive_per_token": rel(o_naive[-1], o_ref[-1])}
    print(f"[quality] {wl.name} {variant} units={U} tokens={T} W={W} n_c={wl.n_comp}: "
          + " ".join(f"{k}={v:.3e}" for k, v in e.items())
          + f" | last token: leapquant={last['leapquant']:.3e} naive={last['naive_per_token']:.3e}", flush=True)
    assert e["leapquant"] < e["naive_per_token"]
    assert e["fp32_kernel"] < 1e-4
    assert e["leapquant_vs_oracle_windowed"] < 1e-3
