"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every unit runs on the GPU, the oracle follows a sample of
units (first, last and seeded random ones) through every decode token and
window boundary, with the tolerances and teacher forcing of tests/parity.py.
Sampled units start from the oracle's own prefill of the workload's
prefill stream; the others from seeded stand-in states.  Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from linear_attention_recurrent_gdn_amd import inputs as I  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def sample_units(wl, n=24, seed=7):
    rng = np.random.default_rng(seed)
    U = wl.n_units
    picks = {0, 1, wl.n_v_heads, U // 2, U - 1}
    picks.update(int(x) for x in rng.choice(U, n, replace=False))
    return sorted(picks)


@pytest.mark.parametrize("name,fmt", [("tiny_gdn", "int8"), ("gdn_decode", "int8"), ("kda_decode", "int8"),
                                      ("gdn_serving", "int8"), ("gdn_decode", "e4m3"), ("kda_decode", "e4m3"),
                                      ("gdn_decode", "int8+fp16"), ("kda_decode", "int8+fp16"),
                                      ("gdn_decode", "int8+nform"), ("gdn_serving", "int8+nform")])
def test_fullsize_parity(name, fmt):
    code, _, buf = fmt.partition("+")
    wl = I.WORKLOADS[name].scaled(code_format=code, buffer_format=buf or "fp32")
    checked = None if wl.n_units == 1 else sample_units(wl)
    n_tok = wl.decode + (wl.window if wl.stagger else 0)  # staggered: warm-up window first
    rep = parity.run(wl, n_tokens=n_tok, checked=checked, dequant_every=wl.window // 2 + 1)
    assert rep.decode_calls == n_tok
    assert rep.flushes >= 1


@pytest.mark.parametrize("layer", [0, 35])
def test_fullsize_parity_hybrid_stack_layer(layer):
    # layers are independent blobs with their own projection weights; two of
    # the 36 are followed here (first and last), each at the full 256 x 32
    # units with GQA (16 key heads), 64 tokens and one window boundary
    wl = I.WORKLOADS["hybrid_stack"]
    rep = parity.run(wl, n_tokens=wl.decode, checked=sample_units(wl, 16), layer=layer,
                     dequant_every=33)
    assert rep.flushes == 1


@pytest.mark.parametrize("name,layer", [("gdn_decode", 0), ("kda_decode", 0), ("hybrid_stack", 0)])
def test_fp32_kernel_fullsize_sampled(name, layer):
    # the FP32-state comparison kernel at the full launch size the benchmark
    # times (every unit of the workload in one launch), its outputs and states
    # followed unit by unit on a sample against the oracle's plain recurrence
    import linear_attention_recurrent_gdn_amd as lq
    import oracle as orc

    wl = I.WORKLOADS[name]
    cfg = parity.config_of(wl)
    U, d = wl.n_units, wl.d
    checked = np.asarray(sample_units(wl, 16))
    gen = torch.Generator("cuda").manual_seed(11)
    S = torch.randn((U, d, d), device="cuda", generator=gen) * 0.5
    chk = torch.as_tensor(checked, device="cuda")
    S_ref = S.index_select(0, chk).double().cpu().numpy()
    src = parity.TokenSource(wl, layer)
    o = torch.empty((wl.n_seq, wl.n_v_heads, d), device="cuda")
    worst = 0.0
    for t in range(6):
        tk = src.token(t)
        dev = {k: torch.from_numpy(v).cuda() for k, v in tk.items()}
        lq.lq_fp32_decode_step(cfg, S, dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], o)
        pu = I.tokens_per_unit(wl, {k: v[None] for k, v in tk.items()})
        sel = lambda a: np.ascontiguousarray(a[:, checked])
        S_ref, o_ref = orc.recurrence(S_ref, sel(pu["q"]), sel(pu["k"]), sel(pu["v"]), sel(pu["beta"]),
                                      sel(pu["gate"]))
        per = parity.unit_rel_l2(o.view(U, d).index_select(0, chk).cpu().numpy(), o_ref[0])
        assert per.max() <= 1e-5, (t, checked[int(np.argmax(per))], per.max())
        worst = max(worst, float(per.max()))
    per_s = parity.unit_rel_l2(S.index_select(0, chk).cpu().numpy(), S_ref)
    assert per_s.max() <= 1e-5, per_s.max()
    print(f"[fp32 kernel] {name}: {U} units per launch, {len(checked)} followed, worst unit output "
          f"rel-L2 {worst:.3g}, state {per_s.max():.3g}", flush=True)


# launches of more than 2048 units take the large-launch form of the decode
# kernel (no early code conversion, non-temporal 512-byte stores): a unit
# count that is no multiple of the XCD grouping (4102 units, two value heads
# per key head), four value heads per key head with more compensators than
# the form holds in registers, and a window above 128 with E4M3 codes and the
# binary16 buffer, each on a sample of units with a boundary inside the run
LARGE_CASES = {
    "large_odd_gqa2": I.WORKLOADS["gdn_decode"].scaled(
        name="large_odd_gqa2", n_seq=2051, n_v_heads=2, n_k_heads=1, window=16, n_comp=3, prefill=24,
        decode=40, outlier_rows=0, outlier_cols=0),
    "large_gqa4_nc7": I.WORKLOADS["gdn_decode"].scaled(
        name="large_gqa4_nc7", n_seq=256, n_v_heads=16, n_k_heads=4, window=32, n_comp=7, prefill=24,
        decode=45),
    "large_kda_w200_e4m3_h16": I.WORKLOADS["kda_decode"].scaled(
        name="large_kda_w200_e4m3_h16", n_seq=1024, n_v_heads=4, n_k_heads=4, window=200, n_comp=8,
        prefill=16, decode=210, code_format="e4m3", buffer_format="fp16"),
}


@pytest.mark.parametrize("name", list(LARGE_CASES))
def test_large_launch_parity(name):
    wl = LARGE_CASES[name]
    assert wl.n_units > 2048
    picks = {0, 1, 2, 3, wl.n_units - 1, wl.n_units - 2, wl.n_units // 2}
    rng = np.random.default_rng(5)
    picks.update(int(x) for x in rng.choice(wl.n_units, 9, replace=False))
    rep = parity.run(wl, checked=sorted(picks), dequant_every=wl.window // 2 + 3)
    assert rep.flushes >= 1 and rep.decode_calls == wl.decode


@pytest.mark.parametrize("d,n_seq,gate", [(128, 640, "scalar"), (64, 1280, "scalar"), (128, 640, "channel")])
def test_flush_more_than_64_items_per_workgroup(d, n_seq, gate):
    # Every unit due at each boundary, more units than 64 per resident
    # workgroup of the boundary kernel (256 workgroups at d = 128, 512 at
    # d = 64): each workgroup reads its part of the work list 64 items at a
    # time, so the later items come from a second read.  Sampled units include
    # the last ones (item 79 of their workgroup at d = 128).
    base = "gdn_decode" if gate == "scalar" else "kda_decode"
    wl = I.WORKLOADS[base].scaled(name=f"many_{d}_{gate}", n_seq=n_seq, n_v_heads=32, n_k_heads=32, d=d,
                                  window=2, prefill=8, decode=4, outlier_rows=0, outlier_cols=0)
    assert wl.n_units > 64 * (256 if d == 128 else 512)
    units = sample_units(wl, 12)
    units += list(range(wl.n_units - 4, wl.n_units))
    rep = parity.run(wl, n_tokens=4, checked=units, dequant_every=3)
    assert rep.flushes == 2
