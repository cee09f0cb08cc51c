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
                                      ("gdn_decode", "int8+fp16"), ("kda_decode", "int8+fp16")])
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
