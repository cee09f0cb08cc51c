"""lq_config.load_policy only changes how the decode step's loads use the
caches (streaming or ordinary), never what they read: outputs and every blob
byte must be the same bit for bit under LQ_LOADS_AUTO, LQ_LOADS_STREAM and
LQ_LOADS_CACHED, for launches of the small form (up to 2,048 units) and of
the large form, with each gate and buffer format.  Parity of the automatic
policy with the oracle is covered by the parity tests.  Needs an MI355X."""
import dataclasses

import pytest

torch = pytest.importorskip("torch")

import linear_attention_recurrent_gdn_amd as lq  # noqa: E402
from linear_attention_recurrent_gdn_amd import inputs as I  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

POLICIES = (lq.LQ_LOADS_AUTO, lq.LQ_LOADS_STREAM, lq.LQ_LOADS_CACHED)


# (workload, n_seq, buffer format, code format): 16 sequences give the small
# form, 72 x 32 heads = 2,304 units the large one
@pytest.mark.parametrize("name,n_seq,buf,code", [
    ("gdn_serving", 16, "fp32", "int8"),
    ("gdn_serving", 72, "fp32", "int8"),
    ("kda_decode", 16, "fp32", "int8"),
    ("kda_decode", 72, "fp32", "e4m3"),
    ("hybrid_stack", 72, "fp16", "int8"),
    ("gdn_serving", 72, "nform", "int8"),
    ("gdn_serving", 16, "nform", "e4m3"),
])
def test_load_policies_bitwise_equal(name, n_seq, buf, code):
    wl = I.WORKLOADS[name].scaled(name=f"{name}_lp", window=8, prefill=0, n_seq=n_seq, buffer_format=buf,
                                  code_format=code, projected=False, layers=1)
    base = parity.config_of(wl)
    cfgs = [dataclasses.replace(base, load_policy=p) for p in POLICIES]
    U, d = wl.n_units, wl.d
    print(f"[load policy] {name}: {U} units, buffer {buf}, codes {code}", flush=True)
    gen = torch.Generator("cuda").manual_seed(23)
    S0 = torch.randn((U, d, d), device="cuda", generator=gen)
    blobs = [lq.new_state(c) for c in cfgs]
    for c, b in zip(cfgs, blobs):
        b.zero_()
        lq.lq_state_init(c, b, S0)
    outs = [torch.empty((wl.n_seq, wl.n_v_heads, d), device="cuda") for _ in cfgs]
    for t in range(wl.window + 5):  # a full window, its boundary, then a partial one
        x = {k: torch.from_numpy(v).cuda() for k, v in I.token(wl, t, layer=0).items()}
        for c, b, o in zip(cfgs, blobs, outs):
            lq.lq_decode_step(c, b, x["q"], x["k"], x["v"], x["beta"], x["gate"], o)
        torch.cuda.synchronize()
        assert torch.isfinite(outs[0]).all(), t
        for p, o in zip(POLICIES[1:], outs[1:]):
            assert torch.equal(outs[0], o), (t, p)
        if t == wl.window - 1:
            for c, b in zip(cfgs, blobs):
                lq.lq_window_flush(c, b)
    torch.cuda.synchronize()
    va = lq.state_views(cfgs[0], blobs[0])
    for p, c, b in zip(POLICIES[1:], cfgs[1:], blobs[1:]):
        vb = lq.state_views(c, b)
        for key in va:
            assert torch.equal(va[key], vb[key]), (p, key)
        assert lq.lq_read_status(c, b) == 0
