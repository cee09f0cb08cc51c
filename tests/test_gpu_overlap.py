"""The boundary call beside the decode: a persistent grid limited to part of
the CUs (lq_config.flush_cus), and a multi-layer schedule that runs each
layer's boundary call on a second stream while the next layers decode, as
the benchmark does for a stack of layers.  Both must leave every output and
every byte of every blob exactly as the plain schedule does: the work per
unit is the same, only its placement and timing differ.  Needs an MI355X."""
import dataclasses

import pytest

torch = pytest.importorskip("torch")

import linear_attention_recurrent_gdn_amd as lq  # noqa: E402
from linear_attention_recurrent_gdn_amd import inputs as I  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _tok(wl, t, layer):
    return {k: torch.from_numpy(v).cuda() for k, v in I.token(wl, t, layer=layer).items()}


def _blob_equal(cfg, a, b, what):
    va, vb = lq.state_views(cfg, a), lq.state_views(cfg, b)
    for key in va:
        assert torch.equal(va[key], vb[key]), (what, key)


@pytest.mark.parametrize("name,cus,buf", [("gdn_decode", 5, "fp32"), ("gdn_decode", 96, "fp32"),
                                          ("kda_decode", 13, "fp32"), ("gdn_decode", 7, "nform")])
def test_flush_on_fewer_cus_is_bitwise_equal(name, cus, buf):
    wl = I.WORKLOADS[name].scaled(name=f"{name}_cus", window=8, prefill=0, n_seq=16, buffer_format=buf)
    cfg = parity.config_of(wl)
    few = dataclasses.replace(cfg, flush_cus=cus)
    U, d = wl.n_units, wl.d
    gen = torch.Generator("cuda").manual_seed(11)
    S0 = torch.randn((U, d, d), device="cuda", generator=gen)
    a, b = lq.new_state(cfg), lq.new_state(cfg)
    a.zero_()
    b.zero_()
    lq.lq_state_init(cfg, a, S0)
    lq.lq_state_init(few, b, S0)  # the same kernel on the smaller grid
    _blob_equal(cfg, a, b, "init")
    o = torch.empty((wl.n_seq, wl.n_v_heads, d), device="cuda")
    mask = torch.zeros(wl.n_seq, dtype=torch.uint8, device="cuda")
    mask[3] = 1
    for t in range(2 * wl.window + 3):
        x = _tok(wl, t, 0)
        for st in (a, b):
            lq.lq_decode_step(cfg, st, x["q"], x["k"], x["v"], x["beta"], x["gate"], o)
        if t % wl.window == wl.window - 1 or t == 2 * wl.window + 1:
            fm = mask if t == 2 * wl.window + 1 else None  # a forced partial window too
            lq.lq_window_flush(cfg, a, fm)
            lq.lq_window_flush(few, b, fm)
    torch.cuda.synchronize()
    _blob_equal(cfg, a, b, "flush")
    Sa = torch.empty((U, d, d), device="cuda")
    Sb = torch.empty((U, d, d), device="cuda")
    lq.lq_dequant_state(cfg, a, Sa, include_buffer=True)
    lq.lq_dequant_state(few, a, Sb, include_buffer=True)
    torch.cuda.synchronize()
    assert torch.equal(Sa, Sb)


def test_flush_cus_rejects_negative():
    wl = I.WORKLOADS["tiny_gdn"]
    cfg = dataclasses.replace(parity.config_of(wl), flush_cus=-1)
    with pytest.raises(lq.LQError) as e:
        lq.lq_state_bytes(cfg)
    assert e.value.code == lq.LQ_EINVAL


class _Stack:
    """L layers (one blob each) of a small GQA workload with windows
    staggered across layers like the benchmark's stack: layer l starts
    floor(l W / L) tokens later (forced partial flushes during the first
    window)."""

    def __init__(self, L=3, seed=5):
        self.wl = I.WORKLOADS["hybrid_stack"].scaled(name="stack_small", layers=L, n_seq=8, n_v_heads=4,
                                                    n_k_heads=2, window=8, n_comp=2, prefill=0,
                                                    projected=False)
        self.cfg = parity.config_of(self.wl)
        self.L, self.W = L, self.wl.window
        self.offsets = [(l * self.W) // L for l in range(L)]
        gen = torch.Generator("cuda").manual_seed(seed)
        U, d = self.wl.n_units, self.wl.d
        self.S0 = [torch.randn((U, d, d), device="cuda", generator=gen) * 0.3 for _ in range(L)]
        self.toks = [[_tok(self.wl, t, l) for t in range(64)] for l in range(L)]
        self.all_seq = torch.ones(self.wl.n_seq, dtype=torch.uint8, device="cuda")

    def states(self):
        out = []
        for l in range(self.L):
            st = lq.new_state(self.cfg)
            st.zero_()
            lq.lq_state_init(self.cfg, st, self.S0[l])
            out.append(st)
        return out

    def due(self, l, t):
        """Whether layer l's boundary follows token t, and its force mask: the
        first window is cut short (forced) after W - offset tokens, later
        ones are full every W tokens."""
        first = self.W - 1 - self.offsets[l]
        if t < first or (t - first) % self.W != 0:
            return False, None
        return True, (self.all_seq if t == first and self.offsets[l] > 0 else None)

    def run(self, blobs, outs, t0, t1, side=None, flush_cus=0):
        """Tokens t0..t1-1; with `side` (a stream), each layer's boundary call
        runs there right after that layer's decode, and the layer's next
        decode waits for it."""
        cur = torch.cuda.current_stream()
        cfg_side = dataclasses.replace(self.cfg, flush_cus=flush_cus)
        pending = [None] * self.L
        for t in range(t0, t1):
            for l in range(self.L):
                if pending[l] is not None:
                    cur.wait_event(pending[l])
                    pending[l] = None
                x = self.toks[l][t % 64]
                lq.lq_decode_step(self.cfg, blobs[l], x["q"], x["k"], x["v"], x["beta"], x["gate"], outs[t][l])
                due, fm = self.due(l, t)
                if due:
                    if side is None:
                        lq.lq_window_flush(self.cfg, blobs[l], fm)
                    else:
                        ev = torch.cuda.Event()
                        ev.record(cur)
                        side.wait_event(ev)
                        lq.lq_window_flush(cfg_side, blobs[l], fm, stream=side)
                        done = torch.cuda.Event()
                        done.record(side)
                        pending[l] = done
        for l in range(self.L):
            if pending[l] is not None:
                cur.wait_event(pending[l])

    def out_buffers(self, n):
        wl = self.wl
        return [[torch.full((wl.n_seq, wl.n_v_heads, wl.d), float("nan"), device="cuda") for _ in range(self.L)]
                for _ in range(n)]


def test_boundary_beside_decode_matches_plain_schedule():
    sk = _Stack()
    n = 4 * sk.W + 3
    ref, ovl = sk.states(), sk.states()
    o_ref, o_ovl = sk.out_buffers(n), sk.out_buffers(n)
    sk.run(ref, o_ref, 0, n)
    side = torch.cuda.Stream()
    sk.run(ovl, o_ovl, 0, n, side=side, flush_cus=3)
    torch.cuda.synchronize()
    for t in range(n):
        for l in range(sk.L):
            assert torch.equal(o_ref[t][l], o_ovl[t][l]), (t, l)
    for l in range(sk.L):
        _blob_equal(sk.cfg, ref[l], ovl[l], f"layer {l}")
        flags = lq.lq_read_status(sk.cfg, ovl[l])
        assert flags == 0, flags


def test_boundary_beside_decode_in_a_graph():
    # the same schedule captured as one HIP graph (the second stream forks
    # from and joins the capture stream through events) and replayed once,
    # against the plain schedule run eagerly
    sk = _Stack(seed=9)
    n0, n = sk.W, 3 * sk.W + 2
    ref, ovl = sk.states(), sk.states()
    o_ref, o_ovl = sk.out_buffers(n), sk.out_buffers(n)
    sk.run(ref, o_ref, 0, n)
    sk.run(ovl, o_ovl, 0, n0)  # eager up to the captured tokens
    cap = torch.cuda.Stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        sk.run(ovl, o_ovl, n0, n, side=side, flush_cus=8)
    g.replay()
    torch.cuda.synchronize()
    for t in range(n):
        for l in range(sk.L):
            assert torch.equal(o_ref[t][l], o_ovl[t][l]), (t, l)
    for l in range(sk.L):
        _blob_equal(sk.cfg, ref[l], ovl[l], f"layer {l}")
