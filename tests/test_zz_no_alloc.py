"""The allocation-free boundary call (lq_window_flush_noalloc) against
lq_window_flush, through the C ABI, on two calls in a row (the second with
fewer units, so the library's scratch array still holds the first call's
longer list).  Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linear_attention_recurrent_gdn_amd as lq  # noqa: E402
from linear_attention_recurrent_gdn_amd import inputs as I  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

SECTIONS = ("status", "fill", "codes", "sigma", "smooth", "comp_idx", "comp_vec", "buf_k", "buf_v",
            "buf_beta", "buf_gate")


def _flush_both(wl, n_tok, forced_seq, seed):
    cfg = parity.config_of(wl)
    U, d = wl.n_units, wl.d
    gen = torch.Generator("cuda").manual_seed(seed)
    S0 = torch.randn((U, d, d), device="cuda", generator=gen)
    a, b = lq.new_state(cfg), lq.new_state(cfg)
    a.zero_()  # buffer entries past the tokens written stay equal (zero) in both
    b.zero_()
    o = torch.empty((wl.n_seq, wl.n_v_heads, d), device="cuda")
    for st in (a, b):
        lq.lq_state_init(cfg, st, S0)
    for t in range(n_tok):
        x = {k: torch.from_numpy(v).cuda() for k, v in I.token(wl, t).items()}
        for st in (a, b):
            lq.lq_decode_step(cfg, st, x["q"], x["k"], x["v"], x["beta"], x["gate"], o)
    mask = torch.zeros(wl.n_seq, dtype=torch.uint8, device="cuda")
    mask[forced_seq] = 1
    lq.lq_window_flush(cfg, a, mask)
    lq.lq_window_flush_noalloc(cfg, b, mask)
    torch.cuda.synchronize()
    va, vb = lq.state_views(cfg, a), lq.state_views(cfg, b)
    for key in SECTIONS:
        assert torch.equal(va[key], vb[key]), (wl.name, key)
    fill = va["fill"].cpu().numpy()
    return fill


def test_noalloc_flush_matches_flush_twice_second_smaller():
    # first call: 1,024 units, some sequences full (W tokens), the forced ones partial
    big = I.WORKLOADS["gdn_decode"].scaled(name="noalloc_big", window=8, prefill=0)
    fill = _flush_both(big, 8, [3, 40, 63], seed=1)
    assert (fill == 0).all()
    # second call: 6 units (the array still holds the longer list), channel gate,
    # a partial window flushed only where forced
    small = I.WORKLOADS["kda_decode"].scaled(name="noalloc_small", n_seq=2, n_v_heads=3, n_k_heads=3,
                                            window=16, n_comp=3, prefill=0)
    fill = _flush_both(small, 5, [1], seed=2)
    assert fill.tolist() == [5, 5, 5, 0, 0, 0]


def test_noalloc_rejects_more_units_than_its_scratch():
    wl = I.WORKLOADS["gdn_decode"].scaled(n_seq=lq.LQ_NOALLOC_MAX_UNITS // 16 + 1, window=1, prefill=0)
    cfg = parity.config_of(wl)
    # rejected on the host before anything is launched or touched: a small
    # allocation passed as a raw pointer stands in for the (22 GB) blob
    dummy = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(lq.LQError) as e:
        lq.lq_window_flush_noalloc(cfg, dummy.data_ptr(), None)
    assert e.value.code == lq.LQ_ESCRATCH


def test_noalloc_flush_matches_flush_chain_free_buffer():
    # the chain-free buffer's boundary kernel through the same scratch array:
    # a full window for most units, a forced partial one, then a smaller call
    big = I.WORKLOADS["gdn_decode"].scaled(name="noalloc_nf", window=8, prefill=0, buffer_format="nform")
    fill = _flush_both(big, 8, [5, 17], seed=3)
    assert (fill == 0).all()
    small = I.WORKLOADS["gdn_decode"].scaled(name="noalloc_nf_small", n_seq=3, n_v_heads=2, n_k_heads=1,
                                             window=12, n_comp=2, prefill=0, buffer_format="nform")
    fill = _flush_both(small, 7, [0, 2], seed=4)
    assert fill.tolist() == [0, 0, 7, 7, 0, 0]
