"""The C-ABI library loads, exports every symbol include/lq.h declares, and its
host-side logic (layout, argument checks) behaves as documented.  CPU only:
nothing here launches a kernel; every rejected call returns before any HIP
call."""
import ctypes
import os
import re

import pytest

import linear_attention_recurrent_gdn_amd as lq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lq.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(lq_[a-z_0-9]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lq.LIB_PATH):
        from linear_attention_recurrent_gdn_amd import _build

        _build.build()
    return lq.load_library()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(lq.EXPORTS) == set(names), names
    for n in names:
        assert hasattr(lib, n), n


def cfg(**kw):
    base = dict(n_seq=3, n_v_heads=4, n_k_heads=2, d_k=128, d_v=128, window=64, n_comp=4,
                gate_kind=lq.LQ_GATE_SCALAR)
    base.update(kw)
    return lq.Config(**base)


def test_layout_sections_aligned_and_disjoint(lib):
    for c in (cfg(), cfg(gate_kind=lq.LQ_GATE_CHANNEL, d_k=64, d_v=64, window=7, n_comp=0),
              cfg(n_seq=512, n_v_heads=32, n_k_heads=32), cfg(buffer_format=lq.LQ_BUFFER_FP16, window=5)):
        L = lq.lq_state_layout(c)
        U, D, W, nc = c.n_units, c.d_k, c.window, c.n_comp
        g = D if c.gate_kind == lq.LQ_GATE_CHANNEL else 1
        e = 2 if c.buffer_format == lq.LQ_BUFFER_FP16 else 4
        sizes = {
            "status": 4, "fill": 4 * U, "codes": U * D * D, "sigma": 4 * U * D,
            "smooth": 4 * U * D, "comp_idx": 4 * U * nc, "comp_vec": 4 * U * nc * D,
            "buf_k": e * c.n_seq * c.n_k_heads * W * D, "buf_v": e * U * W * D,
            "buf_beta": 4 * U * W, "buf_gate": 4 * U * W * g, "work": 4 * (U + 1),
        }
        spans = sorted((L[k], L[k] + n, k) for k, n in sizes.items())
        for (a0, a1, ka), (b0, b1, kb) in zip(spans, spans[1:]):
            assert a1 <= b0, (ka, kb)
        for k in sizes:
            assert L[k] % 256 == 0, k
        assert spans[-1][1] <= L["total_bytes"] == lq.lq_state_bytes(c)
        assert L["total_bytes"] % 256 == 0


def test_state_bytes_matches_int8_footprint(lib):
    # 16 KiB of codes per (sequence, head) at d = 128: a quarter of the FP32 state
    c = cfg(n_seq=512, n_v_heads=32, n_k_heads=32)
    L = lq.lq_state_layout(c)
    assert L["sigma"] - L["codes"] >= 512 * 32 * 128 * 128


@pytest.mark.parametrize("bad,code", [
    (dict(n_seq=0), lq.LQ_EINVAL),
    (dict(n_v_heads=3, n_k_heads=2), lq.LQ_EINVAL),
    (dict(gate_kind=7), lq.LQ_EINVAL),
    (dict(code_format=2), lq.LQ_EINVAL),
    (dict(flush_cus=-1), lq.LQ_EINVAL),
    (dict(load_policy=3), lq.LQ_EINVAL),
    (dict(load_policy=-1), lq.LQ_EINVAL),
    (dict(buffer_format=3), lq.LQ_EINVAL),
    (dict(buffer_format=lq.LQ_BUFFER_NFORM, gate_kind=lq.LQ_GATE_CHANNEL), lq.LQ_EUNSUPPORTED),
    (dict(buffer_format=lq.LQ_BUFFER_NFORM, d_k=64, d_v=64), lq.LQ_EUNSUPPORTED),
    (dict(window=0), lq.LQ_EINVAL),
    (dict(n_comp=-1), lq.LQ_EINVAL),
    (dict(d_k=96, d_v=96), lq.LQ_EUNSUPPORTED),
    (dict(d_k=64, d_v=128), lq.LQ_EUNSUPPORTED),
    (dict(window=257), lq.LQ_EUNSUPPORTED),
    (dict(n_comp=17), lq.LQ_EUNSUPPORTED),
    (dict(n_seq=1 << 26, n_v_heads=64, n_k_heads=64), lq.LQ_EUNSUPPORTED),
])
def test_config_rejected(lib, bad, code):
    c = cfg(**bad).c()
    n = ctypes.c_size_t(0)
    assert lib.lq_state_bytes(ctypes.byref(c), ctypes.byref(n)) == code
    assert lib.lq_state_init(ctypes.byref(c), ctypes.c_void_p(1 << 20), None, None) == code
    with pytest.raises(lq.LQError):
        lq.lq_state_bytes(cfg(**bad))


def test_null_and_misaligned_pointers_rejected(lib):
    c = cfg().c()
    P = ctypes.c_void_p
    ok = P(1 << 20)  # aligned, never dereferenced: every call below fails validation first
    assert lib.lq_state_bytes(None, ctypes.byref(ctypes.c_size_t())) == lq.LQ_EINVAL
    assert lib.lq_state_bytes(ctypes.byref(c), None) == lq.LQ_EINVAL
    assert lib.lq_state_init(ctypes.byref(c), None, None, None) == lq.LQ_EINVAL
    assert lib.lq_state_init(ctypes.byref(c), P((1 << 20) + 16), None, None) == lq.LQ_EINVAL
    assert lib.lq_state_init(ctypes.byref(c), ok, P((1 << 20) + 4), None) == lq.LQ_EINVAL
    args = [ok] * 7
    for i in range(7):
        a = list(args)
        a[i] = None
        assert lib.lq_decode_step(ctypes.byref(c), *a, None) == lq.LQ_EINVAL
        assert lib.lq_fp32_decode_step(ctypes.byref(c), *a, None) == lq.LQ_EINVAL
    a = list(args)
    a[1] = P((1 << 20) + 8)  # q not 16-byte aligned
    assert lib.lq_decode_step(ctypes.byref(c), *a, None) == lq.LQ_EINVAL
    assert lib.lq_window_flush(ctypes.byref(c), None, None, None) == lq.LQ_EINVAL
    assert lib.lq_dequant_state(ctypes.byref(c), ok, None, 0, None) == lq.LQ_EINVAL
    assert lib.lq_read_status(ctypes.byref(c), ok, None, None) == lq.LQ_EINVAL
    assert lib.lq_read_status(ctypes.byref(c), None, ctypes.byref(ctypes.c_uint32()), None) == lq.LQ_EINVAL
    assert lib.lq_clear_status(ctypes.byref(c), None, None) == lq.LQ_EINVAL
    assert lib.lq_clear_status(ctypes.byref(c), P((1 << 20) + 16), None) == lq.LQ_EINVAL
    # prefill: a negative prompt length, a missing input for a non-empty prompt,
    # misaligned pointers; an empty prompt needs no inputs (then it is an init)
    assert lib.lq_prefill(ctypes.byref(c), ok, None, -1, ok, ok, ok, ok, ok, ok, None) == lq.LQ_EINVAL
    assert lib.lq_prefill(ctypes.byref(c), None, None, 0, None, None, None, None, None, None, None) == lq.LQ_EINVAL
    pargs = [ok] * 5
    for i in range(5):
        a = list(pargs)
        a[i] = None
        assert lib.lq_prefill(ctypes.byref(c), ok, None, 3, *a, ok, None) == lq.LQ_EINVAL
    a = list(pargs)
    a[2] = P((1 << 20) + 4)  # v not 16-byte aligned
    assert lib.lq_prefill(ctypes.byref(c), ok, None, 3, *a, ok, None) == lq.LQ_EINVAL
    assert lib.lq_prefill(ctypes.byref(c), ok, None, 3, *pargs, P((1 << 20) + 8), None) == lq.LQ_EINVAL
    big = cfg(n_seq=1 << 15, n_v_heads=64, n_k_heads=64).c()  # 16 tokens of v reach 2^32 elements
    assert lib.lq_prefill(ctypes.byref(big), ok, None, 3, *pargs, ok, None) == lq.LQ_EUNSUPPORTED


def test_strerror_is_static(lib):
    for code in (0, -1, -2, -3, 42):
        assert isinstance(lq.lq_strerror(code), str) and lq.lq_strerror(code)


def test_binding_checks_tensor_sizes():
    torch = pytest.importorskip("torch")
    c = cfg()
    with pytest.raises(ValueError):
        lq.lq_decode_step(c, torch.zeros(8, dtype=torch.uint8), *([torch.zeros(1)] * 6))
