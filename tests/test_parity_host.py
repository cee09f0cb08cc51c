"""Host logic of the parity harness (CPU only): the per-unit gate catches a
single bad unit that the aggregate over all checked units lets through."""
import numpy as np

from tests import parity


def test_per_unit_gate_catches_one_bad_unit():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((29, 128))
    got = ref * (1 + 1e-7 * rng.standard_normal(ref.shape))
    bad = ref[7] + 5e-4 * np.linalg.norm(ref[7]) * rng.standard_normal(128) / np.sqrt(128)
    got[7] = bad
    agg = parity.rel_l2(got, ref)
    per = parity.unit_rel_l2(got, ref)
    assert agg <= parity.TOL_OUT < per.max()
    assert int(np.argmax(per)) == 7


def test_unit_rel_l2_zero_reference_is_absolute():
    ref = np.zeros((2, 4))
    got = np.array([[0.0, 0, 0, 0], [3.0, 4.0, 0, 0]])
    assert parity.unit_rel_l2(got, ref).tolist() == [0.0, 5.0]
