"""The per-group error metric of the gradient parity tests, on the CPU: an
error confined to one token group's tile must fail it even where the
whole-tensor relative error would pass."""
import numpy as np

from tests.gpu_util import TOL, rel_l2, rel_l2_groups


def test_one_wrong_group_is_not_diluted():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((32, 64, 48))
    got = ref * (1 + 1e-3 * rng.standard_normal(ref.shape))
    assert rel_l2_groups(got, ref, 1) <= TOL["bf16"]
    got[5, 32:] = 0.0  # one group's ragged tail tile dropped
    assert rel_l2(got, ref) <= 0.15  # the whole tensor barely notices
    assert rel_l2_groups(got, ref, 1) > 0.5


def test_small_groups_are_measured_against_the_typical_group():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((8, 4, 16))
    ref[3] *= 1e-6  # a group that nearly cancels
    got = ref + 1e-4 * rng.standard_normal(ref.shape)
    assert rel_l2_groups(got, ref, 2) <= 1e-3
    # a wrong small group still reads as wrong against the typical group norm
    got[3, 1] = 1.0
    assert rel_l2_groups(got, ref, 2) > 0.1
    # all-zero reference: only an all-zero result passes
    z = np.zeros((2, 3))
    assert rel_l2_groups(z, z, 1) == 0.0
    assert rel_l2_groups(z + 1e-9, z, 1) == float("inf")
