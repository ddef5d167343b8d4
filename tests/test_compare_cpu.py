"""The GPU tests' comparison (tests.gpu_util.compare) on the CPU: an error confined to one tile
of keys, small enough to pass the pooled NMSE bar, must fail the per-row bound."""
import numpy as np
import pytest

from oracle import fa_back_oracle as O
from tests import gpu_util as U


def _noisy(ref, rel, rng):
    return ref + rel * rng.standard_normal(ref.shape) * np.sqrt(np.mean(ref ** 2))


def test_tile_error_hides_in_nmse_but_not_per_key():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((4, 20000, 16))
    got = _noisy(ref, 3e-4, rng)
    got[2, 5000:5128] *= 1.05                        # one 128-key tile 5% off
    assert O.nmse(got, ref) <= U.TOL                  # the pooled bar does not see it
    assert U.local_error(got, ref, vector=True) > 1.0
    assert U.local_error(_noisy(ref, 3e-4, rng), ref, vector=True) <= 1.0


def test_scalar_entry_error():
    rng = np.random.default_rng(8)
    ref = rng.standard_normal(50000)
    got = _noisy(ref, 1e-4, rng)
    assert U.local_error(got, ref, vector=False) <= 1.0
    i = int(np.argmax(np.abs(ref)))
    got[i] *= 1.1                                      # one row's delta 10% off
    assert O.nmse(got, ref) <= U.TOL
    assert U.local_error(got, ref, vector=False) > 1.0


def test_compare_raises_on_local_error():
    rng = np.random.default_rng(9)
    ref = {k: rng.standard_normal((3, 4000, 8)) for k in ("dq", "dk", "dv")}
    ref.update({k: rng.standard_normal((3, 4000)) for k in ("lse", "delta")})
    got = {k: v.copy() for k, v in ref.items()}
    U.compare(got, ref)
    got["dv"][1, 100] *= 1.2
    with pytest.raises(AssertionError, match="per-row"):
        U.compare(got, ref)


def test_zero_reference_rows_need_exact_zeros():
    ref = np.zeros((2, 5, 4))
    assert U.local_error(ref.copy(), ref, vector=True) == 0.0
    got = ref.copy()
    got[0, 1, 2] = 1e-30
    assert U.local_error(got, ref, vector=True) == float("inf")
