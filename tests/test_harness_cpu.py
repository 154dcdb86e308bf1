"""The parity helpers themselves (CPU): the per-row bound sees a localised error that the
whole-tensor relative Frobenius norm lets through."""
import numpy as np

from harness import ROW_TOL, TOL, rel_fro, rel_fro_rows


def test_row_bound_catches_one_wrong_block():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((2048, 4096))
    got = ref * (1 + 1e-4 * rng.standard_normal(ref.shape))  # storage-rounding-sized noise
    assert rel_fro(got, ref) <= TOL["bf16"] and rel_fro_rows(got, ref) <= ROW_TOL["bf16"]
    got[100:108, 512:528] = 0.0                               # one wrong 8 x 16 block
    assert rel_fro(got, ref) <= TOL["bf16"]                   # the whole-tensor norm misses it
    assert rel_fro_rows(got, ref) > ROW_TOL["bf16"]           # the row bound does not


def test_row_bound_zero_rows_must_stay_zero():
    ref = np.zeros((4, 8))
    ref[1] = 1.0
    assert rel_fro_rows(ref.copy(), ref) == 0.0
    got = ref.copy()
    got[2, 3] = 1e-30
    assert rel_fro_rows(got, ref) == float("inf")
