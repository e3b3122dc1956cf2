"""The parity gate's absolute bound for stress inputs (no GPU needed)."""

from tests.parity import ABS_TOL, assert_gate, bf16_abs_tol


def test_stress_bound_is_one_bf16_ulp_from_four_on():
    assert bf16_abs_tol(0.0) == ABS_TOL
    assert bf16_abs_tol(1.999) == ABS_TOL
    assert bf16_abs_tol(3.999) == ABS_TOL     # half a bf16 ulp (2^-7) fits in 1e-2
    assert bf16_abs_tol(4.0) == 2.0 ** -5      # bf16 ulp on [4, 8)
    assert bf16_abs_tol(7.99) == 2.0 ** -5
    assert bf16_abs_tol(300.0) == 2.0 ** 1


def test_gate_applies_each_bound():
    ok = dict(max_abs=0.009, row_rel=0.007, dead_rows_nonzero=0, lse_abs=9e-4, lse_nan=0,
              lse_inf_mismatch=0)
    assert_gate(ok)
    for key, bad in (("max_abs", 0.011), ("row_rel", 0.008), ("dead_rows_nonzero", 1),
                     ("lse_abs", 1.1e-3), ("lse_nan", 1), ("lse_inf_mismatch", 1)):
        try:
            assert_gate({**ok, key: bad})
        except AssertionError:
            continue
        raise AssertionError(f"{key}={bad} passed the gate")
    assert_gate({**ok, "max_abs": 0.03}, abs_tol=bf16_abs_tol(5.0))
