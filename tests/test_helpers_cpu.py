"""The small-unit output rule of the GPU comparisons (helpers.output_unit_ok),
checked on constructed units: valid roundings pass, real errors fail."""
import numpy as np
import torch

from tests.helpers import REL_L2_TOL, bf16_ulp, output_unit_ok


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _from_bits(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _unit(n=160, seed=3):
    r = np.random.default_rng(seed)
    return r.standard_normal(n) * 0.5


def test_identical_roundings_pass_the_stated_rule():
    ex = _unit()
    ok, stated, excess = output_unit_ok(_bf16_bits(ex), _bf16_bits(ex), ex)
    assert ok and stated == 0.0


def test_one_flip_at_a_midpoint_passes_as_valid_roundings():
    ex = _unit()
    i = int(np.argmax(np.abs(ex)))
    ex[i] = 2.7890625 + 8e-6          # just above a bf16 rounding midpoint
    want = _bf16_bits(ex)              # rounds up
    got = want.copy()
    got[i] = _bf16_bits(2.78125)       # the neighbouring bf16 value below
    ok, stated, excess = output_unit_ok(got, want, ex)
    assert stated > REL_L2_TOL and excess < 1e-4 and ok


def test_near_zero_output_with_unit_scale_error_passes():
    ex = _unit()
    i = int(np.argmax(np.abs(ex)))
    ex[i] = 2.7890625 + 8e-6
    ex[7] = 1.5e-4                     # far below the unit's RMS
    want = _bf16_bits(ex)
    got = want.copy()
    got[i] = _bf16_bits(2.78125)
    got[7] = _bf16_bits(1.5e-4 + 1.5e-6)   # 3e-6 of the RMS off: more than its own spacing
    assert abs(_from_bits(got[7]) - ex[7]) > bf16_ulp(ex[7])
    assert output_unit_ok(got, want, ex)[0]


def test_real_errors_fail():
    ex = _unit()
    i = int(np.argmax(np.abs(ex)))
    ex[i] = 2.7890625 + 8e-6
    want = _bf16_bits(ex)
    # every output 0.5% too large (a wrong scale): beyond the valid roundings
    assert not output_unit_ok(_bf16_bits(ex * 1.005), want, ex)[0]
    # one output four spacings off
    got = want.copy()
    got[3] = _bf16_bits(ex[3] + 4 * bf16_ulp(ex[3]))
    got[i] = _bf16_bits(2.78125)
    assert not output_unit_ok(got, want, ex)[0]
    # a near-zero output off by 2e-3 of the RMS: small next to the unit (its excess
    # passes), but many spacings of the floor at 1/16 of the RMS
    got = want.copy()
    got[i] = _bf16_bits(2.78125)
    ex[11] = 1e-4
    want[11] = _bf16_bits(ex[11])
    got[11] = _bf16_bits(ex[11] + 2e-3 * np.sqrt(np.mean(ex * ex)))
    ok, stated, excess = output_unit_ok(got, want, ex)
    assert excess < REL_L2_TOL and not ok
