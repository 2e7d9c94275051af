"""The GPU parity comparator for 16-bit error buffers, checked on the CPU.

Where a chunk's scale matched, the stored bf16 / fp16 error words must be unique: nearest-even
storage (the error format reading of the gradient-compression survey, bmjup.com, Q&A Q3, on keeping
the error term in FP16) or the stochastic rule with the same random bits.  These tests feed
tests/_parity.assert_err_close stores made here with numpy under other rounding rules -- truncation,
ties away from zero, ties toward zero, a rounding point just below the midpoint, a stochastic store
drawn from another stream -- and require it to reject every one of them, while it accepts the
nearest-even store and allows one unit of the format only on chunks whose scale differed.
"""
import numpy as np
import pytest

import oracle
import _parity as P

_PREC = {"bf16": 8, "f16": 11}


def _values(fmt, n=1 << 18, seed=3):
    """fp32 errors over many binades (fp16: the subnormal range too), with exact midpoints between
    two neighbouring format values (both parities of the lower neighbour) and their fp32 neighbours."""
    rng = np.random.default_rng([seed, _PREC[fmt]])
    lo_e, hi_e = (-30, 30) if fmt == "bf16" else (-26, 15)
    x = (rng.standard_normal(n) * 2.0 ** rng.integers(lo_e, hi_e, n)).astype(np.float32)
    # exact midpoints: a format value plus half its quantum
    base = oracle.to_format(x[: n // 4], fmt)
    base32 = P.widen_err(base).astype(np.float64)
    ex = np.floor(np.log2(np.maximum(np.abs(base32), 2.0 ** -24)))
    if fmt == "f16":
        ex = np.maximum(ex, -14.0)
    q = 2.0 ** (ex - (_PREC[fmt] - 1))
    mid = (base32 + np.sign(base32) * q / 2).astype(np.float32)
    finite = np.isfinite(mid) & (np.abs(mid.astype(np.float64)) < (65504.0 if fmt == "f16" else 3e38))
    mid = mid[finite & (base32 != 0)]
    near = np.concatenate([np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))])
    return np.concatenate([x, mid, near]).astype(np.float32)


def _from_f64(r, fmt):
    """Bits of exact format values given in double (truncation / ties-away results below)."""
    return oracle.to_format(r.astype(np.float32), fmt)


def _neighbours(x, fmt):
    """(lo, hi, q): the format values toward and away from zero around |x|, and the quantum."""
    a = np.abs(x.astype(np.float64))
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -149)))
    emin = -126 if fmt == "bf16" else -14
    q = 2.0 ** (np.maximum(ex, emin) - (_PREC[fmt] - 1))
    lo = np.floor(a / q) * q
    return lo, lo + q, q


def _round_with(x, fmt, rule):
    """Stores of x under another rounding rule, as bits of the format (numpy arithmetic in double)."""
    lo, hi, q = _neighbours(x, fmt)
    a = np.abs(x.astype(np.float64))
    frac = a - lo
    if rule == "truncate":
        r = lo
    elif rule == "ties_away":
        r = np.where(frac >= q / 2, hi, lo)
    elif rule == "ties_toward_zero":
        r = np.where(frac > q / 2, hi, lo)
    elif rule == "below_midpoint":
        # rounds up from 1.5 fp32 ulps under the midpoint, so values one fp32 ulp below it go up
        ulp32 = 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 23)
        r = np.where(frac >= q / 2 - 1.5 * ulp32, hi, lo)
    else:
        raise ValueError(rule)
    r = np.copysign(r, x.astype(np.float64))
    top = 65504.0 if fmt == "f16" else (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > top, np.copysign(np.inf, r), r)
    return _from_f64(r, fmt)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_nearest_even_store_passes(fmt):
    x = _values(fmt)
    ref = oracle.to_format(x, fmt)
    P.assert_err_close(ref.copy(), ref, fmt)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("rule", ["truncate", "ties_away", "ties_toward_zero", "below_midpoint"])
def test_other_rounding_rules_are_rejected(fmt, rule):
    x = _values(fmt)
    ref = oracle.to_format(x, fmt)
    bad = _round_with(x, fmt, rule)
    differ = np.count_nonzero(bad.view(np.uint16) != ref.view(np.uint16))
    assert differ > 0, f"the {rule} store must differ from nearest-even somewhere on this fixture"
    with pytest.raises(AssertionError, match="differ where the scale matched"):
        P.assert_err_close(bad, ref, f"{fmt} {rule}")
    # a chunk whose scale differed allows one unit of the format: the same store passes there
    P.assert_err_close(bad, ref, f"{fmt} {rule}, scale differed", exact=False)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_stochastic_store_from_another_stream_is_rejected(fmt):
    x = _values(fmt, n=1 << 16)
    ref = oracle.to_format_sr(x, fmt, seed=11, step=4, index0=0)
    P.assert_err_close(ref.copy(), ref, fmt)
    for other in (dict(seed=11, step=5, index0=0), dict(seed=12, step=4, index0=0),
                  dict(seed=11, step=4, index0=4)):
        bad = oracle.to_format_sr(x, fmt, **other)
        with pytest.raises(AssertionError, match="differ where the scale matched"):
            P.assert_err_close(bad, ref, f"{fmt} sr {other}")


def test_exact_mask_is_per_element():
    """Only elements outside the mask get the one-unit allowance."""
    x = _values("bf16", n=1 << 12)
    ref = oracle.to_format(x, "bf16")
    bad = _round_with(x, "bf16", "truncate")
    d = bad.view(np.uint16) != ref.view(np.uint16)
    P.assert_err_close(bad, ref, "mask covers every difference", exact=~d)
    k = int(np.argmax(d))
    mask = ~d
    mask[k] = True
    with pytest.raises(AssertionError):
        P.assert_err_close(bad, ref, "one difference inside the mask", exact=mask)


def test_nan_payloads_are_not_compared_but_nan_must_meet_nan():
    ref = np.array([0x7FC0, 0x3F80, 0xFFC0], np.uint16)            # bf16 NaN, 1.0, -NaN
    P.assert_err_close(np.array([0x7FC1, 0x3F80, 0x7FC0], np.uint16), ref, "payloads")
    with pytest.raises(AssertionError):
        P.assert_err_close(np.array([0x7F80, 0x3F80, 0xFFC0], np.uint16), ref, "Inf for NaN")
