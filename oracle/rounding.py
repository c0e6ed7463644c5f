"""Rounding to the storage formats the method uses (test infrastructure only).

The stored summary is bfloat16 (round-to-nearest-even from the float64 value)
and the packed tiers keep a float16 scale and zero per 32-element group.  Both
are written here from the IEEE 754 definition of round-to-nearest-even: a value
x = m * 2**e with 0.5 <= |m| < 1 has quantum 2**(e - p) for a format with p
significant bits, never below the format's subnormal spacing.

Pinned in tests/test_oracle_rounding.py against numpy's own float16 cast (an
independent IEEE implementation) and against hand-checked boundary values.
"""

import numpy as np

# (significant bits, log2 of the subnormal spacing, largest finite value)
_BF16 = (8, -133, float.fromhex("0x1.fep127"))
_FP16 = (11, -24, 65504.0)


def _round_to_format(x, sig_bits, min_exp2, max_finite):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(x)
        quantum_exp = np.maximum(e.astype(np.int64) - sig_bits, min_exp2)
        y = np.ldexp(np.rint(np.ldexp(x, -quantum_exp)), quantum_exp)
    return y, max_finite


def round_bf16(x):
    """Nearest bfloat16 value (ties to even) of a float64 array, as float64.

    Overflow rounds to +-inf, as IEEE round-to-nearest does.
    """
    y, mx = _round_to_format(x, *_BF16)
    with np.errstate(invalid="ignore"):
        y = np.where(np.isfinite(y) & (np.abs(y) > mx), np.sign(y) * np.inf, y)
    return y


def round_fp16_sat(x):
    """Nearest float16 value (ties to even), saturating at +-65504, as float64.

    The packed-tier scale and zero saturate instead of overflowing: a group
    whose range exceeds float16 keeps the largest finite scale.
    """
    y, mx = _round_to_format(x, *_FP16)
    return np.clip(y, -mx, mx)


def as_float32(x):
    """float64 -> float32 with IEEE round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
