"""Element decoding for the oracle: bf16 bit patterns and FP8 E4M3FN codes to float64.

Test infrastructure only (see the package docstring).

[Triton-hd512], section "Approach": an FP8 KV cache keeps working because the kernels cast
on load, so the cache is dequantised in-kernel.  The oracle therefore reads the stored
bytes and dequantises them itself: value = e4m3fn(byte) * scale.  [VO-split], commit
"test asymmetric NVFP4 prefill ...", states the same rule for its own check: the reference
consumes the exact quantised bytes the kernel reads (a dequantisation oracle, not a
requantised approximation).

The format is OCP E4M3FN (the pages say only "FP8"; the workload calls it e4m3): 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, and NaN only at
S.1111.111.  bf16 is the upper half of an IEEE-754 binary32.
"""

import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16 / int16 array) as float64.

    A bf16 value is the binary32 whose upper 16 bits are the pattern and whose lower
    16 bits are zero.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Closed-form value of one E4M3FN code (0..255)."""
    code = int(code)
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:  # subnormal: 2^(1-7) * m/8
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


# All 256 codes, built from the closed form above.
E4M3FN_VALUES = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def kv_values(raw: np.ndarray, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """Dequantised float64 values of stored KV elements.

    kv_dtype "bf16": raw holds bf16 bit patterns; the scale must be 1.
    kv_dtype "fp8":  raw holds E4M3FN codes (uint8); value = e4m3fn(code) * scale.
    """
    if kv_dtype == "bf16":
        if scale != 1.0:
            raise ValueError("bf16 KV takes no scale")
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        return E4M3FN_VALUES[np.asarray(raw).astype(np.uint8)] * float(scale)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")
