"""Element decoding for the oracle: bf16 bit patterns, FP8 E4M3FN codes and NVFP4 blocks to
float64.

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

NVFP4 ([VO-split], sections "Summary" and "NVFP4 split-KV correctness (added)", and its
commit on the split-KV gate): K and V are stored as packed uint8, two E2M1 values per byte,
with one FP8 block scale per 16 consecutive head_dim elements of one token, kept in a
separate scale-factor tensor laid out like the data ("[all-data | all-SF]", with no
per-page swizzle).  Readings taken where the pages are silent:
  * E2M1 is the OCP 4-bit float: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit,
    no infinities or NaN (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
  * Element 2i of a row is the low nibble of byte i, element 2i + 1 the high nibble.
  * The block scale is an E4M3FN code; the tensor-wide fp32 scale (k_scale / v_scale)
    multiplies on top, so value = e2m1(nibble) * e4m3fn(block scale) * tensor scale.
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


def e2m1_value(code: int) -> float:
    """Closed-form value of one E2M1 code (0..15): sign, exponent (bias 1), mantissa."""
    code = int(code)
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:  # subnormal: 2^(1-1) * m/2
        return sign * (m / 2.0)
    return sign * math.ldexp(1.0 + m / 2.0, e - 1)


# All 16 codes, built from the closed form above.
E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)

NVFP4_BLOCK = 16  # head_dim elements per block scale


def nvfp4_values(packed: np.ndarray, block_scales: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Dequantised float64 values of NVFP4 rows.

    packed ``[..., D/2]`` uint8 (element 2i = low nibble of byte i, 2i + 1 = high nibble),
    block_scales ``[..., D/16]`` uint8 E4M3FN codes -> ``[..., D]`` float64, with
    value = e2m1(nibble) * e4m3fn(block scale of element // 16) * scale.
    """
    packed = np.asarray(packed).astype(np.uint8)
    block_scales = np.asarray(block_scales).astype(np.uint8)
    d = 2 * packed.shape[-1]
    if block_scales.shape[-1] * NVFP4_BLOCK != d:
        raise ValueError(f"{block_scales.shape[-1]} block scales do not cover {d} elements")
    codes = np.empty(packed.shape[:-1] + (d,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0x0F
    codes[..., 1::2] = packed >> 4
    per_elem = np.repeat(E4M3FN_VALUES[block_scales], NVFP4_BLOCK, axis=-1)
    return E2M1_VALUES[codes] * per_elem * float(scale)


def kv_values(raw: np.ndarray, kv_dtype: str, scale: float = 1.0, block_scales=None) -> np.ndarray:
    """Dequantised float64 values of stored KV elements.

    kv_dtype "bf16":  raw holds bf16 bit patterns; the scale must be 1.
    kv_dtype "fp8":   raw holds E4M3FN codes (uint8); value = e4m3fn(code) * scale.
    kv_dtype "nvfp4": raw holds packed E2M1 pairs and block_scales the E4M3FN block scales
                      (see nvfp4_values).
    """
    if kv_dtype != "nvfp4" and block_scales is not None:
        raise ValueError(f"{kv_dtype} KV takes no block scales")
    if kv_dtype == "nvfp4":
        if block_scales is None:
            raise ValueError("nvfp4 KV needs its block scales")
        return nvfp4_values(raw, block_scales, scale)
    if kv_dtype == "bf16":
        if scale != 1.0:
            raise ValueError("bf16 KV takes no scale")
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        return E4M3FN_VALUES[np.asarray(raw).astype(np.uint8)] * float(scale)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")
