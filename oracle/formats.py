"""Storage-format decoders for the oracle (test infrastructure only).

The pages never state the KV-cache element type.  The library stores K/V as
float32, bfloat16 or OCP FP8 E4M3 ("e4m3fn") with one float32 scale per KV head;
these decoders turn stored codes into exact float64 values.

* bfloat16 is, by definition, the upper 16 bits of an IEEE-754 binary32 word:
  decoding is a 16-bit left shift and a reinterpretation (exact).
* OCP E4M3 (OCP 8-bit Floating Point Specification, E4M3 encoding): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  subnormals m/8 * 2**(1-7); there are no infinities; S.1111.111 is NaN, so the
  largest finite magnitude is S.1111.110 = 1.75 * 2**8 = 448.

Pinned in tests/test_formats.py against torch's float8_e4m3fn / bfloat16 ->
float64 conversions for every code, and against the specification's named
points in tests/golden/e4m3_spec_points.txt.
"""
import numpy as np


def _e4m3_code_value(code):
    """Value of one E4M3 byte, written out from the format definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return float("nan")
    if exponent == 0:
        return sign * (mantissa / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


def e4m3_value_table():
    """float64[256]: value of every E4M3 code (NaN for the two NaN codes)."""
    return np.array([_e4m3_code_value(c) for c in range(256)], dtype=np.float64)


_E4M3 = e4m3_value_table()


def decode_e4m3(codes):
    """uint8 array of E4M3 codes -> float64 array of the same shape."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return _E4M3[codes]


def decode_bf16(bits):
    """uint16 array of bfloat16 bit patterns -> float64 array (exact)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bfloat16 bit patterns must be uint16")
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode(arr, fmt, scale=None):
    """Stored K/V (or Q) values -> float64.

    fmt: "float" (any numpy float array, taken at its stored value),
         "bf16"  (uint16 bit patterns),
         "e4m3"  (uint8 codes; multiplied by ``scale`` when one is given).
    """
    if fmt == "float":
        out = np.asarray(arr, dtype=np.float64)
    elif fmt == "bf16":
        out = decode_bf16(arr)
    elif fmt == "e4m3":
        out = decode_e4m3(arr)
    else:
        raise ValueError(f"unknown storage format {fmt!r}")
    if scale is not None:
        out = out * np.float64(scale)
    return out
