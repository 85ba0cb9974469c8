"""OCP FP8 E4M3 ("e4m3fn") code -> value, in fp64.  Test infrastructure only.

The pages only say that the KV cache can be stored in FP8, halving its
memory ("TensorRT-LLM, in depth", aicassindra.com, section "Quantization:
fewer bytes per weight and per cached token"; the course glossary "Key terms
in this lesson" defines FP8 as an 8-bit floating-point format).  The exact
format is the OCP 8-bit floating point E4M3 encoding:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0: subnormal, value = (-1)^s * (m / 8) * 2^(1 - 7);
* exponent field 1..15: normal, value = (-1)^s * (1 + m / 8) * 2^(e - 7);
* no infinities; S.1111.111 (0x7F, 0xFF) is NaN, so the largest finite
  magnitude is S.1111.110 = 1.75 * 2^8 = 448.

Each entry is built from the fields above; nothing is read from a library.
"""
from __future__ import annotations

import functools

import numpy as np


def _code_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


@functools.lru_cache(maxsize=1)
def e4m3_decode_table() -> np.ndarray:
    """float64[256]: value of every E4M3 code."""
    t = np.array([_code_value(c) for c in range(256)], dtype=np.float64)
    t.setflags(write=False)
    return t


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (same shape)."""
    return e4m3_decode_table()[np.asarray(codes, dtype=np.uint8)]
