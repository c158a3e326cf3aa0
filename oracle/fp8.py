"""OCP fp8 e4m3fn decode, written from the format's bit definition.

The KvQuantSparseAttnSharedkv page stores KV as FLOAT8_E4M3FN; the same
8-bit layout is used here for q, ori_kv and cmp_kv:

  bit 7      sign
  bits 6..3  exponent, bias 7
  bits 2..0  mantissa
  exponent 0: subnormal, value = mantissa/8 * 2^-6
  exponent 15 with mantissa 7: NaN (there are no infinities; max finite 448)

Test infrastructure only (see the package docstring).
Pinned by tests/test_oracle_fp8.py against torch.float8_e4m3fn decoding.
"""
import numpy as np


def _decode_one(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_LUT = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes (any shape) -> float64 values."""
    return E4M3_LUT[np.asarray(codes, dtype=np.uint8)]
