"""Decoders of the bf16 and packed-640 KV formats, written from the formats'
bit definitions (test infrastructure only; see the package docstring).

bf16 (q of the KvQuantSparseAttnSharedkv page; q and KV of the
SparseCompressedFlashAttention page): the upper 16 bits of an IEEE binary32
value: bit 15 sign, bits 14..7 exponent with bias 127, bits 6..0 mantissa;
exponent 0 is subnormal (mantissa / 128 * 2^-126), exponent 255 is inf
(mantissa 0) or NaN.

e8m0 (the nope_quant_scale bytes of the KvQuantSparseAttnSharedkv row, type
float8_e8m0fnu): an unsigned power of two, value 2^(E - 127) for E in
0..254; E = 255 is NaN.  No sign, no zero, no infinity.

Packed KV row (KvQuantSparseAttnSharedkv, 约束说明: D of ori_kv / cmp_kv is
640): bytes [0, 128) are the rope part, 64 bf16 values (little-endian);
bytes [128, 576) the nope part, 448 fp8 e4m3 codes; bytes [576, 583) seven
e8m0 scales, one per 64-wide nope tile (tile_size 64, 参数说明); bytes
[583, 640) pad.  The row's logical 512-wide vector is rope then nope, nope
column 64 j + i of tile j being code * 2^(E_j - 127).
"""
import numpy as np

from .fp8 import decode_e4m3

ROPE_DIM = 64
NOPE_DIM = 448
TILE = 64
PACKED_ROW_BYTES = 640


def _decode_bf16_one(bits: int) -> float:
    sign = -1.0 if (bits >> 15) & 1 else 1.0
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        return float("nan") if man else sign * float("inf")
    if exp == 0:
        return sign * (man / 128.0) * 2.0 ** (-126)
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


BF16_LUT = np.array([_decode_bf16_one(b) for b in range(1 << 16)], dtype=np.float64)


def decode_bf16(bits) -> np.ndarray:
    """uint16 bit patterns (any shape) -> float64 values."""
    return BF16_LUT[np.asarray(bits, dtype=np.uint16)]


def decode_e8m0(codes) -> np.ndarray:
    """uint8 e8m0 codes (any shape) -> float64 powers of two (NaN for 255)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


def decode_packed640(rows) -> np.ndarray:
    """uint8 rows [n, 640] -> float64 [n, 512] (rope, then scaled nope)."""
    rows = np.asarray(rows, dtype=np.uint8)
    assert rows.shape[-1] == PACKED_ROW_BYTES
    rope_bits = rows[..., 0:2 * ROPE_DIM:2].astype(np.uint16) | (rows[..., 1:2 * ROPE_DIM:2].astype(np.uint16) << 8)
    rope = decode_bf16(rope_bits)
    nope = decode_e4m3(rows[..., 2 * ROPE_DIM:2 * ROPE_DIM + NOPE_DIM])
    scale = decode_e8m0(rows[..., 2 * ROPE_DIM + NOPE_DIM:2 * ROPE_DIM + NOPE_DIM + NOPE_DIM // TILE])
    nope = nope * np.repeat(scale, TILE, axis=-1)
    return np.concatenate([rope, nope], axis=-1)
