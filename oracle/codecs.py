"""Number-format codecs of the CPU oracle (test infrastructure only).

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module. It shares no code with the HIP path.

The FP8 format is the one the "GPT-OSS on day 0" post serves the experts in
(section "GPT-OSS on Hopper": FP8 with 128x128 block scaling).  Its element
type is OCP E4M3 ("fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, no infinities, NaN = S.1111.111, largest finite 448, smallest
subnormal 2^-9.  The MXFP8 variant (the "Hosting Qwen on Blackwell"
post, section "Quantization": microscaling on Blackwell) adds the OCP E8M0 scale: 8 exponent bits with bias
127, no sign and no mantissa, code 0xFF = NaN.  The FP4 weights (the post's
section "GPT-OSS on Hopper": the checkpoints ship in MXFP4) use the OCP E2M1
element: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no
infinities or NaN, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Everything here is
written from those definitions.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6          # subnormal
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)    # normal


#: value of every e4m3 code, fp64 (exact)
E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)

# the 127 non-negative finite codes 0x00..0x7E have increasing values
_POS_VALUES = E4M3_TABLE[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(v: np.ndarray) -> np.ndarray:
    """Values (fp32 or fp64) -> nearest e4m3 code, ties to even mantissa.

    Magnitudes above 448 saturate to 448; NaN maps to 0x7F. The sign of
    zero is kept (a negative value that rounds to zero gives 0x80).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(a)                          # a = m * 2^ex, m in [0.5, 1)
        e_unb = np.maximum(ex - 1, -6)               # binade; subnormals share 2^-6
        quantum = np.ldexp(1.0, e_unb - 3)           # spacing of codes in that binade
        n = np.rint(a / quantum)                     # exact quotient, half-to-even
        r = np.minimum(n * quantum, E4M3_MAX)
    r = np.where(a == 0, 0.0, r)
    idx = np.searchsorted(_POS_VALUES, r)            # r is exactly a table value
    codes = idx.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), codes).astype(np.uint8)


E8M0_BIAS = 127


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes (uint8) -> fp64 powers of two 2^(c - 127); 0xFF -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, c - E8M0_BIAS)
    return np.where(c == 0xFF, np.nan, v)


def _e2m1_value(code: int) -> float:
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * (m / 2.0)                      # subnormal: 0 or 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


#: value of every e2m1 code 0..15, fp64 (exact)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_E2M1_POS = E2M1_TABLE[:8]                           # 0, 0.5, 1, 1.5, 2, 3, 4, 6
assert np.all(np.diff(_E2M1_POS) > 0)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15, any integer dtype) -> fp64 values."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode_rne(v: np.ndarray) -> np.ndarray:
    """Values -> nearest e2m1 code, ties to the even mantissa; magnitudes above 6
    saturate to 6; the sign of zero is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 6.0)
    # nearest of the 8 magnitudes; on a tie the lower index wins only if its code is even
    d = np.abs(a[..., None] - _E2M1_POS)
    best = d.argmin(axis=-1)
    dmin = d.min(axis=-1)
    nxt = np.minimum(best + 1, 7)
    tie = np.take_along_axis(d, nxt[..., None], axis=-1)[..., 0] == dmin
    best = np.where(tie & (nxt != best) & (best % 2 == 1), nxt, best)
    return (best.astype(np.uint8) | np.where(np.signbit(v), 0x8, 0).astype(np.uint8)).astype(np.uint8)


def unpack_fp4_k(packed: np.ndarray) -> np.ndarray:
    """[K/2, N] bytes, two 4-bit codes per byte along K (low nibble = even K)
    -> [K, N] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((2 * p.shape[0],) + p.shape[1:], dtype=np.uint8)
    out[0::2] = p & 0xF
    out[1::2] = p >> 4
    return out


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """fp64 values -> nearest bf16 value (as fp64), ties to even.

    Written directly on the binary64 representation: keep 8 significant bits.
    Reports the rounding floor of bf16 outputs and rounds the optional bf16
    gate weights.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(np.abs(v))
        e_unb = np.maximum(ex - 1, -126)             # bf16 subnormals below 2^-126
        quantum = np.ldexp(1.0, e_unb - 7)
        r = np.rint(v / quantum) * quantum
    return np.where(v == 0, v, r)
