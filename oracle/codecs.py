"""Number formats of the oracle: bf16 and OCP FP8 E4M3FN, plus per-row FP8 activation scaling.

Test infrastructure only (see the package docstring).

bf16: 1 sign, 8 exponent, 7 stored mantissa bits (8 significant); the kernels' rounding points
([S] §BF16 MoE Kernel Optimization) round to nearest, ties to even.
E4M3FN (OCP 8-bit floating point spec, "FN" = finite, NaN only): exponent bias 7, 3 mantissa bits,
largest finite 448 = 1.75 * 2^8, smallest normal 2^-6, subnormals m * 2^-9; no infinities.
Dynamic FP8 ([S] §Highlights, §BF16, NVFP4 and FP8 Model Support; [H] §专家混合): per-row scale
amax / 448, codes = e4m3(x * (448 / amax)), rounded to nearest-even and saturated to +-448.
"""
from __future__ import annotations

import numpy as np

_F64_DROP = 52 - 7            # float64 stored mantissa bits minus bf16 stored mantissa bits
_HALF = np.uint64(1 << (_F64_DROP - 1))
_LOW_MASK = np.uint64((1 << _F64_DROP) - 1)
_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(v) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each element of `v`, returned as float64.

    Works on the float64 bit pattern: keep 8 significant bits, round the 45 dropped bits to
    nearest-even. Defined here for zero and for normal magnitudes of the bf16 range, which is all
    the block produces; anything else (NaN, inf, overflow, bf16-subnormal) raises.
    """
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    mag = np.abs(a)
    bad = ~np.isfinite(a) | ((mag != 0) & (mag < _BF16_MIN_NORMAL)) | (mag > _BF16_MAX)
    if np.any(bad):
        raise ValueError("bf16_round: value outside the normal bf16 range")
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(_F64_DROP)) & np.uint64(1)
    r = (bits + (_HALF - np.uint64(1) + lsb)) & ~_LOW_MASK
    out = r.view(np.float64)
    if np.any(np.abs(out) > _BF16_MAX):
        raise ValueError("bf16_round: rounded past the largest bf16")
    return out


def bf16_bits_to_f64(u16) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to float64 (exact)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3FN code (uint8) as float64; 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(v) -> np.ndarray:
    """E4M3FN code (uint8) of each value: round to nearest, ties to even, saturate to +-448.

    The sign bit follows the sign of the input, so -0 and negative values that round to zero get
    code 0x80. NaN inputs raise.
    """
    a = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(a)):
        raise ValueError("e4m3_encode: NaN input")
    sign = np.signbit(a).astype(np.int64)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    # binade of each magnitude; below 2^-6 the grid is the subnormal spacing 2^-9
    _, ex = np.frexp(np.where(mag > 0, mag, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    quantum = np.exp2((e - 3).astype(np.float64))
    steps = np.rint(mag / quantum)                 # np.rint rounds half to even; division is exact
    q = steps * quantum                            # exact; may carry into the next binade
    q = np.minimum(q, E4M3_MAX)                    # 448 < v < 464 rounds down; >= 464 saturates
    _, qex = np.frexp(np.where(q > 0, q, 1.0))
    qe = qex.astype(np.int64) - 1
    normal = q >= 2.0 ** -6
    exp_field = np.where(normal, qe + 7, 0)
    mant = np.where(normal, np.rint(q / np.exp2(qe.astype(np.float64)) * 8.0) - 8.0,
                    np.rint(q / 2.0 ** -9)).astype(np.int64)
    code = (sign << 7) | (exp_field << 3) | mant
    return code.astype(np.uint8)


def quant_rows_fp8(rows) -> tuple:
    """Dynamic per-row FP8 scaling in fp32 arithmetic, as the quantising kernel computes it.

    For each row r (values exactly representable in fp32 — bf16 x or bf16 h):
      amax = max |r|;  scale = fp32(amax / 448);  inv = fp32(448 / amax);
      code = e4m3(fp32(r * inv)).
    amax = 0 gives scale 1 and all-zero codes. Returns (codes uint8 [n][m], scale fp32 [n]).
    The scale step decides integer codes, so it is taken in fp32, the precision the GPU uses.
    """
    r = np.asarray(rows, dtype=np.float32)
    if r.ndim == 1:
        r = r[None, :]
    amax = np.max(np.abs(r), axis=1).astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(448.0)).astype(np.float32)
    inv = (np.float32(448.0) / safe).astype(np.float32)
    t = (r * inv[:, None]).astype(np.float32)
    codes = e4m3_encode(t)
    codes[zero, :] = 0
    return codes, scale
