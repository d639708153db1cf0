"""Bit-level decoders and the fp8 encoder of the oracle (test infrastructure only).

The pages store K/V in the activation dtype (fp16 / bf16) and name KV-cache
quantization as a throughput lever ("vLLM 推理全流程深度解析", the PagedAttention
remark on KV cache int8).  The fp8 cache format used here is the OCP
``e4m3fn`` format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals at exponent field 0, no infinities, and only ``S.1111.111`` as NaN,
so the largest finite magnitude is 1.75 * 2**8 = 448.

Reading taken where the pages are silent: one float32 scale per tensor
(K and V separately); a stored code means ``code_value * scale``; encoding is
``round_to_nearest_even(saturate(float32(x) * float32(1/scale)))`` with the
single multiply done in IEEE float32, saturation to +-448 for every finite or
infinite overflow, and NaN kept as NaN.

The int8 cache (the pages' own example of KV-cache quantization) is read the
same way: symmetric signed codes -127..127 (two's complement bytes; -128 is
never produced), one float32 scale per tensor, a code means ``code * scale``,
encoding ``round_to_nearest_even(saturate(float32(x) * float32(1/scale)))``
with saturation to +-127; int8 has no NaN, and a NaN input becomes 0.

Both quantized formats also take the per-K/V-head option the int8 row of the
build names (the same reading applied per head): one float32 scale per K/V
head of a tensor, so a code of head ``h`` means ``code * scale[h]`` and is
encoded with ``float32(1/scale[h])``.  The encoders below multiply by
whatever inverse scale they are given, a number or an array that broadcasts
against the values (``[Hkv, 1]`` against ``[..., Hkv, D]``).
"""

import numpy as np

E4M3_MAX = 448.0


def f16_bits_to_f64(bits):
    """IEEE binary16 bit patterns (uint16) -> float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64.

    A bfloat16 is the upper half of an IEEE binary32, so widening the bits by a
    16-bit left shift gives the binary32 with the same value, exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_value(code):
    """Value of one e4m3fn code (0..255), straight from the bit definition."""
    code = int(code)
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)       # subnormal
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)   # normal


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_to_f64(codes):
    """uint8 e4m3fn codes -> float64 values (table lookup)."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


# Non-negative finite codes 0x00..0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def e4m3fn_encode(x_f32, inv_scale_f32):
    """Encode float32 values as e4m3fn codes with the tensor's (or each head's) scale.

    ``y = float32(x * inv_scale)`` (one IEEE float32 multiply), then ``y`` is
    clamped to [-448, 448] (saturation; 448 is representable, so clamping first
    and rounding second equals rounding first and saturating second), then the
    nearest representable e4m3fn magnitude is chosen, with a tie going to the
    code whose mantissa is even.  The sign bit is the sign of ``y`` (so -0.0 and
    negative values rounding to zero give 0x80).  NaN gives 0x7F / 0xFF.

    The search over all 127 non-negative finite codes is the definition of
    round-to-nearest-even written out; it is slow and meant to be obvious.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (x * np.asarray(inv_scale_f32, dtype=np.float32)).astype(np.float32)   # float32 multiply
    neg = np.signbit(y)
    nan = np.isnan(y)
    mag = np.abs(y.astype(np.float64))
    mag = np.where(nan, 0.0, np.minimum(mag, E4M3_MAX))
    flat = mag.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    step = 1 << 16
    for lo in range(0, flat.size, step):
        m = flat[lo:lo + step, None]
        dist = np.abs(m - _POS_VALUES[None, :])
        best = dist.min(axis=1, keepdims=True)
        is_best = dist == best
        # candidates at the minimal distance: at most two (a tie); prefer the even code
        even = (_POS_CODES[None, :] & 1) == 0
        pick_even = is_best & even
        has_even = pick_even.any(axis=1)
        idx_even = np.argmax(pick_even, axis=1)
        idx_any = np.argmax(is_best, axis=1)
        out[lo:lo + step] = np.where(has_even, idx_even, idx_any)
    codes = out.reshape(mag.shape).astype(np.uint8)
    codes = codes | np.where(neg, 0x80, 0).astype(np.uint8)
    codes = np.where(nan, codes | 0x7F, codes)
    return codes.astype(np.uint8)


INT8_MAX = 127


def int8_encode(x_f32, inv_scale_f32):
    """Encode float32 values as symmetric int8 codes with the tensor's (or each head's) scale.

    ``y = float32(x * inv_scale)`` (one IEEE float32 multiply); NaN gives 0;
    ``y`` is clamped to [-127, 127] (127 is an integer, so clamping first and
    rounding second equals rounding first and saturating second); then the
    nearer of the two integers around ``y`` is chosen, and on a tie the even
    one.  Returns int8 codes.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (x * np.asarray(inv_scale_f32, dtype=np.float32)).astype(np.float32)   # float32 multiply
    y = y.astype(np.float64)
    nan = np.isnan(y)
    y = np.where(nan, 0.0, np.clip(y, -INT8_MAX, INT8_MAX))
    lo = np.floor(y)                    # the integer at or below y
    hi = lo + 1.0                       # the integer above
    d_lo = y - lo
    d_hi = hi - y
    lo_even = np.mod(lo, 2.0) == 0.0
    q = np.where((d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even), hi, lo)
    return q.astype(np.int8)


def int8_to_f64(codes):
    """Stored int8 code bytes (uint8 or int8) -> float64 code values."""
    return np.asarray(codes).astype(np.uint8).view(np.int8).astype(np.float64)


def f32_to_bf16_bits(x_f32):
    """float32 values -> bfloat16 bit patterns, round to nearest, ties to even.

    Written out as the definition: the two bfloat16 neighbours of x are the
    float32 bit patterns with the low 16 bits cleared (toward zero) and that
    plus one bfloat16 ulp (away from zero); pick the nearer, and on a tie the
    one whose last kept bit is 0.  The neighbour past the largest finite value
    is infinity, which for rounding counts as 2**128 (IEEE overflow rule).
    NaN becomes a quiet NaN of the same sign; infinities stay.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    sign = bits & 0x80000000
    mag = bits & 0x7FFFFFFF
    lo = mag & 0x7FFF0000                     # toward zero
    hi = lo + 0x10000                         # away from zero (0x7F800000 = inf)

    def value(b):
        # magnitude of a float32 bit pattern as float64; 0x7F800000 counts as 2**128
        f = b.astype(np.uint32).view(np.float32).astype(np.float64)
        return np.where(b == 0x7F800000, 2.0 ** 128, f)

    with np.errstate(invalid="ignore"):        # NaN inputs are handled below
        v = mag.astype(np.uint32).view(np.float32).astype(np.float64)
        d_lo = v - value(lo)
        d_hi = value(hi) - v
    lo_even = ((lo >> 16) & 1) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(pick_hi, hi, lo)
    is_nan = mag > 0x7F800000
    is_inf = mag == 0x7F800000
    out = np.where(is_inf, 0x7F800000, out)
    out = np.where(is_nan, 0x7FC00000, out)
    return ((out | sign) >> 16).astype(np.uint16)


def f32_to_act_bits(x_f32, dtype):
    """float32 values -> stored bits of the activation dtype ('f16' or 'bf16'),
    round to nearest even (fp16: IEEE binary16 conversion)."""
    x = np.asarray(x_f32, dtype=np.float32)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def decode(bits, dtype):
    """Decode stored bits of ``dtype`` ('f16', 'bf16', 'fp8_e4m3', 'int8') to
    float64 (for the quantized formats: the code value, before the scale)."""
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "fp8_e4m3":
        return e4m3fn_to_f64(bits)
    if dtype == "int8":
        return int8_to_f64(bits)
    raise ValueError(dtype)
