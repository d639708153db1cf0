"""Pins of the oracle's codecs against library routines and the format definitions.

The decoders are checked against torch's own CPU casts (an independent
implementation) over every bit pattern; the e4m3fn table against hand-computed
values of the OCP format; the encoder against torch's float8_e4m3fn cast
(round-to-nearest-even) after an explicit clamp to +-448, over every bf16 and
fp16 input under a power-of-two scale (where the float32 multiply is exact)
and a generic scale.
"""

import numpy as np
import pytest
import torch

from oracle import codecs as C

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


def test_bf16_decoder_all_patterns_vs_torch():
    ref = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(C.bf16_bits_to_f64(ALL16), ref)


def test_f16_decoder_all_patterns_vs_torch():
    ref = torch.from_numpy(ALL16.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    assert _same(C.f16_bits_to_f64(ALL16), ref)


def test_bf16_known_values():
    assert C.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert C.bf16_bits_to_f64(np.array([0xC000], np.uint16))[0] == -2.0
    assert C.bf16_bits_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -133


def test_e4m3fn_table_known_values():
    t = C.E4M3FN_TABLE
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0                # exponent field 7 = bias
    assert t[0x7E] == 448.0              # largest finite
    assert t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2      # no infinities, only S.1111.111 is NaN
    assert np.all(np.diff(t[:0x7F]) > 0)  # monotone over the non-negative codes


def test_e4m3fn_table_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(C.E4M3FN_TABLE, ref)


def _torch_encode(x_f32, inv_scale):
    with np.errstate(over="ignore", invalid="ignore"):
        y = (np.asarray(x_f32, np.float32) * np.float32(inv_scale)).astype(np.float32)
    y = np.clip(y, -448.0, 448.0).astype(np.float32)   # NaN passes through clip
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("src", ["bf16", "f16"])
@pytest.mark.parametrize("inv_scale", [np.float32(8.0), np.float32(1.0) / np.float32(0.0137)])
def test_e4m3fn_encoder_exhaustive_vs_torch(src, inv_scale):
    with np.errstate(invalid="ignore"):
        x = C.decode(ALL16, src).astype(np.float32)
    finite = np.isfinite(x)
    mine = C.e4m3fn_encode(x, inv_scale)
    ref = _torch_encode(x, inv_scale)
    # finite inputs: bit-identical codes (torch keeps -0.0's sign too)
    assert np.array_equal(mine[finite], ref[finite])
    # infinities saturate, NaN stays NaN
    inf = np.isinf(x)
    assert np.all(C.E4M3FN_TABLE[mine[inf]] == np.sign(x[inf]) * 448.0)
    nan = np.isnan(x)
    assert np.all((mine[nan] & 0x7F) == 0x7F)


def test_e4m3fn_encoder_ties_and_saturation():
    enc = lambda v: int(C.e4m3fn_encode(np.array([v], np.float32), np.float32(1.0))[0])
    assert enc(1.0) == 0x38
    # 1 + 1/16 is halfway between 1.0 (mantissa 000) and 1.125 (001): even wins
    assert enc(1.0625) == 0x38
    # 1.1875 halfway between 1.125 (001) and 1.25 (010): even wins
    assert enc(1.1875) == 0x3A
    assert enc(464.0) == 0x7E and enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(2.0 ** -10) == 0x00      # halfway between 0 and 2^-9: even (0) wins
    assert enc(3 * 2.0 ** -10) == 0x02  # halfway between 1 and 2 (x 2^-9): even wins
    assert enc(-0.0) == 0x80
    assert enc(float("nan")) & 0x7F == 0x7F


def test_e4m3fn_roundtrip_all_codes():
    vals = C.E4M3FN_TABLE.astype(np.float32)
    codes = np.arange(256, dtype=np.uint8)
    back = C.e4m3fn_encode(vals, np.float32(1.0))
    finite = np.isfinite(vals)
    assert np.array_equal(back[finite], codes[finite])


# ---------------------------------------------------------------- int8 --
# The pages name int8 as their example of KV-cache quantization ("vLLM 推理全流程
# 深度解析", PagedAttention remark); the format is the symmetric one described
# in oracle.codecs.  The independent reference is torch's per-tensor
# quantization (qint8, zero point 0: round to nearest even of x * (1 / scale)
# with saturation), whose only difference is that it also produces -128.

def _torch_int8(x_f32, scale):
    q = torch.quantize_per_tensor(torch.from_numpy(np.asarray(x_f32, np.float32)), float(scale), 0,
                                  torch.qint8)
    return np.maximum(q.int_repr().numpy(), -127)   # the symmetric range stops at -127


@pytest.mark.parametrize("src", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [np.float32(0.125), np.float32(0.0137)])
def test_int8_encoder_exhaustive_vs_torch(src, scale):
    with np.errstate(invalid="ignore"):
        x = C.decode(ALL16, src).astype(np.float32)
    finite = np.isfinite(x)
    mine = C.int8_encode(x, np.float32(1.0) / scale)
    assert mine.dtype == np.int8
    assert np.array_equal(mine[finite], _torch_int8(x[finite], scale))
    # infinities saturate, NaN encodes as 0, -128 never appears
    inf = np.isinf(x)
    assert np.all(mine[inf] == np.sign(x[inf]) * 127)
    assert np.all(mine[np.isnan(x)] == 0)
    assert mine.min() >= -127


def test_int8_encoder_ties_and_saturation():
    enc = lambda v: int(C.int8_encode(np.array([v], np.float32), np.float32(1.0))[0])
    assert [enc(v) for v in (0.5, 1.5, 2.5, -0.5, -1.5, -2.5)] == [0, 2, 2, 0, -2, -2]
    assert [enc(v) for v in (0.49, 0.51, -0.51, 126.5, 126.6)] == [0, 1, -1, 126, 127]
    assert enc(127.5) == 127 and enc(1e9) == 127 and enc(-127.5) == -127 and enc(-1e9) == -127
    assert enc(float("inf")) == 127 and enc(float("-inf")) == -127 and enc(float("nan")) == 0
    # the scale is applied as one float32 multiply before rounding
    assert int(C.int8_encode(np.array([0.3], np.float32), np.float32(10.0))[0]) == 3


def test_int8_codes_roundtrip_and_decoder_vs_torch():
    codes = np.arange(-127, 128, dtype=np.int8)
    assert np.array_equal(C.int8_encode(codes.astype(np.float32), np.float32(1.0)), codes)
    raw = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(raw).view(torch.int8).to(torch.float64).numpy()
    assert np.array_equal(C.int8_to_f64(raw), ref)
    assert np.array_equal(C.decode(raw, "int8"), ref)


def test_int8_error_bound():
    # in range, the decoded value is within half a step of the input
    rng = np.random.default_rng(0)
    scale = np.float32(0.0137)
    x = (rng.standard_normal(100000) * 0.5).astype(np.float32)
    x = x[np.abs(x) < 127 * scale]
    back = C.int8_to_f64(C.int8_encode(x, np.float32(1.0) / scale).view(np.uint8)) * float(scale)
    assert np.max(np.abs(back - x.astype(np.float64))) <= float(scale) * 0.5 * (1 + 1e-6)
