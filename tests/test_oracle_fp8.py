"""Pins for the oracle's e4m3 KV-cache format, quantisation and attention (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import block_attention, from_bf16
from oracle.fp8 import (block_attention_fp8, dequantize_kv, e4m3_decode, e4m3_encode,
                        quantize_kv)
from synth import f32_to_bf16_bits

ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[(ALL & 0x7F) != 0x7F]


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_landmark_codes_have_their_closed_form_values():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in cases.items():
        assert e4m3_decode(np.uint8(c)) == v, hex(c)
    assert np.signbit(e4m3_decode(np.uint8(0x80)))
    assert np.isnan(e4m3_decode(np.uint8(0x7F))) and np.isnan(e4m3_decode(np.uint8(0xFF)))


def test_decoding_matches_torch_float8_e4m3fn_for_all_codes():
    ours, ref = e4m3_decode(ALL), torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_pure_python_decoding_agrees():
    for c in FINITE:
        s, e, m = int(c) >> 7, (int(c) >> 3) & 15, int(c) & 7
        v = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
        assert e4m3_decode(c) == (-v if s else v)


def test_every_finite_code_round_trips():
    assert np.array_equal(e4m3_encode(e4m3_decode(FINITE)), FINITE)


def test_rounding_matches_torch_for_in_range_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (1e-3, 0.05, 1.0, 30.0)])
    x = x[np.abs(x) < 448.0].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)


def test_midpoints_round_to_the_even_code():
    pos = FINITE[FINITE < 0x7F]
    v = e4m3_decode(pos)
    for c in range(len(pos) - 1):
        mid = (v[c] + v[c + 1]) / 2
        even = pos[c] if pos[c] % 2 == 0 else pos[c + 1]
        assert e4m3_encode(mid) == even
        assert e4m3_encode(np.nextafter(mid, 0.0)) == pos[c]
        assert e4m3_encode(np.nextafter(mid, 1e9)) == pos[c + 1]
        assert e4m3_encode(-mid) == (even | 0x80)


def test_saturation_and_signed_zero():
    assert list(e4m3_encode([448.0, 463.9, 464.0, 480.0, 1e30])) == [0x7E] * 5
    assert list(e4m3_encode([-448.0, -1e30])) == [0xFE, 0xFE]
    assert list(e4m3_encode([0.0, -0.0, 2.0 ** -11, -2.0 ** -11])) == [0x00, 0x80, 0x00, 0x80]
    assert list(e4m3_encode([np.inf, -np.inf])) == [0x7E, 0xFE]
    with pytest.raises(ValueError):
        e4m3_encode([np.nan])
    # an fp32 quotient that overflows is an infinity and saturates
    big = f32_to_bf16_bits(np.array([[3.0e38, -3.0e38]], np.float32)).reshape(1, 2, 1)
    assert list(quantize_kv(big, np.array([1e-5], np.float32)).ravel()) == [0x7E, 0xFE]


def test_quantisation_divides_by_the_scale_of_each_head():
    rng = np.random.default_rng(1)
    x = f32_to_bf16_bits(rng.standard_normal((5, 4, 3, 16)).astype(np.float32))
    xf = from_bf16(x)
    # power-of-two scales: fp32 division is exact, so the code is that of x / s
    scale = np.array([1.0, 0.25, 4.0], np.float32)
    got = quantize_kv(x, scale)
    for h in range(3):
        assert np.array_equal(got[:, :, h], e4m3_encode(xf[:, :, h] / float(scale[h])))
    # scale 1: torch's conversion of the bf16 values
    bf = torch.from_numpy(x.astype(np.int16)).view(torch.bfloat16)
    ones = np.ones(3, np.float32)
    assert np.array_equal(quantize_kv(x, ones), bf.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    # the head axis of pages [num_pages, Hkv, 16, D]
    xp = np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    assert np.array_equal(quantize_kv(xp, scale, head_axis=1), got.transpose(0, 2, 1, 3))
    # an fp32 quotient that lies between two e4m3 values: the fp32 rounding decides
    big = f32_to_bf16_bits(np.array([[[3.0]]], np.float32))
    assert quantize_kv(big, np.array([3.0], np.float32)) == 0x38          # exactly 1.0


def test_dequantisation_multiplies_each_head_by_its_scale():
    rng = np.random.default_rng(2)
    codes = rng.choice(FINITE, size=(6, 3, 16, 8)).astype(np.uint8)
    scale = np.array([0.5, 3.0, 0.01], np.float32)
    got = dequantize_kv(codes, scale, head_axis=1)
    for h in range(3):
        assert np.array_equal(got[:, h], e4m3_decode(codes[:, h]) * float(scale[h]))


def _case(seed, L=45, K=5, Hq=4, Hkv=2, D=16, num_pages=8):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits((rng.standard_normal((1, K, Hq, D)) * 0.5).astype(np.float32))
    pick = lambda shape: rng.choice(FINITE, size=shape).astype(np.uint8)   # noqa: E731
    kp, vp = pick((num_pages, Hkv, 16, D)), pick((num_pages, Hkv, 16, D))
    kb, vb = pick((1, K, Hkv, D)), pick((1, K, Hkv, D))
    table = rng.permutation(num_pages).astype(np.int32)[None, :]
    return q, kb, vb, kp, vp, table, np.array([L], np.int32)


@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_k_scale_acts_as_a_per_head_score_scale(mode):
    q, kb, vb, kp, vp, table, lens = _case(3)
    ks = np.array([0.02, 0.05], np.float32)
    vs = np.array([1.0, 1.0], np.float32)
    got = block_attention_fp8(q, kb, vb, kp, vp, ks, vs, table, lens, mode)
    unit = np.ones(2, np.float32)
    for g in range(2):
        sc = 0.25 * float(ks[g])
        ref = block_attention_fp8(q, kb, vb, kp, vp, unit, vs, table, lens, mode, scale=sc)
        np.testing.assert_allclose(got[:, :, 2 * g:2 * g + 2], ref[:, :, 2 * g:2 * g + 2], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mode", ["draft", "verify"])
def test_v_scale_multiplies_the_head_output(mode):
    q, kb, vb, kp, vp, table, lens = _case(4)
    ks = np.array([0.03, 0.03], np.float32)
    base = block_attention_fp8(q, kb, vb, kp, vp, ks, np.ones(2, np.float32), table, lens, mode)
    vs = np.array([0.5, 7.0], np.float32)
    got = block_attention_fp8(q, kb, vb, kp, vp, ks, vs, table, lens, mode)
    for g in range(2):
        np.testing.assert_allclose(got[:, :, 2 * g:2 * g + 2], float(vs[g]) * base[:, :, 2 * g:2 * g + 2],
                                   rtol=1e-12, atol=1e-14)


def test_constant_values_come_out_unchanged():
    q, kb, vb, kp, vp, table, lens = _case(5)
    vb[:] = 0x3A          # 1.25
    vp[:] = 0x3A
    vs = np.array([2.0, 0.5], np.float32)
    out = block_attention_fp8(q, kb, vb, kp, vp, np.array([0.1, 0.1], np.float32), vs, table, lens, "draft")
    np.testing.assert_allclose(out[:, :, :2], 2.5, rtol=1e-13)
    np.testing.assert_allclose(out[:, :, 2:], 0.625, rtol=1e-13)


def test_fp8_attention_is_bf16_attention_on_the_decoded_values():
    q, kb, vb, kp, vp, table, lens = _case(6)
    ks, vs = np.array([0.04, 0.02], np.float32), np.array([0.3, 0.6], np.float32)
    got = block_attention_fp8(q, kb, vb, kp, vp, ks, vs, table, lens, "verify")
    dec = lambda c, s, ax: np.moveaxis(np.moveaxis(e4m3_decode(c), ax, -1) * s.astype(np.float64), -1, ax)  # noqa: E731
    ref = block_attention(from_bf16(q), dec(kb, ks, 2), dec(vb, vs, 2), dec(kp, ks, 1), dec(vp, vs, 1),
                          table, lens, "verify")
    np.testing.assert_array_equal(got, ref)
