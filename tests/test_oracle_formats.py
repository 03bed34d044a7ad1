"""Pins for oracle/formats.py: exact decoders against library routines and the OCP tables,
and the blob decoder against independently quantised copies of the generator's weights."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import formats as F


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # S.1111.111 for both signs
    assert np.array_equal(ours[~nan], ref[~nan])
    # a few values from the OFP8 table
    assert F.e4m3fn_to_f64(np.uint8(0x7E)) == 448.0
    assert F.e4m3fn_to_f64(np.uint8(0x01)) == 2.0 ** -9
    assert F.e4m3fn_to_f64(np.uint8(0x08)) == 2.0 ** -6
    assert F.e4m3fn_to_f64(np.uint8(0x38)) == 1.0


def test_e2m1_all_codes_match_ocp_table():
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    expect = np.array(table + [-v for v in table])
    ours = F.e2m1_to_f64(np.arange(16))
    assert np.array_equal(ours, expect)
    assert np.signbit(ours[8])  # -0


def test_e8m0():
    c = np.array([0, 1, 126, 127, 128, 254, 255], dtype=np.uint8)
    v = F.e8m0_to_f64(c)
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126 and v[2] == 0.5 and v[3] == 1.0
    assert v[4] == 2.0 and v[5] == 2.0 ** 127 and np.isnan(v[6])
    if hasattr(torch, "float8_e8m0fnu"):
        ref = torch.from_numpy(c[:-1].copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        assert np.array_equal(v[:-1], ref)


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 1 << 16, size=100000, dtype=np.uint16)
    u = u[(u & 0x7F80) != 0x7F80]  # drop inf/nan patterns
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_to_f64(u), ref)


SHAPES = [(256, 128), (512, 256)]


@pytest.mark.parametrize("H,I", SHAPES)
def test_blob_bf16_exact(H, I):
    """Decoded bf16 blob == torch bf16 rounding of the generator's fp32 weights, element by
    element: pins the gate/up interleave, the transposed down projection and the decode."""
    Wg, Wu, Wd = mi.expert_f32(0, 2, 3, 5, H, I)
    blob = mi.expert_blob(0, 0, 2, 3, 5, H, I)
    dg, du, dd = F.decode_blob(blob, 0, H, I)

    def r(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()

    assert np.array_equal(dg, r(Wg))
    assert np.array_equal(du, r(Wu))
    assert np.array_equal(dd, r(Wd))


def _fp8_expected(W, axis_blocks):
    """Independent fp8 quantisation: per 128-block of the contraction axis (last axis),
    s = max|w|/448 in fp32, codes by torch's e4m3fn conversion of w/s."""
    W = W.astype(np.float32)
    n = W.shape[-1]
    Wb = W.reshape(*W.shape[:-1], n // 128, 128)
    amax = np.abs(Wb).max(axis=-1, keepdims=True)
    s = (amax / np.float32(448.0)).astype(np.float32)
    q = torch.from_numpy((Wb / s).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (q * s.astype(np.float64)).reshape(W.shape)


@pytest.mark.parametrize("H,I", SHAPES)
def test_blob_fp8_exact(H, I):
    Wg, Wu, Wd = mi.expert_f32(0, 2, 1, 2, H, I)
    blob = mi.expert_blob(0, 1, 2, 1, 2, H, I)
    dg, du, dd = F.decode_blob(blob, 1, H, I)
    assert np.array_equal(dg, _fp8_expected(Wg, 128))
    assert np.array_equal(du, _fp8_expected(Wu, 128))
    assert np.array_equal(dd, _fp8_expected(Wd, 128))  # Wd[H][I]: blocks along I
    # quantisation error bound of e4m3: half an ulp (2^-4 relative) or the subnormal step
    for d, W in ((dg, Wg), (dd, Wd)):
        s = np.repeat(np.abs(W.reshape(W.shape[0], -1, 128)).max(-1) / 448.0, 128, axis=1)
        err = np.abs(d - W)
        assert np.all(err <= np.maximum(np.abs(W) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6))


def _e2m1_nearest_even(v):
    """Independent e2m1 rounding: nearest of the 8 magnitudes, ties to the even code,
    saturating at 6."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.abs(v)
    d = np.abs(a[..., None] - mags)
    best = d.min(-1, keepdims=True)
    cand = d == best
    first = np.argmax(cand, -1)
    last = 7 - np.argmax(cand[..., ::-1], -1)
    codes = np.where(first % 2 == 0, first, last)  # two nearest codes differ in parity
    return np.sign(v) * mags[codes]


def _mx_expected(W):
    W = W.astype(np.float32)
    n = W.shape[-1]
    Wb = W.reshape(*W.shape[:-1], n // 32, 32).astype(np.float64)
    amax = np.abs(Wb).max(-1, keepdims=True)
    _, e = np.frexp(amax)
    X = (e - 1) - 2
    q = _e2m1_nearest_even(Wb / np.exp2(X))
    return (q * np.exp2(X)).reshape(W.shape)


@pytest.mark.parametrize("H,I", SHAPES)
def test_blob_mxfp4_exact(H, I):
    Wg, Wu, Wd = mi.expert_f32(0, 2, 0, 7, H, I)
    blob = mi.expert_blob(0, 2, 2, 0, 7, H, I)
    dg, du, dd = F.decode_blob(blob, 2, H, I)
    assert np.array_equal(dg, _mx_expected(Wg))
    assert np.array_equal(du, _mx_expected(Wu))
    assert np.array_equal(dd, _mx_expected(Wd))


def test_blob_sizes_match_layout_table():
    assert F.blob_size(0, 2048, 768) == 9437184
    assert F.blob_size(1, 4096, 2048) == 25952256
    assert F.blob_size(2, 6144, 2048) == 20054016
    assert F.blob_size(0, 256, 128) == 196608
