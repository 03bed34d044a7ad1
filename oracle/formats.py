"""Exact float64 decoding of the weight and activation formats (test oracle only).

Definitions followed:
* bf16: the upper 16 bits of an IEEE-754 binary32.
* e4m3fn: OCP 8-bit Floating Point Specification (OFP8) rev 1.0, E4M3 - bias 7,
  no infinities, S.1111.111 is NaN, subnormals 2^-6 * m/8.
* e2m1: OCP Microscaling Formats (MX) v1.0, FP4 E2M1 - bias 1, subnormal 0.5*m,
  values {0, 0.5, 1, 1.5, 2, 3, 4, 6} with sign.
* e8m0: OCP MX v1.0 shared scale, 2^(c - 127), c = 255 is NaN.
* Expert blob layout: the FreeToken paper summary's execution-layer paragraph
  says weights are pre-merged into their runtime layout so a load lands in its
  final place; here one (layer, expert) blob is byte-identical in the host pool
  and in a GPU slot.  Element order:
    bf16 : Wgu[I][2][H] (gate row i then up row i), WdT[I][H] (column i of Wd[H][I]);
    fp8  : the same code arrays, then s_gu[I][2][H/128] fp32, s_d[I/128][H] fp32,
           one scale per 128 consecutive contraction elements;
    mxfp4: codes two per byte (even element in the low nibble), then
           s_gu[I][2][H/32] e8m0, s_d[I/32][H] e8m0, one scale per 32.
"""
from __future__ import annotations

import numpy as np

FMT_BF16, FMT_FP8, FMT_MXFP4 = 0, 1, 2


def bf16_to_f64(u16) -> np.ndarray:
    a = np.asarray(u16, dtype=np.uint16)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 15
    man = c & 7
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    sub = (man / 8.0) * 2.0 ** -6
    val = np.where(exp == 0, sub, normal)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


def e2m1_to_f64(nibbles) -> np.ndarray:
    n = np.asarray(nibbles).astype(np.int64) & 15
    sign = np.where((n >> 3) & 1, -1.0, 1.0)
    exp = (n >> 1) & 3
    man = n & 1
    normal = (1.0 + man / 2.0) * np.exp2(exp.astype(np.float64) - 1.0)
    sub = man * 0.5
    return sign * np.where(exp == 0, sub, normal)


def e8m0_to_f64(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def blob_size(fmt: int, H: int, I: int) -> int:
    if fmt == FMT_BF16:
        return 6 * I * H
    if fmt == FMT_FP8:
        return 3 * I * H + 4 * 2 * I * (H // 128) + 4 * (I // 128) * H
    if fmt == FMT_MXFP4:
        return 3 * I * H // 2 + 2 * I * (H // 32) + (I // 32) * H
    raise ValueError(fmt)


def _unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """bytes [..., n] -> nibbles [..., 2n], element 2j from the low nibble of byte j."""
    lo = b & 15
    hi = b >> 4
    return np.stack([lo, hi], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2)


def decode_blob(blob, fmt: int, H: int, I: int):
    """Decode one expert blob to float64 (Wg [I,H], Wu [I,H], Wd [H,I])."""
    b = np.asarray(blob, dtype=np.uint8).reshape(-1)
    assert b.size == blob_size(fmt, H, I), (b.size, blob_size(fmt, H, I))
    if fmt == FMT_BF16:
        v = b.view(np.uint16)
        Wgu = bf16_to_f64(v[: 2 * I * H]).reshape(I, 2, H)
        WdT = bf16_to_f64(v[2 * I * H: 3 * I * H]).reshape(I, H)
    elif fmt == FMT_FP8:
        o = 0
        cgu = b[o: o + 2 * I * H].reshape(I, 2, H); o += 2 * I * H
        cd = b[o: o + I * H].reshape(I, H); o += I * H
        sgu = b[o: o + 4 * 2 * I * (H // 128)].view(np.float32).astype(np.float64)
        sgu = sgu.reshape(I, 2, H // 128); o += 4 * 2 * I * (H // 128)
        sd = b[o: o + 4 * (I // 128) * H].view(np.float32).astype(np.float64).reshape(I // 128, H)
        Wgu = e4m3fn_to_f64(cgu) * np.repeat(sgu, 128, axis=2)
        WdT = e4m3fn_to_f64(cd) * np.repeat(sd, 128, axis=0)
    elif fmt == FMT_MXFP4:
        o = 0
        cgu = _unpack_nibbles(b[o: o + I * H].reshape(I, 2, H // 2)); o += I * H
        cd = _unpack_nibbles(b[o: o + I * H // 2].reshape(I, H // 2)); o += I * H // 2
        sgu = e8m0_to_f64(b[o: o + 2 * I * (H // 32)].reshape(I, 2, H // 32)); o += 2 * I * (H // 32)
        sd = e8m0_to_f64(b[o: o + (I // 32) * H].reshape(I // 32, H))
        Wgu = e2m1_to_f64(cgu) * np.repeat(sgu, 32, axis=2)
        WdT = e2m1_to_f64(cd) * np.repeat(sd, 32, axis=0)
    else:
        raise ValueError(fmt)
    return Wgu[:, 0, :].copy(), Wgu[:, 1, :].copy(), WdT.T.copy()
