"""Budget-driven cache sizing (C ABI, host arithmetic) against oracle/sizing.py, and expert pool
files in the runtime layout (write, read back into host memory, rejection of mismatches)."""
import os

import numpy as np
import pytest

import moe_inputs as mi
from oracle.sizing import auto_capacity

ecoa = pytest.importorskip("expert_cache_offload_amd")
SLOT_LIMIT = 4096


def _shape(name):
    wl = mi.WORKLOADS[name]
    return wl, ecoa.make_shape(wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.fmt,
                               wl.has_shared, wl.tokens_per_step)


@pytest.mark.parametrize("name", ["tiny", "qwen35b_decode", "glm_mxfp4_4stream"])
def test_auto_capacity_matches_oracle(name):
    wl, shape = _shape(name)
    S = wl.blob_bytes
    ws = lambda c: ecoa.moe_workspace_bytes(shape, c)  # noqa: E731
    floor = min(wl.tokens_per_step * wl.top_k, wl.experts)
    rng = np.random.default_rng(5)
    for _ in range(25):
        free = int(rng.uniform(0.2, 1.3) * wl.n_keys * S)
        reserve = int(rng.uniform(0.0, 0.2) * free)
        for ratio in (None, 0.8, 0.3):
            want = auto_capacity(free, reserve, S, wl.n_keys, floor, SLOT_LIMIT, ws, ratio)
            if want is None:
                with pytest.raises(ecoa.MoeError):
                    ecoa.moe_auto_capacity(shape, free, reserve, -1.0 if ratio is None else ratio)
                continue
            got = ecoa.moe_auto_capacity(shape, free, reserve, -1.0 if ratio is None else ratio)
            assert got == want, (free, reserve, ratio, got, want)
            # the budget holds, and one more slot would break it unless a limit stops first
            assert got * S + ws(got) <= free - reserve
            top = min(wl.n_keys, SLOT_LIMIT)
            if ratio is not None:
                top = min(top, int((1 - ratio) * wl.n_keys))
            assert got == top or (got + 1) * S + ws(got + 1) > free - reserve


def test_auto_capacity_hand_cases():
    wl, shape = _shape("tiny")  # 16 experts of 192 KiB, floor 2
    S = wl.blob_bytes
    ws = lambda c: ecoa.moe_workspace_bytes(shape, c)  # noqa: E731
    assert ecoa.moe_auto_capacity(shape, 10 * S + ws(10), 0) == 10     # exactly ten slots
    assert ecoa.moe_auto_capacity(shape, 10 * S + ws(10) - 1, 0) == 9  # one byte short
    assert ecoa.moe_auto_capacity(shape, 10 * S + ws(10) + S, S) == 10  # the reserve comes off
    assert ecoa.moe_auto_capacity(shape, 100 * S, 0) == 16              # the whole pool fits
    assert ecoa.moe_auto_capacity(shape, 100 * S, 0, 0.75) == 4         # keep a quarter
    with pytest.raises(ecoa.MoeError):
        ecoa.moe_auto_capacity(shape, S, 0)                              # below the floor
    with pytest.raises(ecoa.MoeError):
        ecoa.moe_auto_capacity(shape, 100 * S, 0, 1.0)
    # the 35B shape on a 288 GB device: the whole 58 GB pool would fit; the handle's slot
    # limit decides
    wl35, s35 = _shape("qwen35b_decode")
    assert ecoa.moe_auto_capacity(s35, 288 * 10**9, 20 * 10**9) == SLOT_LIMIT


def test_pool_file_round_trip(tmp_path):
    wl, shape = _shape("tiny")
    pool = np.empty(wl.pool_bytes, np.uint8)
    mi.fill_pool(wl.seed, wl.fmt, 0, wl.layers, wl.experts, wl.hidden, wl.inter, pool)
    path = str(tmp_path / "tiny.moepool")
    ecoa.moe_pool_write(path, shape, pool.ctypes.data, 3)
    assert os.path.getsize(path) == 64 + wl.pool_bytes
    back = np.zeros_like(pool)
    ecoa.moe_pool_read(path, shape, back.ctypes.data, 5)
    assert np.array_equal(back, pool)
    with open(path, "rb") as f:
        head = f.read(64)
    assert head[:8] == b"MOEPOOL1"


def test_pool_file_rejects_mismatch(tmp_path):
    wl, shape = _shape("tiny")
    pool = np.zeros(wl.pool_bytes, np.uint8)
    path = str(tmp_path / "p.moepool")
    ecoa.moe_pool_write(path, shape, pool.ctypes.data, 1)
    other = ecoa.make_shape(wl.layers, wl.experts * 2, wl.top_k, wl.hidden, wl.inter, wl.fmt,
                            wl.has_shared, wl.tokens_per_step)
    big = np.zeros(2 * wl.pool_bytes, np.uint8)
    with pytest.raises(ecoa.MoeError):
        ecoa.moe_pool_read(path, other, big.ctypes.data, 2)
    with open(path, "r+b") as f:  # truncated
        f.truncate(64 + wl.pool_bytes - 1)
    with pytest.raises(ecoa.MoeError):
        ecoa.moe_pool_read(path, shape, pool.ctypes.data, 2)
    with pytest.raises(ecoa.MoeError):
        ecoa.moe_pool_read(str(tmp_path / "missing"), shape, pool.ctypes.data, 2)
