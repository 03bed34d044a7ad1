"""Sanity of the seeded input generator (moe_inputs): distributions, encoders against
library conversions, determinism, addressability, and the workload table."""
import numpy as np
import torch

import moe_inputs as mi


def test_normals_moments_and_addressability():
    k = mi.stream_key(0, 2, 1, 2, 0)
    a = mi.normals(k, 0, 400000)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    assert abs(np.mean(a ** 4) - 3) < 0.05  # Gaussian kurtosis
    # any window of the stream equals the same slice of a longer draw
    b = mi.normals(k, 12345, 1001)
    assert np.array_equal(b, a[12345:13346])
    assert not np.array_equal(mi.normals(mi.stream_key(0, 2, 1, 2, 1), 0, 100), a[:100])


def test_e4m3_encoder_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 100, rng.standard_normal(20000) * 0.01,
                        [0.0, 448.0, 449.0, 463.9, 464.0, 500.0, 2.0 ** -6, 2.0 ** -10, 2.0 ** -9 * 1.5]])
    x = x.astype(np.float32)
    ours = np.array([mi.enc_e4m3(float(v)) for v in x], np.uint8)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e2m1_encoder_nearest_even():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for v in np.arange(0, 8.0, 0.125):
        c = mi.enc_e2m1(float(v))
        d = [abs(v - m) for m in mags]
        best = min(d)
        cand = [i for i in range(8) if d[i] == best]
        want = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
        assert c == want, (v, c, want)
        assert mi.enc_e2m1(float(-v)) == (want | 8)


def test_generator_deterministic_and_distinct():
    a = mi.expert_blob(0, 0, 2, 0, 1, 256, 128)
    b = mi.expert_blob(0, 0, 2, 0, 1, 256, 128)
    c = mi.expert_blob(0, 0, 2, 0, 2, 256, 128)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    pool = np.empty(4 * a.size, np.uint8)
    mi.fill_pool(0, 0, 0, 1, 4, 256, 128, pool)
    assert np.array_equal(pool[a.size:2 * a.size], a)


def test_decode_acts_ar1():
    acts = mi.decode_acts(0, 0, 2, 3, 200, 512)
    assert acts.shape == (200, 2, 3, 512)
    x = torch.from_numpy(acts.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    # lag-1 autocorrelation of the AR(1) stream is 0.8
    r = np.mean(x[1:] * x[:-1]) / np.mean(x * x)
    assert abs(r - 0.8) < 0.02
    assert abs(x.std() - 1) < 0.05


def test_workload_table():
    W = mi.WORKLOADS
    assert W["qwen35b_decode"].capacity == 1843 and W["qwen35b_decode"].blob_bytes == 9437184
    assert W["dsv4_fp8_decode"].capacity == 1871 and W["dsv4_fp8_decode"].blob_bytes == 25952256
    g = W["glm_mxfp4_4stream"]
    assert g.capacity == 819 and g.resize_capacity == 307 and g.blob_bytes == 20054016
    assert W["tiny"].capacity == 8 and W["tiny"].blob_bytes == 196608
    assert W["qwen35b_decode"].pool_bytes == 57982058496
