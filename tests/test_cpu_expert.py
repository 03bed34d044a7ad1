"""The CPU expert FFN of the hybrid decode path (host code of the C-ABI library, no GPU)
against the float64 oracle, per token relative L2, at the tiny shape and the 35B shape,
1..8 tokens with routing weights; and its measured rate is positive."""
import numpy as np
import pytest

import moe_inputs as mi
from oracle.ffn import expert_ffn
from oracle.formats import FMT_BF16, bf16_to_f64, decode_blob

ecoa = pytest.importorskip("expert_cache_offload_amd")


def _shape(H, I, T=8):
    S = ecoa.moe_blob_bytes(ecoa.MOE_FMT_BF16, H, I)
    return ecoa.make_shape(1, 4, 2, H, I, ecoa.MOE_FMT_BF16, 0, T), S


@pytest.mark.parametrize("H,I", [(256, 128), (2048, 768)])
@pytest.mark.parametrize("T,threads", [(1, 1), (3, 4), (8, 7)])
def test_cpu_expert_matches_oracle(H, I, T, threads):
    shape, S = _shape(H, I)
    blob = mi.expert_blob(11, FMT_BF16, mi.PURPOSE_EXPERT, 0, 3, H, I)
    assert blob.size == S
    rng = np.random.default_rng(T * 100 + H)
    xf = rng.standard_normal((T, H)).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation (any bf16 input)
    w = rng.uniform(0.05, 1.0, T).astype(np.float32)
    y0 = rng.standard_normal((T, H)).astype(np.float32)  # the call adds to y
    y = y0.copy()
    ecoa.moe_cpu_expert_ffn(shape, blob.ctypes.data, x.ctypes.data, T, w.ctypes.data,
                            y.ctypes.data, threads)
    Wg, Wu, Wd = decode_blob(blob, FMT_BF16, H, I)
    ref = expert_ffn(bf16_to_f64(x), Wg, Wu, Wd) * w[:, None].astype(np.float64)
    got = y.astype(np.float64) - y0.astype(np.float64)
    for t in range(T):
        err = np.linalg.norm(got[t] - ref[t]) / np.linalg.norm(ref[t])
        assert err < 1e-4, (t, err)


def test_cpu_expert_rejects_other_formats_and_sizes():
    shape, S = _shape(256, 128)
    blob = np.zeros(S, np.uint8)
    x = np.zeros((9, 256), np.uint16)
    w = np.zeros(9, np.float32)
    y = np.zeros((9, 256), np.float32)
    with pytest.raises(ecoa.MoeError):
        ecoa.moe_cpu_expert_ffn(shape, blob.ctypes.data, x.ctypes.data, 9, w.ctypes.data,
                                y.ctypes.data, 2)
    fp8 = ecoa.make_shape(1, 4, 2, 256, 128, ecoa.MOE_FMT_FP8_E4M3_K128, 0, 1)
    with pytest.raises(ecoa.MoeError):
        ecoa.moe_cpu_expert_ffn(fp8, blob.ctypes.data, x.ctypes.data, 1, w.ctypes.data,
                                y.ctypes.data, 2)


def test_cpu_expert_rate_positive():
    shape, S = _shape(256, 128)
    pool = np.concatenate([mi.expert_blob(11, FMT_BF16, mi.PURPOSE_EXPERT, 0, e, 256, 128)
                           for e in range(4)])
    g = ecoa.moe_cpu_expert_rate(shape, pool.ctypes.data, 4, 2, 3)
    assert g > 0


def test_mode_choice_threshold():
    """The library's mode rule (moe_choose_mode) against the oracle's hybrid_mode and the
    pages' printed probe rows."""
    import json
    import os

    from oracle.split import hybrid_mode
    assert not ecoa.choose_hybrid(52.4, 51.5)   # the pages' bf16 probe: 1.02x -> offload
    assert ecoa.choose_hybrid(124.5, 56.0)
    assert not ecoa.choose_hybrid(0.0, 51.3)    # no CPU rate
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "mode_probe_ceilings.json")))
    fmt_of = {"bf16": ecoa.MOE_FMT_BF16, "fp8": ecoa.MOE_FMT_FP8_E4M3_K128}
    for row in g["rows"]:
        got = ecoa.moe_choose_mode(fmt_of[row["dtype"]], row["cpu_GBps"] or 0.0,
                                   row["offload_GBps"])
        assert got == (1 if row["mode"] == "hybrid" else 0), row
    rng = np.random.default_rng(3)
    for _ in range(5000):
        cpu, fill = (float(v) for v in rng.uniform(0.0, 300.0, 2))
        if rng.random() < 0.1:
            cpu = 2.0 * fill  # exactly at the threshold: hybrid
        assert ecoa.moe_choose_mode(0, cpu, fill) == int(hybrid_mode(cpu, fill)), (cpu, fill)
        assert ecoa.moe_choose_mode(1, cpu, fill) == 0  # fp8: no CPU expert path
        assert ecoa.moe_choose_mode(2, cpu, fill) == 0  # MXFP4: none either
    assert ecoa.moe_choose_mode(0, -1.0, 50.0) == -1
    assert ecoa.moe_choose_mode(0, float("nan"), 50.0) == -1
    assert ecoa.moe_choose_mode(3, 100.0, 50.0) == -1


def test_kernel_closed_form_split_equals_oracle_minimiser():
    """The route kernel's closed form (floor of the equal-finish point or the next integer),
    called on the host, against the oracle's exhaustive makespan minimiser."""
    from oracle.split import miss_split
    rng = np.random.default_rng(9)
    cases = [(m, bc, bp) for m in range(0, 130) for bc, bp in
             ((0, 56_000), (56_000, 0), (50_000, 50_000), (124_500, 56_000), (7, 3), (1, 10**6))]
    cases += [(int(rng.integers(0, 129)), int(rng.integers(0, 400_000)),
               int(rng.integers(0, 400_000))) for _ in range(3000)]
    for m, bc, bp in cases:
        if bc == 0 and bp == 0:
            continue
        assert ecoa.moe_miss_split(m, bc, bp) == miss_split(m, bc, bp), (m, bc, bp)
    assert ecoa.moe_miss_split(-1, 1, 1) == -1
