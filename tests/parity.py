"""Shared comparison helpers for the GPU parity tests (the HIP path against the oracle)."""
from __future__ import annotations

import numpy as np

TOL_REL_L2 = {0: 2e-2, 1: 5e-2, 2: 5e-2}  # layer-output tolerance by weight format
TOL_TOPK_W = 1e-6


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def rel_l2_rows(a: np.ndarray, b: np.ndarray) -> float:
    """Largest per-token relative L2 error over the rows of [T][H] outputs."""
    a = a.reshape(-1, a.shape[-1])
    b = b.reshape(-1, b.shape[-1])
    return max(rel_l2(a[i], b[i]) for i in range(a.shape[0]))


def compare_step(wb, ref, ctx: str, check_state: bool = True, check_y: bool = True):
    """Compare one executed layer step of the Workbench with the oracle's LayerStep.

    Integer results are compared bit-exactly; topk weights within TOL_TOPK_W relative; the
    layer output within the format's relative-L2 tolerance.  Returns the output error."""
    wl = wb.wl
    l = ref.layer
    idx = wb.topk_idx[l].cpu().numpy()
    w = wb.topk_w[l].cpu().numpy().astype(np.float64)
    assert np.array_equal(idx, ref.topk_idx), f"{ctx}: topk idx {idx} vs {ref.topk_idx}"
    assert np.allclose(w, ref.topk_w, rtol=TOL_TOPK_W, atol=0), f"{ctx}: topk w"
    p = wb.plan()
    rec = ref.rec
    assert p["step"] == ref.s, f"{ctx}: step {p['step']} vs {ref.s}"
    assert list(p["unique"]) == rec.U, f"{ctx}: U {p['unique']} vs {rec.U}"
    assert list(p["hit"]) == rec.hit, f"{ctx}: hit {p['hit']} vs {rec.hit}"
    assert list(p["slot"]) == rec.slot, f"{ctx}: slot {p['slot']} vs {rec.slot}"
    got_m = list(zip(p["miss_key"].tolist(), p["miss_slot"].tolist(), p["miss_victim"].tolist()))
    assert got_m == [tuple(m) for m in rec.misses], f"{ctx}: misses {got_m} vs {rec.misses}"
    assert list(p["cpu_key"]) == list(rec.cpu), f"{ctx}: cpu misses {p['cpu_key']} vs {rec.cpu}"
    assert list(p["count"]) == [int(ref.count[e]) for e in rec.U], f"{ctx}: counts"
    A = wb.T * wl.top_k
    assert np.array_equal(p["perm"][:A], ref.perm), f"{ctx}: perm"
    if check_state:
        key_of, stamp, slot_of, n, step, cap = wb.snapshot()
        assert n == rec.n, f"{ctx}: n {n} vs {rec.n}"
        assert list(key_of) == rec.key_of, f"{ctx}: key_of"
        assert list(stamp) == rec.stamp, f"{ctx}: stamp"
        exp_slot_of = np.full(wl.n_keys, -1, np.int32)
        for sl, k in enumerate(rec.key_of):
            if k >= 0:
                exp_slot_of[k] = sl
        assert np.array_equal(slot_of, exp_slot_of), f"{ctx}: slot_of"
        assert step == ref.s + 1
    err = None
    if check_y and ref.y is not None:
        err = rel_l2_rows(wb.y_f64(l), ref.y)
        assert err <= TOL_REL_L2[wl.fmt], f"{ctx}: output rel-L2 {err}"
    return err
