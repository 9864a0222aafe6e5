"""Host checks of the parity helpers themselves: the id check must flag an
exact mismatch, accept a valid near-tie id and flag an invalid one."""
import numpy as np

from helpers import ids_match, rel_l2_rows


def _lm(V=40, H=8, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((V, H)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    return {"fmt": "bf16", "n": V, "k": H, "group": 0, "data": bits, "scales": None}


def test_ids_match_exact_and_near_ties():
    lm = _lm()
    E = (lm["data"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(1)
    f = rng.standard_normal((3, 8))
    z = f @ E.T
    order = np.argsort(-z, axis=1)
    top = order[:, 0]
    top1 = z[np.arange(3), top]
    second = z[np.arange(3), order[:, 1]]
    gap = top1 - second
    # clear rows: the oracle's id passes, another id fails
    n, bad, near = ids_match(top, top, gap, top1, f, lm)
    assert (n, bad, near) == (3, 0, 0)
    n, bad, near = ids_match(order[:, 1], top, gap, top1, f, lm)
    assert bad == 3
    # a near-tie row: the runner-up is valid when within the threshold, the
    # last-ranked id is not, an out-of-range id is not
    fake_gap = np.array([0.0, 5.0, 5.0])
    thr = float(gap[0]) + 1e-9
    n, bad, near = ids_match(np.array([order[0, 1], top[1], top[2]]), top, fake_gap, top1, f, lm, thr=thr)
    assert (bad, near) == (0, 1)
    n, bad, near = ids_match(np.array([order[0, -1], top[1], top[2]]), top, fake_gap, top1, f, lm, thr=thr)
    assert bad == 1
    n, bad, near = ids_match(np.array([-1, top[1], top[2]]), top, fake_gap, top1, f, lm, thr=thr)
    assert bad == 1


def test_rel_l2_rows_sees_one_bad_row():
    rng = np.random.default_rng(2)
    b = rng.standard_normal((1024, 64))
    a = b.copy()
    a[517] *= 1.03
    assert rel_l2_rows(a, b, 64) > 0.029
    whole = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert whole < 2e-3   # the whole-tensor norm alone would have passed it
