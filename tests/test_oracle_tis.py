"""Pins for the oracle's token-level importance weights (CPU).

* brute force on small batches by a separate route: the binary32 difference
  and ln C rounded from exact rationals by integer arithmetic, the cap
  decision compared as rationals, Python's math.exp, exact rational sums
  for the log-probability statistic;
* closed forms: identical policies give weight 1 and a zero statistic; a
  constant shift c between the policies gives weight e^c on every token and
  a statistic of -c per token;
* limits: C = +inf gives the plain ratio and no token over the cap (TIS and
  MIS agree); a tiny C puts every response token over the cap;
* invariants on the batch recipe: weights in [0, C] up to one rounding,
  TIS = MIS below the cap, TIS = C and MIS = 0 above it, padding ignored
  even when it holds NaN or infinities;
* planted mistakes (swapped policies, the cap decided in the ratio domain
  with a different exp, padding not masked, TIS/MIS exchanged) fail these.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import tis
from precision_rl_rollout_amd import workloads
from tests import pins


def _brute(lt, lr, mask, cap, mode):
    B, T = lt.shape
    c32 = float(np.float32(cap))
    lnc = pins.fl32(Fraction(math.log(c32))) if math.isfinite(c32) else None
    w = np.zeros((B, T))
    row = np.zeros((B, 4))
    for b in range(B):
        n = over_n = 0
        sw = 0.0
        kl = Fraction(0)
        for t in range(T):
            if not mask[b, t]:
                continue
            n += 1
            d = pins.fl32(Fraction(float(lt[b, t])) - Fraction(float(lr[b, t])))
            over = lnc is not None and Fraction(float(d)) > Fraction(float(lnc))
            rho = math.exp(float(d))
            if over:
                over_n += 1
                wt = float(np.float32(cap)) if mode == tis.TRUNCATE else 0.0
            else:
                wt = rho
            w[b, t] = wt
            sw += wt
            kl += Fraction(float(lr[b, t])) - Fraction(float(lt[b, t]))
        row[b] = (n, over_n, sw, float(kl))
    return w, row


def _batch(B, T, seed):
    p = workloads.tis_batch(B, T, seed)
    return p["lp_train"], p["lp_rollout"], p["mask"]


@pytest.mark.parametrize("mode", [tis.TRUNCATE, tis.MASK])
@pytest.mark.parametrize("cap", [2.0, 1.0, 1.05, 0.5, 1.3])
def test_matches_brute_force(mode, cap):
    lt, lr, mask = _batch(6, 40, seed=int(cap * 100) + mode)
    w, row, tot = tis.importance_weights(lt, lr, mask, cap, mode)
    bw, brow = _brute(lt, lr, mask, cap, mode)
    assert np.allclose(w, bw, rtol=1e-15, atol=0)
    assert np.array_equal(row[:, :2], brow[:, :2])
    assert np.allclose(row[:, 2:], brow[:, 2:], rtol=1e-13, atol=1e-13)
    assert np.allclose(tot, row.sum(axis=0), rtol=1e-15, atol=0)


def test_tail_tokens_cross_the_cap():
    # the recipe's 1% tail must put some tokens over C = 2 for the tests
    # above and on the GPU to exercise both branches
    lt, lr, mask = _batch(64, 512, seed=0)
    _, row, _ = tis.importance_weights(lt, lr, mask, 2.0, tis.TRUNCATE)
    assert 0 < row[:, 1].sum() < 0.01 * row[:, 0].sum()


def test_identical_policies():
    lt, lr, mask = _batch(4, 100, seed=1)
    for mode in (tis.TRUNCATE, tis.MASK):
        w, row, _ = tis.importance_weights(lr, lr, mask, 1.0, mode)
        assert np.array_equal(w, mask.astype(np.float64))
        assert np.array_equal(row[:, 1], np.zeros(4)) and np.array_equal(row[:, 3], np.zeros(4))
        assert np.array_equal(row[:, 2], row[:, 0])


@pytest.mark.parametrize("c", [0.25, -0.375, 1.5])
def test_constant_shift(c):
    # log-probabilities on a 2^-10 grid in [-4, 0]: lr + c is exact in binary32
    rng = np.random.default_rng(7)
    lr = (-rng.integers(0, 4096, size=(3, 50)) / 1024.0).astype(np.float32)
    lt = (lr + np.float32(c)).astype(np.float32)
    mask = np.ones((3, 50), np.uint8)
    mask[1, 30:] = 0
    w, row, _ = tis.importance_weights(lt, lr, mask, math.inf, tis.TRUNCATE)
    assert np.allclose(w[mask != 0], math.exp(c), rtol=1e-15)
    assert np.array_equal(row[:, 3], -c * row[:, 0])
    assert np.array_equal(row[:, 1], np.zeros(3))


def test_limits_of_the_cap():
    lt, lr, mask = _batch(5, 80, seed=3)
    wt, rt, _ = tis.importance_weights(lt, lr, mask, math.inf, tis.TRUNCATE)
    wm, rm, _ = tis.importance_weights(lt, lr, mask, math.inf, tis.MASK)
    d = (lt - lr).astype(np.float32).astype(np.float64)
    assert np.array_equal(wt, wm)
    assert np.allclose(wt, np.where(mask != 0, np.exp(d), 0.0), rtol=1e-15, atol=0)
    assert rt[:, 1].sum() == 0
    tiny = 1e-30
    wt, rt, _ = tis.importance_weights(lt, lr, mask, tiny, tis.TRUNCATE)
    wm, rm, _ = tis.importance_weights(lt, lr, mask, tiny, tis.MASK)
    assert np.array_equal(rt[:, 1], rt[:, 0])
    assert np.array_equal(wt, np.where(mask != 0, float(np.float32(tiny)), 0.0))
    assert np.array_equal(wm, np.zeros_like(wm))


def test_invariants_and_padding():
    lt, lr, mask = _batch(16, 300, seed=5)
    cap = 2.0
    lt2, lr2 = lt.copy(), lr.copy()
    pad = mask == 0
    lt2[pad] = np.nan
    lr2[pad] = np.where(np.arange(pad.sum()) % 2 == 0, np.inf, -np.inf).astype(np.float32)
    wt, rt, tt = tis.importance_weights(lt2, lr2, mask, cap, tis.TRUNCATE)
    wm, rm, tm = tis.importance_weights(lt2, lr2, mask, cap, tis.MASK)
    w0, r0, _ = tis.importance_weights(lt, lr, mask, cap, tis.TRUNCATE)
    assert np.array_equal(wt, w0) and np.array_equal(rt, r0)
    assert np.all(wt[pad] == 0) and np.all(wm[pad] == 0)
    assert np.all(wt >= 0) and np.all(wt <= cap * (1 + 2.0 ** -22))
    d = (lt - lr).astype(np.float32)
    over = (mask != 0) & (d > np.float32(math.log(float(np.float32(cap)))))
    assert np.array_equal(wt[over], np.full(over.sum(), cap))
    assert np.all(wm[over] == 0)
    assert np.array_equal(wt[~over], wm[~over])
    assert np.array_equal(rt[:, 1], over.sum(axis=1)) and np.array_equal(rt[:, 1], rm[:, 1])


def test_rejects_bad_arguments():
    lt, lr, mask = _batch(2, 8, seed=0)
    with pytest.raises(ValueError):
        tis.importance_weights(lt, lr, mask, 0.0, tis.TRUNCATE)
    with pytest.raises(ValueError):
        tis.importance_weights(lt, lr, mask, 2.0, 7)
    bad = lt.copy()
    bad[0, 0] = np.nan
    with pytest.raises(ValueError):
        tis.importance_weights(bad, lr, mask, 2.0, tis.TRUNCATE)


# ---------------------------------------------------------------- mutants
def _swapped(lt, lr, mask, cap, mode):
    return tis.importance_weights(lr, lt, mask, cap, mode)


def _unmasked(lt, lr, mask, cap, mode):
    return tis.importance_weights(lt, lr, np.ones_like(mask), cap, mode)


def _exchanged(lt, lr, mask, cap, mode):
    return tis.importance_weights(lt, lr, mask, cap, tis.MASK if mode == tis.TRUNCATE else tis.TRUNCATE)


def _ratio_domain(lt, lr, mask, cap, mode):
    """The cap decided as exp(d) > C with an exp evaluated in binary32
    through a reciprocal (a different rounding)."""
    w, row, tot = tis.importance_weights(lt, lr, mask, math.inf, tis.TRUNCATE)
    d = (lt - lr).astype(np.float32)
    rho32 = (np.float32(1) / np.exp(-d)).astype(np.float32)
    over = (mask != 0) & (rho32 > np.float32(cap))
    w = np.where(over, cap if mode == tis.TRUNCATE else 0.0, w)
    row = row.copy()
    row[:, 1] = over.sum(axis=1)
    return w, row, row.sum(axis=0)


@pytest.mark.parametrize("mutant", [_swapped, _unmasked, _exchanged])
def test_mutants_fail_the_pins(mutant):
    lt, lr, mask = _batch(6, 40, seed=11)
    mask[2, :] = 0
    bw, brow = _brute(lt, lr, mask, 1.05, tis.TRUNCATE)
    w, row, _ = mutant(lt, lr, mask, 1.05, tis.TRUNCATE)
    assert not (np.allclose(w, bw, rtol=1e-15, atol=0) and np.array_equal(row[:, :2], brow[:, :2]))


def test_ratio_domain_mutant_fails_at_the_boundary():
    # tokens placed exactly at d = fl32(ln C) and one binary32 step either
    # side: the log-space decision is fixed; a ratio-domain one with another
    # exp rounding disagrees on some of them
    cap = 1.3
    lnc = np.float32(math.log(float(np.float32(cap))))
    steps = np.arange(-40, 41, dtype=np.int32)
    d = (lnc.view(np.int32) + steps).view(np.float32)
    lr = np.full((1, d.size), np.float32(-1.0))
    lt = (lr + d[None, :]).astype(np.float32)
    dd = (lt - lr).astype(np.float32)
    mask = np.ones_like(lt, dtype=np.uint8)
    bw, brow = _brute(lt, lr, mask, cap, tis.MASK)
    w, row, _ = tis.importance_weights(lt, lr, mask, cap, tis.MASK)
    assert np.array_equal(row[:, :2], brow[:, :2])
    assert row[0, 1] == np.count_nonzero(dd > lnc)
    mw, mrow, _ = _ratio_domain(lt, lr, mask, cap, tis.MASK)
    assert not np.array_equal(mrow[:, 1], brow[:, 1]) or not np.array_equal(mw, bw)
