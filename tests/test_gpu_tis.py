"""GPU parity of tis_token_weights against the oracle.

* counts (valid tokens, tokens over the cap) bit for bit; weights exactly C
  (TIS) or 0 (MIS) where the cap decides, exactly 0 on padding, and within
  2 binary32 ulp of the oracle's fp64 exp(d) elsewhere;
* per-sequence sums within the worst-case error of an fp32 sum of the
  terms (n u sum |x|, u = 2^-24) plus the terms' own rounding; batch totals
  within the sum of those bounds;
* shapes with T % 4 == 0 (vector path) and not (per-token path), one token,
  a long row, the full batch of 1024 x 8192; padding holding NaN and
  infinities; caps 2, 1.05, +inf and 1e-30; bitwise repeatability; the call
  without statistics; empty batches.
"""

import math

import numpy as np
import pytest
import torch

from oracle import tis
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import announce, host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run(p, cap, mode, stats=True):
    w, rs, tt = binding.tis_token_weights(_dev(p["lp_train"]), _dev(p["lp_rollout"]),
                                          _dev(p["mask"]), cap, mode, stats=stats)
    return host(w), (host(rs) if rs is not None else None), (host(tt) if tt is not None else None)


def _poison_padding(p, seed):
    lt, lr = p["lp_train"].copy(), p["lp_rollout"].copy()
    pad = p["mask"] == 0
    vals = np.array([np.nan, np.inf, -np.inf, 1e30], dtype=np.float32)
    idx = np.random.default_rng(seed).integers(0, 4, size=pad.sum())
    lt[pad] = vals[idx]
    lr[pad] = vals[(idx + 1) % 4]
    return dict(lp_train=lt, lp_rollout=lr, mask=p["mask"])


def _check(p, cap, mode, got, label):
    w, rs, tt = got
    ref_w, ref_row, ref_tot = tis.importance_weights(p["lp_train"], p["lp_rollout"], p["mask"],
                                                     cap, mode)
    valid = p["mask"] != 0
    d = (p["lp_train"] - p["lp_rollout"]).astype(np.float32)
    over = valid & (d > tis.log_cap(cap))
    free = valid & ~over
    assert np.all(w[~valid] == 0), f"{label}: padding weight"
    want_over = np.float32(cap) if mode == tis.TRUNCATE else np.float32(0)
    assert np.all(w[over] == want_over), f"{label}: weight at the cap"
    err = np.abs(w[free].astype(np.float64) - ref_w[free])
    bound = 2.0 ** -22 * ref_w[free] + 2.0 ** -148
    assert np.all(err <= bound), f"{label}: weight off by {float((err / np.maximum(bound, 1e-300)).max()):.2f} bounds"
    if rs is None:
        return
    assert np.array_equal(rs[:, 0], ref_row[:, 0]) and np.array_equal(rs[:, 1], ref_row[:, 1]), \
        f"{label}: counts"
    n = valid.sum(axis=1).astype(np.float64)
    kl_abs = np.where(valid, np.abs(p["lp_rollout"].astype(np.float64) - p["lp_train"]), 0.0).sum(axis=1)
    b_w = (n * U + 2.0 ** -22) * ref_row[:, 2] + 1e-30
    b_kl = (n * U + U) * kl_abs + 1e-30
    assert np.all(np.abs(rs[:, 2] - ref_row[:, 2]) <= b_w), f"{label}: sum of weights"
    assert np.all(np.abs(rs[:, 3] - ref_row[:, 3]) <= b_kl), f"{label}: log-probability sum"
    assert tt[0] == ref_tot[0] and tt[1] == ref_tot[1], f"{label}: total counts"
    assert abs(tt[2] - ref_tot[2]) <= b_w.sum() and abs(tt[3] - ref_tot[3]) <= b_kl.sum(), \
        f"{label}: totals"


@pytest.mark.parametrize("B,T", [(1, 1), (3, 5), (7, 40), (16, 1000), (33, 4097), (5, 65536)])
@pytest.mark.parametrize("mode", [tis.TRUNCATE, tis.MASK])
def test_matches_oracle(B, T, mode):
    p = _poison_padding(workloads.tis_batch(B, T, seed=B + T), seed=B)
    for cap in (2.0, 1.05):
        announce(f"tis_token_weights B{B} T{T} mode{mode} cap{cap}")
        _check(p, cap, mode, _run(p, cap, mode), f"B{B} T{T} mode{mode} cap{cap}")


@pytest.mark.parametrize("cap", [math.inf, 1e-30])
def test_cap_limits(cap):
    p = workloads.tis_batch(9, 300, seed=4)
    for mode in (tis.TRUNCATE, tis.MASK):
        announce(f"tis_token_weights cap {cap} mode {mode}")
        got = _run(p, cap, mode)
        _check(p, cap, mode, got, f"cap {cap} mode {mode}")
        if cap == math.inf:
            assert got[1][:, 1].sum() == 0
        else:
            assert np.array_equal(got[1][:, 1], got[1][:, 0])


def test_repeatable_and_without_statistics():
    p = workloads.tis_batch(64, 2048, seed=6)
    announce("tis_token_weights repeatability")
    a = _run(p, 2.0, tis.TRUNCATE)
    b = _run(p, 2.0, tis.TRUNCATE)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    w, rs, tt = _run(p, 2.0, tis.TRUNCATE, stats=False)
    assert rs is None and tt is None
    assert np.array_equal(w, a[0])


def test_empty_batches():
    announce("tis_token_weights empty")
    z = np.zeros((0, 16), np.float32)
    w, rs, tt = _run(dict(lp_train=z, lp_rollout=z, mask=np.zeros((0, 16), np.uint8)), 2.0, 0)
    assert w.shape == (0, 16) and rs.shape == (0, 4) and np.array_equal(tt, np.zeros(4))
    z = np.zeros((5, 0), np.float32)
    w, rs, tt = _run(dict(lp_train=z, lp_rollout=z, mask=np.zeros((5, 0), np.uint8)), 2.0, 1)
    assert np.array_equal(rs, np.zeros((5, 4), np.float32)) and np.array_equal(tt, np.zeros(4))


def test_full_rollout_batch():
    cfg = workloads.TIS_BATCH
    p = workloads.tis_batch(cfg["B"], cfg["T"], seed=0)
    for mode in (tis.TRUNCATE, tis.MASK):
        announce(f"tis_token_weights full B{cfg['B']} T{cfg['T']} mode {mode}")
        _check(p, cfg["cap"], mode, _run(p, cfg["cap"], mode), f"full mode {mode}")
