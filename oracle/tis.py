"""Token-level importance weights for rollout correction (CPU oracle).
TEST INFRASTRUCTURE ONLY (see the package header).

"FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
Learning", abstract, item (iii): the mismatch between the low-precision
rollout policy and the higher-precision policy the trainer assumes is
corrected by importance sampling at token level, in a truncated (TIS) and a
masked (MIS) variant.  The FlashRL article (section on the rollout-training
mismatch) introduces truncated importance sampling for the same purpose and
plots the KL divergence between the trainer's and the rollout engine's
policies (figure 2, right).  Neither page prints a formula or a constant;
the readings taken here:

* per generated token t of a response, the ratio of the sampled token's
  probability under the trainer's policy to that under the rollout policy,
  from the two log-probabilities: ``rho = exp(lp_train - lp_rollout)``;
* TIS: ``w = min(rho, C)``; MIS: ``w = rho`` where ``rho <= C`` and ``0``
  (the token left out of the update) where ``rho > C``; C is the caller's
  truncation constant, ``C = +inf`` gives plain importance weights;
* tokens outside the response (mask 0, padding) get ``w = 0`` and count in
  no statistic;
* "over the cap" is decided in binary32, in log space:
  ``d = fl32(lp_train - lp_rollout) > fl32(ln C)``, with C itself a
  binary32 value and ``ln C`` taken in fp64 and rounded once (both inputs
  are binary32 log-probabilities; a decision that sets a weight to C or 0
  must not depend on how an implementation evaluates exp);
* per sequence: valid tokens, tokens over the cap, the sum of the weights,
  and the sum of ``lp_rollout - lp_train`` over valid tokens (divided by the
  valid count, the sample estimate of KL(rollout || trainer) for tokens drawn
  from the rollout policy); batch totals are the sums of these.

Weights are returned in fp64 from ``exp`` of the binary32 difference ``d``;
statistics in fp64 (counts exact).
"""

from __future__ import annotations

import math

import numpy as np

TRUNCATE = 0      # TIS
MASK = 1          # MIS


def log_cap(cap: float) -> np.float32:
    """fl32(ln C) for C > 0 (+inf for C = +inf).  C is a binary32 value (the
    constant is passed as one), so the logarithm is taken of fl32(C)."""
    c = float(np.float32(cap))
    if not c > 0:
        raise ValueError("oracle: the truncation constant must be positive")
    return np.float32(math.log(c)) if math.isfinite(c) else np.float32(np.inf)


def importance_weights(lp_train, lp_rollout, mask, cap: float, mode: int):
    """lp_train, lp_rollout: float32 [B, T]; mask: uint8 [B, T] (nonzero =
    response token).  Returns (w fp64 [B, T], row_stats fp64 [B, 4],
    totals fp64 [4]) with row_stats[b] = (valid tokens, tokens over the cap,
    sum of w, sum of lp_rollout - lp_train)."""
    lt = np.asarray(lp_train, dtype=np.float32)
    lr = np.asarray(lp_rollout, dtype=np.float32)
    valid = np.asarray(mask) != 0
    if lt.shape != lr.shape or lt.shape != valid.shape or lt.ndim != 2:
        raise ValueError("oracle: inputs must share one [B, T] shape")
    if not (np.all(np.isfinite(lt[valid])) and np.all(np.isfinite(lr[valid]))):
        raise ValueError("oracle: non-finite log-probability on a response token")
    if mode not in (TRUNCATE, MASK):
        raise ValueError("oracle: mode is TRUNCATE or MASK")
    with np.errstate(over="ignore", invalid="ignore"):
        d = (lt - lr).astype(np.float32)                 # binary32 difference
    over = valid & (d > log_cap(cap))
    with np.errstate(over="ignore"):
        rho = np.exp(d.astype(np.float64))
    if mode == TRUNCATE:
        w = np.where(over, np.float64(np.float32(cap)), rho)
    else:
        w = np.where(over, 0.0, rho)
    w = np.where(valid, w, 0.0)
    lr64 = lr.astype(np.float64)
    lt64 = lt.astype(np.float64)
    kl = np.where(valid, lr64 - lt64, 0.0)               # exact in fp64
    row = np.stack([valid.sum(axis=1).astype(np.float64),
                    over.sum(axis=1).astype(np.float64),
                    w.sum(axis=1),
                    kl.sum(axis=1)], axis=1)
    return w, row, row.sum(axis=0)
