"""Seeded synthetic inputs for the 8-bit rollout hot path.

This module only draws inputs.  It holds none of the method's arithmetic (no
amax, no scale, no e4m3/int8 code, no GEMM): both the CPU oracle's tests and
the GPU path's tests and benchmark take their inputs from here, so the two
sides are compared on identical bits.

Recipe (the pages fix none of it; they speak of 7B/32B-class policies whose
weights change every step, of small-batch long-tail decode and of prefill
batches of up to 16,384 tokens):

* generator: numpy PCG64 ``default_rng([seed, stream])``, one stream per
  tensor, ``standard_normal`` drawn in float32;
* weights ``Wt`` ~ N(0, 0.02) (sigma = 0.02), stored ``[N, K]`` row-major
  (output channels x input features, K contiguous);
* activations ``A`` ~ N(0, 1), ``[M, K]``; for the decode and prefill shapes
  ``round(0.01 K)`` columns, chosen without replacement by a separate stream,
  are multiplied by 20 (outlier channels) before rounding;
* every value is rounded float32 -> bfloat16 with round-to-nearest-even and
  returned as raw ``uint16`` bit patterns.

The layer shapes stand in for the real Qwen2.5-7B / 32B-class models and RL
datasets that the pages measure on; none of those is needed here.
"""

from __future__ import annotations

import numpy as np

# Stream ids: one independent PCG64 stream per tensor of a workload.
_STREAMS = {
    "A": 1, "W": 2, "A_down": 3, "W_down": 4, "A_cols": 5, "A_down_cols": 6,
    "q": 11, "k": 12, "v": 13, "o": 14, "gate": 15, "up": 16, "down": 17,
    "special": 21,
    "kv_K": 31, "kv_V": 32, "kv_K_cols": 33, "kv_V_cols": 34, "kv_slots": 35,
    "moe_A": 41, "moe_A_cols": 42, "moe_route": 43, "moe_W": 100,
    "tis_len": 51, "tis_lr": 52, "tis_d": 53, "tis_tail": 54,
    "att_q": 61, "att_len": 62, "att_pages": 63, "att_codes": 64,
}

# Mixture-of-experts decode layer (a 30B-A3B-class model: 128 experts, top-8
# routing, expert up/gate N = 2 x 768, hidden K = 2048), 128 decoding tokens.
MOE_DECODE = dict(E=128, topk=8, tokens=128, N=1536, K=2048)

# Decode attention over an FP8 KV cache of a 32B-class layer (40 query heads,
# 8 KV heads of 128), 64 sequences of 1024-8192 cached tokens, 16-slot pages.
ATT_32B = dict(B=64, Hq=40, Hkv=8, D=128, page=16, min_len=1024, max_len=8192)

# Rollout-correction batch: 1024 responses of up to 8192 tokens, truncation
# constant 2.
TIS_BATCH = dict(B=1024, T=8192, cap=2.0)

# FP8 KV cache of a 32B-class layer: 8 KV heads of 128 (C = 1024 per token),
# a prefill batch of 16,384 tokens written into a cache of 65,536 slots in
# 16-slot pages.
KV_32B = dict(T=16384, C=1024, num_slots=65536, page=16)

# Layer shapes as Wt [N, K] of one 32B-class decoder layer (hidden 5120,
# 8 KV heads of 128, FFN 27648).
STACK_32B = (
    ("q", 5120, 5120),
    ("k", 1024, 5120),
    ("v", 1024, 5120),
    ("o", 5120, 5120),
    ("gate", 27648, 5120),
    ("up", 27648, 5120),
    ("down", 5120, 27648),
)

DECODE_SWEEP_M = (1, 2, 4, 8, 32, 128)

# Named workloads.  "gemms" lists (M, N, K, outliers) GEMM problems.
CONFIGS = {
    "tiny": dict(gemms=[(16, 256, 256, False)]),
    "decode7b_upgate": dict(gemms=[(64, 37888, 3584, True)]),
    "decode32b_sweep": dict(gemms=[(m, 27648, 5120, True) for m in DECODE_SWEEP_M]),
    "prefill32b": dict(gemms=[(8192, 27648, 5120, True), (8192, 5120, 27648, True)]),
    "stack32b_requant": dict(layers=STACK_32B, gemm_m=64),
    "kv32b_prefill": dict(kv=KV_32B),
    "moe_decode": dict(moe=MOE_DECODE),
}


def _rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), _STREAMS[stream]])


def _rng_expert(seed: int, e: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), _STREAMS["moe_W"], int(e)])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def outlier_columns(K: int, seed: int, stream: str = "A_cols") -> np.ndarray:
    """The round(0.01 K) activation columns that carry x20 outliers."""
    n = int(round(0.01 * K))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed, stream).choice(K, size=n, replace=False))


def bf16_normal(shape, sigma: float, seed: int, stream: str,
                outlier_cols: np.ndarray | None = None) -> np.ndarray:
    """N(0, sigma^2) draws rounded to bf16 bits; optional x20 columns."""
    x = _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if outlier_cols is not None and len(outlier_cols):
        x[..., outlier_cols] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


def weight(N: int, K: int, seed: int = 0, stream: str = "W") -> np.ndarray:
    """Wt [N, K] bf16 bits, N(0, 0.02)."""
    return bf16_normal((N, K), 0.02, seed, stream)


def activation(M: int, K: int, seed: int = 0, outliers: bool = True,
               stream: str = "A") -> np.ndarray:
    """A [M, K] bf16 bits, N(0, 1), optionally with x20 outlier columns."""
    cols = outlier_columns(K, seed, stream + "_cols") if outliers else None
    return bf16_normal((M, K), 1.0, seed, stream, cols)


def gemm_problem(M: int, N: int, K: int, outliers: bool, seed: int = 0,
                 down: bool = False) -> dict:
    """The bf16 inputs of one linear layer: A [M, K] and Wt [N, K]."""
    a_stream, w_stream = ("A_down", "W_down") if down else ("A", "W")
    return dict(A=activation(M, K, seed, outliers, a_stream),
                Wt=weight(N, K, seed, w_stream), M=M, N=N, K=K)


def decode_sweep(seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """32B decode sweep: one W draw and the M = 128 activation draw; the
    problem at batch M uses the first M rows of that draw."""
    Mmax = max(DECODE_SWEEP_M)
    A = activation(Mmax, 5120, seed, True, "A")
    Wt = weight(27648, 5120, seed, "W")
    return A, Wt


def stack_layer(name: str, seed: int = 0) -> np.ndarray:
    """One weight of the 32B-class layer stack, Wt [N, K] bf16 bits."""
    for lname, N, K in STACK_32B:
        if lname == name:
            return weight(N, K, seed, name)
    raise KeyError(name)


def special_values_bf16() -> np.ndarray:
    """Every finite bf16 bit pattern (65,536 minus the 512 inf/NaN codes)."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (allbits >> np.uint16(7)) & np.uint16(0xFF)
    return allbits[exp != 0xFF]


def kv_rows(T: int, C: int, seed: int = 0, which: str = "K") -> np.ndarray:
    """New K or V rows [T, C] bf16 bits: N(0, 1) with x20 outlier channels
    (the activation recipe; projection outputs carry outlier channels)."""
    return activation(T, C, seed, True, "kv_" + which)


def kv_slot_mapping(T: int, num_slots: int, page: int = 16, seed: int = 0,
                    pad_every: int = 0) -> np.ndarray:
    """int64 [T]: token t goes to slot page_order[t // page] * page + t % page
    for a random order of the cache's pages (paged-cache style); with
    pad_every > 0, every pad_every-th token is a padding token (slot -1)."""
    pages = num_slots // page
    need = -(-T // page)
    if need > pages:
        raise ValueError("cache too small for T tokens")
    order = _rng(seed, "kv_slots").permutation(pages)[:need]
    t = np.arange(T, dtype=np.int64)
    slots = order[t // page].astype(np.int64) * page + t % page
    if pad_every > 0:
        slots[::pad_every] = -1
    return slots


def moe_routing(tokens: int, E: int, topk: int, seed: int = 0) -> np.ndarray:
    """Expert counts [E] of a batch: each token picks topk distinct experts
    uniformly at random (a synthetic router), so the counts vary around
    tokens * topk / E and some experts may get none."""
    rng = _rng(seed, "moe_route")
    picks = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(tokens)])
    return np.bincount(picks.ravel(), minlength=E).astype(np.int64)


def moe_problem(counts, N: int, K: int, seed: int = 0) -> dict:
    """bf16 inputs of a grouped layer: A [sum(counts), K] (rows sorted by
    expert, activation recipe), one weight Wt_e [N, K] per expert, and the
    row offsets [E + 1]."""
    counts = np.asarray(counts, dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    cols = outlier_columns(K, seed, "moe_A_cols")
    A = bf16_normal((M, K), 1.0, seed, "moe_A", cols)
    Wt = np.stack([f32_to_bf16_bits(_rng_expert(seed, e).standard_normal((N, K), dtype=np.float32)
                                    * np.float32(0.02)) for e in range(len(counts))])
    return dict(A=A, Wt=Wt, offsets=offsets, M=M, N=N, K=K)


def tis_batch(B: int, T: int, seed: int = 0) -> dict:
    """Per-token log-probabilities of a batch of B responses padded to T:
    response lengths uniform in [max(1, T/8), T]; the rollout policy's
    log-probability of each sampled token is -Exp(0.3) (mostly confident
    tokens, a tail of unlikely ones, floored at -30); the trainer's differs
    by N(0, 0.02) on 99% of the tokens and by N(0, 1) on the other 1% (the
    precision mismatch and its tail).  Padding holds zeros.  float32 [B, T]
    x 2 and the uint8 response mask."""
    lens = _rng(seed, "tis_len").integers(max(1, T // 8), T + 1, size=B)
    mask = (np.arange(T)[None, :] < lens[:, None]).astype(np.uint8)
    lr = -_rng(seed, "tis_lr").exponential(0.3, size=(B, T))
    lr = np.maximum(lr, -30.0).astype(np.float32)
    r = _rng(seed, "tis_d")
    d = r.standard_normal((B, T), dtype=np.float32) * np.float32(0.02)
    tail = _rng(seed, "tis_tail").random((B, T)) < 0.01
    d = np.where(tail, r.standard_normal((B, T), dtype=np.float32), d).astype(np.float32)
    lt = (lr + d).astype(np.float32)
    lr = np.where(mask != 0, lr, np.float32(0)).astype(np.float32)
    lt = np.where(mask != 0, lt, np.float32(0)).astype(np.float32)
    return dict(lp_train=lt, lp_rollout=lr, mask=mask)


def att_lengths(B: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Cached tokens per sequence, uniform in [lo, hi] (the length mix of
    long outputs)."""
    return _rng(seed, "att_len").integers(lo, hi + 1, size=B).astype(np.int32)


def att_block_table(seq_lens, page: int, seed: int = 0) -> tuple[np.ndarray, int]:
    """A block table [B, max_blocks] int32 that gives every sequence its own
    pages, taken from one seeded random permutation of the whole pool;
    returns (table, num_slots).  Unused entries hold -1."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    need = (lens + page - 1) // page
    total = int(need.sum())
    perm = _rng(seed, "att_pages").permutation(max(total, 1)).astype(np.int32)
    mb = int(max(1, need.max() if len(need) else 1))
    table = np.full((len(lens), mb), -1, dtype=np.int32)
    pos = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[pos:pos + k]
        pos += int(k)
    return table, max(total, 1) * page


def att_query(B: int, Hq: int, D: int, seed: int = 0) -> np.ndarray:
    """The new token's queries, bf16 [B, Hq, D] (activation recipe, no
    outlier channels)."""
    return bf16_normal((B, Hq * D), 1.0, seed, "att_q").reshape(B, Hq, D)


def att_random_codes(num_slots: int, C: int, seed: int = 0) -> np.ndarray:
    """Cache contents for timing: uniform random finite e4m3 codes (every
    byte but the two NaN codes), uint8 [num_slots, C]."""
    r = _rng(seed, "att_codes").integers(0, 254, size=(num_slots, C), dtype=np.uint8)
    return np.where(r >= 0x7F, r + 1, r).astype(np.uint8)    # skip 0x7F; 0xFF is never drawn
