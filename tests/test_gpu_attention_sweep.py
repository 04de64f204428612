"""A seeded sweep of FP8-KV decode attention configurations against the
fp64 CPU oracle through the C ABI, on both launch forms (the split with the
library's workspace and the one-pass kernel).

The fixed cases elsewhere pin the 32B layer, group sizes and chosen length
patterns; this sweep draws 16 configurations (seed 11): KV heads 1-8 and
12, 1-8 query heads per KV head, 1-24 sequences whose lengths mix empty,
short and up-to-3000-token sequences, and page sizes from 1 to 256 tokens.
The bar is the one test_gpu_attention.py uses (relative Frobenius error at
most 1e-3 against the oracle's bf16 output, every element within 2^-7 of
itself plus 1e-3 of the rms).
"""

import numpy as np
import pytest

from tests.gpu_util import announce
from tests.test_gpu_attention import WS, _build, _check, _gpu

pytestmark = pytest.mark.gpu


def _configs(seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(16):
        Hkv = int(rng.choice([1, 2, 4, 8, 12]))
        G = int(rng.integers(1, 9))
        B = int(rng.integers(1, 25))
        kinds = rng.integers(0, 4, size=B)
        lens = [0 if k == 0 else int(rng.integers(1, 40)) if k == 1
                else int(rng.integers(40, 700)) if k == 2 else int(rng.integers(700, 3001))
                for k in kinds]
        page = int(rng.choice([1, 5, 16, 32, 64, 128, 256]))
        out.append((Hkv * G, Hkv, tuple(lens), page, i))
    return out


CONFIGS = _configs(11)


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("Hq,Hkv,lens,page,i", CONFIGS)
def test_attention_sweep(Hq, Hkv, lens, page, i, ws):
    announce(f"fp8_kv_decode_attention sweep #{i}: Hq{Hq} Hkv{Hkv} B{len(lens)} "
             f"tokens {sum(lens)} page {page} workspace {ws}")
    p = _build(len(lens), Hq, Hkv, list(lens), page, seed=100 + i)
    _check(_gpu(p, ws), p, f"sweep #{i}")
