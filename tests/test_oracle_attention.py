"""Pins for the oracle's decode attention over an FP8 KV cache (CPU).

* a library route: torch's scaled_dot_product_attention in fp64 on the
  decoded, scaled query, keys and values (GQA by repeating the cache heads),
  gathered through the block table by the test itself;
* closed forms: one cached token gives s_v D(v) exactly; identical keys give
  the mean of the values; an empty sequence gives zeros;
* paging: permuting the cache's pages (and the block table with them)
  leaves every output unchanged;
* the query's codes against the brute-force nearest-code search of
  fl32(q / s_q);
* planted mistakes (query head h read against cache head h mod Hkv, a page
  index taken as a slot index, the softmax scale left out) fail the library
  route.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, e4m3, kv
from oracle.gemm import bf16_bits_to_f64
from precision_rl_rollout_amd import workloads
from tests import pins


def _problem(B, Hq, Hkv, D, lens, page, seed):
    lens = np.asarray(lens, dtype=np.int32)
    table, num_slots = workloads.att_block_table(lens, page, seed)
    q = workloads.att_query(B, Hq, D, seed)
    kb = workloads.kv_rows(num_slots, Hkv * D, seed, "K")
    vb = workloads.kv_rows(num_slots, Hkv * D, seed, "V")
    sk, sv, sq = kv.kv_scale(kb), kv.kv_scale(vb), kv.kv_scale(q)
    kc, vc = kv.kv_encode_rows(kb, sk), kv.kv_encode_rows(vb, sv)
    return dict(q=q, sq=sq, kc=kc, vc=vc, sk=sk, sv=sv, table=table, lens=lens, Hkv=Hkv,
                page=page)


def _oracle(p, f64=True, **kw):
    fn = attention.decode_attention_f64 if f64 else attention.decode_attention
    return fn(p["q"], p["sq"], p["kc"], p["vc"], p["sk"], p["sv"], p["table"], p["lens"],
              p["Hkv"], p["page"], **kw)


def _torch_route(p, softmax_scale=None, head_map=None, slot_of=None):
    B, Hq, D = p["q"].shape
    Hkv, page = p["Hkv"], p["page"]
    c = float(np.float32(1 / math.sqrt(D) if softmax_scale is None else softmax_scale))
    qd = torch.from_numpy(e4m3.decode(attention.quantize_query(p["q"], p["sq"]))) * float(p["sq"])
    kd = torch.from_numpy(e4m3.decode(p["kc"])).reshape(-1, Hkv, D) * float(p["sk"])
    vd = torch.from_numpy(e4m3.decode(p["vc"])).reshape(-1, Hkv, D) * float(p["sv"])
    out = torch.zeros((B, Hq, D), dtype=torch.float64)
    for b in range(B):
        n = int(p["lens"][b])
        if n == 0:
            continue
        t = np.arange(n)
        slots = (p["table"][b, t // page].astype(np.int64) * page + t % page) if slot_of is None \
            else slot_of(p, b, t)
        heads = (np.arange(Hq) // (Hq // Hkv)) if head_map is None else head_map(Hq, Hkv)
        k = kd[slots][:, heads, :].permute(1, 0, 2)          # [Hq, n, D]
        v = vd[slots][:, heads, :].permute(1, 0, 2)
        out[b] = torch.nn.functional.scaled_dot_product_attention(
            qd[b][:, None, :], k, v, scale=c)[:, 0, :]
    return out.numpy()


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,page", [
    (3, 8, 2, 128, [17, 1, 40], 16),
    (2, 5, 1, 64, [33, 64], 8),
    (4, 6, 6, 32, [5, 0, 130, 16], 4),
])
def test_matches_library_route(B, Hq, Hkv, D, lens, page):
    p = _problem(B, Hq, Hkv, D, lens, page, seed=B + Hq)
    assert np.allclose(_oracle(p), _torch_route(p), rtol=1e-12, atol=1e-12)


def test_single_token_and_empty():
    p = _problem(2, 4, 2, 64, [1, 0], 16, seed=3)
    out = _oracle(p)
    slot = p["table"][0, 0] * 16
    vd = e4m3.decode(p["vc"][slot]).reshape(2, 64) * float(p["sv"])
    assert np.array_equal(out[0], vd[np.arange(4) // 2])
    assert np.array_equal(out[1], np.zeros((4, 64)))


def test_identical_keys_average_the_values():
    p = _problem(1, 4, 1, 32, [50], 16, seed=4)
    slots = attention.token_slots(p["table"], 50, 0, 16)
    p["kc"][slots] = p["kc"][slots[0]]
    out = _oracle(p)
    want = (e4m3.decode(p["vc"][slots]).mean(axis=0) * float(p["sv"]))
    assert np.allclose(out[0], np.broadcast_to(want, (4, 32)), rtol=1e-13, atol=0)


def test_page_permutation_invariance():
    p = _problem(3, 4, 2, 64, [40, 7, 33], 8, seed=5)
    base = _oracle(p)
    npages = p["kc"].shape[0] // 8
    perm = np.random.default_rng(9).permutation(npages)      # new page of old page i: perm[i]
    kc2, vc2 = np.empty_like(p["kc"]), np.empty_like(p["vc"])
    for i in range(npages):
        kc2[perm[i] * 8:(perm[i] + 1) * 8] = p["kc"][i * 8:(i + 1) * 8]
        vc2[perm[i] * 8:(perm[i] + 1) * 8] = p["vc"][i * 8:(i + 1) * 8]
    t2 = np.where(p["table"] >= 0, perm[np.maximum(p["table"], 0)], -1).astype(np.int32)
    p2 = dict(p, kc=kc2, vc=vc2, table=t2)
    assert np.array_equal(_oracle(p2), base)


def test_query_codes_match_brute_force():
    q = workloads.att_query(2, 3, 16, seed=6)
    s = kv.kv_scale(q)
    codes = attention.quantize_query(q, s)
    x = pins.f32_of_bf16(q).ravel()
    from fractions import Fraction
    quo = np.array([pins.fl32(Fraction(float(v)) / Fraction(float(s))) for v in x], np.float32)
    assert np.array_equal(codes.ravel(), pins.e4m3_nearest(np.copysign(quo, x)))


def test_rounding_is_one_bf16_step():
    p = _problem(2, 4, 2, 64, [20, 9], 16, seed=7)
    f = _oracle(p)
    r = bf16_bits_to_f64(_oracle(p, f64=False))
    assert np.all(np.abs(r - f) <= 2.0 ** -8 * np.abs(f) + 1e-300)   # half a bf16 ulp


# ---------------------------------------------------------------- mutants
def test_mutants_fail_the_library_route():
    p = _problem(2, 8, 2, 64, [30, 12], 16, seed=8)
    good = _oracle(p)
    wrong_heads = _torch_route(p, head_map=lambda Hq, Hkv: np.arange(Hq) % Hkv)
    wrong_pages = _torch_route(
        p, slot_of=lambda pp, b, t: pp["table"][b, t // pp["page"]].astype(np.int64) + t % pp["page"])
    no_scale = _torch_route(p, softmax_scale=1.0)
    for bad in (wrong_heads, wrong_pages, no_scale):
        assert not np.allclose(good, bad, rtol=1e-6, atol=1e-9)
