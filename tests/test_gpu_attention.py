"""GPU parity of fp8_kv_decode_attention against the oracle.

Each case builds a paged FP8 cache with the oracle (K and V rows of the
activation recipe, per-tensor scales, codes), a random block table and a
length mix, runs the kernel, and compares every output with the oracle's
fp64 result rounded once to bf16: relative Frobenius error <= 1e-3 over the
batch, and element by element within two bf16 roundings plus 1e-3 of the
output's rms.  Cases: group sizes 1 to 8, lengths 0, 1, a partial page and
several thousand tokens, page sizes 16 and 5, tokens skipped through
invalid block-table entries, lengths beyond the table (clamped), and the
32B-class layout (40 query heads over 8 KV heads) on sampled sequences of
the full 64-sequence batch.
"""

import numpy as np
import pytest
import torch

from oracle import attention, kv
from oracle.gemm import bf16_bits_to_f64, rel_frobenius
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import announce, bits_to_dev, host

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _build(B, Hq, Hkv, lens, page, seed, D=128):
    lens = np.asarray(lens, dtype=np.int32)
    table, num_slots = workloads.att_block_table(lens, page, seed)
    q = workloads.att_query(B, Hq, D, seed)
    kb = workloads.kv_rows(num_slots, Hkv * D, seed, "K")
    vb = workloads.kv_rows(num_slots, Hkv * D, seed, "V")
    sk, sv, sq = kv.kv_scale(kb), kv.kv_scale(vb), kv.kv_scale(q)
    return dict(q=q, sq=sq, kc=kv.kv_encode_rows(kb, sk), vc=kv.kv_encode_rows(vb, sv), sk=sk,
                sv=sv, table=table, lens=lens, Hkv=Hkv, page=page)


def _gpu(p):
    f = lambda x: torch.tensor([x], dtype=torch.float32, device="cuda:0")
    B, Hq, D = p["q"].shape
    out = binding.fp8_kv_decode_attention(
        bits_to_dev(p["q"].reshape(B, -1)).view(B, Hq, D), f(p["sq"]), _dev(p["kc"]),
        _dev(p["vc"]), f(p["sk"]), f(p["sv"]), _dev(p["table"]), _dev(p["lens"]), p["Hkv"],
        p["page"])
    return host(out)


def _check(got, p, label, rows=None):
    ref = attention.decode_attention(p["q"], p["sq"], p["kc"], p["vc"], p["sk"], p["sv"],
                                     p["table"], p["lens"], p["Hkv"], p["page"],
                                     batch_rows=rows)
    g = got if rows is None else got[rows]
    err = rel_frobenius(g, ref)
    assert err <= TOL, f"{label}: relative Frobenius error {err:.3e}"
    gf, rf = bf16_bits_to_f64(g), bf16_bits_to_f64(ref)
    rms = np.sqrt(np.mean(rf * rf)) if rf.size else 0.0
    bad = np.abs(gf - rf) > 2.0 ** -7 * np.abs(rf) + 1e-3 * rms
    assert not bad.any(), f"{label}: {int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (12, 4), (8, 2), (10, 2), (12, 2),
                                    (14, 2), (8, 1)])
def test_group_sizes(Hq, Hkv):
    p = _build(3, Hq, Hkv, [37, 300, 1], 16, seed=Hq + Hkv)
    announce(f"fp8_kv_decode_attention Hq{Hq} Hkv{Hkv}")
    _check(_gpu(p), p, f"Hq{Hq} Hkv{Hkv}")


@pytest.mark.parametrize("lens,page", [([0, 1, 15, 16, 17], 16), ([33, 3000, 5], 5),
                                       ([4100, 31, 64], 16), ([1, 1, 1, 2], 1)])
def test_lengths_and_pages(lens, page):
    p = _build(len(lens), 10, 2, lens, page, seed=sum(lens))
    announce(f"fp8_kv_decode_attention lens {lens} page {page}")
    _check(_gpu(p), p, f"lens {lens} page {page}")


def test_skipped_tokens_and_clamped_lengths():
    p = _build(3, 8, 2, [40, 40, 40], 8, seed=11)
    # sequence 0: one page entry negative, sequence 1: one past the cache;
    # the oracle is given the same tokens removed (their page dropped)
    num_slots = p["kc"].shape[0]
    t = p["table"].copy()
    t[0, 1] = -3
    t[1, 2] = num_slots // 8 + 5
    q = dict(p, table=t)
    announce("fp8_kv_decode_attention skipped tokens")
    got = _gpu(q)
    for b, drop in ((0, 1), (1, 2)):
        keep_pages = [pg for i, pg in enumerate(p["table"][b, :5]) if i != drop]
        ref_table = np.array([keep_pages], dtype=np.int32)
        r = dict(p, q=p["q"][b:b + 1], table=ref_table, lens=np.array([32], np.int32))
        _check(got[b:b + 1], r, f"skipped page of sequence {b}")
    # lengths beyond max_blocks * page are clamped to it
    c = dict(p, lens=np.array([40, 500, 41], np.int32))
    got = _gpu(c)
    _check(got, dict(p, lens=np.array([40, 40, 40], np.int32)), "clamped lengths")


def test_full_32b_batch_sampled():
    cfg = workloads.ATT_32B
    B, Hq, Hkv, D, page = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page"]
    lens = workloads.att_lengths(B, cfg["min_len"], cfg["max_len"], 0)
    table, num_slots = workloads.att_block_table(lens, page, 0)
    announce(f"fp8_kv_decode_attention full 32B batch B{B} slots{num_slots}")
    q = workloads.att_query(B, Hq, D, 0)
    kc = workloads.att_random_codes(num_slots, Hkv * D, 0)
    vc = workloads.att_random_codes(num_slots, Hkv * D, 1)
    # scales that keep the scores of random codes in a softmax-relevant range
    p = dict(q=q, sq=kv.kv_scale(q), kc=kc, vc=vc, sk=np.float32(2.0 ** -12),
             sv=np.float32(2.0 ** -8), table=table, lens=lens, Hkv=Hkv, page=page)
    got = _gpu(p)
    rows = [0, 17, 40, 63]
    _check(got, p, "32B batch", rows=rows)
