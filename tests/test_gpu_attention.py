"""GPU parity of fp8_kv_decode_attention (the one-pass kernel, workspace
None) and fp8_kv_decode_attention_ws (the batch split over the CUs, with the
workspace the library asks for) against the oracle.

Each case builds a paged FP8 cache with the oracle (K and V rows of the
activation recipe, per-tensor scales, codes), a random block table and a
length mix, runs the kernel, and compares every output with the oracle's
fp64 result rounded once to bf16: relative Frobenius error <= 1e-3 over the
batch, and element by element within two bf16 roundings plus 1e-3 of the
output's rms.  Cases: group sizes 1 to 8, lengths 0, 1, a partial page and
several thousand tokens, page sizes 16 and 5, tokens skipped through
invalid block-table entries, lengths beyond the table (clamped), and the
32B-class layout (40 query heads over 8 KV heads) on all of the full
64-sequence batch; for the split: one long sequence cut over every
CU, hundreds of short sequences sharing workgroups, the most sequences it
takes (2048), one-token pages with a workgroup range of more than 1024
pages (its page table staged in several chunks), shapes it does not take
(more than 8 KV heads, more than 2048 sequences, a workspace too small),
and bitwise-repeatable results.
"""

import functools
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import attention, kv
from oracle.gemm import bf16_bits_to_f64, rel_frobenius
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import announce, bits_to_dev, host, oracle_workers

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


WS = ["auto", None]     # the split with the library's workspace; the one-pass kernel


def _gpu(p, ws="auto"):
    f = lambda x: torch.tensor([x], dtype=torch.float32, device="cuda:0")
    B, Hq, D = p["q"].shape
    out = binding.fp8_kv_decode_attention(
        bits_to_dev(p["q"].reshape(B, -1)).view(B, Hq, D), f(p["sq"]), _dev(p["kc"]),
        _dev(p["vc"]), f(p["sk"]), f(p["sv"]), _dev(p["table"]), _dev(p["lens"]), p["Hkv"],
        p["page"], workspace=ws)
    return host(out)


def _check(got, p, label, ref=None):
    if ref is None:
        ref = attention.decode_attention(p["q"], p["sq"], p["kc"], p["vc"], p["sk"], p["sv"],
                                         p["table"], p["lens"], p["Hkv"], p["page"])
    g = got
    err = rel_frobenius(g, ref)
    assert err <= TOL, f"{label}: relative Frobenius error {err:.3e}"
    gf, rf = bf16_bits_to_f64(g), bf16_bits_to_f64(ref)
    rms = np.sqrt(np.mean(rf * rf)) if rf.size else 0.0
    bad = np.abs(gf - rf) > 2.0 ** -7 * np.abs(rf) + 1e-3 * rms
    assert not bad.any(), f"{label}: {int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (12, 4), (8, 2), (10, 2), (12, 2),
                                    (14, 2), (8, 1), (40, 8), (24, 3), (35, 5), (18, 6),
                                    (14, 7), (36, 12)])
def test_group_sizes(Hq, Hkv, ws):
    p = _build(3, Hq, Hkv, [37, 300, 1], 16, seed=Hq + Hkv)
    announce(f"fp8_kv_decode_attention Hq{Hq} Hkv{Hkv} workspace {ws}")
    _check(_gpu(p, ws), p, f"Hq{Hq} Hkv{Hkv}")


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("lens,page", [([0, 1, 15, 16, 17], 16), ([33, 3000, 5], 5),
                                       ([4100, 31, 64], 16), ([1, 1, 1, 2], 1),
                                       ([0, 0, 0], 16)])
def test_lengths_and_pages(lens, page, ws):
    p = _build(len(lens), 10, 2, lens, page, seed=sum(lens))
    announce(f"fp8_kv_decode_attention lens {lens} page {page} workspace {ws}")
    _check(_gpu(p, ws), p, f"lens {lens} page {page}")


def test_one_long_sequence_over_every_cu():
    # 9000 tokens of one sequence: ~36 per workgroup, ranges starting inside
    # pages (page 7), every KV head of the 32B layout
    p = _build(1, 40, 8, [9000], 7, seed=5)
    announce("fp8_kv_decode_attention_ws one sequence of 9000 tokens")
    _check(_gpu(p, "auto"), p, "one long sequence")


def test_many_short_sequences_share_workgroups():
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 40, size=300).astype(np.int32)
    lens[::7] = 0
    p = _build(300, 16, 4, lens, 16, seed=7)
    announce("fp8_kv_decode_attention_ws 300 short sequences")
    _check(_gpu(p, "auto"), p, "300 short sequences")


def test_split_not_taken_falls_back():
    # more than 8 KV heads (one wave each would not do); more than 2048
    # sequences; a workspace below the size asked for: all run the one-pass
    # kernel
    assert binding.attention_workspace_bytes(4, 36, 12, 128) == 0
    assert binding.attention_workspace_bytes(4, 12, 3, 128) > 0
    assert binding.attention_workspace_bytes(2049, 8, 2, 128) == 0
    n = binding.attention_workspace_bytes(3, 10, 2, 128)
    assert n > 0
    p = _build(3, 10, 2, [50, 700, 3], 16, seed=21)
    small = torch.empty((n - 16,), dtype=torch.uint8, device="cuda:0")
    announce("fp8_kv_decode_attention_ws workspace too small")
    _check(_gpu(p, small), p, "workspace too small")
    lens = np.full(2100, 3, dtype=np.int32)
    q = _build(2100, 8, 2, lens, 4, seed=2)
    announce("fp8_kv_decode_attention_ws 2100 sequences")
    _check(_gpu(q, "auto"), q, "2100 sequences")


def test_split_is_bitwise_repeatable():
    p = _build(5, 40, 8, [3000, 10, 2047, 0, 513], 16, seed=9)
    announce("fp8_kv_decode_attention_ws repeated")
    a, b = _gpu(p, "auto"), _gpu(p, "auto")
    assert np.array_equal(a, b)
    _check(a, p, "repeatable")


@pytest.mark.parametrize("ws", WS)
def test_skipped_tokens_and_clamped_lengths(ws):
    p = _build(3, 8, 2, [40, 40, 40], 8, seed=11)
    # sequence 0: one page entry negative, sequence 1: one past the cache;
    # the oracle is given the same tokens removed (their page dropped)
    num_slots = p["kc"].shape[0]
    t = p["table"].copy()
    t[0, 1] = -3
    t[1, 2] = num_slots // 8 + 5
    q = dict(p, table=t)
    announce(f"fp8_kv_decode_attention skipped tokens workspace {ws}")
    got = _gpu(q, ws)
    for b, drop in ((0, 1), (1, 2)):
        keep_pages = [pg for i, pg in enumerate(p["table"][b, :5]) if i != drop]
        ref_table = np.array([keep_pages], dtype=np.int32)
        r = dict(p, q=p["q"][b:b + 1], table=ref_table, lens=np.array([32], np.int32))
        _check(got[b:b + 1], r, f"skipped page of sequence {b}")
    # lengths beyond max_blocks * page are clamped to it
    c = dict(p, lens=np.array([40, 500, 41], np.int32))
    got = _gpu(c, ws)
    _check(got, dict(p, lens=np.array([40, 40, 40], np.int32)), "clamped lengths")


@functools.lru_cache(maxsize=1)
def _full_32b_case():
    """The 64-sequence 32B-class batch and the oracle's output for all of
    it, computed once for both launch forms: sequences in pairs on worker
    threads (each pair's output depends on that pair alone)."""
    cfg = workloads.ATT_32B
    B, Hq, Hkv, D, page = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page"]
    lens = workloads.att_lengths(B, cfg["min_len"], cfg["max_len"], 0)
    table, num_slots = workloads.att_block_table(lens, page, 0)
    q = workloads.att_query(B, Hq, D, 0)
    kc = workloads.att_random_codes(num_slots, Hkv * D, 0)
    vc = workloads.att_random_codes(num_slots, Hkv * D, 1)
    # scales that keep the scores of random codes in a softmax-relevant range
    p = dict(q=q, sq=kv.kv_scale(q), kc=kc, vc=vc, sk=np.float32(2.0 ** -12),
             sv=np.float32(2.0 ** -8), table=table, lens=lens, Hkv=Hkv, page=page)
    pairs = [list(range(b, min(B, b + 2))) for b in range(0, B, 2)]
    with ThreadPoolExecutor(oracle_workers()) as ex:
        parts = list(ex.map(lambda rows: attention.decode_attention(
            q, p["sq"], kc, vc, p["sk"], p["sv"], table, lens, Hkv, page, batch_rows=rows),
            pairs))
    return p, np.concatenate(parts, axis=0), num_slots


@pytest.mark.parametrize("ws", WS)
def test_full_32b_batch(ws):
    p, ref, num_slots = _full_32b_case()
    B = p["q"].shape[0]
    announce(f"fp8_kv_decode_attention full 32B batch B{B} slots{num_slots} workspace {ws}")
    got = _gpu(p, ws)
    _check(got, p, "32B batch", ref=ref)


def test_split_at_most_sequences():
    lens = np.full(2048, 3, dtype=np.int32)
    lens[::5] = 0
    p = _build(2048, 8, 2, lens, 4, seed=2)
    assert binding.attention_workspace_bytes(2048, 8, 2, 128) > 0
    announce("fp8_kv_decode_attention_ws 2048 sequences")
    _check(_gpu(p, "auto"), p, "2048 sequences")


def test_split_long_ranges_of_one_token_pages():
    # 270,000 tokens over the CUs: more than 1024 one-token pages per
    # workgroup, so each range's page table is staged in several chunks
    p = _build(2, 2, 1, [140000, 130000], 1, seed=13)
    announce("fp8_kv_decode_attention_ws 270,000 tokens in one-token pages")
    _check(_gpu(p, "auto"), p, "one-token pages")
