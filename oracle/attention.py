"""Decode attention over an FP8 KV cache (CPU oracle).  TEST INFRASTRUCTURE
ONLY (see the package header).

"FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
Learning", abstract, item (ii): the KV cache is kept in FP8, with the Q, K
and V scales recalibrated every step, to remove the memory bottleneck of
long contexts.  The pages describe no attention kernel; the readings taken
here (with those of ``oracle.kv`` for the cache itself):

* one new token per sequence (decode); its query has Hq heads of D values,
  the cache Hkv heads (grouped-query attention: query head h reads cache
  head h // (Hq / Hkv));
* a Q scale implies that the query, too, is quantized per tensor:
  ``q^ = E4M3_sat_RNE(fl32(q / s_q))`` (the cache's encode, scale from
  ``kv_scale``); K and V are the cache's codes with their scales;
* score of cached token t: ``s_q s_k c (D(q^) . D(k^_t))`` with c the
  softmax scale (1 / sqrt(D) unless the caller gives another); weights
  ``softmax`` over the sequence's ``len`` cached tokens (the new token's K
  and V are written to the cache before the read);
* output ``s_v sum_t p_t D(v^_t)``, rounded once to bf16; a sequence with no
  cached token gives zeros;
* the cache is paged: token t of sequence b is in slot
  ``block_table[b, t // page] * page + t % page``.

Everything after the codes is fp64 (the dot products of decoded e4m3 values
are exact in fp64).
"""

from __future__ import annotations

import numpy as np

from . import e4m3
from .gemm import round_bf16
from .kv import kv_encode_rows


def quantize_query(q_bits, s_q) -> np.ndarray:
    """bf16 [B, Hq, D] -> e4m3 codes (per-tensor scale s_q)."""
    q = np.asarray(q_bits, dtype=np.uint16)
    return kv_encode_rows(q.reshape(q.shape[0], -1), np.float32(s_q)).reshape(q.shape)


def token_slots(block_table, seq_len: int, b: int, page: int) -> np.ndarray:
    t = np.arange(seq_len)
    return np.asarray(block_table)[b, t // page].astype(np.int64) * page + t % page


def decode_attention_f64(q_bits, s_q, k_cache, v_cache, s_k, s_v, block_table, seq_lens,
                         Hkv: int, page: int, softmax_scale: float | None = None,
                         batch_rows=None) -> np.ndarray:
    """q_bits bf16 [B, Hq, D]; k_cache, v_cache e4m3 codes [num_slots, Hkv * D];
    block_table int [B, max_blocks]; seq_lens int [B].  Returns the fp64
    result [len(batch_rows), Hq, D] for the sequences batch_rows (default:
    all), before the bf16 rounding."""
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    B, Hq, D = q_bits.shape
    if Hq % Hkv != 0:
        raise ValueError("oracle: Hq must be a multiple of Hkv")
    grp = Hq // Hkv
    c = np.float32(1.0 / np.sqrt(D)) if softmax_scale is None else np.float32(softmax_scale)
    qc = e4m3.decode(quantize_query(q_bits, s_q))                 # [B, Hq, D] fp64
    sqk = float(np.float32(s_q)) * float(np.float32(s_k)) * float(c)
    sv = float(np.float32(s_v))
    rows = range(B) if batch_rows is None else batch_rows
    out = np.zeros((len(rows), Hq, D))
    for i, b in enumerate(rows):
        n = int(seq_lens[b])
        if n == 0:
            continue
        slots = token_slots(block_table, n, b, page)
        kd = e4m3.decode(np.asarray(k_cache)[slots]).reshape(n, Hkv, D)
        vd = e4m3.decode(np.asarray(v_cache)[slots]).reshape(n, Hkv, D)
        for h in range(Hq):
            kh = h // grp
            s = (kd[:, kh, :] @ qc[b, h]) * sqk                    # [n]
            p = np.exp(s - s.max())
            p /= p.sum()
            out[i, h] = sv * (p @ vd[:, kh, :])
    return out


def decode_attention(q_bits, s_q, k_cache, v_cache, s_k, s_v, block_table, seq_lens,
                     Hkv: int, page: int, softmax_scale: float | None = None,
                     batch_rows=None) -> np.ndarray:
    """As decode_attention_f64, rounded once to bf16 bits."""
    return round_bf16(decode_attention_f64(q_bits, s_q, k_cache, v_cache, s_k, s_v, block_table,
                                           seq_lens, Hkv, page, softmax_scale, batch_rows))
