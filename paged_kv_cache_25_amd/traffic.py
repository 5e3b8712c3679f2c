"""Algorithmic bytes and FLOPs of a decode step (host-side accounting).

The roofline numbers the library reports are algorithmic: what the method must
move and compute, not what a kernel happens to move.

* KV bytes per token: ``2 * layers * n_kv * d_h * e`` (K and V).  The serving
  lesson (learn.mohebi.ai, "KV-cache memory and the batch that fits") and the
  KV-cache posts give 131,072 B for Llama-3-8B in bf16.
* Decode-step proposition (serving lesson, "Proposition (decode step: bytes,
  FLOPs, intensity and time)"): bytes >= W + B*C*k, FLOPs ~ B*W + g*B*C*k in
  bf16, attention costs 4*C*d_h*a*L FLOPs per sequence, so g FLOP per cache
  byte (2g/e_kv for other formats).
* For one attention call (one layer) the algorithmic traffic is every
  attended token's K and V row of every KV head, plus the queries, the
  outputs, the block-table entries walked, the context lengths and, for e4m3,
  one float32 scale per (block, kv head) for K and for V.  Partial results of
  a split-KV launch and the unread tail of a sequence's last block are
  implementation overhead and are not counted.
"""

from __future__ import annotations

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}

# MI355X published peaks used for roofline fractions.
HBM_PEAK_GBPS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3


def kv_bytes_per_token(layers: int, n_kv: int, d_h: int, e: float) -> float:
    """K and V bytes one token adds to the cache over all layers."""
    return 2 * layers * n_kv * d_h * e


def blocks_needed(n_tokens, block_size: int):
    """Whole blocks a sequence of n tokens occupies: ceil(n / block_size)."""
    n = np.asarray(n_tokens, dtype=np.int64)
    return -(-n // block_size)


def paged_slots(live_lengths, block_size: int) -> int:
    """Token slots held by paged sequences (whole blocks allocated on demand)."""
    return int(block_size * blocks_needed(live_lengths, block_size).sum())


def decode_step_model(*, W, B, C, k, layers, a, d_h, psi, peak_flops, bw):
    """The serving lesson's decode-step roofline: bytes, FLOPs, intensity,
    memory time and compute time for batch(es) ``B`` at context ``C``."""
    B = np.asarray(B, dtype=np.float64)
    kv = B * C * k
    n_bytes = W + kv
    flops = 2 * psi * B + 4 * B * C * layers * a * d_h
    return dict(bytes=n_bytes, flops=flops, intensity=flops / n_bytes,
                t_mem=n_bytes / bw, t_comp=flops / peak_flops,
                tokens_per_s=B / np.maximum(n_bytes / bw, flops / peak_flops))


def attention_call_traffic(context_lens, *, num_q_heads, num_kv_heads, head_dim,
                           q_dtype, kv_dtype, block_size=16):
    """Algorithmic bytes and FLOPs of one paged decode-attention call (one layer).

    Returns a dict with ``kv_bytes`` (K+V rows of every attended token),
    ``total_bytes`` (plus q, out, tables, lengths, e4m3 scales) and ``flops``
    (4 * D * Hq per attended token: q.k and p.v).
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    tokens = int(ctx.sum())
    e_kv = ELEM_BYTES[kv_dtype]
    e_q = ELEM_BYTES[q_dtype]
    B = len(ctx)
    kv = tokens * 2 * num_kv_heads * head_dim * e_kv
    nblk = int(blocks_needed(ctx, block_size).sum())
    scales = nblk * num_kv_heads * 4 * 2 if kv_dtype == "fp8_e4m3" else 0
    qo = 2 * B * num_q_heads * head_dim * e_q
    tables = 4 * nblk + 4 * B
    return dict(tokens=tokens, kv_bytes=kv, scale_bytes=scales, qo_bytes=qo,
                table_bytes=tables, total_bytes=kv + scales + qo + tables,
                flops=4 * head_dim * num_q_heads * tokens)


def append_traffic(num_seqs, *, num_kv_heads, head_dim, kv_dtype):
    """Bytes the append moves: each new K and V row read once and written once."""
    row = num_kv_heads * head_dim * ELEM_BYTES[kv_dtype]
    return dict(bytes=num_seqs * row * 2 * 2)


def multi_query_traffic(context_lens, new_tokens, *, num_q_heads, num_kv_heads, head_dim,
                        q_dtype, kv_dtype, block_size=16):
    """Algorithmic bytes and FLOPs of one multi-token attention call: sequence b
    brings new_tokens[b] queries that share one read of its ctx_b cached K/V
    rows (the newest sees them all, and the others a prefix of them).  Bytes:
    those rows, q and out of every new token, the tables and lengths (and the
    query offsets); FLOPs: 4 * D * Hq per (query, visible token) pair, where
    query j of t sees ctx - t + j + 1 tokens."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    t = np.asarray(new_tokens, dtype=np.int64)
    base = attention_call_traffic(ctx, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                                  head_dim=head_dim, q_dtype=q_dtype, kv_dtype=kv_dtype,
                                  block_size=block_size)
    rows = int(t.sum())
    qo = 2 * rows * num_q_heads * head_dim * ELEM_BYTES[q_dtype]
    tables = base["table_bytes"] + 4 * (len(ctx) + 1)
    # sum over j < t of max(ctx - t + j + 1, 0)
    pairs = 0
    for c, n in zip(ctx.tolist(), t.tolist()):
        pairs += sum(max(c - n + j + 1, 0) for j in range(n))
    return dict(tokens=base["tokens"], rows=rows, kv_bytes=base["kv_bytes"],
                scale_bytes=base["scale_bytes"], qo_bytes=qo, table_bytes=tables,
                total_bytes=base["kv_bytes"] + base["scale_bytes"] + qo + tables,
                flops=4 * head_dim * num_q_heads * pairs)


def quant_append_traffic(num_rows, *, num_kv_heads, head_dim, new_dtype):
    """Bytes quantise-on-append must move in fixed-scale mode: each new K and V
    row read in its input dtype, its e4m3 codes written, and the slice's scale
    read.  (A running-amax append that grows a scale also rewrites the slice's
    earlier rows: up to 15 more code rows read and written.)"""
    row = num_kv_heads * head_dim
    per = 2 * (row * ELEM_BYTES[new_dtype] + row + num_kv_heads * 4)
    return dict(bytes=num_rows * per)


def mla_numbers_per_token(kv_lora_rank: int, rope_dim: int) -> int:
    """Numbers an MLA layer caches per token: the latent plus the shared rotary key."""
    return kv_lora_rank + rope_dim


def mla_attention_traffic(context_lens, *, num_heads, kv_lora_rank, rope_dim, dtype="bf16",
                          block_size=16):
    """Algorithmic bytes and FLOPs of one absorbed MLA decode-attention call.
    Bytes: every attended token's one shared row (d_c + d_r numbers), the
    absorbed queries, the latent outputs, table entries and lengths.  FLOPs:
    per token and head, 2 (d_c + d_r) for the score and 2 d_c for the
    weighted sum of latents."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    tokens = int(ctx.sum())
    e = ELEM_BYTES[dtype]
    d = kv_lora_rank + rope_dim
    B = len(ctx)
    kv = tokens * d * e
    nblk = int(blocks_needed(ctx, block_size).sum())
    qo = B * num_heads * (d + kv_lora_rank) * e
    tables = 4 * nblk + 4 * B
    return dict(tokens=tokens, kv_bytes=kv, qo_bytes=qo, table_bytes=tables,
                total_bytes=kv + qo + tables,
                flops=tokens * num_heads * 2 * (d + kv_lora_rank))
