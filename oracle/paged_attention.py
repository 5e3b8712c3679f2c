"""CPU float64 oracle: one decode step of attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library's
product path never calls it, and it shares no code with the HIP kernels.

What it computes, written out plainly and slowly from the pages:

* Storage formats are decoded from their bits (bfloat16 = the top half of a
  float32; OCP float8 e4m3fn = 1 sign, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals at exponent 0, the all-ones codes are NaN).  Each
  decoded e4m3 value is multiplied by its (block, kv head) float32 scale; the
  product is exact in float64.

* ``kv_append``: the new token's key and value go to position ``ctx - 1`` of
  its sequence: logical block ``(ctx - 1) // block_size`` looked up in the
  block table, slot ``(ctx - 1) % block_size`` of that physical block, for
  every KV head.  (KV-cache post, "A toy vLLM": the locker/shelf addressing of
  ``write_kv``; brunomaga.github.io inference post, "PagedAttention: memory
  management for the KV cache", ``PagedKVCache.append``.)  ``ctx`` counts the
  appended token: the appended key is attended in the same step (KV-cache
  post, "Prefill and decode": the token's own K/V are appended first).

* ``gather_sequence``: follow the block table in logical order, take each
  block's rows, line the slots up and drop the slots at or beyond ``ctx``
  (``read_kv`` in the toy vLLM; the padded gather of ``paged_decode_attention``
  in the brunomaga post).  Table entries past ``ceil(ctx / block_size)`` are
  never read.

* ``attend``: for query head ``i`` and KV head ``h = i // g`` (consecutive
  grouping: 32 query heads in 8 groups of 4 for Llama-3-8B, kongchang.com
  "What the KV Cache Is"), ``s_t = scale * q_i . k_t``, softmax over the
  ``ctx`` tokens, output ``sum_t p_t v_t``.  No causal mask beyond ``ctx``:
  in decode the newest token may look at every cached token (4yush.com,
  "Adding the cache to GPT-2": the decode mask is all ones).

* ``kv_append_tokens`` / ``multi_query_attention``: several new tokens per
  sequence (chunked prefill, a prefix-cache tail, a speculative verify pass).
  The t newest tokens are appended, then query j of them attends over the
  tokens up to its own position: ``ctx - t + j + 1`` of them (the shifted
  causal mask of the KV post's ``attn_cached``, the brunomaga post's
  ``causal_mask`` and the 4yush post's mask with a start offset).

* ``partition_partials`` / ``merge_partials``: the softmax over a range of
  tokens splits into per-range normalised outputs ``o_p`` and their
  log-sum-exp ``lse_p = m_p + ln sum exp(s - m_p)``; the whole-range output is
  ``sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M)`` with ``M = max_p lse_p``
  (learn.mohebi.ai serving lesson, "PagedAttention" and "Where it shows up":
  block-by-block reading merged with the online-softmax update, split-KV
  decoding for long contexts).  An empty range has ``lse = -inf`` and does not
  contribute.

Every function is pinned in ``tests/test_oracle.py`` against something other
than itself: torch's float64 ``scaled_dot_product_attention`` with a causal
mask (the routine the KV-cache post's own check uses), exhaustive format
tables, closed forms and invariants.
"""

from __future__ import annotations

import numpy as np

LN2 = float(np.log(2.0))


# --------------------------------------------------------------------------
# Storage formats
# --------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the bits are the top half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP float8 e4m3fn codes (uint8) -> float64, from the bit layout.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    exponent 0: subnormal, value = m/8 * 2**-6; otherwise (1 + m/8) * 2**(e-7).
    Exponent 15 with mantissa 7 is NaN; there are no infinities (max 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(exp == 0,
                   (man / 8.0) * 2.0 ** -6,
                   (1.0 + man / 8.0) * np.exp2((exp - 7).astype(np.float64)))
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def to_float64(storage: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array of ``dtype`` ('f32', 'bf16' bits, 'fp8_e4m3' codes) -> float64 (exact)."""
    if dtype == "f32":
        return np.asarray(storage, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(storage)
    if dtype == "fp8_e4m3":
        # An e4m3 value depends on its 8-bit code alone: decode all 256 codes
        # from their bits, then look every stored code up (same values as
        # decoding each element, far faster on a whole cache).
        table = decode_e4m3fn(np.arange(256, dtype=np.uint8))
        return table[np.asarray(storage, dtype=np.uint8)]
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Append: the new token's K/V into its slot
# --------------------------------------------------------------------------

def slot_of(table_row: np.ndarray, position: int, block_size: int) -> tuple[int, int]:
    """(physical block, slot) of a logical token position through one block table row."""
    return int(table_row[position // block_size]), position % block_size


def kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens, block_size,
              inplace=False):
    """Write each sequence's new K/V rows ([B, Hkv, D], pool storage format) to
    slot ``ctx - 1``.  Returns the (copied unless ``inplace``) pools.  A
    sequence with ``ctx <= 0`` has nothing to append."""
    if not inplace:
        k_pool = k_pool.copy()
        v_pool = v_pool.copy()
    for b in range(len(context_lens)):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        blk, off = slot_of(block_tables[b], ctx - 1, block_size)
        k_pool[blk, :, off, :] = k_new[b]
        v_pool[blk, :, off, :] = v_new[b]
    return k_pool, v_pool


# --------------------------------------------------------------------------
# Gather through the block table
# --------------------------------------------------------------------------

def gather_sequence(pool, table_row, ctx, block_size, dtype, scales=None):
    """One sequence's cache as a contiguous float64 array [Hkv, ctx, D].

    ``pool`` is [num_blocks, Hkv, block_size, D] in storage format; ``scales``
    ([num_blocks, Hkv]) multiplies each e4m3 block-head slice.
    """
    nb = -(-ctx // block_size)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = to_float64(pool[ids], dtype)                      # [nb, Hkv, bs, D]
    if scales is not None:
        blocks = blocks * np.asarray(scales, np.float32)[ids].astype(np.float64)[:, :, None, None]
    hkv, d = blocks.shape[1], blocks.shape[3]
    seq = blocks.transpose(1, 0, 2, 3).reshape(hkv, nb * block_size, d)
    return seq[:, :ctx, :]


# --------------------------------------------------------------------------
# Attention of one query per head over a contiguous cache
# --------------------------------------------------------------------------

def attend(q, K, V, scale, return_weights=False):
    """q [Hq, D], K/V [Hkv, T, D] (float64) -> out [Hq, D].

    Query head i reads KV head i // (Hq // Hkv).  Softmax over all T tokens.
    """
    hq = q.shape[0]
    hkv = K.shape[0]
    g = hq // hkv
    out = np.empty((hq, V.shape[2]), dtype=np.float64)
    weights = []
    for i in range(hq):
        h = i // g
        s = scale * (K[h] @ q[i])                   # [T]
        m = s.max()
        p = np.exp(s - m)
        z = p.sum()
        out[i] = (p @ V[h]) / z
        weights.append(p / z)
    if return_weights:
        return out, np.stack(weights)
    return out


def decode_attention(q, k_pool, v_pool, block_tables, context_lens, *, block_size,
                     softmax_scale, q_dtype, kv_dtype, k_scales=None, v_scales=None,
                     seqs=None):
    """Decode-step attention over pools that already hold the appended tokens.

    q: [B, Hq, D] storage; pools [NB, Hkv, bs, D] storage; returns float64
    [len(seqs), Hq, D] (all sequences by default).  A sequence with ctx == 0
    attends over nothing and returns zeros.
    """
    seqs = range(len(context_lens)) if seqs is None else seqs
    outs = []
    for b in seqs:
        ctx = int(context_lens[b])
        qb = to_float64(q[b], q_dtype)
        if ctx <= 0:
            outs.append(np.zeros_like(qb))
            continue
        K = gather_sequence(k_pool, block_tables[b], ctx, block_size, kv_dtype, k_scales)
        V = gather_sequence(v_pool, block_tables[b], ctx, block_size, kv_dtype, v_scales)
        outs.append(attend(qb, K, V, softmax_scale))
    return np.stack(outs) if outs else np.zeros((0,) + q.shape[1:], np.float64)


# --------------------------------------------------------------------------
# Split over token ranges, then merge by log-sum-exp
# --------------------------------------------------------------------------

def partition_partials(q, K, V, scale, partition_size):
    """q [Hq, D], K/V [Hkv, T, D] -> (o [Hq, nP, D], lse [Hq, nP]).

    Partition p covers tokens [p*P, min((p+1)*P, T)); o_p is the softmax of
    that range applied to V; lse_p is its natural-log log-sum-exp.
    """
    hq, d = q.shape
    T = K.shape[1]
    g = hq // K.shape[0]
    n_p = -(-T // partition_size)
    o = np.zeros((hq, n_p, d))
    lse = np.full((hq, n_p), -np.inf)
    for i in range(hq):
        h = i // g
        for p in range(n_p):
            lo, hi = p * partition_size, min((p + 1) * partition_size, T)
            s = scale * (K[h, lo:hi] @ q[i])
            m = s.max()
            w = np.exp(s - m)
            l = w.sum()
            o[i, p] = (w @ V[h, lo:hi]) / l
            lse[i, p] = m + np.log(l)
    return o, lse


def merge_partials(o, lse):
    """o [..., nP, D], lse [..., nP] -> [..., D].  Partitions with lse = -inf
    are empty and skipped (never multiplied); if all are empty the result is 0.
    Any other lse counts, so a NaN partial propagates."""
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    out = np.zeros(o.shape[:-2] + (o.shape[-1],))
    flat_o = o.reshape(-1, o.shape[-2], o.shape[-1])
    flat_l = lse.reshape(-1, lse.shape[-1])
    flat_out = out.reshape(-1, o.shape[-1])
    for r in range(flat_l.shape[0]):
        valid = ~np.isneginf(flat_l[r])
        if not valid.any():
            continue
        M = flat_l[r][valid].max()
        w = np.exp(flat_l[r][valid] - M)
        flat_out[r] = (w @ flat_o[r][valid]) / w.sum()
    return out


def decode_partials(q, k_pool, v_pool, block_tables, context_lens, *, block_size,
                    softmax_scale, q_dtype, kv_dtype, partition_size, max_partitions,
                    k_scales=None, v_scales=None):
    """Per-partition outputs of every sequence, padded to ``max_partitions``:
    (o [B, Hq, maxP, D], lse [B, Hq, maxP]); missing partitions hold o = 0,
    lse = -inf."""
    B, hq, d = q.shape
    o = np.zeros((B, hq, max_partitions, d))
    lse = np.full((B, hq, max_partitions), -np.inf)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        K = gather_sequence(k_pool, block_tables[b], ctx, block_size, kv_dtype, k_scales)
        V = gather_sequence(v_pool, block_tables[b], ctx, block_size, kv_dtype, v_scales)
        ob, lb = partition_partials(to_float64(q[b], q_dtype), K, V, softmax_scale, partition_size)
        o[b, :, :ob.shape[1]] = ob
        lse[b, :, :lb.shape[1]] = lb
    return o, lse


# --------------------------------------------------------------------------
# Several new tokens per sequence: the shifted causal mask
# --------------------------------------------------------------------------

def visible_tokens(ctx: int, t: int, j: int) -> int:
    """How many cached tokens query j (0-based) of a sequence's t newest tokens
    sees: the tokens up to its own position ctx - t + j (KV post, "A KV cache in
    PyTorch": mask tril(T - t); brunomaga post, causal_mask(Sq, Sk) =
    tril(Sk - Sq); 4yush post, "Adding the cache to GPT-2": new token r at
    position start + r sees keys 0 .. start + r)."""
    return ctx - t + j + 1


def kv_append_tokens(k_pool, v_pool, k_new, v_new, block_tables, context_lens, query_start_loc,
                     block_size, inplace=False):
    """Write the t_b = qsl[b+1] - qsl[b] newest rows of every sequence: row
    qsl[b] + j of k_new/v_new ([total, Hkv, D]) goes to position ctx_b - t_b + j."""
    if not inplace:
        k_pool = k_pool.copy()
        v_pool = v_pool.copy()
    for b in range(len(context_lens)):
        ctx = int(context_lens[b])
        q0, q1 = int(query_start_loc[b]), int(query_start_loc[b + 1])
        t = q1 - q0
        for j in range(t):
            pos = ctx - t + j
            if pos < 0:
                continue
            blk, off = slot_of(block_tables[b], pos, block_size)
            k_pool[blk, :, off, :] = k_new[q0 + j]
            v_pool[blk, :, off, :] = v_new[q0 + j]
    return k_pool, v_pool


def multi_query_attention(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, *,
                          block_size, softmax_scale, q_dtype, kv_dtype, k_scales=None,
                          v_scales=None):
    """q [total, Hq, D]: rows qsl[b] .. qsl[b+1]-1 are sequence b's newest
    tokens, in order.  Query j of sequence b attends over its first
    visible_tokens(ctx_b, t_b, j) cached tokens.  Returns float64 [total, Hq, D]."""
    total = int(query_start_loc[-1])
    out = np.zeros((total,) + q.shape[1:])
    for b in range(len(context_lens)):
        ctx = int(context_lens[b])
        q0, q1 = int(query_start_loc[b]), int(query_start_loc[b + 1])
        if q1 == q0 or ctx <= 0:
            continue
        K = gather_sequence(k_pool, block_tables[b], ctx, block_size, kv_dtype, k_scales)
        V = gather_sequence(v_pool, block_tables[b], ctx, block_size, kv_dtype, v_scales)
        for j in range(q1 - q0):
            n = visible_tokens(ctx, q1 - q0, j)
            if n <= 0:
                continue
            out[q0 + j] = attend(to_float64(q[q0 + j], q_dtype), K[:, :n], V[:, :n], softmax_scale)
    return out


def decode_step(q, k_pool, v_pool, k_new, v_new, block_tables, context_lens, *,
                block_size, softmax_scale, q_dtype, kv_dtype, k_scales=None,
                v_scales=None, seqs=None):
    """Append, then attend: one whole decode step.  Returns (out float64,
    k_pool after, v_pool after)."""
    kp, vp = kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens, block_size)
    out = decode_attention(q, kp, vp, block_tables, context_lens, block_size=block_size,
                           softmax_scale=softmax_scale, q_dtype=q_dtype, kv_dtype=kv_dtype,
                           k_scales=k_scales, v_scales=v_scales, seqs=seqs)
    return out, kp, vp
