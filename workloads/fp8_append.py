"""Seeded synthetic state for appending to an e4m3 paged cache with
quantisation: pools of random e4m3 codes (no NaN codes), positive float32
scales per (block, KV head) around 1/448, sequences with shuffled blocks, and
new K/V rows as float32 values (bf16-exact when ``new_dtype`` is "bf16").
No quantisation arithmetic happens here: the codes and scales are drawn
directly."""

from __future__ import annotations

import numpy as np
import torch


def fp8_append_state(seed=0, num_seqs=5, num_kv_heads=3, head_dim=64, block_size=16,
                     new_tokens=None, ctx_range=(1, 69), new_dtype="bf16", spare_blocks=3,
                     new_std=1.5):
    """Returns a dict with k_pool/v_pool (uint8 [NB, Hkv, bs, D]),
    k_scales/v_scales (float32 [NB, Hkv]), k_new/v_new (float32 [rows, Hkv, D]),
    block_tables (int32, -1 padded, one spare column), context_lens (int32) and
    query_start_loc (int32 [B+1], or None for one new row per sequence).
    ``new_tokens``: None, an int, or a list of per-sequence counts."""
    rng = np.random.default_rng(seed)
    B = num_seqs
    ctx = rng.integers(ctx_range[0], ctx_range[1], B, endpoint=True)
    if new_tokens is None:
        t = None
    else:
        t = np.resize(np.asarray(new_tokens, np.int64), B)
        ctx = np.maximum(ctx, t)
    nblk = -(-ctx // block_size)
    NB = int(nblk.sum()) + spare_blocks
    perm = rng.permutation(NB)
    tables = np.full((B, int(nblk.max()) + 1), -1, np.int32)
    c = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[c:c + nblk[b]]
        c += nblk[b]
    shape = (NB, num_kv_heads, block_size, head_dim)
    pools = []
    for fill in (0x11, 0x22):
        p = rng.integers(0, 256, shape).astype(np.uint8)
        p[(p & 0x7F) == 0x7F] = fill                     # no NaN codes in the state
        pools.append(p)
    ks = (rng.uniform(0.5, 2.0, (NB, num_kv_heads)) / 448).astype(np.float32)
    vs = (rng.uniform(0.5, 2.0, (NB, num_kv_heads)) / 448).astype(np.float32)
    if t is None:
        qsl, rows = None, B
    else:
        qsl = np.concatenate([[0], np.cumsum(t)]).astype(np.int32)
        rows = int(qsl[-1])
    new = []
    for scale in (new_std, 1.0):
        x = rng.standard_normal((rows, num_kv_heads, head_dim)).astype(np.float32) * np.float32(scale)
        if new_dtype == "bf16":
            x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        new.append(x)
    return dict(k_pool=pools[0], v_pool=pools[1], k_scales=ks, v_scales=vs, k_new=new[0],
                v_new=new[1], block_tables=tables, context_lens=ctx.astype(np.int32),
                query_start_loc=qsl)
