"""Seeded synthetic inputs for MLA decode over a paged latent cache.

A latent pool [num_blocks, block_size, d_c + d_r] (one 576-number row per
token for the DeepSeek-V2 shape: a 512-number latent and a 64-number rotary
key), absorbed queries [B, H, d_c + d_r], the new token's latent rows
[B, d_c + d_r], block tables and context lengths.  Same recipe as the
attention workloads: lengths first, then a random permutation of the pool,
then N(0,1) values (bf16 round-to-nearest-even), unused slots poisoned with
NaN.  No attention arithmetic happens here."""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from .configs import _context_lengths, _draw_pool, _poison_value, _to_storage


@dataclasses.dataclass
class MLAInputs:
    name: str
    num_seqs: int
    num_heads: int
    kv_lora_rank: int
    rope_dim: int
    block_size: int
    num_blocks: int
    dtype: str
    softmax_scale: float
    partition_size: int
    context_lens: np.ndarray      # int32 [B]
    block_tables: np.ndarray      # int32 [B, max_blocks], -1 padded
    q: np.ndarray                 # [B, H, d_c + d_r] storage format
    latent_pool: np.ndarray       # [NB, block_size, d_c + d_r], state before the append
    latent_new: np.ndarray        # [B, d_c + d_r]
    seed: int = 0

    @property
    def row_dim(self) -> int:
        return self.kv_lora_rank + self.rope_dim

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


MLA_WORKLOADS = {
    # DeepSeek-V2/V3 attention shape (128 heads, 512 + 64 latent row, softmax
    # scale 1/sqrt(128 + 64)), the batch-64 decode layer with the same context
    # lengths as the Llama-3-8B workload.  The balanced split (-1): at most 256
    # chunks of nearly equal size, one round on the 256 CUs.
    "deepseek_mla_b64": dict(num_seqs=64, num_heads=128, ctx=("uniform", 512, 4096), seed=2,
                             partition_size=-1),
    # DeepSeek-V2-Lite's 16 heads, a small batch the oracle finishes quickly.
    # Partitions of one pair of blocks: with one wave per workgroup the time
    # grows with the pairs each wave walks.
    "deepseek_lite_mla_b8": dict(num_seqs=8, num_heads=16, ctx=("uniform", 1, 700), seed=12,
                                 partition_size=32),
}


def make_mla_inputs(*, num_seqs, num_heads, ctx, kv_lora_rank=512, rope_dim=64, block_size=16,
                    dtype="bf16", pool_used_fraction=1.0, partition_size=512, seed=0,
                    poison=True, softmax_scale=None, name="custom_mla", qk_head_dim=128):
    rng = np.random.default_rng(seed)
    ctx_lens = _context_lengths(rng, ctx, num_seqs)
    nblk = -(-ctx_lens // block_size)
    total = int(nblk.sum())
    num_blocks = max(1, int(math.ceil(total / pool_used_fraction)))
    perm = rng.permutation(num_blocks)
    tables = np.full((num_seqs, max(int(nblk.max()) if num_seqs else 1, 1)), -1, np.int32)
    valid = np.zeros(num_blocks, np.int64)
    cur = 0
    for b in range(num_seqs):
        ids = perm[cur:cur + nblk[b]]
        cur += nblk[b]
        tables[b, :nblk[b]] = ids
        v = np.full(nblk[b], block_size, np.int64)
        if nblk[b]:
            v[-1] = ctx_lens[b] - (nblk[b] - 1) * block_size
        valid[ids] = v
    d = kv_lora_rank + rope_dim
    pool4, _ = _draw_pool([seed, 3], num_blocks, 1, block_size, d, dtype, valid, poison)
    pool = pool4[:, 0]
    q = _to_storage(rng.standard_normal((num_seqs, num_heads, d), dtype=np.float32), dtype)
    new = np.empty((num_seqs, d), pool.dtype)
    pv = _poison_value(dtype)
    for b in range(num_seqs):
        if ctx_lens[b] <= 0:
            new[b] = pv
            continue
        pos = ctx_lens[b] - 1
        blk, off = tables[b, pos // block_size], pos % block_size
        new[b] = pool[blk, off]
        if poison:
            pool[blk, off] = pv
    scale = (1.0 / math.sqrt(qk_head_dim + rope_dim)) if softmax_scale is None else softmax_scale
    return MLAInputs(name=name, num_seqs=num_seqs, num_heads=num_heads, kv_lora_rank=kv_lora_rank,
                     rope_dim=rope_dim, block_size=block_size, num_blocks=num_blocks, dtype=dtype,
                     softmax_scale=scale, partition_size=partition_size,
                     context_lens=ctx_lens.astype(np.int32), block_tables=tables, q=q,
                     latent_pool=pool, latent_new=new, seed=seed)


def named_mla(name, **overrides):
    r = dict(MLA_WORKLOADS[name])
    r.update(overrides)
    return make_mla_inputs(name=name, **r)
