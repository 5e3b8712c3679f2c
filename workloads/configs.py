"""Seeded synthetic workloads for one decode step over a paged KV cache.

Nothing here computes attention.  The module draws:

1. context lengths (tokens attended, counting the token appended this step),
2. a random placement of every sequence's logical blocks in the shared pool,
3. K pool values, then V pool values (each from its own seed sequence,
   [seed, 1] and [seed, 2], in chunks of 256 blocks), then queries, all N(0, 1),

and stores them in the storage format of the requested dtype:

* ``f32``       float32 values,
* ``bf16``      uint16 bit patterns, rounded to nearest even from float32,
* ``fp8_e4m3``  uint8 bit patterns of OCP float8 e4m3fn, with one float32
                scale per (block, kv head) equal to the block's max |value|
                over its valid slots divided by 448 (1 when that max is 0).

The new token's K/V rows are drawn as part of the pool; they are then taken
out of their slot (``k_new``/``v_new``) and the slot is poisoned, so that a
decode step that forgets to append reads poison.  Unused blocks and the tail
slots of each sequence's last block are poisoned too (NaN, or 0x7F for e4m3),
and block-table padding is -1: none of them may ever reach an output.

The five named workloads follow the decode configurations the pages analyse:
the Llama-3-8B layer shape (32 query heads, 8 KV heads, head dim 128, blocks
of 16 tokens) that the serving lesson's worked example and the KV-cache posts
use, plus a tiny float32 case, a 131,072-token split-KV case, a
continuous-batching length mix and an fp8 multi-head case.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np
import torch

DTYPES = ("f32", "bf16", "fp8_e4m3")
STORAGE_NP = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}
E4M3_MAX = 448.0
BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F

CONFIG_NAMES = {
    1: "tiny_fp32",
    2: "llama3_8b_b64",
    3: "long_context_131k",
    4: "continuous_batching_mix",
    5: "fp8_mha_b128",
}

# Shape and length recipe of each named workload.  ``ctx`` is one of
#   ("fixed", [lengths...])                  explicit per-sequence lengths
#   ("const", n)                             every sequence n tokens
#   ("uniform", lo, hi)                      integers in [lo, hi], both ends
#   ("lognormal", median, sigma, lo, hi)     round(exp(ln median + sigma*N)),
#                                            clipped to [lo, hi]
# ``pool`` is ("blocks", n) for a pool of n blocks, or ("used_fraction", f) for
# ceil(blocks needed / f) blocks (f = 1: exactly the blocks needed).
# ``partition_size`` is the one-token decode's default split: 512 tokens where
# the workload names it (the long-context one) or where one partition holds
# every sequence, else -1, the balanced split (chunks of nearly equal size
# chosen from the context lengths), for one new token per sequence or
# several.
_RECIPES = {
    1: dict(num_seqs=4, num_q_heads=4, num_kv_heads=4, head_dim=64,
            ctx=("fixed", [17, 33, 64, 100]), pool=("blocks", 64),
            q_dtype="f32", kv_dtype="f32", partition_size=512),
    2: dict(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
            ctx=("uniform", 512, 4096), pool=("used_fraction", 1.0),
            q_dtype="bf16", kv_dtype="bf16", partition_size=-1),
    3: dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
            ctx=("const", 131072), pool=("used_fraction", 1.0),
            q_dtype="bf16", kv_dtype="bf16", partition_size=512),
    4: dict(num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
            ctx=("lognormal", 1024, 1.0, 1, 32768), pool=("used_fraction", 0.7),
            q_dtype="bf16", kv_dtype="bf16", partition_size=-1),
    5: dict(num_seqs=128, num_q_heads=32, num_kv_heads=32, head_dim=128,
            ctx=("const", 2048), pool=("used_fraction", 1.0),
            q_dtype="bf16", kv_dtype="fp8_e4m3", partition_size=-1),
}


@dataclasses.dataclass
class PagedDecodeInputs:
    """Host-side inputs of one decode step (storage formats, see module doc)."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    partition_size: int
    q_dtype: str
    kv_dtype: str
    softmax_scale: float
    context_lens: np.ndarray      # int32 [B]
    block_tables: np.ndarray      # int32 [B, max_blocks_per_seq], -1 padded
    q: np.ndarray                 # [B, Hq, D]
    k_pool: np.ndarray            # [NB, Hkv, bs, D], state before the append
    v_pool: np.ndarray
    k_new: np.ndarray             # [B, Hkv, D]
    v_new: np.ndarray
    k_scales: np.ndarray | None   # float32 [NB, Hkv] (fp8 only)
    v_scales: np.ndarray | None
    seed: int = 0
    # Several new tokens per sequence: rows qsl[b] .. qsl[b+1]-1 of q, k_new and
    # v_new belong to sequence b (its newest tokens, in order).  None: one each.
    query_start_loc: np.ndarray | None = None

    @property
    def total_queries(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_new_tokens(self) -> int:
        if self.query_start_loc is None:
            return 1
        return int(np.diff(self.query_start_loc).max()) if self.num_seqs else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def num_partitions(self, partition_size: int | None = None) -> np.ndarray:
        p = self.partition_size if partition_size is None else partition_size
        if p < 0:
            raise ValueError("the balanced split has no fixed partition count")
        if p == 0:
            return np.minimum(self.context_lens, 1).astype(np.int64)
        return -(-self.context_lens.astype(np.int64) // p)

    def subset(self, seqs) -> "PagedDecodeInputs":
        """The same pools, with only the chosen sequences in the batch (one new
        token per sequence)."""
        if self.query_start_loc is not None:
            raise ValueError("subset() is for one new token per sequence")
        seqs = np.asarray(seqs, dtype=np.int64)
        return dataclasses.replace(
            self,
            num_seqs=len(seqs),
            context_lens=self.context_lens[seqs].copy(),
            block_tables=self.block_tables[seqs].copy(),
            q=self.q[seqs].copy(),
            k_new=self.k_new[seqs].copy(),
            v_new=self.v_new[seqs].copy(),
        )


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage format.  bf16 and e4m3 use torch's round-to-nearest-even casts."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8_e4m3":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def _poison_value(dtype: str):
    return {"f32": np.float32(np.nan), "bf16": np.uint16(BF16_NAN_BITS),
            "fp8_e4m3": np.uint8(E4M3_NAN_CODE)}[dtype]


_POOL_CHUNK_BLOCKS = 256


def _draw_pool(seed_words, num_blocks, hkv, bs, d, dtype, valid_count, poison):
    """Draw one pool (post-append contents).  Blocks are drawn in chunks of
    256, chunk i from its own generator ``SeedSequence(seed_words).spawn(n)[i]``
    (so the result does not depend on how many threads draw it)."""
    pool = np.empty((num_blocks, hkv, bs, d), STORAGE_NP[dtype])
    scales = np.full((num_blocks, hkv), np.nan, np.float32) if dtype == "fp8_e4m3" else None
    pv = _poison_value(dtype)
    starts = list(range(0, num_blocks, _POOL_CHUNK_BLOCKS))
    kids = np.random.SeedSequence(seed_words).spawn(len(starts))

    def one(i):
        c0 = starts[i]
        c1 = min(num_blocks, c0 + _POOL_CHUNK_BLOCKS)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        x = g.standard_normal((c1 - c0, hkv, bs, d), dtype=np.float32)
        vc = valid_count[c0:c1]
        slot_ok = np.arange(bs)[None, :] < vc[:, None]                     # [n, bs]
        if dtype == "fp8_e4m3":
            mag = np.abs(x)
            mag *= slot_ok[:, None, :, None]
            amax = mag.max(axis=(2, 3))
            sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
            x /= sc[:, :, None, None]
            np.clip(x, -E4M3_MAX, E4M3_MAX, out=x)
            scales[c0:c1] = np.where(vc[:, None] > 0, sc, np.float32(np.nan))
        pool[c0:c1] = _to_storage(x, dtype)
        if poison:
            bad = ~slot_ok                                                   # [n, bs]
            if bad.any():
                view = pool[c0:c1].transpose(0, 2, 1, 3)                     # [n, bs, hkv, d]
                view[bad] = pv

    with concurrent.futures.ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(one, range(len(starts))))
    return pool, scales


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _context_lengths(rng, spec, num_seqs):
    kind = spec[0]
    if kind == "fixed":
        vals = np.asarray(spec[1], dtype=np.int64)
        if num_seqs != len(vals):
            vals = np.resize(vals, num_seqs)
        return vals
    if kind == "const":
        return np.full(num_seqs, spec[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=num_seqs, endpoint=True).astype(np.int64)
    if kind == "lognormal":
        _, median, sigma, lo, hi = spec
        z = rng.standard_normal(num_seqs)
        return np.clip(np.round(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)
    raise ValueError(spec)


def make_inputs(*, num_seqs, num_q_heads, num_kv_heads, head_dim, ctx, pool,
                q_dtype, kv_dtype, partition_size=512, block_size=16, seed=0,
                poison=True, extra_table_cols=0, name="custom", softmax_scale=None,
                new_tokens=None):
    """Draw one decode step's inputs.  See the module docstring for the recipe.

    ``new_tokens`` (a length spec like ``ctx``, or None for one per sequence)
    gives each sequence several new tokens: they are its newest positions, and
    a context shorter than its new tokens is raised to their count."""
    if q_dtype not in ("f32", "bf16") or kv_dtype not in DTYPES:
        raise ValueError((q_dtype, kv_dtype))
    rng = np.random.default_rng(seed)
    ctx_lens = _context_lengths(rng, ctx, num_seqs)
    if new_tokens is None:
        t_new = np.ones(num_seqs, dtype=np.int64) * (ctx_lens > 0)
        qsl = None
    else:
        t_new = _context_lengths(rng, new_tokens, num_seqs)
        ctx_lens = np.maximum(ctx_lens, t_new)
        qsl = np.concatenate([[0], np.cumsum(t_new)]).astype(np.int32)
    nblk = -(-ctx_lens // block_size)
    total = int(nblk.sum())
    if pool[0] == "blocks":
        num_blocks = int(pool[1])
    else:
        num_blocks = max(1, int(math.ceil(total / pool[1])))
    if total > num_blocks:
        raise RuntimeError(f"out of KV cache blocks: {total} needed, pool has {num_blocks}")
    perm = rng.permutation(num_blocks)
    max_blk = int(nblk.max()) + extra_table_cols if num_seqs else max(1, extra_table_cols)
    tables = np.full((num_seqs, max(max_blk, 1)), -1, dtype=np.int32)
    valid_count = np.zeros(num_blocks, dtype=np.int64)
    cursor = 0
    for b in range(num_seqs):
        ids = perm[cursor:cursor + nblk[b]]
        cursor += nblk[b]
        tables[b, :nblk[b]] = ids
        valid = np.full(nblk[b], block_size, dtype=np.int64)
        if nblk[b]:
            valid[-1] = ctx_lens[b] - (nblk[b] - 1) * block_size
        valid_count[ids] = valid

    k_pool, k_scales = _draw_pool([seed, 1], num_blocks, num_kv_heads, block_size, head_dim,
                                  kv_dtype, valid_count, poison)
    v_pool, v_scales = _draw_pool([seed, 2], num_blocks, num_kv_heads, block_size, head_dim,
                                  kv_dtype, valid_count, poison)
    n_rows = num_seqs if qsl is None else int(qsl[-1])
    q = _to_storage(rng.standard_normal((n_rows, num_q_heads, head_dim), dtype=np.float32), q_dtype)

    # Take the new tokens' rows out of their slots, and poison the slots.
    k_new = np.empty((n_rows, num_kv_heads, head_dim), STORAGE_NP[kv_dtype])
    v_new = np.empty_like(k_new)
    pv = _poison_value(kv_dtype)
    row = 0
    for b in range(num_seqs):
        t = int(t_new[b]) if qsl is not None else 1
        if qsl is None and ctx_lens[b] <= 0:
            k_new[b] = pv
            v_new[b] = pv
            row += 1
            continue
        for j in range(t):
            pos = ctx_lens[b] - t + j
            blk = tables[b, pos // block_size]
            off = pos % block_size
            k_new[row] = k_pool[blk, :, off]
            v_new[row] = v_pool[blk, :, off]
            if poison:
                k_pool[blk, :, off] = pv
                v_pool[blk, :, off] = pv
            row += 1

    return PagedDecodeInputs(
        name=name, num_seqs=num_seqs, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
        max_blocks_per_seq=tables.shape[1], partition_size=partition_size,
        q_dtype=q_dtype, kv_dtype=kv_dtype,
        softmax_scale=(1.0 / math.sqrt(head_dim)) if softmax_scale is None else softmax_scale,
        context_lens=ctx_lens.astype(np.int32), block_tables=tables, q=q,
        k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
        k_scales=k_scales, v_scales=v_scales, seed=seed, query_start_loc=qsl)


def recipe(config: int) -> dict:
    return dict(_RECIPES[config])


def named_config(config: int, *, seed=None, **overrides) -> PagedDecodeInputs:
    """One of the five named workloads; ``overrides`` replace recipe fields
    (e.g. ``num_seqs`` for a smaller batch of the same shape, or ``kv_dtype``
    and ``q_dtype`` for a float32 twin of a bf16 workload)."""
    name = overrides.pop("name", CONFIG_NAMES[config])
    r = recipe(config)
    r.update(overrides)
    return make_inputs(seed=config if seed is None else seed, name=name, **r)
