"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function returns the worst deviation it found (0 = exact) so
that ``test_oracle.py`` can assert on it, and ``test_oracle_mutations.py`` can
plant mistakes in the oracle and see which pins catch them.  The references
here are independent of the oracle's code: torch's float64
``scaled_dot_product_attention`` (the routine the KV-cache post checks its own
cache against), torch's float8/bfloat16 casts, scipy's ``logsumexp``, a
padded torch gather, closed forms and invariants.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle.paged_attention as pa
from workloads import make_inputs, named_config


def _sdpa(q, k, v, **kw):
    """float64 CPU SDPA; q [..., Hq, T, D]; k/v [..., Hkv, T, D] expanded with
    consecutive grouping (query head i reads KV head i // g)."""
    g = q.shape[-3] // k.shape[-3]
    k = k.repeat_interleave(g, dim=-3)
    v = v.repeat_interleave(g, dim=-3)
    return F.scaled_dot_product_attention(q, k, v, **kw)


# --------------------------------------------------------------------------
# Pin 1: append + paged decode step by step == full causal attention
# --------------------------------------------------------------------------

def pin_incremental_vs_causal(*, n_seqs=3, Hq=4, Hkv=2, D=16, T=37, bs=4, seed=0):
    """Every sequence decodes T tokens one step at a time through a paged
    pool whose blocks are handed out on demand from a shuffled free list
    (sequences interleaved).  Output of step t must equal row t-1 of full
    causal attention over all T tokens."""
    rng = np.random.default_rng(seed)
    q_all = rng.standard_normal((n_seqs, Hq, T, D)).astype(np.float32)
    k_all = rng.standard_normal((n_seqs, Hkv, T, D)).astype(np.float32)
    v_all = rng.standard_normal((n_seqs, Hkv, T, D)).astype(np.float32)
    ref = _sdpa(torch.from_numpy(q_all).double(), torch.from_numpy(k_all).double(),
                torch.from_numpy(v_all).double(), is_causal=True).numpy()
    nbmax = -(-T // bs)
    NB = n_seqs * nbmax + 5
    free = [int(x) for x in rng.permutation(NB)]
    k_pool = np.full((NB, Hkv, bs, D), np.nan, np.float32)
    v_pool = np.full((NB, Hkv, bs, D), np.nan, np.float32)
    tables = np.full((n_seqs, nbmax + 2), -1, np.int32)
    used = [0] * n_seqs
    worst = 0.0
    for t in range(1, T + 1):
        for b in range(n_seqs):
            if (t - 1) % bs == 0:
                tables[b, used[b]] = free.pop()
                used[b] += 1
        ctx = np.full(n_seqs, t, np.int32)
        pa.kv_append(k_pool, v_pool, k_all[:, :, t - 1], v_all[:, :, t - 1], tables, ctx, bs,
                     inplace=True)
        out = pa.decode_attention(q_all[:, :, t - 1], k_pool, v_pool, tables, ctx,
                                  block_size=bs, softmax_scale=1.0 / math.sqrt(D),
                                  q_dtype="f32", kv_dtype="f32")
        worst = max(worst, float(np.nan_to_num(np.abs(out - ref[:, :, t - 1]), nan=np.inf).max()))
    return worst


# --------------------------------------------------------------------------
# Pin 9: library cross-check with a torch padded gather (the brunomaga form)
# --------------------------------------------------------------------------

def torch_decode_storage(t, dtype):
    """Storage numpy array -> float64 torch tensor, decoded by torch's own dtypes."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t)).double()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t).view(np.int16)).view(torch.bfloat16).double()
    if dtype == "fp8_e4m3":
        return torch.from_numpy(np.ascontiguousarray(t)).view(torch.float8_e4m3fn).double()
    raise ValueError(dtype)


def torch_padded_decode(inp, k_pool, v_pool, seqs=None):
    """Gather every sequence's blocks into a padded [B, Hkv, L, D] tensor with
    torch indexing, mask the slots at or beyond ctx, and run float64 SDPA."""
    seqs = list(range(inp.num_seqs)) if seqs is None else list(seqs)
    bs, D = inp.block_size, inp.head_dim
    ctx = torch.from_numpy(inp.context_lens[seqs].astype(np.int64))
    nb = int(((ctx + bs - 1) // bs).max())
    tab = torch.from_numpy(inp.block_tables[seqs][:, :nb].astype(np.int64))
    valid_blk = torch.arange(nb)[None, :] < ((ctx + bs - 1) // bs)[:, None]
    safe = torch.where(valid_blk, tab, torch.zeros_like(tab))
    kp = torch_decode_storage(k_pool, inp.kv_dtype)
    vp = torch_decode_storage(v_pool, inp.kv_dtype)
    if inp.k_scales is not None:
        kp = kp * torch.from_numpy(inp.k_scales).double()[:, :, None, None]
        vp = vp * torch.from_numpy(inp.v_scales).double()[:, :, None, None]
    B = len(seqs)
    L = nb * bs
    k = kp[safe].permute(0, 2, 1, 3, 4).reshape(B, inp.num_kv_heads, L, D)
    v = vp[safe].permute(0, 2, 1, 3, 4).reshape(B, inp.num_kv_heads, L, D)
    mask = torch.arange(L)[None, :] < ctx[:, None]                      # [B, L]
    k = torch.where(mask[:, None, :, None], k, torch.zeros_like(k))      # poison never multiplies
    v = torch.where(mask[:, None, :, None], v, torch.zeros_like(v))
    q = torch_decode_storage(inp.q[seqs], inp.q_dtype)[:, :, None, :]   # [B, Hq, 1, D]
    out = _sdpa(q, k, v, attn_mask=mask[:, None, None, :], scale=inp.softmax_scale)
    return out[:, :, 0].numpy()


def pin_library_crosscheck(inp, seqs=None):
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, inp.block_size)
    ref = torch_padded_decode(inp, kp, vp, seqs)
    out = pa.decode_attention(inp.q, kp, vp, inp.block_tables, inp.context_lens,
                              block_size=inp.block_size, softmax_scale=inp.softmax_scale,
                              q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype,
                              k_scales=inp.k_scales, v_scales=inp.v_scales, seqs=seqs)
    return float(np.nan_to_num(np.abs(out - ref), nan=np.inf).max())


# --------------------------------------------------------------------------
# Pin 10: storage formats, exhaustively
# --------------------------------------------------------------------------

def pin_e4m3_table():
    codes = np.arange(256, dtype=np.uint8)
    mine = pa.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    if not np.array_equal(np.isnan(mine), np.isnan(ref)):
        return math.inf
    ok = ~np.isnan(ref)
    return float(np.abs(mine[ok] - ref[ok]).max())


def pin_bf16_table():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = pa.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    if not np.array_equal(np.isnan(mine), np.isnan(ref)):
        return math.inf
    ok = ~np.isnan(ref)
    if not np.array_equal(np.isinf(mine[ok]), np.isinf(ref[ok])):
        return math.inf
    fin = ok & np.isfinite(ref)
    return float(np.abs(mine[fin] - ref[fin]).max())


# --------------------------------------------------------------------------
# Pin 6: split + merge == unsplit; lse against scipy; two-stage merge
# --------------------------------------------------------------------------

def pin_split_merge(inp, partition_sizes=(16, 64, 512, 0)):
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, inp.block_size)
    kw = dict(block_size=inp.block_size, softmax_scale=inp.softmax_scale, q_dtype=inp.q_dtype,
              kv_dtype=inp.kv_dtype, k_scales=inp.k_scales, v_scales=inp.v_scales)
    whole = pa.decode_attention(inp.q, kp, vp, inp.block_tables, inp.context_lens, **kw)
    worst = 0.0
    for P in partition_sizes:
        P = P or int(inp.max_context_len)
        maxp = int(-(-inp.max_context_len // P))
        o, lse = pa.decode_partials(inp.q, kp, vp, inp.block_tables, inp.context_lens,
                                    partition_size=P, max_partitions=maxp, **kw)
        worst = max(worst, float(np.abs(pa.merge_partials(o, lse) - whole).max()))
        # two-stage merge: halves first, each half's lse = logsumexp of its parts
        h = max(1, maxp // 2)
        parts_o, parts_l = [], []
        for lo, hi in ((0, h), (h, maxp)):
            if hi <= lo:
                continue
            sub_l = lse[:, :, lo:hi]
            parts_o.append(pa.merge_partials(o[:, :, lo:hi], sub_l))
            with np.errstate(divide="ignore"):
                parts_l.append(logsumexp(sub_l, axis=-1))
        two = pa.merge_partials(np.stack(parts_o, axis=2), np.stack(parts_l, axis=2))
        worst = max(worst, float(np.abs(two - whole).max()))
        # each lse_p against scipy's logsumexp of the partition's scores (torch gather)
        for b in range(min(inp.num_seqs, 3)):
            ctx = int(inp.context_lens[b])
            nb = -(-ctx // inp.block_size)
            ids = torch.from_numpy(inp.block_tables[b, :nb].astype(np.int64))
            K = torch_decode_storage(kp, inp.kv_dtype)[ids]
            if inp.k_scales is not None:
                K = K * torch.from_numpy(inp.k_scales).double()[ids][:, :, None, None]
            K = K.permute(1, 0, 2, 3).reshape(inp.num_kv_heads, nb * inp.block_size, -1)[:, :ctx]
            q = torch_decode_storage(inp.q[b], inp.q_dtype)
            g = inp.group_size
            for i in range(inp.num_q_heads):
                s = (K[i // g] @ q[i]).numpy() * inp.softmax_scale
                for p in range(-(-ctx // P)):
                    ref = logsumexp(s[p * P:(p + 1) * P])
                    worst = max(worst, abs(float(lse[b, i, p]) - ref))
    return worst


def pin_merge_edge_cases():
    """One partition is the identity; empty (-inf) partitions are skipped; all
    empty gives 0."""
    rng = np.random.default_rng(7)
    o = rng.standard_normal((3, 1, 5))
    lse = rng.standard_normal((3, 1))
    worst = float(np.abs(pa.merge_partials(o, lse) - o[:, 0]).max())
    o2 = np.concatenate([o, np.full((3, 2, 5), np.nan)], axis=1)
    lse2 = np.concatenate([lse, np.full((3, 2), -np.inf)], axis=1)
    worst = max(worst, float(np.nan_to_num(np.abs(pa.merge_partials(o2, lse2) - o[:, 0]), nan=np.inf).max()))
    empty = pa.merge_partials(np.full((2, 3, 4), np.nan), np.full((2, 3), -np.inf))
    worst = max(worst, float(np.nan_to_num(np.abs(empty), nan=np.inf).max()))
    return worst


# --------------------------------------------------------------------------
# Pins 2, 4, 5, 7, 8: invariants and closed forms
# --------------------------------------------------------------------------

def _step(inp, k_pool=None, v_pool=None, tables=None, k_new=None, v_new=None,
          k_scales=None, v_scales=None, num_kv_heads=None):
    k_pool = inp.k_pool if k_pool is None else k_pool
    v_pool = inp.v_pool if v_pool is None else v_pool
    tables = inp.block_tables if tables is None else tables
    out, _, _ = pa.decode_step(inp.q, k_pool, v_pool,
                               inp.k_new if k_new is None else k_new,
                               inp.v_new if v_new is None else v_new,
                               tables, inp.context_lens, block_size=inp.block_size,
                               softmax_scale=inp.softmax_scale, q_dtype=inp.q_dtype,
                               kv_dtype=inp.kv_dtype,
                               k_scales=inp.k_scales if k_scales is None else k_scales,
                               v_scales=inp.v_scales if v_scales is None else v_scales)
    return out


def pin_placement_invariance(inp, seed=11):
    """Move every physical block elsewhere and rewrite the tables: the output
    must be bit-identical."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(inp.num_blocks)
    kp = np.empty_like(inp.k_pool)
    vp = np.empty_like(inp.v_pool)
    kp[perm] = inp.k_pool
    vp[perm] = inp.v_pool
    ks = vs = None
    if inp.k_scales is not None:
        ks = np.empty_like(inp.k_scales)
        vs = np.empty_like(inp.v_scales)
        ks[perm] = inp.k_scales
        vs[perm] = inp.v_scales
    tab = np.where(inp.block_tables >= 0, perm[np.maximum(inp.block_tables, 0)], -1).astype(np.int32)
    a = _step(inp)
    b = _step(inp, kp, vp, tab, k_scales=ks, v_scales=vs)
    return 0.0 if np.array_equal(a, b) else float(np.nan_to_num(np.abs(a - b), nan=np.inf).max() or np.inf)


def pin_single_token_is_v(kv_dtype="f32", q_dtype="f32"):
    """ctx = 1: the only weight is exp(0)/1 = 1, so the output is the appended V row."""
    inp = make_inputs(num_seqs=3, num_q_heads=6, num_kv_heads=3, head_dim=64, ctx=("const", 1),
                      pool=("blocks", 16), q_dtype=q_dtype, kv_dtype=kv_dtype, seed=5)
    out = _step(inp)
    v = pa.to_float64(inp.v_new, kv_dtype)                            # [B, Hkv, D]
    if inp.v_scales is not None:
        blk = inp.block_tables[:, 0]
        v = v * inp.v_scales[blk].astype(np.float64)[:, :, None]
    ref = np.repeat(v, inp.group_size, axis=1)
    return 0.0 if np.array_equal(out, ref) else float(np.nan_to_num(np.abs(out - ref), nan=np.inf).max() or np.inf)


def pin_gqa_equals_repeated_mha(kv_dtype="bf16"):
    """Hq = 8 over Hkv = 2 equals Hq = 8 over the K/V heads repeated 4 times
    (query head i reads KV head i // 4)."""
    inp = make_inputs(num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                      ctx=("uniform", 20, 90), pool=("used_fraction", 0.8),
                      q_dtype="bf16", kv_dtype=kv_dtype, seed=9)
    g = inp.group_size
    a = _step(inp)
    rep = dict(k_pool=np.repeat(inp.k_pool, g, axis=1), v_pool=np.repeat(inp.v_pool, g, axis=1),
               k_new=np.repeat(inp.k_new, g, axis=1), v_new=np.repeat(inp.v_new, g, axis=1))
    if inp.k_scales is not None:
        rep["k_scales"] = np.repeat(inp.k_scales, g, axis=1)
        rep["v_scales"] = np.repeat(inp.v_scales, g, axis=1)
    b = _step(inp, **rep)
    return 0.0 if np.array_equal(a, b) else float(np.nan_to_num(np.abs(a - b), nan=np.inf).max() or np.inf)


def _pool_from_contiguous(K, V, bs, rng):
    """Lay contiguous per-sequence caches [B, Hkv, T, D] into a pool of blocks
    of bs tokens at random places; tail slots NaN."""
    B, hkv, T, D = K.shape
    nb = -(-T // bs)
    NB = B * nb + 2
    perm = rng.permutation(NB)
    kp = np.full((NB, hkv, bs, D), np.nan, np.float32)
    vp = np.full((NB, hkv, bs, D), np.nan, np.float32)
    tab = np.full((B, nb), -1, np.int32)
    for b in range(B):
        for j in range(nb):
            blk = perm[b * nb + j]
            tab[b, j] = blk
            lo, hi = j * bs, min((j + 1) * bs, T)
            kp[blk, :, :hi - lo] = K[b, :, lo:hi]
            vp[blk, :, :hi - lo] = V[b, :, lo:hi]
    return kp, vp, tab


def pin_block_size_invariance(T=45, seed=13):
    rng = np.random.default_rng(seed)
    B, hq, hkv, D = 2, 4, 2, 32
    K = rng.standard_normal((B, hkv, T, D)).astype(np.float32)
    V = rng.standard_normal((B, hkv, T, D)).astype(np.float32)
    q = rng.standard_normal((B, hq, D)).astype(np.float32)
    ctx = np.full(B, T, np.int32)
    outs = []
    for bs in (1, 4, 16, T):
        kp, vp, tab = _pool_from_contiguous(K, V, bs, rng)
        outs.append(pa.decode_attention(q, kp, vp, tab, ctx, block_size=bs, softmax_scale=0.3,
                                        q_dtype="f32", kv_dtype="f32"))
    worst = 0.0
    for o in outs[1:]:
        if not np.array_equal(o, outs[0]):
            worst = max(worst, float(np.nan_to_num(np.abs(o - outs[0]), nan=np.inf).max() or np.inf))
    return worst


def pin_closed_forms(seed=17):
    """Equal keys -> mean of V; q = 0 -> mean of V; one key far along q -> that key's V."""
    rng = np.random.default_rng(seed)
    T, D = 29, 64
    V = rng.standard_normal((1, T, D))
    q = rng.standard_normal((1, D))
    K_eq = np.repeat(rng.standard_normal((1, 1, D)), T, axis=1)
    worst = float(np.abs(pa.attend(q, K_eq, V, 0.125) - V[0].mean(axis=0)).max())
    K = rng.standard_normal((1, T, D))
    worst = max(worst, float(np.abs(pa.attend(np.zeros((1, D)), K, V, 0.125) - V[0].mean(axis=0)).max()))
    t_star = 11
    K_dom = K.copy()
    K_dom[0, t_star] = 400.0 * q[0] / np.linalg.norm(q[0]) / np.linalg.norm(q[0]) * 8.0
    # score of t_star = 0.125 * 400 * 8 / 1 = 400; the others are O(1): weights < e^-300
    worst = max(worst, float(np.abs(pa.attend(q, K_dom, V, 0.125) - V[0, t_star]).max()))
    return worst


def pin_weights_sum_to_one(seed=19):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for T in (1, 7, 300, 5000):
        q = rng.standard_normal((4, 32))
        K = rng.standard_normal((2, T, 32)) * 3
        V = rng.standard_normal((2, T, 32))
        _, w = pa.attend(q, K, V, 0.5, return_weights=True)
        if (w < 0).any():
            return math.inf
        worst = max(worst, float(np.abs(w.sum(axis=1) - 1).max()) / (1e-14 * T))
    return worst   # in units of 1e-14 * T


def pin_config_crosscheck(config, seqs=None, **overrides):
    return pin_library_crosscheck(named_config(config, **overrides), seqs)


# --------------------------------------------------------------------------
# Several new tokens per sequence (chunked prefill / verify): shifted causal mask
# --------------------------------------------------------------------------

def pin_chunked_vs_causal(*, schedules, Hq=4, Hkv=2, D=16, bs=4, seed=23):
    """Each sequence s processes its T_s tokens in chunks schedules[s] (all
    sequences advance one chunk per step, ragged): append the chunk's K/V,
    then every query of the chunk attends.  The outputs, in token order, must
    equal full causal attention over the T_s tokens (the KV post's check: a
    6-token prefill then 4 single-token decodes against attention over all 10)."""
    rng = np.random.default_rng(seed)
    n = len(schedules)
    T = [sum(sc) for sc in schedules]
    Tm = max(T)
    q_all = rng.standard_normal((n, Hq, Tm, D)).astype(np.float32)
    k_all = rng.standard_normal((n, Hkv, Tm, D)).astype(np.float32)
    v_all = rng.standard_normal((n, Hkv, Tm, D)).astype(np.float32)
    worst = 0.0
    refs = [_sdpa(torch.from_numpy(q_all[s:s + 1, :, :T[s]]).double(),
                  torch.from_numpy(k_all[s:s + 1, :, :T[s]]).double(),
                  torch.from_numpy(v_all[s:s + 1, :, :T[s]]).double(), is_causal=True).numpy()[0]
            for s in range(n)]
    nbmax = -(-Tm // bs)
    NB = n * nbmax + 3
    free = [int(x) for x in rng.permutation(NB)]
    k_pool = np.full((NB, Hkv, bs, D), np.nan, np.float32)
    v_pool = np.full((NB, Hkv, bs, D), np.nan, np.float32)
    tables = np.full((n, nbmax + 1), -1, np.int32)
    used = [0] * n
    done = [0] * n
    for step in range(max(len(sc) for sc in schedules)):
        t = [schedules[s][step] if step < len(schedules[s]) else 0 for s in range(n)]
        ctx = np.array([done[s] + t[s] for s in range(n)], np.int32)
        for s in range(n):
            while used[s] * bs < ctx[s]:
                tables[s, used[s]] = free.pop()
                used[s] += 1
        qsl = np.concatenate([[0], np.cumsum(t)]).astype(np.int32)
        rows_q = np.concatenate([q_all[s, :, done[s]:done[s] + t[s]].transpose(1, 0, 2) for s in range(n)])
        rows_k = np.concatenate([k_all[s, :, done[s]:done[s] + t[s]].transpose(1, 0, 2) for s in range(n)])
        rows_v = np.concatenate([v_all[s, :, done[s]:done[s] + t[s]].transpose(1, 0, 2) for s in range(n)])
        pa.kv_append_tokens(k_pool, v_pool, rows_k, rows_v, tables, ctx, qsl, bs, inplace=True)
        out = pa.multi_query_attention(rows_q, k_pool, v_pool, tables, ctx, qsl, block_size=bs,
                                       softmax_scale=1.0 / math.sqrt(D), q_dtype="f32",
                                       kv_dtype="f32")
        for s in range(n):
            got = out[qsl[s]:qsl[s + 1]]                              # [t, Hq, D]
            ref = refs[s][:, done[s]:done[s] + t[s]].transpose(1, 0, 2)
            if got.size:
                worst = max(worst, float(np.nan_to_num(np.abs(got - ref), nan=np.inf).max()))
        done = [done[s] + t[s] for s in range(n)]
    return worst


def torch_padded_multi_query(inp, k_pool, v_pool):
    """Padded torch gather + float64 SDPA with each query's mask
    arange(L) < ctx - t + j + 1."""
    bs, D = inp.block_size, inp.head_dim
    qsl = inp.query_start_loc
    out = np.zeros((inp.total_queries, inp.num_q_heads, D))
    kp = torch_decode_storage(k_pool, inp.kv_dtype)
    vp = torch_decode_storage(v_pool, inp.kv_dtype)
    if inp.k_scales is not None:
        kp = kp * torch.from_numpy(inp.k_scales).double()[:, :, None, None]
        vp = vp * torch.from_numpy(inp.v_scales).double()[:, :, None, None]
    q_all = torch_decode_storage(inp.q, inp.q_dtype)
    for b in range(inp.num_seqs):
        ctx = int(inp.context_lens[b])
        t = int(qsl[b + 1] - qsl[b])
        nb = -(-ctx // bs)
        ids = torch.from_numpy(inp.block_tables[b, :nb].astype(np.int64))
        L = nb * bs
        k = kp[ids].permute(1, 0, 2, 3).reshape(inp.num_kv_heads, L, D)[None]
        v = vp[ids].permute(1, 0, 2, 3).reshape(inp.num_kv_heads, L, D)[None]
        keep = torch.arange(L)[None, :] < torch.arange(ctx - t + 1, ctx + 1)[:, None]  # [t, L]
        valid = torch.arange(L) < ctx
        k = torch.where(valid[None, None, :, None], k, torch.zeros_like(k))
        v = torch.where(valid[None, None, :, None], v, torch.zeros_like(v))
        q = q_all[qsl[b]:qsl[b + 1]].permute(1, 0, 2)[None]                            # [1, Hq, t, D]
        o = _sdpa(q, k, v, attn_mask=keep[None, None], scale=inp.softmax_scale)
        out[qsl[b]:qsl[b + 1]] = o[0].permute(1, 0, 2).numpy()
    return out


def pin_multi_query_library(inp):
    kp, vp = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                                 inp.context_lens, inp.query_start_loc, inp.block_size)
    ref = torch_padded_multi_query(inp, kp, vp)
    out = pa.multi_query_attention(inp.q, kp, vp, inp.block_tables, inp.context_lens,
                                   inp.query_start_loc, block_size=inp.block_size,
                                   softmax_scale=inp.softmax_scale, q_dtype=inp.q_dtype,
                                   kv_dtype=inp.kv_dtype, k_scales=inp.k_scales,
                                   v_scales=inp.v_scales)
    return float(np.nan_to_num(np.abs(out - ref), nan=np.inf).max())
