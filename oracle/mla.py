"""CPU float64 oracle: multi-head latent attention (MLA) decode over a paged
latent cache, in its absorbed form.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP kernels.

From the pages (KV-cache post, "MLA: how does decode get full-size keys and
values back?"; serving lesson, "Smaller caches: GQA, MQA, MLA and quantized
caches"; 4yush post, "Compressing it (MLA)"):

* Each token caches one latent vector c = W_DKV h of d_c = 512 numbers plus
  a 64-number rotary key part shared by all heads: 576 numbers per token and
  layer, against 2 x 128 heads x 128 = 32,768 for standard multi-head
  attention.  Head i's key is k_i = [W_UK,i c ; k_rope] and its value
  v_i = W_UV,i c.

* Expand: rebuild every token's full keys and values and run ordinary
  attention.  Absorb (what decode does): everything is linear, so
  q_i . k_i,t = [W_UK,i^T q_nope,i ; q_rope,i] . [c_t ; k_rope,t] and
  sum_t p_t v_i,t = W_UV,i (sum_t p_t c_t).  Every head then attends over the
  one shared 576-number row per token (key = the whole row, value = its first
  d_c numbers), like multi-query attention with a wide head, and the latent
  output is projected up once.

``mla_decode_absorbed`` is that attention over the paged latent cache (the
part the kernel computes); ``absorb_query`` / ``project_out`` are the two
folded projections; ``mla_decode_expanded`` is the expand form, written
independently as ordinary per-head attention over rebuilt K and V, which the
pins compare against.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import gather_sequence, to_float64


def mla_decode_absorbed(q_abs, latent_pool, block_tables, context_lens, *, block_size,
                        softmax_scale, kv_lora_rank, dtype, seqs=None):
    """q_abs [B, H, d_c + d_r] (storage format), latent_pool [NB, block_size,
    d_c + d_r] -> latent outputs [B, H, d_c] float64.

    For head i of sequence b: s_t = scale * q_abs[b, i] . row_t over its ctx
    cached rows, p = softmax(s), out = sum_t p_t row_t[:d_c].  ctx = 0 gives 0."""
    B, H, _ = q_abs.shape
    out = np.zeros((B, H, kv_lora_rank))
    pool4 = latent_pool[:, None]                       # one shared "KV head"
    for b in (range(B) if seqs is None else seqs):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        rows = gather_sequence(pool4, block_tables[b], ctx, block_size, dtype)[0]   # [T, 576]
        q = to_float64(q_abs[b], dtype)                                            # [H, 576]
        for i in range(H):
            s = softmax_scale * (rows @ q[i])
            p = np.exp(s - s.max())
            out[b, i] = (p @ rows[:, :kv_lora_rank]) / p.sum()
    return out


def absorb_query(q_nope, q_rope, w_uk):
    """q_nope [H, d_h], q_rope [H, d_r], W_UK [H, d_h, d_c] ->
    q_abs [H, d_c + d_r] = [W_UK,i^T q_nope,i ; q_rope,i] (float64)."""
    lat = np.einsum("hkc,hk->hc", np.asarray(w_uk, np.float64), np.asarray(q_nope, np.float64))
    return np.concatenate([lat, np.asarray(q_rope, np.float64)], axis=1)


def project_out(o_lat, w_uv):
    """o_lat [H, d_c], W_UV [H, d_h, d_c] -> per-head outputs [H, d_h] = W_UV,i o_lat,i."""
    return np.einsum("hkc,hc->hk", np.asarray(w_uv, np.float64), np.asarray(o_lat, np.float64))


def mla_decode_expanded(q_nope, q_rope, latents, rope_keys, w_uk, w_uv, softmax_scale):
    """The expand form for one sequence: latents [T, d_c], rope_keys [T, d_r];
    K_i = [latents W_UK,i^T ; rope_keys], V_i = latents W_UV,i^T; ordinary
    softmax attention per head.  Returns [H, d_h] float64."""
    c = np.asarray(latents, np.float64)
    kr = np.asarray(rope_keys, np.float64)
    H = w_uk.shape[0]
    out = np.zeros((H, w_uv.shape[1]))
    for i in range(H):
        K = np.concatenate([c @ np.asarray(w_uk[i], np.float64).T, kr], axis=1)   # [T, d_h + d_r]
        V = c @ np.asarray(w_uv[i], np.float64).T                                 # [T, d_h]
        q = np.concatenate([np.asarray(q_nope[i], np.float64), np.asarray(q_rope[i], np.float64)])
        s = softmax_scale * (K @ q)
        p = np.exp(s - s.max())
        out[i] = (p @ V) / p.sum()
    return out
