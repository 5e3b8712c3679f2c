"""CPU oracle: appending new K/V rows to an fp8 (e4m3) paged cache,
quantising them on the way in.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP kernels.

The pages say only that storing the cache in 8-bit floats halves its bytes
(KV-cache post, "The KV cache is big": fewer bytes per number; serving
lesson, "Smaller caches: GQA, MQA, MLA and quantized caches" and "Where it
shows up"; 4yush post, ways to shrink the cache).  Everything below is the
plainest reading that the rest of this library supports:

* Format: OCP float8 e4m3fn (bias 7, 3 mantissa bits, subnormals, no
  infinities, S.1111.111 is NaN, largest finite 448).  A stored code c of a
  (block, KV head) slice means the real value ``decode(c) * scale``.

* ``encode_e4m3fn``: float32 -> code by rounding to the nearest e4m3 value,
  ties to the even code, saturating at +-448 (an infinity also saturates);
  NaN gives 0x7F.  Written out from the format, not from any library cast.

* Quantising a value x for a slice with scale s is ``encode(f32(x / s))``:
  one float32 division, correctly rounded, then the rounding above.  The
  decision is taken in float32 on both sides (the new rows arrive as bf16 or
  float32, and scales are float32).

* ``SCALE_FIXED``: each slice keeps the scale its block was given when it
  was allocated; new rows are quantised with it (values beyond 448 * s
  saturate).

* ``SCALE_RUNNING_AMAX``: the slice's scale grows to cover the new rows.
  For the new rows landing in one slice: amax = max |x| over them (float32),
  candidate = f32(amax / 448); the slice's earlier rows are those before the
  first new row's slot, and if there are none the old scale is ignored
  (treated as 0: a freshly allocated block).  new scale = max(old, candidate).
  If it grew and earlier rows exist, each earlier code is requantised:
  ``encode(f32(f32(decode(c) * old) / new))``.  The new rows are then
  quantised with the new scale; a scale of 0 (every value so far is 0) stores
  code 0.  Scales never shrink.

Placement (which slot a row goes to) is that of ``kv_append_tokens``:
row qsl[b] + j of sequence b goes to position ctx_b - t_b + j; rows at a
negative position, and sequences with ctx <= 0 or past the table's capacity,
are skipped.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import decode_e4m3fn

SCALE_FIXED = 0
SCALE_RUNNING_AMAX = 1
E4M3_MAX = 448.0


def encode_e4m3fn(x) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8): round to nearest, ties to even
    code, saturate at +-448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    for i, v in enumerate(flat.tolist()):
        res[i] = _encode_one(v)
    return out


def _encode_one(v: float) -> int:
    if v != v:
        return 0x7F
    sign = 0x80 if (v < 0 or (v == 0 and np.signbit(v))) else 0
    a = abs(v)
    if a >= E4M3_MAX:
        return sign | 0x7E
    # the exponent of a in the e4m3 grid: normal for a >= 2**-6
    if a < 2.0 ** -6:
        q = _round_half_even(a / 2.0 ** -9)            # subnormal quantum 2**-9; q in 0..8
        return sign | q                                 # q = 8 is the code of 2**-6
    e = int(np.floor(np.log2(a)))
    if 2.0 ** e > a:                                    # guard log2 rounding
        e -= 1
    elif 2.0 ** (e + 1) <= a:
        e += 1
    q = _round_half_even(a / 2.0 ** (e - 3))           # 8 <= q <= 16
    if q == 16:
        e, q = e + 1, 8
    code = ((e + 7) << 3) | (q - 8)
    return sign | min(code, 0x7E)


def _round_half_even(y: float) -> int:
    """Nearest integer to y (exact in float64 here), ties to even."""
    f = np.floor(y)
    d = y - f
    if d > 0.5 or (d == 0.5 and int(f) % 2 == 1):
        f += 1
    return int(f)


def quantize(x, scale) -> np.ndarray:
    """Codes of the real values x (float32) for a slice with float32 scale s:
    encode(f32(x / s))."""
    x = np.asarray(x, dtype=np.float32)
    return encode_e4m3fn(x / np.float32(scale))


def _positions(context_lens, query_start_loc, b, max_blocks, block_size):
    ctx = int(context_lens[b])
    if query_start_loc is None:
        q0, q1 = b, b + 1
    else:
        q0, q1 = int(query_start_loc[b]), int(query_start_loc[b + 1])
    t = q1 - q0
    if ctx <= 0 or ctx > max_blocks * block_size:
        return []
    return [(q0 + j, ctx - t + j) for j in range(t) if ctx - t + j >= 0]


def kv_append_quant(k_pool, v_pool, k_scales, v_scales, k_new, v_new, block_tables,
                    context_lens, block_size, mode, query_start_loc=None):
    """Quantise and append.  Pools: uint8 codes [NB, Hkv, bs, D]; scales
    float32 [NB, Hkv]; k_new/v_new float32 values [rows, Hkv, D] (a bf16 input
    is widened exactly first).  Returns new (k_pool, v_pool, k_scales,
    v_scales); the inputs are not modified."""
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    k_scales = np.asarray(k_scales, np.float32).copy()
    v_scales = np.asarray(v_scales, np.float32).copy()
    k_new = np.asarray(k_new, np.float32)
    v_new = np.asarray(v_new, np.float32)
    hkv = k_pool.shape[1]
    B, max_blocks = block_tables.shape
    for b in range(B):
        rows = _positions(context_lens, query_start_loc, b, max_blocks, block_size)
        if not rows:
            continue
        # group the rows by the block they land in, in order
        by_block = {}
        for r, pos in rows:
            by_block.setdefault(pos // block_size, []).append((r, pos % block_size))
        for lblk, items in by_block.items():
            phys = int(block_tables[b, lblk])
            if not 0 <= phys < k_pool.shape[0]:
                continue
            n_old = items[0][1]                       # slots before the first new row
            for pool, scales, new in ((k_pool, k_scales, k_new), (v_pool, v_scales, v_new)):
                for h in range(hkv):
                    _append_slice(pool, scales, new, phys, h, items, n_old, mode)
    return k_pool, v_pool, k_scales, v_scales


def _append_slice(pool, scales, new, phys, h, items, n_old, mode):
    if mode == SCALE_FIXED:
        s = scales[phys, h]
        for r, slot in items:
            pool[phys, h, slot] = quantize(new[r, h], s)
        return
    if mode != SCALE_RUNNING_AMAX:
        raise ValueError(mode)
    vals = np.stack([new[r, h] for r, _ in items])
    amax = np.float32(np.abs(vals).max())
    cand = np.float32(amax / np.float32(E4M3_MAX))
    old = scales[phys, h] if n_old > 0 else np.float32(0.0)
    s = np.float32(max(old, cand))
    if s > old and n_old > 0:
        prev = decode_e4m3fn(pool[phys, h, :n_old]).astype(np.float32)
        real = (prev * old).astype(np.float32)
        pool[phys, h, :n_old] = encode_e4m3fn(real / s)
    scales[phys, h] = s
    for r, slot in items:
        pool[phys, h, slot] = 0 if s == 0 else quantize(new[r, h], s)
