"""The CPU oracle against what the pages and the mathematics fix (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import oracle.paged_attention as pa
from tests import oracle_pins as pins
from workloads import make_inputs, named_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# Pin 1 -----------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,bs,T", [(4, 4, 4, 40), (4, 2, 4, 37), (8, 2, 16, 33), (3, 1, 1, 12)])
def test_cached_decode_equals_full_causal(Hq, Hkv, bs, T):
    assert pins.pin_incremental_vs_causal(Hq=Hq, Hkv=Hkv, bs=bs, T=T) < 1e-12


# Pin 9 -----------------------------------------------------------------------

def test_library_crosscheck_config1_full():
    assert pins.pin_config_crosscheck(1) < 1e-12


@pytest.mark.parametrize("config", [2, 4])
def test_library_crosscheck_bf16_shapes(config):
    assert pins.pin_config_crosscheck(config, num_seqs=5) < 1e-12


def test_library_crosscheck_fp8():
    assert pins.pin_config_crosscheck(5, num_seqs=3, ctx=("uniform", 17, 300)) < 1e-12


def test_library_crosscheck_long_context_sample():
    inp = named_config(3, num_seqs=1, ctx=("const", 8192 + 37))
    assert pins.pin_library_crosscheck(inp) < 1e-12


# Pin 10 ----------------------------------------------------------------------

def test_e4m3_decode_exhaustive():
    assert pins.pin_e4m3_table() == 0.0


def test_e4m3_known_codes():
    # bias 7, max normal 448 = 1.75 * 2^8, min subnormal 2^-9, NaN at S.1111.111
    vals = pa.decode_e4m3fn(np.array([0x00, 0x01, 0x08, 0x38, 0x7E, 0xFE, 0x80], np.uint8))
    assert list(vals) == [0.0, 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -448.0, 0.0]
    assert np.isnan(pa.decode_e4m3fn(np.array([0x7F, 0xFF], np.uint8))).all()


def test_bf16_decode_exhaustive():
    assert pins.pin_bf16_table() == 0.0


# Pin 6 -----------------------------------------------------------------------

def test_split_merge_equals_unsplit():
    inp = named_config(2, num_seqs=3, ctx=("uniform", 100, 1500))
    assert pins.pin_split_merge(inp) < 1e-13


def test_split_merge_fp32_config1():
    assert pins.pin_split_merge(named_config(1)) < 1e-13


def test_merge_edge_cases():
    assert pins.pin_merge_edge_cases() == 0.0


# Pins 2, 3, 4, 5, 7, 8 -------------------------------------------------------

@pytest.mark.parametrize("config,over", [(1, {}), (2, dict(num_seqs=4)),
                                          (5, dict(num_seqs=3, ctx=("uniform", 40, 200)))])
def test_placement_invariance(config, over):
    assert pins.pin_placement_invariance(named_config(config, **over)) == 0.0


def test_weights_sum_to_one():
    assert pins.pin_weights_sum_to_one() <= 1.0


@pytest.mark.parametrize("kv,q", [("f32", "f32"), ("bf16", "bf16"), ("fp8_e4m3", "bf16")])
def test_single_token_context_returns_v(kv, q):
    assert pins.pin_single_token_is_v(kv, q) == 0.0


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3", "f32"])
def test_gqa_equals_repeated_mha(kv):
    assert pins.pin_gqa_equals_repeated_mha(kv) == 0.0


def test_block_size_invariance():
    assert pins.pin_block_size_invariance() == 0.0


def test_closed_forms():
    assert pins.pin_closed_forms() < 1e-13


# Worked examples printed on the pages ---------------------------------------

def test_locker_addressing_golden():
    g = _golden("kv_post_lockers.json")
    bs = g["block_size"]
    for case in g["cases"]:
        table = np.array(case["table"], np.int32)
        assert pa.slot_of(table, case["position"], bs) == (case["block"], case["slot"])
        # the append writes there and nowhere else
        NB, H, D = 8, 2, 3
        kp = np.zeros((NB, H, bs, D), np.float32)
        vp = np.zeros((NB, H, bs, D), np.float32)
        kn = np.full((1, H, D), 5.0, np.float32)
        kp2, vp2 = pa.kv_append(kp, vp, kn, -kn, table[None], np.array([case["position"] + 1]), bs)
        touched = np.argwhere(kp2 != 0)
        assert {(int(b), int(s)) for b, _, s, _ in touched} == {(case["block"], case["slot"])}
        assert (vp2[case["block"], :, case["slot"]] == -5.0).all()


def test_hundred_token_prompt_blocks_golden():
    """100 tokens in 16-token blocks: 7 blocks, 6 full and 4 tokens in the last;
    the gather reads exactly those, never the padding or the tail slots."""
    g = _golden("serving_lesson_numbers.json")["exercise_parallel_sampling"]
    bs, n = g["block"], g["prompt_tokens"]
    NB, H, D = 12, 1, 4
    pool = np.full((NB, H, bs, D), np.nan, np.float32)
    ids = [3, 9, 0, 5, 11, 2, 7]
    assert len(ids) == g["blocks"]
    for j, blk in enumerate(ids):
        fill = bs if j < g["full_blocks"] else g["tokens_in_last_block"]
        pool[blk, :, :fill] = j + 1
    table = np.array(ids + [-1, -1], np.int32)
    seq = pa.gather_sequence(pool, table, n, bs, "f32")
    assert seq.shape == (H, n, D)
    assert not np.isnan(seq).any()
    assert (seq[0, -g["tokens_in_last_block"]:, 0] == g["blocks"]).all()


def test_decode_mask_all_ones():
    """Decode has no causal mask beyond ctx: with start = 6 cached tokens and
    one new one, the new query sees all 7 keys (4yush.com, 'Adding the cache to
    GPT-2').  A key placed at the newest position with a dominant score must
    therefore win."""
    inp = make_inputs(num_seqs=1, num_q_heads=2, num_kv_heads=2, head_dim=64, ctx=("const", 7),
                      pool=("blocks", 4), q_dtype="f32", kv_dtype="f32", seed=3)
    qv = pa.to_float64(inp.q[0], "f32")
    inp.k_new[0] = (200.0 * qv / (qv * qv).sum(axis=1, keepdims=True) * 8).astype(np.float32)
    out = pins._step(inp)
    assert np.abs(out[0] - inp.v_new[0].astype(np.float64)).max() < 1e-12


def test_empty_context_gives_zeros():
    inp = make_inputs(num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=64,
                      ctx=("fixed", [5, 0, 9]), pool=("blocks", 4), q_dtype="f32",
                      kv_dtype="f32", seed=1)
    out = pins._step(inp)
    assert (out[1] == 0).all() and np.isfinite(out).all()


def test_workload_recipes_shapes():
    """The named workloads have the shapes and length mixes they are named for."""
    c1 = named_config(1)
    assert list(c1.context_lens) == [17, 33, 64, 100] and c1.num_blocks == 64
    assert c1.k_pool.dtype == np.float32 and c1.head_dim == 64
    # new-token offsets in their blocks: first slot, first slot, last slot, 4th slot
    assert [int((c - 1) % 16) for c in c1.context_lens] == [0, 0, 15, 3]
    c2 = named_config(2, num_seqs=64)
    assert c2.context_lens.min() >= 512 and c2.context_lens.max() <= 4096
    assert c2.num_blocks == int((-(-c2.context_lens // 16)).sum())
    c4 = named_config(4, num_seqs=256, head_dim=64, num_q_heads=4, num_kv_heads=1)
    used = int((-(-c4.context_lens // 16)).sum())
    assert c4.num_blocks == math.ceil(used / 0.7)
    assert 700 < np.median(c4.context_lens) < 1400
    c5 = named_config(5, num_seqs=2, ctx=("const", 64))
    assert c5.k_scales.shape == (c5.num_blocks, 32) and c5.k_pool.dtype == np.uint8


# Several new tokens per sequence ----------------------------------------------

@pytest.mark.parametrize("schedules,Hq,Hkv,bs", [
    ([[6, 1, 1, 1, 1]], 4, 4, 4),                                   # the KV post's own check
    ([[6, 1, 1, 1, 1], [3, 3, 3, 1], [1, 1, 8, 2]], 4, 2, 4),       # ragged chunks, GQA
    ([[17, 16, 1, 5], [40], [1] * 12], 8, 2, 16),                   # a whole prefill, blocks of 16
])
def test_chunked_equals_full_causal(schedules, Hq, Hkv, bs):
    assert pins.pin_chunked_vs_causal(schedules=schedules, Hq=Hq, Hkv=Hkv, bs=bs) < 1e-12


def test_visibility_golden():
    g = _golden("gpt2_cache_masks.json")
    for case in g["cases"]:
        start, t = case["start"], case["new"]
        for j, row in enumerate(case["mask"]):
            assert pa.visible_tokens(start + t, t, j) == sum(row)
            assert row == [1] * sum(row) + [0] * (len(row) - sum(row))


@pytest.mark.parametrize("kv,q", [("bf16", "bf16"), ("fp8_e4m3", "bf16"), ("f32", "f32")])
def test_multi_query_library_crosscheck(kv, q):
    inp = make_inputs(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                      ctx=("uniform", 1, 700), pool=("used_fraction", 0.8), q_dtype=q,
                      kv_dtype=kv, seed=41, new_tokens=("uniform", 1, 9))
    assert pins.pin_multi_query_library(inp) < 1e-12


def test_one_new_token_is_decode():
    inp = named_config(2, num_seqs=3)
    qsl = np.arange(4, dtype=np.int32)
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, 16)
    kw = dict(block_size=16, softmax_scale=inp.softmax_scale, q_dtype="bf16", kv_dtype="bf16")
    a = pa.decode_attention(inp.q, kp, vp, inp.block_tables, inp.context_lens, **kw)
    b = pa.multi_query_attention(inp.q, kp, vp, inp.block_tables, inp.context_lens, qsl, **kw)
    assert np.array_equal(a, b)
