"""GPU parity of several new tokens per sequence: pkv_kv_append_tokens then
pkv_paged_multi_query_attention, against the oracle's kv_append_tokens and
multi_query_attention (the causal mask shifted by the cache length).

Covers both kernels (matrix cores for bf16 over bf16 with 2+ queries per KV
head, the vector kernel otherwise), column tiles that span several new tokens
and a ragged last tile, partition boundaries inside the new tokens,
sequences with no new token, rows that see nothing, a prompt prefilled in
chunks, the one-token case against the decode entry point bit for bit, and
the balanced split (partial rows [slot, max_query_len, Hq]) on the same
cases."""

import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
from tests.gpu_util import (DeviceMultiStep, DeviceStep, check_tolerance, dev_tensor,
                            host_storage, log, oracle_multi)
from workloads import make_inputs, named_config

pytestmark = pytest.mark.gpu
BAL = -1                             # PKV_PARTITION_BALANCED


def _shape(config, **over):
    """A named workload's head layout and dtypes, with a small batch."""
    from workloads.configs import recipe
    r = recipe(config)
    r.update(over)
    return r


def _same_bits(a, b):
    """Bitwise equality (the pools hold NaN poison, which == would reject)."""
    return a.dtype == b.dtype and a.shape == b.shape and np.array_equal(
        np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def _check(inp, label, partition_size=None):
    log(f"[case] {label}: B={inp.num_seqs} T={inp.total_queries} maxq={inp.max_new_tokens} "
        f"g={inp.group_size} D={inp.head_dim} {inp.q_dtype}/{inp.kv_dtype} "
        f"P={inp.partition_size if partition_size is None else partition_size}")
    dev = DeviceMultiStep(inp)
    gpu = dev.step(partition_size).detach().float().cpu().double().numpy()
    pools = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                                inp.context_lens, inp.query_start_loc, inp.block_size)
    ref = oracle_multi(inp, pools)
    check_tolerance(inp.kv_dtype, gpu, ref, label, out_dtype=inp.q_dtype)
    # the append is a bitwise scatter: the pools match the oracle's exactly
    assert _same_bits(host_storage(dev.k_pool), pools[0])
    assert _same_bits(host_storage(dev.v_pool), pools[1])
    return dev, gpu, ref


@pytest.mark.parametrize("t", [1, 2, 4, 5, 8, 16])
def test_fixed_new_tokens_f32(t):
    """Tiny f32 MHA workload (vector kernel), every sequence with t new tokens."""
    r = _shape(1)
    r["ctx"] = ("fixed", [17, 33, 64, 100])
    inp = make_inputs(seed=10 + t, name=f"tiny_f32_t{t}", new_tokens=("const", t), **r)
    _check(inp, f"f32 t={t}")
    _check(inp, f"f32 t={t} P=32", partition_size=32)
    _check(inp, f"f32 t={t} balanced", partition_size=BAL)


@pytest.mark.parametrize("t", [1, 2, 4, 5, 8, 16])
def test_fixed_new_tokens_gqa_bf16(t):
    """Llama-3-8B heads (g=4) in bf16: the matrix-core kernel; 16-column tiles
    hold 4 new tokens, so t=5 leaves a ragged tile."""
    inp = named_config(2, seed=20 + t, num_seqs=6, ctx=("uniform", 16, 1400),
                       new_tokens=("const", t), name=f"gqa_bf16_t{t}")
    _check(inp, f"gqa bf16 t={t} balanced (the workload's default)")
    _check(inp, f"gqa bf16 t={t} P=64", partition_size=64)


@pytest.mark.parametrize("group,head_dim,dtypes", [
    (1, 128, ("bf16", "bf16")),      # MHA: the matrix cores serve t tokens of one head
    (1, 128, ("bf16", "fp8_e4m3")),  # fp8 MHA (vector kernel)
    (4, 128, ("f32", "bf16")),
    (8, 64, ("bf16", "bf16")),
    (8, 64, ("f32", "f32")),
    (2, 64, ("bf16", "fp8_e4m3")),
])
def test_group_and_dtype_mix(group, head_dim, dtypes):
    qd, kd = dtypes
    hkv = 4
    inp = make_inputs(num_seqs=5, num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=head_dim,
                      ctx=("uniform", 1, 700), pool=("used_fraction", 0.8), q_dtype=qd,
                      kv_dtype=kd, partition_size=128, seed=30 + group,
                      new_tokens=("uniform", 1, 9), name=f"g{group}_d{head_dim}_{qd}_{kd}")
    _check(inp, inp.name)
    _check(inp, inp.name + " balanced", partition_size=BAL)


def test_ragged_new_tokens_and_empty_sequences():
    """t_b from 0 to 33 in one batch: sequences with no new token produce no
    rows; a 33-token tail spans three 16-column tiles even at g=1 ... g=4."""
    r = _shape(2, num_seqs=7, ctx=("fixed", [5, 300, 40, 1030, 33, 600, 100]))
    r["new_tokens"] = ("fixed", [3, 0, 33, 1, 16, 0, 7])
    inp = make_inputs(seed=41, name="ragged", **r)
    assert inp.total_queries == 60
    _check(inp, "ragged bf16 P=512")
    _check(inp, "ragged bf16 P=32", partition_size=32)
    _check(inp, "ragged bf16 balanced", partition_size=BAL)
    r.update(q_dtype="f32", kv_dtype="f32")
    _check(make_inputs(seed=41, name="ragged_f32", **r), "ragged f32", partition_size=48)


def test_prefill_from_empty_cache():
    """ctx == t: the whole prompt is new (plain causal attention)."""
    inp = named_config(2, seed=50, num_seqs=3, ctx=("fixed", [40, 77, 16]),
                       new_tokens=("fixed", [40, 77, 16]), name="prefill")
    _check(inp, "prefill bf16")
    _check(inp, "prefill bf16 P=16", partition_size=16)


def test_rows_that_see_nothing():
    """A context shorter than the new tokens (ctx < t): rows whose position
    would be negative are not appended and attend to nothing (zeros)."""
    r = _shape(1)
    inp = make_inputs(seed=60, name="short", ctx=("fixed", [20, 40, 64, 100]),
                      new_tokens=("fixed", [6, 2, 9, 4]),
                      **{k: v for k, v in r.items() if k != "ctx"})
    inp.context_lens[0] = 3          # 6 new rows, 3 positions: rows 0..2 see nothing
    inp.context_lens[2] = 5
    _, gpu, ref = _check(inp, "ctx < t")
    assert np.all(gpu[0:3] == 0) and np.all(ref[0:3] == 0)
    _, gpu, ref = _check(inp, "ctx < t balanced", partition_size=BAL)
    assert np.all(gpu[0:3] == 0)


def test_one_token_matches_decode_entry_point():
    """With t_b = 1 everywhere the multi-token entry point computes exactly
    what the decode entry point does (same kernels, same rounding) at the same
    fixed partition size."""
    for cfg, label in ((2, "gqa bf16"), (5, "fp8 mha"), (1, "f32")):
        over = dict(num_seqs=8) if cfg != 1 else {}
        if cfg == 5:
            over["ctx"] = ("uniform", 100, 1500)
        one = named_config(cfg, seed=70 + cfg, **over)
        multi = named_config(cfg, seed=70 + cfg, new_tokens=("const", 1), **over)
        assert np.array_equal(one.context_lens, multi.context_lens)
        assert _same_bits(one.q, multi.q) and _same_bits(one.k_new, multi.k_new)
        a = DeviceStep(one).step(512).detach().cpu()
        dm = DeviceMultiStep(multi)
        b = dm.step(512).detach().cpu()
        log(f"[case] t=1 {label}: bit-identical {torch.equal(a, b)}")
        assert torch.equal(a, b), label


def test_chunked_prefill_equals_one_pass():
    """A prompt written and attended in chunks (6, 1, 1, 9, 16, 3 tokens) gives
    the oracle's one-pass causal attention over the whole prompt, row by row."""
    chunks = [6, 1, 1, 9, 16, 3]
    total = sum(chunks)
    full = named_config(2, seed=80, num_seqs=1, ctx=("const", total),
                        new_tokens=("const", total), name="prefill_one_pass")
    ref = oracle_multi(full)
    dev = DeviceMultiStep(full)
    rows = []
    done = 0
    qsl = torch.zeros(2, dtype=torch.int32, device="cuda")
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    from paged_kv_cache_25_amd import ops
    for c in chunks:
        qsl[1] = c
        lens[0] = done + c
        sl = slice(done, done + c)
        q = dev.q[sl].contiguous()
        out = torch.empty_like(q)
        ops.kv_append_tokens(dev.k_pool, dev.v_pool, dev.k_new[sl].contiguous(),
                             dev.v_new[sl].contiguous(), dev.tables, lens, qsl)
        ops.paged_multi_query_attention(out, q, dev.k_pool, dev.v_pool, dev.tables, lens, qsl,
                                        c, done + c, full.softmax_scale, 16)
        torch.cuda.synchronize()
        rows.append(out.float().cpu().double().numpy())
        done += c
    gpu = np.concatenate(rows)
    check_tolerance("bf16", gpu, ref, "chunked prefill")


@pytest.mark.parametrize("t", [4, 16])
def test_batch64_new_tokens_full(t):
    """The Llama-3-8B batch-64 layer with t new tokens per sequence (t = 4: three
    drafts and the token before them, as a verify pass sees them; t = 16: a
    chunk of a prompt), at full size in the launch configuration the
    benchmark times (the balanced split; at t = 16 its 32,768 merged rows go
    through the merge's several-items-per-workgroup shape): every row of every
    sequence against the oracle."""
    inp = named_config(2, new_tokens=("const", t), name=f"llama3_8b_b64_t{t}")
    dev = DeviceMultiStep(inp)
    gpu = dev.step().detach().float().cpu().double().numpy()
    pools = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                                inp.context_lens, inp.query_start_loc, inp.block_size)
    assert _same_bits(host_storage(dev.k_pool), pools[0])
    assert _same_bits(host_storage(dev.v_pool), pools[1])
    ref = np.zeros_like(gpu)
    for b in range(inp.num_seqs):
        q0, q1 = int(inp.query_start_loc[b]), int(inp.query_start_loc[b + 1])
        ref[q0:q1] = pa.multi_query_attention(inp.q[q0:q1], pools[0], pools[1],
                                              inp.block_tables[b:b + 1], inp.context_lens[b:b + 1],
                                              np.array([0, q1 - q0]), block_size=inp.block_size,
                                              softmax_scale=inp.softmax_scale, q_dtype=inp.q_dtype,
                                              kv_dtype=inp.kv_dtype)
    check_tolerance("bf16", gpu, ref, f"batch-64 t={t} (all {inp.num_seqs} sequences)",
                    out_dtype="bf16")


@pytest.mark.parametrize("kv,q,P", [("bf16", "bf16", 64), ("f32", "f32", 32),
                                    ("fp8_e4m3", "bf16", 128)])
def test_partials_match_oracle_and_merge(kv, q, P):
    """pkv_paged_multi_query_partials against the oracle's per-partition
    results of each row's visible prefix; partitions a row does not see carry
    lse = -inf; merging the partials gives the attention call bit for bit."""
    from paged_kv_cache_25_amd import ops
    inp = make_inputs(num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                      ctx=("fixed", [3, 300, 40, 520]), pool=("used_fraction", 0.8),
                      q_dtype=q, kv_dtype=kv, seed=90, new_tokens=("fixed", [5, 1, 19, 8]))
    inp.context_lens[0] = 3               # ctx < t: two rows see nothing
    maxp = -(-inp.max_context_len // P)
    log(f"[case] multi partials kv={kv} q={q} P={P} maxP={maxp}")
    dev = DeviceMultiStep(inp)
    dev.append()
    R = inp.total_queries
    po = torch.full((R, 8, maxp, 128), float("nan"), device="cuda")
    pl = torch.full((R, 8, maxp), float("nan"), device="cuda")
    ops.paged_multi_query_partials(po, pl, dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.lens,
                                   dev.qsl, inp.max_new_tokens, inp.softmax_scale, P,
                                   dev.k_scales, dev.v_scales)
    torch.cuda.synchronize()
    got_l = pl.cpu().double().numpy()
    got_o = po.cpu().double().numpy()
    kp, vp = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                                 inp.context_lens, inp.query_start_loc, inp.block_size)
    tol_l = 1e-5 if kv == "f32" else 2e-3
    tol_o = 1e-5 if kv == "f32" else (2e-2 if kv == "bf16" else 6e-2)
    for b in range(inp.num_seqs):
        ctx = int(inp.context_lens[b])
        q0, q1 = int(inp.query_start_loc[b]), int(inp.query_start_loc[b + 1])
        K = pa.gather_sequence(kp, inp.block_tables[b], ctx, 16, kv, inp.k_scales)
        V = pa.gather_sequence(vp, inp.block_tables[b], ctx, 16, kv, inp.v_scales)
        for j in range(q1 - q0):
            r = q0 + j
            n = pa.visible_tokens(ctx, q1 - q0, j)
            seen = -(-n // P) if n > 0 else 0
            assert np.all(np.isneginf(got_l[r, :, seen:])), (b, j)
            if seen == 0:
                continue
            o_ref, l_ref = pa.partition_partials(pa.to_float64(inp.q[r], q), K[:, :n], V[:, :n],
                                                 inp.softmax_scale, P)
            assert np.abs(got_l[r, :, :seen] - l_ref).max() < tol_l, (b, j)
            assert np.abs(got_o[r, :, :seen] - o_ref).max() < tol_o, (b, j)
    merged = torch.empty_like(dev.q)
    ops.merge_partials(merged, po, pl)
    whole = dev.attend(P).clone()
    torch.cuda.synchronize()
    check_tolerance(kv, merged.float().cpu().double().numpy(), oracle_multi(inp, (kp, vp)),
                    f"multi partials+merge {kv}", out_dtype=q)
    assert torch.equal(merged, whole)


@pytest.mark.parametrize("kv,q", [("bf16", "bf16"), ("f32", "f32"), ("fp8_e4m3", "bf16")])
def test_balanced_partials_planned_match_chunk_oracle(kv, q):
    """pkv_paged_multi_query_partials_planned: the schedule's chunk starts are
    those of the definition, every (slot, new token, head) row is the oracle's
    attention restricted to the chunk's tokens that the token sees (-inf when
    it sees none), and the log-sum-exp merge of each row over its sequence's
    slots is the oracle's multi-token output."""
    from paged_kv_cache_25_amd import ops
    from tests.test_gpu_balanced import expected_plan
    inp = make_inputs(num_seqs=6, num_q_heads=8, num_kv_heads=2, head_dim=128,
                      ctx=("fixed", [3, 300, 40, 520, 1300, 17]), pool=("used_fraction", 0.8),
                      q_dtype=q, kv_dtype=kv, seed=96, new_tokens=("fixed", [5, 1, 19, 8, 4, 0]))
    inp.context_lens[0] = 3                  # ctx < t: two rows see nothing
    B, hq, D = inp.num_seqs, inp.num_q_heads, inp.head_dim
    mq = inp.max_new_tokens
    dev = DeviceMultiStep(inp)
    dev.append()
    R = ops.multi_query_plan_slots(B, mq, hq, inp.num_kv_heads, D, dev.q.dtype, dev.k_pool.dtype)
    log(f"[case] multi planned partials kv={kv} q={q} R={R}")
    plan = torch.empty(ops.load().pkv_decode_plan_bytes(B, R), dtype=torch.uint8, device="cuda")
    po = torch.full((R, mq, hq, D), float("nan"), device="cuda")
    pl = torch.full((R, mq, hq), float("nan"), device="cuda")
    ops.paged_multi_query_partials_planned(po, pl, plan, dev.q, dev.k_pool, dev.v_pool, dev.tables,
                                           dev.lens, dev.qsl, mq, inp.softmax_scale, dev.k_scales,
                                           dev.v_scales)
    torch.cuda.synchronize()
    first, info = expected_plan(inp.context_lens, R, inp.max_blocks_per_seq)
    assert np.array_equal(host_storage(plan)[:4 * (B + 1)].view(np.int32), first)
    got_l, got_o = pl.cpu().double().numpy(), po.cpu().double().numpy()
    kp, vp = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                                 inp.context_lens, inp.query_start_loc, inp.block_size)
    tol_l = 1e-5 if kv == "f32" else 2e-3
    tol_o = 1e-5 if kv == "f32" else (2e-2 if kv == "bf16" else 6e-2)
    merged = np.zeros((inp.total_queries, hq, D))
    for b in range(B):
        ctx = int(inp.context_lens[b])
        q0, q1 = int(inp.query_start_loc[b]), int(inp.query_start_loc[b + 1])
        slots = range(first[b], first[b + 1])
        K = pa.gather_sequence(kp, inp.block_tables[b], max(ctx, 1), 16, kv, inp.k_scales)
        V = pa.gather_sequence(vp, inp.block_tables[b], max(ctx, 1), 16, kv, inp.v_scales)
        for j in range(q1 - q0):
            n = pa.visible_tokens(ctx, q1 - q0, j)
            for s in slots:
                lo, hi = 16 * info[s, 1], min(16 * info[s, 2], max(n, 0))
                if hi <= lo:
                    assert np.all(np.isneginf(got_l[s, j])), (b, j, s)
                    continue
                o_ref, l_ref = pa.partition_partials(pa.to_float64(inp.q[q0 + j], q),
                                                     K[:, lo:hi], V[:, lo:hi], inp.softmax_scale,
                                                     hi - lo)
                assert np.abs(got_l[s, j] - l_ref[:, 0]).max() < tol_l, (b, j, s)
                assert np.abs(got_o[s, j] - o_ref[:, 0]).max() < tol_o, (b, j, s)
            merged[q0 + j] = pa.merge_partials(got_o[list(slots), j].transpose(1, 0, 2),
                                               got_l[list(slots), j].T)
    check_tolerance(kv, merged, oracle_multi(inp, (kp, vp)), f"multi planned partials {kv}",
                    out_dtype="f32")


@pytest.mark.parametrize("P", [0, BAL])
def test_unit_longer_than_the_table_window(P):
    """Sixteen new tokens per sequence over contexts of 9,000 and 8,300
    tokens (563 and 519 blocks): with one partition per sequence a unit walks
    more blocks than the 512 table entries the LDS-ring kernel holds at once,
    so it drains the ring and reloads the entries mid-sequence."""
    inp = named_config(2, seed=120, num_seqs=2, ctx=("fixed", [9000, 8300]),
                       new_tokens=("const", 16), name="long_unit_t16")
    _check(inp, f"long unit t=16 P={P}", partition_size=P)


@pytest.mark.parametrize("P", [0, 32, BAL])
def test_bad_table_entry_with_new_tokens(P):
    """A table entry outside [0, num_blocks) in a sequence with 16 new tokens
    (64 query columns per KV head: the LDS-ring kernel) is an empty block:
    the result is the oracle's attention with that block taken out of the
    table and its 16 tokens out of the context (every new row sees the whole
    block, so its removal shifts no visibility)."""
    inp = make_inputs(num_seqs=3, num_q_heads=16, num_kv_heads=4, head_dim=128,
                      ctx=("fixed", [200, 300, 150]), pool=("used_fraction", 0.8),
                      q_dtype="bf16", kv_dtype="bf16", seed=121, new_tokens=("const", 16),
                      name="bad_entry_t16")
    pools = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                                inp.context_lens, inp.query_start_loc, inp.block_size)
    good = inp.block_tables.copy()
    bad_seq, bad_blk = 1, 1
    inp.block_tables[bad_seq, bad_blk] = inp.num_blocks + 7
    log(f"[case] bad entry t=16 P={P}")
    dev = DeviceMultiStep(inp)
    dev.k_pool = dev_tensor(pools[0], inp.kv_dtype)       # appended already: attend only
    dev.v_pool = dev_tensor(pools[1], inp.kv_dtype)
    gpu = dev.attend(P)
    torch.cuda.synchronize()
    gpu = gpu.detach().float().cpu().double().numpy()
    tables = good.copy()
    row = [x for k, x in enumerate(tables[bad_seq]) if k != bad_blk] + [-1]
    tables[bad_seq] = np.asarray(row, dtype=tables.dtype)
    lens = inp.context_lens.copy()
    lens[bad_seq] -= 16
    ref = pa.multi_query_attention(inp.q, pools[0], pools[1], tables, lens, inp.query_start_loc,
                                   block_size=inp.block_size, softmax_scale=inp.softmax_scale,
                                   q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    check_tolerance("bf16", gpu, ref, f"bad entry t=16 P={P}")
