"""GPU parity of the balanced split of the one-token decode
(partition_size = PKV_PARTITION_BALANCED), through the C ABI.

The split only regroups the partial sums: each sequence's blocks are cut into
n_b >= 1 runs of nearly equal length, each run is attended on its own and the
runs are merged by their log-sum-exps, which combine any split of the tokens.
So the attention output is checked against the oracle at the usual bars, and
each run's partial result against the oracle restricted to that run's tokens.

The schedule itself is integer work, checked bit for bit against its
definition written out below: u_b = ceil(min(max(ctx_b, 0), cap) / 16)
blocks, n_b = max(1, ceil(u_b / t)) with t the smallest positive integer for
which sum_b n_b <= R = max(num_slots, num_seqs), chunk k of n_b covering
blocks [k u_b // n_b, (k+1) u_b // n_b).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.paged_attention as pa  # noqa: E402
from paged_kv_cache_25_amd import ops  # noqa: E402
from tests.gpu_util import (DeviceStep, FullReference, check_guard,  # noqa: E402
                            check_tolerance, host_storage, log, oracle_out)
from workloads import make_inputs, named_config  # noqa: E402

pytestmark = pytest.mark.gpu
BAL = ops.PKV_PARTITION_BALANCED
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()


def expected_plan(lens, num_slots, max_blocks, block_size=16):
    """(chunk_first [B + 1], slot_info [num_slots, 4]) from the definition."""
    B = len(lens)
    cap = max_blocks * block_size
    u = [-(-min(max(int(c), 0), cap) // block_size) for c in lens]
    R = max(num_slots, B)

    def count(t):
        return sum(max(1, -(-x // t)) for x in u)

    lo, hi = 1, max(max(u, default=1), 1)          # count(hi) = B <= R
    while lo < hi:
        mid = (lo + hi) // 2
        if count(mid) <= R:
            hi = mid
        else:
            lo = mid + 1
    n = [max(1, -(-x // lo)) for x in u]
    first = np.zeros(B + 1, np.int32)
    first[1:] = np.cumsum(n)
    info = np.tile(np.array([-1, 0, 0, 0], np.int32), (num_slots, 1))
    for b in range(B):
        for k in range(n[b]):
            info[first[b] + k] = (b, k * u[b] // n[b], (k + 1) * u[b] // n[b], n[b])
    return first, info


def device_plan(lens, num_slots, max_blocks):
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    plan = ops.decode_plan(lens_d, num_slots, max_blocks)
    torch.cuda.synchronize()
    raw = host_storage(plan).view(np.uint8)
    B = len(lens)
    first = raw[:4 * (B + 1)].view(np.int32)
    off = ops.plan_info_offset(B)
    info = raw[off:off + 16 * num_slots].view(np.int32).reshape(num_slots, 4)
    return first, info, plan


# --- the schedule --------------------------------------------------------------

def plan_case(case):
    """(context lengths, slots, max_blocks_per_seq) of a schedule test."""
    if case.startswith("config"):
        inp = named_config(int(case[6]))
        return inp.context_lens, 384, inp.max_blocks_per_seq
    return {
        "long_and_short": (np.array([3000, 5, 17, 64, 1, 33, 100, 0, 48]), 384, 200),
        "many_short": (np.random.default_rng(61).integers(0, 41, 600), 600, 3),
        "all_empty": (np.zeros(4, np.int64), 384, 4),
        "one_long": (np.array([6000]), 384, 375),
        "clamped": (np.array([-5, 10 ** 6, 129, 128]), 384, 8),   # past the table / negative
        "few_slots": (np.array([100, 200, 300]), 7, 19),
        "as_many_slots_as_seqs": (np.array([5000, 16, 17, 0]), 4, 313),
    }[case]


@pytest.mark.parametrize("case", ["long_and_short", "many_short", "all_empty", "one_long",
                                  "clamped", "few_slots", "as_many_slots_as_seqs",
                                  "config2_lens", "config4_lens"])
def test_plan_matches_definition(case):
    lens, slots, mb = plan_case(case)
    log(f"[case] plan {case}: B={len(lens)} slots={slots} max_blocks={mb}")
    first, info, _ = device_plan(lens, slots, mb)
    want_first, want_info = expected_plan(lens, slots, mb)
    assert np.array_equal(first, want_first)
    assert np.array_equal(info, want_info)


def test_plan_slots_of_the_workloads():
    """R for the five workloads' shapes: one wave of resident decode
    workgroups (S), or max(2S, 2B) when 2B > S."""
    assert ops.decode_plan_slots(64, 32, 8, 128, torch.bfloat16, torch.bfloat16) == 384
    assert ops.decode_plan_slots(256, 32, 8, 128, torch.bfloat16, torch.bfloat16) == 768
    assert ops.decode_plan_slots(128, 32, 32, 128, torch.bfloat16, torch.float8_e4m3fn) == 256
    assert ops.decode_plan_slots(4, 4, 4, 64, torch.float32, torch.float32) == 768


# --- attention and the fused step -------------------------------------------------

def run_balanced(inp, label, seqs=None, fused=False, full=None):
    """``full``: a FullReference of ``inp`` (its oracle results, shared with the
    other tests of the same workload)."""
    label = f"{label} balanced" + (" [fused step]" if fused else "")
    log(f"[case] {label}: B={inp.num_seqs} Hq={inp.num_q_heads} Hkv={inp.num_kv_heads} "
        f"D={inp.head_dim} kv={inp.kv_dtype} q={inp.q_dtype} max_ctx={inp.max_context_len}")
    d = DeviceStep(inp)
    d.step(BAL, fused=fused)
    if full is not None:
        kp, vp = full.pools
    else:
        kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                              inp.context_lens, inp.block_size)
    assert np.array_equal(host_storage(d.k_pool).view(np.uint8), kp.view(np.uint8)), "K pool"
    assert np.array_equal(host_storage(d.v_pool).view(np.uint8), vp.view(np.uint8)), "V pool"
    if full is not None:
        ref, absv = full.ref, full.absv
    else:
        ref, absv = oracle_out(inp, seqs=seqs, pools=(kp, vp)), None
    gpu = d.out_f64() if seqs is None else d.out_f64()[list(seqs)]
    check_tolerance(inp.kv_dtype, gpu, ref, label, out_dtype=inp.q_dtype)
    check_guard(inp, gpu, ref, label, seqs=seqs, pools=(kp, vp), absv=absv)
    return d


FUSED = pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused_step"])


@FUSED
def test_config1_tiny_fp32(fused):
    run_balanced(named_config(1), "config1 tiny fp32", fused=fused)


@FUSED
def test_config2_llama3_8b_b64(fused):
    run_balanced(named_config(2), "config2 llama3-8b b64", fused=fused)


@FUSED
def test_config3_long_context_full(fused):
    full = FullReference.get("config3", lambda: named_config(3))
    run_balanced(full.inp, "config3 131072 ctx", full=full, fused=fused)


@FUSED
def test_config4_continuous_batching(fused):
    run_balanced(named_config(4), "config4 lognormal mix b256", fused=fused)


@FUSED
def test_config5_fp8_full(fused):
    full = FullReference.get("config5", lambda: named_config(5))
    run_balanced(full.inp, "config5 fp8 b128", full=full, fused=fused)


EDGE_CTX = [0, 1, 15, 16, 17, 300, 2500, 33]


@FUSED
@pytest.mark.parametrize("q,kv", [("f32", "f32"), ("f32", "bf16"), ("f32", "fp8_e4m3"),
                                  ("bf16", "f32"), ("bf16", "bf16"), ("bf16", "fp8_e4m3")])
@pytest.mark.parametrize("d", [64, 128])
def test_dtypes_and_edge_lengths(q, kv, d, fused):
    """Every kernel family, with empty, one-token, one-block, block-edge and
    long contexts in one batch (the long one is cut into many chunks)."""
    inp = make_inputs(num_seqs=len(EDGE_CTX), num_q_heads=8, num_kv_heads=2, head_dim=d,
                      ctx=("fixed", EDGE_CTX), pool=("used_fraction", 0.85), q_dtype=q,
                      kv_dtype=kv, seed=91)
    dev = run_balanced(inp, f"edges q={q} kv={kv} d={d}", fused=fused)
    assert np.all(dev.out_f64()[0] == 0)                    # ctx 0: zeros


@pytest.mark.parametrize("hq,hkv,d", [(48, 2, 128), (32, 1, 64), (6, 2, 128), (16, 16, 64)])
def test_group_shapes(hq, hkv, d):
    """Several column tiles per KV head (48 and 32 heads per group on the
    matrix cores), a vector tile of 3, and no grouping."""
    inp = make_inputs(num_seqs=5, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      ctx=("fixed", [4000, 7, 160, 0, 1234]), pool=("used_fraction", 0.9),
                      q_dtype="bf16", kv_dtype="bf16", seed=92)
    run_balanced(inp, f"groups Hq={hq} Hkv={hkv} d={d}")


@FUSED
def test_more_sequences_than_planned_in_kernel(fused):
    """Batches of more than 256 sequences are scheduled by the one-wave plan
    kernel before the decode kernel (smaller ones plan inside it): 300
    sequences, mostly short, three long."""
    lens = np.random.default_rng(94).integers(0, 200, 300)
    lens[[7, 150, 299]] = [3000, 2200, 1700]
    inp = make_inputs(num_seqs=300, num_q_heads=8, num_kv_heads=2, head_dim=64,
                      ctx=("fixed", lens.tolist()), pool=("used_fraction", 0.9), q_dtype="bf16",
                      kv_dtype="bf16", seed=94)
    run_balanced(inp, "300 sequences", fused=fused)


def test_planned_partials_with_many_slots():
    """50,000 slots (more than the decode kernel plans for itself, whose chunk
    bounds stay in 32 bits below 46,341 slots): the planned pieces take the
    plan kernel, and merging them still gives the oracle's attention."""
    lens = [0, 5, 900, 3100]
    inp = make_inputs(num_seqs=4, num_q_heads=2, num_kv_heads=1, head_dim=64,
                      ctx=("fixed", lens), pool=("used_fraction", 0.9), q_dtype="bf16",
                      kv_dtype="bf16", seed=95)
    d = DeviceStep(inp)
    d.append()
    slots = 50000
    log(f"[case] planned partials, {slots} slots")
    lens_d = torch.from_numpy(inp.context_lens.astype(np.int32)).cuda()
    plan = torch.empty(ops.load().pkv_decode_plan_bytes(4, slots), dtype=torch.uint8, device="cuda")
    po = torch.empty((slots, 2, 64), device="cuda")
    pl = torch.empty((slots, 2), device="cuda")
    ops.paged_decode_partials_planned(po, pl, plan, d.q, d.k_pool, d.v_pool, d.tables, lens_d,
                                      inp.softmax_scale)
    torch.cuda.synchronize()
    first, info = expected_plan(inp.context_lens, slots, inp.max_blocks_per_seq)
    raw = host_storage(plan).view(np.uint8)
    assert np.array_equal(raw[:20].view(np.int32), first)
    off = ops.plan_info_offset(4)
    assert np.array_equal(raw[off:off + 16 * slots].view(np.int32).reshape(slots, 4), info)
    merged = torch.empty_like(d.q)
    ops.merge_partials_planned(merged, po, pl, plan)
    torch.cuda.synchronize()
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, inp.block_size)
    check_tolerance("bf16", merged.float().cpu().double().numpy(), oracle_out(inp, pools=(kp, vp)),
                    "planned, 50000 slots", out_dtype="bf16")


@pytest.mark.parametrize("B,kind,slot_mult,q,kv", [
    (1, "uniform", 1, "bf16", "bf16"), (7, "mixed", 3, "f32", "f32"),
    (64, "lognormal", 1, "bf16", "bf16"), (100, "short", 2, "bf16", "bf16"),
    (255, "uniform", 1, "f32", "bf16"), (256, "lognormal", 4, "bf16", "bf16")])
def test_in_kernel_plan_random_batches(B, kind, slot_mult, q, kv):
    """The schedule each decode workgroup derives for itself (up to 256
    sequences), on random batches and slot counts: the chunk starts it
    publishes equal the definition bit for bit, and merging its chunks gives
    the oracle's attention (a wrong chunk range would drop or repeat tokens)."""
    rng = np.random.default_rng(1000 + B)
    lens = {"uniform": lambda: rng.integers(1, 3000, B),
            "mixed": lambda: np.where(rng.random(B) < 0.5, rng.integers(0, 20, B),
                                      rng.integers(500, 4000, B)),
            "lognormal": lambda: np.clip(np.exp(rng.normal(np.log(400), 1.2, B)), 0, 6000),
            "short": lambda: rng.integers(0, 40, B)}[kind]().astype(np.int64)
    inp = make_inputs(num_seqs=B, num_q_heads=2, num_kv_heads=1, head_dim=64,
                      ctx=("fixed", lens.tolist()), pool=("used_fraction", 0.95), q_dtype=q,
                      kv_dtype=kv, seed=2000 + B)
    slots = max(1, slot_mult * ops.decode_plan_slots(B, 2, 1, 64, TORCH_DT[q], TORCH_DT[kv]) // 2)
    slots = max(slots, B)
    log(f"[case] in-kernel plan: B={B} {kind} slots={slots} {q}/{kv}")
    d = DeviceStep(inp)
    d.append()
    plan = torch.full((ops.load().pkv_decode_plan_bytes(B, slots),), 0xFF, dtype=torch.uint8,
                      device="cuda")
    po = torch.empty((slots, 2, 64), device="cuda")
    pl = torch.empty((slots, 2), device="cuda")
    ops.paged_decode_partials_planned(po, pl, plan, d.q, d.k_pool, d.v_pool, d.tables, d.lens,
                                      inp.softmax_scale)
    merged = torch.empty_like(d.q)
    ops.merge_partials_planned(merged, po, pl, plan)
    torch.cuda.synchronize()
    first, _ = expected_plan(inp.context_lens, slots, inp.max_blocks_per_seq)
    got_first = host_storage(plan)[:4 * (B + 1)].view(np.int32)
    assert np.array_equal(got_first, first)
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, inp.block_size)
    check_tolerance(kv, merged.float().cpu().double().numpy(), oracle_out(inp, pools=(kp, vp)),
                    f"in-kernel plan B={B}", out_dtype=q)


def test_huge_table_takes_the_integer_division():
    """A table row of 2^22 + 5 entries whose context fills it (67M tokens)
    makes the in-kernel planner divide in integers (its float-reciprocal
    quotient is exact only below 2^22 blocks) and sum block counts past 16
    bits.  Only the first three entries are valid; the rest are outside the
    pool, i.e. empty blocks, so the result is attention over 48 tokens."""
    inp = make_inputs(num_seqs=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
                      ctx=("fixed", [48]), pool=("used_fraction", 1.0), q_dtype="bf16",
                      kv_dtype="bf16", seed=98)
    d = DeviceStep(inp)
    d.append()                                              # position 47 gets its row
    mb = (1 << 22) + 5
    table = np.full((1, mb), -1, np.int32)
    table[0, :3] = inp.block_tables[0, :3]
    d.tables = torch.from_numpy(table).cuda()
    d.lens = torch.tensor([mb * 16], dtype=torch.int32, device="cuda")
    log(f"[case] huge table: {mb} entries, ctx {mb * 16}")
    ws = ops.alloc_workspace(1, 2, 64, mb * 16, BAL, "cuda")
    ops.paged_decode_attention(d.out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, mb * 16,
                               inp.softmax_scale, BAL, workspace=ws)
    torch.cuda.synchronize()
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, inp.block_size)
    check_tolerance("bf16", d.out_f64(), oracle_out(inp, pools=(kp, vp)), "huge table",
                    out_dtype="bf16")


def test_deterministic_and_equal_to_split_math():
    """Two calls give the same bits; the result agrees with the fixed
    512-token split within float rounding (only the grouping differs)."""
    inp = named_config(2, num_seqs=16)
    log("[case] balanced determinism")
    d = DeviceStep(inp)
    d.append()
    a = d.decode(BAL).clone()
    b = d.decode(BAL).clone()
    c = d.decode(512).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    diff = (a.float() - c.float()).abs().max().item()
    assert diff <= 2.0 ** -7 * max(1.0, c.float().abs().max().item()), diff


# --- the planned pieces -------------------------------------------------------------

@pytest.mark.parametrize("kv,q", [("bf16", "bf16"), ("f32", "f32"), ("fp8_e4m3", "bf16")])
def test_planned_partials_and_merge(kv, q):
    """pkv_paged_decode_partials_planned: it writes the schedule's chunk
    starts (planned inside the decode kernel at this batch size) equal to
    pkv_decode_plan's; each chunk's normalised output and natural-log lse
    against the oracle over the chunk's tokens as pkv_decode_plan's slot
    records give them; an empty sequence's chunk has lse = -inf; unused slots
    are not written; merging with pkv_merge_partials_planned gives the
    attention output."""
    lens = [1, 700, 63, 1500, 0, 2900]
    inp = make_inputs(num_seqs=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                      ctx=("fixed", lens), pool=("used_fraction", 0.8), q_dtype=q, kv_dtype=kv,
                      seed=93)
    d = DeviceStep(inp)
    d.append()
    slots = ops.decode_plan_slots(len(lens), 8, 2, 128, TORCH_DT[q], TORCH_DT[kv])
    log(f"[case] planned partials kv={kv} q={q} slots={slots}")
    first, info, plan = device_plan(inp.context_lens, slots, inp.max_blocks_per_seq)
    po = torch.full((slots, 8, 128), float("nan"), device="cuda")
    pl = torch.full((slots, 8), float("nan"), device="cuda")
    plan[:4 * (len(lens) + 1)] = 0xFF                     # chunk_first is rewritten by the call
    ops.paged_decode_partials_planned(po, pl, plan, d.q, d.k_pool, d.v_pool, d.tables, d.lens,
                                      inp.softmax_scale, d.k_scales, d.v_scales)
    torch.cuda.synchronize()
    assert np.array_equal(host_storage(plan)[:4 * (len(lens) + 1)].view(np.int32), first)
    got_o = po.cpu().double().numpy()
    got_l = pl.cpu().double().numpy()
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, inp.block_size)
    used = int(first[-1])
    assert np.isnan(got_l[used:]).all() and np.isnan(got_o[used:]).all()
    tol_l = 1e-5 if kv == "f32" else 2e-3
    tol_o = 1e-5 if kv == "f32" else (2e-2 if kv == "bf16" else 6e-2)
    for s in range(used):
        b, k0, k1, _ = (int(x) for x in info[s])
        ctx = int(inp.context_lens[b])
        if ctx <= 0:
            assert np.isneginf(got_l[s]).all()
            continue
        K = pa.gather_sequence(kp, inp.block_tables[b], ctx, 16, kv, inp.k_scales)
        V = pa.gather_sequence(vp, inp.block_tables[b], ctx, 16, kv, inp.v_scales)
        lo, hi = 16 * k0, min(16 * k1, ctx)
        o_ref, l_ref = pa.partition_partials(pa.to_float64(inp.q[b], q), K[:, lo:hi],
                                             V[:, lo:hi], inp.softmax_scale, hi - lo)
        assert np.abs(got_l[s] - l_ref[:, 0]).max() < tol_l, s
        assert np.abs(got_o[s] - o_ref[:, 0]).max() < tol_o, s
    merged = torch.empty_like(d.q)
    ops.merge_partials_planned(merged, po, pl, plan)
    whole = d.decode(BAL)
    torch.cuda.synchronize()
    ref = oracle_out(inp, pools=(kp, vp))
    check_tolerance(kv, merged.float().cpu().double().numpy(), ref, f"planned merge {kv}",
                    out_dtype=q)
    # Sequences of two or more chunks go through the same kernels either way.
    multi = [b for b in range(len(lens)) if first[b + 1] - first[b] >= 2]
    assert multi and torch.equal(merged[multi], whole[multi])


def test_workspace_reuse_across_sizes():
    """One workspace, sized for the largest call, serves calls of different
    sizes and kinds in turn (balanced calls on 12 sequences of the
    Llama-3-8B layer and on 9 sequences with 8 q / 2 kv heads, a
    fixed-partition call between them, each leaving its partial rows and plan
    behind for the next): every result matches the oracle."""
    a = named_config(2, num_seqs=12)
    b = make_inputs(num_seqs=9, num_q_heads=8, num_kv_heads=2, head_dim=128,
                    ctx=("fixed", [1, 40, 700, 1500, 17, 3000, 260, 33, 900]),
                    pool=("used_fraction", 0.9), q_dtype="bf16", kv_dtype="bf16", seed=97)
    n = max(ops.workspace_bytes(a.num_seqs, a.num_q_heads, a.head_dim, a.max_context_len, BAL),
            ops.workspace_bytes(a.num_seqs, a.num_q_heads, a.head_dim, a.max_context_len, 512),
            ops.workspace_bytes(b.num_seqs, b.num_q_heads, b.head_dim, b.max_context_len, BAL))
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    refs = {}
    devs = {}
    for name, inp in (("a", a), ("b", b)):
        d = DeviceStep(inp)
        d.append()
        devs[name] = d
        refs[name] = oracle_out(inp)
    for name, P in (("a", BAL), ("b", BAL), ("a", 512), ("a", BAL), ("b", BAL)):
        d, inp = devs[name], devs[name].inp
        log(f"[case] workspace reuse: {name} P={P}")
        d.out.fill_(float("nan"))
        ops.paged_decode_attention(d.out, d.q, d.k_pool, d.v_pool, d.tables, d.lens,
                                   inp.max_context_len, inp.softmax_scale, P, workspace=ws)
        torch.cuda.synchronize()
        check_tolerance("bf16", d.out_f64(), refs[name], f"reuse {name} P={P}", out_dtype="bf16")
