"""The balanced calls inside a captured HIP graph.

The balanced split schedules the batch on the device from context_lens, with
no host copy and no memset, so a decode step can be captured once and
replayed.  Each case runs the call eagerly, captures the same call, then
replays the graph several times with other eager work and synchronisations
between the replays, and requires every replay to give the eager result bit
for bit (the kernels are deterministic; a replay re-appends the same rows to
the same slots).  The eager result itself is checked against the oracle."""

import numpy as np
import pytest
import torch

import oracle.mla as mla
import oracle.paged_attention as pa
from paged_kv_cache_25_amd import ops
from tests.gpu_util import DeviceMultiStep, DeviceStep, check_tolerance, log, oracle_multi
from tests.test_gpu_mla import DevMLA, _appended_pool
from workloads import named_config
from workloads.mla import make_mla_inputs

pytestmark = pytest.mark.gpu
BAL = ops.PKV_PARTITION_BALANCED
REPLAYS = 4


def _replays_match(run, out, label):
    """Eager result of run(), then REPLAYS graph replays of it, each equal."""
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(REPLAYS):
        out.fill_(0)
        scratch.mul_(1.0001).add_(1.0)                # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"{label}: replay {r} differs from the eager call"
    log(f"[graph] {label}: {REPLAYS} replays equal the eager call")
    return eager


def test_balanced_decode_step_in_a_graph():
    inp = named_config(2, num_seqs=24)
    log(f"[case] graph: fused balanced step B={inp.num_seqs}")
    d = DeviceStep(inp)
    ws = ops.alloc_workspace(inp.num_seqs, inp.num_q_heads, inp.head_dim, inp.max_context_len,
                             BAL, "cuda")

    def run():
        ops.decode_step(d.out, d.q, d.k_pool, d.v_pool, d.k_new, d.v_new, d.tables, d.lens,
                        inp.max_context_len, inp.softmax_scale, BAL, workspace=ws, fused=True)

    eager = _replays_match(run, d.out, "fused balanced step")
    kp, vp = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                          inp.context_lens, inp.block_size)
    ref = pa.decode_attention(inp.q, kp, vp, inp.block_tables, inp.context_lens,
                              block_size=inp.block_size, softmax_scale=inp.softmax_scale,
                              q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    check_tolerance("bf16", eager.float().cpu().double().numpy(), ref, "graph step",
                    out_dtype="bf16")


def test_balanced_mla_in_a_graph():
    inp = make_mla_inputs(num_seqs=6, num_heads=128, ctx=("fixed", [1, 17, 64, 300, 700, 1500]),
                          seed=96)
    log("[case] graph: balanced MLA decode")
    dev = DevMLA(inp)
    ops.mla_append(dev.pool, dev.new, dev.tables, dev.lens)
    n = int(ops.load().pkv_mla_workspace_bytes(inp.num_seqs, inp.num_heads, 512,
                                               inp.max_context_len, BAL))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def run():
        ops.mla_decode_attention(dev.out, dev.q, dev.pool, dev.tables, dev.lens,
                                 inp.max_context_len, inp.softmax_scale, BAL, workspace=ws)

    eager = _replays_match(run, dev.out, "balanced MLA")
    pool = _appended_pool(inp)
    ref = mla.mla_decode_absorbed(inp.q, pool, inp.block_tables, inp.context_lens, block_size=16,
                                  softmax_scale=inp.softmax_scale, kv_lora_rank=inp.kv_lora_rank,
                                  dtype=inp.dtype)
    check_tolerance("bf16", eager.float().cpu().double().numpy(), ref, "graph MLA",
                    out_dtype="bf16")


def test_balanced_multi_token_in_a_graph():
    inp = named_config(2, seed=97, num_seqs=6, ctx=("uniform", 16, 1400),
                       new_tokens=("const", 4), name="graph_t4")
    log("[case] graph: balanced attention with 4 new tokens")
    dev = DeviceMultiStep(inp)
    dev.append()
    mq = inp.max_new_tokens
    n = int(ops.load().pkv_multi_query_balanced_workspace_bytes(
        inp.num_seqs, mq, inp.num_q_heads, inp.num_kv_heads, inp.head_dim,
        ops.dtype_code(dev.q.dtype), ops.dtype_code(dev.k_pool.dtype)))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def run():
        ops.paged_multi_query_attention(dev.out, dev.q, dev.k_pool, dev.v_pool, dev.tables,
                                        dev.lens, dev.qsl, mq, inp.max_context_len,
                                        inp.softmax_scale, BAL, workspace=ws)

    eager = _replays_match(run, dev.out, "balanced multi-token")
    pools = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                                inp.context_lens, inp.query_start_loc, inp.block_size)
    check_tolerance("bf16", eager.float().cpu().double().numpy(), oracle_multi(inp, pools),
                    "graph multi-token", out_dtype="bf16")
