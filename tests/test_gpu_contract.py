"""The device-side contract of include/pkv.h when it is violated: a table
entry outside [0, num_blocks) is treated as an empty block.  Its tokens get
no weight and nothing is read from or written to the pool for it; every other
token is attended as usual.

Decode attention has no positional term, so the expected output is the
oracle's attention over the same sequence with that block taken out of its
table (and its 16 tokens out of the context).  Every kernel family is run:
the matrix-core kernel (bf16 over bf16, grouped heads), the vector kernel
(float32, and e4m3 with scales, whose scale reads the bad entry must not
reach), and the absorbed MLA kernel."""

import numpy as np
import pytest

import oracle.mla as mla
import oracle.paged_attention as pa
from tests.gpu_util import DeviceStep, check_tolerance, host_storage, log
from tests.test_gpu_mla import DevMLA, _appended_pool
from workloads.configs import make_inputs
from workloads.mla import make_mla_inputs

pytestmark = pytest.mark.gpu

CTX = [40, 100, 70]            # sequence 1 loses block 1 (tokens 16..31)
BAD_SEQ, BAD_BLK = 1, 1


def _without_block(tables, lens, b, j, block_size=16):
    """The table row of sequence b with entry j removed, and its context 16 shorter."""
    t, n = tables.copy(), lens.copy()
    row = [x for k, x in enumerate(t[b]) if k != j] + [-1]
    t[b] = np.asarray(row, dtype=t.dtype)
    n[b] = n[b] - block_size
    return t, n


@pytest.mark.parametrize("q_dtype,kv_dtype,heads", [("bf16", "bf16", (16, 4)), ("f32", "f32", (4, 4)),
                                                     ("bf16", "fp8_e4m3", (4, 4))])
@pytest.mark.parametrize("P", [0, 32, 512, -1])
def test_decode_bad_table_entry_is_an_empty_block(q_dtype, kv_dtype, heads, P):
    hq, hkv = heads
    inp = make_inputs(num_seqs=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                      ctx=("fixed", CTX), pool=("used_fraction", 0.8), q_dtype=q_dtype,
                      kv_dtype=kv_dtype, seed=77)
    good_tables = inp.block_tables.copy()
    pools = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, good_tables,
                         inp.context_lens, inp.block_size)
    inp.block_tables[BAD_SEQ, BAD_BLK] = inp.num_blocks + 7
    label = f"bad entry {q_dtype}/{kv_dtype} Hq={hq} P={P}"
    log(f"[case] {label}")
    dev = DeviceStep(inp)
    gpu = dev.step(P)
    gpu = gpu.detach().float().cpu().double().numpy()
    # The pool holds exactly the appended rows (the bad entry wrote nothing).
    assert np.array_equal(host_storage(dev.k_pool).view(np.uint8), pools[0].view(np.uint8))
    assert np.array_equal(host_storage(dev.v_pool).view(np.uint8), pools[1].view(np.uint8))
    tables, lens = _without_block(good_tables, inp.context_lens, BAD_SEQ, BAD_BLK)
    ref = pa.decode_attention(inp.q, pools[0], pools[1], tables, lens, block_size=inp.block_size,
                              softmax_scale=inp.softmax_scale, q_dtype=q_dtype, kv_dtype=kv_dtype,
                              k_scales=inp.k_scales, v_scales=inp.v_scales)
    check_tolerance(kv_dtype, gpu, ref, label, out_dtype=q_dtype)


@pytest.mark.parametrize("P", [0, 32, 64, -1])
def test_mla_bad_table_entry_is_an_empty_block(P):
    inp = make_mla_inputs(num_seqs=3, num_heads=128, ctx=("fixed", CTX), seed=78,
                          pool_used_fraction=0.8)
    pool = _appended_pool(inp)
    good_tables = inp.block_tables.copy()
    inp.block_tables[BAD_SEQ, BAD_BLK] = inp.num_blocks + 3
    log(f"[case] mla bad entry P={P}")
    dev = DevMLA(inp)
    gpu = dev.step(P)
    assert np.array_equal(host_storage(dev.pool), pool)
    tables, lens = _without_block(good_tables, inp.context_lens, BAD_SEQ, BAD_BLK)
    ref = mla.mla_decode_absorbed(inp.q, pool, tables, lens, block_size=16,
                                  softmax_scale=inp.softmax_scale, kv_lora_rank=inp.kv_lora_rank,
                                  dtype=inp.dtype)
    check_tolerance("bf16", gpu, ref, f"mla bad entry P={P}", out_dtype="bf16")
