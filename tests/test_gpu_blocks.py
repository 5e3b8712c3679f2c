"""GPU parity of copy-on-write: pkv_copy_blocks against the oracle's
copy_blocks (bit for bit, every pool dtype, e4m3 scales, skipped bad pairs),
and parallel sampling end to end: a prompt prefilled once, forked into
samples through the library's allocator, each sample decoding several
tokens (copies, append, attention through the C ABI) against the oracle's
allocator, copies, append and attention."""

import numpy as np
import pytest
import torch

import oracle.block_manager as obm
import oracle.paged_attention as pa
from paged_kv_cache_25_amd import ops
from tests.gpu_util import check_tolerance, dev_tensor, host_storage, log
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("kv,head_dim,hkv", [("bf16", 128, 8), ("f32", 64, 4), ("fp8_e4m3", 128, 32)])
def test_copy_blocks_matches_oracle(kv, head_dim, hkv):
    inp = make_inputs(num_seqs=4, num_q_heads=hkv, num_kv_heads=hkv, head_dim=head_dim,
                      ctx=("uniform", 20, 300), pool=("blocks", 96), q_dtype="bf16",
                      kv_dtype=kv, seed=5)
    rng = np.random.default_rng(6)
    ids = rng.permutation(96)
    pairs = [(int(ids[i]), int(ids[40 + i])) for i in range(30)]     # 30 distinct dsts, no dst a src
    pairs_dev = pairs + [(97, 3), (3, -1)]                            # out of range: skipped
    log(f"[case] copy_blocks {kv} D={head_dim} Hkv={hkv}: {len(pairs)} pairs")
    kp = dev_tensor(inp.k_pool, kv)
    vp = dev_tensor(inp.v_pool, kv)
    ks = None if inp.k_scales is None else dev_tensor(inp.k_scales, None)
    vs = None if inp.v_scales is None else dev_tensor(inp.v_scales, None)
    pr = torch.tensor(pairs_dev, dtype=torch.int32, device="cuda")
    ops.copy_blocks(kp, vp, pr, ks, vs)
    torch.cuda.synchronize()
    pools = [inp.k_pool, inp.v_pool] + ([inp.k_scales, inp.v_scales] if ks is not None else [])
    ref = obm.copy_blocks(pools, pairs)
    assert _bits_equal(host_storage(kp), ref[0]) and _bits_equal(host_storage(vp), ref[1])
    if ks is not None:
        assert _bits_equal(ks.cpu().numpy(), ref[2]) and _bits_equal(vs.cpu().numpy(), ref[3])
    log(f"[parity] copy_blocks {kv}: bit-identical")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_parallel_sampling_end_to_end(kv):
    """4 samples of a 100-token prompt (Llama-3-8B heads, blocks of 16) decode
    5 tokens each.  Every step: the allocator's append_slots (copy-on-write on
    the shared last block), pkv_copy_blocks, pkv_kv_append, then
    pkv_paged_decode_attention for all samples at once."""
    hq, hkv, D, bs, NB = 32, 8, 128, 16, 64
    n_samples, prompt, steps = 4, 100, 5
    rng = np.random.default_rng(9)

    def rows(n):
        x = rng.standard_normal((n, hkv, D)).astype(np.float32)
        if kv == "bf16":
            return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return torch.from_numpy(x * 0.5).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    store = np.uint16 if kv == "bf16" else np.uint8
    k_pool = np.zeros((NB, hkv, bs, D), store)
    v_pool = np.zeros_like(k_pool)
    scales = None if kv == "bf16" else np.full((NB, hkv), 1.0 / 64, np.float32)
    kd, vd = dev_tensor(k_pool, kv), dev_tensor(v_pool, kv)
    ksd = None if scales is None else dev_tensor(scales, None)
    vsd = None if scales is None else dev_tensor(scales.copy(), None)
    ref_k, ref_v = k_pool.copy(), v_pool.copy()
    ref_ks = None if scales is None else scales.copy()
    ref_vs = None if scales is None else scales.copy()

    lib_m, ref_m = ops.BlockManager(NB, bs), obm.BlockManager(NB, bs)
    # prefill the prompt into sample 0: K/V rows written through its table
    lib_m.add(0); ref_m.add(0)
    assert lib_m.append_slots(0, prompt) == ref_m.append_slots(0, prompt) == []
    pk, pv = rows(prompt), rows(prompt)
    t, lens = lib_m.block_tables([0], 8)
    qsl = torch.tensor([0, prompt], dtype=torch.int32, device="cuda")
    ops.kv_append_tokens(kd, vd, dev_tensor(pk, kv), dev_tensor(pv, kv), dev_tensor(t, None),
                         dev_tensor(lens, None), qsl)
    ref_k, ref_v = pa.kv_append_tokens(ref_k, ref_v, pk, pv, t, lens, np.array([0, prompt]), bs)
    for s in range(1, n_samples):
        lib_m.fork(0, s); ref_m.fork(0, s)
    seqs = list(range(n_samples))
    for step in range(steps):
        copies = []
        for s in seqs:
            got = lib_m.append_slots(s, 1)
            want = ref_m.append_slots(s, 1)
            assert got == want, (step, s)
            copies += got
        if copies:
            ops.copy_blocks(kd, vd, torch.tensor(copies, dtype=torch.int32, device="cuda"), ksd, vsd)
            pools = [ref_k, ref_v] + ([ref_ks, ref_vs] if ksd is not None else [])
            out = obm.copy_blocks(pools, copies)
            ref_k, ref_v = out[0], out[1]
            if ksd is not None:
                ref_ks, ref_vs = out[2], out[3]
        tables, lens = lib_m.block_tables(seqs, 8)
        rt, rl = ref_m.block_tables(seqs, 8)
        assert np.array_equal(tables, rt) and np.array_equal(lens, rl)
        nk, nv = rows(n_samples), rows(n_samples)
        td, ld = dev_tensor(tables, None), dev_tensor(lens, None)
        ops.kv_append(kd, vd, dev_tensor(nk, kv), dev_tensor(nv, kv), td, ld)
        ref_k, ref_v = pa.kv_append(ref_k, ref_v, nk, nv, tables, lens, bs)
        q = torch.from_numpy(rng.standard_normal((n_samples, hq, D)).astype(np.float32)).to(
            torch.bfloat16).cuda()
        outd = torch.empty_like(q)
        ops.paged_decode_attention(outd, q, kd, vd, td, ld, int(lens.max()), D ** -0.5, 64,
                                   ksd, vsd)
        torch.cuda.synchronize()
        qb = q.cpu().view(torch.int16).numpy().view(np.uint16)
        ref = pa.decode_attention(qb, ref_k, ref_v, tables, lens, block_size=bs,
                                  softmax_scale=D ** -0.5, q_dtype="bf16", kv_dtype=kv,
                                  k_scales=ref_ks, v_scales=ref_vs)
        check_tolerance(kv, outd.float().cpu().double().numpy(), ref,
                        f"sampling {kv} step {step} ({len(copies)} copies)", out_dtype="bf16")
    assert _bits_equal(host_storage(kd), ref_k) and _bits_equal(host_storage(vd), ref_v)
    # exercise 3's shape: 7 prompt blocks shared, then one private last block per writer
    # but the last sharer, which writes in place
    assert NB - lib_m.num_free() == 7 + (n_samples - 1)
