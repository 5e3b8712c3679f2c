"""Helpers for the GPU parity tests: move workload inputs to the device, run
the HIP path through the C ABI, and compare against the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.paged_attention as pa
from paged_kv_cache_25_amd import ops

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_tensor(arr: np.ndarray, dtype: str | None, device="cuda"):
    """Storage numpy array -> device tensor of the matching torch dtype."""
    if dtype is None:
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "fp8_e4m3":
        t = torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def host_storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy storage array (float32 / uint16 bits / uint8 codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


class DeviceStep:
    """One workload on the device, ready to run append + decode."""

    def __init__(self, inp, device="cuda"):
        self.inp = inp
        self.q = dev_tensor(inp.q, inp.q_dtype, device)
        self.k_pool = dev_tensor(inp.k_pool, inp.kv_dtype, device)
        self.v_pool = dev_tensor(inp.v_pool, inp.kv_dtype, device)
        self.k_new = dev_tensor(inp.k_new, inp.kv_dtype, device)
        self.v_new = dev_tensor(inp.v_new, inp.kv_dtype, device)
        self.tables = dev_tensor(inp.block_tables, None, device)
        self.lens = dev_tensor(inp.context_lens, None, device)
        self.k_scales = None if inp.k_scales is None else dev_tensor(inp.k_scales, None, device)
        self.v_scales = None if inp.v_scales is None else dev_tensor(inp.v_scales, None, device)
        self.out = torch.empty(inp.num_seqs, inp.num_q_heads, inp.head_dim,
                               dtype=TORCH_DT[inp.q_dtype], device=device)

    def append(self):
        ops.kv_append(self.k_pool, self.v_pool, self.k_new, self.v_new, self.tables, self.lens)

    def decode(self, partition_size=None, max_context_len=None):
        inp = self.inp
        P = inp.partition_size if partition_size is None else partition_size
        mcl = inp.max_context_len if max_context_len is None else max_context_len
        ops.paged_decode_attention(self.out, self.q, self.k_pool, self.v_pool, self.tables,
                                   self.lens, mcl, inp.softmax_scale, P, self.k_scales,
                                   self.v_scales)
        return self.out

    def step(self, partition_size=None, fused=False):
        """Append then attend: two ABI calls, or pkv_paged_decode_step when fused."""
        if fused:
            inp = self.inp
            P = inp.partition_size if partition_size is None else partition_size
            ops.decode_step(self.out, self.q, self.k_pool, self.v_pool, self.k_new, self.v_new,
                            self.tables, self.lens, inp.max_context_len, inp.softmax_scale, P,
                            self.k_scales, self.v_scales, fused=True)
            out = self.out
        else:
            self.append()
            out = self.decode(partition_size)
        torch.cuda.synchronize()
        return out

    def out_f64(self):
        return self.out.detach().float().cpu().double().numpy()


def oracle_out(inp, seqs=None, pools=None):
    """Oracle output (float64) after the append; ``pools`` = already-appended pools."""
    if pools is None:
        pools = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                             inp.context_lens, inp.block_size)
    return pa.decode_attention(inp.q, pools[0], pools[1], inp.block_tables, inp.context_lens,
                               block_size=inp.block_size, softmax_scale=inp.softmax_scale,
                               q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype,
                               k_scales=inp.k_scales, v_scales=inp.v_scales, seqs=seqs)


def uses_matrix_cores(inp):
    """bf16 queries over a bf16 cache with a shared KV head take the MFMA kernel."""
    return inp.q_dtype == "bf16" and inp.kv_dtype == "bf16" and inp.group_size >= 2


def abs_v_attention(inp, seqs=None, pools=None):
    """A = sum_t p_t |v_t| / sum_t p_t per output element (the oracle applied
    to |V|): bounds how far rounding each weight to bf16 can move the output."""
    if pools is None:
        pools = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.block_tables,
                             inp.context_lens, inp.block_size)
    vabs = pools[1] & np.uint16(0x7FFF) if inp.kv_dtype == "bf16" else np.abs(pools[1])
    return pa.decode_attention(inp.q, pools[0], vabs, inp.block_tables, inp.context_lens,
                               block_size=inp.block_size, softmax_scale=inp.softmax_scale,
                               q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype, seqs=seqs)


def check_guard(inp, gpu, ref, label, seqs=None, pools=None, absv=None):
    """A bound from the kernels' own arithmetic, much tighter than the bars:
    fp32 products, sums and softmax (relative error ~1e-6), the output rounded
    once to its dtype (2^-9 relative for bf16) and, on the matrix-core path,
    every weight rounded to bf16 (at most 2^-9 A).  Margins of 2x.  ``absv``:
    A already computed (abs_v_attention of the same sequences)."""
    out_r = 2.0 ** -8 if inp.q_dtype == "bf16" else 0.0
    bound = out_r * np.abs(ref) + 2e-5 * (1.0 + np.abs(ref))
    if uses_matrix_cores(inp):
        if absv is None:
            absv = abs_v_attention(inp, seqs, pools)
        bound = bound + 2.0 ** -8 * absv
    err = np.abs(gpu - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    assert (err <= bound).all(), f"{label}: error exceeds the arithmetic bound ({worst:.2f}x)"
    log(f"[guard] {label}: max err / bound = {worst:.3f}")
    return worst


class FullReference:
    """A full-size workload with its oracle results, built once per process and
    shared by every test that runs it (the fixed and balanced splits, the two
    calls and the fused step): the inputs, the pools after the append, the
    oracle output of every sequence and, for the matrix-core path, A of
    check_guard.  The oracle runs one sequence at a time, so host memory holds
    one sequence's gathered float64 cache at most, and each sequence logs."""

    _cache: dict = {}

    @classmethod
    def get(cls, key, make):
        if key not in cls._cache:
            cls._cache[key] = cls(key, make())
        return cls._cache[key]

    def __init__(self, key, inp):
        self.inp = inp
        self.pools = pa.kv_append(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                  inp.block_tables, inp.context_lens, inp.block_size)
        refs, absv = [], []
        for b in range(inp.num_seqs):
            refs.append(oracle_out(inp, seqs=[b], pools=self.pools)[0])
            if uses_matrix_cores(inp):
                absv.append(abs_v_attention(inp, [b], self.pools)[0])
            if b % 16 == 15 or b == inp.num_seqs - 1 or inp.num_seqs <= 16:
                log(f"[oracle] {key}: {b + 1}/{inp.num_seqs} sequences")
        self.ref = np.stack(refs)
        self.absv = np.stack(absv) if absv else None


def check_tolerance(kv_dtype, gpu, ref, label="", out_dtype="f32"):
    """The bars: f32 KV max-abs 1e-5; bf16 KV |d| <= max(2e-2 |ref|, 1e-2);
    e4m3 KV max-abs 6e-2 (against the oracle on the same dequantised values).
    An f32-KV result written as bf16 (bf16 queries) also carries the output's
    round-to-nearest error, at most 2^-9 |ref| (2^-8 |ref| allowed).
    Returns the max abs error; asserts on the bar and on finiteness."""
    assert np.isfinite(gpu).all(), f"{label}: non-finite output"
    err = np.abs(gpu - ref)
    mx = float(err.max()) if err.size else 0.0
    if kv_dtype == "f32":
        bound = 1e-5 + (2.0 ** -8 * np.abs(ref) if out_dtype == "bf16" else 0.0)
        assert (err <= bound).all(), f"{label}: max abs err {mx}"
    elif kv_dtype == "bf16":
        bound = np.maximum(2e-2 * np.abs(ref), 1e-2)
        assert (err <= bound).all(), f"{label}: max abs err {mx}"
    else:
        assert mx <= 6e-2, f"{label}: max abs err {mx}"
    log(f"[parity] {label}: max|gpu-oracle| = {mx:.3e}")
    return mx


class DeviceMultiStep:
    """A workload with several new tokens per sequence on the device: append
    them (pkv_kv_append_tokens), then attend (pkv_paged_multi_query_attention)."""

    def __init__(self, inp, device="cuda"):
        assert inp.query_start_loc is not None
        self.inp = inp
        self.q = dev_tensor(inp.q, inp.q_dtype, device)
        self.k_pool = dev_tensor(inp.k_pool, inp.kv_dtype, device)
        self.v_pool = dev_tensor(inp.v_pool, inp.kv_dtype, device)
        self.k_new = dev_tensor(inp.k_new, inp.kv_dtype, device)
        self.v_new = dev_tensor(inp.v_new, inp.kv_dtype, device)
        self.tables = dev_tensor(inp.block_tables, None, device)
        self.lens = dev_tensor(inp.context_lens, None, device)
        self.qsl = dev_tensor(inp.query_start_loc.astype(np.int32), None, device)
        self.k_scales = None if inp.k_scales is None else dev_tensor(inp.k_scales, None, device)
        self.v_scales = None if inp.v_scales is None else dev_tensor(inp.v_scales, None, device)
        self.out = torch.empty(inp.total_queries, inp.num_q_heads, inp.head_dim,
                               dtype=TORCH_DT[inp.q_dtype], device=device)

    def append(self):
        ops.kv_append_tokens(self.k_pool, self.v_pool, self.k_new, self.v_new, self.tables,
                             self.lens, self.qsl)

    def attend(self, partition_size=None, max_query_len=None):
        inp = self.inp
        P = inp.partition_size if partition_size is None else partition_size
        mq = max(inp.max_new_tokens, 1) if max_query_len is None else max_query_len
        ops.paged_multi_query_attention(self.out, self.q, self.k_pool, self.v_pool, self.tables,
                                        self.lens, self.qsl, mq, inp.max_context_len,
                                        inp.softmax_scale, P, self.k_scales, self.v_scales)
        return self.out

    def step(self, partition_size=None):
        self.append()
        out = self.attend(partition_size)
        torch.cuda.synchronize()
        return out

    def out_f64(self):
        return self.out.detach().float().cpu().double().numpy()


def oracle_multi(inp, pools=None):
    """Oracle output (float64, [total, Hq, D]) after appending the new tokens."""
    if pools is None:
        pools = pa.kv_append_tokens(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                    inp.block_tables, inp.context_lens, inp.query_start_loc,
                                    inp.block_size)
    return pa.multi_query_attention(inp.q, pools[0], pools[1], inp.block_tables,
                                    inp.context_lens, inp.query_start_loc,
                                    block_size=inp.block_size, softmax_scale=inp.softmax_scale,
                                    q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype,
                                    k_scales=inp.k_scales, v_scales=inp.v_scales)
