"""ctypes binding of libpkv (include/pkv.h) over torch tensors.

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI.  torch provides the device memory and the current
HIP stream.  If ``libpkv.so`` has not been built, every call raises; there is
no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB names another build of the library to load instead (libpkv_vector.so:
# every decode on the vector kernel, the baseline of the matrix-core kernel).
LIB_PATH = os.environ.get("PKV_LIB") or os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
PKV_SCALE_FIXED, PKV_SCALE_RUNNING_AMAX = 0, 1
PKV_PARTITION_BALANCED = -1        # decode / MLA decode: balanced split of the batch's work
STATUS = {0: "PKV_OK", 1: "PKV_ERR_INVALID_ARG", 2: "PKV_ERR_UNSUPPORTED",
          3: "PKV_ERR_WORKSPACE", 4: "PKV_ERR_HIP", 5: "PKV_ERR_OUT_OF_BLOCKS"}
PKV_ERR_OUT_OF_BLOCKS = 5
BLOCK_SIZE = 16

_lib = None


class PkvError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


def load():
    """Load libpkv.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_25_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    L.pkv_abi_version.restype = ctypes.c_int
    L.pkv_abi_version.argtypes = []
    L.pkv_status_string.restype = ctypes.c_char_p
    L.pkv_status_string.argtypes = [ctypes.c_int]
    L.pkv_kv_append.restype = ctypes.c_int
    L.pkv_kv_append.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, ctypes.c_int, P]
    L.pkv_decode_workspace_bytes.restype = Z
    L.pkv_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    L.pkv_paged_decode_attention.restype = ctypes.c_int
    L.pkv_paged_decode_attention.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I,
                                             P, Z, ctypes.c_int, ctypes.c_int, P]
    L.pkv_paged_decode_step.restype = ctypes.c_int
    L.pkv_paged_decode_step.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I,
                                        P, Z, ctypes.c_int, ctypes.c_int, P]
    L.pkv_paged_decode_step_noalloc.restype = ctypes.c_int
    L.pkv_paged_decode_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                                I, F, I, ctypes.c_int, ctypes.c_int, P]
    L.pkv_paged_decode_partials.restype = ctypes.c_int
    L.pkv_paged_decode_partials.argtypes = [P, P, I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I,
                                            ctypes.c_int, ctypes.c_int, P]
    L.pkv_merge_partials.restype = ctypes.c_int
    L.pkv_merge_partials.argtypes = [P, P, P, P, I, I, I, I, ctypes.c_int, P]
    L.pkv_decode_plan_slots.restype = I
    L.pkv_decode_plan_slots.argtypes = [I, I, I, I, ctypes.c_int, ctypes.c_int]
    L.pkv_decode_plan_bytes.restype = Z
    L.pkv_decode_plan_bytes.argtypes = [I, I]
    L.pkv_decode_plan.restype = ctypes.c_int
    L.pkv_decode_plan.argtypes = [P, Z, P, I, I, I, I, P]
    L.pkv_paged_decode_partials_planned.restype = ctypes.c_int
    L.pkv_paged_decode_partials_planned.argtypes = [P, P, P, Z, I, P, P, P, P, P, P, P, I, I, I,
                                                    I, I, I, I, F, ctypes.c_int, ctypes.c_int, P]
    L.pkv_merge_partials_planned.restype = ctypes.c_int
    L.pkv_merge_partials_planned.argtypes = [P, P, P, P, I, I, I, I, ctypes.c_int, P]
    L.pkv_kv_append_tokens.restype = ctypes.c_int
    L.pkv_kv_append_tokens.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, ctypes.c_int, P]
    L.pkv_multi_query_workspace_bytes.restype = Z
    L.pkv_multi_query_workspace_bytes.argtypes = [I, I, I, I, I]
    L.pkv_multi_query_balanced_workspace_bytes.restype = Z
    L.pkv_multi_query_balanced_workspace_bytes.argtypes = [I, I, I, I, I, ctypes.c_int,
                                                           ctypes.c_int]
    L.pkv_paged_multi_query_attention.restype = ctypes.c_int
    L.pkv_paged_multi_query_attention.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                                  I, I, I, F, I, P, Z, ctypes.c_int,
                                                  ctypes.c_int, P]
    L.pkv_multi_query_plan_slots.restype = I
    L.pkv_multi_query_plan_slots.argtypes = [I, I, I, I, I, ctypes.c_int, ctypes.c_int]
    L.pkv_paged_multi_query_partials_planned.restype = ctypes.c_int
    L.pkv_paged_multi_query_partials_planned.argtypes = [P, P, P, Z, I, P, P, P, P, P, P, P, P, I,
                                                         I, I, I, I, I, I, I, I, F, ctypes.c_int,
                                                         ctypes.c_int, P]
    L.pkv_paged_multi_query_partials.restype = ctypes.c_int
    L.pkv_paged_multi_query_partials.argtypes = [P, P, I, P, P, P, P, P, P, P, P, I, I, I, I, I,
                                                 I, I, I, I, F, I, ctypes.c_int, ctypes.c_int, P]
    L.pkv_kv_append_quant.restype = ctypes.c_int
    L.pkv_kv_append_quant.argtypes = [P, P, P, P, P, P, ctypes.c_int, P, P, P, I, I, I, I, I, I, I,
                                      ctypes.c_int, P]
    I64 = ctypes.c_int64
    L.pkv_bm_create.restype = P
    L.pkv_bm_create.argtypes = [I, I]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_destroy.argtypes = [P]
    L.pkv_bm_add_seq.restype = ctypes.c_int
    L.pkv_bm_add_seq.argtypes = [P, I64]
    L.pkv_bm_fork.restype = ctypes.c_int
    L.pkv_bm_fork.argtypes = [P, I64, I64]
    L.pkv_bm_free_seq.restype = ctypes.c_int
    L.pkv_bm_free_seq.argtypes = [P, I64]
    L.pkv_bm_append_slots.restype = ctypes.c_int
    L.pkv_bm_append_slots.argtypes = [P, I64, I, P, P, I, P]
    L.pkv_bm_num_free.restype = I
    L.pkv_bm_num_free.argtypes = [P]
    L.pkv_bm_refcount.restype = I
    L.pkv_bm_refcount.argtypes = [P, I]
    L.pkv_bm_seq_len.restype = I64
    L.pkv_bm_seq_len.argtypes = [P, I64]
    L.pkv_bm_free_list.restype = I
    L.pkv_bm_free_list.argtypes = [P, P, I]
    L.pkv_bm_block_tables.restype = ctypes.c_int
    L.pkv_bm_block_tables.argtypes = [P, P, I, P, I, P]
    L.pkv_copy_blocks.restype = ctypes.c_int
    L.pkv_copy_blocks.argtypes = [P, P, P, P, P, I, I, I, I, I, ctypes.c_int, P]
    L.pkv_stream_read.restype = ctypes.c_int
    L.pkv_stream_read.argtypes = [P, P, Z, I, P]
    L.pkv_gather_read.restype = ctypes.c_int
    L.pkv_gather_read.argtypes = [P, P, Z, P, I, I, P]
    L.pkv_stream_read_out_words.restype = I
    L.pkv_stream_read_out_words.argtypes = [I]
    L.pkv_mla_append.restype = ctypes.c_int
    L.pkv_mla_append.argtypes = [P, P, P, P, I, I, I, I, I, P]
    L.pkv_mla_workspace_bytes.restype = Z
    L.pkv_mla_workspace_bytes.argtypes = [I, I, I, I, I]
    L.pkv_mla_decode_attention.restype = ctypes.c_int
    L.pkv_mla_decode_attention.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, Z, P]
    L.pkv_mla_decode_partials.restype = ctypes.c_int
    L.pkv_mla_decode_partials.argtypes = [P, P, I, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    _lib = L
    return L


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return PKV_F32
    if t == torch.bfloat16:
        return PKV_BF16
    if t in (torch.float8_e4m3fn, torch.uint8):
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise PkvError(fn, status)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


_KV_DTYPES = (torch.float32, torch.bfloat16, torch.float8_e4m3fn, torch.uint8)
_Q_DTYPES = (torch.float32, torch.bfloat16)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _want(name, t, dtypes, shape, optional=False):
    """Check one tensor argument before anything is launched: the C ABI takes
    raw pointers, so a wrong dtype or shape here would make a kernel read or
    write past the caller's buffers.  ``dtypes``: allowed torch dtypes (None:
    any); ``shape``: expected sizes, None for a size not fixed by the others.
    Raises TypeError (dtype) or ValueError (missing tensor, rank or size)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    if t.dim() != len(shape) or any(e is not None and e != g for e, g in zip(shape, t.shape)):
        want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")


def _want_pools(k_pool, v_pool, dtypes=_KV_DTYPES):
    """Pools [NB, Hkv, 16, D] of one dtype; returns (NB, Hkv, block_size, D)."""
    _want("k_pool", k_pool, dtypes, (None, None, None, None))
    nb, hkv, bs, d = k_pool.shape
    _want("v_pool", v_pool, (k_pool.dtype,), (nb, hkv, bs, d))
    return nb, hkv, bs, d


def _want_tables(block_tables, context_lens, num_seqs=None):
    """Tables int32 [B, max_blocks], lengths int32 [B]; returns B."""
    _want("block_tables", block_tables, _I32, (num_seqs, None))
    B = block_tables.shape[0]
    _want("context_lens", context_lens, _I32, (B,))
    return B


def _want_scales(k_scales, v_scales, nb, hkv):
    _want("k_scales", k_scales, _F32, (nb, hkv), optional=True)
    _want("v_scales", v_scales, _F32, (nb, hkv), optional=True)


def _want_query(q, out, num_rows=None):
    """q [rows, Hq, D] float32/bfloat16 and out of the same dtype and shape."""
    _want("q", q, _Q_DTYPES, (num_rows, None, None))
    _want("out", out, (q.dtype,), tuple(q.shape))


def _want_workspace(workspace):
    _want("workspace", workspace, None, (None,), optional=True)


def _nbytes(t):
    return t.numel() * t.element_size()


def kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens, stream=None):
    """Write every sequence's new K/V rows [B, Hkv, D] into slot ctx-1 (pkv_kv_append)."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want("k_new", k_new, (k_pool.dtype,), (B, hkv, d))
    _want("v_new", v_new, (k_pool.dtype,), (B, hkv, d))
    _need_cuda(k_pool, v_pool, k_new, v_new, block_tables, context_lens)
    _check("pkv_kv_append", load().pkv_kv_append(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
        _ptr(context_lens), B, hkv, d, bs, nb, block_tables.shape[1], dtype_code(k_pool.dtype),
        _stream(stream)))


def workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size):
    return int(load().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                 max_context_len, partition_size))


def alloc_workspace(num_seqs, num_q_heads, head_dim, max_context_len, partition_size, device):
    n = workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def paged_decode_attention(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                           softmax_scale, partition_size=512, k_scales=None, v_scales=None,
                           workspace=None, stream=None):
    """out[B, Hq, D] (q's dtype) = attention of q over each sequence's paged cache."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want_query(q, out, B)
    _want("q", q, None, (B, None, d))
    _want_scales(k_scales, v_scales, nb, hkv)
    _want_workspace(workspace)
    _need_cuda(out, q, k_pool, v_pool, block_tables, context_lens, k_scales, v_scales, workspace)
    hq = q.shape[1]
    if workspace is None:
        workspace = alloc_workspace(B, hq, d, max_context_len, partition_size, q.device)
    _check("pkv_paged_decode_attention", load().pkv_paged_decode_attention(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), _ptr(context_lens), B, hq, hkv, d, bs, nb, block_tables.shape[1],
        int(max_context_len), float(softmax_scale), int(partition_size), _ptr(workspace),
        _nbytes(workspace), dtype_code(q.dtype), dtype_code(k_pool.dtype), _stream(stream)))
    return out


def paged_decode_partials(partial_out, partial_lse, q, k_pool, v_pool, block_tables,
                          context_lens, softmax_scale, partition_size=512, k_scales=None,
                          v_scales=None, stream=None):
    """Unmerged split-KV results: partial_out [B, Hq, P, D] fp32, partial_lse [B, Hq, P] fp32."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want("q", q, _Q_DTYPES, (B, None, d))
    hq = q.shape[1]
    _want("partial_out", partial_out, _F32, (B, hq, None, d))
    _want("partial_lse", partial_lse, _F32, (B, hq, partial_out.shape[2]))
    _want_scales(k_scales, v_scales, nb, hkv)
    _need_cuda(partial_out, partial_lse, q, k_pool, v_pool, block_tables, context_lens,
               k_scales, v_scales)
    _check("pkv_paged_decode_partials", load().pkv_paged_decode_partials(
        _ptr(partial_out), _ptr(partial_lse), partial_out.shape[2], _ptr(q), _ptr(k_pool),
        _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), _ptr(context_lens), B,
        hq, hkv, d, bs, nb, block_tables.shape[1], float(softmax_scale), int(partition_size),
        dtype_code(q.dtype), dtype_code(k_pool.dtype), _stream(stream)))
    return partial_out, partial_lse


def merge_partials(out, partial_out, partial_lse, num_partitions=None, stream=None):
    """out[B, Hq, D] = LSE merge of partial_out [B, Hq, P, D] with partial_lse [B, Hq, P]."""
    _want("partial_out", partial_out, _F32, (None, None, None, None))
    B, hq, maxp, d = partial_out.shape
    _want("partial_lse", partial_lse, _F32, (B, hq, maxp))
    _want("out", out, _Q_DTYPES, (B, hq, d))
    _want("num_partitions", num_partitions, _I32, (B,), optional=True)
    _need_cuda(out, partial_out, partial_lse, num_partitions)
    _check("pkv_merge_partials", load().pkv_merge_partials(
        _ptr(out), _ptr(partial_out), _ptr(partial_lse), _ptr(num_partitions), B, hq, d, maxp,
        dtype_code(out.dtype), _stream(stream)))
    return out


def decode_plan_slots(num_seqs, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype):
    """Chunk slots of a balanced split for this shape (pkv_decode_plan_slots)."""
    n = int(load().pkv_decode_plan_slots(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         dtype_code(q_dtype), dtype_code(kv_dtype)))
    if n <= 0:
        raise PkvError("pkv_decode_plan_slots", 1)
    return n


def decode_plan(context_lens, num_slots, max_blocks_per_seq, plan=None, stream=None):
    """The balanced split's schedule (pkv_decode_plan) in a uint8 device
    buffer: chunk_first int32 [B + 1], then slot_info int32x4 [num_slots] at
    the offset plan_info_offset(B)."""
    _want("context_lens", context_lens, _I32, (None,))
    _want("plan", plan, (torch.uint8,), (None,), optional=True)
    _need_cuda(context_lens, plan)
    B = context_lens.shape[0]
    n = int(load().pkv_decode_plan_bytes(B, num_slots))
    if n == 0:
        raise PkvError("pkv_decode_plan_bytes", 1)
    if plan is None:
        plan = torch.empty(n, dtype=torch.uint8, device=context_lens.device)
    _check("pkv_decode_plan", load().pkv_decode_plan(
        _ptr(plan), plan.numel(), _ptr(context_lens), B, int(num_slots), BLOCK_SIZE,
        int(max_blocks_per_seq), _stream(stream)))
    return plan


def plan_info_offset(num_seqs):
    """Byte offset of slot_info in a plan: chunk_first rounded up to 256 bytes."""
    return (4 * (num_seqs + 1) + 255) // 256 * 256


def paged_decode_partials_planned(partial_out, partial_lse, plan, q, k_pool, v_pool,
                                  block_tables, context_lens, softmax_scale, k_scales=None,
                                  v_scales=None, stream=None):
    """Chunk results of a balanced split over R = partial_out.shape[0] slots:
    partial_out [R, Hq, D] fp32, partial_lse [R, Hq] fp32; the schedule is
    written into ``plan`` (uint8, pkv_decode_plan_bytes(B, R) bytes)."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want("q", q, _Q_DTYPES, (B, None, d))
    hq = q.shape[1]
    _want("partial_out", partial_out, _F32, (None, hq, d))
    _want("partial_lse", partial_lse, _F32, (partial_out.shape[0], hq))
    _want("plan", plan, (torch.uint8,), (None,))
    _want_scales(k_scales, v_scales, nb, hkv)
    _need_cuda(partial_out, partial_lse, plan, q, k_pool, v_pool, block_tables, context_lens,
               k_scales, v_scales)
    _check("pkv_paged_decode_partials_planned", load().pkv_paged_decode_partials_planned(
        _ptr(partial_out), _ptr(partial_lse), _ptr(plan), _nbytes(plan),
        partial_out.shape[0], _ptr(q),
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), _ptr(block_tables),
        _ptr(context_lens), B, hq, hkv, d, bs, nb, block_tables.shape[1], float(softmax_scale),
        dtype_code(q.dtype), dtype_code(k_pool.dtype), _stream(stream)))
    return partial_out, partial_lse


def merge_partials_planned(out, partial_out, partial_lse, plan, stream=None):
    """out[B, Hq, D] = LSE merge of each sequence's chunk rows of partial_out [R, Hq, D]."""
    _want("out", out, _Q_DTYPES, (None, None, None))
    B, hq, d = out.shape
    _want("partial_out", partial_out, _F32, (None, hq, d))
    _want("partial_lse", partial_lse, _F32, (partial_out.shape[0], hq))
    _want("plan", plan, (torch.uint8,), (None,))
    _need_cuda(out, partial_out, partial_lse, plan)
    _check("pkv_merge_partials_planned", load().pkv_merge_partials_planned(
        _ptr(out), _ptr(partial_out), _ptr(partial_lse), _ptr(plan), partial_out.shape[0], B, hq,
        d, dtype_code(out.dtype), _stream(stream)))
    return out


def decode_step(out, q, k_pool, v_pool, k_new, v_new, block_tables, context_lens,
                max_context_len, softmax_scale, partition_size=512, k_scales=None,
                v_scales=None, workspace=None, stream=None, fused=True):
    """One decode step: append the new K/V, then attend.  ``fused`` runs it as
    pkv_paged_decode_step (the append inside the decode kernel); otherwise as
    pkv_kv_append then pkv_paged_decode_attention on the same stream."""
    if not fused:
        kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens, stream)
        return paged_decode_attention(out, q, k_pool, v_pool, block_tables, context_lens,
                                      max_context_len, softmax_scale, partition_size, k_scales,
                                      v_scales, workspace, stream)
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want_query(q, out, B)
    _want("q", q, None, (B, None, d))
    _want("k_new", k_new, (k_pool.dtype,), (B, hkv, d))
    _want("v_new", v_new, (k_pool.dtype,), (B, hkv, d))
    _want_scales(k_scales, v_scales, nb, hkv)
    _want_workspace(workspace)
    _need_cuda(out, q, k_pool, v_pool, k_new, v_new, block_tables, context_lens, k_scales,
               v_scales, workspace)
    hq = q.shape[1]
    if workspace is None:
        workspace = alloc_workspace(B, hq, d, max_context_len, partition_size, q.device)
    _check("pkv_paged_decode_step", load().pkv_paged_decode_step(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(k_scales),
        _ptr(v_scales), _ptr(block_tables), _ptr(context_lens), B, hq, hkv, d, bs, nb,
        block_tables.shape[1], int(max_context_len), float(softmax_scale), int(partition_size),
        _ptr(workspace), _nbytes(workspace), dtype_code(q.dtype), dtype_code(k_pool.dtype),
        _stream(stream)))
    return out


PKV_NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_step_noalloc(out, q, k_pool, v_pool, k_new, v_new, block_tables, context_lens,
                        max_context_len, softmax_scale, partition_size=PKV_PARTITION_BALANCED,
                        k_scales=None, v_scales=None, stream=None):
    """pkv_paged_decode_step_noalloc: the fused decode step with the partial
    results in the library's own per-GPU device array (no workspace, nothing
    allocated); calls that overlap on one GPU race on that array."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want_query(q, out, B)
    _want("q", q, None, (B, None, d))
    _want("k_new", k_new, (k_pool.dtype,), (B, hkv, d))
    _want("v_new", v_new, (k_pool.dtype,), (B, hkv, d))
    _want_scales(k_scales, v_scales, nb, hkv)
    _need_cuda(out, q, k_pool, v_pool, k_new, v_new, block_tables, context_lens, k_scales,
               v_scales)
    _check("pkv_paged_decode_step_noalloc", load().pkv_paged_decode_step_noalloc(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(k_scales),
        _ptr(v_scales), _ptr(block_tables), _ptr(context_lens), B, q.shape[1], hkv, d, bs, nb,
        block_tables.shape[1], int(max_context_len), float(softmax_scale), int(partition_size),
        dtype_code(q.dtype), dtype_code(k_pool.dtype), _stream(stream)))
    return out


def kv_append_tokens(k_pool, v_pool, k_new, v_new, block_tables, context_lens, query_start_loc,
                     stream=None):
    """Write rows qsl[b] .. qsl[b+1]-1 of k_new/v_new [T, Hkv, D] into positions
    ctx_b - t_b .. ctx_b - 1 of sequence b (pkv_kv_append_tokens)."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want("query_start_loc", query_start_loc, _I32, (B + 1,))
    _want("k_new", k_new, (k_pool.dtype,), (None, hkv, d))
    _want("v_new", v_new, (k_pool.dtype,), (k_new.shape[0], hkv, d))
    _need_cuda(k_pool, v_pool, k_new, v_new, block_tables, context_lens, query_start_loc)
    _check("pkv_kv_append_tokens", load().pkv_kv_append_tokens(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start_loc), B, k_new.shape[0], hkv, d, bs, nb,
        block_tables.shape[1], dtype_code(k_pool.dtype), _stream(stream)))


def multi_query_workspace_bytes(num_tokens, num_q_heads, head_dim, max_context_len,
                                partition_size):
    return int(load().pkv_multi_query_workspace_bytes(num_tokens, num_q_heads, head_dim,
                                                      max_context_len, partition_size))


def paged_multi_query_attention(out, q, k_pool, v_pool, block_tables, context_lens,
                                query_start_loc, max_query_len, max_context_len, softmax_scale,
                                partition_size=512, k_scales=None, v_scales=None, workspace=None,
                                stream=None):
    """out[T, Hq, D] (q's dtype): row qsl[b] + j attends over the first
    ctx_b - t_b + j + 1 cached tokens of sequence b (pkv_paged_multi_query_attention)."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want("query_start_loc", query_start_loc, _I32, (B + 1,))
    _want_query(q, out)
    _want("q", q, None, (None, None, d))
    _want_scales(k_scales, v_scales, nb, hkv)
    _want_workspace(workspace)
    _need_cuda(out, q, k_pool, v_pool, block_tables, context_lens, query_start_loc, k_scales,
               v_scales, workspace)
    T, hq, _ = q.shape
    if workspace is None:
        if partition_size == PKV_PARTITION_BALANCED:
            n = int(load().pkv_multi_query_balanced_workspace_bytes(
                B, int(max_query_len), hq, hkv, d, dtype_code(q.dtype), dtype_code(k_pool.dtype)))
        else:
            n = multi_query_workspace_bytes(T, hq, d, max_context_len, partition_size)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check("pkv_paged_multi_query_attention", load().pkv_paged_multi_query_attention(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc), B, T, int(max_query_len),
        hq, hkv, d, bs, nb, block_tables.shape[1], int(max_context_len), float(softmax_scale),
        int(partition_size), _ptr(workspace), _nbytes(workspace), dtype_code(q.dtype),
        dtype_code(k_pool.dtype), _stream(stream)))
    return out


def paged_multi_query_partials(partial_out, partial_lse, q, k_pool, v_pool, block_tables,
                               context_lens, query_start_loc, max_query_len, softmax_scale,
                               partition_size=512, k_scales=None, v_scales=None, stream=None):
    """Unmerged split-KV results of the multi-token attention: partial_out
    [T, Hq, P, D] fp32, partial_lse [T, Hq, P] fp32 (pkv_paged_multi_query_partials)."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want("query_start_loc", query_start_loc, _I32, (B + 1,))
    _want("q", q, _Q_DTYPES, (None, None, d))
    T, hq, _ = q.shape
    _want("partial_out", partial_out, _F32, (T, hq, None, d))
    _want("partial_lse", partial_lse, _F32, (T, hq, partial_out.shape[2]))
    _want_scales(k_scales, v_scales, nb, hkv)
    _need_cuda(partial_out, partial_lse, q, k_pool, v_pool, block_tables, context_lens,
               query_start_loc, k_scales, v_scales)
    _check("pkv_paged_multi_query_partials", load().pkv_paged_multi_query_partials(
        _ptr(partial_out), _ptr(partial_lse), partial_out.shape[2], _ptr(q), _ptr(k_pool),
        _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start_loc), B, T, int(max_query_len), hq, hkv, d, bs, nb,
        block_tables.shape[1], float(softmax_scale), int(partition_size), dtype_code(q.dtype),
        dtype_code(k_pool.dtype), _stream(stream)))
    return partial_out, partial_lse


def multi_query_plan_slots(num_seqs, max_query_len, num_q_heads, num_kv_heads, head_dim, q_dtype,
                           kv_dtype):
    """Chunk slots of a balanced multi-token split for this shape (pkv_multi_query_plan_slots)."""
    n = int(load().pkv_multi_query_plan_slots(num_seqs, max_query_len, num_q_heads, num_kv_heads,
                                              head_dim, dtype_code(q_dtype), dtype_code(kv_dtype)))
    if n <= 0:
        raise PkvError("pkv_multi_query_plan_slots", 1)
    return n


def paged_multi_query_partials_planned(partial_out, partial_lse, plan, q, k_pool, v_pool,
                                       block_tables, context_lens, query_start_loc,
                                       max_query_len, softmax_scale, k_scales=None,
                                       v_scales=None, stream=None):
    """Chunk results of a balanced multi-token split over R = partial_out.shape[0]
    slots: partial_out [R, max_query_len, Hq, D] fp32, partial_lse [R,
    max_query_len, Hq] fp32; the schedule is written into ``plan`` (uint8,
    pkv_decode_plan_bytes(B, R) bytes)."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    B = _want_tables(block_tables, context_lens)
    _want("query_start_loc", query_start_loc, _I32, (B + 1,))
    _want("q", q, _Q_DTYPES, (None, None, d))
    T, hq, _ = q.shape
    _want("partial_out", partial_out, _F32, (None, int(max_query_len), hq, d))
    _want("partial_lse", partial_lse, _F32, (partial_out.shape[0], int(max_query_len), hq))
    _want("plan", plan, (torch.uint8,), (None,))
    _want_scales(k_scales, v_scales, nb, hkv)
    _need_cuda(partial_out, partial_lse, plan, q, k_pool, v_pool, block_tables, context_lens,
               query_start_loc, k_scales, v_scales)
    _check("pkv_paged_multi_query_partials_planned", load().pkv_paged_multi_query_partials_planned(
        _ptr(partial_out), _ptr(partial_lse), _ptr(plan), _nbytes(plan), partial_out.shape[0],
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start_loc), B, T, int(max_query_len), hq, hkv, d, bs, nb,
        block_tables.shape[1], float(softmax_scale), dtype_code(q.dtype), dtype_code(k_pool.dtype),
        _stream(stream)))
    return partial_out, partial_lse


def kv_append_quant(k_pool, v_pool, k_scales, v_scales, k_new, v_new, block_tables,
                    context_lens, query_start_loc=None, mode=PKV_SCALE_FIXED, stream=None):
    """Quantise bf16/fp32 rows [R, Hkv, D] into the e4m3 pools and append them
    (pkv_kv_append_quant); ``mode`` PKV_SCALE_FIXED or PKV_SCALE_RUNNING_AMAX."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool, (torch.float8_e4m3fn, torch.uint8))
    B = _want_tables(block_tables, context_lens)
    _want("k_scales", k_scales, _F32, (nb, hkv))
    _want("v_scales", v_scales, _F32, (nb, hkv))
    _want("query_start_loc", query_start_loc, _I32, (B + 1,), optional=True)
    _want("k_new", k_new, _Q_DTYPES, (B if query_start_loc is None else None, hkv, d))
    _want("v_new", v_new, (k_new.dtype,), (k_new.shape[0], hkv, d))
    _need_cuda(k_pool, v_pool, k_scales, v_scales, k_new, v_new, block_tables, context_lens,
               query_start_loc)
    _check("pkv_kv_append_quant", load().pkv_kv_append_quant(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), _ptr(k_new), _ptr(v_new),
        dtype_code(k_new.dtype), _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc), B,
        k_new.shape[0], hkv, d, bs, nb, block_tables.shape[1], int(mode), _stream(stream)))


class BlockManager:
    """The library's host-side block allocator (pkv_bm_*): on-demand blocks,
    reference counts, forks and copy-on-write.  ``append_slots`` returns the
    (src, dst) copies to run with ``copy_blocks`` before writing."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        self._L = load()
        self._h = self._L.pkv_bm_create(num_blocks, block_size)
        if not self._h:
            raise ValueError("pkv_bm_create failed")
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self):
        if self._h:
            self._L.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, seq: int):
        _check("pkv_bm_add_seq", self._L.pkv_bm_add_seq(self._h, seq))

    def fork(self, parent: int, child: int):
        _check("pkv_bm_fork", self._L.pkv_bm_fork(self._h, parent, child))

    def free_seq(self, seq: int):
        _check("pkv_bm_free_seq", self._L.pkv_bm_free_seq(self._h, seq))

    def append_slots(self, seq: int, n: int):
        src, dst, cnt = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pkv_bm_append_slots", self._L.pkv_bm_append_slots(
            self._h, seq, n, ctypes.byref(src), ctypes.byref(dst), 1, ctypes.byref(cnt)))
        return [(src.value, dst.value)] if cnt.value else []

    def num_free(self) -> int:
        return self._L.pkv_bm_num_free(self._h)

    def refcount(self, block: int) -> int:
        return self._L.pkv_bm_refcount(self._h, block)

    def seq_len(self, seq: int) -> int:
        return self._L.pkv_bm_seq_len(self._h, seq)

    def free_list(self):
        n = self._L.pkv_bm_free_list(self._h, None, 0)
        buf = (ctypes.c_int32 * max(n, 1))()
        self._L.pkv_bm_free_list(self._h, buf, n)
        return list(buf)[:n]

    def block_tables(self, seqs, max_blocks: int):
        """int32 numpy [len(seqs), max_blocks] tables (-1 padded) and lengths."""
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        tables = np.empty((len(ids), max_blocks), np.int32)
        lens = np.empty(len(ids), np.int32)
        _check("pkv_bm_block_tables", self._L.pkv_bm_block_tables(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), len(ids),
            tables.ctypes.data_as(ctypes.c_void_p), max_blocks,
            lens.ctypes.data_as(ctypes.c_void_p)))
        return tables, lens


def copy_blocks(k_pool, v_pool, pairs, k_scales=None, v_scales=None, stream=None):
    """Run copy-on-write copies: pairs int32 [n, 2] (src, dst) on the device."""
    nb, hkv, bs, d = _want_pools(k_pool, v_pool)
    _want("pairs", pairs, _I32, (None, 2))
    _want_scales(k_scales, v_scales, nb, hkv)
    _need_cuda(k_pool, v_pool, pairs, k_scales, v_scales)
    _check("pkv_copy_blocks", load().pkv_copy_blocks(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), _ptr(pairs),
        pairs.shape[0] if pairs.numel() else 0, nb, hkv, d, bs, dtype_code(k_pool.dtype),
        _stream(stream)))


def stream_read(src, num_workgroups, out=None, stream=None):
    """Read every byte of src once (pkv_stream_read, a bandwidth measurement);
    returns out, int32 [pkv_stream_read_out_words(num_workgroups)], whose XOR
    is the XOR of src's 32-bit words."""
    _want("out", out, _I32, (None,), optional=True)
    _need_cuda(src, out)
    words = int(load().pkv_stream_read_out_words(num_workgroups))
    if words == 0:
        raise ValueError(f"num_workgroups {num_workgroups} out of range")
    if out is None:
        out = torch.empty(words, dtype=torch.int32, device=src.device)
    elif out.numel() < words:
        raise ValueError(f"out holds {out.numel()} words, {words} needed")
    _check("pkv_stream_read", load().pkv_stream_read(
        _ptr(out), _ptr(src), src.numel() * src.element_size(), num_workgroups, _stream(stream)))
    return out


def gather_read(src, chunk_ids, chunks_per_workgroup, out=None, stream=None):
    """Read the 4 KiB chunks chunk_ids (int32) of src once (pkv_gather_read, a
    bandwidth measurement of the decode kernels' access pattern); returns out,
    int32 [64 * len(chunk_ids) / chunks_per_workgroup]: lane l of workgroup w
    holds the XOR of the 32-bit words it read."""
    _want("chunk_ids", chunk_ids, _I32, (None,))
    _want("out", out, _I32, (None,), optional=True)
    _need_cuda(src, chunk_ids, out)
    n = chunk_ids.shape[0]
    if chunks_per_workgroup <= 0 or n % chunks_per_workgroup:
        raise ValueError("the chunk count must be a multiple of chunks_per_workgroup")
    words = 64 * (n // chunks_per_workgroup)
    if out is None:
        out = torch.empty(words, dtype=torch.int32, device=src.device)
    elif out.numel() < words:
        raise ValueError(f"out holds {out.numel()} words, {words} needed")
    _check("pkv_gather_read", load().pkv_gather_read(
        _ptr(out), _ptr(src), _nbytes(src), _ptr(chunk_ids), n, int(chunks_per_workgroup),
        _stream(stream)))
    return out


def mla_append(latent_pool, latent_new, block_tables, context_lens, stream=None):
    """Write each sequence's new 576-number row into slot ctx-1 (pkv_mla_append)."""
    _want("latent_pool", latent_pool, (torch.bfloat16,), (None, None, None))
    nb, bs, d = latent_pool.shape
    B = _want_tables(block_tables, context_lens)
    _want("latent_new", latent_new, (torch.bfloat16,), (B, d))
    _need_cuda(latent_pool, latent_new, block_tables, context_lens)
    _check("pkv_mla_append", load().pkv_mla_append(
        _ptr(latent_pool), _ptr(latent_new), _ptr(block_tables), _ptr(context_lens),
        block_tables.shape[0], d, bs, nb, block_tables.shape[1], _stream(stream)))


def mla_decode_attention(out, q, latent_pool, block_tables, context_lens, max_context_len,
                         softmax_scale, partition_size=512, kv_lora_rank=512, workspace=None,
                         stream=None):
    """out [B, H, 512] bf16: absorbed MLA decode of q [B, H, 576] over the paged
    latent rows (pkv_mla_decode_attention); partition_size PKV_PARTITION_BALANCED
    splits the batch's work into balanced chunks."""
    _want("latent_pool", latent_pool, (torch.bfloat16,), (None, None, None))
    nb, bs, d = latent_pool.shape
    B = _want_tables(block_tables, context_lens)
    _want("q", q, (torch.bfloat16,), (B, None, d))
    H = q.shape[1]
    _want("out", out, (torch.bfloat16,), (B, H, kv_lora_rank))
    _want_workspace(workspace)
    _need_cuda(out, q, latent_pool, block_tables, context_lens, workspace)
    if workspace is None:
        n = int(load().pkv_mla_workspace_bytes(B, H, kv_lora_rank, max_context_len,
                                               partition_size))
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check("pkv_mla_decode_attention", load().pkv_mla_decode_attention(
        _ptr(out), _ptr(q), _ptr(latent_pool), _ptr(block_tables), _ptr(context_lens), B, H,
        kv_lora_rank, d - kv_lora_rank, bs, nb, block_tables.shape[1], int(max_context_len),
        float(softmax_scale), int(partition_size), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))
    return out


def mla_decode_partials(partial_out, partial_lse, q, latent_pool, block_tables, context_lens,
                        softmax_scale, partition_size=512, kv_lora_rank=512, stream=None):
    """Unmerged MLA split-KV results: partial_out [B, H, P, 512], partial_lse [B, H, P]."""
    _want("latent_pool", latent_pool, (torch.bfloat16,), (None, None, None))
    nb, bs, d = latent_pool.shape
    B = _want_tables(block_tables, context_lens)
    _want("q", q, (torch.bfloat16,), (B, None, d))
    H = q.shape[1]
    _want("partial_out", partial_out, _F32, (B, H, None, kv_lora_rank))
    _want("partial_lse", partial_lse, _F32, (B, H, partial_out.shape[2]))
    _need_cuda(partial_out, partial_lse, q, latent_pool, block_tables, context_lens)
    _check("pkv_mla_decode_partials", load().pkv_mla_decode_partials(
        _ptr(partial_out), _ptr(partial_lse), partial_out.shape[2], _ptr(q), _ptr(latent_pool),
        _ptr(block_tables), _ptr(context_lens), B, H, kv_lora_rank, d - kv_lora_rank, bs, nb,
        block_tables.shape[1], float(softmax_scale), int(partition_size), _stream(stream)))
    return partial_out, partial_lse
