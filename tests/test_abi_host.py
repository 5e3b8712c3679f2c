"""The C ABI on the host: the library loads, exports every entry point the
header declares, and rejects bad arguments before launching anything.  No
GPU is needed: every call here fails validation, so no HIP call is made."""

import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_cache_25_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(pkv_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libpkv.so not built")
    return ops.load()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "pkv_abi_version", "pkv_status_string", "pkv_kv_append", "pkv_decode_workspace_bytes",
        "pkv_paged_decode_attention", "pkv_paged_decode_step", "pkv_paged_decode_partials",
        "pkv_merge_partials", "pkv_kv_append_tokens", "pkv_multi_query_workspace_bytes",
        "pkv_paged_multi_query_attention", "pkv_paged_multi_query_partials",
        "pkv_kv_append_quant", "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_add_seq",
        "pkv_bm_fork", "pkv_bm_free_seq", "pkv_bm_append_slots", "pkv_bm_num_free",
        "pkv_bm_refcount", "pkv_bm_seq_len", "pkv_bm_free_list", "pkv_bm_block_tables",
        "pkv_copy_blocks", "pkv_mla_append", "pkv_mla_workspace_bytes",
        "pkv_mla_decode_attention", "pkv_mla_decode_partials"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(lib):
    assert lib.pkv_abi_version() == 1
    for code, name in ops.STATUS.items():
        assert lib.pkv_status_string(code).decode() == name
    assert lib.pkv_status_string(99).decode() == "PKV_UNKNOWN_STATUS"


def _append(lib, **over):
    a = dict(k_pool=FAKE, v_pool=FAKE, k_new=FAKE, v_new=FAKE, tables=FAKE, lens=FAKE, B=2, hkv=2,
             d=128, bs=16, nb=8, mbps=4, kv=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_kv_append(a["k_pool"], a["v_pool"], a["k_new"], a["v_new"], a["tables"],
                             a["lens"], a["B"], a["hkv"], a["d"], a["bs"], a["nb"], a["mbps"],
                             a["kv"], None)


def test_append_validation(lib):
    assert _append(lib, k_pool=None) == INVALID
    assert _append(lib, lens=None) == INVALID
    assert _append(lib, hkv=0) == INVALID
    assert _append(lib, B=-1) == INVALID
    assert _append(lib, kv=7) == INVALID
    assert _append(lib, d=96) == UNSUPPORTED
    assert _append(lib, bs=8) == UNSUPPORTED
    assert _append(lib, B=0, k_pool=None) == OK       # empty batch: nothing to do


def _decode(lib, **over):
    a = dict(out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, ks=None, vs=None, tables=FAKE, lens=FAKE, B=2,
             hq=8, hkv=2, d=128, bs=16, nb=8, mbps=4, maxctx=64, scale=0.088, P=16, ws=None,
             wsb=0, qt=ops.PKV_BF16, kvt=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_paged_decode_attention(
        a["out"], a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["tables"], a["lens"], a["B"],
        a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mbps"], a["maxctx"], a["scale"], a["P"],
        a["ws"], a["wsb"], a["qt"], a["kvt"], None)


def test_decode_validation(lib):
    assert _decode(lib, q=None) == INVALID
    assert _decode(lib, tables=None) == INVALID
    assert _decode(lib, hq=6, hkv=4) == INVALID           # Hq % Hkv != 0
    assert _decode(lib, P=24) == INVALID                  # not a multiple of the block size
    assert _decode(lib, P=-16) == INVALID
    assert _decode(lib, maxctx=-1) == INVALID
    assert _decode(lib, scale=float("nan")) == INVALID
    assert _decode(lib, d=256) == UNSUPPORTED
    assert _decode(lib, bs=32, P=32) == UNSUPPORTED
    assert _decode(lib, qt=ops.PKV_FP8_E4M3) == UNSUPPORTED
    assert _decode(lib, kvt=ops.PKV_FP8_E4M3) == INVALID  # e4m3 without scales
    assert _decode(lib, kvt=ops.PKV_FP8_E4M3, ks=FAKE) == INVALID
    assert _decode(lib) == WORKSPACE                      # 4 partitions and no workspace
    need = lib.pkv_decode_workspace_bytes(2, 8, 128, 64, 16)
    assert _decode(lib, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _decode(lib, B=0, q=None) == OK


def test_alignment_checked(lib):
    odd = ctypes.c_void_p(0x10008)                        # 8-byte aligned only
    assert _append(lib, k_pool=odd) == INVALID
    assert _append(lib, tables=ctypes.c_void_p(0x10002)) == INVALID
    need = lib.pkv_decode_workspace_bytes(2, 8, 128, 64, 16)
    assert _decode(lib, q=odd, ws=FAKE, wsb=need) == INVALID
    assert _decode(lib, out=odd, ws=FAKE, wsb=need) == INVALID
    assert _decode(lib, ws=odd, wsb=need) == INVALID
    f = lib.pkv_merge_partials
    assert f(FAKE, odd, FAKE, None, 2, 4, 128, 3, ops.PKV_BF16, None) == INVALID


def _step(lib, **over):
    a = dict(out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, kn=FAKE, vn=FAKE, ks=None, vs=None, tables=FAKE,
             lens=FAKE, B=2, hq=8, hkv=2, d=128, bs=16, nb=8, mbps=4, maxctx=64, scale=0.088,
             P=16, ws=None, wsb=0, qt=ops.PKV_BF16, kvt=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_paged_decode_step(
        a["out"], a["q"], a["kp"], a["vp"], a["kn"], a["vn"], a["ks"], a["vs"], a["tables"],
        a["lens"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mbps"], a["maxctx"],
        a["scale"], a["P"], a["ws"], a["wsb"], a["qt"], a["kvt"], None)


def test_step_validation(lib):
    assert _step(lib, kn=None) == INVALID
    assert _step(lib, vn=ctypes.c_void_p(0x10008)) == INVALID
    assert _step(lib, q=None) == INVALID
    assert _step(lib, hq=6, hkv=4) == INVALID
    assert _step(lib, d=96) == UNSUPPORTED
    assert _step(lib) == WORKSPACE
    assert _step(lib, B=0, kn=None, q=None) == OK


def _partials(lib, **over):
    a = dict(po=FAKE, pl=FAKE, maxp=4, q=FAKE, kp=FAKE, vp=FAKE, ks=None, vs=None, tables=FAKE,
             lens=FAKE, B=2, hq=8, hkv=2, d=128, bs=16, nb=8, mbps=4, scale=0.088, P=16,
             qt=ops.PKV_BF16, kvt=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_paged_decode_partials(
        a["po"], a["pl"], a["maxp"], a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["tables"],
        a["lens"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mbps"], a["scale"],
        a["P"], a["qt"], a["kvt"], None)


def test_partials_validation(lib):
    assert _partials(lib, po=None) == INVALID
    assert _partials(lib, pl=None) == INVALID
    assert _partials(lib, maxp=0) == INVALID
    assert _partials(lib, po=ctypes.c_void_p(0x10008)) == INVALID
    assert _partials(lib, hq=6, hkv=4) == INVALID
    assert _partials(lib, P=24) == INVALID
    assert _partials(lib, d=96) == UNSUPPORTED
    assert _partials(lib, kvt=ops.PKV_FP8_E4M3) == INVALID
    assert _partials(lib, B=0, po=None) == OK


def test_workspace_size(lib):
    # maxP = ceil(4096 / 512) = 8; o: 64*32*8*128*4 B; lse 64*32*8*4 B, both 256-aligned
    assert lib.pkv_decode_workspace_bytes(64, 32, 128, 4096, 512) == 64 * 32 * 8 * 128 * 4 + 64 * 32 * 8 * 4
    assert lib.pkv_decode_workspace_bytes(4, 4, 64, 100, 512) == 0      # one partition
    assert lib.pkv_decode_workspace_bytes(4, 4, 64, 100, 0) == 0
    assert lib.pkv_decode_workspace_bytes(1, 1, 64, 17, 16) == 512 + 256   # maxP = 2


def test_merge_validation(lib):
    f = lib.pkv_merge_partials
    assert f(None, FAKE, FAKE, None, 2, 4, 128, 3, ops.PKV_BF16, None) == INVALID
    assert f(FAKE, FAKE, FAKE, None, 2, 4, 128, 0, ops.PKV_BF16, None) == INVALID
    assert f(FAKE, FAKE, FAKE, None, 2, 4, 96, 3, ops.PKV_BF16, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, None, 2, 4, 128, 3, ops.PKV_FP8_E4M3, None) == UNSUPPORTED
    assert f(None, None, None, None, 0, 4, 128, 3, ops.PKV_F32, None) == OK


def _append_tokens(lib, **over):
    a = dict(k_pool=FAKE, v_pool=FAKE, k_new=FAKE, v_new=FAKE, tables=FAKE, lens=FAKE, qsl=FAKE,
             B=2, T=5, hkv=2, d=128, bs=16, nb=8, mbps=4, kv=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_kv_append_tokens(a["k_pool"], a["v_pool"], a["k_new"], a["v_new"],
                                    a["tables"], a["lens"], a["qsl"], a["B"], a["T"], a["hkv"],
                                    a["d"], a["bs"], a["nb"], a["mbps"], a["kv"], None)


def test_append_tokens_validation(lib):
    assert _append_tokens(lib, qsl=None) == INVALID
    assert _append_tokens(lib, qsl=ctypes.c_void_p(0x10002)) == INVALID
    assert _append_tokens(lib, k_new=ctypes.c_void_p(0x10008)) == INVALID
    assert _append_tokens(lib, T=-1) == INVALID
    assert _append_tokens(lib, hkv=0) == INVALID
    assert _append_tokens(lib, d=96) == UNSUPPORTED
    assert _append_tokens(lib, T=0, k_pool=None, qsl=None) == OK     # no new rows
    assert _append_tokens(lib, B=0, k_pool=None, qsl=None) == OK


def _multi(lib, **over):
    a = dict(out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, ks=None, vs=None, tables=FAKE, lens=FAKE,
             qsl=FAKE, B=2, T=6, maxq=4, hq=8, hkv=2, d=128, bs=16, nb=8, mbps=4, maxctx=64,
             scale=0.088, P=16, ws=None, wsb=0, qt=ops.PKV_BF16, kvt=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_paged_multi_query_attention(
        a["out"], a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["tables"], a["lens"], a["qsl"],
        a["B"], a["T"], a["maxq"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mbps"],
        a["maxctx"], a["scale"], a["P"], a["ws"], a["wsb"], a["qt"], a["kvt"], None)


def test_multi_query_validation(lib):
    need = lib.pkv_multi_query_workspace_bytes(6, 8, 128, 64, 16)
    assert need == lib.pkv_decode_workspace_bytes(6, 8, 128, 64, 16) > 0
    assert _multi(lib, qsl=None, ws=FAKE, wsb=need) == INVALID
    assert _multi(lib, qsl=ctypes.c_void_p(0x10002), ws=FAKE, wsb=need) == INVALID
    assert _multi(lib, maxq=0, ws=FAKE, wsb=need) == INVALID
    assert _multi(lib, maxq=-1) == INVALID
    assert _multi(lib, T=-1) == INVALID
    assert _multi(lib, maxctx=-1) == INVALID
    assert _multi(lib, hq=6, hkv=4) == INVALID
    assert _multi(lib, P=24) == INVALID
    assert _multi(lib, d=96) == UNSUPPORTED
    assert _multi(lib, qt=ops.PKV_FP8_E4M3) == UNSUPPORTED
    assert _multi(lib, kvt=ops.PKV_FP8_E4M3) == INVALID        # e4m3 without scales
    assert _multi(lib, out=ctypes.c_void_p(0x10008), ws=FAKE, wsb=need) == INVALID
    assert _multi(lib) == WORKSPACE                            # 4 partitions, no workspace
    assert _multi(lib, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _multi(lib, B=0, q=None, qsl=None) == OK
    assert _multi(lib, T=0, q=None, qsl=None) == OK


def _multi_partials(lib, **over):
    a = dict(po=FAKE, pl=FAKE, maxp=4, q=FAKE, kp=FAKE, vp=FAKE, ks=None, vs=None, tables=FAKE,
             lens=FAKE, qsl=FAKE, B=2, T=6, maxq=4, hq=8, hkv=2, d=128, bs=16, nb=8, mbps=4,
             scale=0.088, P=16, qt=ops.PKV_BF16, kvt=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_paged_multi_query_partials(
        a["po"], a["pl"], a["maxp"], a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["tables"],
        a["lens"], a["qsl"], a["B"], a["T"], a["maxq"], a["hq"], a["hkv"], a["d"], a["bs"],
        a["nb"], a["mbps"], a["scale"], a["P"], a["qt"], a["kvt"], None)


def test_multi_query_partials_validation(lib):
    assert _multi_partials(lib, po=None) == INVALID
    assert _multi_partials(lib, pl=None) == INVALID
    assert _multi_partials(lib, maxp=0) == INVALID
    assert _multi_partials(lib, qsl=None) == INVALID
    assert _multi_partials(lib, maxq=0) == INVALID
    assert _multi_partials(lib, po=ctypes.c_void_p(0x10008)) == INVALID
    assert _multi_partials(lib, P=24) == INVALID
    assert _multi_partials(lib, d=96) == UNSUPPORTED
    assert _multi_partials(lib, kvt=ops.PKV_FP8_E4M3) == INVALID
    assert _multi_partials(lib, T=0, po=None, qsl=None) == OK


def _quant(lib, **over):
    a = dict(kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, kn=FAKE, vn=FAKE, nd=ops.PKV_BF16, tables=FAKE,
             lens=FAKE, qsl=None, B=2, R=2, hkv=2, d=128, bs=16, nb=8, mbps=4,
             mode=ops.PKV_SCALE_RUNNING_AMAX)
    a.update(over)
    return lib.pkv_kv_append_quant(a["kp"], a["vp"], a["ks"], a["vs"], a["kn"], a["vn"], a["nd"],
                                   a["tables"], a["lens"], a["qsl"], a["B"], a["R"], a["hkv"],
                                   a["d"], a["bs"], a["nb"], a["mbps"], a["mode"], None)


def test_quant_append_validation(lib):
    assert _quant(lib, ks=None) == INVALID
    assert _quant(lib, vn=None) == INVALID
    assert _quant(lib, nd=ops.PKV_FP8_E4M3) == INVALID       # new rows must be wider
    assert _quant(lib, mode=2) == INVALID
    assert _quant(lib, kn=ctypes.c_void_p(0x10008)) == INVALID
    assert _quant(lib, ks=ctypes.c_void_p(0x10002)) == INVALID
    assert _quant(lib, qsl=ctypes.c_void_p(0x10002)) == INVALID
    assert _quant(lib, hkv=0) == INVALID
    assert _quant(lib, d=96) == UNSUPPORTED
    assert _quant(lib, bs=8) == UNSUPPORTED
    assert _quant(lib, B=0, kp=None) == OK
    assert _quant(lib, R=0, kp=None) == OK


def _copy(lib, **over):
    a = dict(kp=FAKE, vp=FAKE, ks=None, vs=None, pairs=FAKE, n=3, nb=8, hkv=2, d=128, bs=16,
             kv=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_copy_blocks(a["kp"], a["vp"], a["ks"], a["vs"], a["pairs"], a["n"], a["nb"],
                               a["hkv"], a["d"], a["bs"], a["kv"], None)


def test_copy_blocks_validation(lib):
    assert _copy(lib, pairs=None) == INVALID
    assert _copy(lib, kp=None) == INVALID
    assert _copy(lib, n=-1) == INVALID
    assert _copy(lib, kv=ops.PKV_FP8_E4M3) == INVALID          # e4m3 without scales
    assert _copy(lib, kp=ctypes.c_void_p(0x10008)) == INVALID
    assert _copy(lib, pairs=ctypes.c_void_p(0x10002)) == INVALID
    assert _copy(lib, d=96) == UNSUPPORTED
    assert _copy(lib, hkv=300) == UNSUPPORTED
    assert _copy(lib, n=0, kp=None, pairs=None) == OK


def _mla(lib, **over):
    a = dict(out=FAKE, q=FAKE, pool=FAKE, tables=FAKE, lens=FAKE, B=2, H=128, dc=512, dr=64,
             bs=16, nb=8, mbps=4, maxctx=64, scale=0.07, P=32, ws=None, wsb=0)
    a.update(over)
    return lib.pkv_mla_decode_attention(a["out"], a["q"], a["pool"], a["tables"], a["lens"],
                                        a["B"], a["H"], a["dc"], a["dr"], a["bs"], a["nb"],
                                        a["mbps"], a["maxctx"], a["scale"], a["P"], a["ws"],
                                        a["wsb"], None)


def test_mla_validation(lib):
    need = lib.pkv_mla_workspace_bytes(2, 128, 512, 64, 32)       # maxP = 2
    assert need == 2 * 128 * 2 * 512 * 4 + 2 * 128 * 2 * 4
    assert lib.pkv_mla_workspace_bytes(2, 128, 512, 32, 32) == 0
    assert _mla(lib, q=None, ws=FAKE, wsb=need) == INVALID
    assert _mla(lib, P=24) == INVALID
    assert _mla(lib, maxctx=-1) == INVALID
    assert _mla(lib, scale=float("nan")) == INVALID
    assert _mla(lib, dc=256) == UNSUPPORTED
    assert _mla(lib, dr=32) == UNSUPPORTED
    assert _mla(lib, H=24) == UNSUPPORTED
    assert _mla(lib, bs=32, P=32) == UNSUPPORTED
    assert _mla(lib) == WORKSPACE
    assert _mla(lib, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _mla(lib, out=ctypes.c_void_p(0x10008), ws=FAKE, wsb=need) == INVALID
    assert _mla(lib, B=0, q=None) == OK
    f = lib.pkv_mla_append
    assert f(None, FAKE, FAKE, FAKE, 2, 576, 16, 8, 4, None) == INVALID
    assert f(FAKE, ctypes.c_void_p(0x10008), FAKE, FAKE, 2, 576, 16, 8, 4, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 512, 16, 8, 4, None) == UNSUPPORTED
    assert f(None, None, None, None, 0, 576, 16, 8, 4, None) == OK
    g = lib.pkv_mla_decode_partials
    args = [FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, 2, 128, 512, 64, 16, 8, 4, 0.07, 32, None]
    for i, bad in ((0, None), (2, 0), (3, None), (8, 24), (15, 24)):
        a = list(args)
        a[i] = bad
        assert g(*a) in (INVALID, UNSUPPORTED), i
    a = list(args); a[9] = 256
    assert g(*a) == UNSUPPORTED
    a = list(args); a[15] = -1                                     # balanced: attention only
    assert g(*a) == INVALID


def _align(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("B,H,slots", [(2, 128, 256), (2, 64, 512), (2, 16, 512), (300, 128, 300),
                                       (700, 16, 700)])
def test_mla_balanced_workspace(lib, B, H, slots):
    """PKV_PARTITION_BALANCED: o [R, H, 512] f32 | lse [R, H] f32 | chunk starts
    [B + 1] int32, each 256-byte aligned, R = max(256 for 8-wave workgroups
    (more than 64 heads) or 512, B); max_context_len does not enter."""
    want = _align(slots * H * 512 * 4) + _align(slots * H * 4) + _align((B + 1) * 4)
    for maxctx in (0, 17, 100000):
        assert lib.pkv_mla_workspace_bytes(B, H, 512, maxctx, -1) == want
    assert lib.pkv_mla_workspace_bytes(B, H, 512, 64, -2) == 0


def test_mla_balanced_validation(lib):
    need = lib.pkv_mla_workspace_bytes(2, 128, 512, 64, -1)
    assert _mla(lib, P=-1) == WORKSPACE                             # nothing launched
    assert _mla(lib, P=-1, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _mla(lib, P=-2, ws=FAKE, wsb=need) == INVALID
    assert _mla(lib, P=-1, H=24, ws=FAKE, wsb=need) == UNSUPPORTED
    assert _mla(lib, P=-1, ws=ctypes.c_void_p(0x10008), wsb=need) == INVALID
    assert _mla(lib, P=-1, B=0, q=None) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros(4, 2, 16, 64)
    with pytest.raises(ValueError):
        ops.kv_append(t, t, t[:, :, 0], t[:, :, 0], torch.zeros(1, 1, dtype=torch.int32),
                      torch.zeros(1, dtype=torch.int32))
