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
        "pkv_paged_decode_attention", "pkv_paged_decode_step", "pkv_paged_decode_step_noalloc",
        "pkv_paged_decode_partials",
        "pkv_merge_partials", "pkv_kv_append_tokens", "pkv_multi_query_workspace_bytes",
        "pkv_paged_multi_query_attention", "pkv_paged_multi_query_partials",
        "pkv_multi_query_plan_slots", "pkv_paged_multi_query_partials_planned",
        "pkv_kv_append_quant", "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_add_seq",
        "pkv_bm_fork", "pkv_bm_free_seq", "pkv_bm_append_slots", "pkv_bm_num_free",
        "pkv_bm_refcount", "pkv_bm_seq_len", "pkv_bm_free_list", "pkv_bm_block_tables",
        "pkv_copy_blocks", "pkv_mla_append", "pkv_mla_workspace_bytes",
        "pkv_mla_decode_attention", "pkv_mla_decode_partials", "pkv_decode_plan_slots",
        "pkv_decode_plan_bytes", "pkv_decode_plan", "pkv_paged_decode_partials_planned",
        "pkv_merge_partials_planned", "pkv_multi_query_balanced_workspace_bytes",
        "pkv_stream_read", "pkv_stream_read_out_words", "pkv_gather_read"])


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


def _step_noalloc(lib, **over):
    a = dict(out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, kn=FAKE, vn=FAKE, ks=None, vs=None, tables=FAKE,
             lens=FAKE, B=2, hq=8, hkv=2, d=128, bs=16, nb=8, mbps=4, maxctx=64, scale=0.088,
             P=16, qt=ops.PKV_BF16, kvt=ops.PKV_BF16)
    a.update(over)
    return lib.pkv_paged_decode_step_noalloc(
        a["out"], a["q"], a["kp"], a["vp"], a["kn"], a["vn"], a["ks"], a["vs"], a["tables"],
        a["lens"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mbps"], a["maxctx"],
        a["scale"], a["P"], a["qt"], a["kvt"], None)


def test_step_noalloc_validation(lib):
    """Argument checks and the size limit come before the device is touched."""
    assert _step_noalloc(lib, kn=None) == INVALID
    assert _step_noalloc(lib, out=ctypes.c_void_p(0x10008)) == INVALID
    assert _step_noalloc(lib, q=None) == INVALID
    assert _step_noalloc(lib, hq=6, hkv=4) == INVALID
    assert _step_noalloc(lib, d=96) == UNSUPPORTED
    assert _step_noalloc(lib, B=0, kn=None, q=None) == OK
    # 256 sequences x 32 heads x head dim 128 with up to 64 partitions of 512
    # tokens: 270 MB of partials, past the 32 MiB array
    assert _step_noalloc(lib, B=256, hq=32, hkv=8, mbps=2048, maxctx=32768, P=512) == WORKSPACE
    assert ops.PKV_NOALLOC_SCRATCH_BYTES == 32 << 20


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
    assert _partials(lib, P=-1) == INVALID                # balanced: the planned call
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
    # the balanced split: sized by its own function, checked before any launch
    bal = lib.pkv_multi_query_balanced_workspace_bytes(2, 4, 8, 2, 128, ops.PKV_BF16, ops.PKV_BF16)
    assert bal > 0
    assert _multi(lib, P=-1) == WORKSPACE
    assert _multi(lib, P=-1, ws=FAKE, wsb=bal - 1) == WORKSPACE
    assert _multi(lib, P=-2, ws=FAKE, wsb=bal) == INVALID
    assert _multi(lib, P=-1, qsl=None, ws=FAKE, wsb=bal) == INVALID
    assert _multi_partials(lib, P=-1) == INVALID                 # no balanced partials call


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


def test_stream_read_validation(lib):
    big = 1 << 20                                                   # the header's maximum
    assert lib.pkv_stream_read_out_words(1) == 4                    # one word per wave
    assert lib.pkv_stream_read_out_words(big) == 4 * big
    assert lib.pkv_stream_read_out_words(0) == 0
    assert lib.pkv_stream_read_out_words(big + 1) == 0
    read = lambda out, src, n, g: lib.pkv_stream_read(out, src, n, g, None)
    assert read(FAKE, FAKE, 1024, 0) == INVALID
    assert read(FAKE, FAKE, 1024, big + 1) == INVALID
    assert read(FAKE, FAKE, 1000, 8) == INVALID                     # not a multiple of 16
    assert read(None, FAKE, 1024, 8) == INVALID
    assert read(ctypes.c_void_p(0x10002), FAKE, 1024, 8) == INVALID
    assert read(FAKE, None, 1024, 8) == INVALID
    assert read(FAKE, ctypes.c_void_p(0x10008), 1024, 8) == INVALID


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


@pytest.mark.parametrize("B,hq,hkv,kind,slots", [
    (64, 32, 8, "mfma", 384),       # 8 KV heads x 1 tile of 16 columns: S = 3072 / 8
    (256, 32, 8, "mfma", 768),      # 2B > S: two waves' worth
    (128, 32, 32, "vector", 256),   # S = 3072 / 32 = 96: 2B
    (192, 32, 8, "mfma", 384),      # 2B = S: one wave
    (193, 32, 8, "mfma", 768),
    (3, 4, 4, "f32", 768),          # vector tiles of one column: 3072 / 4
    (2, 64, 1, "mfma", 768),        # 64 columns = 4 tiles of 16
    (5000, 8, 1, "mfma", 10000)])
def test_decode_plan_slots(lib, B, hq, hkv, kind, slots):
    """R = S if 2B <= S else max(2S, 2B), S = 3072 // (KV heads x column
    tiles): the one-wave decode workgroups MI355X holds at once (256 CUs x 4
    SIMDs x 3 waves)."""
    qt, kvt = {"mfma": (ops.PKV_BF16, ops.PKV_BF16), "vector": (ops.PKV_BF16, ops.PKV_FP8_E4M3),
               "f32": (ops.PKV_F32, ops.PKV_F32)}[kind]
    assert lib.pkv_decode_plan_slots(B, hq, hkv, 128, qt, kvt) == slots
    # The workspace function, which does not know num_kv_heads, bounds it.
    ws = lib.pkv_decode_workspace_bytes(B, hq, 128, 0, -1)
    used = _align(slots * hq * 128 * 4) + _align(slots * hq * 4) + lib.pkv_decode_plan_bytes(B, slots)
    assert ws >= used


def test_decode_plan_layout(lib):
    """chunk_first int32 [B + 1] then slot_info int32x4 [R], each 256-aligned;
    the balanced workspace is o | lse | plan at the bound
    R = max(2 x 3072 // ceil(Hq/16), 2B)."""
    assert lib.pkv_decode_plan_bytes(64, 384) == 512 + 384 * 16
    assert lib.pkv_decode_plan_bytes(0, 1) == 256 + 256
    assert lib.pkv_decode_plan_bytes(10, 9) == 0                   # fewer slots than sequences
    assert lib.pkv_decode_plan_bytes(1, 0) == 0
    r = 2 * (3072 // 2)
    assert lib.pkv_decode_workspace_bytes(64, 32, 128, 4096, -1) == (
        _align(r * 32 * 128 * 4) + _align(r * 32 * 4) + lib.pkv_decode_plan_bytes(64, r))
    assert lib.pkv_decode_workspace_bytes(64, 32, 128, 0, -1) == lib.pkv_decode_workspace_bytes(
        64, 32, 128, 100000, -1)                                  # max_context_len does not enter
    assert lib.pkv_decode_workspace_bytes(64, 32, 128, 4096, -2) == 0
    assert lib.pkv_multi_query_workspace_bytes(64, 32, 128, 4096, -1) == 0
    # several new tokens: [R, max_q, Hq, D] | [R, max_q, Hq] | plan; t = 4, g = 4: one
    # 16-column tile per KV head, so R = 384 as for one token
    t = 4
    assert lib.pkv_multi_query_balanced_workspace_bytes(64, t, 32, 8, 128, ops.PKV_BF16,
                                                        ops.PKV_BF16) == (
        _align(384 * t * 32 * 128 * 4) + _align(384 * t * 32 * 4) + lib.pkv_decode_plan_bytes(64, 384))
    # t = 16: 64 columns = 2 waves of two tiles each (two waves per SIMD resident, 2048 in
    # all): units 8 x 2 = 16, S = 128, 2B = 128 <= S
    assert lib.pkv_multi_query_balanced_workspace_bytes(64, 16, 32, 8, 128, ops.PKV_BF16,
                                                        ops.PKV_BF16) == (
        _align(128 * 16 * 32 * 128 * 4) + _align(128 * 16 * 32 * 4) + lib.pkv_decode_plan_bytes(64, 128))
    assert lib.pkv_multi_query_balanced_workspace_bytes(64, 0, 32, 8, 128, ops.PKV_BF16,
                                                        ops.PKV_BF16) == 0
    assert ops.plan_info_offset(64) == 512 and ops.plan_info_offset(63) == 256


def test_decode_balanced_validation(lib):
    # What a call with these sizes uses (the workspace function bounds it from above).
    r = lib.pkv_decode_plan_slots(2, 8, 2, 128, ops.PKV_BF16, ops.PKV_BF16)
    assert r == 3072 // 2
    used = _align(r * 8 * 128 * 4) + _align(r * 8 * 4) + lib.pkv_decode_plan_bytes(2, r)
    need = lib.pkv_decode_workspace_bytes(2, 8, 128, 64, -1)
    assert need >= used
    assert _decode(lib, P=-1) == WORKSPACE                          # nothing launched
    assert _decode(lib, P=-1, ws=FAKE, wsb=used - 1) == WORKSPACE
    assert _decode(lib, P=-2, ws=FAKE, wsb=need) == INVALID
    assert _decode(lib, P=-1, d=96, ws=FAKE, wsb=need) == UNSUPPORTED
    assert _decode(lib, P=-1, ws=ctypes.c_void_p(0x10008), wsb=need) == INVALID
    assert _decode(lib, P=-1, mbps=1 << 28, ws=FAKE, wsb=need) == INVALID   # tokens overflow int32
    assert _step(lib, P=-1) == WORKSPACE
    assert _step(lib, P=-1, kn=None) == INVALID
    assert _decode(lib, P=-1, B=0, q=None) == OK


def test_decode_plan_validation(lib):
    f = lib.pkv_decode_plan
    need = lib.pkv_decode_plan_bytes(2, 384)
    assert f(FAKE, need, FAKE, 2, 1, 16, 4, None) == INVALID         # fewer slots than sequences
    assert f(FAKE, need, FAKE, 2, 384, 0, 4, None) == INVALID
    assert f(FAKE, need, FAKE, 2, 384, 16, 0, None) == INVALID
    assert f(FAKE, need, FAKE, 2, 384, 16, 1 << 28, None) == INVALID
    assert f(None, need, FAKE, 2, 384, 16, 4, None) == INVALID
    assert f(ctypes.c_void_p(0x10008), need, FAKE, 2, 384, 16, 4, None) == INVALID
    assert f(FAKE, need - 1, FAKE, 2, 384, 16, 4, None) == WORKSPACE
    assert f(FAKE, need, None, 2, 384, 16, 4, None) == INVALID
    assert f(FAKE, need, ctypes.c_void_p(0x10002), 2, 384, 16, 4, None) == INVALID
    assert f(FAKE, lib.pkv_decode_plan_bytes(0, 384), None, 0, 384, 16, 4, None) == OK
    g = lib.pkv_paged_decode_partials_planned
    args = [FAKE, FAKE, FAKE, need, 384, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 2, 8, 2, 128, 16,
            8, 4, 0.088, ops.PKV_BF16, ops.PKV_BF16, None]
    for i, bad in [(0, None), (1, None), (2, None), (2, ctypes.c_void_p(0x10008)), (4, 1),
                   (4, 0), (5, None), (13, 7), (15, 96), (16, 32), (19, float("nan")),
                   (21, ops.PKV_FP8_E4M3)]:
        a = list(args)
        a[i] = bad
        assert g(*a) in (INVALID, UNSUPPORTED), i
    a = list(args); a[3] = need - 1
    assert g(*a) == WORKSPACE                                     # plan buffer too small
    a = list(args); a[12] = 0; a[5] = None
    assert g(*a) == OK
    m = lib.pkv_merge_partials_planned
    margs = [FAKE, FAKE, FAKE, FAKE, 384, 2, 8, 128, ops.PKV_BF16, None]
    for i, bad in [(0, None), (3, None), (3, ctypes.c_void_p(0x10008)), (4, 1), (7, 96),
                   (8, ops.PKV_FP8_E4M3)]:
        a = list(margs)
        a[i] = bad
        assert m(*a) in (INVALID, UNSUPPORTED), i
    a = list(margs); a[5] = 0; a[0] = None
    assert m(*a) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros(4, 2, 16, 64)
    with pytest.raises(ValueError):
        ops.kv_append(t, t, t[:, :, 0], t[:, :, 0], torch.zeros(1, 1, dtype=torch.int32),
                      torch.zeros(1, dtype=torch.int32))
