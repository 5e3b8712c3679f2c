"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  This is what makes the pins worth trusting: a dropped term,
a wrong index, a wrong sign or a transposed operand must fail at least one."""

import numpy as np
import pytest

import oracle.paged_attention as pa
from tests import oracle_pins as pins
from workloads import named_config


def _mut_gqa_modulo(monkeypatch):
    def attend(q, K, V, scale, return_weights=False):
        hq, hkv = q.shape[0], K.shape[0]
        out = np.empty((hq, V.shape[2]))
        for i in range(hq):
            h = i % hkv                      # strided grouping instead of i // g
            s = scale * (K[h] @ q[i])
            p = np.exp(s - s.max())
            out[i] = (p @ V[h]) / p.sum()
        return out
    monkeypatch.setattr(pa, "attend", attend)


def _mut_append_slot(monkeypatch):
    orig = pa.slot_of
    monkeypatch.setattr(pa, "slot_of", lambda row, pos, bs: orig(row, pos + 1, bs))


def _mut_no_scale(monkeypatch):
    orig = pa.attend
    monkeypatch.setattr(pa, "attend", lambda q, K, V, scale, return_weights=False:
                        orig(q, K, V, 1.0, return_weights))


def _mut_keep_tail(monkeypatch):
    def gather(pool, row, ctx, bs, dtype, scales=None):
        nb = -(-ctx // bs)
        ids = np.asarray(row[:nb], np.int64)
        blk = pa.to_float64(pool[ids], dtype)
        if scales is not None:
            blk = blk * np.asarray(scales, np.float64)[ids][:, :, None, None]
        return blk.transpose(1, 0, 2, 3).reshape(blk.shape[1], nb * bs, blk.shape[3])
    monkeypatch.setattr(pa, "gather_sequence", gather)


def _mut_block_order(monkeypatch):
    orig = pa.gather_sequence
    monkeypatch.setattr(pa, "gather_sequence",
                        lambda pool, row, ctx, bs, dtype, scales=None:
                        orig(pool, np.concatenate([row[:-(-ctx // bs)][::-1], row[-(-ctx // bs):]]),
                             ctx, bs, dtype, scales))


def _mut_v_from_k(monkeypatch):
    def attend(q, K, V, scale, return_weights=False):
        g = q.shape[0] // K.shape[0]
        out = np.empty((q.shape[0], V.shape[2]))
        for i in range(q.shape[0]):
            s = scale * (K[i // g] @ q[i])
            p = np.exp(s - s.max())
            out[i] = (p @ K[i // g]) / p.sum()          # wrong operand
        return out
    monkeypatch.setattr(pa, "attend", attend)


def _mut_no_max_shift_sign(monkeypatch):
    def attend(q, K, V, scale, return_weights=False):
        g = q.shape[0] // K.shape[0]
        out = np.empty((q.shape[0], V.shape[2]))
        for i in range(q.shape[0]):
            s = scale * (K[i // g] @ q[i])
            p = np.exp(-(s - s.max()))                 # wrong sign
            out[i] = (p @ V[i // g]) / p.sum()
        return out
    monkeypatch.setattr(pa, "attend", attend)


def _mut_merge_weights(monkeypatch):
    def merge(o, lse):
        o = np.asarray(o, np.float64)
        lse = np.asarray(lse, np.float64)
        w = np.where(np.isfinite(lse), 1.0, 0.0)       # dropped exp(lse - M) term
        return np.einsum("...p,...pd->...d", w, np.nan_to_num(o)) / np.maximum(w.sum(-1), 1)[..., None]
    monkeypatch.setattr(pa, "merge_partials", merge)


def _mut_e4m3_bias(monkeypatch):
    orig = pa.decode_e4m3fn
    monkeypatch.setattr(pa, "decode_e4m3fn", lambda c: orig(c) * 0.5)   # bias 8


def _mut_fp8_scale_transposed(monkeypatch):
    orig = pa.gather_sequence
    def gather(pool, row, ctx, bs, dtype, scales=None):
        if scales is not None:
            scales = np.ascontiguousarray(np.asarray(scales)[:, ::-1])   # head order reversed
        return orig(pool, row, ctx, bs, dtype, scales)
    monkeypatch.setattr(pa, "gather_sequence", gather)


def _mut_bf16_shift(monkeypatch):
    def dec(bits):
        u = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(15)
        return u.view(np.float32).astype(np.float64)
    monkeypatch.setattr(pa, "decode_bf16", dec)


def _mut_partition_overlap(monkeypatch):
    orig = pa.partition_partials
    monkeypatch.setattr(pa, "partition_partials",
                        lambda q, K, V, scale, P: orig(q, K[:, 1:], V[:, 1:], scale, P))


def _mut_visibility(monkeypatch):
    monkeypatch.setattr(pa, "visible_tokens", lambda ctx, t, j: ctx - t + j + 2)


def _mut_append_tokens_order(monkeypatch):
    orig = pa.kv_append_tokens
    def app(kp, vp, kn, vn, tab, ctx, qsl, bs, inplace=False):
        return orig(kp, vp, kn[::-1].copy(), vn[::-1].copy(), tab, ctx, qsl, bs, inplace)
    monkeypatch.setattr(pa, "kv_append_tokens", app)


def _caught(check):
    with np.errstate(all="ignore"):
        try:
            return check()
        except Exception:           # a crash is also a catch
            return True


PIN_SUITE = {
    "causal_mha": lambda: pins.pin_incremental_vs_causal(Hq=4, Hkv=4, T=20) > 1e-9,
    "causal_gqa": lambda: pins.pin_incremental_vs_causal(Hq=4, Hkv=2, T=20) > 1e-9,
    "library_cfg1": lambda: pins.pin_config_crosscheck(1) > 1e-9,
    "library_fp8": lambda: pins.pin_config_crosscheck(5, num_seqs=2, ctx=("uniform", 17, 60)) > 1e-9,
    "e4m3": lambda: pins.pin_e4m3_table() > 0,
    "bf16": lambda: pins.pin_bf16_table() > 0,
    "split_merge": lambda: pins.pin_split_merge(named_config(1), (16, 64)) > 1e-9,
    "closed_forms": lambda: pins.pin_closed_forms() > 1e-9,
    "chunked": lambda: pins.pin_chunked_vs_causal(schedules=[[6, 1, 1, 1, 1], [3, 3, 3, 1]],
                                                  Hkv=2) > 1e-9,
}


@pytest.mark.parametrize("mutant", [
    _mut_gqa_modulo, _mut_append_slot, _mut_no_scale, _mut_keep_tail, _mut_block_order,
    _mut_v_from_k, _mut_no_max_shift_sign, _mut_merge_weights, _mut_e4m3_bias,
    _mut_fp8_scale_transposed, _mut_bf16_shift, _mut_partition_overlap, _mut_visibility,
    _mut_append_tokens_order,
])
def test_planted_mistake_is_caught(monkeypatch, mutant):
    mutant(monkeypatch)
    caught = [name for name, check in PIN_SUITE.items() if _caught(check)]
    assert caught, f"{mutant.__name__} slipped past every pin"
