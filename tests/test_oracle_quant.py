"""Pins of the fp8 quantise-on-append oracle (oracle/kv_quant.py), against
what the format and the arithmetic fix: every code round-trips, ties go to
the even code, torch's float8 cast agrees wherever it does not overflow,
saturation, and the append's results checked through properties computed
independently of the oracle's own steps (error within half a quantum, the
scale a closed form of the new rows' maximum, untouched slots bit-identical).
A last test plants mistakes in the oracle and checks that a pin catches each."""

import numpy as np
import pytest
import torch

import oracle.kv_quant as kq
from oracle.paged_attention import decode_e4m3fn
from workloads.fp8_append import fp8_append_state

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


# --- the encoder ----------------------------------------------------------------

def pin_roundtrip():
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_e4m3fn(codes).astype(np.float32)
    finite = np.isfinite(vals)
    enc = kq.encode_e4m3fn(vals)
    return bool(np.array_equal(enc[finite], codes[finite]) and np.all(enc[~finite] == 0x7F))


def pin_ties():
    """Midpoints of neighbouring codes go to the even code; a hair off goes to
    the nearer one.  Both signs."""
    ok = True
    for c in range(0, 0x7E):
        lo, hi = float(decode_e4m3fn(np.uint8(c))), float(decode_e4m3fn(np.uint8(c + 1)))
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2           # exact in float32
        even = c if c % 2 == 0 else c + 1
        eps = (hi - lo) / 64
        for sgn, bit in ((1, 0), (-1, 0x80)):
            ok &= int(kq.encode_e4m3fn(sgn * mid)) == (even | bit) or (c == 0 and sgn < 0 and
                                                                       int(kq.encode_e4m3fn(sgn * mid)) == 0x80)
            ok &= int(kq.encode_e4m3fn(np.float32(sgn * (mid - eps)))) == (c | bit) or c == 0
            ok &= int(kq.encode_e4m3fn(np.float32(sgn * (mid + eps)))) == ((c + 1) | bit)
    return bool(ok)


def pin_torch_in_range(n=20000, seed=0):
    """torch's float8_e4m3fn cast rounds to nearest even; it agrees wherever it
    does not overflow (|x| < 464)."""
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.uniform(-463.9, 463.9, n),
        rng.standard_normal(n) * 3,
        rng.uniform(-2.0 ** -5, 2.0 ** -5, n),        # the subnormal range and its edge
        np.ldexp(rng.integers(1, 2 ** 12, n), rng.integers(-20, -2, n)) * rng.choice([-1, 1], n),
    ]).astype(np.float32)
    x = x[np.abs(x) < 464]
    return bool(np.array_equal(kq.encode_e4m3fn(x), torch_e4m3(x)))


def pin_saturation():
    big = np.array([448, 449, 463.99, 464, 465, 1e6, 3.4e38, np.inf], np.float32)
    return bool(np.all(kq.encode_e4m3fn(big) == 0x7E) and np.all(kq.encode_e4m3fn(-big) == 0xFE)
                and int(kq.encode_e4m3fn(np.float32(np.nan))) == 0x7F)


def test_encoder_roundtrip():
    assert pin_roundtrip()


def test_encoder_ties_to_even():
    assert pin_ties()


def test_encoder_matches_torch_in_range():
    assert pin_torch_in_range()


def test_encoder_saturates():
    assert pin_saturation()


# --- the append ------------------------------------------------------------------

def _state(seed=0, B=5, hkv=3, D=64, t=None):
    return fp8_append_state(seed=seed, num_seqs=B, num_kv_heads=hkv, head_dim=D, new_tokens=t)


def _placed(st, bs=16):
    """(row, phys, slot) of every placed new row, from the addressing alone."""
    out = []
    B = len(st["context_lens"])
    for b in range(B):
        ctx = int(st["context_lens"][b])
        qsl = st["query_start_loc"]
        q0, q1 = (b, b + 1) if qsl is None else (int(qsl[b]), int(qsl[b + 1]))
        for j in range(q1 - q0):
            pos = ctx - (q1 - q0) + j
            if pos >= 0:
                out.append((q0 + j, int(st["block_tables"][b, pos // bs]), pos % bs, b))
    return out


def _half_quantum(real_over_scale):
    """Half the e4m3 spacing at |y| (y = value / scale), in units of y, plus
    the float32 rounding of the quotient (and of a product before it), which
    may move y onto a midpoint."""
    a = np.abs(real_over_scale)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 3) / 2 + a * 2.0 ** -22


def _append(st, mode):
    return kq.kv_append_quant(st["k_pool"], st["v_pool"], st["k_scales"], st["v_scales"],
                              st["k_new"], st["v_new"], st["block_tables"], st["context_lens"], 16,
                              mode, query_start_loc=st["query_start_loc"])


def pin_fixed(st):
    kp, vp, ks, vs = _append(st, kq.SCALE_FIXED)
    placed = _placed(st)
    touched = np.zeros(st["k_pool"].shape[:3], bool)
    for pool, scales, new in ((kp, ks, st["k_new"]), (vp, vs, st["v_new"])):
        for r, phys, slot, _ in placed:
            for h in range(pool.shape[1]):
                s = np.float64(scales[phys, h])
                y = new[r, h] / s
                got = decode_e4m3fn(pool[phys, h, slot])
                inside = np.abs(y) <= 448
                if not np.all(np.abs(got[inside] - y[inside]) <= _half_quantum(y[inside]) * 1.0000001):
                    return False
                if not np.all(np.abs(got[~inside]) == 448):
                    return False
                touched[phys, h, slot] = True
    untouched = ~touched
    return bool(np.array_equal(ks, st["k_scales"]) and np.array_equal(vs, st["v_scales"]) and
                np.array_equal(kp[untouched], st["k_pool"][untouched]) and
                np.array_equal(vp[untouched], st["v_pool"][untouched]))


def pin_running(st):
    kp, vp, ks, vs = _append(st, kq.SCALE_RUNNING_AMAX)
    placed = _placed(st)
    groups = {}
    for r, phys, slot, b in placed:
        groups.setdefault((b, phys), []).append((r, slot))
    touched = np.zeros(st["k_pool"].shape[:3], bool)
    ok = True
    for pool0, s0, pool, scales, new in ((st["k_pool"], st["k_scales"], kp, ks, st["k_new"]),
                                         (st["v_pool"], st["v_scales"], vp, vs, st["v_new"])):
        for (b, phys), items in groups.items():
            first = min(sl for _, sl in items)
            for h in range(pool.shape[1]):
                vals = np.stack([new[r, h] for r, _ in items])
                amax = np.float32(np.max(np.abs(vals)))
                old = np.float32(s0[phys, h]) if first > 0 else np.float32(0)
                expect = max(old, np.float32(amax / np.float32(448)))
                ok &= scales[phys, h] == expect
                s = np.float64(scales[phys, h])
                for r, slot in items:
                    y = new[r, h] / s
                    got = decode_e4m3fn(pool[phys, h, slot])
                    ok &= bool(np.all(np.abs(y) <= 448 * (1 + 1e-7)))
                    ok &= bool(np.all(np.abs(got - y) <= _half_quantum(y) * 1.0000001))
                    touched[phys, h, slot] = True
                if first > 0:
                    prev = decode_e4m3fn(pool0[phys, h, :first]) * np.float64(old)
                    now = decode_e4m3fn(pool[phys, h, :first]) * s
                    if expect == old:
                        ok &= bool(np.array_equal(pool[phys, h, :first], pool0[phys, h, :first]))
                    else:
                        ok &= bool(np.all(np.abs(now - prev) <= _half_quantum(prev / s) * s * 1.000001))
                    touched[phys, h, :first] = True
    untouched = ~touched
    ok &= bool(np.array_equal(kp[untouched], st["k_pool"][untouched]))
    ok &= bool(np.array_equal(vp[untouched], st["v_pool"][untouched]))
    return bool(ok)


@pytest.mark.parametrize("t", [None, 1, 3, 20])
def test_fixed_scale_append(t):
    assert pin_fixed(_state(seed=1, t=t))


@pytest.mark.parametrize("t", [None, 1, 3, 20])
def test_running_amax_append(t):
    st = _state(seed=2, t=t)
    st["k_scales"][::2] *= np.float32(0.25)              # half the slices must grow
    assert pin_running(st)


def test_running_scale_grows_and_requantises():
    """A slice whose scale is too small for the new row: the scale becomes
    amax/448 and the earlier rows' real values move by at most half a quantum."""
    st = _state(seed=3, B=1, hkv=1, D=64)
    st["context_lens"][:] = 9                            # 8 earlier rows, new row at slot 8
    st["k_scales"][:] = np.float32(1e-3)
    st["k_new"][0, 0, 5] = 100.0
    kp, _, ks, _ = _append(st, kq.SCALE_RUNNING_AMAX)
    phys = int(st["block_tables"][0, 0])
    assert ks[phys, 0] == np.float32(np.float32(100.0) / np.float32(448))
    assert kp[phys, 0, 8, 5] == 0x7E                     # the max maps to 448 exactly
    assert not np.array_equal(kp[phys, 0, :8], st["k_pool"][phys, 0, :8])
    assert pin_running(st)


def test_fresh_block_ignores_old_scale():
    """A new row at slot 0 starts a block: the stale scale is not kept."""
    st = _state(seed=4, B=1, hkv=1, D=64)
    st["context_lens"][:] = 17                           # position 16: slot 0 of block 1
    st["block_tables"][0, 1] = st["block_tables"][0, 1] if st["block_tables"][0, 1] >= 0 else 0
    phys = int(st["block_tables"][0, 1])
    st["k_scales"][phys, 0] = np.float32(1e3)            # a huge stale scale
    _, _, ks, _ = _append(st, kq.SCALE_RUNNING_AMAX)
    amax = np.float32(np.abs(st["k_new"][0, 0]).max())
    assert ks[phys, 0] == np.float32(amax / np.float32(448))


def test_zero_rows_give_zero_scale():
    st = _state(seed=5, B=1, hkv=1, D=64)
    st["context_lens"][:] = 1
    st["k_new"][:] = 0.0
    kp, _, ks, _ = _append(st, kq.SCALE_RUNNING_AMAX)
    phys = int(st["block_tables"][0, 0])
    assert ks[phys, 0] == 0 and np.all(kp[phys, 0, 0] == 0)


# --- planted mistakes ----------------------------------------------------------------

def _mut_truncate(mp):
    mp.setattr(kq, "_round_half_even", lambda y: int(np.floor(y)))


def _mut_ties_away(mp):
    mp.setattr(kq, "_round_half_even", lambda y: int(np.floor(y + 0.5)))


def _mut_no_saturation(mp):
    orig = kq._encode_one
    mp.setattr(kq, "_encode_one", lambda v: 0x7F if abs(v) >= 464 else orig(v))


def _mut_bias8(mp):
    orig = kq._encode_one

    def enc(v):
        c = orig(v)
        e = (c >> 3) & 0xF
        return c if e in (0, 15) else (c & 0x87) | ((e + 1) << 3)
    mp.setattr(kq, "_encode_one", enc)


def _mut_no_requant(mp):
    orig = kq._append_slice

    def app(pool, scales, new, phys, h, items, n_old, mode):
        keep = pool[phys, h, :n_old].copy()
        orig(pool, scales, new, phys, h, items, n_old, mode)
        pool[phys, h, :n_old] = keep
    mp.setattr(kq, "_append_slice", app)


def _mut_keep_stale_scale(mp):
    orig = kq._append_slice
    mp.setattr(kq, "_append_slice", lambda pool, scales, new, phys, h, items, n_old, mode:
               orig(pool, scales, new, phys, h, items, max(n_old, 1) if mode else n_old, mode))


def _mut_scale_from_first_row(mp):
    orig = kq._append_slice
    mp.setattr(kq, "_append_slice", lambda pool, scales, new, phys, h, items, n_old, mode:
               orig(pool, scales, new, phys, h, items[:1], n_old, mode) or
               [orig(pool, scales, new, phys, h, [it], it[1], kq.SCALE_FIXED) for it in items[1:]])


def _mut_wrong_slot(mp):
    orig = kq._positions
    mp.setattr(kq, "_positions", lambda c, q, b, m, bs: [(r, p - 1) for r, p in orig(c, q, b, m, bs)
                                                         if p >= 1])


def _mut_scale_multiply(mp):
    mp.setattr(kq, "quantize", lambda x, s: kq.encode_e4m3fn(np.asarray(x, np.float32) *
                                                             np.float32(s)))


def _running_cases():
    st = _state(seed=2, t=3)
    st["k_scales"][::2] *= np.float32(0.25)
    return st


QUANT_PINS = {
    "roundtrip": pin_roundtrip,
    "ties": pin_ties,
    "torch": lambda: pin_torch_in_range(n=3000),
    "saturation": pin_saturation,
    "fixed": lambda: pin_fixed(_state(seed=1, t=3)),
    "running": lambda: pin_running(_running_cases()),
    "fresh": lambda: _fresh_ok(),
}


def _fresh_ok():
    try:
        test_fresh_block_ignores_old_scale()
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("mutant", [_mut_truncate, _mut_ties_away, _mut_no_saturation, _mut_bias8,
                                    _mut_no_requant, _mut_keep_stale_scale,
                                    _mut_scale_from_first_row, _mut_wrong_slot,
                                    _mut_scale_multiply])
def test_planted_quant_mistake_is_caught(monkeypatch, mutant):
    mutant(monkeypatch)
    failed = []
    for name, pin in QUANT_PINS.items():
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"{mutant.__name__} slipped past every pin"
