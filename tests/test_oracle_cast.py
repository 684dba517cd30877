"""Pins of the oracle's fp32 -> bf16/fp16 casts: brute-force nearest value, torch, special values."""

import numpy as np
import torch

import oracle as O


def _decode(bits, exp_bits, man_bits):
    """Exact float64 value of every 16-bit pattern, decoded from the IEEE field definition."""
    bits = bits.astype(np.int64)
    bias = (1 << (exp_bits - 1)) - 1
    s = (bits >> 15) & 1
    e = (bits >> man_bits) & ((1 << exp_bits) - 1)
    m = bits & ((1 << man_bits) - 1)
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), 1 - bias - man_bits),
                   np.ldexp((m + (1 << man_bits)).astype(np.float64), e - bias - man_bits))
    mag = np.where(e == (1 << exp_bits) - 1, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def _nearest_even(x32, exp_bits, man_bits):
    """Round each fp32 value to the 16-bit format by search: nearest value, ties to even mantissa,
    at or beyond (max + half an ulp) to infinity. Returns bit patterns."""
    pats = np.arange(0, 1 << 15, dtype=np.int64)                 # non-negative patterns
    vals = _decode(pats, exp_bits, man_bits)
    fin = np.isfinite(vals)
    pats, vals = pats[fin], vals[fin]                            # increasing in both
    x = x32.astype(np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo, dhi = np.abs(a - vals[lo]), np.abs(vals[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (pats[hi] % 2 == 0))
    res = np.where(pick_hi, pats[hi], pats[lo])
    vmax = vals[-1]
    ulp_max = vals[-1] - vals[-2]
    inf_pat = ((1 << exp_bits) - 1) << man_bits
    res = np.where(a >= vmax + ulp_max / 2, inf_pat, res)
    res = np.where(np.signbit(x), res | 0x8000, res)
    return res.astype(np.uint16)


def _boundary_inputs(exp_bits, man_bits, rng):
    """fp32 inputs at and around every 16-bit value and every rounding midpoint, plus randoms."""
    pats = np.arange(0, 1 << 16, dtype=np.int64)
    vals = _decode(pats, exp_bits, man_bits)
    vals = vals[np.isfinite(vals)]
    v32 = vals.astype(np.float32)
    pos = np.sort(vals[vals >= 0])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)        # exact in fp32 for both formats
    cands = [v32, mids, -mids, np.nextafter(mids, np.float32(np.inf)),
             np.nextafter(mids, np.float32(-np.inf))]
    rnd = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    cands.append(rnd[np.isfinite(rnd)])
    return np.concatenate(cands).astype(np.float32)


def test_bf16_matches_nearest_even_search():
    rng = np.random.default_rng(11)
    x = _boundary_inputs(8, 7, rng)
    # every high half with the low halves that decide rounding
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    grid = (hi[:, None] | lows[None, :]).reshape(-1).view(np.float32)
    x = np.concatenate([x, grid[np.isfinite(grid)]])
    got = O.cast_bf16_rne(x)
    want = _nearest_even(x, 8, 7)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(x[i:i+1].view(np.uint32)[0])), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_fp16_matches_nearest_even_search():
    rng = np.random.default_rng(12)
    x = _boundary_inputs(5, 10, rng)
    x = np.concatenate([x, np.float32([65504, 65519.996, 65520, 70000, 2.0**-24, 2.0**-25,
                                        2.0**-25 * 1.0000001, 2.0**-26, -2.0**-25, 1e-30, -0.0])])
    got = O.cast_fp16_rne(x)
    want = _nearest_even(x, 5, 10)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_casts_agree_with_torch_cpu():
    rng = np.random.default_rng(13)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    t = torch.from_numpy(x.copy())
    tb = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    th = t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert (O.cast_bf16_rne(x) == tb).all()
    assert (O.cast_fp16_rne(x) == th).all()


def test_special_values():
    x = np.float32([0.0, -0.0, 1.0, -2.0, np.inf, -np.inf, 3.4e38, 1e-45])
    assert O.cast_bf16_rne(x).tolist() == [0x0000, 0x8000, 0x3F80, 0xC000, 0x7F80, 0xFF80, 0x7F80, 0x0000]
    assert O.cast_fp16_rne(x).tolist() == [0x0000, 0x8000, 0x3C00, 0xC000, 0x7C00, 0xFC00, 0x7C00, 0x0000]
    # ties: 1 + 2^-8 lies halfway between bf16 1.0 and 1+2^-7 -> even (1.0); 1 + 3*2^-8 -> up
    assert O.cast_bf16_rne(np.float32([1 + 2.0**-8, 1 + 3 * 2.0**-8])).tolist() == [0x3F80, 0x3F82]
    nan = O.cast_bf16_rne(np.float32([np.nan, -np.nan]))
    assert ((nan & 0x7F80) == 0x7F80).all() and ((nan & 0x7F) != 0).all()
    assert nan[1] & 0x8000


def test_widen_round_trips_exactly():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    wb = O.widen_bf16(b)
    ok = ~np.isnan(wb)
    assert (O.cast_bf16_rne(wb[ok]) == b[ok]).all()
    assert np.array_equal(wb[ok].astype(np.float64), _decode(b, 8, 7)[ok])
    wh = O.widen_fp16(b)
    ok = ~np.isnan(wh)
    assert np.array_equal(wh[ok].astype(np.float64), _decode(b, 5, 10)[ok])


def test_cast_slice_checker_catches_planted_mistakes():
    """The checker behind the exhaustive GPU cast test: silent on the oracle's own casts (any NaN
    payload allowed), loud on a wrong bit, a NaN turned into infinity, or a changed master."""
    from cast_check import check_cast_slice
    lo = 0x7F7FFF00                         # the top of the finite range, infinity and NaNs
    pats = np.arange(lo, lo + 4096, dtype=np.uint64).astype(np.uint32)
    x = pats.view(np.float32)
    good = {"bf16": O.cast_bf16_rne(x), "f16": O.cast_fp16_rne(x)}
    assert check_cast_slice(lo, good, pats.copy()) is None
    nan = (pats & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    quiet = {"bf16": np.uint16(0x0040), "f16": np.uint16(0x0200)}       # another NaN payload
    payload = {k: np.where(nan, v | quiet[k], v) for k, v in good.items()}
    assert any((payload[k] != good[k]).any() for k in good)
    assert check_cast_slice(lo, payload, pats.copy()) is None        # NaN payloads are free
    for dt in ("bf16", "f16"):
        bad = dict(good)
        bad[dt] = good[dt].copy()
        bad[dt][10] ^= 1                                              # a finite pattern's cast
        assert "casts to" in check_cast_slice(lo, bad, pats.copy())
        bad[dt] = good[dt].copy()
        bad[dt][np.argmax(nan)] = 0x7F80 if dt == "bf16" else 0x7C00   # NaN -> infinity
        assert "NaN" in check_cast_slice(lo, bad, pats.copy())
    p2 = pats.copy()
    p2[3] ^= 1
    assert check_cast_slice(lo, good, p2) == "non-NaN master changed"
