"""The host half of ZeRO-Offload on the CPU: zero_host_adam_step against the oracle, bit for bit
(the same fp32 operation order and round-to-nearest-even casts as the GPU kernel). No GPU needed."""

import numpy as np
import pytest

import oracle as O
import zero_partition_plan_amd as Z
from bitcmp import assert_bits_equal_nan
from workloads.extremes import EXTREME_CASES, mixed_state

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _case(rng, n, warm=True):
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32) if warm else np.zeros(n, np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32) if warm else np.zeros(n, np.float32)
    return master, g, m, v


@pytest.mark.parametrize("odt", ["bf16", "f16", None])
@pytest.mark.parametrize("mode", ["adamw", "l2"])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_host_step_matches_oracle(odt, mode, threads):
    n = 200_003
    rng = np.random.default_rng(hash((odt, mode, threads)) % 1000)
    master, g, m, v = _case(rng, n)
    hp = {**HP, "wd_mode": mode, "step": 7}
    out = np.full(n, 0x1234, np.uint16) if odt else None
    p2, m2, v2 = master.copy(), m.copy(), v.copy()
    Z.zero_host_adam_step(g, n, 0.5, p2, m2, v2, Z.adam_hparams(**hp), out=out,
                          out_dtype={"bf16": Z.ZERO_BF16, "f16": Z.ZERO_F16, None: Z.ZERO_BF16}[odt],
                          threads=threads)
    wp, wm, wv, wo = O.sharded_step([g], "f32", 0.5, master, m, v, O.AdamHParams(**hp), odt)
    assert np.array_equal(p2.view(np.uint32), wp.view(np.uint32))
    assert np.array_equal(m2.view(np.uint32), wm.view(np.uint32))
    assert np.array_equal(v2.view(np.uint32), wv.view(np.uint32))
    if odt:
        assert np.array_equal(out, wo)


def test_host_step_unaligned_and_ragged():
    rng = np.random.default_rng(5)
    for n in (1, 2, 63, 64, 65, 4099, 70_001):
        for off in (0, 1, 3):
            master, g, m, v = _case(rng, n + off)
            out = np.zeros(n + off, np.uint16)
            p2, m2, v2 = master.copy(), m.copy(), v.copy()
            Z.zero_host_adam_step(g[off:], n, 1.0, p2[off:], m2[off:], v2[off:], Z.adam_hparams(step=2, **HP),
                                  out=out[off:], threads=4)
            wp, wm, wv, wo = O.sharded_step([g[off:]], "f32", 1.0, master[off:], m[off:], v[off:],
                                            O.AdamHParams(step=2, **HP), "bf16")
            assert np.array_equal(p2[off:].view(np.uint32), wp.view(np.uint32)), (n, off)
            assert np.array_equal(out[off:], wo), (n, off)
            assert np.array_equal(p2[:off], master[:off]) and not out[:off].any()


def _edge_patterns(rng):
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x7FFF, 0x8000, 0x8001, 0xFFFF],
                    dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    # dense sweep over the binary16 subnormal / underflow region and the overflow boundary
    sub = np.arange(0x33000000 - 64, 0x38800000 + 64, 97, dtype=np.uint32)
    top = np.arange(0x477FE000 - 4096, 0x47800000 + 4096, dtype=np.uint32)
    rnd = rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    pats = np.concatenate([pats, sub, sub | 0x80000000, top, top | 0x80000000, rnd])
    x = pats.view(np.float32)
    return x[~np.isnan(x)].copy()


@pytest.mark.parametrize("odt,cast", [("bf16", O.cast_bf16_rne), ("f16", O.cast_fp16_rne)])
def test_host_casts_on_edge_patterns(odt, cast):
    """Zero gradient on zero state with wd = 0 leaves p unchanged, so the output is the cast of
    arbitrary fp32 patterns: ties, subnormals, the binary16 underflow and overflow boundaries."""
    x = _edge_patterns(np.random.default_rng(17))
    n = x.size
    z = np.zeros(n, np.float32)
    p, m, v, out = x.copy(), z.copy(), z.copy(), np.zeros(n, np.uint16)
    Z.zero_host_adam_step(z, n, 1.0, p, m, v, Z.adam_hparams(lr=1e-3, weight_decay=0.0, step=1), out=out,
                          out_dtype=Z.ZERO_BF16 if odt == "bf16" else Z.ZERO_F16, threads=8)
    assert np.array_equal(p.view(np.uint32), x.view(np.uint32))
    want = cast(x)
    bad = np.nonzero(out != want)[0]
    assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), hex(int(out[i])), hex(int(want[i]))) for i in bad[:5]]


def test_host_nan_cast_is_a_nan_of_the_same_sign():
    x = np.array([0x7FC00000, 0xFFC00001, 0x7F800001, 0xFFBFFFFF, 0x7FFFFFFF], np.uint32).view(np.float32)
    n = x.size
    z = np.zeros(n, np.float32)
    for odt, expo in ((Z.ZERO_BF16, 0x7F80), (Z.ZERO_F16, 0x7C00)):
        p, out = x.copy(), np.zeros(n, np.uint16)
        Z.zero_host_adam_step(z, n, 1.0, p, z.copy(), z.copy(), Z.adam_hparams(weight_decay=0.0), out=out,
                              out_dtype=odt, threads=1)
        assert ((out & expo) == expo).all() and (out & (expo ^ 0x7FFF)).all()     # NaN, quiet payload
        assert ((out >> 15) == (x.view(np.uint32) >> 31)).all()                   # sign kept
    # bf16 follows the oracle's rule exactly
    out = np.zeros(n, np.uint16)
    Z.zero_host_adam_step(z, n, 1.0, x.copy(), z.copy(), z.copy(), Z.adam_hparams(weight_decay=0.0), out=out,
                          out_dtype=Z.ZERO_BF16, threads=1)
    assert np.array_equal(out, O.cast_bf16_rne(x))


def test_host_step_errors():
    n = 16
    a = [np.zeros(n, np.float32) for _ in range(4)]
    with pytest.raises(Z.ZeroError):
        Z.zero_host_adam_step(a[0], n, 1.0, a[1], a[1], a[2], Z.adam_hparams())       # master is m
    with pytest.raises(Z.ZeroError):
        Z.zero_host_adam_step(a[0], n, 1.0, a[1], a[2], a[3], Z.adam_hparams(step=0))
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_host_adam_step(a[0], n, 1.0, a[1], a[2], a[3], Z.adam_hparams(), out=np.zeros(n, np.uint16),
                              out_dtype=Z.ZERO_F32)
    assert e.value.status == 3
    Z.zero_host_adam_step(None, 0, 1.0, None, None, None, Z.adam_hparams())              # n = 0 no-op


@pytest.mark.parametrize("case", range(len(EXTREME_CASES)))
@pytest.mark.parametrize("threads", [1, 4])
def test_host_step_ieee_special_cases(case, threads):
    """Operands over the whole binary32 range (subnormals, overflow, 0/0, inf/inf, signed zeros):
    every non-NaN result equals the oracle's bit for bit, and NaN results are NaN on both sides
    (operand order inside a vector loop may pick a different NaN's payload)."""
    regimes, gs, hpx = EXTREME_CASES[case]
    n = 70_001
    rng = np.random.default_rng(900 + case)
    g, p, m, v = mixed_state(rng, n, regimes)
    hp = {**HP, "step": 3, **hpx}
    for odt in ("bf16", "f16"):
        p2, m2, v2, out = p.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
        Z.zero_host_adam_step(g, n, gs, p2, m2, v2, Z.adam_hparams(**hp), out=out,
                              out_dtype={"bf16": Z.ZERO_BF16, "f16": Z.ZERO_F16}[odt], threads=threads)
        with np.errstate(all="ignore"):
            wp, wm, wv, wo = O.sharded_step([g], "f32", gs, p, m, v, O.AdamHParams(**hp), odt)
        for got, want, what in ((p2, wp, "master"), (m2, wm, "m"), (v2, wv, "v")):
            assert_bits_equal_nan(got.view(np.uint32), want.view(np.uint32), f"{what} ({odt})")
        assert_bits_equal_nan(out, wo, f"out {odt}", odt)


def _aligned(n, dtype, fill=0):
    """n elements of dtype whose first element sits on a 64-byte boundary."""
    item = np.dtype(dtype).itemsize
    raw = np.full(n + 64 // item, fill, dtype)
    k = (-raw.ctypes.data % 64) // item
    a = raw[k:k + n]
    assert a.ctypes.data % 64 == 0
    return a


@pytest.mark.parametrize("odt", ["bf16", "f16", None])
@pytest.mark.parametrize("mode", ["adamw", "l2"])
def test_host_step_array_phases(odt, mode):
    """Master, m, v, the gradient and the 16-bit output each start at their own offset within a
    32-byte line, so every form of the host loop runs: streamed state with a streamed or a plain
    16-bit store (scalar head and tail around the vector body), and the plain loop when m or v is
    out of master's phase. Bit for bit against the oracle, nothing written outside the arrays."""
    rng = np.random.default_rng(hash((odt, mode)) % 1000)
    hp = {**HP, "wd_mode": mode, "step": 3}
    for n in (1, 7, 8, 9, 100, 4099, 70_001):
        # (master, m, v, gradient, output) offsets in elements from 64-byte aligned bases: all on
        # the boundary; a 5-element head with the output still streamed after it; a 7-element head
        # leaving the output off its 16 bytes (plain 16-bit stores); v and then m out of master's
        # phase (the plain loop)
        for offs in ((0, 0, 0, 0, 0), (3, 3, 3, 5, 3), (1, 1, 1, 1, 7), (0, 0, 4, 0, 0), (5, 2, 5, 6, 1)):
            op, om, ov, og, oo = offs
            master, g, m, v = _case(rng, n)
            P = _aligned(n + 16, np.float32); P[op:op + n] = master
            M = _aligned(n + 16, np.float32); M[om:om + n] = m
            V = _aligned(n + 16, np.float32); V[ov:ov + n] = v
            G = _aligned(n + 16, np.float32); G[og:og + n] = g
            out = _aligned(n + 16, np.uint16, 0x5A5A)
            Z.zero_host_adam_step(G[og:og + n], n, 0.5, P[op:op + n], M[om:om + n], V[ov:ov + n],
                                  Z.adam_hparams(**hp), out=out[oo:oo + n] if odt else None,
                                  out_dtype={"bf16": Z.ZERO_BF16, "f16": Z.ZERO_F16, None: Z.ZERO_BF16}[odt],
                                  threads=3)
            wp, wm, wv, wo = O.sharded_step([g], "f32", 0.5, master, m, v, O.AdamHParams(**hp), odt)
            what = (n, offs)
            assert np.array_equal(P[op:op + n].view(np.uint32), wp.view(np.uint32)), what
            assert np.array_equal(M[om:om + n].view(np.uint32), wm.view(np.uint32)), what
            assert np.array_equal(V[ov:ov + n].view(np.uint32), wv.view(np.uint32)), what
            for arr, o in ((P, op), (M, om), (V, ov)):
                assert not arr[:o].any() and not arr[o + n:].any(), what
            if odt:
                assert np.array_equal(out[oo:oo + n], wo), what
            keep = np.ones(n + 16, bool)
            if odt:
                keep[oo:oo + n] = False
            assert (out[keep] == 0x5A5A).all(), what


@pytest.mark.parametrize("odt", ["bf16", "f16"])
def test_host_step_ignores_callers_flush_to_zero(odt):
    """A caller running with flush-to-zero and denormals-are-zero (torch.set_flush_denormal) gets
    the IEEE results all the same: the host update sets IEEE mode in every thread it runs on, and
    the caller's mode is back afterwards. The state is put where the update and the casts meet
    subnormals: fp32 subnormal parameters and moments, and parameters in binary16's subnormal range."""
    import torch
    rng = np.random.default_rng(23)
    n = 70_001
    sub32 = (rng.integers(1, 1 << 23, n, dtype=np.uint64).astype(np.uint32)
             | (rng.integers(0, 2, n, dtype=np.uint64).astype(np.uint32) << 31)).view(np.float32)
    sub16 = (rng.standard_normal(n) * 3e-6).astype(np.float32)        # binary16 subnormals
    master = np.where(rng.random(n) < 0.5, sub32, sub16).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-30).astype(np.float32)
    m = sub32[::-1].copy()
    v = np.abs(sub32)
    hp = {**HP, "step": 2}
    wp, wm, wv, wo = O.sharded_step([g], "f32", 1.0, master, m, v, O.AdamHParams(**hp), odt)
    if not torch.set_flush_denormal(True):
        pytest.skip("this CPU has no flush-to-zero control")
    try:
        p2, m2, v2, out = master.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
        Z.zero_host_adam_step(g, n, 1.0, p2, m2, v2, Z.adam_hparams(**hp), out=out,
                              out_dtype=Z.ZERO_BF16 if odt == "bf16" else Z.ZERO_F16, threads=4)
        flushed = float(np.float32(1e-40) * np.float32(1.0)) == 0.0       # the caller's mode is back
    finally:
        torch.set_flush_denormal(False)
    assert flushed
    assert np.array_equal(p2.view(np.uint32), wp.view(np.uint32))
    assert np.array_equal(m2.view(np.uint32), wm.view(np.uint32))
    assert np.array_equal(v2.view(np.uint32), wv.view(np.uint32))
    assert np.array_equal(out, wo)


def test_host_arithmetic_ignores_callers_rounding_mode():
    """Under each directed rounding mode set by the caller (C fesetround), the derived step
    constants and the host update equal their round-to-nearest results bit for bit, and the caller's
    mode is back afterwards."""
    import ctypes
    libc = ctypes.CDLL(None)
    modes = {"downward": 0x400, "upward": 0x800, "toward zero": 0xC00}       # x86 <fenv.h> values
    rng = np.random.default_rng(29)
    n = 20_003
    master, g, m, v = _case(rng, n)
    hp = Z.adam_hparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=777)
    want_k = Z.zero_adam_derive(hp)
    want = [a.copy() for a in (master, m, v)] + [np.zeros(n, np.uint16)]
    Z.zero_host_adam_step(g, n, 0.25, *want[:3], hp, out=want[3], threads=3)
    for name, mode in modes.items():
        got = [a.copy() for a in (master, m, v)] + [np.zeros(n, np.uint16)]
        assert libc.fesetround(mode) == 0
        try:
            k = Z.zero_adam_derive(hp)
            Z.zero_host_adam_step(g, n, 0.25, *got[:3], hp, out=got[3], threads=3)
            back = libc.fegetround()
        finally:
            libc.fesetround(0)
        assert back == mode, name
        assert bytes(k) == bytes(want_k), name
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), name
