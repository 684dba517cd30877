"""Checks that pin the oracle's Adam/AdamW update to facts outside itself.

Each check takes the update and scalar functions as arguments (defaulting to the oracle's) so the
mutation tests can run the same checks against deliberately wrong copies and see them fail.

Pins used:
  * closed form under a constant gradient g from m = v = 0: m_t = (1-b1^t) g, v_t = (1-b2^t) g^2,
    so the bias-corrected moments are g and g^2 and every step moves p by lr*g/(|g| + eps); with
    AdamW decay d = 1 - lr*wd first, p_t = d^t p_0 - lr*u*(1-d^t)/(1-d), u = g/(|g| + eps);
  * a zero gradient on zero state leaves p unchanged (Adam) or multiplies it by d (AdamW), so
    padding stays inert;
  * with eps = 0, scaling g by 2^k scales m by 2^k and v by 2^(2k) exactly and leaves p bit-equal;
  * torch.optim.Adam / AdamW on the CPU (a library implementation with its own operation order).
"""

from __future__ import annotations


import numpy as np
import torch

import oracle as O


def _run_steps(p0, g_seq, hp_base, steps, update_fn, scalars_fn):
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    hist = []
    for t in range(1, steps + 1):
        hp = O.AdamHParams(**{**hp_base.__dict__, "step": t})
        g = g_seq(t)
        p, m, v = update_fn(p, m, v, g, scalars_fn(hp), hp.wd_mode)
        hist.append((p.copy(), m.copy(), v.copy()))
    return hist


def check_constant_grad_closed_form(update_fn=O.adam_update, scalars_fn=O.adam_scalars,
                                    steps=6, wd=0.0, seed=0):
    rng = np.random.default_rng(seed)
    n = 20000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[:8] = [1e-9, -1e-9, 1e-3, -5e-2, 3e-7, 0.5, -2.0, 1e-6]    # |g| near, below and above eps
    hp = O.AdamHParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, wd_mode="adamw")
    hist = _run_steps(p0, lambda t: g, hp, steps, update_fn, scalars_fn)
    g64, p64 = g.astype(np.float64), p0.astype(np.float64)
    u = g64 / (np.abs(g64) + hp.eps)
    d = 1.0 - hp.lr * wd
    for t, (p, m, v) in enumerate(hist, start=1):
        m_ref = (1.0 - hp.beta1 ** t) * g64
        v_ref = (1.0 - hp.beta2 ** t) * g64 * g64
        np.testing.assert_allclose(m, m_ref, rtol=4 * t * 2.0 ** -24, atol=0)
        np.testing.assert_allclose(v, v_ref, rtol=6 * t * 2.0 ** -24, atol=0)
        if wd == 0.0:
            p_ref = p64 - t * hp.lr * u
        else:
            p_ref = d ** t * p64 - hp.lr * u * (1.0 - d ** t) / (1.0 - d)
        tol = t * (2.0 ** -23 * np.abs(p_ref) + 2.0 ** -20 * hp.lr)
        err = np.abs(p.astype(np.float64) - p_ref)
        assert (err <= tol).all(), f"step {t}: max err {err.max():.3e} vs tol {tol[np.argmax(err)]:.3e}"


def check_l2_first_step(update_fn=O.adam_update, scalars_fn=O.adam_scalars, seed=1):
    """Adam with L2 decay, first step from zero state: g' = g + wd*p, p1 = p0 - lr*g'/(|g'|+eps)."""
    rng = np.random.default_rng(seed)
    n = 20000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    hp = O.AdamHParams(lr=1e-3, weight_decay=0.05, wd_mode="l2", step=1)
    p, m, v = update_fn(p0, np.zeros_like(p0), np.zeros_like(p0), g, scalars_fn(hp), "l2")
    gp = g.astype(np.float64) + 0.05 * p0.astype(np.float64)
    p_ref = p0.astype(np.float64) - hp.lr * gp / (np.abs(gp) + hp.eps)
    # g' is one fp32 sum: its error is bounded by the size of its terms, not of the result
    m_tol = 0.1 * 2.0 ** -22 * (np.abs(g) + 0.05 * np.abs(p0)).astype(np.float64)
    assert (np.abs(m - 0.1 * gp) <= m_tol).all()
    # first-order propagation of that error through lr*g'/(|g'| + eps), steep where |g'| ~ eps
    dg = 2.0 ** -23 * (np.abs(g) + 0.05 * np.abs(p0)).astype(np.float64)
    cond = hp.lr * hp.eps * dg / (np.abs(gp) + hp.eps) ** 2
    tol = 2.0 ** -23 * np.abs(p_ref) + 2.0 ** -18 * hp.lr + 2 * cond
    assert (np.abs(p - p_ref) <= tol).all()


def check_zero_grad_inert(update_fn=O.adam_update, scalars_fn=O.adam_scalars):
    rng = np.random.default_rng(2)
    p0 = (rng.standard_normal(4096) * 0.02).astype(np.float32)
    z = np.zeros_like(p0)
    for wd, mode in ((0.0, "adamw"), (0.1, "adamw"), (0.0, "l2")):
        for t in (1, 7):
            hp = O.AdamHParams(weight_decay=wd, wd_mode=mode, step=t)
            p, m, v = update_fn(p0, z, z, z, scalars_fn(hp), mode)
            assert not m.any() and not v.any()
            want = p0 * np.float32(1.0 - hp.lr * wd) if mode == "adamw" else p0
            assert np.array_equal(p, want)


def check_scale_invariance(update_fn=O.adam_update, scalars_fn=O.adam_scalars, k=7):
    rng = np.random.default_rng(3)
    n = 8192
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(3)]
    hp = O.AdamHParams(eps=0.0, weight_decay=0.01)
    s = np.float32(2.0 ** k)
    a = _run_steps(p0, lambda t: gs[t - 1], hp, 3, update_fn, scalars_fn)
    b = _run_steps(p0, lambda t: gs[t - 1] * s, hp, 3, update_fn, scalars_fn)
    for (pa, ma, va), (pb, mb, vb) in zip(a, b):
        assert np.array_equal(pa, pb)
        assert np.array_equal(ma * s, mb)
        assert np.array_equal(va * s * s, vb)


def check_against_torch(update_fn=O.adam_update, scalars_fn=O.adam_scalars, steps=3):
    """torch.optim.Adam/AdamW (fp32 CPU, single-tensor path) within 1e-6 relative.

    The gradients keep one sign per element and stay above wd*|p|, so neither m nor the L2 sum
    cancels; p may still cross zero, so its floor is a few ulps of its starting size.
    """
    rng = np.random.default_rng(4)
    n = 50000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    gs = [(sign * (1e-3 + 1e-3 * np.abs(rng.standard_normal(n)))).astype(np.float32)
          for _ in range(steps)]
    cases = [("adam", 0.0, "adamw"), ("adamw", 0.01, "adamw"), ("adam", 0.01, "l2")]
    for opt_name, wd, mode in cases:
        tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
        cls = torch.optim.AdamW if opt_name == "adamw" else torch.optim.Adam
        opt = cls([tp], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd, foreach=False)
        p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
        for t in range(1, steps + 1):
            tp.grad = torch.from_numpy(gs[t - 1].copy())
            opt.step()
            hp = O.AdamHParams(weight_decay=wd, wd_mode=mode, step=t)
            p, m, v = update_fn(p, m, v, gs[t - 1], scalars_fn(hp), mode)
        st = opt.state[tp]
        p_floor = steps * 2.0 ** -22 * (np.abs(p0) + steps * 1e-3)
        assert (np.abs(p - tp.detach().numpy()) <= 1e-6 * np.abs(tp.detach().numpy()) + p_floor).all()
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-6, atol=0)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-6, atol=0)


ALL_CHECKS = {
    "constant_grad_adam": lambda u, s: check_constant_grad_closed_form(u, s, wd=0.0),
    "constant_grad_adamw": lambda u, s: check_constant_grad_closed_form(u, s, wd=0.1),
    "l2_first_step": check_l2_first_step,
    "zero_grad_inert": check_zero_grad_inert,
    "scale_invariance": check_scale_invariance,
    "torch_optim": check_against_torch,
}
