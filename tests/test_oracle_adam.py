"""Pins of the oracle's Adam / AdamW update (CPU only).

Checked against Adam's closed forms (first step, constant gradient,
decay only, the moment recurrences summed in float64), against
torch.optim.AdamW / torch.optim.Adam in float64 (an independent library
implementation of the textbook update), and against the skip rule.
"""
import numpy as np
import pytest
import torch

import oracle

LR, B1, B2, EPS, WD = 1e-3, 0.9, 0.999, 1e-8, 0.01


def _f16(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _zeros(n):
    return np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)


def test_first_step_is_lr_times_sign():
    # t = 1, wd = 0, m = v = 0, p = 0:  p1 = -lr * g / (|g| + eps)  ->  -lr * sign(g)
    g = np.array([1.0, -1.0, 3e-3, -7.5e-4, 0.25, -0.125, 2.0e-2, -6.0], np.float32)
    h = _f16(g)
    gf = h.view(np.float16).astype(np.float64)
    for eps in (1e-8, 1e-30):
        p, m, v = _zeros(g.size)
        assert oracle.adam_step(1, 1.0, h, "f16", p, m, v, LR, B1, B2, eps, 0.0) == 0
        closed = -LR * gf / (np.abs(gf) + eps)
        assert np.allclose(p, closed, rtol=1e-6, atol=0)
        if eps == 1e-30:
            assert np.allclose(p, -LR * np.sign(gf), rtol=1e-6, atol=0)
        # the moments after one step
        assert np.allclose(m, (1 - B1) * gf, rtol=1e-6, atol=0)
        assert np.allclose(v, (1 - B2) * gf * gf, rtol=1e-6, atol=0)


def test_constant_gradient_gives_the_same_step_every_time():
    # with g constant, mhat = g and vhat = g^2 exactly, so every step moves by
    # -lr * g / (|g| + eps)
    g = np.array([0.5, -0.25, 1e-2, -3e-3, 1.0, -2.0], np.float32)
    h = _f16(g)
    gf = h.view(np.float16).astype(np.float64)
    p, m, v = _zeros(g.size)
    prev = p.astype(np.float64)
    step = -LR * gf / (np.abs(gf) + EPS)
    for t in range(1, 51):
        oracle.adam_step(t, 1.0, h, "f16", p, m, v, LR, B1, B2, EPS, 0.0)
        cur = p.astype(np.float64)
        assert np.allclose(cur - prev, step, rtol=2e-5, atol=0), t
        prev = cur


def test_zero_gradient_only_decays():
    # g = 0 and m = v = 0: u = 0 / eps = 0, so AdamW gives p_t = p_0 (1 - lr wd)^t
    p0 = np.array([1.0, -0.5, 3.0, 1e-3, -7.0], np.float32)
    p, m, v = p0.copy(), *_zeros(p0.size)[1:]
    h = np.zeros(p0.size, np.uint16)
    for t in range(1, 11):
        oracle.adam_step(t, 1.0, h, "f16", p, m, v, LR, B1, B2, EPS, WD)
        assert np.allclose(p, p0.astype(np.float64) * (1 - LR * WD) ** t, rtol=1e-6, atol=0)
    assert not m.any() and not v.any()
    # Adam with an L2 term instead: the first step sees g = wd * p0 and moves
    # by -lr * g / (|g| + eps)
    p = p0.copy()
    m[:] = 0
    v[:] = 0
    oracle.adam_step(1, 1.0, h, "f16", p, m, v, LR, B1, B2, EPS, WD, adamw=False)
    g = WD * p0.astype(np.float64)
    closed = p0 - LR * g / (np.abs(g) + EPS)
    assert np.all(np.abs(p - closed) <= 2e-7 * np.abs(p0) + 1e-12)


@pytest.mark.parametrize("n", [4, 9, 16])
def test_moment_recurrences_match_float64_sums(n):
    rng = np.random.default_rng(n)
    T = 12
    gs = [_f16(rng.normal(0, 1, n)) for _ in range(T)]
    p, m, v = _zeros(n)
    for t in range(1, T + 1):
        oracle.adam_step(t, 1.0, gs[t - 1], "f16", p, m, v, LR, B1, B2, EPS, 0.0)
    gf = [g.view(np.float16).astype(np.float64) for g in gs]
    m_ref = (1 - B1) * sum(B1 ** (T - k) * gf[k - 1] for k in range(1, T + 1))
    v_ref = (1 - B2) * sum(B2 ** (T - k) * gf[k - 1] ** 2 for k in range(1, T + 1))
    scale_m = (1 - B1) * sum(B1 ** (T - k) * np.abs(gf[k - 1]) for k in range(1, T + 1))
    assert np.all(np.abs(m - m_ref) <= 1e-6 * scale_m)
    assert np.allclose(v, v_ref, rtol=1e-6, atol=0)


def _torch_run(cls, p0, grads, scale, wd, steps):
    w = torch.nn.Parameter(torch.from_numpy(p0.astype(np.float64)))
    opt = cls([w], lr=LR, betas=(B1, B2), eps=EPS, weight_decay=wd, foreach=False)
    for t in range(steps):
        w.grad = torch.from_numpy(grads[t].astype(np.float64) / scale)
        opt.step()
    st = opt.state[w]
    return w.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("adamw", [True, False])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_matches_torch_optim_in_float64(adamw, dt):
    rng = np.random.default_rng(7)
    n, steps, scale = 4096, 10, (1024.0 if dt == "f16" else 1.0)
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    raw = [(rng.normal(0, 1e-3, n) * scale).astype(np.float32) for _ in range(steps)]
    if dt == "f16":
        hs = [r.astype(np.float16).view(np.uint16) for r in raw]
    elif dt == "bf16":
        hs = [torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
              for r in raw]
    else:
        hs = [r.view(np.uint32) for r in raw]
    gvals = [(r.astype(np.float64) if dt == "f32" else
              oracle.half_to_float(h, dt).astype(np.float64)) for r, h in zip(raw, hs)]
    p, m, v = p0.copy(), *_zeros(n)[1:]
    for t in range(1, steps + 1):
        assert oracle.adam_step(t, scale, hs[t - 1], dt, p, m, v, LR, B1, B2, EPS, WD, adamw) == 0
    cls = torch.optim.AdamW if adamw else torch.optim.Adam
    tp, tm, tv = _torch_run(cls, p0, gvals, scale, WD, steps)
    # fp32 state vs the float64 library: a few fp32 roundings per step
    assert np.max(np.abs(p - tp) / np.maximum(np.abs(tp), 1e-3)) < 2e-6
    assert np.max(np.abs(m - tm)) < 2e-6 * np.max(np.abs(tm))
    assert np.max(np.abs(v - tv) / tv) < 2e-6


def test_unscale_is_exact_for_power_of_two_scales():
    # grads scaled by 2^10 then unscaled equal the unscaled grads bit for bit
    rng = np.random.default_rng(3)
    base = rng.normal(0, 1.0, 512).astype(np.float32).astype(np.float16)
    mag = np.abs(base.astype(np.float32))
    base = base[(mag >= 2.0 ** -14) & (mag < 32)]       # normal, and x * 1024 stays finite
    assert base.size > 400
    h1 = base.view(np.uint16)
    h2 = (base.astype(np.float32) * 1024).astype(np.float16).view(np.uint16)
    a = [x.copy() for x in (np.full(base.size, 0.1, np.float32), *_zeros(base.size)[1:])]
    b = [x.copy() for x in a]
    oracle.adam_step(3, 1.0, h1, "f16", *a)
    oracle.adam_step(3, 1024.0, h2, "f16", *b)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    # and a scale that is not undone changes the result
    c = [np.full(base.size, 0.1, np.float32), *_zeros(base.size)[1:]]
    oracle.adam_step(3, 1.0, h2, "f16", *c)
    assert not np.array_equal(c[1], a[1])


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00, 0x7D01])
def test_overflow_step_changes_nothing(bad):
    rng = np.random.default_rng(1)
    n = 300
    h = _f16(rng.normal(0, 1, n))
    h[rng.integers(0, n)] = bad
    p = rng.normal(0, 1, n).astype(np.float32)
    m = rng.normal(0, 1e-3, n).astype(np.float32)
    v = np.abs(rng.normal(0, 1e-6, n)).astype(np.float32)
    keep = [x.copy() for x in (p, m, v)]
    assert oracle.adam_step(5, 65536.0, h, "f16", p, m, v) == 1
    for x, y in zip((p, m, v), keep):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_largest_finite_gradient_does_not_skip():
    h = np.array([0x7BFF, 0xFBFF, 0x0001, 0x8000], np.uint16)   # fp16 max, -max, subnormal, -0
    p, m, v = _zeros(4)
    assert oracle.adam_step(1, 65536.0, h, "f16", p, m, v) == 0
    hb = np.array([0x7F7F, 0xFF7F], np.uint16)                   # bf16 max finite
    p, m, v = _zeros(2)
    assert oracle.adam_step(1, 1.0, hb, "bf16", p, m, v) == 0


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_f32_gradients_equal_the_half_path_on_values_it_represents(dt):
    # fp32 gradients that are exactly fp16 / bf16 values give the half path's
    # state bit for bit: the update reads the value, not the encoding
    rng = np.random.default_rng(11)
    n, scale = 2049, (1024.0 if dt == "f16" else 1.0)
    h = oracle.float_to_half((rng.normal(0, 1e-3, n) * scale).astype(np.float32), dt)
    f = oracle.half_to_float(h, dt)
    a = [rng.normal(0, 0.02, n).astype(np.float32), *_zeros(n)[1:]]
    b = [x.copy() for x in a]
    for t in range(1, 6):
        for adamw in (True, False):
            assert oracle.adam_step(t, scale, h, dt, *a, adamw=adamw) == 0
            assert oracle.adam_step(t, scale, f, "f32", *b, adamw=adamw) == 0
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("bad", [0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001])
def test_f32_overflow_step_changes_nothing(bad):
    rng = np.random.default_rng(2)
    n = 300
    g = rng.normal(0, 1e-3, n).astype(np.float32).view(np.uint32).copy()
    g[rng.integers(0, n)] = bad
    p = rng.normal(0, 1, n).astype(np.float32)
    m = rng.normal(0, 1e-3, n).astype(np.float32)
    v = np.abs(rng.normal(0, 1e-6, n)).astype(np.float32)
    keep = [x.copy() for x in (p, m, v)]
    assert oracle.adam_step(5, 1.0, g, "f32", p, m, v) == 1
    for x, y in zip((p, m, v), keep):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    g[g == bad] = 0x7F7FFFFF                       # the largest finite value does not skip
    assert oracle.adam_step(5, 1.0, g, "f32", p, m, v) == 0
