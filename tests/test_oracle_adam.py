"""Pins of the oracle's Adam(W) update, clipping and loss-scale policy.

Closed forms: with m0 = v0 = 0 and a constant gradient g, bias-corrected Adam
has m_hat = g and v_hat = g^2 exactly in real arithmetic, so every step moves
the parameter by lr * g / (|g| + eps) (Kingma and Ba, cited on the ZeRO pages
for the optimizer states: "ZeRO: Memory Optimizations Toward Training Trillion
Parameter Models" summary, 3.4 "Model-State Memory Analysis").  Decoupled
weight decay ("ZeRO Stage 1/2/3" guide, section 5, AdamW with weight_decay)
adds a geometric factor.  torch.optim.AdamW in fp32 on the CPU is an
independent library cross-check.
"""
import numpy as np
import pytest
import torch

rng = np.random.default_rng(7)
ULP = 2.0 ** -23


def _run(O, p0, grads, hp, clip=1.0):
    p = np.array(p0, np.float32)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    st = O.new_scalars(1.0)
    for g in grads:
        acc = O.SumSq().add(g)
        rep = O.finalize(hp, st, 0, acc)
        O.adam(p, m, v, np.asarray(g, np.float32), hp, rep.clip if clip else 1.0, st.pow1,
               st.pow2)
    return p, m, v, st


@pytest.mark.parametrize("t", [1, 2, 5, 20])
def test_constant_gradient_closed_form(O, t):
    n = 4096
    g = (rng.normal(0, 1e-3, n) * rng.choice([1e-2, 1, 10], n)).astype(np.float32)
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    hp = O.hparams(lr=1e-3)
    p, m, v, _ = _run(O, p0, [g] * t, hp)
    g64 = g.astype(np.float64)
    u = g64 / (np.abs(g64) + 1e-8)
    closed = p0.astype(np.float64) - t * 1e-3 * u
    # each step: u to a few ulps (m and v carry t roundings), p rounded once
    tol = t * (1e-3 * np.abs(u) * 8 * t * ULP + np.abs(closed) * ULP) + 1e-12
    assert np.all(np.abs(p - closed) <= tol)
    # m_t = (1 - beta1^t) g and v_t = (1 - beta2^t) g^2 in reals, with the
    # betas being the binary32 hyperparameters 0.9f and 0.999f
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    mt = (1 - b1 ** t) * g64
    vt = (1 - b2 ** t) * g64 ** 2
    assert np.all(np.abs(m - mt) <= 4 * t * ULP * np.abs(mt) + 1e-45)
    assert np.all(np.abs(v - vt) <= 6 * t * ULP * vt + 1e-45)


@pytest.mark.parametrize("t", [1, 3, 10])
def test_constant_gradient_with_decoupled_weight_decay(O, t):
    n = 2048
    lr, wd = 1e-3, 0.01
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    hp = O.hparams(lr=lr, weight_decay=wd)
    p, _, _, _ = _run(O, p0, [g] * t, hp)
    u = g.astype(np.float64) / (np.abs(g.astype(np.float64)) + 1e-8)
    a = 1 - lr * wd
    closed = a ** t * p0.astype(np.float64) - lr * u * sum(a ** j for j in range(t))
    tol = t * (lr * 8 * t * ULP + np.abs(closed) * 2 * ULP)
    assert np.all(np.abs(p - closed) <= tol)


def test_first_step_any_gradient(O):
    n = 10_000
    g = (rng.normal(0, 1, n) * 10.0 ** rng.uniform(-6, 1, n)).astype(np.float32)
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    hp = O.hparams(lr=3e-4, weight_decay=0.1)
    p, _, _, st = _run(O, p0, [g], hp)
    g64, p64 = g.astype(np.float64), p0.astype(np.float64)
    closed = p64 - 3e-4 * (g64 / (np.abs(g64) + 1e-8) + 0.1 * p64)
    assert st.t == 1
    assert np.all(np.abs(p - closed) <= 3e-4 * 6 * ULP + 2 * ULP * np.abs(closed))


def test_epsilon_sits_outside_the_square_root(O):
    # with |g| = 1e-4, g^2 = eps: inside the root would change the step by ~29%
    g = np.full(16, 1e-4, np.float32)
    p, _, _, _ = _run(O, np.zeros(16, np.float32), [g], O.hparams(lr=1.0))
    assert np.allclose(p, -1e-4 / (1e-4 + 1e-8), rtol=1e-6)


def test_matches_torch_adamw(O):
    """torch.optim.AdamW (fp32, CPU, same binary32 betas) orders the same
    arithmetic differently (lerp for m, sqrt(v)/sqrt(bc2), decay before the
    step), so the two agree to rounding: within 1e-5 of each array's RMS
    after 12 steps, where a wrong term would differ by O(1) of the update."""
    n, steps = 50_000, 12
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    grads = [rng.normal(0, 1e-3, n).astype(np.float32) for _ in range(steps)]
    hp = O.hparams(lr=1e-3, weight_decay=0.01)
    p, m, v, _ = _run(O, p0, grads, hp)
    betas = (float(np.float32(0.9)), float(np.float32(0.999)))
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=1e-3, betas=betas, eps=1e-8, weight_decay=0.01,
                            foreach=False)
    for g in grads:
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
    s = opt.state[tp]
    for ours, ref in ((p, tp.detach().numpy()), (m, s["exp_avg"].numpy()),
                      (v, s["exp_avg_sq"].numpy())):
        rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
        assert np.abs(ours - ref).max() <= 1e-5 * rms
    # the accumulated update itself agrees to 1e-4 of its RMS
    du, dref = p - p0, tp.detach().numpy() - p0
    assert np.abs(du - dref).max() <= 1e-4 * float(np.sqrt(np.mean(dref.astype(np.float64) ** 2)))


# ------------------------------------------------------------------------- clip
def test_clip_leaves_small_gradients_bitwise(O):
    g = rng.normal(0, 1e-3, 1000).astype(np.float32)
    hp = O.hparams(max_grad_norm=1.0)
    st = O.new_scalars(1.0)
    rep = O.finalize(hp, st, 0, O.SumSq().add(g))
    assert rep.norm < 1.0 and rep.clip == 1.0
    assert np.array_equal(g * np.float32(rep.clip), g)


@pytest.mark.parametrize("target_norm", [316.0, 1.25])
def test_clip_rescales_to_max_norm(O, target_norm):
    # post-clip norm is max * norm / (norm + 1e-6); near max (1.25) the 1e-6
    # term moves it by 8e-7 relative, well outside the 1e-7 tolerance
    g = rng.normal(0, 1.0, 100_000)
    g = (g * (target_norm / np.linalg.norm(g))).astype(np.float32)
    hp = O.hparams(max_grad_norm=1.0)
    rep = O.finalize(hp, O.new_scalars(1.0), 0, O.SumSq().add(g))
    gc = g * np.float32(rep.clip)
    post = float(np.linalg.norm(gc.astype(np.float64)))
    assert abs(rep.norm - target_norm) < 1e-3 * target_norm
    assert abs(post - rep.norm / (rep.norm + 1e-6)) <= 1e-7


# ------------------------------------------------------------------------- loss scale
def _flags_step(O, hp, st, bad):
    g = np.array([np.inf if bad else 1e-3], np.float32)
    return O.finalize(hp, st, int(bad), O.SumSq().add(g))


def test_dynamic_scaler_trace(O):
    """Hand-derived from the adopted reading: skip on overflow and halve S,
    otherwise apply the step; S doubles after growth_interval clean steps."""
    hp = O.hparams(scaler=2, min_scale=1.0, growth_interval=1000)
    st = O.new_scalars(2.0 ** 15)
    trace = []
    for bad in (0, 1, 0, 0, 0):
        rep = _flags_step(O, hp, st, bad)
        trace.append((rep.scale_used, rep.skip, st.t))
    assert trace == [(2.0 ** 15, 0, 1), (2.0 ** 15, 1, 1), (2.0 ** 14, 0, 2), (2.0 ** 14, 0, 3),
                     (2.0 ** 14, 0, 4)]
    assert st.scale == 2.0 ** 14


def test_dynamic_scaler_growth_and_floor(O):
    hp = O.hparams(scaler=2, min_scale=4.0, growth_interval=2)
    st = O.new_scalars(8.0)
    scales = []
    for bad in (0, 0, 0, 0, 1, 1, 1, 0, 0):
        _flags_step(O, hp, st, bad)
        scales.append(st.scale)
    # grows after every 2 clean steps (twice in a row), halves per skip, floor 4
    assert scales == [8.0, 16.0, 16.0, 32.0, 16.0, 8.0, 4.0, 4.0, 8.0]


def test_skip_without_scaler_keeps_scale_and_step(O):
    hp = O.hparams(scaler=0)
    st = O.new_scalars(1.0)
    rep = _flags_step(O, hp, st, 1)
    assert rep.skip == 1 and st.t == 0 and st.scale == 1.0 and st.pow1 == 1.0
    rep = _flags_step(O, hp, st, 0)
    assert rep.skip == 0 and st.t == 1 and st.pow1 == np.float64(np.float32(0.9))


def test_bias_correction_powers_are_running_products(O):
    hp = O.hparams()
    st = O.new_scalars(1.0)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    e1 = e2 = 1.0
    for _ in range(50):
        _flags_step(O, hp, st, 0)
        e1 *= b1
        e2 *= b2
        assert st.pow1 == e1 and st.pow2 == e2
