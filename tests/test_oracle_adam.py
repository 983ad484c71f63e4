"""Pins of the oracle's Adam(W) update, clipping and loss-scale policy.

Closed forms: with m0 = v0 = 0 and a constant gradient g, bias-corrected Adam
has m_hat = g and v_hat = g^2 exactly in real arithmetic, so every step moves
the parameter by lr * g / (|g| + eps) (Kingma and Ba, cited on the ZeRO pages
for the optimizer states: "ZeRO: Memory Optimizations Toward Training Trillion
Parameter Models" summary, 3.4 "Model-State Memory Analysis").  Decoupled
weight decay ("ZeRO Stage 1/2/3" guide, section 5, AdamW with weight_decay)
adds a geometric factor.  torch.optim.AdamW in fp32 on the CPU is an
independent library cross-check.

The pages give no clip rule and no loss-scale schedule; the readings taken
are PyTorch's, and these tests pin the oracle's decisions to PyTorch's own
CPU routines: torch.nn.utils.clip_grads_with_norm_ (coefficient
min(1, max / (norm + 1e-6)), here given the oracle's binary64 norm) and
torch._amp_update_scale_ (halve on overflow, double after growth_interval
clean steps unless the doubled scale is not finite).  The one departure,
the min_scale floor, has its own test.
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


def _torch_clipped(g: np.ndarray, norm: float, max_norm: float) -> np.ndarray:
    """g (fp32) after torch.nn.utils.clip_grads_with_norm_ with total norm `norm`."""
    t = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float32))
    t.grad = torch.from_numpy(g.copy())
    torch.nn.utils.clip_grads_with_norm_([t], max_norm, torch.tensor(norm, dtype=torch.float64),
                                         foreach=False)
    return t.grad.numpy()


def _clip_case_grads():
    """Gradients whose norms fall far below, just below, inside the window
    (max - 1e-6, max], exactly on, just above and far above max = 1, and
    around other thresholds."""
    cases = []
    for x in (0.5, 0.999998, 0.9999990, 0.9999995, np.nextafter(np.float32(1), np.float32(0)),
              1.0, np.nextafter(np.float32(1), np.float32(2)), 1.0000010, 1.5, 34.7, 1e6):
        cases.append((np.array([x], np.float32), 1.0))   # norm = |x| exactly
    for max_norm in (1.0, 0.25, 3.0, 1e-3):
        for target in (0.3, 0.9999999, 1.0, 1.0000003, 2.0, 316.0):
            g = rng.normal(0, 1.0, 4096)
            g = (g * (target * max_norm / np.linalg.norm(g))).astype(np.float32)
            cases.append((g, max_norm))
    for _ in range(200):
        g = rng.normal(0, 1.0, int(rng.integers(1, 64))).astype(np.float32)
        cases.append((g * np.float32(10.0 ** rng.uniform(-3, 3)), float(np.float32(rng.uniform(0.1, 5)))))
    return cases


def test_clip_rule_matches_torch():
    """For every norm, the oracle's clipped gradient equals, bit for bit,
    torch's clip_grads_with_norm_ given the same binary64 norm: the same
    coefficient (rounded once to fp32, 1 where torch clamps it) applied by the
    same fp32 multiplication.  Includes norms in (max - 1e-6, max], which
    torch scales and a rule 'clip only when norm > max' would not."""
    import oracle as O
    in_window = 0
    for g, max_norm in _clip_case_grads():
        max_norm = float(np.float32(max_norm))  # the threshold is an fp32 setting
        hp = O.hparams(max_grad_norm=max_norm)
        rep = O.finalize(hp, O.new_scalars(1.0), 0, O.SumSq().add(g))
        ref = _torch_clipped(g, rep.norm, max_norm)
        ours = g * np.float32(rep.clip)
        assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32)), (max_norm, rep.norm, rep.clip)
        coef = max_norm / (rep.norm + 1e-6)
        assert (rep.clip == 1.0) == (coef >= 1.0), (max_norm, rep.norm, rep.clip)
        if max_norm - 1e-6 < rep.norm <= max_norm:
            in_window += 1
            assert rep.clip < 1.0
    assert in_window >= 3


# ------------------------------------------------------------------------- loss scale
def _torch_scaler(scale0: float, flags, growth_interval: int):
    """(scale, growth tracker) after each step of torch._amp_update_scale_
    with growth factor 2 and backoff 0.5 (GradScaler's defaults)."""
    s = torch.tensor([scale0], dtype=torch.float32)
    tracker = torch.zeros(1, dtype=torch.int32)
    out = []
    for bad in flags:
        torch._amp_update_scale_(s, tracker, torch.tensor([1.0 if bad else 0.0]), 2.0, 0.5,
                                 growth_interval)
        out.append((float(s[0]), int(tracker[0])))
    return out


@pytest.mark.parametrize("scale0,growth_interval,p_bad", [
    (2.0 ** 15, 1000, 0.2), (2.0 ** 15, 1, 0.3), (2.0 ** 16, 2, 0.25), (1.0, 3, 0.1),
    (0.75, 1, 0.0), (2.0 ** 126, 1, 0.0), (2.0 ** 127, 1, 0.05), (3.0e38, 2, 0.05),
    (2.0 ** 120, 5, 0.02), (1.5 * 2.0 ** 100, 1, 0.5)])
def test_scaler_matches_torch(O, scale0, growth_interval, p_bad):
    """The dynamic scaler's trace equals torch._amp_update_scale_'s (scale and
    run count after every step), including growth that would overflow fp32:
    torch keeps the scale there and so does the oracle."""
    flags = [int(b) for b in np.random.default_rng(int(scale0 % 977) + growth_interval).random(300)
             < p_bad]
    flags[:3] = [0, 0, 0]
    hp = O.hparams(scaler=2, min_scale=2.0 ** -126, growth_interval=growth_interval)
    st = O.new_scalars(scale0)
    ref = _torch_scaler(scale0, flags, growth_interval)
    for i, (bad, (s_ref, tr_ref)) in enumerate(zip(flags, ref)):
        assert s_ref >= 2.0 ** -126  # the floor never binds in these traces
        _flags_step(O, hp, st, bad)
        assert (st.scale, st.good) == (s_ref, tr_ref), (i, st.scale, st.good, s_ref, tr_ref)
        assert np.isfinite(st.scale)


def test_scaler_growth_never_reaches_infinity(O):
    """From 2^127 with growth_interval 1 every applied step asks to double: the
    scale stays 2^127 (as torch's does) instead of becoming inf."""
    hp = O.hparams(scaler=2, min_scale=1.0, growth_interval=1)
    st = O.new_scalars(2.0 ** 127)
    for _ in range(5):
        rep = _flags_step(O, hp, st, 0)
        assert rep.skip == 0 and st.scale == 2.0 ** 127 and st.good == 0
    assert _torch_scaler(2.0 ** 127, [0] * 5, 1)[-1] == (2.0 ** 127, 0)


def test_scaler_floor_departs_from_torch(O):
    """The one departure: torch halves below any floor (down to 0); the
    oracle's scale stops at min_scale."""
    hp = O.hparams(scaler=2, min_scale=0.25, growth_interval=1000)
    st = O.new_scalars(1.0)
    flags = [1, 1, 1, 1]
    ref = _torch_scaler(1.0, flags, 1000)
    ours = []
    for bad in flags:
        _flags_step(O, hp, st, bad)
        ours.append(st.scale)
    assert [s for s, _ in ref] == [0.5, 0.25, 0.125, 0.0625]
    assert ours == [0.5, 0.25, 0.25, 0.25]
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
