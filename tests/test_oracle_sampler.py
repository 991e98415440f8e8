"""Oracle pins for the sampler steps around the denoiser.

What pins them (none of it re-types the oracle's formulas):
  * the forward process of cv-learn "Sora / DiT" (Method, training objective
    bullet) composed step by step reproduces the schedule's abar;
  * Gaussian conditioning of the joint law of (x_s, x_t) given x_0, done with
    a 2x2 covariance and a linear solve, gives the reverse-step mean and
    variance;
  * the learned-covariance endpoints (v = +1 -> beta, v = -1 -> beta_tilde);
  * for Gaussian data every ideal predictor is affine and has a closed form,
    so an ancestral chain with the ideal mean and variance must return the
    data law exactly, an ODE solver must converge to the exact flow map at
    its order (DDIM first, DPM-Solver++(2M) second, rectified-flow Euler
    first), and a point-mass data law must be hit exactly;
  * DPM-Solver++ at first order equals the deterministic DDIM update written
    from DDIM's definition.
"""
import math

import numpy as np
import pytest

from oracle import sampler_oracle as so


# --- schedule ---------------------------------------------------------------

def test_schedule_matches_composed_forward_process():
    betas, abar = so.linear_beta_schedule()
    assert betas.shape == (1000,) and abar.shape == (1000,)
    assert betas[0] == pytest.approx(1e-4, rel=1e-14)
    assert betas[-1] == pytest.approx(0.02, rel=1e-14)
    assert np.allclose(np.diff(betas), (0.02 - 1e-4) / 999, rtol=1e-10, atol=0)
    # q(x_t | x_{t-1}) = N(sqrt(1 - beta_t) x_{t-1}, beta_t): push mean (per unit
    # x_0) and variance through t + 1 single steps; the marginal must be
    # N(sqrt(abar_t) x_0, 1 - abar_t).
    m, v = 1.0, 0.0
    for t in range(1000):
        m = math.sqrt(1.0 - betas[t]) * m
        v = (1.0 - betas[t]) * v + betas[t]
        assert m == pytest.approx(math.sqrt(abar[t]), rel=1e-12)
        assert v == pytest.approx(1.0 - abar[t], rel=1e-12, abs=1e-16)


def test_even_timesteps():
    assert list(so.even_timesteps(1)) == [999]
    assert list(so.even_timesteps(2)) == [999, 0]
    full = so.even_timesteps(1000)
    assert list(full) == list(range(999, -1, -1))
    for S in (25, 50, 250):
        ts = so.even_timesteps(S)
        assert len(ts) == S and ts[0] == 999 and ts[-1] == 0
        assert np.all(np.diff(ts) < 0)
        gaps = -np.diff(ts)
        assert gaps.max() - gaps.min() <= 1


# --- DDPM reverse step ------------------------------------------------------

def _conditioning(abar_t, abar_s):
    """Law of x_s given (x_t, x_0) by Gaussian conditioning.  x_s = a_s x_0 + n_s,
    x_t = r x_s + n, with a_s = sqrt(abar_s), Var n_s = 1 - abar_s,
    r = sqrt(abar_t/abar_s), Var n = 1 - abar_t/abar_s.  Returns the weights
    of x_0 and x_t in the conditional mean and the conditional variance."""
    a_s = math.sqrt(abar_s)
    r = math.sqrt(abar_t / abar_s)
    var_s = 1.0 - abar_s
    var_n = 1.0 - abar_t / abar_s
    # (x_s, x_t) - E[. | x_0] has covariance S; E[x_s | x_0] = a_s x_0,
    # E[x_t | x_0] = r a_s x_0.
    S = np.array([[var_s, r * var_s], [r * var_s, r * r * var_s + var_n]])
    k = np.linalg.solve(S[1:, 1:], S[1:, :1])[0, 0]   # Cov(x_s,x_t)/Var(x_t)
    var = S[0, 0] - k * S[1, 0]
    w_x0 = a_s - k * r * a_s
    w_xt = k
    return w_x0, w_xt, var


@pytest.mark.parametrize("abar_t,abar_s", [(0.3, 0.5), (4e-5, 0.02), (0.9, 0.9999),
                                          (0.0123, 0.0124)])
def test_ddpm_step_is_gaussian_conditioning(abar_t, abar_s):
    rng = np.random.default_rng(3)
    C = 3
    x0 = rng.standard_normal((2, C, 4, 4))
    eps = rng.standard_normal((2, C, 4, 4))
    x_t = math.sqrt(abar_t) * x0 + math.sqrt(1 - abar_t) * eps
    w_x0, w_xt, var = _conditioning(abar_t, abar_s)
    mean = w_x0 * x0 + w_xt * x_t
    # The true noise as the model output: the step's mean is E[x_s | x_t, x_0].
    got = so.ddpm_step(x_t, eps, C, abar_t, abar_s, np.zeros_like(x_t))
    assert np.allclose(got, mean, rtol=1e-10, atol=1e-10)
    # Cout == C: the variance is beta_tilde, the conditional variance.
    got1 = so.ddpm_step(x_t, eps, C, abar_t, abar_s, np.ones_like(x_t))
    assert np.allclose(got1 - got, math.sqrt(var), rtol=1e-10, atol=0)
    q = so.ddpm_transition(abar_t, abar_s)
    assert q["beta_tilde"] == pytest.approx(var, rel=1e-10)


def test_predict_x0_inverts_forward_process():
    rng = np.random.default_rng(4)
    x0 = rng.standard_normal((3, 4, 8, 8))
    eps = rng.standard_normal((3, 4, 8, 8))
    for abar in (1e-4, 0.5, 0.9999):
        x_t = math.sqrt(abar) * x0 + math.sqrt(1 - abar) * eps
        assert np.allclose(so.predict_x0(x_t, eps, abar), x0, rtol=0, atol=1e-9)


@pytest.mark.parametrize("v,which", [(1.0, "beta"), (-1.0, "beta_tilde"), (0.0, "geo")])
def test_learned_variance_endpoints(v, which):
    abar_t, abar_s = 0.2, 0.35
    C = 2
    x = np.zeros((1, C, 2, 2))
    mo = np.concatenate([np.zeros_like(x), np.full_like(x, v)], axis=1)
    q = so.ddpm_transition(abar_t, abar_s)
    beta = 1 - abar_t / abar_s
    bt = beta * (1 - abar_s) / (1 - abar_t)
    want = {"beta": math.sqrt(beta), "beta_tilde": math.sqrt(bt),
            "geo": (beta * bt) ** 0.25}[which]
    noise = so.ddpm_step(x, mo, C, abar_t, abar_s, np.ones_like(x))
    assert np.allclose(noise, want, rtol=1e-12, atol=0)
    assert q["beta"] == pytest.approx(beta, rel=1e-14)


def test_last_step_is_x0_prediction_and_reads_no_noise():
    rng = np.random.default_rng(5)
    C = 4
    x = rng.standard_normal((2, C, 4, 4))
    mo = rng.standard_normal((2, 2 * C, 4, 4))
    z = np.full_like(x, np.nan)
    abar_t = 0.9999
    got = so.ddpm_step(x, mo, C, abar_t, 1.0, z)
    want = (x - math.sqrt(1 - abar_t) * mo[:, :C]) / math.sqrt(abar_t)
    assert np.all(np.isfinite(got))
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


# --- Gaussian data: ideal predictors in closed form ---------------------------

def _gauss_posterior(x, abar, mu, s):
    """Data x_0 ~ N(mu, s^2), x_t = sqrt(abar) x_0 + sqrt(1-abar) eps:
    E[x_0 | x_t = x] and Var(x_0 | x_t)."""
    a = math.sqrt(abar)
    tot = abar * s * s + 1 - abar
    mean = mu + a * s * s * (x - a * mu) / tot
    var = s * s * (1 - abar) / tot
    return mean, var


def _ideal_eps(x, abar, mu, s):
    m, _ = _gauss_posterior(x, abar, mu, s)
    return (x - math.sqrt(abar) * m) / math.sqrt(1 - abar)


@pytest.mark.parametrize("S", [1, 7, 50])
def test_ddpm_point_mass_is_hit_exactly(S):
    _, abar = so.linear_beta_schedule()
    ts = so.even_timesteps(S)
    mu = 0.7
    rng = np.random.default_rng(6)
    xT = rng.standard_normal((2, 3, 4, 4))
    noise = rng.standard_normal((S,) + xT.shape)

    def model(x, t):
        ab = abar[int(t)]
        eps = (x - math.sqrt(ab) * mu) / math.sqrt(1 - ab)
        return np.concatenate([eps, np.zeros_like(eps)], axis=1)

    out = so.sample_ddpm(model, xT, ts, noise, 3, abar)
    assert np.allclose(out, mu, rtol=0, atol=1e-9)
    out2 = so.sample_dpmpp_2m(model, xT, ts, 3, abar)
    assert np.allclose(out2, mu, rtol=0, atol=1e-9)


@pytest.mark.parametrize("S,mu,s", [(50, 0.4, 1.3), (250, -1.0, 0.5), (10, 0.0, 1.0)])
def test_ddpm_chain_with_ideal_mean_and_variance_returns_data_law(S, mu, s):
    """The chain is affine-Gaussian, so push mean and variance through it
    exactly: each step x -> A x + B + sig z is read off the oracle step by
    evaluating it at x in {0, 1} and z in {0, 1}."""
    _, abar = so.linear_beta_schedule()
    ts = so.even_timesteps(S)
    levels = [float(abar[t]) for t in ts] + [1.0]
    C = 1
    m = math.sqrt(levels[0]) * mu
    v = levels[0] * s * s + 1 - levels[0]
    for k in range(S):
        ab_t, ab_s = levels[k], levels[k + 1]
        _, var0 = _gauss_posterior(0.0, ab_t, mu, s)
        if ab_s < 1.0:
            w_x0, _, var_c = _conditioning(ab_t, ab_s)
            true_var = var_c + w_x0 * w_x0 * var0     # law of x_s given x_t
            beta = 1 - ab_t / ab_s
            bt = beta * (1 - ab_s) / (1 - ab_t)
            v_raw = 2 * (math.log(true_var) - math.log(bt)) / (math.log(beta) - math.log(bt)) - 1
        else:
            v_raw = 0.0

        def step(x, z):
            xa = np.full((1, C, 1, 1), x)
            mo = np.concatenate([_ideal_eps(xa, ab_t, mu, s), np.full_like(xa, v_raw)], axis=1)
            lbt = so.ddpm_last_log_beta_tilde(levels[:-1]) if ab_s >= 1.0 else None
            return float(so.ddpm_step(xa, mo, C, ab_t, ab_s, np.full_like(xa, z),
                                      log_beta_tilde=lbt)[0, 0, 0, 0])

        B0 = step(0.0, 0.0)
        A = step(1.0, 0.0) - B0
        sig = step(0.0, 1.0) - B0
        m, v = A * m + B0, A * A * v + sig * sig
        if ab_s < 1.0:   # every intermediate marginal is the forward process's
            assert m == pytest.approx(math.sqrt(ab_s) * mu, rel=1e-9, abs=1e-12)
            assert v == pytest.approx(ab_s * s * s + 1 - ab_s, rel=1e-9)
    # The last step adds no noise: its output is E[x_0 | x_{tau_1}], whose
    # variance falls short of s^2 by Var(x_0 | x_{tau_1}).
    _, var_last = _gauss_posterior(0.0, levels[-2], mu, s)
    assert m == pytest.approx(mu, rel=1e-9, abs=1e-12)
    assert v == pytest.approx(s * s - var_last, rel=1e-9)


# --- ODE solvers --------------------------------------------------------------

def _vp_flow(x_from, ab_from, ab_to, mu, s):
    """Exact probability-flow map for Gaussian data: the standardised
    coordinate (x - sqrt(abar) mu) / sqrt(abar s^2 + 1 - abar) is conserved."""
    z = (x_from - math.sqrt(ab_from) * mu) / math.sqrt(ab_from * s * s + 1 - ab_from)
    return math.sqrt(ab_to) * mu + math.sqrt(ab_to * s * s + 1 - ab_to) * z


def _lambda_grid(ab_start, ab_end, S):
    lam = np.linspace(so.log_snr_half(ab_start), so.log_snr_half(ab_end), S + 1)
    return [1.0 / (1.0 + math.exp(-2 * l)) for l in lam]   # abar from lambda


def _solve(levels, x, mu, s, second):
    x0_prev = None
    for k in range(len(levels) - 1):
        eps = _ideal_eps(x, levels[k], mu, s)
        use2 = second and x0_prev is not None
        x, x0 = so.dpmpp_step(x, eps, levels[k], levels[k + 1],
                              x0_prev if use2 else None, levels[k - 1] if use2 else None)
        x0_prev = x0
    return x


def test_dpmpp_first_order_equals_ddim():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 4, 3, 3))
    eps = rng.standard_normal((2, 4, 3, 3))
    for ab_t, ab_s in [(0.01, 0.2), (0.5, 0.9), (4e-5, 1e-3)]:
        x0 = (x - math.sqrt(1 - ab_t) * eps) / math.sqrt(ab_t)
        ddim = math.sqrt(ab_s) * x0 + math.sqrt(1 - ab_s) * eps   # DDIM, eta = 0
        got, gx0 = so.dpmpp_step(x, eps, ab_t, ab_s)
        assert np.allclose(got, ddim, rtol=1e-12, atol=1e-12)
        assert np.allclose(gx0, x0, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("second,lo,hi", [(False, 1.7, 2.3), (True, 3.3, 4.7)])
def test_dpmpp_converges_at_its_order(second, lo, hi):
    _, abar = so.linear_beta_schedule()
    ab0, ab1 = float(abar[999]), float(abar[0])
    mu, s = 0.3, 0.8
    x = np.linspace(-3, 3, 13)
    exact = _vp_flow(x, ab0, ab1, mu, s)
    errs = []
    for S in (16, 32, 64, 128):
        got = _solve(_lambda_grid(ab0, ab1, S), x, mu, s, second)
        errs.append(np.max(np.abs(got - exact)))
    ratios = [errs[i] / errs[i + 1] for i in range(len(errs) - 1)]
    assert all(lo < r < hi for r in ratios[1:]), (errs, ratios)


def test_dpmpp_loop_converges_on_the_discrete_schedule():
    """sample_dpmpp_2m on even kept steps; the reference is the exact flow to
    tau_1 = 0 followed by the exact posterior mean (the first-order jump into
    sigma = 0 is exactly E[x_0 | x])."""
    _, abar = so.linear_beta_schedule()
    mu, s = -0.2, 1.1
    xT = np.linspace(-2.5, 2.5, 11).reshape(1, 1, 11, 1)
    model = lambda x, t: _ideal_eps(x, float(abar[int(t)]), mu, s)
    errs = []
    for S in (25, 50, 100):
        got = so.sample_dpmpp_2m(model, xT, so.even_timesteps(S), 1, abar)
        xl = _vp_flow(xT, float(abar[999]), float(abar[0]), mu, s)
        want, _ = _gauss_posterior(xl, float(abar[0]), mu, s)
        errs.append(np.max(np.abs(got - want)))
    # The even grid takes large log-SNR steps near tau = 0, so the error at
    # 25 steps is large; what is pinned is the second-order decay.
    assert errs[0] < 0.25 and errs[1] < errs[0] / 3.3 and errs[2] < errs[1] / 3.3, errs


# --- rectified flow -----------------------------------------------------------

def test_rf_point_mass_path_is_straight_and_exact():
    """Data at a single point mu: the ideal velocity (mu - x)/(1 - t) is
    constant along each path, so Euler is exact on any grid."""
    mu = 1.5
    rng = np.random.default_rng(8)
    x0 = rng.standard_normal((2, 16, 2, 4, 4))
    times = np.sort(np.concatenate([[0.0, 1.0], rng.uniform(0.01, 0.99, 6)]))
    x = x0.copy()
    for k in range(len(times) - 1):
        v = (mu - x) / (1 - times[k])
        x = so.rf_euler_step(x, v, times[k], times[k + 1])
        assert np.allclose(x, (1 - times[k + 1]) * x0 + times[k + 1] * mu, atol=1e-12)
    model = lambda xx, t: (mu - xx) / (1 - t)
    out = so.sample_rf_euler(model, x0, times)
    assert np.allclose(out, mu, atol=1e-12)


def test_rf_euler_first_order_on_gaussian_data():
    """x_1 ~ N(mu, s^2), x_0 ~ N(0, 1), x_t = t x_1 + (1-t) x_0.  The ideal
    velocity E[x_1 - x_0 | x_t = x] is affine in x; the exact flow keeps
    (x - t mu) / sqrt(t^2 s^2 + (1-t)^2) fixed."""
    mu, s = 0.5, 0.6

    def vel(x, t):
        var = t * t * s * s + (1 - t) ** 2
        cov = t * s * s - (1 - t)
        return mu + cov / var * (x - t * mu)

    x0 = np.linspace(-3, 3, 13)
    exact = mu + s * x0
    errs = [np.max(np.abs(so.sample_rf_euler(vel, x0, so.rf_uniform_times(S)) - exact))
            for S in (32, 64, 128, 256)]
    ratios = [errs[i] / errs[i + 1] for i in range(3)]
    assert all(1.7 < r < 2.3 for r in ratios), (errs, ratios)
