"""fp64 reference of the sampler steps that run around the denoiser.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every array is
converted to float64 on entry; nothing is rounded in between.

What the pages fix, and the readings taken where they stop:
  * [Sora-cvl] Method / training objective bullet: the forward process
    x_t = sqrt(abar_t) x_0 + sqrt(1 - abar_t) eps; the reverse-process
    covariance Sigma_theta is learned (trained with the full KL term) and the
    decoder emits noise and covariance, 2C channels per latent element.
  * [DiT-wiki] Inference with diffusers: sampling runs a multistep
    DPM-Solver scheduler for 25 steps with guidance.
  * [Goku] 2.3 rectified flow: x_t = t x_1 + (1 - t) x_0 with x_0 ~ N(0, I)
    noise and x_1 data; the network predicts the velocity that carries x_t
    toward x_1; inference integrates that velocity from noise to data.
Readings (none of this is printed on the pages):
  * noise schedule: 1000 training steps, beta linear from 1e-4 to 0.02
    (the DDPM schedule; consistent with integer t in 0..999 fed to the
    timestep sinusoid).
  * sampling on a subset of steps tau_S > ... > tau_1 keeps abar at the kept
    steps; the step from tau_k goes to tau_{k-1}, and the last step goes to
    the clean latent (abar = 1).  Default subset: tau = round(j (1000-1)/(S-1)).
  * learned Sigma: the raw channel value v in [C, 2C) sets
    log var = f log(beta) + (1 - f) log(beta_tilde) with f = (v + 1) / 2,
    i.e. an interpolation between the two classical DDPM variances (the
    published "learned range" parameterisation, Nichol and Dhariwal 2021).
    Channels [0, C) are eps.  With C output channels the variance is
    beta_tilde.
  * no clipping of the predicted x_0 (the pages bound no latent range).
  * DPM-Solver++(2M) (Lu et al. 2022, data-prediction multistep solver,
    second order): first step first order; the last step into sigma = 0 is
    first order (the second-order weights are undefined there).
  * rectified flow: explicit Euler from t = 0 (noise) to t = 1 (data),
    uniform grid by default; the model is evaluated at the grid time as is.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Schedule

def linear_beta_schedule(train_steps=1000, beta_start=1e-4, beta_end=0.02):
    """betas [train_steps] on a straight line, and abar_t = prod_{j<=t}(1 - beta_j)."""
    betas = np.linspace(beta_start, beta_end, train_steps, dtype=np.float64)
    abar = np.cumprod(1.0 - betas)
    return betas, abar


def even_timesteps(S, train_steps=1000):
    """S kept steps, evenly spread over [0, train_steps - 1], in sampling
    order (largest first).  Rounds half away from zero."""
    if S < 1 or S > train_steps:
        raise ValueError("S must be in [1, train_steps]")
    if S == 1:
        return np.array([train_steps - 1], dtype=np.int64)
    ks = [int(math.floor(j * (train_steps - 1) / (S - 1) + 0.5)) for j in range(S)]
    return np.array(ks[::-1], dtype=np.int64)


# ---------------------------------------------------------------------------
# DDPM ancestral step with learned covariance ([Sora-cvl] Method)

def ddpm_transition(abar_t, abar_s):
    """Quantities of the reverse step from a level with abar_t to one with
    abar_s >= abar_t (abar_s = 1 is the clean latent).
    Returns dict with beta (of this step), beta_tilde (posterior variance),
    c_x0 and c_xt (posterior-mean weights of x_0 and x_t)."""
    beta = 1.0 - abar_t / abar_s
    alpha = 1.0 - beta
    beta_tilde = beta * (1.0 - abar_s) / (1.0 - abar_t)
    c_x0 = beta * math.sqrt(abar_s) / (1.0 - abar_t)
    c_xt = (1.0 - abar_s) * math.sqrt(alpha) / (1.0 - abar_t)
    return dict(beta=beta, beta_tilde=beta_tilde, c_x0=c_x0, c_xt=c_xt)


def predict_x0(x_t, eps, abar_t):
    """Invert the forward process for x_0 given the predicted noise."""
    return (_f64(x_t) - math.sqrt(1.0 - abar_t) * _f64(eps)) / math.sqrt(abar_t)


def learned_log_variance(v, beta, log_beta_tilde):
    """log var = f log(beta) + (1 - f) log(beta_tilde), f = (v + 1) / 2."""
    f = (_f64(v) + 1.0) / 2.0
    return f * math.log(beta) + (1.0 - f) * log_beta_tilde


def ddpm_step(x_t, model_out, C, abar_t, abar_s, z, log_beta_tilde=None):
    """One ancestral step x_t -> x_s.

    model_out: [B, Cout, ...] with eps in channels [0, C) and, if Cout == 2C,
    the raw covariance values in [C, 2C).  z: noise of x's shape (ignored
    when abar_s == 1: the step into the clean latent adds no noise).
    log_beta_tilde overrides log(beta_tilde) (used at the last step, where
    beta_tilde is 0)."""
    x_t = _f64(x_t)
    mo = _f64(model_out)
    eps = mo[:, :C]
    q = ddpm_transition(abar_t, abar_s)
    x0 = predict_x0(x_t, eps, abar_t)
    mean = q["c_x0"] * x0 + q["c_xt"] * x_t
    if abar_s >= 1.0:
        return mean
    lbt = math.log(q["beta_tilde"]) if log_beta_tilde is None else log_beta_tilde
    if mo.shape[1] == 2 * C:
        logvar = learned_log_variance(mo[:, C:], q["beta"], lbt)
    else:
        logvar = lbt
    return mean + np.exp(0.5 * logvar) * _f64(z)


def ddpm_last_log_beta_tilde(levels):
    """Reading for the last step (into abar = 1, where beta_tilde = 0).
    levels: abar at the kept steps in sampling order.  Use log(beta_tilde) of
    the step before the last (levels[-2] -> levels[-1]), or log(beta) of the
    only step.  It never reaches a sample: that step adds no noise."""
    if len(levels) >= 2:
        q = ddpm_transition(levels[-2], levels[-1])
        return math.log(q["beta_tilde"])
    return math.log(1.0 - levels[-1])


# ---------------------------------------------------------------------------
# DPM-Solver++ (2M) in data prediction, variance-preserving parameters
# alpha = sqrt(abar), sigma = sqrt(1 - abar), lambda = log(alpha / sigma).

def vp_alpha_sigma(abar):
    return math.sqrt(abar), math.sqrt(1.0 - abar)


def log_snr_half(abar):
    """lambda = log(alpha / sigma); +inf for abar = 1."""
    if abar >= 1.0:
        return math.inf
    a, s = vp_alpha_sigma(abar)
    return math.log(a) - math.log(s)


def dpmpp_step(x_t, eps, abar_t, abar_s, x0_prev=None, abar_prev=None):
    """One DPM-Solver++ step from abar_t to abar_s (> abar_t).

    x0 = (x_t - sigma_t eps) / alpha_t.  First order:
        x_s = (sigma_s / sigma_t) x_t + alpha_s (1 - e^{-h}) x0,
        h = lambda_s - lambda_t.
    Second order (multistep, x0_prev from the level abar_prev < abar_t):
        r = (lambda_t - lambda_prev) / h,
        D = (1 + 1/(2r)) x0 - (1/(2r)) x0_prev, used in place of x0.
    abar_s = 1 (sigma_s = 0) gives x_s = x0 (first order only).
    Returns (x_s, x0)."""
    x_t = _f64(x_t)
    at, st = vp_alpha_sigma(abar_t)
    x0 = (x_t - st * _f64(eps)) / at
    if abar_s >= 1.0:
        return x0.copy(), x0
    as_, ss = vp_alpha_sigma(abar_s)
    h = log_snr_half(abar_s) - log_snr_half(abar_t)
    D = x0
    if x0_prev is not None:
        r = (log_snr_half(abar_t) - log_snr_half(abar_prev)) / h
        D = (1.0 + 0.5 / r) * x0 - (0.5 / r) * _f64(x0_prev)
    x_s = (ss / st) * x_t + as_ * (-math.expm1(-h)) * D
    return x_s, x0


# ---------------------------------------------------------------------------
# Rectified flow ([Goku] 2.3)

def rf_euler_step(x, v, t, t_next):
    """x(t_next) = x(t) + (t_next - t) v, v the predicted velocity toward data."""
    return _f64(x) + (t_next - t) * _f64(v)


def rf_uniform_times(S):
    return np.arange(S + 1, dtype=np.float64) / S


# ---------------------------------------------------------------------------
# Sampling loops around a model callable

def sample_ddpm(model, x_T, timesteps, noise, C, abar, model_input=None):
    """model(x, t_scalar) -> [B, Cout, ...].  timesteps: kept steps in
    sampling order; noise[k] is the z of step k.  model_input maps the fp64
    state to what the model is fed (e.g. a rounding to the model dtype)."""
    x = _f64(x_T).copy()
    abars = [float(abar[t]) for t in timesteps] + [1.0]
    last_lbt = ddpm_last_log_beta_tilde(abars[:-1]) if len(timesteps) else None
    for k, t in enumerate(timesteps):
        xin = x if model_input is None else model_input(x)
        mo = model(xin, float(t))
        lbt = last_lbt if abars[k + 1] >= 1.0 else None
        x = ddpm_step(x, mo, C, abars[k], abars[k + 1], noise[k], log_beta_tilde=lbt)
    return x


def sample_dpmpp_2m(model, x_T, timesteps, C, abar, model_input=None):
    """DPM-Solver++(2M) over the kept steps, ending at the clean latent."""
    x = _f64(x_T).copy()
    abars = [float(abar[t]) for t in timesteps] + [1.0]
    x0_prev = None
    for k, t in enumerate(timesteps):
        xin = x if model_input is None else model_input(x)
        eps = _f64(model(xin, float(t)))[:, :C]
        second = x0_prev is not None and abars[k + 1] < 1.0
        x, x0 = dpmpp_step(x, eps, abars[k], abars[k + 1],
                           x0_prev if second else None,
                           abars[k - 1] if second else None)
        x0_prev = x0
    return x


def sample_rf_euler(model, x_0, times, model_input=None):
    """Euler integration of the predicted velocity over times[0] < ... < times[S]."""
    x = _f64(x_0).copy()
    for k in range(len(times) - 1):
        xin = x if model_input is None else model_input(x)
        v = model(xin, float(times[k]))
        x = rf_euler_step(x, v, float(times[k]), float(times[k + 1]))
    return x
