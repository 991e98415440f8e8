"""Pins of the training-step oracle (oracle/train_oracle.py).

  * the torch restatement of the forward pass equals the numpy oracle;
  * autograd gradients of every parameter field equal central finite
    differences of the numpy loss (the KL term evaluated with the predicted
    mean frozen at the base point, which is what the stop-gradient means);
  * the posterior coefficients equal the product-of-Gaussians posterior of
    q(x_{t-1} | x_0) and q(x_t | x_{t-1}), derived independently;
  * the per-element KL and NLL equal numerical integration / scipy's normal
    log-density;
  * L_simple of a model whose output is a per-channel constant has a closed
    form; the gradient of the loss with respect to the output is
    2 (eps_theta - eps) / n on the eps channels and only the KL part on the
    covariance channels;
  * AdamW's first step is -lr g / (|g| + eps) (the bias corrections cancel).
"""
import math

import numpy as np
import pytest
import torch
from scipy import integrate, stats

import dit_inputs
from oracle import dit_oracle as D
from oracle import sampler_oracle as S
from oracle import train_oracle as TR


def tiny_cfg(**kw):
    cfg = dict(name="tiny train", C=2, Cout=4, F=1, H=4, W=4, p=2, pt=1, d=16, N=2, heads=2,
               mlp_hidden=32, num_classes=3, cond_dim=0, freq_dim=8, qk_norm=0, rope3d=0,
               dtype=dit_inputs.DTYPE_F32, ln_eps=1e-6, batch=3, cfg=False, scale=1.0, guided=2,
               conditioning=0, seed_idx=11)
    cfg.update(kw)
    return cfg


def batch(cfg, seed=5):
    rng = np.random.default_rng(seed)
    B = cfg["batch"]
    x0 = rng.standard_normal((B, cfg["C"], cfg["H"], cfg["W"]))
    eps = rng.standard_normal(x0.shape)
    t = np.array([0, 7, 900][:B])
    y = np.array([0, cfg["num_classes"], 2][:B])        # one null-label row
    return x0, y, t, eps


def test_torch_forward_equals_numpy_oracle():
    cfg = tiny_cfg()
    w = dit_inputs.make_weights(cfg, std=0.2)
    x0, y, t, eps = batch(cfg)
    x_t = TR.noised(x0, eps, t)
    ref = D.forward(cfg, w, x_t, t.astype(np.float64), y)
    P = {k: TR._t(w[k]) for k in TR.TRAIN_FIELDS}
    got = TR.forward_torch(cfg, P, x_t, t.astype(np.float64), y).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    ls_n, lv_n = TR.loss_terms(cfg, ref, x0, x_t, eps, t)
    ls_t, lv_t = TR.loss_torch(cfg, torch.as_tensor(ref), x0, x_t, eps, t)
    assert abs(float(ls_t) - ls_n) < 1e-12 and abs(float(lv_t) - lv_n) < 1e-12
    assert lv_n != 0.0


@pytest.mark.parametrize("Cout", [4, 2])
def test_gradients_match_finite_differences(Cout):
    cfg = tiny_cfg(Cout=Cout)
    w = dit_inputs.make_weights(cfg, std=0.2)
    x0, y, t, eps = batch(cfg)
    ls, lv, g = TR.gradients(cfg, w, x0, y, t, eps)
    x_t = TR.noised(x0, eps, t)
    base_out = D.forward(cfg, w, x_t, t.astype(np.float64), y)
    e_frozen = base_out[:, :cfg["C"]]

    def f(wp):
        a, b = TR.train_loss(cfg, wp, x0, y, t, eps, eps_for_mean=e_frozen)
        return a + b

    assert abs(f(w) - (ls + lv)) < 1e-12
    rng = np.random.default_rng(1)
    h = 1e-5
    for k in TR.TRAIN_FIELDS:
        flat = w[k].reshape(-1)
        idx = rng.choice(flat.size, size=min(4, flat.size), replace=False)
        if k == "y_table":
            idx = np.array([0, 3 * cfg["d"] + 1, 2 * cfg["d"] + 5])   # used rows only
        for i in idx:
            wp = {kk: vv.astype(np.float64) for kk, vv in w.items()}
            wm = {kk: vv.astype(np.float64) for kk, vv in w.items()}
            wp[k].reshape(-1)[i] += h
            wm[k].reshape(-1)[i] -= h
            fd = (f(wp) - f(wm)) / (2 * h)
            got = g[k].reshape(-1)[i]
            assert abs(fd - got) <= 1e-7 + 1e-5 * abs(got), (k, i, fd, got)
    # the unused class row gets no gradient
    assert np.all(g["y_table"][1] == 0.0)


def test_posterior_coefficients_from_product_of_gaussians():
    betas, abar = S.linear_beta_schedule()
    for t in (1, 2, 50, 999):
        r = TR.row_coefficients([t])[0]
        a_prev, alpha, beta = abar[t - 1], 1.0 - betas[t], betas[t]
        # q(x_{t-1} | x_0) = N(sqrt(a_prev) x_0, 1 - a_prev); q(x_t | x_{t-1}) =
        # N(sqrt(alpha) x_{t-1}, beta): precision-weighted combination
        prec = 1.0 / (1.0 - a_prev) + alpha / beta
        var = 1.0 / prec
        assert math.isclose(math.exp(r["lbt"]), var, rel_tol=1e-10)
        assert math.isclose(r["c_x0"], var * math.sqrt(a_prev) / (1.0 - a_prev), rel_tol=1e-10)
        assert math.isclose(r["c_xt"], var * math.sqrt(alpha) / beta, rel_tol=1e-10)
        assert math.isclose(r["beta"], beta, rel_tol=1e-12)
        assert math.isclose(r["sa"] ** 2 + r["sb"] ** 2, 1.0, rel_tol=1e-14)
    r0, r1 = TR.row_coefficients([0, 1])
    assert r0["lbt"] == r1["lbt"] and math.isclose(r0["c_x0"], 1.0, rel_tol=1e-14)
    assert r0["c_xt"] == 0.0


def test_kl_and_nll_against_integration():
    rng = np.random.default_rng(3)
    for _ in range(4):
        mu1, mu2 = rng.normal(size=2)
        lv1, lv2 = rng.normal(size=2) * 0.5
        s1, s2 = math.exp(0.5 * lv1), math.exp(0.5 * lv2)

        def integrand(x):
            lp = stats.norm.logpdf(x, mu1, s1)
            return math.exp(lp) * (lp - stats.norm.logpdf(x, mu2, s2))

        ref, _ = integrate.quad(integrand, mu1 - 12 * s1, mu1 + 12 * s1, epsabs=1e-13)
        assert abs(TR.kl_gauss(mu1, lv1, mu2, lv2) - ref) < 1e-9
        x = rng.normal()
        assert abs(TR.gauss_nll(x, mu2, lv2) + stats.norm.logpdf(x, mu2, s2)) < 1e-12


def test_constant_output_closed_form_and_output_gradient():
    cfg = tiny_cfg()
    x0, y, t, eps = batch(cfg)
    x_t = TR.noised(x0, eps, t)
    B, C = x0.shape[:2]
    rng = np.random.default_rng(9)
    const = rng.normal(size=2 * C)
    out = np.broadcast_to(const[None, :, None, None], (B, 2 * C, 4, 4)).copy()
    ls, _ = TR.loss_terms(cfg, out, x0, x_t, eps, t)
    want = np.mean([(const[c] - eps[b, c]) ** 2 for b in range(B) for c in range(C)])
    assert abs(ls - want) < 1e-12
    ot = torch.as_tensor(out).requires_grad_(True)
    a, b = TR.loss_torch(cfg, ot, x0, x_t, eps, t)
    ga = torch.autograd.grad(a, ot, retain_graph=True)[0].numpy()
    gb = torch.autograd.grad(b, ot)[0].numpy()
    n = eps.size
    np.testing.assert_allclose(ga[:, :C], 2.0 * (out[:, :C] - eps) / n, rtol=1e-12, atol=1e-15)
    assert np.all(ga[:, C:] == 0.0) and np.all(gb[:, :C] == 0.0)
    assert np.all(gb[:, C:] != 0.0)


def test_adamw_first_step_and_ema():
    rng = np.random.default_rng(4)
    p, g = rng.normal(size=50), rng.normal(size=50)
    z = np.zeros(50)
    pn, m, v = TR.adamw(p, g, z, z, 1, 1e-4, 0.9, 0.999, 1e-8, 0.0)
    np.testing.assert_allclose(pn, p - 1e-4 * g / (np.abs(g) + 1e-8), rtol=1e-12)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-12)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-12)
    pn, _, _ = TR.adamw(p, g, z, z, 1, 1e-4, 0.9, 0.999, 1e-8, 0.1)
    np.testing.assert_allclose(pn, p - 1e-4 * (g / (np.abs(g) + 1e-8) + 0.1 * p), rtol=1e-12)
    e = rng.normal(size=50)
    np.testing.assert_allclose(TR.ema(e, p, 0.9999), e + 1e-4 * (p - e), rtol=1e-12)
