"""fp64 reference of one training step of the adaLN-Zero DiT.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * [Sora-cvl] Method / training objective bullet: the forward process
    x_t = sqrt(abar_t) x_0 + sqrt(1 - abar_t) eps with eps ~ N(0, I); the
    denoiser minimises L_simple = ||eps_theta(x_t) - eps||^2; the reverse
    covariance Sigma_theta is trained with the full KL term, the decoder
    emitting noise and covariance (2C channels).
  * [DiT-wiki] Results / training notes: AdamW, constant learning rate 1e-4,
    no weight decay, batch 256, an EMA of the weights with decay 0.9999.
Readings (the pages stop there):
  * schedule and learned variance as in ``sampler_oracle`` (1000 steps,
    linear beta 1e-4 .. 0.02; log var = f log beta + (1 - f) log beta_tilde,
    f = (v + 1) / 2; at t = 0, where beta_tilde is 0, log beta_tilde of
    t = 1 is used);
  * loss = mean over all B C H W latent elements of (eps_theta - eps)^2
    + mean over the same elements of the per-element KL term, in nats;
    the KL term sees the predicted mean through a stop-gradient, so it
    trains only the covariance channels;
  * KL term at t > 0: KL(q(x_{t-1} | x_t, x_0) || p_theta(x_{t-1} | x_t))
    between the two diagonal Gaussians; at t = 0 (no x_{t-1}): the Gaussian
    negative log-likelihood -log N(x_0; mu_theta, sigma^2);
  * with Cout = C (no covariance channels) the loss is L_simple alone;
  * AdamW with beta = (0.9, 0.999), eps 1e-8, bias correction, decoupled
    weight decay; the EMA is taken of the updated weights;
  * label dropout for guidance and the horizontal flip are choices of the
    caller's batch (y may hold the null label; x_0 is taken as given).

The gradient is computed by torch autograd (CPU, float64) over a torch
restatement of the forward pass; ``tests/test_oracle_train.py`` pins that
restatement to the numpy oracle and its gradient to central finite
differences of the numpy loss.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import dit_oracle as D
from . import sampler_oracle as S

# Parameters of the adaLN-Zero class-conditional image model, in the order of
# the flat parameter layout.
TRAIN_FIELDS = ("pe_w", "pe_b", "t1_w", "t1_b", "t2_w", "t2_b", "y_table", "ada_w", "ada_b",
                "qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b", "out_w",
                "out_b")

ADAMW = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, ema_decay=0.9999)


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------------------
# Forward process and per-row coefficients

def row_coefficients(t, train_steps=1000):
    """Per-row constants of the loss for integer steps t [B]: sqrt(abar_t),
    sqrt(1 - abar_t), beta_t, log beta_tilde_t (t = 0: that of t = 1), the
    posterior-mean weights c_x0, c_xt, and 1 / sqrt(abar_t)."""
    betas, abar = S.linear_beta_schedule(train_steps)
    t = np.asarray(t).astype(np.int64)
    if np.any(t < 0) or np.any(t >= train_steps):
        raise ValueError("t out of range")
    out = []
    for ti in t:
        a_t = abar[ti]
        a_prev = abar[ti - 1] if ti > 0 else 1.0
        q = S.ddpm_transition(a_t, a_prev)
        if ti > 0:
            lbt = math.log(q["beta_tilde"])
        else:
            lbt = math.log(S.ddpm_transition(abar[1], abar[0])["beta_tilde"])
        out.append(dict(sa=math.sqrt(a_t), sb=math.sqrt(1.0 - a_t), beta=q["beta"], lbt=lbt,
                        c_x0=q["c_x0"], c_xt=q["c_xt"], t=int(ti)))
    return out


def noised(x0, eps, t, train_steps=1000):
    """x_t = sqrt(abar_t) x_0 + sqrt(1 - abar_t) eps, per row."""
    x0, eps = D._f64(x0), D._f64(eps)
    rc = row_coefficients(t, train_steps)
    sa = np.array([r["sa"] for r in rc]).reshape(-1, *([1] * (x0.ndim - 1)))
    sb = np.array([r["sb"] for r in rc]).reshape(-1, *([1] * (x0.ndim - 1)))
    return sa * x0 + sb * eps


# ---------------------------------------------------------------------------
# Loss (numpy; also the target of the finite-difference pins)

def kl_gauss(mu1, logv1, mu2, logv2):
    """KL(N(mu1, e^logv1) || N(mu2, e^logv2)) elementwise."""
    return 0.5 * (-1.0 + logv2 - logv1 + np.exp(logv1 - logv2)
                  + (mu1 - mu2) ** 2 * np.exp(-logv2))


def gauss_nll(x, mu, logv):
    """-log N(x; mu, e^logv) elementwise."""
    return 0.5 * (math.log(2.0 * math.pi) + logv + (x - mu) ** 2 * np.exp(-logv))


def loss_terms(cfg, out, x0, x_t, eps, t, eps_for_mean=None):
    """(L_simple, L_vlb) for model output ``out`` [B, Cout, H, W].

    eps_for_mean: the eps prediction used inside mu_theta of the KL term
    (default: out's own eps channels).  Passing a fixed array evaluates the
    stop-gradient semantics: the KL term then varies only through the
    covariance channels."""
    out, x0, x_t, eps = D._f64(out), D._f64(x0), D._f64(x_t), D._f64(eps)
    C = cfg["C"]
    e_th = out[:, :C]
    n = e_th.size
    l_simple = float(((e_th - eps) ** 2).sum() / n)
    if out.shape[1] == C:
        return l_simple, 0.0
    e_m = e_th if eps_for_mean is None else D._f64(eps_for_mean)
    v = out[:, C:]
    total = 0.0
    for b, r in enumerate(row_coefficients(t)):
        x0h = (x_t[b] - r["sb"] * e_m[b]) / r["sa"]
        mu_th = r["c_x0"] * x0h + r["c_xt"] * x_t[b]
        logv = S.learned_log_variance(v[b], r["beta"], r["lbt"])
        if r["t"] > 0:
            mu_q = r["c_x0"] * x0[b] + r["c_xt"] * x_t[b]
            total += kl_gauss(mu_q, r["lbt"], mu_th, logv).sum()
        else:
            total += gauss_nll(x0[b], mu_th, logv).sum()
    return l_simple, float(total / n)


def train_loss(cfg, w, x0, y, t, eps, eps_for_mean=None):
    """Loss of one batch with the numpy forward: returns (L_simple, L_vlb)."""
    x_t = noised(x0, eps, t)
    out = D.forward(cfg, w, x_t, np.asarray(t, np.float64), y)
    return loss_terms(cfg, out, x0, x_t, eps, t, eps_for_mean)


# ---------------------------------------------------------------------------
# torch restatement of the adaLN-Zero forward pass (float64, autograd)

def _ln(z, eps):
    mu = z.mean(-1, keepdim=True)
    var = ((z - mu) ** 2).mean(-1, keepdim=True)
    return (z - mu) / torch.sqrt(var + eps)


def _gelu(z):
    return 0.5 * z * (1.0 + torch.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def _lin(x, w, b):
    return x @ w.T + b


def forward_torch(cfg, P, x_t, t, y):
    """The adaLN-Zero forward of ``dit_oracle.forward`` with torch ops on the
    parameter dict P (float64 tensors).  x_t: [B, C, H, W] numpy; t: [B];
    y: [B].  Returns the output [B, Cout, H, W] as a tensor."""
    C, H, W, p, d, N = cfg["C"], cfg["H"], cfg["W"], cfg["p"], cfg["d"], cfg["N"]
    Hh = cfg["heads"]
    dh = d // Hh
    eps = cfg["ln_eps"]
    gf, gh, gw = D.token_grid(1, H, W, p, 1)
    x = np.asarray(x_t, np.float64)
    B = x.shape[0]
    patches = _t(D.patchify(x[:, :, None], p, 1))                 # fixed input
    X = _lin(patches, P["pe_w"], P["pe_b"]) + _t(D.pos_embed_2d(gh, gw, d))[None]
    e = _t(D.timestep_embedding(np.asarray(t, np.float64), cfg["freq_dim"]))
    h1 = _lin(e, P["t1_w"], P["t1_b"])
    temb = _lin(h1 * torch.sigmoid(h1), P["t2_w"], P["t2_b"])
    c = temb + P["y_table"][torch.as_tensor(np.asarray(y).astype(np.int64))]
    mod = _lin(c * torch.sigmoid(c), P["ada_w"], P["ada_b"])
    T = X.shape[1]
    for l in range(N):
        m = mod[:, 6 * d * l:6 * d * (l + 1)]
        sh1, sc1, g1, sh2, sc2, g2 = (m[:, i * d:(i + 1) * d][:, None, :] for i in range(6))
        h = _ln(X, eps) * (1.0 + sc1) + sh1
        qkv = _lin(h, P["qkv_w"][l], P["qkv_b"][l])
        q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(B, T, Hh, dh).transpose(1, 2)
                   for i in range(3))
        s = (q @ k.transpose(-1, -2)) / math.sqrt(dh)
        a = torch.softmax(s, dim=-1) @ v
        a = a.transpose(1, 2).reshape(B, T, d)
        X = X + g1 * _lin(a, P["o_w"][l], P["o_b"][l])
        h = _ln(X, eps) * (1.0 + sc2) + sh2
        f = _lin(_gelu(_lin(h, P["fc1_w"][l], P["fc1_b"][l])), P["fc2_w"][l], P["fc2_b"][l])
        X = X + g2 * f
    fb = 6 * d * N
    Hf = _ln(X, eps) * (1.0 + mod[:, None, fb + d:fb + 2 * d]) + mod[:, None, fb:fb + d]
    Y = _lin(Hf, P["out_w"], P["out_b"])                           # [B, T, p p Cout]
    Cout = cfg["Cout"]
    Y = Y.reshape(B, gh, gw, p, p, Cout).permute(0, 5, 1, 3, 2, 4)
    return Y.reshape(B, Cout, H, W)


def loss_torch(cfg, out, x0, x_t, eps, t):
    """torch version of ``loss_terms`` with the stop-gradient on the mean."""
    C = cfg["C"]
    x0, x_t, eps = _t(x0), _t(x_t), _t(eps)
    e_th = out[:, :C]
    n = e_th.numel()
    l_simple = ((e_th - eps) ** 2).sum() / n
    if out.shape[1] == C:
        return l_simple, torch.zeros((), dtype=torch.float64)
    v = out[:, C:]
    e_m = e_th.detach()
    total = torch.zeros((), dtype=torch.float64)
    for b, r in enumerate(row_coefficients(t)):
        x0h = (x_t[b] - r["sb"] * e_m[b]) / r["sa"]
        mu_th = r["c_x0"] * x0h + r["c_xt"] * x_t[b]
        f = (v[b] + 1.0) / 2.0
        logv = f * math.log(r["beta"]) + (1.0 - f) * r["lbt"]
        if r["t"] > 0:
            mu_q = r["c_x0"] * x0[b] + r["c_xt"] * x_t[b]
            kl = 0.5 * (-1.0 + logv - r["lbt"] + torch.exp(r["lbt"] - logv)
                        + (mu_q - mu_th) ** 2 * torch.exp(-logv))
        else:
            kl = 0.5 * (math.log(2.0 * math.pi) + logv + (x0[b] - mu_th) ** 2 * torch.exp(-logv))
        total = total + kl.sum()
    return l_simple, total / n


def gradients(cfg, w, x0, y, t, eps):
    """Loss terms and d(L_simple + L_vlb)/d(parameter) for every field of
    TRAIN_FIELDS, at the parameter values w (numpy).  Returns
    (l_simple, l_vlb, grads dict of numpy arrays)."""
    P = {k: _t(w[k]).clone().requires_grad_(True) for k in TRAIN_FIELDS}
    x_t = noised(x0, eps, t)
    out = forward_torch(cfg, P, x_t, np.asarray(t, np.float64), y)
    ls, lv = loss_torch(cfg, out, x0, x_t, eps, t)
    (ls + lv).backward()
    return float(ls.detach()), float(lv.detach()), {k: P[k].grad.numpy().copy() for k in TRAIN_FIELDS}


# ---------------------------------------------------------------------------
# Optimizer

def adamw(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay):
    """One AdamW update at step number ``step`` (1-based).  Returns
    (p_new, m_new, v_new)."""
    p, g, m, v = D._f64(p), D._f64(g), D._f64(m), D._f64(v)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    p = p - lr * (mh / (np.sqrt(vh) + eps) + weight_decay * p)
    return p, m, v


def ema(e, p, decay):
    return decay * D._f64(e) + (1.0 - decay) * D._f64(p)


def train_step(cfg, w, state, x0, y, t, eps, step, hp=None):
    """One optimizer step.  w: the weights the forward uses (model dtype
    values); state: dict field -> dict(master, m, v, ema) (fp32 values).
    Returns (l_simple, l_vlb, grads, new_state)."""
    hp = dict(ADAMW, **(hp or {}))
    ls, lv, g = gradients(cfg, w, x0, y, t, eps)
    new = {}
    for k in TRAIN_FIELDS:
        s = state[k]
        p, m, v = adamw(s["master"], g[k], s["m"], s["v"], step, hp["lr"], hp["beta1"],
                        hp["beta2"], hp["eps"], hp["weight_decay"])
        new[k] = dict(master=p, m=m, v=v, ema=ema(s["ema"], p, hp["ema_decay"]))
    return ls, lv, g, new
