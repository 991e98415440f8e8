"""fp64 reference implementation of the DiT denoiser forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every array is
converted to float64 on entry; no intermediate rounding is applied.  Library
primitives used as steps: numpy matmul, exp, tanh, sin, cos, sqrt.

Citations use the page keys listed in ``oracle/__init__.py``.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Patchify / unpatchify
# [DiT-wiki] Structure / Latent space and patchify: an I x I x C latent is cut
# into p x p patches, each linearly mapped to a d-dim token, T = (I/p)^2; the
# decoder emits p x p x 2C values per token that are put back in the spatial
# layout.  [Sora-obs] Architecture details / spacetime patch tokenisation:
# video latents are cut into (time x height x width) patches.
# Reading taken: raster token order over (frame, row, col); patch vector order
# (frame offset, row offset, col offset, channel) with channel fastest, at
# both ends.

def token_grid(F, H, W, p, pt=1):
    """(frames, rows, cols) of the token grid."""
    if F % pt or H % p or W % p:
        raise ValueError("latent extent not divisible by the patch size")
    return F // pt, H // p, W // p


def patchify(x, p, pt=1):
    """x: [B, C, H, W] or [B, C, F, H, W]  ->  P: [B, T, pt*p*p*C].

    P[b, (f*gh + i)*gw + j, ((a*p + py)*p + px)*C + c]
        = x[b, c, f*pt + a, i*p + py, j*p + px]
    """
    x = np.asarray(x)
    if x.ndim == 4:
        x = x[:, :, None]
    B, C, F, H, W = x.shape
    gf, gh, gw = token_grid(F, H, W, p, pt)
    v = x.reshape(B, C, gf, pt, gh, p, gw, p)
    # -> [B, gf, gh, gw, pt, py, px, C]
    v = v.transpose(0, 2, 4, 6, 3, 5, 7, 1)
    return np.ascontiguousarray(v.reshape(B, gf * gh * gw, pt * p * p * C))


def unpatchify(Y, Cout, F, H, W, p, pt=1, frames_axis=None):
    """Y: [B, T, pt*p*p*Cout] -> out [B, Cout, H, W] (F == 1 and
    frames_axis falsy) or [B, Cout, F, H, W].  Inverse index map of
    :func:`patchify`."""
    Y = np.asarray(Y)
    B = Y.shape[0]
    gf, gh, gw = token_grid(F, H, W, p, pt)
    v = Y.reshape(B, gf, gh, gw, pt, p, p, Cout)
    # -> [B, Cout, gf, pt, gh, py, gw, px]
    v = v.transpose(0, 7, 1, 4, 2, 5, 3, 6)
    out = np.ascontiguousarray(v.reshape(B, Cout, F, H, W))
    if frames_axis is None:
        frames_axis = F > 1
    return out if frames_axis else out[:, :, 0]


# ---------------------------------------------------------------------------
# Embeddings

def timestep_embedding(t, dim=256, max_period=10000.0):
    """[Sora-cvl] / [DiT-wiki] adaLN-Zero: c is the sum of a timestep
    embedding and a class embedding.  The pages give no formula; the reading
    taken is the 256-dim sinusoid [cos(t f_k) | sin(t f_k)] with
    f_k = max_period^(-k/(dim/2)), k = 0..dim/2-1, t used as given."""
    t = _f64(t).reshape(-1)
    half = dim // 2
    k = np.arange(half, dtype=np.float64)
    freqs = np.exp(-math.log(max_period) * k / half)
    args = t[:, None] * freqs[None, :]
    return np.concatenate([np.cos(args), np.sin(args)], axis=1)


def pos_embed_2d(gh, gw, d):
    """[DiT-wiki] Structure / Latent space and patchify, and [Sora-cvl]
    Method (patchify bullet): ViT-style fixed 2-D sine-cosine position
    embedding added to every token.  Reading taken: d/4 frequencies
    w_k = 10000^(-k/(d/4)); token (i, j) gets
    [sin(i w) | cos(i w) | sin(j w) | cos(j w)], row axis first."""
    if d % 4:
        raise ValueError("d must be a multiple of 4")
    dq = d // 4
    omega = 1.0 / 10000.0 ** (np.arange(dq, dtype=np.float64) / dq)
    ii, jj = np.meshgrid(np.arange(gh, dtype=np.float64),
                         np.arange(gw, dtype=np.float64), indexing="ij")
    i = ii.reshape(-1)[:, None] * omega[None, :]
    j = jj.reshape(-1)[:, None] * omega[None, :]
    return np.concatenate([np.sin(i), np.cos(i), np.sin(j), np.cos(j)], axis=1)


# ---------------------------------------------------------------------------
# Elementwise pieces

def layer_norm(z, eps=1e-6):
    """[DiT-wiki] adaLN-Zero: LN has no learnable affine parameters;
    Implementation / adaLN-Zero block: eps = 1e-6.  Biased variance over the
    last axis, eps inside the square root."""
    z = _f64(z)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + eps)


def modulate(h, shift, scale):
    """[DiT-wiki] adaLN-Zero equations: LN(x)(1 + gamma) + beta, the same
    (gamma, beta) for every token of a row.  h: [B, T, d]; shift, scale:
    [B, d]."""
    return h * (1.0 + scale[:, None, :]) + shift[:, None, :]


def silu(z):
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z):
    """[DiT-wiki] Implementation / adaLN-Zero block: the MLP uses the
    tanh-approximate GELU."""
    z = _f64(z)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def linear(x, w, b=None):
    """x @ w.T + b with w stored [out, in]."""
    y = _f64(x) @ _f64(w).T
    if b is not None:
        y = y + _f64(b)
    return y


# ---------------------------------------------------------------------------
# Attention
# [DiT-wiki] Implementation / adaLN-Zero block: nn.MultiheadAttention(d, heads),
# i.e. packed q|k|v projection with bias, per-head softmax(q k^T / sqrt(dh)) v,
# heads as contiguous dh-slices, output projection with bias.  [Goku] 2.2:
# full attention over every spacetime token.

def attention(q, k, v, q_chunk=2048):
    """q, k, v: [B, H, T, dh] -> [B, H, T, dh].  Queries are processed in
    chunks only to bound memory; each query row's arithmetic is unchanged."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hh, T, dh = q.shape
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(dh)
    for b in range(B):
        for h in range(Hh):
            kt = k[b, h].T
            for s in range(0, T, q_chunk):
                e = min(T, s + q_chunk)
                sc = (q[b, h, s:e] @ kt) * scale
                sc = sc - sc.max(axis=1, keepdims=True)
                pr = np.exp(sc)
                pr /= pr.sum(axis=1, keepdims=True)
                out[b, h, s:e] = pr @ v[b, h]
    return out


def qk_layernorm(x, eps=1e-6):
    """[Goku] 2.2 Q-K normalisation (the variant [DiT-wiki] MMDiT names is
    RMSNorm).  Reading taken: LayerNorm without affine over each head's
    dh-vector, eps 1e-6, applied to q and k before the rotary embedding."""
    return layer_norm(x, eps)


def rope3d_tables(gf, gh, gw, dh, base=10000.0):
    """cos/sin tables [T, dh/2] for the 3-D rotary embedding.

    [Goku] 2.2 3D RoPE over (time, height, width).  Reading taken: dh is
    split into three equal segments (frame, row, col) of size da = dh/3
    (even); pair k of a segment rotates by angle pos * base^(-2k/da), with
    integer positions; pairs are adjacent elements (x_2k, x_2k+1)."""
    if dh % 6:
        raise ValueError("3-D RoPE needs dh divisible by 6")
    da = dh // 3
    theta = base ** (-2.0 * np.arange(da // 2, dtype=np.float64) / da)
    ff, ii, jj = np.meshgrid(np.arange(gf, dtype=np.float64),
                             np.arange(gh, dtype=np.float64),
                             np.arange(gw, dtype=np.float64), indexing="ij")
    pos = [ff.reshape(-1), ii.reshape(-1), jj.reshape(-1)]
    ang = np.concatenate([p[:, None] * theta[None, :] for p in pos], axis=1)
    return np.cos(ang), np.sin(ang)


def rope3d(x, cos, sin):
    """x: [B, H, T, dh]; cos/sin: [T, dh/2].  Rotates pairs (x_2k, x_2k+1)."""
    x = _f64(x)
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


# ---------------------------------------------------------------------------
# Conditioning

def embed_condition(cfg, w, t, y=None, pooled=None):
    """c = t_emb + y_emb (+ pooled projection).

    [DiT-wiki] adaLN-Zero: c is the sum of the time embedding and the class
    embedding; [Sora-cvl] Method (CFG bullet): the null label is a class of its
    own; [DiT-wiki] MMDiT: a pooled vector and the time embedding enter through
    adaLN.  Readings taken: t_emb = Linear(d,d)(SiLU(Linear(256,d)(e(t))));
    the class table has num_classes + 1 rows, the last being the null label;
    the pooled vector enters through one Linear(cond_dim, d).
    Returns (e, t_emb, c)."""
    e = timestep_embedding(t, cfg["freq_dim"])
    temb = linear(silu(linear(e, w["t1_w"], w["t1_b"])), w["t2_w"], w["t2_b"])
    c = temb.copy()
    if cfg["num_classes"] > 0:
        y = np.asarray(y).astype(np.int64)
        if np.any(y < 0) or np.any(y > cfg["num_classes"]):
            raise ValueError("class label out of range")
        c = c + _f64(w["y_table"])[y]
    if cfg["cond_dim"] > 0:
        c = c + linear(pooled, w["pool_w"], w["pool_b"])
    return e, temb, c


def modulation(cfg, w, c):
    """[DiT-wiki] adaLN-Zero: (beta1, gamma1, alpha1, beta2, gamma2, alpha2)
    = MLP(c); Implementation: the MLP is SiLU followed by Linear(d, 6d).
    All blocks' rows and the final layer's (beta_f, gamma_f) rows are stacked
    in one weight.  Returns [B, (6N+2) d]."""
    return linear(silu(c), w["ada_w"], w["ada_b"])


# ---------------------------------------------------------------------------
# Transformer block

def block(cfg, wl, X, mod_l, rope=None):
    """One adaLN-Zero DiT block.

    [DiT-wiki] adaLN-Zero equations:
        x <- x + alpha1 * Attn(LN(x)(1 + gamma1) + beta1)
        x <- x + alpha2 * FFN(LN(x)(1 + gamma2) + beta2)
    with the six vectors in the order (beta1, gamma1, alpha1, beta2, gamma2,
    alpha2) (same page, Implementation / adaLN-Zero block: shift, scale, gate
    twice).  FFN = Linear(d, 4d), tanh-GELU, Linear(4d, d).

    wl: dict with qkv_w [3d,d], qkv_b, o_w, o_b, fc1_w, fc1_b, fc2_w, fc2_b.
    X: [B, T, d]; mod_l: [B, 6d].  Returns (X_out, o, f) where o and f are the
    attention and FFN branches before their gates.
    """
    X = _f64(X)
    B, T, d = X.shape
    Hh = cfg["heads"]
    dh = d // Hh
    eps = cfg["ln_eps"]
    sh1, sc1, g1, sh2, sc2, g2 = np.split(_f64(mod_l), 6, axis=1)

    h = modulate(layer_norm(X, eps), sh1, sc1)
    qkv = linear(h, wl["qkv_w"], wl["qkv_b"])
    q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(B, T, Hh, dh).transpose(0, 2, 1, 3)
               for i in range(3))
    if cfg["qk_norm"]:
        q, k = qk_layernorm(q, eps), qk_layernorm(k, eps)
    if cfg["rope3d"]:
        cos, sin = rope
        q, k = rope3d(q, cos, sin), rope3d(k, cos, sin)
    a = attention(q, k, v).transpose(0, 2, 1, 3).reshape(B, T, d)
    o = linear(a, wl["o_w"], wl["o_b"])
    X = X + g1[:, None, :] * o

    h = modulate(layer_norm(X, eps), sh2, sc2)
    f = linear(gelu_tanh(linear(h, wl["fc1_w"], wl["fc1_b"])), wl["fc2_w"], wl["fc2_b"])
    X = X + g2[:, None, :] * f
    return X, o, f


def block_weights(w, l):
    keys = ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b",
            "ln_p", "xq_w", "xq_b", "xkv_w", "xkv_b", "xo_w", "xo_b")
    return {k: w[k][l] for k in keys if k in w}


# ---------------------------------------------------------------------------
# The other two conditioning designs ([DiT-wiki] Conditioning methods table;
# [DiT-coin] DiT block description).  Both use standard pre-LN blocks without
# regressed modulation.  Readings taken: each LayerNorm has a learned affine
# written like the adaLN form with constants, LN(x)(1 + g) + b, with
# ln_p[l, i] = (b, g) for the i-th LN of block l; residual adds have no gate.

IN_CONTEXT, CROSS_ATTENTION = 1, 2


def _self_attention(cfg, wl, h):
    B, T, d = h.shape
    Hh = cfg["heads"]
    dh = d // Hh
    qkv = linear(h, wl["qkv_w"], wl["qkv_b"])
    q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(B, T, Hh, dh).transpose(0, 2, 1, 3)
               for i in range(3))
    a = attention(q, k, v).transpose(0, 2, 1, 3).reshape(B, T, d)
    return linear(a, wl["o_w"], wl["o_b"])


def cross_attention(cfg, wl, h, ctx):
    """Multi-head attention of the tokens h [B, T, d] over the context tokens
    ctx [B, S, d]: q = Linear(d, d)(h), [k | v] = Linear(d, 2d)(ctx), per head
    softmax(q k^T / sqrt(dh)) v, output Linear(d, d).  ([DiT-coin]: a
    multi-head cross-attention layer added after the self-attention layer.)"""
    B, T, d = h.shape
    S = ctx.shape[1]
    Hh = cfg["heads"]
    dh = d // Hh
    q = linear(h, wl["xq_w"], wl["xq_b"]).reshape(B, T, Hh, dh).transpose(0, 2, 1, 3)
    kv = linear(ctx, wl["xkv_w"], wl["xkv_b"])
    k = kv[..., :d].reshape(B, S, Hh, dh).transpose(0, 2, 1, 3)
    v = kv[..., d:].reshape(B, S, Hh, dh).transpose(0, 2, 1, 3)
    a = attention(q, k, v).transpose(0, 2, 1, 3).reshape(B, T, d)
    return linear(a, wl["xo_w"], wl["xo_b"])


def _ffn(wl, h):
    return linear(gelu_tanh(linear(h, wl["fc1_w"], wl["fc1_b"])), wl["fc2_w"], wl["fc2_b"])


def _affine_ln(X, lnp_i, eps):
    B = X.shape[0]
    b = np.broadcast_to(_f64(lnp_i[0]), (B, X.shape[-1]))
    g = np.broadcast_to(_f64(lnp_i[1]), (B, X.shape[-1]))
    return modulate(layer_norm(X, eps), b, g)


def block_in_context(cfg, wl, X):
    """[DiT-wiki] Conditioning methods, in-context row: the time and class
    embeddings ride along as two extra tokens of the sequence (like ViT's cls
    token) through standard blocks:
        x <- x + Attn(LN1(x)),  x <- x + FFN(LN2(x)).
    X: [B, T + 2, d].  Returns X."""
    X = _f64(X)
    eps = cfg["ln_eps"]
    X = X + _self_attention(cfg, wl, _affine_ln(X, wl["ln_p"][0], eps))
    return X + _ffn(wl, _affine_ln(X, wl["ln_p"][1], eps))


def block_cross_attention(cfg, wl, X, ctx):
    """[DiT-wiki] Conditioning methods, cross-attention row; [DiT-coin]: the
    time and class embeddings form a separate length-2 sequence, and each block
    gains a multi-head cross-attention layer after its self-attention:
        x <- x + Attn(LN1(x)),  x <- x + CrossAttn(LN2(x), ctx),
        x <- x + FFN(LN3(x)).
    X: [B, T, d]; ctx: [B, 2, d].  Returns X."""
    X = _f64(X)
    eps = cfg["ln_eps"]
    X = X + _self_attention(cfg, wl, _affine_ln(X, wl["ln_p"][0], eps))
    X = X + cross_attention(cfg, wl, _affine_ln(X, wl["ln_p"][1], eps), _f64(ctx))
    return X + _ffn(wl, _affine_ln(X, wl["ln_p"][2], eps))


def class_embedding(cfg, w, y):
    """Row y of the class table (num_classes + 1 rows, the last the null label)."""
    y = np.asarray(y).astype(np.int64)
    if np.any(y < 0) or np.any(y > cfg["num_classes"]):
        raise ValueError("class label out of range")
    return _f64(w["y_table"])[y]


# ---------------------------------------------------------------------------
# Whole denoiser

def forward(cfg, w, x_t, t, y=None, pooled=None, taps=None, blocks=None):
    """eps_theta(x_t, t, c) for a batch of rows.

    [Sora-cvl] Method and architecture; [DiT-wiki] Structure: patchify +
    linear embedding + position embedding, N adaLN-Zero blocks, final norm
    followed by a linear decoder to p x p x 2C per token, unpatchify.
    Reading taken for the final layer: LayerNorm (no affine), adaLN modulate
    with (beta_f, gamma_f) regressed from c, then Linear(d, p*p*Cout).
    Video ([Goku] 2.2): no additive position embedding; 3-D RoPE and QK
    normalisation inside attention.

    x_t: [B, C, H, W] or [B, C, F, H, W]; t: [B]; y: [B] ints in
    [0, num_classes] (num_classes is the null label); pooled: [B, cond_dim].
    ``taps`` (a dict) receives intermediate tensors.  ``blocks`` limits the
    number of blocks run (default: all N).
    Returns out [B, Cout, H, W] or [B, Cout, F, H, W].
    """
    x = _f64(x_t)
    video = x.ndim == 5
    x5 = x if video else x[:, :, None]
    B = x5.shape[0]
    C, F, H, W = cfg["C"], cfg["F"], cfg["H"], cfg["W"]
    p, pt, d, N = cfg["p"], cfg["pt"], cfg["d"], cfg["N"]
    if x5.shape[1:] != (C, F, H, W):
        raise ValueError(f"x_t shape {x.shape} does not match the config")
    gf, gh, gw = token_grid(F, H, W, p, pt)

    P = patchify(x5, p, pt)
    X = linear(P, w["pe_w"], w["pe_b"])
    rope = None
    if cfg["rope3d"]:
        rope = rope3d_tables(gf, gh, gw, d // cfg["heads"])
    else:
        if gf != 1:
            raise ValueError("2-D position embedding needs a single frame")
        X = X + pos_embed_2d(gh, gw, d)[None]

    cond = cfg.get("conditioning", 0)
    if cond in (IN_CONTEXT, CROSS_ATTENTION):
        return _forward_variant(cfg, w, X, t, y, taps, blocks, (F, H, W, video))

    e, temb, c = embed_condition(cfg, w, t, y, pooled)
    mod = modulation(cfg, w, c)
    if taps is not None:
        taps.update(e=e, temb=temb, c=c, mod=mod, X0=X.copy(), X=[], o=[], f=[])

    nb = N if blocks is None else blocks
    for l in range(nb):
        X, o, f = block(cfg, block_weights(w, l), X, mod[:, 6 * d * l:6 * d * (l + 1)], rope)
        if taps is not None:
            taps["X"].append(X.copy())
            taps["o"].append(o)
            taps["f"].append(f)

    shf = mod[:, 6 * d * N:6 * d * N + d]
    scf = mod[:, 6 * d * N + d:6 * d * N + 2 * d]
    Hf = modulate(layer_norm(X, cfg["ln_eps"]), shf, scf)
    Y = linear(Hf, w["out_w"], w["out_b"])
    out = unpatchify(Y, cfg["Cout"], F, H, W, p, pt, frames_axis=video)
    if taps is not None:
        taps.update(Hf=Hf, Y=Y, out=out)
    return out


def _forward_variant(cfg, w, X, t, y, taps, blocks, geom):
    """The in-context and cross-attention designs after the patch embedding X
    [B, T, d].  Readings taken: the time-embedding token is the timestep MLP's
    output and the class token is the class table's row, both without a
    position embedding; in-context appends them after the T patch tokens;
    the final layer is LN (learned affine) + Linear on the T patch tokens."""
    F, H, W, video = geom
    p, pt, N = cfg["p"], cfg["pt"], cfg["N"]
    if cfg["cond_dim"] > 0 or cfg["num_classes"] <= 0:
        raise ValueError("the in-context and cross-attention designs are class-conditional")
    T = X.shape[1]
    e = timestep_embedding(t, cfg["freq_dim"])
    temb = linear(silu(linear(e, w["t1_w"], w["t1_b"])), w["t2_w"], w["t2_b"])
    yemb = class_embedding(cfg, w, y)
    in_ctx = cfg["conditioning"] == IN_CONTEXT
    ctx = None
    if in_ctx:
        X = np.concatenate([X, temb[:, None, :], yemb[:, None, :]], axis=1)
    else:
        ctx = np.stack([temb, yemb], axis=1)
    if taps is not None:
        taps.update(e=e, temb=temb, yemb=yemb, X0=X.copy(), X=[])
    nb = N if blocks is None else blocks
    for l in range(nb):
        wl = block_weights(w, l)
        X = block_in_context(cfg, wl, X) if in_ctx else block_cross_attention(cfg, wl, X, ctx)
        if taps is not None:
            taps["X"].append(X.copy())
    Hf = _affine_ln(X[:, :T], w["final_ln"], cfg["ln_eps"])
    Y = linear(Hf, w["out_w"], w["out_b"])
    out = unpatchify(Y, cfg["Cout"], F, H, W, p, pt, frames_axis=video)
    if taps is not None:
        taps.update(Hf=Hf, Y=Y, out=out)
    return out


def cfg_combine(cond, uncond, s, guided):
    """[Sora-cvl] Method (classifier-free guidance bullet):
        eps_hat = eps(x, null) + s * (eps(x, c) - eps(x, null)).
    [DiT-wiki] Results / ImageNet notes: the official code guides only the
    first three output channels; guiding all channels is standard.  Channels
    >= ``guided`` are taken from the conditional output."""
    cond, uncond = _f64(cond), _f64(uncond)
    out = cond.copy()
    g = guided
    out[:, :g] = uncond[:, :g] + s * (cond[:, :g] - uncond[:, :g])
    return out


def cfg_forward(cfg, w, x_t, t, y, s, guided, taps=None, blocks=None):
    """Guided prediction for Bh rows: the trunk runs 2*Bh rows
    [(x_t, t, y) ; (x_t, t, null)], then :func:`cfg_combine`."""
    x = _f64(x_t)
    Bh = x.shape[0]
    t = _f64(t).reshape(-1)
    y = np.asarray(y).astype(np.int64).reshape(-1)
    x2 = np.concatenate([x, x], axis=0)
    t2 = np.concatenate([t, t])
    y2 = np.concatenate([y, np.full(Bh, cfg["num_classes"], dtype=np.int64)])
    both = forward(cfg, w, x2, t2, y2, taps=taps, blocks=blocks)
    return cfg_combine(both[:Bh], both[Bh:], s, guided)


# ---------------------------------------------------------------------------
# Packed sequences ([Goku] 2.2 Patch n' Pack: images and videos of different
# sizes share one sequence batch, each attending only to its own tokens).
# The packed forward is, by definition, every sequence's own forward; the
# packing is a layout of the same computation.

def forward_packed(cfg, w, latents, t, y=None, pooled=None):
    """latents: list of [C, H_i, W_i] (or [C, F_i, H_i, W_i]) arrays; t, y,
    pooled: one entry per sequence.  Returns the list of outputs
    [Cout, H_i, W_i] (or [Cout, F_i, H_i, W_i])."""
    outs = []
    for i, x in enumerate(latents):
        x = _f64(x)
        dims = x.shape[1:]
        F, H, W = (1,) + tuple(dims) if len(dims) == 2 else tuple(dims)
        ci = dict(cfg, F=F, H=H, W=W)
        yi = None if y is None else np.asarray(y)[i:i + 1]
        pi = None if pooled is None else _f64(pooled)[i:i + 1]
        outs.append(forward(ci, w, x[None], _f64(t)[i:i + 1], yi, pi)[0])
    return outs


# ---------------------------------------------------------------------------
# MMDiT ([DiT-wiki] MMDiT section): text tokens and image patch tokens are one
# sequence for attention, but each modality keeps its own weights for the
# normalisation, the QKV projection and the MLP (two transformers that meet
# only inside attention); the pooled vector and the time embedding still enter
# through adaLN modulation; Q and K get RMSNorm.
# Readings taken: each stream has its own adaLN-Zero modulation (six vectors
# per block from SiLU(c)) and output projection; the context tokens are a
# Linear(ctx_dim, d) of the given text embeddings, without position embedding,
# and come first in the joint sequence; QK RMSNorm is per head, eps 1e-6, with
# a learned scale 1 + g (g a dh-vector per stream for q and for k, written
# like the LayerNorm affines); the final layer reads the image stream only.

MMDIT = 3


def rms_norm(x, w, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = _f64(x)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * _f64(w)


def mmdit_block(cfg, wl, Xc, Xi, mod_c, mod_i):
    """One MMDiT block.  Xc: [B, L, d] context stream, Xi: [B, T, d] image
    stream; mod_c, mod_i: [B, 6d] (beta1, gamma1, alpha1, beta2, gamma2,
    alpha2) of each stream.  wl holds the image stream's qkv/o/fc1/fc2 weights,
    the context stream's c-prefixed ones, and qk_rms [4, dh] (g of q, k of the
    image stream, then of the context stream).  Returns (Xc, Xi)."""
    Xc, Xi = _f64(Xc), _f64(Xi)
    B, L, d = Xc.shape
    T = Xi.shape[1]
    Hh = cfg["heads"]
    dh = d // Hh
    eps = cfg["ln_eps"]
    mc = np.split(_f64(mod_c), 6, axis=1)
    mi = np.split(_f64(mod_i), 6, axis=1)
    rms = _f64(wl["qk_rms"])

    def heads_qkv(h, w, b, wq, wk):
        n = h.shape[1]
        qkv = linear(h, w, b)
        q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(B, n, Hh, dh).transpose(0, 2, 1, 3)
                   for i in range(3))
        return rms_norm(q, wq, eps), rms_norm(k, wk, eps), v

    qc, kc, vc = heads_qkv(modulate(layer_norm(Xc, eps), mc[0], mc[1]), wl["cqkv_w"],
                           wl["cqkv_b"], 1.0 + rms[2], 1.0 + rms[3])
    qi, ki, vi = heads_qkv(modulate(layer_norm(Xi, eps), mi[0], mi[1]), wl["qkv_w"],
                           wl["qkv_b"], 1.0 + rms[0], 1.0 + rms[1])
    a = attention(np.concatenate([qc, qi], axis=2), np.concatenate([kc, ki], axis=2),
                  np.concatenate([vc, vi], axis=2)).transpose(0, 2, 1, 3).reshape(B, L + T, d)
    Xc = Xc + mc[2][:, None, :] * linear(a[:, :L], wl["co_w"], wl["co_b"])
    Xi = Xi + mi[2][:, None, :] * linear(a[:, L:], wl["o_w"], wl["o_b"])

    def ffn(X, m, pre):
        h = modulate(layer_norm(X, eps), m[3], m[4])
        f = linear(gelu_tanh(linear(h, wl[pre + "fc1_w"], wl[pre + "fc1_b"])),
                   wl[pre + "fc2_w"], wl[pre + "fc2_b"])
        return X + m[5][:, None, :] * f

    return ffn(Xc, mc, "c"), ffn(Xi, mi, "")


def mmdit_block_weights(w, l):
    keys = ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b", "cqkv_w",
            "cqkv_b", "co_w", "co_b", "cfc1_w", "cfc1_b", "cfc2_w", "cfc2_b", "qk_rms")
    return {k: w[k][l] for k in keys}


def mmdit_forward(cfg, w, x_t, t, ctx, pooled, taps=None):
    """MMDiT denoiser: image latent x_t [B, C, H, W], time t [B], text
    embeddings ctx [B, L, ctx_dim], pooled vector [B, cond_dim].  Returns
    [B, Cout, H, W]."""
    x = _f64(x_t)
    B = x.shape[0]
    C, H, W, p, d, N = cfg["C"], cfg["H"], cfg["W"], cfg["p"], cfg["d"], cfg["N"]
    gf, gh, gw = token_grid(1, H, W, p, 1)
    Xi = linear(patchify(x[:, :, None], p, 1), w["pe_w"], w["pe_b"]) + pos_embed_2d(gh, gw, d)[None]
    Xc = linear(ctx, w["ctx_w"], w["ctx_b"])
    _, temb, c = embed_condition(dict(cfg, num_classes=0), w, t, None, pooled)
    mod_i = modulation(cfg, w, c)
    mod_c = linear(silu(c), w["cada_w"], w["cada_b"])
    if taps is not None:
        taps.update(c=c, mod=mod_i, cmod=mod_c, Xi0=Xi.copy(), Xc0=Xc.copy(), Xi=[], Xc=[])
    for l in range(N):
        Xc, Xi = mmdit_block(cfg, mmdit_block_weights(w, l), Xc, Xi,
                             mod_c[:, 6 * d * l:6 * d * (l + 1)], mod_i[:, 6 * d * l:6 * d * (l + 1)])
        if taps is not None:
            taps["Xi"].append(Xi.copy())
            taps["Xc"].append(Xc.copy())
    fb = 6 * d * N
    Hf = modulate(layer_norm(Xi, cfg["ln_eps"]), mod_i[:, fb:fb + d], mod_i[:, fb + d:fb + 2 * d])
    Y = linear(Hf, w["out_w"], w["out_b"])
    out = unpatchify(Y, cfg["Cout"], 1, H, W, p, 1)
    if taps is not None:
        taps.update(Y=Y, out=out)
    return out
