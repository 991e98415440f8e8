"""Oracle pins for the DiT block, the whole denoiser and the CFG combine.

* An independent torch.nn fp64 composition of the block structure named by
  itwiki "확산 트랜스포머", Implementation / adaLN-Zero block (LayerNorm without
  affine at eps 1e-6, MultiheadAttention, Linear-GELU(tanh)-Linear, SiLU +
  Linear regressing six vectors, shift/scale/gate twice) and of the whole
  denoiser (Conv2d/Conv3d patch embedding, fold/rearrange unpatchify).
* The zero-initialised modulation makes a block the identity, bit for bit
  (same page, adaLN-Zero section and the identity check in Implementation).
* Guidance invariants from cv-learn "Sora / DiT", Method (CFG bullet).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn as nn
import torch.nn.functional as Fnn
from einops import rearrange

import dit_inputs
import oracle



@pytest.fixture(autouse=True)
def _float64_default():
    # fp64 torch modules for this module's tests only; restored afterwards so the
    # GPU tests collected in the same session keep torch's fp32 default.
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def tiny_image_cfg(**kw):
    cfg = dict(name="tiny", C=4, Cout=8, F=1, H=8, W=8, p=2, pt=1, d=24, N=2, heads=3,
               mlp_hidden=96, num_classes=10, cond_dim=0, freq_dim=256, qk_norm=0, rope3d=0,
               dtype=dit_inputs.DTYPE_F32, ln_eps=1e-6, batch=3, cfg=False, scale=1.5, guided=4,
               seed_idx=99)
    cfg.update(kw)
    return cfg


def tiny_video_cfg(**kw):
    cfg = dict(name="tinyvid", C=4, Cout=4, F=2, H=4, W=6, p=2, pt=1, d=36, N=2, heads=2,
               mlp_hidden=144, num_classes=0, cond_dim=16, freq_dim=256, qk_norm=1, rope3d=1,
               dtype=dit_inputs.DTYPE_F32, ln_eps=1e-6, batch=2, cfg=False, scale=1.0, guided=4,
               seed_idx=98)
    cfg.update(kw)
    return cfg


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# --- independent torch composition --------------------------------------------

class RefBlock(nn.Module):
    """adaLN-Zero block assembled from torch.nn modules."""

    def __init__(self, cfg, wl):
        super().__init__()
        d, H = cfg["d"], cfg["heads"]
        self.cfg = cfg
        self.ln = nn.LayerNorm(d, elementwise_affine=False, eps=1e-6)
        self.mha = nn.MultiheadAttention(d, H, batch_first=True)
        self.fc1 = nn.Linear(d, cfg["mlp_hidden"])
        self.fc2 = nn.Linear(cfg["mlp_hidden"], d)
        self.act = nn.GELU(approximate="tanh")
        with torch.no_grad():
            self.mha.in_proj_weight.copy_(_t(wl["qkv_w"]))
            self.mha.in_proj_bias.copy_(_t(wl["qkv_b"]))
            self.mha.out_proj.weight.copy_(_t(wl["o_w"]))
            self.mha.out_proj.bias.copy_(_t(wl["o_b"]))
            self.fc1.weight.copy_(_t(wl["fc1_w"]))
            self.fc1.bias.copy_(_t(wl["fc1_b"]))
            self.fc2.weight.copy_(_t(wl["fc2_w"]))
            self.fc2.bias.copy_(_t(wl["fc2_b"]))

    def attn(self, h, rope):
        cfg = self.cfg
        if not (cfg["qk_norm"] or cfg["rope3d"]):
            return self.mha(h, h, h, need_weights=False)[0]
        B, T, d = h.shape
        H = cfg["heads"]
        dh = d // H
        q, k, v = Fnn.linear(h, self.mha.in_proj_weight, self.mha.in_proj_bias).chunk(3, dim=-1)
        q, k, v = (z.reshape(B, T, H, dh).transpose(1, 2) for z in (q, k, v))
        if cfg["qk_norm"]:
            q = Fnn.layer_norm(q, (dh,), eps=1e-6)
            k = Fnn.layer_norm(k, (dh,), eps=1e-6)
        if cfg["rope3d"]:
            q, k = rope(q), rope(k)
        a = Fnn.scaled_dot_product_attention(q, k, v)
        return self.mha.out_proj(a.transpose(1, 2).reshape(B, T, d))

    def forward(self, x, m, rope=None):
        shift1, scale1, gate1, shift2, scale2, gate2 = m.chunk(6, dim=1)
        h = self.ln(x) * (1 + scale1[:, None]) + shift1[:, None]
        o = self.attn(h, rope)
        x = x + gate1[:, None] * o
        h = self.ln(x) * (1 + scale2[:, None]) + shift2[:, None]
        f = self.fc2(self.act(self.fc1(h)))
        return x + gate2[:, None] * f, o, f


def complex_rope(cfg):
    gf, gh, gw = cfg["F"] // cfg["pt"], cfg["H"] // cfg["p"], cfg["W"] // cfg["p"]
    dh = cfg["d"] // cfg["heads"]
    da = dh // 3
    theta = 10000.0 ** (-2.0 * torch.arange(da // 2) / da)
    f, i, j = torch.meshgrid(torch.arange(gf), torch.arange(gh), torch.arange(gw), indexing="ij")
    ang = torch.cat([p.reshape(-1, 1).double() * theta for p in (f, i, j)], dim=1)
    rot = torch.polar(torch.ones_like(ang), ang)

    def apply(x):
        xc = torch.view_as_complex(x.reshape(*x.shape[:-1], -1, 2).contiguous())
        return torch.view_as_real(xc * rot).reshape(x.shape)
    return apply


def torch_forward(cfg, w, x_t, t, y=None, pooled=None):
    d, N, p, pt, C, Cout = cfg["d"], cfg["N"], cfg["p"], cfg["pt"], cfg["C"], cfg["Cout"]
    x = _t(x_t)
    video = x.ndim == 5
    kin = pt * p * p * C
    if video:
        conv = nn.Conv3d(C, d, kernel_size=(pt, p, p), stride=(pt, p, p))
        wc = _t(w["pe_w"]).reshape(d, pt, p, p, C).permute(0, 4, 1, 2, 3)
    else:
        conv = nn.Conv2d(C, d, kernel_size=p, stride=p)
        wc = _t(w["pe_w"]).reshape(d, p, p, C).permute(0, 3, 1, 2)
    with torch.no_grad():
        conv.weight.copy_(wc)
        conv.bias.copy_(_t(w["pe_b"]))
    X = conv(x).flatten(2).transpose(1, 2)
    gf, gh, gw = cfg["F"] // pt, cfg["H"] // p, cfg["W"] // p
    rope = None
    if cfg["rope3d"]:
        rope = complex_rope(cfg)
    else:
        X = X + _t(oracle.pos_embed_2d(gh, gw, d))[None]

    tmlp = nn.Sequential(nn.Linear(cfg["freq_dim"], d), nn.SiLU(), nn.Linear(d, d))
    with torch.no_grad():
        tmlp[0].weight.copy_(_t(w["t1_w"])); tmlp[0].bias.copy_(_t(w["t1_b"]))
        tmlp[2].weight.copy_(_t(w["t2_w"])); tmlp[2].bias.copy_(_t(w["t2_b"]))
    c = tmlp(_t(oracle.timestep_embedding(t, cfg["freq_dim"])))
    if cfg["num_classes"]:
        emb = nn.Embedding(cfg["num_classes"] + 1, d)
        with torch.no_grad():
            emb.weight.copy_(_t(w["y_table"]))
        c = c + emb(torch.from_numpy(np.asarray(y, dtype=np.int64)))
    if cfg["cond_dim"]:
        c = c + Fnn.linear(_t(pooled), _t(w["pool_w"]), _t(w["pool_b"]))
    ada = nn.Sequential(nn.SiLU(), nn.Linear(d, (6 * N + 2) * d))
    with torch.no_grad():
        ada[1].weight.copy_(_t(w["ada_w"])); ada[1].bias.copy_(_t(w["ada_b"]))
    m = ada(c)
    for l in range(N):
        blk = RefBlock(cfg, {k: w[k][l] for k in ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w",
                                                   "fc1_b", "fc2_w", "fc2_b")})
        X, _, _ = blk(X, m[:, 6 * d * l:6 * d * (l + 1)], rope)
    shift, scale = m[:, 6 * d * N:].chunk(2, dim=1)
    Hf = Fnn.layer_norm(X, (d,), eps=1e-6) * (1 + scale[:, None]) + shift[:, None]
    Y = Fnn.linear(Hf, _t(w["out_w"]), _t(w["out_b"]))
    if video:
        return rearrange(Y, "b (f h w) (a py px c) -> b c (f a) (h py) (w px)",
                         f=gf, h=gh, w=gw, a=pt, py=p, px=p, c=Cout).detach().numpy()
    cols = rearrange(Y, "b l (py px c) -> b (c py px) l", py=p, px=p, c=Cout)
    return Fnn.fold(cols, (cfg["H"], cfg["W"]), kernel_size=p, stride=p).detach().numpy()


# --- block ------------------------------------------------------------------------

@pytest.mark.parametrize("video", [False, True])
def test_block_matches_torch_composition(video):
    cfg = tiny_video_cfg() if video else tiny_image_cfg()
    w = dit_inputs.make_weights(cfg, seed=11, std=0.2)
    rng = np.random.default_rng(12)
    B = 2
    T = dit_inputs.tokens(cfg)
    X = rng.standard_normal((B, T, cfg["d"]))
    mod = rng.standard_normal((B, 6 * cfg["d"])) * 0.5
    wl = {k: w[k][0] for k in ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")}
    rope = None
    if video:
        gf, gh, gw = oracle.token_grid(cfg["F"], cfg["H"], cfg["W"], cfg["p"], cfg["pt"])
        rope = oracle.rope3d_tables(gf, gh, gw, cfg["d"] // cfg["heads"])
    Xo, o, f = oracle.block(cfg, wl, X, mod, rope)
    ref = RefBlock(cfg, wl)
    with torch.no_grad():
        rX, ro, rf = ref(_t(X), _t(mod), complex_rope(cfg) if video else None)
    np.testing.assert_allclose(o, ro.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f, rf.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Xo, rX.numpy(), rtol=1e-10, atol=1e-12)


def test_zero_gate_block_is_identity():
    # adaLN-Zero: zero-initialised last Linear of the modulation => alpha = 0
    # => every block returns its input bit for bit.  DiT-S width, 256 tokens.
    cfg = tiny_image_cfg(d=384, heads=6, mlp_hidden=1536, H=32, W=32, p=2, N=1)
    w = dit_inputs.zero_gates(cfg, dit_inputs.make_weights(cfg, seed=13))
    rng = np.random.default_rng(14)
    X = rng.standard_normal((2, 256, 384))
    c = rng.standard_normal((2, 384))
    mod = oracle.modulation(cfg, w, c)[:, :6 * 384]
    assert np.all(mod == 0.0)
    Xo, _, _ = oracle.block(cfg, {k: w[k][0] for k in ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w",
                                                       "fc1_b", "fc2_w", "fc2_b")}, X, mod)
    assert np.array_equal(Xo, X)


def test_unit_gate_is_plain_adaln():
    # Gate rows W = 0, b = 1 => alpha = 1: x + Attn(...), x + FFN(...)  (adaLN row of the table).
    cfg = tiny_image_cfg()
    w = dit_inputs.set_gate_bias(cfg, dit_inputs.make_weights(cfg, seed=15, std=0.2), 1.0,
                                 zero_rows=True)
    rng = np.random.default_rng(16)
    X = rng.standard_normal((2, 16, cfg["d"]))
    c = rng.standard_normal((2, cfg["d"]))
    mod = oracle.modulation(cfg, w, c)[:, :6 * cfg["d"]]
    d = cfg["d"]
    assert np.all(mod[:, 2 * d:3 * d] == 1.0) and np.all(mod[:, 5 * d:6 * d] == 1.0)
    wl = {k: w[k][0] for k in ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")}
    Xo, o, f = oracle.block(cfg, wl, X, mod)
    X1 = X + o
    np.testing.assert_allclose(Xo, X1 + f, rtol=1e-13, atol=1e-13)


def test_block_token_permutation_equivariance():
    cfg = tiny_image_cfg()
    w = dit_inputs.make_weights(cfg, seed=17, std=0.2)
    rng = np.random.default_rng(18)
    X = rng.standard_normal((2, 16, cfg["d"]))
    mod = rng.standard_normal((2, 6 * cfg["d"])) * 0.5
    wl = {k: w[k][1] for k in ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")}
    perm = rng.permutation(16)
    a, _, _ = oracle.block(cfg, wl, X[:, perm], mod)
    b, _, _ = oracle.block(cfg, wl, X, mod)
    np.testing.assert_allclose(a, b[:, perm], rtol=1e-12, atol=1e-13)


# --- whole forward ------------------------------------------------------------------

@pytest.mark.parametrize("video", [False, True])
def test_forward_matches_torch_composition(video):
    cfg = tiny_video_cfg() if video else tiny_image_cfg()
    w = dit_inputs.make_weights(cfg, seed=21, std=0.2)
    inp = dit_inputs.make_inputs(cfg, seed=22)
    if not video:
        inp["y"][-1] = cfg["num_classes"]          # one null-label row
    got = oracle.forward(cfg, w, inp["x_t"], inp["t"], inp["y"], inp["pooled"])
    with torch.no_grad():
        ref = torch_forward(cfg, w, inp["x_t"], inp["t"], inp["y"], inp["pooled"])
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-11)


def test_forward_batch_row_independence():
    cfg = tiny_image_cfg()
    w = dit_inputs.make_weights(cfg, seed=23, std=0.2)
    inp = dit_inputs.make_inputs(cfg, seed=24, batch=4)
    full = oracle.forward(cfg, w, inp["x_t"], inp["t"], inp["y"])
    for i in range(4):
        one = oracle.forward(cfg, w, inp["x_t"][i:i + 1], inp["t"][i:i + 1], inp["y"][i:i + 1])
        np.testing.assert_allclose(one[0], full[i], rtol=1e-12, atol=1e-13)


def test_null_label_uses_last_table_row():
    cfg = tiny_image_cfg()
    w = dit_inputs.make_weights(cfg, seed=25, std=0.2)
    t = np.array([5.0, 5.0])
    _, _, c = oracle.embed_condition(cfg, w, t, np.array([3, cfg["num_classes"]]))
    np.testing.assert_allclose(c[1] - c[0], w["y_table"][-1].astype(float) - w["y_table"][3],
                               rtol=1e-12, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.embed_condition(cfg, w, t, np.array([0, cfg["num_classes"] + 1]))


# --- classifier-free guidance ---------------------------------------------------------

def test_cfg_combine_invariants():
    rng = np.random.default_rng(30)
    cond = rng.standard_normal((3, 8, 4, 4))
    unc = rng.standard_normal((3, 8, 4, 4))
    assert np.array_equal(oracle.cfg_combine(cond, unc, 0.0, 8), unc)      # s = 0 => eps(null)
    one = oracle.cfg_combine(cond, unc, 1.0, 8)                             # s = 1 => eps(c)
    # u + (c - u) rounds twice; each rounding is at most half an ulp of max(|c|, |u|, |c - u|).
    big = np.maximum(np.maximum(np.abs(cond), np.abs(unc)), np.abs(cond - unc))
    assert np.all(np.abs(one - cond) <= np.spacing(big))
    a, b, c = (oracle.cfg_combine(cond, unc, s, 8) for s in (0.0, 1.5, 4.0))
    np.testing.assert_allclose(b, a + 1.5 * (oracle.cfg_combine(cond, unc, 1.0, 8) - a),
                               rtol=1e-12, atol=1e-12)                      # affine in s
    np.testing.assert_allclose(c, a + 4.0 * (cond - unc), rtol=1e-12, atol=1e-12)
    g3 = oracle.cfg_combine(cond, unc, 1.5, 3)                              # first 3 channels only
    assert np.array_equal(g3[:, 3:], cond[:, 3:])
    assert np.array_equal(g3[:, :3], b[:, :3])


def test_cfg_forward_pairs_rows():
    cfg = tiny_image_cfg()
    w = dit_inputs.make_weights(cfg, seed=31, std=0.2)
    inp = dit_inputs.make_inputs(cfg, seed=32, batch=2)
    got = oracle.cfg_forward(cfg, w, inp["x_t"], inp["t"], inp["y"], 1.5, 4)
    cond = oracle.forward(cfg, w, inp["x_t"], inp["t"], inp["y"])
    unc = oracle.forward(cfg, w, inp["x_t"], inp["t"], np.full(2, cfg["num_classes"]))
    np.testing.assert_allclose(got[:, :4], unc[:, :4] + 1.5 * (cond[:, :4] - unc[:, :4]),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got[:, 4:], cond[:, 4:], rtol=1e-12, atol=1e-13)
