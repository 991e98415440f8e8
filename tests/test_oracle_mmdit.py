"""Oracle pins for the MMDiT model (itwiki "확산 트랜스포머", MMDiT section):
text and image streams with their own weights, one joint attention, pooled
vector + time adaLN, QK RMSNorm.

  * a block equals an independent torch composition (functional LayerNorm,
    Linear, scaled_dot_product_attention over the concatenated streams);
  * exchanging the two streams together with their weights exchanges the
    outputs (the joint attention does not depend on the concatenation order);
  * information flows both ways: each stream's output depends on the other
    stream's input;
  * zero gates make the block the identity for both streams (adaLN-Zero).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import dit_inputs
import oracle


@pytest.fixture(autouse=True)
def _float64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def small_cfg(**kw):
    cfg = dict(name="MMDiT small", C=4, Cout=4, F=1, H=16, W=16, p=2, pt=1, d=128, N=2, heads=2,
               mlp_hidden=512, num_classes=0, cond_dim=32, freq_dim=256, qk_norm=0, rope3d=0,
               dtype=dit_inputs.DTYPE_F32, ln_eps=1e-6, batch=2, cfg=False, scale=1.0, guided=4,
               conditioning=dit_inputs.COND_MMDIT, ctx_len=7, ctx_dim=64, seed_idx=9)
    cfg.update(kw)
    return cfg


def _block_inputs(cfg, seed):
    rng = np.random.default_rng(seed)
    B, d = 2, cfg["d"]
    Xc = rng.standard_normal((B, cfg["ctx_len"], d))
    Xi = rng.standard_normal((B, 64, d))
    mc = rng.standard_normal((B, 6 * d)) * 0.3
    mi = rng.standard_normal((B, 6 * d)) * 0.3
    return Xc, Xi, mc, mi


def _torch_block(cfg, wl, Xc, Xi, mc, mi):
    d, Hh = cfg["d"], cfg["heads"]
    dh = d // Hh
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    mc = [t(m) for m in np.split(mc, 6, axis=1)]
    mi = [t(m) for m in np.split(mi, 6, axis=1)]
    rms = t(wl["qk_rms"])

    def pre(X, m, i):
        return Fnn.layer_norm(X, (d,), eps=1e-6) * (1 + m[i + 1][:, None]) + m[i][:, None]

    def qkv(h, w, b, gq, gk):
        B, n, _ = h.shape
        y = Fnn.linear(h, t(w), t(b)).view(B, n, 3, Hh, dh).permute(2, 0, 3, 1, 4)
        rmsn = lambda z, g: z * torch.rsqrt(z.pow(2).mean(-1, keepdim=True) + 1e-6) * (1 + g)
        return rmsn(y[0], gq), rmsn(y[1], gk), y[2]

    Xc, Xi = t(Xc), t(Xi)
    L = Xc.shape[1]
    qc, kc, vc = qkv(pre(Xc, mc, 0), wl["cqkv_w"], wl["cqkv_b"], rms[2], rms[3])
    qi, ki, vi = qkv(pre(Xi, mi, 0), wl["qkv_w"], wl["qkv_b"], rms[0], rms[1])
    a = Fnn.scaled_dot_product_attention(torch.cat([qc, qi], 2), torch.cat([kc, ki], 2),
                                         torch.cat([vc, vi], 2))
    a = a.transpose(1, 2).reshape(Xc.shape[0], -1, d)
    Xc = Xc + mc[2][:, None] * Fnn.linear(a[:, :L], t(wl["co_w"]), t(wl["co_b"]))
    Xi = Xi + mi[2][:, None] * Fnn.linear(a[:, L:], t(wl["o_w"]), t(wl["o_b"]))

    def ffn(X, m, p):
        h = pre(X, m, 3)
        f = Fnn.linear(Fnn.gelu(Fnn.linear(h, t(wl[p + "fc1_w"]), t(wl[p + "fc1_b"])),
                                approximate="tanh"), t(wl[p + "fc2_w"]), t(wl[p + "fc2_b"]))
        return X + m[5][:, None] * f

    return ffn(Xc, mc, "c").numpy(), ffn(Xi, mi, "").numpy()


def test_block_matches_torch_composition():
    cfg = small_cfg()
    w = dit_inputs.make_weights(cfg)
    wl = oracle.mmdit_block_weights(w, 1)
    Xc, Xi, mc, mi = _block_inputs(cfg, 1)
    gc, gi = oracle.mmdit_block(cfg, wl, Xc, Xi, mc, mi)
    tc, ti = _torch_block(cfg, wl, Xc, Xi, mc, mi)
    assert np.allclose(gc, tc, rtol=1e-10, atol=1e-10)
    assert np.allclose(gi, ti, rtol=1e-10, atol=1e-10)


def test_stream_swap_symmetry():
    cfg = small_cfg()
    w = dit_inputs.make_weights(cfg)
    wl = oracle.mmdit_block_weights(w, 0)
    Xc, Xi, mc, mi = _block_inputs(cfg, 2)
    sw = dict(wl)
    for a, b in (("qkv", "cqkv"), ("o", "co"), ("fc1", "cfc1"), ("fc2", "cfc2")):
        for s in ("_w", "_b"):
            sw[a + s], sw[b + s] = wl[b + s], wl[a + s]
    sw["qk_rms"] = np.asarray(wl["qk_rms"])[[2, 3, 0, 1]]
    c1, i1 = oracle.mmdit_block(cfg, wl, Xc, Xi, mc, mi)
    c2, i2 = oracle.mmdit_block(cfg, sw, Xi, Xc, mi, mc)
    assert np.allclose(c1, i2, rtol=1e-11, atol=1e-11)
    assert np.allclose(i1, c2, rtol=1e-11, atol=1e-11)


def test_information_flows_both_ways_and_zero_gates_are_identity():
    cfg = small_cfg()
    w = dit_inputs.make_weights(cfg)
    wl = oracle.mmdit_block_weights(w, 0)
    Xc, Xi, mc, mi = _block_inputs(cfg, 3)
    rng = np.random.default_rng(30)
    c0, i0 = oracle.mmdit_block(cfg, wl, Xc, Xi, mc, mi)
    # (a constant shift or a scale of a whole token is removed by LayerNorm)
    c1, i1 = oracle.mmdit_block(cfg, wl, Xc + rng.standard_normal(Xc.shape), Xi, mc, mi)
    c2, i2 = oracle.mmdit_block(cfg, wl, Xc, Xi + rng.standard_normal(Xi.shape), mc, mi)
    assert np.abs(i1 - i0).max() > 1e-6       # image output depends on the text stream
    assert np.abs(c2 - c0).max() > 1e-6       # text output depends on the image stream
    d = cfg["d"]
    for m in (mc, mi):
        m[:, 2 * d:3 * d] = 0.0
        m[:, 5 * d:6 * d] = 0.0
    c3, i3 = oracle.mmdit_block(cfg, wl, Xc, Xi, mc, mi)
    assert np.array_equal(c3, Xc) and np.array_equal(i3, Xi)


def test_rms_norm_definition():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5, 64))
    g = rng.standard_normal(64)
    got = oracle.rms_norm(x, g)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6)
    assert np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


def test_forward_shapes_and_text_dependence():
    cfg = small_cfg()
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_mmdit_inputs(cfg)
    out = oracle.mmdit_forward(cfg, w, inp["x_t"], inp["t"], inp["ctx"], inp["pooled"])
    assert out.shape == (2, cfg["Cout"], 16, 16)
    out2 = oracle.mmdit_forward(cfg, w, inp["x_t"], inp["t"], inp["ctx"] * 0.5, inp["pooled"])
    assert np.abs(out2 - out).max() > 1e-6


def test_mac_count_matches_closed_form(monkeypatch):
    """Every product the oracle's MMDiT forward makes, counted as it runs,
    equals the closed-form count the throughput figures use."""
    from oracle import dit_oracle, flops
    cfg = small_cfg()
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_mmdit_inputs(cfg)
    macs = {"n": 0}
    lin0, att0 = dit_oracle.linear, dit_oracle.attention

    def lin(x, wt, b=None):
        x = np.asarray(x)
        macs["n"] += int(np.prod(x.shape[:-1])) * wt.shape[0] * wt.shape[1]
        return lin0(x, wt, b)

    def att(q, k, v, q_chunk=2048):
        B, H, Tq, dh = np.shape(q)
        macs["n"] += 2 * B * H * Tq * np.shape(k)[2] * dh
        return att0(q, k, v, q_chunk)

    monkeypatch.setattr(dit_oracle, "linear", lin)
    monkeypatch.setattr(dit_oracle, "attention", att)
    oracle.mmdit_forward(cfg, w, inp["x_t"], inp["t"], inp["ctx"], inp["pooled"])
    want = flops.gmac_for(cfg) * 1e9 * cfg["batch"]
    assert macs["n"] == round(want)
