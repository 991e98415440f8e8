"""Oracle pins for the in-context and cross-attention conditioning designs
(itwiki "확산 트랜스포머", Conditioning methods table; cointeeth DiT article,
DiT block description).

  * the multiply-accumulates the oracle's forward performs, counted at every
    matrix product, equal the closed form that reproduces the table's
    119.4 / 137.6 Gflops (pinned in test_oracle_shapes_flops.py), so no layer
    is missing or extra;
  * each block equals an independent torch.nn composition (LayerNorm with
    affine, MultiheadAttention for self- and cross-attention, Linear + GELU);
  * cross-attention over two equal context tokens is the output projection of
    their value, whatever the query;
  * an in-context block is equivariant to permutations of the patch tokens.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn as nn

import dit_inputs
import oracle
from oracle import dit_oracle, flops


@pytest.fixture(autouse=True)
def _float64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def _cfg(cond, **kw):
    base = dict(N=2, batch=2)
    base.update(kw)
    return dit_inputs.workload("dit_s8_f32", conditioning=cond, **base)


@pytest.mark.parametrize("cond,name", [(1, "in-context"), (2, "cross-attention"),
                                       (0, "adaLN-Zero")])
def test_forward_mac_count_matches_closed_form(cond, name, monkeypatch):
    cfg = _cfg(cond)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
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
    oracle.forward(cfg, w, inp["x_t"], inp["t"], inp["y"])
    T = dit_inputs.tokens(cfg)
    want = flops.gmac_per_image(cfg["N"], cfg["d"], T, cfg["p"], cfg["C"], cfg["Cout"],
                                conditioning=name) * 1e9 * cfg["batch"]
    assert macs["n"] == round(want)


def _ln(d, lnp_i):
    m = nn.LayerNorm(d, eps=1e-6)
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(1.0 + np.asarray(lnp_i[1], np.float64)))
        m.bias.copy_(torch.from_numpy(np.asarray(lnp_i[0], np.float64)))
    return m


def _mha(d, heads, w_in, b_in, w_out, b_out):
    m = nn.MultiheadAttention(d, heads, batch_first=True)
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.from_numpy(np.asarray(w_in, np.float64)))
        m.in_proj_bias.copy_(torch.from_numpy(np.asarray(b_in, np.float64)))
        m.out_proj.weight.copy_(torch.from_numpy(np.asarray(w_out, np.float64)))
        m.out_proj.bias.copy_(torch.from_numpy(np.asarray(b_out, np.float64)))
    return m


def _ffn(wl):
    f1 = nn.Linear(*np.shape(wl["fc1_w"])[::-1])
    f2 = nn.Linear(*np.shape(wl["fc2_w"])[::-1])
    with torch.no_grad():
        for m, k in ((f1, "fc1"), (f2, "fc2")):
            m.weight.copy_(torch.from_numpy(np.asarray(wl[k + "_w"], np.float64)))
            m.bias.copy_(torch.from_numpy(np.asarray(wl[k + "_b"], np.float64)))
    return nn.Sequential(f1, nn.GELU(approximate="tanh"), f2)


def test_in_context_block_matches_torch_composition():
    cfg = _cfg(1)
    w = dit_inputs.make_weights(cfg)
    wl = oracle.block_weights(w, 1)
    d, heads = cfg["d"], cfg["heads"]
    rng = np.random.default_rng(5)
    X = rng.standard_normal((2, dit_inputs.tokens(cfg) + 2, d))
    got = oracle.block_in_context(cfg, wl, X)
    ln1, ln2 = _ln(d, wl["ln_p"][0]), _ln(d, wl["ln_p"][1])
    sa = _mha(d, heads, wl["qkv_w"], wl["qkv_b"], wl["o_w"], wl["o_b"])
    ff = _ffn(wl)
    with torch.no_grad():
        x = torch.from_numpy(X)
        h = ln1(x)
        x = x + sa(h, h, h, need_weights=False)[0]
        x = x + ff(ln2(x))
    assert np.allclose(got, x.numpy(), rtol=1e-10, atol=1e-10)


def test_cross_attention_block_matches_torch_composition():
    cfg = _cfg(2)
    w = dit_inputs.make_weights(cfg)
    wl = oracle.block_weights(w, 0)
    d, heads = cfg["d"], cfg["heads"]
    rng = np.random.default_rng(6)
    X = rng.standard_normal((2, dit_inputs.tokens(cfg), d))
    ctx = rng.standard_normal((2, 2, d))
    got = oracle.block_cross_attention(cfg, wl, X, ctx)
    lns = [_ln(d, wl["ln_p"][i]) for i in range(3)]
    sa = _mha(d, heads, wl["qkv_w"], wl["qkv_b"], wl["o_w"], wl["o_b"])
    ca = _mha(d, heads, np.concatenate([wl["xq_w"], wl["xkv_w"]]),
              np.concatenate([wl["xq_b"], wl["xkv_b"]]), wl["xo_w"], wl["xo_b"])
    ff = _ffn(wl)
    with torch.no_grad():
        x = torch.from_numpy(X)
        c = torch.from_numpy(ctx)
        h = lns[0](x)
        x = x + sa(h, h, h, need_weights=False)[0]
        x = x + ca(lns[1](x), c, c, need_weights=False)[0]
        x = x + ff(lns[2](x))
    assert np.allclose(got, x.numpy(), rtol=1e-10, atol=1e-10)


def test_cross_attention_over_equal_context_is_value_projection():
    cfg = _cfg(2)
    w = dit_inputs.make_weights(cfg)
    wl = oracle.block_weights(w, 1)
    d = cfg["d"]
    rng = np.random.default_rng(7)
    h = rng.standard_normal((3, 5, d))
    c0 = rng.standard_normal((3, 1, d))
    out = oracle.cross_attention(cfg, wl, h, np.concatenate([c0, c0], axis=1))
    v = c0[:, 0] @ np.asarray(wl["xkv_w"][d:], np.float64).T + wl["xkv_b"][d:]
    want = v @ np.asarray(wl["xo_w"], np.float64).T + wl["xo_b"]
    assert np.allclose(out, np.broadcast_to(want[:, None, :], out.shape), rtol=1e-12, atol=1e-12)


def test_in_context_block_is_equivariant_to_patch_token_order():
    cfg = _cfg(1)
    w = dit_inputs.make_weights(cfg)
    wl = oracle.block_weights(w, 0)
    T = dit_inputs.tokens(cfg)
    rng = np.random.default_rng(8)
    X = rng.standard_normal((2, T + 2, cfg["d"]))
    perm = np.concatenate([rng.permutation(T), [T, T + 1]])
    a = oracle.block_in_context(cfg, wl, X)[:, perm]
    b = oracle.block_in_context(cfg, wl, X[:, perm])
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)


def test_in_context_tokens_are_the_time_and_class_embeddings():
    cfg = _cfg(1)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    taps = {}
    oracle.forward(cfg, w, inp["x_t"], inp["t"], inp["y"], taps=taps, blocks=0)
    T = dit_inputs.tokens(cfg)
    _, temb, _ = oracle.embed_condition(cfg, w, inp["t"], inp["y"])
    assert np.array_equal(taps["X0"][:, T], temb)
    assert np.array_equal(taps["X0"][:, T + 1], np.asarray(w["y_table"], np.float64)[inp["y"]])
    assert taps["X0"].shape[1] == T + 2


def test_variants_reject_pooled_or_classless_configs():
    cfg = _cfg(2)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    with pytest.raises(ValueError):
        oracle.forward(dict(cfg, num_classes=0), w, inp["x_t"], inp["t"], None)
    with pytest.raises(ValueError):
        oracle.forward(dict(cfg, cond_dim=8), w, inp["x_t"], inp["t"], inp["y"],
                       pooled=np.zeros((2, 8)))
