"""Oracle pins for the per-token pieces: embeddings, LayerNorm, activations,
attention, QK normalisation and 3-D RoPE.

Pinned against torch fp64 library routines (the modules the itwiki
"확산 트랜스포머" Implementation section names), brute-force loops and
closed-form special cases.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle



@pytest.fixture(autouse=True)
def _float64_default():
    # fp64 torch modules for this module's tests only; restored afterwards so the
    # GPU tests collected in the same session keep torch's fp32 default.
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


# --- timestep sinusoid --------------------------------------------------------

def test_timestep_embedding_closed_forms():
    e = oracle.timestep_embedding(np.array([0.0, 1.0, 37.0, 999.0]))
    assert e.shape == (4, 256)
    # t = 0: cos part all ones, sin part all zeros.
    assert np.array_equal(e[0, :128], np.ones(128)) and np.array_equal(e[0, 128:], np.zeros(128))
    # each (cos, sin) pair lies on the unit circle.
    np.testing.assert_allclose(e[:, :128] ** 2 + e[:, 128:] ** 2, 1.0, rtol=0, atol=1e-15)
    # the first frequency is 1 rad per unit t; the last is 10^4^(-127/128).
    assert e[2, 0] == math.cos(37.0) and e[2, 128] == math.sin(37.0)
    f_last = math.atan2(e[1, 255], e[1, 127])
    assert abs(f_last - 10000.0 ** (-127 / 128)) < 1e-15


def test_timestep_embedding_shift_invariance():
    # <e(t), e(t')> = sum_k cos((t - t') f_k) depends only on t - t'.
    t = np.array([3.0, 10.0, 103.0, 110.0])
    e = oracle.timestep_embedding(t)
    a = e[0] @ e[1]
    b = e[2] @ e[3]
    assert abs(a - b) < 1e-9
    assert abs(e[0] @ e[0] - 128.0) < 1e-12


# --- 2-D sin-cos position embedding ------------------------------------------

def test_pos_embed_closed_forms():
    d, gh, gw = 32, 3, 5
    pe = oracle.pos_embed_2d(gh, gw, d)
    assert pe.shape == (gh * gw, d)
    dq = d // 4
    # origin: sin parts 0, cos parts 1.
    assert np.array_equal(pe[0], np.concatenate([np.zeros(dq), np.ones(dq), np.zeros(dq), np.ones(dq)]))
    grid = pe.reshape(gh, gw, d)
    # first half depends only on the row, second half only on the column.
    assert np.all(grid[:, :, :d // 2] == grid[:, :1, :d // 2])
    assert np.all(grid[:, :, d // 2:] == grid[:1, :, d // 2:])
    # frequency 0 of the row half is sin(i), cos(i); the last frequency is 10^4^(-(dq-1)/dq).
    for i in range(gh):
        assert grid[i, 0, 0] == math.sin(i) and grid[i, 0, dq] == math.cos(i)
    ang = math.atan2(grid[0, 1, 2 * dq + dq - 1], grid[0, 1, 3 * dq + dq - 1])
    assert abs(ang - 10000.0 ** (-(dq - 1) / dq)) < 1e-15
    np.testing.assert_allclose(pe[:, :dq] ** 2 + pe[:, dq:2 * dq] ** 2, 1.0, atol=1e-15)


# --- LayerNorm / modulate / activations ---------------------------------------

def test_layer_norm_matches_torch():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((3, 7, 48)) * 3 + 1
    ref = Fnn.layer_norm(torch.from_numpy(z), (48,), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.layer_norm(z, 1e-6), ref, rtol=1e-12, atol=1e-13)


def test_layer_norm_row_stats():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((4, 64)) * 0.01
    h = oracle.layer_norm(z, 1e-6)
    v = z.var(axis=1)
    np.testing.assert_allclose(h.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(h.var(axis=1), v / (v + 1e-6), rtol=1e-10)


def test_modulate_zero_is_layer_norm():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((2, 5, 16))
    h = oracle.layer_norm(z)
    zeros = np.zeros((2, 16))
    assert np.array_equal(oracle.modulate(h, zeros, zeros), h)
    sh = rng.standard_normal((2, 16))
    sc = rng.standard_normal((2, 16))
    ref = torch.from_numpy(h) * (1 + torch.from_numpy(sc)[:, None]) + torch.from_numpy(sh)[:, None]
    np.testing.assert_allclose(oracle.modulate(h, sh, sc), ref.numpy(), rtol=1e-15, atol=1e-15)


def test_gelu_silu_match_torch():
    z = np.linspace(-8, 8, 1001)
    np.testing.assert_allclose(oracle.gelu_tanh(z),
                               Fnn.gelu(torch.from_numpy(z), approximate="tanh").numpy(),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.silu(z), Fnn.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-13, atol=1e-15)


# --- attention ------------------------------------------------------------------

def _attention_loops(q, k, v):
    B, H, T, dh = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                s = [sum(q[b, h, i, e] * k[b, h, j, e] for e in range(dh)) / math.sqrt(dh)
                     for j in range(T)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = sum(w)
                for e in range(dh):
                    out[b, h, i, e] = sum(w[j] * v[b, h, j, e] for j in range(T)) / z
    return out


@pytest.mark.parametrize("T", [1, 2, 3, 5])
def test_attention_brute_force(T):
    rng = np.random.default_rng(T)
    q, k, v = (rng.standard_normal((2, 2, T, 6)) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v), _attention_loops(q, k, v),
                               rtol=1e-12, atol=1e-13)


def test_attention_query_chunking_is_exact():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 2, 37, 8)) for _ in range(3))
    a = oracle.attention(q, k, v, q_chunk=5)
    b = oracle.attention(q, k, v, q_chunk=4096)
    assert np.array_equal(a, b)


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 3, 1, 8))
    k = rng.standard_normal((1, 3, 1, 8))
    v = rng.standard_normal((1, 3, 1, 8))
    np.testing.assert_allclose(oracle.attention(q, k, v), v, rtol=0, atol=1e-15)   # T = 1 => o = v
    T = 9
    q = rng.standard_normal((1, 1, T, 8))
    k = np.repeat(rng.standard_normal((1, 1, 1, 8)), T, axis=2)                    # all keys equal
    v = rng.standard_normal((1, 1, T, 8))
    np.testing.assert_allclose(oracle.attention(q, k, v)[0, 0],
                               np.repeat(v[0, 0].mean(axis=0, keepdims=True), T, axis=0), atol=1e-14)


def test_attention_matches_torch_multihead():
    # nn.MultiheadAttention(d, heads) with the same packed q|k|v and output weights.
    rng = np.random.default_rng(7)
    B, T, d, H = 2, 11, 24, 3
    x = rng.standard_normal((B, T, d))
    w_in = rng.standard_normal((3 * d, d)) * 0.3
    b_in = rng.standard_normal(3 * d) * 0.3
    w_o = rng.standard_normal((d, d)) * 0.3
    b_o = rng.standard_normal(d) * 0.3
    mha = torch.nn.MultiheadAttention(d, H, batch_first=True)
    with torch.no_grad():
        mha.in_proj_weight.copy_(torch.from_numpy(w_in))
        mha.in_proj_bias.copy_(torch.from_numpy(b_in))
        mha.out_proj.weight.copy_(torch.from_numpy(w_o))
        mha.out_proj.bias.copy_(torch.from_numpy(b_o))
        xt = torch.from_numpy(x)
        ref = mha(xt, xt, xt, need_weights=False)[0].numpy()
    qkv = oracle.linear(x, w_in, b_in)
    q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(B, T, H, d // H).transpose(0, 2, 1, 3)
               for i in range(3))
    a = oracle.attention(q, k, v).transpose(0, 2, 1, 3).reshape(B, T, d)
    np.testing.assert_allclose(oracle.linear(a, w_o, b_o), ref, rtol=1e-11, atol=1e-12)


# --- QK normalisation and 3-D RoPE ---------------------------------------------

def test_qk_layernorm_matches_torch():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 2, 5, 72))
    ref = Fnn.layer_norm(torch.from_numpy(x), (72,), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.qk_layernorm(x), ref, rtol=1e-12, atol=1e-13)


def test_rope3d_as_complex_rotation():
    # Independent formulation: pairs as complex numbers times exp(i * pos * theta).
    gf, gh, gw, dh = 2, 3, 4, 12
    cos, sin = oracle.rope3d_tables(gf, gh, gw, dh)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 1, gf * gh * gw, dh))
    got = oracle.rope3d(x, cos, sin)
    da = dh // 3
    xc = x[..., 0::2] + 1j * x[..., 1::2]
    pos = np.array([(f, i, j) for f in range(gf) for i in range(gh) for j in range(gw)], float)
    theta = 10000.0 ** (-2.0 * np.arange(da // 2) / da)
    phase = np.concatenate([pos[:, a:a + 1] * theta[None] for a in range(3)], axis=1)
    rc = xc * np.exp(1j * phase)
    ref = np.empty_like(x)
    ref[..., 0::2] = rc.real
    ref[..., 1::2] = rc.imag
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_rope3d_invariants():
    gf, gh, gw, dh = 3, 4, 5, 72
    cos, sin = oracle.rope3d_tables(gf, gh, gw, dh)
    rng = np.random.default_rng(10)
    T = gf * gh * gw
    x = rng.standard_normal((1, 1, T, dh))
    y = oracle.rope3d(x, cos, sin)
    # rotation: pair norms preserved; position (0,0,0) is the identity.
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-12)
    assert np.array_equal(y[0, 0, 0], x[0, 0, 0])
    # relative position: <R(m) q, R(n) k> depends only on m - n (per axis).
    q = rng.standard_normal(dh)
    k = rng.standard_normal(dh)
    qs = np.repeat(q[None, None, None], T, axis=2)
    ks = np.repeat(k[None, None, None], T, axis=2)
    rq, rk = oracle.rope3d(qs, cos, sin)[0, 0], oracle.rope3d(ks, cos, sin)[0, 0]

    def tok(f, i, j):
        return (f * gh + i) * gw + j
    a = rq[tok(1, 2, 3)] @ rk[tok(0, 1, 1)]
    b = rq[tok(2, 3, 4)] @ rk[tok(1, 2, 2)]
    assert abs(a - b) < 1e-10
