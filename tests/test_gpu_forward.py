"""GPU parity of the whole forward pass (dit_forward / dit_cfg_forward through
the C ABI) against the fp64 oracle.

Bounds: relative L2 <= 1e-4 for the fp32 workload, <= 2e-2 for bf16, for the
output and for every tap (c, mod, embedded tokens, residual stream after each
block, decoder output).  Because the output is weakly sensitive to the blocks,
blocks are also checked teacher-forced (given the same input and modulation)
on their pre-gate attention and FFN branches, with normal and amplified gates.
Full-size workloads are checked on sampled rows the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import dit_inputs
import oracle
from tests.parity import (BF16_TOL, F32_TOL, compare_taps, device_inputs, log, np_,
                          oracle_taps, rel_l2)

pytestmark = pytest.mark.gpu
dmod = pytest.importorskip("diffusion_transformer_denoiser_amd")

BLOCK_KEYS = ("qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dmod.load()
    yield
    torch.cuda.synchronize()


def _model(cfg, w):
    return dmod.DiT(cfg, w, "cuda")


# --- small workloads, whole forward, every tap ----------------------------------------------

def test_fp32_dit_s8_full():
    cfg = dit_inputs.workload("dit_s8_f32")
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    inp["y"] = np.array([inp["y"][0], cfg["num_classes"]], dtype=np.int32)   # one null row
    log(f"fp32 DiT-S/8 B=2 labels={inp['y']}")
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    taps = m.make_taps(2)
    out = np_(m.forward(x, t, y, taps=taps))
    ref, otaps = oracle_taps(cfg, w, inp)
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert err <= F32_TOL
    compare_taps(cfg, taps, otaps, F32_TOL, "fp32 S/8")


def test_bf16_dit_b4_full():
    cfg = dit_inputs.workload("dit_b4_bf16")
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    log("bf16 DiT-B/4 B=32")
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    taps = m.make_taps(32)
    out = np_(m.forward(x, t, y, taps=taps))
    ref, otaps = oracle_taps(cfg, w, inp)
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert err <= BF16_TOL
    compare_taps(cfg, taps, otaps, BF16_TOL, "bf16 B/4")


def test_bf16_xl2_cfg_reduced_depth():
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=3, batch=3)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    log("bf16 DiT-XL/2 256 CFG, N=3, Bh=3")
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    taps = m.make_taps(6)
    out = np_(m.cfg_forward(x, t, y, 1.5, 4, taps=taps))
    ref, otaps = oracle_taps(cfg, w, inp, cfg_mode=True, scale=1.5, guided=4)
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert err <= BF16_TOL
    compare_taps(cfg, taps, otaps, BF16_TOL, "XL/2 CFG")


# --- guidance, determinism, row independence --------------------------------------------------

def test_cfg_invariants_and_determinism():
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=2, batch=3)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    null = torch.full_like(y, cfg["num_classes"])
    f_cond = np_(m.forward(x, t, y))
    f_null = np_(m.forward(x, t, null))
    s0 = np_(m.cfg_forward(x, t, y, 0.0, 8))
    s1 = np_(m.cfg_forward(x, t, y, 1.0, 8))
    g3 = np_(m.cfg_forward(x, t, y, 1.5, 3))
    g3b = np_(m.cfg_forward(x, t, y, 1.5, 3))
    log("CFG s=0 / s=1 / g=3 / determinism")
    assert np.array_equal(s0, f_null)                       # s = 0 -> eps(null), bit for bit
    big = np.maximum(np.abs(f_cond), np.abs(f_null))
    assert np.all(np.abs(s1 - f_cond) <= np.spacing(big.astype(np.float32)) * 2)   # s = 1 -> eps(c)
    assert np.array_equal(g3[:, 3:], f_cond[:, 3:])         # unguided channels = conditional row
    ref = f_null[:, :3] + 1.5 * (f_cond[:, :3] - f_null[:, :3])
    assert np.abs(g3[:, :3] - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
    assert np.array_equal(g3, g3b)                          # deterministic


def test_batch_row_independence():
    cfg = dit_inputs.workload("dit_b4_bf16", N=2, batch=5)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    full = np_(m.forward(x, t, y))
    for i in (0, 3):
        one = np_(m.forward(x[i:i + 1].contiguous(), t[i:i + 1].contiguous(),
                            y[i:i + 1].contiguous()))
        assert np.array_equal(one[0], full[i])


@pytest.mark.parametrize("name", ["dit_s8_f32", "dit_b4_bf16"])
def test_out_of_range_label_poisons_only_its_row(name):
    # Labels are not read on the host: a label outside [0, num_classes] makes
    # that row's conditioning, and so its output, NaN; the other rows are
    # unaffected (bitwise equal to a run with a valid label there).  The fp32
    # and bf16 models take different conditioning kernels.
    cfg = dit_inputs.workload(name, N=2, batch=3)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg, batch=3)
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    good = np_(m.forward(x, t, y))
    for bad in (cfg["num_classes"] + 1, -1):
        yb = y.clone()
        yb[1] = bad
        out = np_(m.forward(x, t, yb))
        log(f"{name} label {bad}: row 1 all-NaN {np.isnan(out[1]).all()}")
        assert np.isnan(out[1]).all()
        assert np.array_equal(out[0], good[0]) and np.array_equal(out[2], good[2])


def test_bf16_single_row_matches_oracle():
    cfg = dit_inputs.workload("dit_b4_bf16", N=3, batch=1)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg, batch=1)
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    out = np_(m.forward(x, t, y))
    ref, _ = oracle_taps(cfg, w, inp)
    err = rel_l2(out, ref)
    log(f"bf16 B/4 depth 3, one row: rel-L2 {err:.2e}")
    assert err <= BF16_TOL


# --- teacher-forced blocks --------------------------------------------------------------------

def _block_case(cfg, w, layer, B, rows, gate_bias=None, seed=7):
    rng = np.random.default_rng(seed)
    T = dit_inputs.tokens(cfg)
    d = cfg["d"]
    X = rng.standard_normal((B, T, d)).astype(np.float32)
    c = rng.standard_normal((B, d))
    mod = oracle.modulation(cfg, w, c)[:, 6 * d * layer:6 * d * (layer + 1)].astype(np.float32)
    if gate_bias is not None:
        mod[:, 2 * d:3 * d] += gate_bias
        mod[:, 5 * d:6 * d] += gate_bias
    m = _model(cfg, w)
    Xd = torch.from_numpy(X.reshape(B * T, d)).cuda()
    md = torch.from_numpy(mod).cuda()
    ob = torch.empty_like(Xd)
    fb = torch.empty_like(Xd)
    Xo = np_(m.block_forward(layer, Xd, md, o_branch=ob, f_branch=fb)).reshape(B, T, d)
    ob, fb = np_(ob).reshape(B, T, d), np_(fb).reshape(B, T, d)
    wl = {k: w[k][layer] for k in BLOCK_KEYS}
    rope = None
    if cfg["rope3d"]:
        gf, gh, gw = oracle.token_grid(cfg["F"], cfg["H"], cfg["W"], cfg["p"], cfg["pt"])
        rope = oracle.rope3d_tables(gf, gh, gw, d // cfg["heads"])
    rXo, ro, rf = oracle.block(cfg, wl, X[rows], mod[rows], rope)
    res = dict(o=rel_l2(ob[rows], ro), f=rel_l2(fb[rows], rf),
               dx=rel_l2(Xo[rows] - X[rows], rXo - X[rows]), x=rel_l2(Xo[rows], rXo))
    return res


@pytest.mark.parametrize("name,depth,layer,B,rows", [
    ("dit_xl2_256_cfg", 2, 1, 64, [0, 31, 32, 63]), ("dit_xl2_512_cfg", 1, 0, 16, [0, 9]),
    ("dit_b4_bf16", 12, 11, 32, [0, 31])])
def test_block_teacher_forced_full_shape(name, depth, layer, B, rows):
    # Full row count and token count of each workload; depth trimmed to the layer tested.
    cfg = dit_inputs.workload(name, N=depth)
    w = dit_inputs.make_weights(cfg)
    for gb in (None, 1.0):
        res = _block_case(cfg, w, layer, B, rows, gate_bias=gb)
        log(f"block {name} l={layer} B={B} rows={rows} gate+={gb}: " +
            ", ".join(f"{k}={v:.2e}" for k, v in res.items()))
        assert all(v <= BF16_TOL for v in res.values()), res


def test_zero_gate_block_is_identity_on_gpu():
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=1)
    w = dit_inputs.zero_gates(cfg, dit_inputs.make_weights(cfg))
    d, T, B = cfg["d"], 256, 2
    rng = np.random.default_rng(3)
    X = rng.standard_normal((B * T, d)).astype(np.float32)
    mod = oracle.modulation(cfg, w, rng.standard_normal((B, d)))[:, :6 * d].astype(np.float32)
    assert np.all(mod == 0)
    m = _model(cfg, w)
    out = np_(m.block_forward(0, torch.from_numpy(X).cuda(), torch.from_numpy(mod).cuda()))
    assert np.array_equal(out, X)


# --- full-size workloads, sampled rows ------------------------------------------------------------

def _full_size_sampled(name, sample_rows, blocks, oracle_rows=()):
    cfg = dit_inputs.workload(name)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    Bh = cfg["batch"]
    rows = 2 * Bh
    T, d, N = dit_inputs.tokens(cfg), cfg["d"], cfg["N"]
    log(f"full-size {name}: trunk rows={rows} T={T}")
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    taps = m.make_taps(rows)
    out = np_(m.cfg_forward(x, t, y, cfg["scale"], cfg["guided"], taps=taps))
    torch.cuda.synchronize()
    # conditioning and embedding: every row
    x2 = np.concatenate([inp["x_t"], inp["x_t"]])
    t2 = np.concatenate([inp["t"], inp["t"]])
    y2 = np.concatenate([inp["y"], np.full(Bh, cfg["num_classes"], np.int32)])
    _, _, c = oracle.embed_condition(cfg, w, t2, y2)
    mod = oracle.modulation(cfg, w, c)
    P = oracle.patchify(x2, cfg["p"])
    X0 = oracle.linear(P, w["pe_w"], w["pe_b"]) + oracle.pos_embed_2d(cfg["H"] // cfg["p"],
                                                                      cfg["W"] // cfg["p"], d)[None]
    res = {"c": rel_l2(np_(taps["c"]), c), "mod": rel_l2(np_(taps["mod"]), mod),
           "x_embed": rel_l2(np_(taps["x_embed"]), X0.reshape(-1, d))}
    xb = taps["x_blocks"]
    for l in blocks:
        prev = taps["x_embed"] if l == 0 else xb[l - 1]
        Xin = np_(prev.reshape(rows, T, d)[sample_rows])
        Xg = np_(xb[l].reshape(rows, T, d)[sample_rows])
        rX, _, _ = oracle.block(cfg, {k: w[k][l] for k in BLOCK_KEYS}, Xin,
                                mod[sample_rows, 6 * d * l:6 * d * (l + 1)])
        res[f"dx_block{l}"] = rel_l2(Xg - Xin, rX - Xin)
    XN = np_(xb[N - 1].reshape(rows, T, d)[sample_rows])
    fb = 6 * d * N
    Hf = oracle.modulate(oracle.layer_norm(XN), mod[sample_rows, fb:fb + d],
                         mod[sample_rows, fb + d:fb + 2 * d])
    Yref = oracle.linear(Hf, w["out_w"], w["out_b"])
    Yg = np_(taps["y_final"]).reshape(rows, T, -1)
    res["y_final"] = rel_l2(Yg[sample_rows], Yref)
    # guidance + unpatchify of the GPU's own decoder output, for every row
    Yall = Yg.astype(np.float64)
    ep = oracle.unpatchify(Yall, cfg["Cout"], 1, cfg["H"], cfg["W"], cfg["p"])
    ref_out = oracle.cfg_combine(ep[:Bh], ep[Bh:], cfg["scale"], cfg["guided"])
    res["cfg_out"] = rel_l2(out, ref_out)
    # The call bench.py times: no taps.  Same kernels, same launch sequence,
    # so the output equals the tapped call's bit for bit; guided rows of it
    # against the oracle's own guided forward of those rows.
    out_nt = np_(m.cfg_forward(x, t, y, cfg["scale"], cfg["guided"]))
    torch.cuda.synchronize()
    assert np.array_equal(out_nt, out), "untapped forward differs from the tapped one"
    # The forward writes every workspace byte before it reads it: with the
    # workspace filled with NaN bytes first, the output is unchanged bit for bit.
    m.workspace(rows).fill_(0xFF)
    out_p = np_(m.cfg_forward(x, t, y, cfg["scale"], cfg["guided"]))
    torch.cuda.synchronize()
    assert np.array_equal(out_p, out_nt), "forward read workspace bytes it had not written"
    if oracle_rows:
        r = list(oracle_rows)
        ref_g = oracle.cfg_forward(cfg, w, inp["x_t"][r], inp["t"][r], inp["y"][r], cfg["scale"],
                                   cfg["guided"])
        res["cfg_forward_untapped"] = rel_l2(out_nt[r], ref_g)
    log(f"  {name} sampled rel-L2: " + ", ".join(f"{k}={v:.2e}" for k, v in res.items()))
    assert res["cfg_out"] <= 1e-6
    assert all(v <= BF16_TOL for v in res.values()), res


def test_full_size_xl2_256_cfg_sampled():
    _full_size_sampled("dit_xl2_256_cfg", [0, 33, 63], blocks=[0, 13, 27], oracle_rows=(0, 31))


def test_full_size_xl2_512_cfg_sampled():
    _full_size_sampled("dit_xl2_512_cfg", [2, 11], blocks=[0, 27])


# --- spacetime video workload ---------------------------------------------------------------------

def test_video_reduced_frames_full_forward():
    cfg = dit_inputs.workload("video_xl_spacetime", F=2, N=2)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    log("video F=2 (T=3120) N=2")
    m = _model(cfg, w)
    x, t, _, pooled = device_inputs(cfg, inp)
    taps = m.make_taps(1)
    out = np_(m.forward(x, t, None, pooled, taps=taps))
    ref, otaps = oracle_taps(cfg, w, inp)
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert out.shape == ref.shape and err <= BF16_TOL
    compare_taps(cfg, taps, otaps, BF16_TOL, "video F=2")


def test_video_full_length_attention_sampled_queries():
    # T = 24960 tokens, 16 heads of 72: the full-length attention of the video workload.
    B, H, T, dh = 1, 16, 24960, 72
    rng = np.random.default_rng(11)
    q, k, v = (dit_inputs.bf16_round(rng.standard_normal((B, H, T, dh)).astype(np.float32))
               for _ in range(3))
    packed = np.concatenate([a.transpose(0, 2, 1, 3).reshape(B, T, H * dh) for a in (q, k, v)],
                            axis=2)
    o = dmod.attention(torch.from_numpy(packed).to(torch.bfloat16).cuda(), H)
    torch.cuda.synchronize()
    qs = np.array([0, 1, 127, 128, 12345, 24895, 24959])
    errs = []
    for h in (0, 9, 15):
        sub = oracle.attention(q[:, h:h + 1, qs], k[:, h:h + 1], v[:, h:h + 1])[0, 0]
        got = np_(o[0, qs, h * dh:(h + 1) * dh])
        errs.append(rel_l2(got, sub))
    log(f"video attention sampled rel-L2 {max(errs):.2e}")
    assert max(errs) <= 1e-2


def test_video_block_teacher_forced_full_length():
    cfg = dit_inputs.workload("video_xl_spacetime", N=1)
    w = dit_inputs.make_weights(cfg)
    d, T = cfg["d"], dit_inputs.tokens(cfg)
    rng = np.random.default_rng(12)
    X = rng.standard_normal((T, d)).astype(np.float32)
    mod = (rng.standard_normal((1, 6 * d)) * 0.2).astype(np.float32)
    m = _model(cfg, w)
    ob = torch.empty(T, d, device="cuda")
    fb = torch.empty(T, d, device="cuda")
    Xo = np_(m.block_forward(0, torch.from_numpy(X).cuda(), torch.from_numpy(mod).cuda(),
                             o_branch=ob, f_branch=fb))
    # oracle on a query subset: q/k/v of every token are needed, outputs only for the sample.
    wl = {kk: w[kk][0] for kk in BLOCK_KEYS}
    sh1, sc1 = mod[:, :d], mod[:, d:2 * d]
    h = oracle.modulate(oracle.layer_norm(X[None]), sh1, sc1)
    qkv = oracle.linear(h, wl["qkv_w"], wl["qkv_b"])
    Hh, dh = cfg["heads"], d // cfg["heads"]
    q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(1, T, Hh, dh).transpose(0, 2, 1, 3)
               for i in range(3))
    q, k = oracle.qk_layernorm(q), oracle.qk_layernorm(k)
    cos, sin = oracle.rope3d_tables(16, 30, 52, dh)
    q, k = oracle.rope3d(q, cos, sin), oracle.rope3d(k, cos, sin)
    qs = np.array([0, 777, 12480, 24959])
    a = oracle.attention(q[:, :, qs], k, v).transpose(0, 2, 1, 3).reshape(1, len(qs), d)
    o_ref = oracle.linear(a, wl["o_w"], wl["o_b"])[0]
    # the rest of the block is token-local: the residual after the attention
    # branch, the FFN branch and the block output of the sampled tokens
    g1, sh2, sc2, g2 = mod[:, 2 * d:3 * d], mod[:, 3 * d:4 * d], mod[:, 4 * d:5 * d], mod[:, 5 * d:]
    X1 = X[qs].astype(np.float64) + g1 * o_ref
    h2 = oracle.modulate(oracle.layer_norm(X1[None]), sh2, sc2)
    f_ref = oracle.linear(oracle.gelu_tanh(oracle.linear(h2, wl["fc1_w"], wl["fc1_b"])),
                          wl["fc2_w"], wl["fc2_b"])[0]
    X_ref = X1 + g2 * f_ref
    err = rel_l2(np_(ob)[qs], o_ref)
    err_f = rel_l2(np_(fb)[qs], f_ref)
    err_x = rel_l2(Xo[qs] - X[qs], X_ref - X[qs])
    log(f"video full-length block sampled rel-L2: attention {err:.2e}, FFN {err_f:.2e}, "
        f"block increment {err_x:.2e}")
    assert err <= BF16_TOL and err_f <= BF16_TOL and err_x <= BF16_TOL
    assert np.isfinite(Xo).all()


def test_fp32_narrow_decoder():
    """p = 2 gives p^2 Cout = 32 decoder outputs per token (a decoder product
    narrower than any GEMM tile); fp32 path: final LayerNorm + modulation,
    then the VALU GEMM with its bias epilogue."""
    cfg = dit_inputs.workload("dit_s8_f32", p=2, N=2)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    log("fp32 DiT-S p=2 (T=256, 32 decoder outputs) B=2")
    m = _model(cfg, w)
    x, t, y, _ = device_inputs(cfg, inp)
    taps = m.make_taps(2)
    out = np_(m.forward(x, t, y, taps=taps))
    ref, otaps = oracle_taps(cfg, w, inp)
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert err <= F32_TOL
    compare_taps(cfg, taps, otaps, F32_TOL, "fp32 S p=2")
