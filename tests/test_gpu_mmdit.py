"""GPU parity of the MMDiT design (itwiki "확산 트랜스포머", MMDiT section)
through the C ABI (dit_forward_ctx) against the fp64 oracle.

Bounds as for the adaLN-Zero model: rel-L2 <= 1e-4 (fp32) and <= 2e-2
(bf16), for the output and for every tap: the conditioning vector, the
image-stream modulation, both embedded streams, both streams after each block
(and each block's increment) and the decoder output.  The call without taps
is checked against the oracle as well, and must equal the tapped call bit for
bit (the taps only add copies).  The 512 x 512 MMDiT runs at its full width and token counts (1024
image + 333 text tokens per row) with two blocks.
"""
import numpy as np
import pytest
import torch

import dit_inputs
import oracle
from tests.parity import BF16_TOL, F32_TOL, log, np_, rel_l2

pytestmark = pytest.mark.gpu
dmod = pytest.importorskip("diffusion_transformer_denoiser_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dmod.load()
    yield
    torch.cuda.synchronize()


def small_cfg(**kw):
    cfg = dict(name="MMDiT small", C=4, Cout=4, F=1, H=16, W=16, p=2, pt=1, d=128, N=2, heads=2,
               mlp_hidden=512, num_classes=0, cond_dim=32, freq_dim=256, qk_norm=0, rope3d=0,
               dtype=dit_inputs.DTYPE_F32, ln_eps=1e-6, batch=2, cfg=False, scale=1.0, guided=4,
               conditioning=dit_inputs.COND_MMDIT, ctx_len=7, ctx_dim=64, seed_idx=9)
    cfg.update(kw)
    return cfg


def _device(cfg, inp):
    dt = torch.bfloat16 if cfg["dtype"] == dit_inputs.DTYPE_BF16 else torch.float32
    x = torch.from_numpy(inp["x_t"]).to(dt).cuda()
    ctx = torch.from_numpy(inp["ctx"]).to(dt).cuda()
    t = torch.from_numpy(inp["t"]).cuda()
    pooled = torch.from_numpy(inp["pooled"]).cuda()
    return x, t, pooled, ctx


def _check_taps(cfg, m, taps, ot, B, tol, label):
    d, N, T, L = cfg["d"], cfg["N"], m.T, m.Lc
    split = B * T      # image-stream rows first, then the text stream's

    def streams(a):
        return a[:split], a[split:]

    xe = np_(taps["x_embed"])
    res = {"c": rel_l2(np_(taps["c"]), ot["c"]),
           "mod": rel_l2(np_(taps["mod"]), ot["mod"]),
           "xi_embed": rel_l2(streams(xe)[0], ot["Xi0"].reshape(-1, d)),
           "xc_embed": rel_l2(streams(xe)[1], ot["Xc0"].reshape(-1, d)),
           "y_final": rel_l2(np_(taps["y_final"]), ot["Y"].reshape(B * T, -1))}
    xb = np_(taps["x_blocks"])
    for l in range(N):
        gi, gc = streams(xb[l])
        pi, pc = streams(xe if l == 0 else xb[l - 1])
        ri, rc_ = ot["Xi"][l].reshape(-1, d), ot["Xc"][l].reshape(-1, d)
        oi = (ot["Xi0"] if l == 0 else ot["Xi"][l - 1]).reshape(-1, d)
        oc = (ot["Xc0"] if l == 0 else ot["Xc"][l - 1]).reshape(-1, d)
        res[f"xi_block{l}"] = rel_l2(gi, ri)
        res[f"xc_block{l}"] = rel_l2(gc, rc_)
        res[f"dxi_block{l}"] = rel_l2(gi - pi, ri - oi)
        res[f"dxc_block{l}"] = rel_l2(gc - pc, rc_ - oc)
    log(f"{label} taps rel-L2: " + ", ".join(f"{k}={v:.2e}" for k, v in res.items()))
    bad = {k: v for k, v in res.items() if not v <= tol}
    assert not bad, f"{label}: stages above {tol}: {bad}"


@pytest.mark.parametrize("dtype,batch,tol", [(dit_inputs.DTYPE_F32, 2, F32_TOL),
                                             (dit_inputs.DTYPE_BF16, 4, BF16_TOL)])
def test_small_mmdit_matches_oracle(dtype, batch, tol):
    cfg = small_cfg(dtype=dtype, batch=batch)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_mmdit_inputs(cfg)
    label = f"MMDiT small dtype={dtype} B={batch}"
    log(label)
    m = dmod.DiT(cfg, w, "cuda")
    x, t, pooled, ctx = _device(cfg, inp)
    ot = {}
    ref = oracle.mmdit_forward(cfg, w, inp["x_t"], inp["t"], inp["ctx"], inp["pooled"], taps=ot)
    taps = m.make_taps(batch)
    out = np_(m.forward_ctx(x, t, pooled, ctx, taps=taps))
    err = rel_l2(out, ref)
    log(f"  out (taps) rel-L2 {err:.2e}")
    assert out.shape == ref.shape and err <= tol
    _check_taps(cfg, m, taps, ot, batch, tol, label)
    # without taps: the same kernels on the same rows
    out2 = np_(m.forward_ctx(x, t, pooled, ctx))
    torch.cuda.synchronize()
    err2 = rel_l2(out2, ref)
    log(f"  out (no taps) rel-L2 {err2:.2e}")
    assert err2 <= tol
    assert np.array_equal(out2, out), "untapped output differs from the tapped one"


def test_text_tokens_reach_the_image_output():
    """Changing one row's text embeddings changes only that row's output, by
    what the oracle says it changes (fp32: the change is about 1e-3 of the
    output, so it is compared as a difference)."""
    cfg = small_cfg(batch=3)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_mmdit_inputs(cfg)
    log("MMDiT small fp32: per-row dependence on the text tokens")
    m = dmod.DiT(cfg, w, "cuda")
    x, t, pooled, ctx = _device(cfg, inp)
    a = np_(m.forward_ctx(x, t, pooled, ctx))
    ctx2 = ctx.clone()
    ctx2[1] = -ctx2[1]
    b = np_(m.forward_ctx(x, t, pooled, ctx2))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    sel = slice(1, 2)
    ra = oracle.mmdit_forward(cfg, w, inp["x_t"][sel], inp["t"][sel], inp["ctx"][sel],
                              inp["pooled"][sel])
    rb = oracle.mmdit_forward(cfg, w, inp["x_t"][sel], inp["t"][sel], -inp["ctx"][sel],
                              inp["pooled"][sel])
    err = rel_l2(b[1] - a[1], (rb - ra)[0])
    log(f"  change of row 1: {rel_l2(rb, ra):.2e} of the output; its rel-L2 error {err:.2e}")
    assert err <= 2e-2


def test_mmdit_512_full_width_two_blocks():
    cfg = dit_inputs.workload("mmdit_d24_512", N=2, batch=2)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_mmdit_inputs(cfg)
    log("MMDiT 512x512 (d 1536, 1024 + 333 tokens) N=2 B=2 bf16")
    m = dmod.DiT(cfg, w, "cuda")
    x, t, pooled, ctx = _device(cfg, inp)
    out = np_(m.forward_ctx(x, t, pooled, ctx))
    torch.cuda.synchronize()
    ref = oracle.mmdit_forward(cfg, w, inp["x_t"], inp["t"], inp["ctx"], inp["pooled"])
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert out.shape == ref.shape and err <= BF16_TOL
