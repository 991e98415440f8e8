"""GPU parity of the sampler (dit_sampler_step / dit_sample through the C ABI)
against the fp64 oracle's steps and loops.

Bounds: relative L2 <= 1e-4 for fp32 models and for the step kernels alone,
<= 2e-2 for bf16 models (the bounds of the forward pass; a step is a few
fp32 FMAs per element on top of it).  The bf16 loop feeds the model the state
rounded to bf16 on both sides.  At full size the loop is checked on sampled
rows (rows are independent) and against the composition of the library's own
guided forward and step entry points.
"""
import numpy as np
import pytest
import torch

import dit_inputs
import oracle
from oracle import sampler_oracle as so
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


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


# --- step kernels alone ---------------------------------------------------------------------

@pytest.mark.parametrize("kind,learned", [("ddpm", True), ("ddpm", False), ("dpmpp_2m", True),
                                          ("dpmpp_2m", False), ("rf_euler", False)])
def test_step_kernel_chain_matches_oracle(kind, learned):
    """Six steps with seeded random predictions; the GPU chain (fp32) and the
    oracle chain (fp64) each carry their own state and x0 history."""
    S, B, C, Hh, Ww = 6, 3, 4, 17, 9          # 1836 elements: 8 blocks, ragged tail
    Cout = 2 * C if learned else C
    rng = np.random.default_rng(41)
    x = dit_inputs.f32_round(rng.standard_normal((B, C, Hh, Ww)))
    mos = dit_inputs.f32_round(rng.standard_normal((S, B, Cout, Hh, Ww)))
    zs = dit_inputs.f32_round(rng.standard_normal((S, B, C, Hh, Ww)))
    sp = dmod.Sampler(kind, S)
    log(f"step chain {kind} Cout={Cout} S={S} shape={x.shape}")
    gx = _dev(x)
    hist = torch.zeros_like(gx)
    _, abar = so.linear_beta_schedule()
    ts = so.even_timesteps(S)
    levels = [float(abar[t]) for t in ts] + [1.0]
    times = so.rf_uniform_times(S)
    ox = x.astype(np.float64)
    ox0 = None
    for k in range(S):
        gx = sp.step(k, gx, _dev(mos[k]), z=_dev(zs[k]), x0_hist=hist)
        if kind == "ddpm":
            lbt = so.ddpm_last_log_beta_tilde(levels[:-1]) if k == S - 1 else None
            ox = so.ddpm_step(ox, mos[k], C, levels[k], levels[k + 1], zs[k], log_beta_tilde=lbt)
        elif kind == "dpmpp_2m":
            second = k >= 1 and k < S - 1
            ox, ox0 = so.dpmpp_step(ox, mos[k][:, :C], levels[k], levels[k + 1],
                                    ox0 if second else None, levels[k - 1] if second else None)
        else:
            ox = so.rf_euler_step(ox, mos[k][:, :C], times[k], times[k + 1])
        err = rel_l2(np_(gx), ox)
        log(f"  step {k}: rel-L2 {err:.2e}")
        assert err <= F32_TOL


def test_step_in_place_and_single_step_without_noise():
    B, C, n = 2, 4, 64
    rng = np.random.default_rng(42)
    x = dit_inputs.f32_round(rng.standard_normal((B, C, n)))
    mo = dit_inputs.f32_round(rng.standard_normal((B, 2 * C, n)))
    sp = dmod.Sampler("ddpm", 1)
    gx = _dev(x)
    out = sp.step(0, gx, _dev(mo), out=gx)             # the only step: no noise read
    assert out.data_ptr() == gx.data_ptr()
    _, abar = so.linear_beta_schedule()
    ref = so.ddpm_step(x, mo, C, float(abar[999]), 1.0, None)
    err = rel_l2(np_(gx), ref)
    log(f"single DDPM step in place: rel-L2 {err:.2e}")
    assert err <= F32_TOL


# --- whole loops on small models ---------------------------------------------------------------

def _oracle_loop(cfg, w, kind, S, inp, scale, guided):
    Bn = inp["x"].shape[0]
    cast = (lambda a: dit_inputs.cast_to(a, dit_inputs.DTYPE_BF16)) \
        if cfg["dtype"] == dit_inputs.DTYPE_BF16 else None

    def model(xx, t):
        tv = np.full(Bn, t, dtype=np.float64)
        if guided > 0:
            return oracle.cfg_forward(cfg, w, xx, tv, inp["y"], scale, guided)
        return oracle.forward(cfg, w, xx, tv, inp["y"], inp["pooled"])

    _, abar = so.linear_beta_schedule()
    if kind == "ddpm":
        return so.sample_ddpm(model, inp["x"], so.even_timesteps(S), inp["noise"], cfg["C"],
                              abar, model_input=cast)
    if kind == "dpmpp_2m":
        return so.sample_dpmpp_2m(model, inp["x"], so.even_timesteps(S), cfg["C"], abar,
                                  model_input=cast)
    return so.sample_rf_euler(model, inp["x"], so.rf_uniform_times(S), model_input=cast)


def _gpu_loop(cfg, w, kind, S, inp, scale, guided):
    m = dmod.DiT(cfg, w, "cuda")
    x = _dev(inp["x"])
    noise = _dev(inp["noise"]) if kind == "ddpm" else None
    m.sample(dmod.Sampler(kind, S), x, y=_dev(inp["y"]), pooled=_dev(inp["pooled"]),
             scale=scale, guided=guided, noise=noise)
    return np_(x)


@pytest.mark.parametrize("name,over,kind,S,guided,tol", [
    ("dit_s8_f32", dict(), "ddpm", 4, 4, F32_TOL),
    ("dit_s8_f32", dict(), "dpmpp_2m", 5, 8, F32_TOL),
    ("dit_s8_f32", dict(), "ddpm", 1, 4, F32_TOL),
    ("dit_s8_f32", dict(batch=3), "ddpm", 3, 0, F32_TOL),
    ("dit_b4_bf16", dict(N=2, batch=4), "ddpm", 3, 4, BF16_TOL),
    ("dit_b4_bf16", dict(N=2, batch=3), "dpmpp_2m", 3, 4, BF16_TOL),
    ("video_xl_spacetime", dict(F=2, H=8, W=8, N=1), "rf_euler", 3, 0, BF16_TOL),
])
def test_sample_loop_matches_oracle(name, over, kind, S, guided, tol):
    cfg = dit_inputs.workload(name, **over)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_sampler_inputs(cfg, S)
    scale = 1.5 if guided else 1.0
    log(f"sample loop {name} {over} {kind} S={S} guided={guided}")
    got = _gpu_loop(cfg, w, kind, S, inp, scale, guided)
    ref = _oracle_loop(cfg, w, kind, S, inp, scale, guided)
    err = rel_l2(got, ref)
    log(f"  final state rel-L2 {err:.2e}")
    assert got.shape == ref.shape and err <= tol


# --- full size -----------------------------------------------------------------------------------

def test_full_size_loop_equals_forward_plus_step_composition():
    """dit_sample (decoder output read in the step kernel) against
    dit_cfg_forward + dit_sampler_step, DiT-XL/2 256x256, 32 + 32 rows."""
    cfg = dit_inputs.workload("dit_xl2_256_cfg")
    w = dit_inputs.make_weights(cfg)
    S = 3
    inp = dit_inputs.make_sampler_inputs(cfg, S)
    log("full-size XL/2 256 DDPM S=3: dit_sample vs forward + step")
    m = dmod.DiT(cfg, w, "cuda")
    x = _dev(inp["x"])
    noise = _dev(inp["noise"])
    y = _dev(inp["y"])
    sp = dmod.Sampler("ddpm", S)
    m.sample(sp, x, y=y, scale=cfg["scale"], guided=cfg["guided"], noise=noise)
    xs = _dev(inp["x"])
    for k in range(S):
        mt, _ = sp.coefficients(k)
        t = torch.full((cfg["batch"],), mt, dtype=torch.float32, device="cuda")
        eps = m.cfg_forward(xs.to(torch.bfloat16), t, y, cfg["scale"], cfg["guided"])
        xs = sp.step(k, xs, eps, z=noise[k])
    a, b = np_(x), np_(xs)
    diff = float(np.max(np.abs(a - b)))
    log(f"  max |loop - composition| = {diff:.3e} (bit-exact: {np.array_equal(a, b)})")
    assert diff <= 1e-5 * float(np.max(np.abs(b)))


def test_full_size_loop_sampled_rows_match_oracle():
    """DiT-XL/2 256x256, 32 conditional rows, two guided DDPM steps; the
    oracle runs the loop for two sampled rows on their own."""
    cfg = dit_inputs.workload("dit_xl2_256_cfg")
    w = dit_inputs.make_weights(cfg)
    S = 2
    inp = dit_inputs.make_sampler_inputs(cfg, S)
    log("full-size XL/2 256 DDPM S=2, sampled rows 0 and 29")
    got = _gpu_loop(cfg, w, "ddpm", S, inp, cfg["scale"], cfg["guided"])
    errs = []
    for r in (0, 29):
        sub = dict(x=inp["x"][r:r + 1], noise=inp["noise"][:, r:r + 1], y=inp["y"][r:r + 1],
                   pooled=None)
        ref = _oracle_loop(cfg, w, "ddpm", S, sub, cfg["scale"], cfg["guided"])
        errs.append(rel_l2(got[r:r + 1], ref))
    log(f"  sampled rows rel-L2 {errs}")
    assert max(errs) <= BF16_TOL
