"""GPU parity of the in-context and cross-attention conditioning designs
(itwiki "확산 트랜스포머", Conditioning methods table; cointeeth DiT article)
through the C ABI against the fp64 oracle.

Bounds as for the adaLN-Zero model: rel-L2 <= 1e-4 (fp32) and <= 2e-2
(bf16), for the output and for every tap: the time embedding, the embedded
tokens (with the two conditioning tokens of the in-context design), the
residual stream after each block and the decoder output on the patch tokens.
"""
import numpy as np
import pytest
import torch

import dit_inputs
import oracle
from tests.parity import BF16_TOL, F32_TOL, device_inputs, log, np_, rel_l2

pytestmark = pytest.mark.gpu
dmod = pytest.importorskip("diffusion_transformer_denoiser_amd")

DESIGNS = [(1, "in-context"), (2, "cross-attention")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dmod.load()
    yield
    torch.cuda.synchronize()


def _check_taps(cfg, m, taps, otaps, rows, tol, label):
    d, N, T, Tt = cfg["d"], cfg["N"], m.T, m.Tt
    res = {"temb": rel_l2(np_(taps["c"]), otaps["temb"]),
           "x_embed": rel_l2(np_(taps["x_embed"]), otaps["X0"].reshape(-1, d))}
    xb = np_(taps["x_blocks"])
    for l in range(N):
        res[f"x_block{l}"] = rel_l2(xb[l], otaps["X"][l].reshape(-1, d))
        prev = otaps["X0"] if l == 0 else otaps["X"][l - 1]
        gprev = np_(taps["x_embed"]) if l == 0 else xb[l - 1]
        res[f"dx_block{l}"] = rel_l2(xb[l] - gprev, (otaps["X"][l] - prev).reshape(-1, d))
    Y = np_(taps["y_final"]).reshape(rows, Tt, -1)[:, :T]
    res["y_final"] = rel_l2(Y, otaps["Y"])
    log(f"{label} taps rel-L2: " + ", ".join(f"{k}={v:.2e}" for k, v in res.items()))
    bad = {k: v for k, v in res.items() if not v <= tol}
    assert not bad, f"{label}: stages above {tol}: {bad}"


@pytest.mark.parametrize("cond,name", DESIGNS)
@pytest.mark.parametrize("wl,over,tol", [("dit_s8_f32", dict(N=3), F32_TOL),
                                         ("dit_b4_bf16", dict(N=3, batch=8), BF16_TOL)])
def test_forward_with_taps_matches_oracle(cond, name, wl, over, tol):
    cfg = dit_inputs.workload(wl, conditioning=cond, **over)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    B = inp["x_t"].shape[0]
    inp["y"][-1] = cfg["num_classes"]          # one null-label row
    log(f"{name} {wl} {over}")
    m = dmod.DiT(cfg, w, "cuda")
    x, t, y, _ = device_inputs(cfg, inp)
    taps = m.make_taps(B)
    out = np_(m.forward(x, t, y, taps=taps))
    otaps = {}
    ref = oracle.forward(cfg, w, inp["x_t"], inp["t"], inp["y"], taps=otaps)
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert out.shape == ref.shape and err <= tol
    _check_taps(cfg, m, taps, otaps, B, tol, f"{name} {wl}")


@pytest.mark.parametrize("cond,name", DESIGNS)
def test_guided_xl2_reduced_depth(cond, name):
    cfg = dit_inputs.workload("dit_xl2_256_cfg", conditioning=cond, N=2, batch=3)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    log(f"{name} XL/2 N=2 guided, 3 + 3 rows")
    m = dmod.DiT(cfg, w, "cuda")
    x, t, y, _ = device_inputs(cfg, inp)
    out = np_(m.cfg_forward(x, t, y, cfg["scale"], cfg["guided"]))
    ref = oracle.cfg_forward(cfg, w, inp["x_t"], inp["t"], inp["y"], cfg["scale"], cfg["guided"])
    err = rel_l2(out, ref)
    log(f"  out rel-L2 {err:.2e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("cond,name", DESIGNS)
def test_full_size_xl2_guided_sampled_row(cond, name):
    """Full DiT-XL/2 256x256 with guidance, 32 + 32 trunk rows; the oracle
    runs one guided row (rows are independent)."""
    cfg = dit_inputs.workload("dit_xl2_256_cfg", conditioning=cond)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    log(f"{name} full-size XL/2 256 guided, sampled row 17")
    m = dmod.DiT(cfg, w, "cuda")
    x, t, y, _ = device_inputs(cfg, inp)
    out = np_(m.cfg_forward(x, t, y, cfg["scale"], cfg["guided"]))
    r = 17
    ref = oracle.cfg_forward(cfg, w, inp["x_t"][r:r + 1], inp["t"][r:r + 1], inp["y"][r:r + 1],
                             cfg["scale"], cfg["guided"])
    err = rel_l2(out[r:r + 1], ref)
    log(f"  row {r} rel-L2 {err:.2e}")
    assert np.all(np.isfinite(out)) and err <= BF16_TOL


@pytest.mark.parametrize("cond,name", DESIGNS)
def test_out_of_range_label_poisons_only_its_row(cond, name):
    cfg = dit_inputs.workload("dit_s8_f32", conditioning=cond, N=2, batch=3)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    x, t, y, _ = device_inputs(cfg, inp)
    y[1] = cfg["num_classes"] + 5
    out = np_(m.forward(x, t, y))
    assert np.all(np.isnan(out[1]))
    for r in (0, 2):
        ref = oracle.forward(cfg, w, inp["x_t"][r:r + 1], inp["t"][r:r + 1], inp["y"][r:r + 1])
        assert rel_l2(out[r:r + 1], ref) <= F32_TOL


def test_sampling_loop_with_in_context_design():
    """dit_sample reads the decoder output with its T + 2 token stride."""
    from oracle import sampler_oracle as so
    cfg = dit_inputs.workload("dit_s8_f32", conditioning=1, N=2)
    w = dit_inputs.make_weights(cfg)
    S = 3
    inp = dit_inputs.make_sampler_inputs(cfg, S)
    m = dmod.DiT(cfg, w, "cuda")
    xg = torch.from_numpy(inp["x"]).cuda()
    m.sample(dmod.Sampler("ddpm", S), xg, y=torch.from_numpy(inp["y"]).cuda(), scale=1.5,
             guided=4, noise=torch.from_numpy(inp["noise"]).cuda())
    _, abar = so.linear_beta_schedule()

    def model(xx, tt):
        return oracle.cfg_forward(cfg, w, xx, np.full(xx.shape[0], tt), inp["y"], 1.5, 4)

    ref = so.sample_ddpm(model, inp["x"], so.even_timesteps(S), inp["noise"], cfg["C"], abar)
    err = rel_l2(np_(xg), ref)
    log(f"in-context DDPM loop S=3 rel-L2 {err:.2e}")
    assert err <= F32_TOL
