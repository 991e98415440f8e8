"""GPU parity of packed sequences (dit_forward_packed, the Patch n' Pack
batching of the GOKU review, section 2.2): latents of different sizes in one
call, attention inside each sequence.  The oracle runs every sequence on its
own; bounds as for the forward pass (1e-4 fp32, 2e-2 bf16, rel-L2 per
sequence).  Same-sized sequences must also reproduce the batched forward.
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


def _inputs(cfg, shapes, seed):
    rng = np.random.default_rng(seed)
    xs = [dit_inputs.cast_to(rng.standard_normal((cfg["C"],) + hw), cfg["dtype"]) for hw in shapes]
    t = rng.integers(0, 1000, size=len(shapes)).astype(np.float32)
    y = rng.integers(0, cfg["num_classes"], size=len(shapes)).astype(np.int32)
    y[-1] = cfg["num_classes"]      # one null-label sequence
    return xs, t, y


def _run(m, cfg, xs, t, y):
    dt = dmod.torch_dtype(cfg["dtype"])
    gx = [torch.from_numpy(a).to(dt).cuda() for a in xs]
    outs = m.forward_packed(gx, torch.from_numpy(t).cuda(), torch.from_numpy(y).cuda())
    return [np_(o) for o in outs]


@pytest.mark.parametrize("wl,over,shapes,tol", [
    ("dit_s8_f32", dict(p=4, N=2), [(32, 32), (64, 32), (32, 64), (64, 64), (16, 32)], F32_TOL),
    ("dit_b4_bf16", dict(p=2, N=3), [(16, 16), (32, 32), (16, 32), (32, 16), (16, 16)], BF16_TOL),
])
def test_packed_matches_per_sequence_oracle(wl, over, shapes, tol):
    cfg = dit_inputs.workload(wl, **over)
    w = dit_inputs.make_weights(cfg)
    xs, t, y = _inputs(cfg, shapes, 71)
    log(f"packed {wl} {over} shapes={shapes}")
    m = dmod.DiT(cfg, w, "cuda")
    got = _run(m, cfg, xs, t, y)
    ref = oracle.forward_packed(cfg, w, xs, t, y)
    errs = [rel_l2(g, r) for g, r in zip(got, ref)]
    log(f"  per-sequence rel-L2 {[f'{e:.2e}' for e in errs]}")
    assert all(g.shape == r.shape for g, r in zip(got, ref))
    assert max(errs) <= tol


@pytest.mark.parametrize("wl,over", [("dit_s8_f32", dict(p=4, N=2)),
                                     ("dit_b4_bf16", dict(N=2, batch=5))])
def test_packed_equal_shapes_reproduce_batched_forward(wl, over):
    cfg = dit_inputs.workload(wl, **over)
    w = dit_inputs.make_weights(cfg)
    B = 5
    inp = dit_inputs.make_inputs(cfg, batch=B)
    m = dmod.DiT(cfg, w, "cuda")
    dt = dmod.torch_dtype(cfg["dtype"])
    x = torch.from_numpy(inp["x_t"]).to(dt).cuda()
    t = torch.from_numpy(inp["t"]).cuda()
    y = torch.from_numpy(inp["y"]).cuda()
    batched = np_(m.forward(x, t, y))
    packed = m.forward_packed([x[i] for i in range(B)], t, y)
    packed = np.stack([np_(o) for o in packed])
    diff = float(np.max(np.abs(packed - batched)))
    log(f"packed vs batched {wl}: max |diff| = {diff:.3e} (bit-exact: {np.array_equal(packed, batched)})")
    assert rel_l2(packed, batched) <= 1e-6


def test_packed_xl2_mixed_256_and_512():
    """DiT-XL/2 (depth 4): four 256x256 latents and one 512x512 latent in one
    call (4 x 256 + 1024 tokens); two sequences checked against the oracle."""
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=4)
    w = dit_inputs.make_weights(cfg)
    shapes = [(32, 32), (64, 64), (32, 32), (32, 32), (32, 32)]
    xs, t, y = _inputs(cfg, shapes, 72)
    log(f"packed XL/2 N=4 shapes={shapes}")
    m = dmod.DiT(cfg, w, "cuda")
    got = _run(m, cfg, xs, t, y)
    errs = {}
    for i in (1, 4):
        ref = oracle.forward_packed(cfg, w, [xs[i]], t[i:i + 1], y[i:i + 1])[0]
        errs[i] = rel_l2(got[i], ref)
    log(f"  rel-L2 {errs}")
    assert all(np.all(np.isfinite(g)) for g in got)
    assert max(errs.values()) <= BF16_TOL
