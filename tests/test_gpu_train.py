"""GPU parity of one training step (dit_train_step) against the fp64 oracle
(oracle/train_oracle.py: autograd over the restated forward, pinned to
finite differences).

Checked per step: both loss terms; the gradient of every trained parameter
field (rel-L2 <= 1e-4 fp32, <= 2e-2 bf16); AdamW and the EMA, by applying the
oracle's update formula in fp64 to the GPU's own gradient and state (the
update normalises each gradient element, so it is compared where it is
unique: given the same gradient); and the model-dtype weights, which must be
the new master weights rounded.  Rows include t = 0 (the negative
log-likelihood branch), t = 1, a null label and repeated labels.
"""
import numpy as np
import pytest
import torch

import dit_inputs
from oracle import train_oracle as TR
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
    cfg = dict(name="train small", C=4, Cout=8, F=1, H=8, W=8, p=2, pt=1, d=128, N=2, heads=2,
               mlp_hidden=512, num_classes=10, cond_dim=0, freq_dim=256, qk_norm=0, rope3d=0,
               dtype=dit_inputs.DTYPE_F32, ln_eps=1e-6, batch=4, cfg=False, scale=1.0, guided=4,
               conditioning=0, seed_idx=12)
    cfg.update(kw)
    return cfg


def make_batch(cfg, seed):
    rng = np.random.default_rng(seed)
    B = cfg["batch"]
    x0 = rng.standard_normal((B, cfg["C"], cfg["H"], cfg["W"])).astype(np.float32)
    eps = rng.standard_normal(x0.shape).astype(np.float32)
    t = np.concatenate([[0, 1], rng.integers(0, 1000, size=B - 2)]).astype(np.int32)
    y = rng.integers(0, cfg["num_classes"] + 1, size=B).astype(np.int32)
    y[0] = cfg["num_classes"]          # null label
    y[-1] = y[1]                       # a repeated label
    return x0, y, t, eps


def to_dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def run_steps(cfg, tol, steps=2, label=""):
    w = dit_inputs.make_weights(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    m.train_init()
    hp = TR.ADAMW
    wcur = {k: v.copy() for k, v in w.items()}
    for k in range(1, steps + 1):
        x0, y, t, eps = make_batch(cfg, 100 + k)
        before = {n: m.train_state[n].clone() for n in ("master", "m", "v", "ema")}
        loss = np_(m.train_step(*to_dev(x0, y, t, eps), step=k))
        torch.cuda.synchronize()
        ls, lv, g = TR.gradients(cfg, wcur, x0, y, t, eps)
        el = (abs(loss[0] - ls) / abs(ls), abs(loss[1] - lv) / abs(lv))
        log(f"{label} step {k}: loss GPU {loss} oracle ({ls:.6f}, {lv:.6f}); rel err {el[0]:.2e} {el[1]:.2e}")
        assert el[0] <= tol and el[1] <= tol
        errs = {}
        for name in TR.TRAIN_FIELDS:
            errs[name] = rel_l2(np_(m.train_view("grad", name)), g[name])
        log("  grad rel-L2: " + ", ".join(f"{n}={e:.1e}" for n, e in errs.items()))
        bad = {n: e for n, e in errs.items() if not e <= tol}
        assert not bad, f"{label} step {k}: gradients above {tol}: {bad}"
        # AdamW / EMA on the GPU's own gradient
        for name in TR.TRAIN_FIELDS:
            off, cnt = m.train_fields[name]
            sl = slice(off, off + cnt)
            gg = np_(m.train_state["grad"][sl])
            p1, m1, v1 = TR.adamw(np_(before["master"][sl]), gg, np_(before["m"][sl]),
                                  np_(before["v"][sl]), k, hp["lr"], hp["beta1"], hp["beta2"],
                                  hp["eps"], hp["weight_decay"])
            dp_gpu = np_(m.train_state["master"][sl]) - np_(before["master"][sl])
            dp_ref = p1 - np_(before["master"][sl])
            assert rel_l2(dp_gpu, dp_ref) <= 1e-4, (name, rel_l2(dp_gpu, dp_ref))
            assert rel_l2(np_(m.train_state["m"][sl]), m1) <= 1e-6, name
            assert rel_l2(np_(m.train_state["v"][sl]), v1) <= 1e-5, name
            e1 = TR.ema(np_(before["ema"][sl]), np_(m.train_state["master"][sl]), hp["ema_decay"])
            assert np.allclose(np_(m.train_state["ema"][sl]), e1, rtol=1e-6, atol=1e-9), name
            # the model-dtype weights are the new master weights rounded
            want = m.train_state["master"][sl].to(m.tensors[name].dtype)
            assert torch.equal(m.tensors[name].reshape(-1), want), name
            wcur[name] = np_(m.tensors[name]).reshape(w[name].shape).astype(np.float64)


def test_train_step_fp32_matches_oracle():
    run_steps(small_cfg(), F32_TOL, label="fp32 d128 T16 B4")


def test_train_step_bf16_matches_oracle():
    run_steps(small_cfg(dtype=dit_inputs.DTYPE_BF16, batch=8), BF16_TOL, label="bf16 d128 T16 B8")


def test_train_step_learned_sigma_off_matches_oracle():
    """Cout == C: the loss is L_simple alone."""
    cfg = small_cfg(Cout=4)
    w = dit_inputs.make_weights(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    x0, y, t, eps = make_batch(cfg, 7)
    loss = np_(m.train_step(*to_dev(x0, y, t, eps), step=1))
    torch.cuda.synchronize()
    ls, lv, g = TR.gradients(cfg, w, x0, y, t, eps)
    assert lv == 0.0 and loss[1] == 0.0
    assert abs(loss[0] - ls) <= F32_TOL * ls
    for name in TR.TRAIN_FIELDS:
        assert rel_l2(np_(m.train_view("grad", name)), g[name]) <= F32_TOL, name


def test_train_step_xl_width_two_blocks():
    """DiT-XL/2 width (d 1152, 16 heads of 72, T = 256) with two blocks, bf16."""
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=2, batch=2)
    w = dit_inputs.make_weights(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    x0, y, t, eps = make_batch(dict(cfg, batch=2), 21)
    log("XL/2 width, N=2, B=2, bf16")
    loss = np_(m.train_step(*to_dev(x0, y, t, eps), step=1))
    torch.cuda.synchronize()
    ls, lv, g = TR.gradients(cfg, w, x0, y, t, eps)
    log(f"  loss GPU {loss} oracle ({ls:.6f}, {lv:.6f})")
    assert abs(loss[0] - ls) <= BF16_TOL * ls and abs(loss[1] - lv) <= BF16_TOL * abs(lv)
    errs = {n: rel_l2(np_(m.train_view("grad", n)), g[n]) for n in TR.TRAIN_FIELDS}
    log("  grad rel-L2: " + ", ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= BF16_TOL}
    assert not bad, bad


def test_train_step_xl_width_batch16():
    """DiT-XL/2 width with one block at batch 16 (M = 4096 token rows, 16 row
    tiles per product): both loss terms and every gradient against the fp64
    oracle's autograd."""
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=1, batch=16)
    w = dit_inputs.make_weights(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    x0, y, t, eps = make_batch(dict(cfg, batch=16), 23)
    log("XL/2 width, N=1, B=16, bf16")
    loss = np_(m.train_step(*to_dev(x0, y, t, eps), step=1))
    torch.cuda.synchronize()
    ls, lv, g = TR.gradients(cfg, w, x0, y, t, eps)
    log(f"  loss GPU {loss} oracle ({ls:.6f}, {lv:.6f})")
    assert abs(loss[0] - ls) <= BF16_TOL * ls and abs(loss[1] - lv) <= BF16_TOL * abs(lv)
    errs = {n: rel_l2(np_(m.train_view("grad", n)), g[n]) for n in TR.TRAIN_FIELDS}
    log("  grad rel-L2: " + ", ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= BF16_TOL}
    assert not bad, bad


def _train_inputs_dev(cfg, B=None):
    inp = dit_inputs.make_train_inputs(cfg, batch=B)
    return to_dev(inp["x0"], inp["y"], inp["t"], inp["noise"])


def test_train_step_full_size_batch_split_consistency():
    """The training workload at full size (DiT-XL/2, batch 256, 28 blocks, bf16), as
    the training benchmark runs it.  The loss is a mean over rows, so the loss and
    every gradient of the 256-row batch must equal the mean of those of its two
    128-row halves; only the summation order of the reductions over rows differs.
    lr = 0 keeps the weights fixed across the three steps."""
    cfg = dit_inputs.workload("dit_xl2_256_train")
    B = cfg["batch"]
    m = dmod.DiT(cfg, dit_inputs.make_weights(cfg), "cuda")
    m.train_init()
    x0, y, t, eps = _train_inputs_dev(cfg)
    log(f"full-size training step: batch {B}, 28 blocks, bf16")
    lf = np_(m.train_step(x0, y, t, eps, step=1, lr=0.0)).astype(np.float64)
    gf = m.train_state["grad"].clone()
    h = B // 2
    la = np_(m.train_step(x0[:h], y[:h], t[:h], eps[:h], step=2, lr=0.0)).astype(np.float64)
    ga = m.train_state["grad"].clone()
    lb = np_(m.train_step(x0[h:], y[h:], t[h:], eps[h:], step=3, lr=0.0)).astype(np.float64)
    gm = (ga + m.train_state["grad"]) * 0.5
    torch.cuda.synchronize()
    el = np.abs(lf - (la + lb) / 2) / np.abs(lf)
    log(f"  loss full {lf}, halves {la} {lb}; rel diff {el}")
    assert np.all(np.isfinite(lf)) and np.all(el <= 1e-5)
    errs = {}
    for name, (off, cnt) in m.train_fields.items():
        errs[name] = rel_l2(np_(gf[off:off + cnt]), np_(gm[off:off + cnt]))
    log("  grad rel-L2 full vs mean of halves: " + ", ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= 1e-4}
    assert not bad, bad


def test_train_step_full_depth_one_row_matches_oracle():
    """One row through all 28 DiT-XL/2 blocks (bf16): both loss terms and every
    gradient field against the fp64 oracle's autograd."""
    cfg = dit_inputs.workload("dit_xl2_256_train", batch=1)
    w = dit_inputs.make_weights(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    inp = dit_inputs.make_train_inputs(cfg, batch=1)
    inp["t"][0] = 500
    log("full-depth training step, one row, bf16")
    loss = np_(m.train_step(*to_dev(inp["x0"], inp["y"], inp["t"], inp["noise"]), step=1))
    torch.cuda.synchronize()
    ls, lv, g = TR.gradients(cfg, w, inp["x0"], inp["y"], inp["t"], inp["noise"])
    log(f"  loss GPU {loss} oracle ({ls:.6f}, {lv:.6f})")
    assert abs(loss[0] - ls) <= BF16_TOL * ls and abs(loss[1] - lv) <= BF16_TOL * abs(lv)
    errs = {n: rel_l2(np_(m.train_view("grad", n)), g[n]) for n in TR.TRAIN_FIELDS}
    log("  grad rel-L2: " + ", ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= BF16_TOL}
    assert not bad, bad
