"""Seeded synthetic workloads for the DiT denoiser forward pass.

This module is shared by the fp64 oracle's tests and by the GPU path's
tests and benchmark.  It draws numbers and casts them; it holds none of
the denoiser's arithmetic (no patchify, embedding, attention, LayerNorm,
guidance ...).

Workload shapes follow the pages:
  * latent 32x32x4 for 256x256 images and 64x64x4 for 512x512 images
    (itwiki "확산 트랜스포머" (Diffusion Transformer), section Structure /
    Latent space and patchify, and section Results / ImageNet table notes);
  * model sizes S/B/L/XL = (N, d, heads) (same page, Model sizes table);
  * the video latent uses the 8x8 spatial / 4x temporal VAE strides
    (blog.outta.ai "GOKU" review, section 2.1) with 16 channels.

Every value is drawn in fp64 from numpy's PCG64 generator, rounded to fp32
(round to nearest even) and, for bf16 workloads, rounded again to bf16
(round to nearest even).  The oracle and the GPU receive the same bits.
"""
from __future__ import annotations

import copy

import numpy as np

# ---------------------------------------------------------------------------
# dtype codes (mirrors the C header's enum values: 0 = fp32, 1 = bf16)
DTYPE_F32 = 0
DTYPE_BF16 = 1

# Conditioning designs (mirrors the C header's codes): adaLN-Zero, the time and
# class embeddings as two extra tokens, or as a cross-attended context
# (itwiki page, Conditioning methods table).
COND_ADALN_ZERO, COND_IN_CONTEXT, COND_CROSS_ATTENTION = 0, 1, 2
# MMDiT (itwiki page, MMDiT section): text and image streams with their own
# weights, joint attention, pooled-vector + time adaLN.
COND_MMDIT = 3

# Model sizes: (depth N, width d, heads) from the Model sizes table.
MODEL_SIZES = {
    "S": (12, 384, 6),
    "B": (12, 768, 12),
    "L": (24, 1024, 16),
    "XL": (28, 1152, 16),
}


def _image_config(size, p, I, dtype, batch, cfg_guidance, name):
    N, d, heads = MODEL_SIZES[size]
    return dict(
        name=name, C=4, Cout=8, F=1, H=I, W=I, p=p, pt=1, d=d, N=N,
        heads=heads, mlp_hidden=4 * d, num_classes=1000, cond_dim=0,
        freq_dim=256, qk_norm=0, rope3d=0, dtype=dtype, ln_eps=1e-6,
        batch=batch, cfg=cfg_guidance, scale=1.5, guided=4, conditioning=COND_ADALN_ZERO,
    )


# The five workloads.  ``batch`` is the number of rows the caller passes in:
# for guided workloads it is the number of conditional rows Bh; the trunk
# then runs 2*Bh rows (conditional + null-label).
WORKLOADS = {
    "dit_s8_f32": dict(_image_config("S", 8, 32, DTYPE_F32, 2, False,
                                     "DiT-S/8 fp32, 32x32x4 latent, batch 2"), seed_idx=1),
    "dit_b4_bf16": dict(_image_config("B", 4, 32, DTYPE_BF16, 32, False,
                                      "DiT-B/4 bf16, 32x32x4 latent, batch 32"), seed_idx=2),
    "dit_xl2_256_cfg": dict(_image_config("XL", 2, 32, DTYPE_BF16, 32, True,
                                          "DiT-XL/2 256x256 (32x32x4 latent) + CFG, 32 cond + 32 null rows"),
                            seed_idx=3),
    "dit_xl2_512_cfg": dict(_image_config("XL", 2, 64, DTYPE_BF16, 8, True,
                                          "DiT-XL/2 512x512 (64x64x4 latent) + CFG, 8 cond + 8 null rows"),
                            seed_idx=4),
    "video_xl_spacetime": dict(
        name="spacetime video DiT-XL, 16x60x104x16 latent, patch 1x2x2, batch 1",
        C=16, Cout=16, F=16, H=60, W=104, p=2, pt=1, d=1152, N=28, heads=16,
        mlp_hidden=4608, num_classes=0, cond_dim=4096, freq_dim=256, qk_norm=1,
        rope3d=1, dtype=DTYPE_BF16, ln_eps=1e-6, batch=1, cfg=False, scale=1.0,
        guided=16, conditioning=COND_ADALN_ZERO, seed_idx=5),
    # The other two conditioning designs of the Conditioning methods table, at
    # the DiT-XL/2 256x256 + CFG shape.
    "dit_xl2_256_cfg_in_context": dict(
        _image_config("XL", 2, 32, DTYPE_BF16, 32, True,
                      "DiT-XL/2 256x256 in-context conditioning + CFG, 32 cond + 32 null rows"),
        conditioning=COND_IN_CONTEXT, seed_idx=6),
    # MMDiT at depth 24 (hidden 64 x 24, 24 heads: the page's size rule),
    # 512x512 images as a 64x64x16 latent with p = 2, 333 text tokens of a
    # 4096-wide text encoder and a 2048-wide pooled vector, velocity output.
    "mmdit_d24_512": dict(
        name="MMDiT depth 24 (d 1536, 24 heads), 64x64x16 latent, 333 text tokens, batch 8",
        C=16, Cout=16, F=1, H=64, W=64, p=2, pt=1, d=1536, N=24, heads=24, mlp_hidden=6144,
        num_classes=0, cond_dim=2048, freq_dim=256, qk_norm=0, rope3d=0, dtype=DTYPE_BF16,
        ln_eps=1e-6, batch=8, cfg=False, scale=1.0, guided=16, conditioning=COND_MMDIT,
        ctx_len=333, ctx_dim=4096, seed_idx=8),
    # The pages' training setup: DiT-XL/2 on 256x256 ImageNet latents, batch 256.
    "dit_xl2_256_train": dict(_image_config("XL", 2, 32, DTYPE_BF16, 256, False,
                                            "DiT-XL/2 256x256 (32x32x4 latent) training, batch 256"),
                              seed_idx=13),
    "dit_xl2_256_cfg_cross_attention": dict(
        _image_config("XL", 2, 32, DTYPE_BF16, 32, True,
                      "DiT-XL/2 256x256 cross-attention conditioning + CFG, 32 cond + 32 null rows"),
        conditioning=COND_CROSS_ATTENTION, seed_idx=7),
}


def workload(name: str, **overrides) -> dict:
    """Return a copy of a named workload, optionally with fields overridden
    (used by tests to shrink depth, batch or frame count)."""
    cfg = copy.deepcopy(WORKLOADS[name])
    for k, v in overrides.items():
        if k not in cfg:
            raise KeyError(f"unknown workload field {k!r}")
        cfg[k] = v
    if "d" in overrides and "mlp_hidden" not in overrides:
        cfg["mlp_hidden"] = 4 * cfg["d"]
    return cfg


def tokens(cfg: dict) -> int:
    """Number of tokens per row (a plain size helper for allocation)."""
    return (cfg["F"] // cfg["pt"]) * (cfg["H"] // cfg["p"]) * (cfg["W"] // cfg["p"])


# ---------------------------------------------------------------------------
# Rounding helpers (casts, not method arithmetic)

def f32_round(a) -> np.ndarray:
    """fp64 -> fp32, round to nearest even (numpy's cast)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def bf16_round(a) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, returned as an fp32 array whose
    values are exactly representable in bf16."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(a.shape)


def bf16_bits(a) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def cast_to(a, dtype: int) -> np.ndarray:
    """fp64 draws -> the workload dtype (returned as fp32 storage)."""
    a32 = f32_round(a)
    return bf16_round(a32) if dtype == DTYPE_BF16 else a32


# ---------------------------------------------------------------------------
# Weights

def weight_shapes(cfg: dict) -> dict:
    """Shapes of every parameter, Linear weights as [out, in] (in fastest).

    GEMM weights are stored in the workload dtype; biases and the class
    table are fp32.  The adaLN weight stacks all blocks' modulation rows
    followed by the final layer's two rows of width d.
    """
    d, N, C, Cout = cfg["d"], cfg["N"], cfg["C"], cfg["Cout"]
    p, pt, hid, fd = cfg["p"], cfg["pt"], cfg["mlp_hidden"], cfg["freq_dim"]
    kin = pt * p * p * C
    kout = pt * p * p * Cout
    shapes = {
        "pe_w": (d, kin), "pe_b": (d,),
        "t1_w": (d, fd), "t1_b": (d,),
        "t2_w": (d, d), "t2_b": (d,),
    }
    if cfg["num_classes"] > 0:
        shapes["y_table"] = (cfg["num_classes"] + 1, d)
    if cfg["cond_dim"] > 0:
        shapes["pool_w"] = (d, cfg["cond_dim"])
        shapes["pool_b"] = (d,)
    cond = cfg.get("conditioning", COND_ADALN_ZERO)
    if cond in (COND_ADALN_ZERO, COND_MMDIT):
        shapes.update({"ada_w": ((6 * N + 2) * d, d), "ada_b": ((6 * N + 2) * d,)})
    shapes.update({
        "qkv_w": (N, 3 * d, d), "qkv_b": (N, 3 * d),
        "o_w": (N, d, d), "o_b": (N, d),
        "fc1_w": (N, hid, d), "fc1_b": (N, hid),
        "fc2_w": (N, d, hid), "fc2_b": (N, d),
    })
    if cond in (COND_IN_CONTEXT, COND_CROSS_ATTENTION):
        # per block: (shift, scale) of each LayerNorm (2 for in-context, 3 with
        # the cross-attention layer); the final layer's LayerNorm
        n_ln = 2 if cond == COND_IN_CONTEXT else 3
        shapes.update({"ln_p": (N, n_ln, 2, d), "final_ln": (2, d)})
    if cond == COND_CROSS_ATTENTION:
        shapes.update({"xq_w": (N, d, d), "xq_b": (N, d),
                       "xkv_w": (N, 2 * d, d), "xkv_b": (N, 2 * d),
                       "xo_w": (N, d, d), "xo_b": (N, d)})
    if cond == COND_MMDIT:
        dh = d // cfg["heads"]
        shapes.update({"ctx_w": (d, cfg["ctx_dim"]), "ctx_b": (d,),
                       "cada_w": (6 * N * d, d), "cada_b": (6 * N * d,),
                       "cqkv_w": (N, 3 * d, d), "cqkv_b": (N, 3 * d),
                       "co_w": (N, d, d), "co_b": (N, d),
                       "cfc1_w": (N, hid, d), "cfc1_b": (N, hid),
                       "cfc2_w": (N, d, hid), "cfc2_b": (N, d),
                       "qk_rms": (N, 4, dh)})
    shapes.update({"out_w": (kout, d), "out_b": (kout,)})
    return shapes


GEMM_WEIGHTS = ("pe_w", "t1_w", "t2_w", "pool_w", "ada_w", "qkv_w", "o_w",
                "fc1_w", "fc2_w", "out_w", "xq_w", "xkv_w", "xo_w", "ctx_w", "cada_w",
                "cqkv_w", "co_w", "cfc1_w", "cfc2_w")


def make_weights(cfg: dict, seed: int | None = None, std: float = 0.02) -> dict:
    """All parameters ~ N(0, std^2), drawn in a fixed key order.

    GEMM weights are cast to the workload dtype; biases and the class
    table to fp32.  Returns fp32 numpy arrays.
    """
    if seed is None:
        seed = 1000 + cfg["seed_idx"]
    rng = np.random.default_rng(seed)
    out = {}
    for key, shape in weight_shapes(cfg).items():
        n = int(np.prod(shape))
        buf = np.empty(n, dtype=np.float32)
        step = 1 << 24
        for s in range(0, n, step):
            e = min(n, s + step)
            buf[s:e] = f32_round(rng.standard_normal(e - s) * std)
        buf = buf.reshape(shape)
        if key in GEMM_WEIGHTS and cfg["dtype"] == DTYPE_BF16:
            buf = bf16_round(buf)
        out[key] = buf
    return out


def zero_gates(cfg: dict, w: dict) -> dict:
    """adaLN-Zero initialisation of the modulation's last Linear: the rows
    and biases of every block's modulation are set to zero, so every gate
    alpha is 0.  (The final layer's rows are left as drawn.)"""
    w = dict(w)
    d, N = cfg["d"], cfg["N"]
    aw = w["ada_w"].copy()
    ab = w["ada_b"].copy()
    aw[: 6 * N * d] = 0.0
    ab[: 6 * N * d] = 0.0
    w["ada_w"], w["ada_b"] = aw, ab
    return w


def set_gate_bias(cfg: dict, w: dict, value: float, zero_rows: bool = False) -> dict:
    """Set every block's gate bias (alpha1, alpha2 chunks) to ``value``;
    with ``zero_rows`` also zero the gate rows of the weight."""
    w = dict(w)
    d, N = cfg["d"], cfg["N"]
    aw = w["ada_w"].copy()
    ab = w["ada_b"].copy()
    for l in range(N):
        for chunk in (2, 5):
            s = (6 * l + chunk) * d
            ab[s:s + d] = value
            if zero_rows:
                aw[s:s + d] = 0.0
    w["ada_w"], w["ada_b"] = aw, ab
    return w


# ---------------------------------------------------------------------------
# Inputs

def make_inputs(cfg: dict, seed: int | None = None, batch: int | None = None) -> dict:
    """Seeded inputs for one call.

    images: x_t ~ N(0,1) [B, C, H, W]; t ~ U{0..999} (as fp32);
            y ~ U{0..num_classes-1} (int32).
    video:  x0, x1 ~ N(0,1) [B, C, F, H, W]; t ~ U(0,1);
            x_t = t*x1 + (1-t)*x0 (the rectified-flow mix of the GOKU
            review, section 2.3), pooled v ~ N(0,1) [B, cond_dim] (fp32).
    """
    if seed is None:
        seed = 2000 + cfg["seed_idx"]
    B = cfg["batch"] if batch is None else batch
    rng = np.random.default_rng(seed)
    C, F, H, W = cfg["C"], cfg["F"], cfg["H"], cfg["W"]
    res = {}
    if cfg["cond_dim"] > 0:
        shape = (B, C, F, H, W)
        x0 = rng.standard_normal(shape)
        x1 = rng.standard_normal(shape)
        t = rng.uniform(0.0, 1.0, size=B)
        tt = t.reshape(B, 1, 1, 1, 1)
        res["x_t"] = cast_to(tt * x1 + (1.0 - tt) * x0, cfg["dtype"])
        res["t"] = f32_round(t)
        res["y"] = None
        res["pooled"] = f32_round(rng.standard_normal((B, cfg["cond_dim"])))
    else:
        shape = (B, C, H, W) if F == 1 else (B, C, F, H, W)
        res["x_t"] = cast_to(rng.standard_normal(shape), cfg["dtype"])
        res["t"] = rng.integers(0, 1000, size=B).astype(np.float32)
        res["y"] = rng.integers(0, cfg["num_classes"], size=B).astype(np.int32)
        res["pooled"] = None
    return res


def make_sampler_inputs(cfg: dict, steps: int, seed: int | None = None,
                        batch: int | None = None) -> dict:
    """Seeded inputs of a sampling loop: the starting state x ~ N(0,1)
    [B, C, (F,) H, W] and the per-step noise z ~ N(0,1) [steps, B, C, ...],
    both fp32; class labels U{0..num_classes-1} or pooled vectors N(0,1) as
    in :func:`make_inputs`."""
    if seed is None:
        seed = 3000 + cfg["seed_idx"]
    B = cfg["batch"] if batch is None else batch
    rng = np.random.default_rng(seed)
    C, F, H, W = cfg["C"], cfg["F"], cfg["H"], cfg["W"]
    shape = (B, C, F, H, W) if (F > 1 or cfg["rope3d"]) else (B, C, H, W)
    res = {"x": f32_round(rng.standard_normal(shape)),
           "noise": f32_round(rng.standard_normal((steps,) + shape))}
    if cfg["num_classes"] > 0:
        res["y"] = rng.integers(0, cfg["num_classes"], size=B).astype(np.int32)
    else:
        res["y"] = None
    res["pooled"] = (f32_round(rng.standard_normal((B, cfg["cond_dim"])))
                     if cfg["cond_dim"] > 0 else None)
    return res


def make_mmdit_inputs(cfg: dict, seed: int | None = None, batch: int | None = None) -> dict:
    """Seeded inputs of an MMDiT call: image latent x_t ~ N(0,1) [B, C, H, W]
    and text embeddings ~ N(0,1) [B, ctx_len, ctx_dim], both in the model
    dtype; flow time t ~ U(0,1); pooled vector ~ N(0,1) [B, cond_dim] fp32."""
    if seed is None:
        seed = 2000 + cfg["seed_idx"]
    B = cfg["batch"] if batch is None else batch
    rng = np.random.default_rng(seed)
    return {"x_t": cast_to(rng.standard_normal((B, cfg["C"], cfg["H"], cfg["W"])), cfg["dtype"]),
            "t": f32_round(rng.uniform(0.0, 1.0, size=B)),
            "ctx": cast_to(rng.standard_normal((B, cfg["ctx_len"], cfg["ctx_dim"])), cfg["dtype"]),
            "pooled": f32_round(rng.standard_normal((B, cfg["cond_dim"])))}


def make_train_inputs(cfg: dict, seed: int | None = None, batch: int | None = None,
                      label_drop: float = 0.1) -> dict:
    """Seeded inputs of one training step: clean latents x0 ~ N(0,1) and noise
    ~ N(0,1) [B, C, H, W] fp32, integer steps t ~ U{0..999}, labels ~
    U{0..num_classes-1} of which a fraction label_drop (drawn per row) is
    replaced by the null label num_classes (training for guidance)."""
    if seed is None:
        seed = 4000 + cfg["seed_idx"]
    B = cfg["batch"] if batch is None else batch
    rng = np.random.default_rng(seed)
    shape = (B, cfg["C"], cfg["H"], cfg["W"])
    x0 = f32_round(rng.standard_normal(shape))
    noise = f32_round(rng.standard_normal(shape))
    t = rng.integers(0, 1000, size=B).astype(np.int32)
    y = rng.integers(0, cfg["num_classes"], size=B).astype(np.int32)
    y[rng.random(B) < label_drop] = cfg["num_classes"]
    return {"x0": x0, "noise": noise, "t": t, "y": y}
