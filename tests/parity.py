"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dit_inputs
import oracle

BF16_TOL = 2e-2      # end-to-end and per-branch bound for the bf16 path
F32_TOL = 1e-4       # bound for the fp32 path


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def device_inputs(cfg, inp, device="cuda"):
    dt = torch.bfloat16 if cfg["dtype"] == dit_inputs.DTYPE_BF16 else torch.float32
    x = torch.from_numpy(inp["x_t"]).to(dt).to(device)
    t = torch.from_numpy(inp["t"]).to(device)
    y = None if inp["y"] is None else torch.from_numpy(inp["y"]).to(device)
    pooled = None if inp["pooled"] is None else torch.from_numpy(inp["pooled"]).to(device)
    return x, t, y, pooled


def oracle_taps(cfg, w, inp, cfg_mode=False, scale=1.5, guided=4):
    taps = {}
    if cfg_mode:
        out = oracle.cfg_forward(cfg, w, inp["x_t"], inp["t"], inp["y"], scale, guided, taps=taps)
    else:
        out = oracle.forward(cfg, w, inp["x_t"], inp["t"], inp["y"], inp["pooled"], taps=taps)
    return out, taps


def compare_taps(cfg, gtaps, otaps, tol, label=""):
    """Per-stage rel-L2 of the GPU taps against the oracle's; returns a dict."""
    d, N = cfg["d"], cfg["N"]
    res = {"c": rel_l2(np_(gtaps["c"]), otaps["c"]),
           "mod": rel_l2(np_(gtaps["mod"]), otaps["mod"]),
           "x_embed": rel_l2(np_(gtaps["x_embed"]), otaps["X0"].reshape(-1, d)),
           "y_final": rel_l2(np_(gtaps["y_final"]), otaps["Y"].reshape(gtaps["y_final"].shape))}
    xb = np_(gtaps["x_blocks"])
    for l in range(N):
        ref = otaps["X"][l].reshape(-1, d)
        res[f"x_block{l}"] = rel_l2(xb[l], ref)
        # the increment of the block isolates its two gated branches
        prev = otaps["X0"].reshape(-1, d) if l == 0 else otaps["X"][l - 1].reshape(-1, d)
        gprev = np_(gtaps["x_embed"]) if l == 0 else xb[l - 1]
        res[f"dx_block{l}"] = rel_l2(xb[l] - gprev, ref - prev)
    log(f"{label} taps rel-L2: " + ", ".join(f"{k}={v:.2e}" for k, v in res.items()))
    bad = {k: v for k, v in res.items() if not v <= tol}
    assert not bad, f"{label}: stages above {tol}: {bad}"
    return res
