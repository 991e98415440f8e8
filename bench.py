"""Benchmark: DiT-XL/2 denoiser forwards/s with classifier-free guidance on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one guided forward pass of the whole hot path (dit_cfg_forward):
32 conditional + 32 null-label rows of a 32x32x4 latent (DiT-XL/2, p = 2,
T = 256, d = 1152, 28 blocks, 16 heads), guidance scale 1.5 on all 4 noise
channels; seeded synthetic inputs and N(0, 0.02) weights, resident in HBM
before timing starts.  Prints one JSON line.

Besides the headline number (K timed steps; the median of five more repeats
of K steps is reported beside it) the line carries
  kernels       every hot kernel of the forward timed alone with HIP events on
                the stream it is launched on, at the forward's shapes and with
                the forward's per-block weights, right after the forward loop
                (at the same sustained clocks): average launch time, launches
                per forward, algorithmic TFLOP/s and GB/s and their fractions
                of the MI355X peaks;
  roofline      the entry of that list with the largest time per forward;
  peaks         the published peaks used, and CU count x max engine clock x
                4096 bf16 FLOP per clock per CU read from rocminfo;
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload on
                this host's cores, extrapolated to whole forwards (CPU model,
                BLAS library and thread count stated).

Other modes (same JSON line, their own metric):
  --workload NAME   another forward configuration; --skip-cpu-baseline for long ones
  --train           one dit_train_step per step at DiT-XL/2 batch 256; roofline
                    of the weight-gradient kernel (dit_linear_wgrad)
  --sample KIND     whole dit_sample loops (ddpm, dpmpp_2m, rf_euler)
  --packed          one packed call over latents of two sizes
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "DiT-XL/2 denoiser forwards/s + TFLOP/s (% MFMA peak) on 1 MI355X"
REPEATS = 5
KERNEL_NAMES = ("layernorm", "qkv", "attention", "out_proj", "fc1", "fc2")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit_xl2_256_cfg")
    ap.add_argument("--kernel-launches", type=int, default=50,
                    help="launches of each hot kernel timed alone (after a few untimed ones)")
    ap.add_argument("--repeats", type=int, default=REPEATS,
                    help="extra repeats of the K timed steps (their median is reported)")
    ap.add_argument("--cpu-rows", type=int, default=2,
                    help="guided rows of the workload the oracle runs for the CPU baseline")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (HBM counter calibration)")
    ap.add_argument("--sample", choices=("ddpm", "dpmpp_2m", "rf_euler"), default=None,
                    help="time whole sampling loops (dit_sample) instead of single forwards")
    ap.add_argument("--sample-steps", type=int, default=25,
                    help="denoiser evaluations per sampling loop")
    ap.add_argument("--train", action="store_true",
                    help="time dit_train_step on the training workload (DiT-XL/2, batch 256)")
    ap.add_argument("--packed", action="store_true",
                    help="time packed mixed-resolution forwards (dit_forward_packed): 16 latents "
                         "of 32x32 and 4 of 64x64 in one call, against the same work as two "
                         "batched calls")
    args = ap.parse_args()
    if args.kernel_launches < 1:
        ap.error("--kernel-launches must be at least 1: the roofline figure comes from "
                 "the hot kernels timed alone")
    return args


# ---------------------------------------------------------------------------
# Work counts (measurement only).

def gmac_per_row(cfg) -> float:
    """Multiply-accumulates (10^9) of one row's forward: every matrix product
    (patch embedding, timestep MLP, pooled projection, per-block modulation,
    q | k | v, attention scores and weighted sum, output projection, FFN, final
    modulation, decoder), the unit of the conditioning-methods table of itwiki
    "확산 트랜스포머" (118.6 for DiT-XL/2 at 256x256).  In-context rows carry two
    more tokens and no modulation; cross-attention adds a query and an output
    projection per token, key/value projections of two context tokens and
    attention over them; MMDiT runs both streams' products and joint
    attention."""
    d, N = cfg["d"], cfg["N"]
    T = (cfg["F"] // cfg["pt"]) * (cfg["H"] // cfg["p"]) * (cfg["W"] // cfg["p"])
    r = cfg["mlp_hidden"] / d
    kin = cfg["pt"] * cfg["p"] ** 2 * cfg["C"]
    kout = cfg["pt"] * cfg["p"] ** 2 * cfg["Cout"]
    cond = cfg.get("conditioning", 0)
    per_tok = (4 + 2 * r) * d * d            # q | k | v, output projection, FFN
    front = T * kin * d + cfg["freq_dim"] * d + d * d + cfg.get("cond_dim", 0) * d
    back = T * d * kout
    if cond == 3:                            # MMDiT: image + text streams, joint attention
        J = T + cfg["ctx_len"]
        blocks = N * (J * per_tok + 2 * J * J * d + 12 * d * d)
        front += cfg["ctx_len"] * cfg["ctx_dim"] * d
        back += 2 * d * d
    elif cond == 1:                          # in-context: two more tokens, no modulation
        T2 = T + 2
        blocks = N * (T2 * per_tok + 2 * T2 * T2 * d)
    elif cond == 2:                          # cross-attention: no modulation
        blocks = N * (T * per_tok + 2 * T * T * d + 2 * T * d * d + 4 * d * d + 4 * T * d)
    else:                                    # adaLN-Zero
        blocks = N * (T * per_tok + 2 * T * T * d + 6 * d * d)
        back += 2 * d * d
    return (blocks + front + back) / 1e9


def tokens_of(cfg) -> int:
    return (cfg["F"] // cfg["pt"]) * (cfg["H"] // cfg["p"]) * (cfg["W"] // cfg["p"])


# ---------------------------------------------------------------------------
# Machine facts (printed beside the numbers).

def rocminfo_peak():
    """(compute units, max engine clock MHz, bf16 TFLOP/s = CUs x clock x 4096)
    of the first gfx950 agent in rocminfo, or None."""
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:
        return None
    for block in txt.split("Agent ")[1:]:
        if "gfx950" not in block:
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", block)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", block)
        if cu and mhz:
            cus, clk = int(cu.group(1)), int(mhz.group(1))
            return cus, clk, round(cus * clk * 1e6 * 4096 / 1e12, 1)
    return None


def cpu_facts():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return model, blas


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def measured_traffic(rec_name: str, src_rel: str, kernel: str, shape):
    """HBM bytes per launch of `kernel` at `shape` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record profiles/`rec_name` (each counter scaled by the
    factor a plain copy of known size gave), or None when there is no record for this
    kernel and shape or the kernel source changed since it was taken."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", rec_name)
    try:
        rec = json.load(open(rec_path))
        src = open(os.path.join(ROOT, src_rel), "rb").read()
    except OSError:
        return None
    if (rec.get("kernel") != kernel or rec.get("shape") != list(shape)
            or rec.get("source_sha256") != hashlib.sha256(src).hexdigest()):
        return None
    return int(rec["traffic_bytes"])


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle (the only use of oracle/ here).

def cpu_baseline_mmdit(cfg, w, inp, rows: int, trunk_rows: int):
    """fp64 oracle on `rows` of the MMDiT workload's rows."""
    import oracle
    t0 = time.perf_counter()
    oracle.mmdit_forward(cfg, w, inp["x_t"][:rows], inp["t"][:rows], inp["ctx"][:rows],
                         inp["pooled"][:rows])
    dt = time.perf_counter() - t0
    return {"value": rows / trunk_rows / dt, "unit": "forwards/s", "cores": blas_threads(),
            "kind": "oracle", "extrapolated": True,
            "sample": f"oracle.mmdit_forward (fp64 NumPy) on {rows} of {trunk_rows} rows (all "
                      f"{cfg['N']} blocks): {dt:.2f} s; value scaled to whole {trunk_rows}-row "
                      f"forwards"}


def cpu_baseline_video(cfg, w, inp):
    """fp64 oracle for the spacetime workload: the embedding and conditioning,
    one full-length block (attention over all T tokens, in query chunks) and
    the final layer, timed on this host; the forward is extrapolated as
    embed + N x block + final."""
    import oracle
    d, N = cfg["d"], cfg["N"]
    t0 = time.perf_counter()
    _, _, c = oracle.embed_condition(cfg, w, inp["t"], None, inp["pooled"])
    mod = oracle.modulation(cfg, w, c)
    P = oracle.patchify(inp["x_t"], cfg["p"], cfg["pt"])
    X = oracle.linear(P, w["pe_w"], w["pe_b"])
    t_embed = time.perf_counter() - t0
    rope = oracle.rope3d_tables(cfg["F"] // cfg["pt"], cfg["H"] // cfg["p"], cfg["W"] // cfg["p"],
                                d // cfg["heads"])
    t0 = time.perf_counter()
    X, _, _ = oracle.block(cfg, oracle.block_weights(w, 0), X, mod[:, :6 * d], rope)
    t_block = time.perf_counter() - t0
    t0 = time.perf_counter()
    fb = 6 * d * N
    H = oracle.modulate(oracle.layer_norm(X), mod[:, fb:fb + d], mod[:, fb + d:fb + 2 * d])
    oracle.linear(H, w["out_w"], w["out_b"])
    t_final = time.perf_counter() - t0
    total = t_embed + N * t_block + t_final
    return {"value": 1.0 / total, "unit": "forwards/s", "cores": blas_threads(), "kind": "oracle",
            "extrapolated": True,
            "sample": f"oracle (fp64 NumPy): embedding {t_embed:.2f} s + one full-length block "
                      f"(T = {tokens_of(cfg)}, attention in 2048-query chunks) {t_block:.2f} s "
                      f"x {N} blocks + final layer {t_final:.2f} s = {total:.1f} s per forward "
                      f"(extrapolated from one block)"}


def cpu_baseline(cfg, w, inp, rows: int, trunk_rows: int):
    """fp64 oracle on `rows` guided rows (2*rows trunk rows) of the workload."""
    import oracle
    if cfg.get("conditioning", 0) == 3:
        r = cpu_baseline_mmdit(cfg, w, inp, rows, trunk_rows)
    elif tokens_of(cfg) >= 4096:
        r = cpu_baseline_video(cfg, w, inp)
    elif cfg["cfg"]:
        t0 = time.perf_counter()
        oracle.cfg_forward(cfg, w, inp["x_t"][:rows], inp["t"][:rows], inp["y"][:rows],
                           cfg["scale"], cfg["guided"])
        dt = time.perf_counter() - t0
        frac = (2 * rows) / trunk_rows
        r = {"value": frac / dt, "unit": "forwards/s", "cores": blas_threads(), "kind": "oracle",
             "extrapolated": True,
             "sample": f"oracle.cfg_forward (fp64 NumPy) on {rows} of {trunk_rows // 2} guided "
                       f"rows ({2 * rows} of {trunk_rows} trunk rows, all {cfg['N']} blocks): "
                       f"{dt:.2f} s; value scaled to whole {trunk_rows}-row forwards"}
    else:
        t0 = time.perf_counter()
        oracle.forward(cfg, w, inp["x_t"][:rows], inp["t"][:rows],
                       None if inp.get("y") is None else inp["y"][:rows],
                       None if inp.get("pooled") is None else inp["pooled"][:rows])
        dt = time.perf_counter() - t0
        r = {"value": rows / trunk_rows / dt, "unit": "forwards/s", "cores": blas_threads(),
             "kind": "oracle", "extrapolated": True,
             "sample": f"oracle.forward (fp64 NumPy) on {rows} of {trunk_rows} rows (all "
                       f"{cfg['N']} blocks): {dt:.2f} s; value scaled to whole forwards"}
    model, blas = cpu_facts()
    r["cpu_model"] = model
    r["blas"] = blas
    return r


# ---------------------------------------------------------------------------
# Hot kernels timed alone.

def time_launches(fn, n, stream):
    """Average ms of one launch of fn over n launches (after 3 untimed), HIP
    events on `stream` (the stream the library launches on)."""
    import torch
    for i in range(3):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def kernel_table(cfg, model, rows, n_launch, dev, in_forward):
    """The forward's hot kernels at its shapes: the four block products
    (wide-tile MFMA GEMM with the forward's epilogue), attention and LayerNorm +
    modulate.

    in_forward: {kernel: [ms per launch]} from the library's launch timer over
    forwards (a HIP event pair on the forward's stream around each launch);
    where a kernel has such launches their average is its figure
    (``"timing": "in forward"``).  Each kernel is also timed alone, n_launch
    launches in a row (the GEMMs cycling through the blocks' weights, as the
    forward does, so no launch finds its weight matrix cached), reported as
    ``avg_launch_us_alone`` and used where the forward has no timed launches
    of it (the designs without adaLN-Zero blocks)."""
    import torch
    import diffusion_transformer_denoiser_amd as dm
    d, hid, H, N = cfg["d"], cfg["mlp_hidden"], cfg["heads"], cfg["N"]
    T = model.Tt
    M = rows * T
    dt = dm.torch_dtype(cfg["dtype"])
    es = 2 if dt == torch.bfloat16 else 4
    dh = d // H
    stream = torch.cuda.current_stream(dev)
    tw = model.tensors
    g = torch.Generator(device=dev).manual_seed(7)

    Hb = torch.randn(M, d, device=dev, generator=g).to(dt)
    Gb = torch.randn(M, hid, device=dev, generator=g).to(dt)
    X = torch.randn(M, d, device=dev, generator=g)
    gate = torch.randn((M + T - 1) // T, d, device=dev, generator=g) * 0.1
    qkv = torch.empty(M, 3 * d, device=dev, dtype=dt)
    G = torch.empty(M, hid, device=dev, dtype=dt)

    def gemm(epi, A, Wkey, bkey, outbuf, gated):
        Ws = [tw[Wkey][l] for l in range(N)]
        bs = [tw[bkey][l] for l in range(N)]
        if gated:
            fn = lambda i: dm.linear(epi, A, Ws[i % N], bs[i % N], outbuf, gate=gate,
                                     gate_stride=d, T=T)
        else:
            fn = lambda i: dm.linear(epi, A, Ws[i % N], bs[i % N], outbuf)
        return time_launches(fn, n_launch, stream)

    alone = {
        "qkv": gemm(dm.DIT_EPI_BIAS_DT, Hb, "qkv_w", "qkv_b", qkv, False),
        "out_proj": gemm(dm.DIT_EPI_GATED, Hb, "o_w", "o_b", X, True),
        "fc1": gemm(dm.DIT_EPI_GELU, Hb, "fc1_w", "fc1_b", G, False),
        "fc2": gemm(dm.DIT_EPI_GATED, Gb, "fc2_w", "fc2_b", X, True),
    }
    del G
    qkv.normal_(generator=g)     # attention over the packed q | k | v of every row
    alone["attention"] = time_launches(lambda i: dm.attention(qkv.view(rows, T, 3 * d), H),
                                       n_launch, stream)
    mod = torch.randn(rows, 6 * d, device=dev, generator=g) * 0.1
    Hn = torch.empty(M, d, device=dev, dtype=dt)
    alone["layernorm"] = time_launches(lambda i: dm.ln_modulate(X, mod, 0, d, T, Hn), n_launch,
                                       stream)
    del Hb, Gb, X, qkv, Hn

    epin = {"qkv": "bias", "out_proj": "bias + gated fp32 residual", "fc1": "bias + tanh-GELU",
            "fc2": "bias + gated fp32 residual"}
    shapes = {"qkv": (3 * d, d, False), "out_proj": (d, d, True), "fc1": (hid, d, False),
              "fc2": (d, hid, True)}
    out = []
    for name in ("qkv", "out_proj", "fc1", "fc2", "attention", "layernorm"):
        if name in shapes:
            n_out, n_in, gated = shapes[name]
            flop = 2.0 * M * n_out * n_in
            out_b = M * n_out * (4 if gated else es) * (2 if gated else 1)  # gated: read + write X
            nbytes = M * n_in * es + n_out * n_in * es + n_out * 4 + out_b
            desc = f"{name}: GEMM M={M} N={n_out} K={n_in}, {epin[name]} epilogue"
            per_fwd = N
        elif name == "attention":
            flop, nbytes = 4.0 * rows * H * T * T * dh, rows * T * 4 * d * es
            desc, per_fwd = f"attention: {rows} rows x {H} heads, T={T}, dh={dh}", N
        else:
            flop, nbytes = 0.0, M * d * (4 + es) + rows * 2 * d * 4
            desc, per_fwd = f"LayerNorm + modulate: M={M}, d={d}", 2 * N + 1
        runs = in_forward.get(name, [])
        ms = sum(runs) / len(runs) if runs else alone[name]
        t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12) if flop else 0.0
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
        tf = flop / (ms * 1e-3) / 1e12 if flop else None
        gbs = nbytes / (ms * 1e-3) / 1e9
        out.append({"name": name, "kernel": desc, "launches_per_forward": per_fwd,
                    "avg_launch_us": round(ms * 1e3, 2),
                    "timing": "in forward" if runs else "alone",
                    "launches_timed": len(runs) if runs else n_launch,
                    "avg_launch_us_alone": round(alone[name] * 1e3, 2),
                    "us_per_forward": round(ms * 1e3 * per_fwd, 1),
                    "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                    "tflops": round(tf, 1) if tf else None,
                    "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4) if tf else None,
                    "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                    "algorithmic_flop": flop, "algorithmic_bytes": nbytes})
    return out


def roofline_of(top, traffic=None):
    flop_bound = top["bound"] == "mfma"
    r = {"bound": top["bound"],
         "achieved": top["tflops"] if flop_bound else top["gbs"],
         "peak": PEAK_BF16_TFLOPS if flop_bound else PEAK_HBM_GBS,
         "unit": "TFLOP/s" if flop_bound else "GB/s",
         "frac": top["mfma_frac"] if flop_bound else top["hbm_frac"],
         "traffic": traffic,
         "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE)",
         "algorithmic_bytes": top["algorithmic_bytes"],
         "kernel": top["kernel"],
         "avg_launch_ms": round(top["avg_launch_us"] / 1e3, 5)}
    if traffic:
        gbs = traffic / (top["avg_launch_us"] * 1e-6) / 1e9
        r["hbm_gbs"] = round(gbs, 1)
        r["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4)
    return r


def train_main(args, cfg, model, dev):
    """Training: each timed step is one dit_train_step (forward with saved
    activations, loss, backward, AdamW + EMA) on one batch resident in HBM."""
    import torch
    import dit_inputs

    B = cfg["batch"]
    inp = dit_inputs.make_train_inputs(cfg)
    x0, noise, t, y = (torch.from_numpy(inp[k]).to(dev) for k in ("x0", "noise", "t", "y"))
    model.train_init()
    loss = torch.empty(2, device=dev)
    k = 0
    for _ in range(args.warmup):
        k += 1
        model.train_step(x0, y, t, noise, step=k, loss=loss)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        k += 1
        model.train_step(x0, y, t, noise, step=k, loss=loss)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1) / args.steps
    lv = loss.cpu().tolist()
    assert all(math.isfinite(v) for v in lv), "non-finite loss"
    # forward MACs x 3 (the backward computes two products per forward product)
    flop_step = 3 * 2.0 * gmac_per_row(cfg) * 1e9 * B

    # Dominant kernel of the step: the weight-gradient product (TN MFMA GEMM
    # over the row-major saved activations, split along the token reduction,
    # accumulating atomically into fp32).  Timed alone at the FFN
    # down-projection's shape, dW2 [d, 4d] += dF^T G over all B T tokens with
    # dF [B T, d] and G [B T, 4d], through dit_linear_wgrad, on the stream it
    # is launched on.
    import diffusion_transformer_denoiser_amd as dm
    d, hid = cfg["d"], cfg["mlp_hidden"]
    R = B * dit_inputs.tokens(cfg)
    dF = torch.randn(R, d, device=dev).to(torch.bfloat16)
    G = torch.randn(R, hid, device=dev).to(torch.bfloat16)
    acc = torch.zeros(d, hid, device=dev)
    for _ in range(10):
        dm.linear_wgrad(dF, G, acc)
    stream = torch.cuda.current_stream(dev)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    nk = max(10, args.kernel_launches // 4)
    for _ in range(nk):
        dm.linear_wgrad(dF, G, acc)
    k1.record(stream)
    torch.cuda.synchronize()
    kms = k0.elapsed_time(k1) / nk
    kflop = 2.0 * d * hid * R
    k_tflops = kflop / (kms * 1e-3) / 1e12
    traffic = measured_traffic("gemm_tn_wgrad_hbm_counters.json",
                               "diffusion_transformer_denoiser_amd/csrc/gemm_mfma.hip",
                               "gemm_tn_kernel", (d, hid, R))
    roofline = {"bound": "mfma", "achieved": round(k_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE)",
                "algorithmic_bytes": (d + hid) * R * 2 + d * hid * 4 * 2,
                "kernel": f"gemm_tn_kernel (FFN down-projection weight gradient: dW [{d}, {hid}] "
                          f"over R={R} rows)",
                "avg_launch_ms": round(kms, 4)}
    if traffic:   # counter-measured HBM bytes over the HIP-event launch time
        roofline["hbm_gbs"] = round(traffic / (kms * 1e-3) / 1e9, 1)
        roofline["hbm_frac"] = round(traffic / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    if args.copy_mib:   # calibration copy for the HBM byte counters
        n = args.copy_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    cpu = None
    if not args.skip_cpu_baseline:
        from oracle import train_oracle as TR
        w = {kk: v for kk, v in model.host_weights.items()}
        t0 = time.perf_counter()
        TR.gradients(cfg, w, inp["x0"][:1], inp["y"][:1], inp["t"][:1], inp["noise"][:1])
        dt = time.perf_counter() - t0
        cpu = {"value": 1.0 / (dt * B), "unit": "steps/s", "cores": blas_threads(),
               "kind": "oracle",
               "sample": f"train_oracle.gradients (fp64 torch autograd, all {cfg['N']} blocks) on 1 "
                         f"of {B} rows: {dt:.2f} s; value scaled to whole {B}-row steps (no "
                         f"optimizer update counted)"}
    line = {
        "metric": "DiT-XL/2 training steps/s (forward + backward + AdamW) on 1 MI355X",
        "value": round(1000.0 / ms, 4),
        "unit": "steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == dit_inputs.DTYPE_BF16 else "f32",
        "data": "synthetic (seeded N(0,1) latents and noise, U{0..999} t, random labels with 10% "
                "null, N(0,0.02) weights)",
        "config": {"workload": cfg["name"], "batch": B, "tokens": dit_inputs.tokens(cfg),
                   "parallelism": "single GPU"},
        "images_per_s": round(B * 1000.0 / ms, 1),
        "tflops": round(flop_step / (ms * 1e-3) / 1e12, 1),
        "loss": [round(v, 5) for v in lv],
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def sample_main(args, cfg, model, dev):
    """Sampling loops: each timed step is one dit_sample call of S denoiser
    evaluations plus S update kernels on the workload's batch."""
    import torch
    import dit_inputs
    import diffusion_transformer_denoiser_amd as dm

    S = args.sample_steps
    Bh = cfg["batch"]
    rows = 2 * Bh if cfg["cfg"] else Bh
    guided = cfg["guided"] if cfg["cfg"] else 0
    scale = cfg["scale"] if cfg["cfg"] else 1.0
    inp = dit_inputs.make_sampler_inputs(cfg, S)
    x0 = torch.from_numpy(inp["x"]).to(dev)
    x = x0.clone()
    y = torch.from_numpy(inp["y"]).to(dev) if inp["y"] is not None else None
    pooled = torch.from_numpy(inp["pooled"]).to(dev) if inp["pooled"] is not None else None
    noise = torch.from_numpy(inp["noise"]).to(dev) if args.sample == "ddpm" else None
    sp = dm.Sampler(args.sample, S)

    def loop():
        x.copy_(x0)
        model.sample(sp, x, y=y, pooled=pooled, scale=scale, guided=guided, noise=noise)

    for _ in range(args.warmup):
        loop()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        loop()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1) / args.steps
    assert torch.isfinite(x).all().item(), "non-finite sample"

    # The update kernel alone (the plain-input variant of the same kernel, via
    # dit_sampler_step) at the loop's state size.  One launch takes a few
    # microseconds, less than issuing it from Python, so the launches are
    # captured in a HIP graph and the graph replays are timed with HIP events.
    n_el = x.numel()
    learned = cfg["Cout"] == 2 * cfg["C"]
    mo = torch.randn((x.shape[0], cfg["Cout"]) + tuple(x.shape[2:]), device=dev)
    z = torch.randn_like(x)
    hist = torch.zeros_like(x)
    xs = x0.clone()
    for _ in range(3):
        sp.step(0, xs, mo, z=z, x0_hist=hist, out=xs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.kernel_launches):
            sp.step(0, xs, mo, z=z, x0_hist=hist, out=xs)
    graph.replay()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    k0.record()
    for _ in range(3):
        graph.replay()
    k1.record()
    torch.cuda.synchronize()
    kms = k0.elapsed_time(k1) / (3 * args.kernel_launches)
    # algorithmic bytes per element of step 0: read x and the prediction channel(s),
    # the noise (DDPM) or the x0 history slot (DPM++ writes it), write x
    per = {"ddpm": 4 * (3 + (1 if learned else 0)) + 4, "dpmpp_2m": 4 * 2 + 4 + 4,
           "rf_euler": 4 * 2 + 4}[args.sample]
    gbs = per * n_el / (kms * 1e-3) / 1e9
    gmac_row = gmac_per_row(cfg)
    flop_loop = 2.0 * gmac_row * 1e9 * rows * S
    line = {
        "metric": f"DiT sampling loop images/s ({args.sample}, {S} steps) on 1 MI355X",
        "value": round(Bh * 1000.0 / ms, 3),
        "unit": "images/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == dit_inputs.DTYPE_BF16 else "f32",
        "data": "synthetic (seeded N(0,1) start state and noise, random labels, N(0,0.02) weights)",
        "config": {"workload": cfg["name"], "sampler": args.sample, "sampling_steps": S,
                   "images_per_loop": Bh, "trunk_rows": rows, "guidance_scale": scale,
                   "guided_channels": guided, "parallelism": "single GPU"},
        "ms_per_denoiser_step": round(ms / S, 4),
        "tflops": round(flop_loop / (ms * 1e-3) / 1e12, 1),
        "wall_s_timed": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes": per * n_el,
                     "kernel": f"sampler_step_kernel ({args.sample}, plain input, {n_el} elements)",
                     "avg_launch_ms": round(kms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def packed_main(args, cfg, model, dev):
    """Packed sequences: one dit_forward_packed call over 16 latents of 32x32
    (256x256 images) and 4 of 64x64 (512x512), 8192 tokens, against the same
    sequences as two batched dit_forward calls."""
    import torch
    import dit_inputs
    import diffusion_transformer_denoiser_amd as dm

    shapes = ([(64, 64)] + [(32, 32)] * 4) * 4
    rng = np.random.default_rng(4242)
    dt = dm.torch_dtype(cfg["dtype"])
    xs = [torch.from_numpy(dit_inputs.cast_to(rng.standard_normal((cfg["C"],) + hw), cfg["dtype"]))
          .to(dt).to(dev) for hw in shapes]
    n = len(shapes)
    t = torch.from_numpy(rng.integers(0, 1000, size=n).astype(np.float32)).to(dev)
    y = torch.from_numpy(rng.integers(0, cfg["num_classes"], size=n).astype(np.int32)).to(dev)
    small = [i for i, hw in enumerate(shapes) if hw == (32, 32)]
    large = [i for i, hw in enumerate(shapes) if hw == (64, 64)]
    xs_s = torch.stack([xs[i] for i in small]); xs_l = torch.stack([xs[i] for i in large])
    t_s, t_l = t[small].contiguous(), t[large].contiguous()
    y_s, y_l = y[small].contiguous(), y[large].contiguous()
    cfg_l = dict(cfg, H=64, W=64)
    model_l = dm.DiT(cfg_l, dit_inputs.make_weights(cfg), dev)   # same weights, 64x64 grid

    def packed():
        model.forward_packed(xs, t, y)

    def separate():
        model.forward(xs_s, t_s, y_s)
        model_l.forward(xs_l, t_l, y_l)

    res = {}
    for name, fn in (("packed", packed), ("separate", separate)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / args.steps
    tokens = sum((h // cfg["p"]) * (w // cfg["p"]) for h, w in shapes)
    gmac = sum(gmac_per_row(dict(cfg, H=h, W=w)) for h, w in shapes)
    ms = res["packed"]
    line = {
        "metric": "DiT-XL/2 packed mixed-resolution forward tokens/s on 1 MI355X",
        "value": round(tokens * 1000.0 / ms, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == dit_inputs.DTYPE_BF16 else "f32",
        "data": "synthetic (seeded N(0,1) latents, random t and labels, N(0,0.02) weights)",
        "config": {"workload": "DiT-XL/2 packed: 16 latents of 32x32x4 + 4 of 64x64x4 in one call",
                   "sequences": n, "tokens": tokens, "parallelism": "single GPU"},
        "tflops": round(2.0 * gmac * 1e9 / (ms * 1e-3) / 1e12, 1),
        "separate_batched_ms": round(res["separate"], 4),
        "packed_over_separate": round(res["separate"] / ms, 4),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def forward_main(args, cfg, model, dev, w, inp, x, t, y, pooled, ctx, out):
    import torch
    import dit_inputs
    import diffusion_transformer_denoiser_amd as dm
    mmdit = cfg.get("conditioning", 0) == dit_inputs.COND_MMDIT
    Bh = cfg["batch"]
    rows = 2 * Bh if cfg["cfg"] else Bh

    def step():
        if mmdit:
            model.forward_ctx(x, t, pooled, ctx, out=out)
        elif cfg["cfg"]:
            model.cfg_forward(x, t, y, cfg["scale"], cfg["guided"], out=out)
        else:
            model.forward(x, t, y, pooled, out=out)

    def timed(k):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        ev0.record()
        for _ in range(k):
            step()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / k, time.perf_counter() - wall0

    for _ in range(args.warmup):
        step()
    ms, wall = timed(args.steps)               # the contract's K timed steps
    reps = [timed(args.steps)[0] for _ in range(args.repeats)]
    assert torch.isfinite(out).all().item(), "non-finite output"

    # The block kernels inside forwards: ceil(kernel_launches / depth) more
    # forwards, identical to the timed ones but with the library's launch timer
    # armed (an event pair around each of the blocks' launches).
    T = model.Tt
    in_forward, timer_ms = {}, None
    if not mmdit:
        nf = -(-args.kernel_launches // cfg["N"])
        dm.launch_timer_start(KERNEL_NAMES, nf * 7 * cfg["N"])
        timer_ms = timed(nf)[0]
        in_forward = dm.launch_timer_stop()
    kernels = [] if mmdit else kernel_table(cfg, model, rows, args.kernel_launches, dev,
                                            in_forward)
    roofline = None
    if kernels:
        top = max(kernels, key=lambda k: k["us_per_forward"])
        shape = {"qkv": (rows * T, 3 * cfg["d"], cfg["d"]), "out_proj": (rows * T, cfg["d"], cfg["d"]),
                 "fc1": (rows * T, cfg["mlp_hidden"], cfg["d"]),
                 "fc2": (rows * T, cfg["d"], cfg["mlp_hidden"])}.get(top["name"])
        traffic = None
        if shape:
            traffic = measured_traffic(f"gemm_{top['name']}_hbm_counters.json",
                                       "diffusion_transformer_denoiser_amd/csrc/gemm_wide.hip",
                                       "gemm_wide_kernel", shape)
        roofline = roofline_of(top, traffic)

    if args.copy_mib:   # calibration copy for the HBM byte counters
        n = args.copy_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.skip_cpu_baseline:
        cpu = cpu_baseline(cfg, w, inp, min(args.cpu_rows, Bh), rows)

    flop_fwd = 2.0 * gmac_per_row(cfg) * 1e9 * rows
    tflops = flop_fwd / (ms * 1e-3) / 1e12
    peak_rocm = rocminfo_peak()
    med = statistics.median(reps) if reps else ms
    line = {
        "metric": METRIC,
        "value": round(1000.0 / ms, 3),
        "unit": "forwards/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == dit_inputs.DTYPE_BF16 else "f32",
        "data": ("synthetic (seeded N(0,1) latents and text embeddings, U(0,1) t, N(0,1) "
                 "pooled vector, N(0,0.02) weights)" if mmdit else
                 "synthetic (seeded N(0,1) latents, U(0,1) flow time, N(0,1) pooled vector, "
                 "N(0,0.02) weights)" if cfg["cond_dim"] else
                 "synthetic (seeded N(0,1) latents, U{0..999} t and labels, N(0,0.02) weights)"),
        "config": ({"workload": cfg["name"], "rows": rows, "image_tokens": tokens_of(cfg),
                    "text_tokens": cfg["ctx_len"], "parallelism": "single GPU"} if mmdit else
                   {"workload": cfg["name"], "guided_rows": Bh if cfg["cfg"] else 0,
                    "trunk_rows": rows, "tokens": tokens_of(cfg),
                    "guidance_scale": cfg["scale"], "guided_channels": cfg["guided"],
                    "parallelism": "single GPU"}),
        "tflops": round(tflops, 1),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(rows * T * 1000.0 / ms, 1),
        "images_per_s": round(Bh * 1000.0 / ms, 1),
        "gflop_per_forward": round(flop_fwd / 1e9, 1),
        "wall_s_timed": round(wall, 3),
        "repeats_ms_per_step": [round(r, 4) for r in reps],
        "median_of_repeats": {"ms_per_step": round(med, 4), "value": round(1000.0 / med, 3),
                              "tflops": round(flop_fwd / (med * 1e-3) / 1e12, 1)},
        "peaks": {"bf16_tflops_published": PEAK_BF16_TFLOPS, "hbm_gbs_published": PEAK_HBM_GBS,
                  "rocminfo": ({"compute_units": peak_rocm[0], "max_sclk_mhz": peak_rocm[1],
                                "bf16_tflops_cu_x_clk_x_4096": peak_rocm[2]}
                               if peak_rocm else None)},
        "kernels": kernels,
        "ms_per_step_launch_timer": round(timer_ms, 4) if timer_ms else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the denoiser runs on one GPU; multi-GPU runs are not "
                                   "supported (use --gpus 1)"}), flush=True)
        sys.exit(2)

    import torch
    import dit_inputs
    import diffusion_transformer_denoiser_amd as dm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dm.load()
    dev = torch.device("cuda", torch.cuda.current_device())
    if args.train and args.workload == "dit_xl2_256_cfg":
        args.workload = "dit_xl2_256_train"
    cfg = dit_inputs.workload(args.workload)
    Bh = cfg["batch"]
    w = dit_inputs.make_weights(cfg)
    mmdit = cfg.get("conditioning", 0) == dit_inputs.COND_MMDIT
    inp = dit_inputs.make_mmdit_inputs(cfg) if mmdit else dit_inputs.make_inputs(cfg)
    model = dm.DiT(cfg, w, dev)
    dt = dm.torch_dtype(cfg["dtype"])
    x = torch.from_numpy(inp["x_t"]).to(dt).to(dev)
    t = torch.from_numpy(inp["t"]).to(dev)
    y = torch.from_numpy(inp["y"]).to(dev) if inp.get("y") is not None else None
    pooled = torch.from_numpy(inp["pooled"]).to(dev) if inp["pooled"] is not None else None
    ctx = torch.from_numpy(inp["ctx"]).to(dt).to(dev) if mmdit else None
    out = torch.empty(model.out_shape(Bh), device=dev, dtype=torch.float32)
    if args.sample:
        return sample_main(args, cfg, model, dev)
    if args.train:
        model.host_weights = w
        return train_main(args, cfg, model, dev)
    if args.packed:
        return packed_main(args, cfg, model, dev)
    return forward_main(args, cfg, model, dev, w, inp, x, t, y, pooled, ctx, out)


if __name__ == "__main__":
    main()
