"""Benchmark: DiT-XL/2 denoiser forwards/s with classifier-free guidance on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one guided forward pass of the whole hot path (dit_cfg_forward):
32 conditional + 32 null-label rows of a 32x32x4 latent (DiT-XL/2, p = 2,
T = 256, d = 1152, 28 blocks, 16 heads), guidance scale 1.5 on all 4 noise
channels; seeded synthetic inputs and N(0, 0.02) weights, resident in HBM
before timing starts.  Prints one JSON line.

Besides the headline number the line carries
  roofline      the dominant kernel, timed alone with HIP events on the same
                stream and launch configuration as in the forward pass, right
                after the forward loop (at the same sustained clocks);
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload, on
                this host's cores.

Other modes (same JSON line, their own metric):
  --workload NAME   another forward configuration (its dominant kernel is fc1,
                    or attention at T >= 4096); --skip-cpu-baseline for long ones
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
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "DiT-XL/2 denoiser forwards/s + TFLOP/s (% MFMA peak) on 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit_xl2_256_cfg")
    ap.add_argument("--kernel-launches", type=int, default=200,
                    help="launches of the dominant kernel timed alone (after as many untimed)")
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
    return ap.parse_args()


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


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline_mmdit(cfg, w, inp, rows: int, trunk_rows: int):
    """fp64 oracle on `rows` of the MMDiT workload's rows."""
    import oracle
    t0 = time.perf_counter()
    oracle.mmdit_forward(cfg, w, inp["x_t"][:rows], inp["t"][:rows], inp["ctx"][:rows],
                         inp["pooled"][:rows])
    dt = time.perf_counter() - t0
    return {"value": rows / trunk_rows / dt, "unit": "forwards/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"oracle.mmdit_forward (fp64 NumPy) on {rows} of {trunk_rows} rows (all "
                      f"{cfg['N']} blocks): {dt:.2f} s; value scaled to whole {trunk_rows}-row "
                      f"forwards"}


def cpu_baseline(cfg, w, inp, rows: int, trunk_rows: int):
    """fp64 oracle on `rows` guided rows (2*rows trunk rows) of the workload."""
    import oracle
    if cfg.get("conditioning", 0) == 3:
        return cpu_baseline_mmdit(cfg, w, inp, rows, trunk_rows)
    t0 = time.perf_counter()
    oracle.cfg_forward(cfg, w, inp["x_t"][:rows], inp["t"][:rows], inp["y"][:rows],
                       cfg["scale"], cfg["guided"])
    dt = time.perf_counter() - t0
    frac = (2 * rows) / trunk_rows
    return {"value": frac / dt, "unit": "forwards/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"oracle.cfg_forward (fp64 NumPy) on {rows} of {trunk_rows // 2} guided rows "
                      f"({2 * rows} of {trunk_rows} trunk rows, all 28 blocks): {dt:.2f} s; "
                      f"value scaled to whole {trunk_rows}-row forwards"}


def train_main(args, cfg, model, dev):
    """Training: each timed step is one dit_train_step (forward with saved
    activations, loss, backward, AdamW + EMA) on one batch resident in HBM."""
    import torch
    import dit_inputs
    from oracle import flops as oflops

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
    flop_step = 3 * 2.0 * oflops.gmac_for(cfg) * 1e9 * B

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
    from oracle import flops as oflops

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
    gmac_row = oflops.gmac_for(cfg)
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
    from oracle import flops as oflops

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
    gmac = sum(oflops.gmac_for(dict(cfg, H=h, W=w)) for h, w in shapes)
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
    from oracle import flops as oflops   # closed-form MAC count (numbers only)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dm.load()
    dev = torch.device("cuda", torch.cuda.current_device())
    if args.train and args.workload == "dit_xl2_256_cfg":
        args.workload = "dit_xl2_256_train"
    cfg = dit_inputs.workload(args.workload)
    Bh = cfg["batch"]
    rows = 2 * Bh if cfg["cfg"] else Bh
    T = dit_inputs.tokens(cfg)
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

    def step():
        if mmdit:
            model.forward_ctx(x, t, pooled, ctx, out=out)
        elif cfg["cfg"]:
            model.cfg_forward(x, t, y, cfg["scale"], cfg["guided"], out=out)
        else:
            model.forward(x, t, y, pooled, out=out)

    # Dominant kernel: the FFN up-projection (N = 4d, K = d, bias + tanh-GELU epilogue), the
    # same MFMA kernel, tile and shape as in the forward pass, timed alone.  The forward runs
    # the two halves of its rows on two streams, so each launch there covers M = rows/2 * T.
    # Its buffers are set up before the forward is timed, and it is timed right after the
    # forward loop, with a warm-up of its own, so it runs at the same sustained clocks as
    # inside the forward (an idle GPU needs ~0.1 s of load to reach them).
    # Consecutive launches cycle through the model's per-block weights, as the forward does,
    # so no launch finds its weight matrix already cached.
    d, hid = cfg["d"], cfg["mlp_hidden"]
    # (MMDiT: the image stream's fc1, its largest)
    M = (rows // 2 if rows >= 2 else rows) * (model.Tf if mmdit else model.Tt)
    A = torch.randn(M, d, device=dev).to(dt)
    W1 = [model.tensors["fc1_w"][l] for l in range(cfg["N"])]
    b1 = [model.tensors["fc1_b"][l] for l in range(cfg["N"])]
    G = torch.empty(M, hid, device=dev, dtype=dt)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    nb = len(W1)
    # At video length (T >= 4096) attention, not the FFN, dominates the forward; its
    # kernel is timed alone instead, on one row half's q | k | v.
    attn_dom = T >= 4096 and not mmdit
    if attn_dom:
        Ba, H = (rows // 2 if rows >= 2 else rows), cfg["heads"]
        qkvs = [torch.randn(Ba, model.Tt, 3 * d, device=dev).to(dt) for _ in range(2)]
        del A, G
        def kernel(i):
            dm.attention(qkvs[i % 2], H)
    else:
        def kernel(i):
            dm.linear(dm.DIT_EPI_GELU, A, W1[i % nb], b1[i % nb], G)
    for i in range(args.kernel_launches):
        kernel(i)
    k0.record()
    for i in range(args.kernel_launches):
        kernel(i)
    k1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    kms = k0.elapsed_time(k1) / args.kernel_launches
    assert torch.isfinite(out).all().item(), "non-finite output"

    gmac_row = oflops.gmac_for(cfg)
    flop_fwd = 2.0 * gmac_row * 1e9 * rows
    tflops = flop_fwd / (ms * 1e-3) / 1e12
    if attn_dom:
        dh = d // H
        kflop = 4.0 * Ba * H * model.Tt * model.Tt * dh
        k_tflops = kflop / (kms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(k_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
                    "traffic": None,
                    "algorithmic_bytes": Ba * model.Tt * (3 * d + d) * 2,
                    "kernel": f"attn_bf16_kernel<{dh}> (attention of {Ba} row(s): H={H}, "
                              f"T={model.Tt}, dh={dh})",
                    "avg_launch_ms": round(kms, 4)}
    else:
        kflop = 2.0 * M * hid * d
        k_tflops = kflop / (kms * 1e-3) / 1e12
        traffic = measured_traffic("gemm_fc1_hbm_counters.json",
                                   "diffusion_transformer_denoiser_amd/csrc/gemm_mfma.hip",
                                   "gemm_bf16_kernel<5, 128, 192, 64, 2, 1, 1, 1>", (M, hid, d))
        roofline = {"bound": "mfma", "achieved": round(k_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic,
                    "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE)",
                    "algorithmic_bytes": (M * d + hid * d) * 2 + hid * 4 + M * hid * 2,
                    "kernel": f"gemm_bf16_kernel<EPI_GELU,128,192,64> (FFN fc1 of one row half: "
                              f"M={M}, N={hid}, K={d})",
                    "avg_launch_ms": round(kms, 4)}
        if traffic:   # counter-measured HBM bytes over the HIP-event launch time
            roofline["hbm_gbs"] = round(traffic / (kms * 1e-3) / 1e9, 1)
            roofline["hbm_frac"] = round(traffic / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.skip_cpu_baseline:
        cpu = cpu_baseline(cfg, w, inp, min(args.cpu_rows, Bh), rows)

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
        "config": ({"workload": cfg["name"], "rows": rows, "image_tokens": T,
                    "text_tokens": cfg["ctx_len"], "parallelism": "single GPU"} if mmdit else
                   {"workload": cfg["name"], "guided_rows": Bh, "trunk_rows": rows, "tokens": T,
                    "guidance_scale": cfg["scale"], "guided_channels": cfg["guided"],
                    "parallelism": "single GPU"}),
        "tflops": round(tflops, 1),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(rows * model.Tt * 1000.0 / ms, 1),
        "images_per_s": round(Bh * 1000.0 / ms, 1),
        "gflop_per_forward": round(flop_fwd / 1e9, 1),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
