"""Seeded generators: determinism, shapes and the bf16 round-to-nearest-even cast."""
import numpy as np
import torch

import dit_inputs


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    # exact ties at bf16 precision, both parities
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], dtype=np.uint32).view(np.float32)
    a = np.concatenate([a, ties])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(dit_inputs.bf16_round(a), ref)
    bits = dit_inputs.bf16_bits(ref)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy(), ref)


def test_generators_are_deterministic_and_shaped():
    cfg = dit_inputs.workload("dit_b4_bf16", N=2, batch=3)
    w1 = dit_inputs.make_weights(cfg)
    w2 = dit_inputs.make_weights(cfg)
    for k, shape in dit_inputs.weight_shapes(cfg).items():
        assert w1[k].shape == shape and np.array_equal(w1[k], w2[k])
        if k in dit_inputs.GEMM_WEIGHTS:
            dit_inputs.bf16_bits(w1[k])          # raises unless bf16-representable
    assert abs(w1["fc1_w"].std() - 0.02) < 1e-3
    i1 = dit_inputs.make_inputs(cfg)
    assert i1["x_t"].shape == (3, 4, 32, 32) and i1["y"].dtype == np.int32
    assert np.all((i1["t"] >= 0) & (i1["t"] <= 999) & (i1["t"] == np.round(i1["t"])))


def test_video_inputs_rectified_flow_mix():
    cfg = dit_inputs.workload("video_xl_spacetime", F=2, H=4, W=6)
    inp = dit_inputs.make_inputs(cfg)
    assert inp["x_t"].shape == (1, 16, 2, 4, 6)
    assert 0.0 < inp["t"][0] < 1.0 and inp["pooled"].shape == (1, 4096)
    assert inp["y"] is None


def test_workload_token_counts():
    T = {n: dit_inputs.tokens(dit_inputs.workload(n)) for n in dit_inputs.WORKLOADS}
    assert T == {"dit_s8_f32": 16, "dit_b4_bf16": 64, "dit_xl2_256_cfg": 256,
                 "dit_xl2_512_cfg": 1024, "video_xl_spacetime": 24960,
                 "dit_xl2_256_cfg_in_context": 256, "dit_xl2_256_cfg_cross_attention": 256,
                 "mmdit_d24_512": 1024, "dit_xl2_256_train": 256}


def test_train_inputs_recipe():
    cfg = dit_inputs.workload("dit_xl2_256_train")
    a = dit_inputs.make_train_inputs(cfg)
    b = dit_inputs.make_train_inputs(cfg)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    assert a["x0"].shape == (256, 4, 32, 32) and a["x0"].dtype == np.float32
    assert a["t"].dtype == np.int32 and a["t"].min() >= 0 and a["t"].max() <= 999
    null = (a["y"] == 1000).mean()
    assert 0.04 < null < 0.18 and a["y"].min() >= 0
