"""The launch timer (dit_launch_timer_start / _stop): the event pairs it
records around the adaLN-Zero block's launches inside forwards.  It times
every launch of the armed kernels up to its capacity, leaves the forward's
result bit for bit unchanged, and sees only the arming thread's forwards."""
import threading

import numpy as np
import pytest
import torch

import dit_inputs
from tests.parity import device_inputs, log, np_

pytestmark = pytest.mark.gpu
dmod = pytest.importorskip("diffusion_transformer_denoiser_amd")

ALL = ("layernorm", "qkv", "attention", "out_proj", "fc1", "fc2")


@pytest.fixture(scope="module")
def case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dmod.load()
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=3, batch=2)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    x, t, y, _ = device_inputs(cfg, inp)
    yield cfg, m, (lambda: m.cfg_forward(x, t, y, 1.5, 4))
    torch.cuda.synchronize()


def test_every_block_launch_timed_and_output_unchanged(case):
    cfg, m, fwd = case
    N = cfg["N"]
    ref = np_(fwd())
    dmod.launch_timer_start(ALL, 7 * N * 2 + 5)
    out1 = np_(fwd())
    out2 = np_(fwd())
    runs = dmod.launch_timer_stop()
    log(f"timed launches: { {k: len(v) for k, v in runs.items()} }")
    assert np.array_equal(out1, ref) and np.array_equal(out2, ref)
    assert {k: len(v) for k, v in runs.items()} == {
        "layernorm": 4 * N, "qkv": 2 * N, "attention": 2 * N, "out_proj": 2 * N, "fc1": 2 * N,
        "fc2": 2 * N}
    for k, v in runs.items():
        assert all(np.isfinite(v)) and min(v) > 0 and max(v) < 1000, (k, v)
    assert dmod.launch_timer_stop() == {}          # stopping disarmed the timer


def test_capacity_and_kind_mask(case):
    cfg, m, fwd = case
    dmod.launch_timer_start(("fc1", "attention"), 4)
    fwd()
    fwd()
    runs = dmod.launch_timer_stop()
    # launch order within a block: attention before fc1
    assert {k: len(v) for k, v in runs.items()} == {"attention": 2, "fc1": 2}
    fwd()                                          # disarmed: nothing recorded
    assert dmod.launch_timer_stop() == {}


def test_other_threads_are_not_timed(case):
    cfg, m, fwd = case
    dmod.launch_timer_start(("qkv",), 100)
    err = []

    def other():
        try:
            fwd()
            torch.cuda.synchronize()
        except Exception as e:                     # reported below
            err.append(e)

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert not err, err
    fwd()
    runs = dmod.launch_timer_stop()
    assert {k: len(v) for k, v in runs.items()} == {"qkv": cfg["N"]}
