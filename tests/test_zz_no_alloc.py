"""dit_forward_noalloc (the forward on the library's static scratch, for
callers that cannot allocate) against dit_forward with a caller workspace, on
two calls in a row, the second with fewer rows: the same kernels run on the
same rows, so the outputs must be equal bit for bit (stricter than the 2e-2
bf16 / 1e-4 fp32 bound of the forward's parity tests).  Also: a batch whose
workspace exceeds the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import dit_inputs
from diffusion_transformer_denoiser_amd import _lib
from tests.parity import device_inputs, log, np_

import diffusion_transformer_denoiser_amd as dmod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw,rows", [
    ("dit_xl2_256_cfg", dict(N=2), (4, 2)),
    ("dit_s8_f32", dict(N=2), (2, 1)),
    ("video_xl_spacetime", dict(F=1, N=1), (1, 1)),
])
def test_noalloc_matches_forward(name, kw, rows):
    cfg = dit_inputs.workload(name, batch=max(rows), **kw)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    x, t, y, pooled = device_inputs(cfg, inp)
    for B in rows:
        args = [a[:B].contiguous() if a is not None else None for a in (x, t, y, pooled)]
        want = np_(m.forward(*args))
        got = np_(m.forward_noalloc(*args))
        torch.cuda.synchronize()
        log(f"noalloc {name} B={B}: max |diff| {np.abs(got - want).max():.3e}")
        assert np.isfinite(got).all()
        assert np.array_equal(got, want)


def test_noalloc_rejects_oversized_batch():
    cfg = dit_inputs.workload("dit_xl2_256_cfg", N=2, batch=64)
    w = dit_inputs.make_weights(cfg)
    inp = dit_inputs.make_inputs(cfg)
    m = dmod.DiT(cfg, w, "cuda")
    x, t, y, _ = device_inputs(cfg, inp)
    out = torch.full(m.out_shape(64), 7.0, device="cuda")
    with pytest.raises(_lib.DitError) as e:
        m.forward_noalloc(x, t, y, out=out)
    assert e.value.code == _lib.DIT_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was written
