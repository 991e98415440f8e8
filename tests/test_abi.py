"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/dit.h, and rejects bad arguments before any launch."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit.h")

from diffusion_transformer_denoiser_amd import _lib  # noqa: E402

needs_lib = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                               reason="libdit.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dit_create", "dit_destroy", "dit_workspace_size", "dit_forward", "dit_cfg_forward",
              "dit_status_string", "dit_patchify", "dit_unpatchify", "dit_timestep_embed",
              "dit_attention", "dit_linear", "dit_linear_wgrad", "dit_block_forward", "dit_sampler_coefficients",
              "dit_sampler_step", "dit_sample_workspace_size", "dit_sample",
              "dit_packed_workspace_size", "dit_forward_packed", "dit_forward_ctx",
              "dit_train_param_count", "dit_train_param_layout", "dit_train_workspace_size",
              "dit_train_step", "dit_forward_noalloc"):
        assert n in names
    assert set(names) == set(_lib.EXPORTS), "binding and header disagree"


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = C.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@needs_lib
def test_config_struct_size_matches_header():
    # 17 ints + 1 float + 3 ints
    assert C.sizeof(_lib.DitConfig) == 21 * 4
    assert C.sizeof(_lib.DitWeights) == 42 * C.sizeof(C.c_void_p)


def _cfg(**kw):
    base = dict(in_channels=4, out_channels=8, frames=1, height=32, width=32, patch=2, patch_t=1,
                hidden=1152, depth=2, heads=16, mlp_hidden=4608, num_classes=1000, cond_dim=0,
                freq_dim=256, qk_norm=0, rope3d=0, dtype=1, ln_eps=1e-6, conditioning=0)
    base.update(kw)
    return _lib.DitConfig(**base)


def _weights(**null):
    # dummy, 256-aligned, never dereferenced by the host code
    w = _lib.DitWeights(**{k: 0x100000 + 256 * i for i, k in enumerate(_lib.WEIGHT_FIELDS)})
    for k in null:
        setattr(w, k, None)
    return w


def _create(cfg, w):
    lib = _lib.load()
    h = C.c_void_p()
    rc = lib.dit_create(C.byref(cfg), C.byref(w), C.byref(h))
    return rc, h


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(height=33), _lib.DIT_EINVAL),            # I % p != 0
    (dict(hidden=1150), _lib.DIT_EINVAL),          # d % heads != 0
    (dict(heads=12), _lib.DIT_EUNSUPPORTED),       # head dim 96
    (dict(hidden=576, heads=9), _lib.DIT_EUNSUPPORTED),   # d % 128 != 0
    (dict(dtype=7), _lib.DIT_EINVAL),
    (dict(freq_dim=255), _lib.DIT_EINVAL),
    (dict(depth=0), _lib.DIT_EINVAL),
    (dict(frames=4), _lib.DIT_EUNSUPPORTED),       # 2-D PE with several frames
    (dict(rope3d=1, hidden=1024), _lib.DIT_EUNSUPPORTED),  # RoPE thirds of dh 64
    (dict(ln_eps=0.0), _lib.DIT_EINVAL),
    (dict(conditioning=4), _lib.DIT_EINVAL),
    (dict(ctx_len=7), _lib.DIT_EINVAL),                              # text tokens without MMDiT
    (dict(conditioning=3, num_classes=0, cond_dim=64, ctx_len=7, ctx_dim=96),
     _lib.DIT_EUNSUPPORTED),                                         # ctx_dim % 64
    (dict(conditioning=3, num_classes=1000, cond_dim=64, ctx_len=7, ctx_dim=64),
     _lib.DIT_EUNSUPPORTED),                                         # MMDiT takes no class table
    (dict(conditioning=3, num_classes=0, cond_dim=0, ctx_len=7, ctx_dim=64),
     _lib.DIT_EUNSUPPORTED),                                         # nor runs without a pooled vector
    (dict(conditioning=3, num_classes=0, cond_dim=64, ctx_len=0, ctx_dim=64),
     _lib.DIT_EUNSUPPORTED),
    (dict(conditioning=1, num_classes=0), _lib.DIT_EUNSUPPORTED),   # needs a class table
    (dict(conditioning=2, cond_dim=4096), _lib.DIT_EUNSUPPORTED),   # no pooled conditioning
])
def test_create_rejects_bad_configs(kw, code):
    rc, h = _create(_cfg(**kw), _weights())
    assert rc == code and not h.value
    assert _lib.load().dit_last_error_message()


@needs_lib
def test_conditioning_designs_check_their_weights():
    lib = _lib.load()
    # the two other designs need no adaLN weights, but their LayerNorm affines
    rc, h = _create(_cfg(conditioning=1), _weights(ada_w=1, ada_b=1))
    assert rc == _lib.DIT_OK
    p = C.c_void_p(0x200000)
    need = C.c_size_t()
    assert lib.dit_workspace_size(h, 4, C.byref(need)) == 0
    assert lib.dit_block_forward(h, 0, 4, p, p, p, None, None, p, need.value,
                                 None) == _lib.DIT_EUNSUPPORTED
    lib.dit_destroy(h)
    rc, _ = _create(_cfg(conditioning=1), _weights(ln_p=1))
    assert rc == _lib.DIT_EINVAL
    rc, _ = _create(_cfg(conditioning=2), _weights(xkv_w=1))
    assert rc == _lib.DIT_EINVAL
    rc, h = _create(_cfg(conditioning=0), _weights(ln_p=1, final_ln=1, xq_w=1))
    assert rc == _lib.DIT_OK
    lib.dit_destroy(h)


@needs_lib
def test_mmdit_design_checks_weights_and_entry_points():
    lib = _lib.load()
    mm = dict(conditioning=3, num_classes=0, cond_dim=64, ctx_len=7, ctx_dim=64)
    rc, _ = _create(_cfg(**mm), _weights(cfc2_w=1))
    assert rc == _lib.DIT_EINVAL
    rc, _ = _create(_cfg(**mm), _weights(qk_rms=1))
    assert rc == _lib.DIT_EINVAL
    rc, h = _create(_cfg(**mm), _weights(y_table=1))
    assert rc == _lib.DIT_OK
    try:
        need = C.c_size_t()
        assert lib.dit_workspace_size(h, 2, C.byref(need)) == 0
        p = C.c_void_p(0x200000)
        # the plain forward takes no text embeddings; the ctx entry needs them
        assert lib.dit_forward(h, p, p, None, p, 2, p, p, need.value, None) == _lib.DIT_EINVAL
        assert lib.dit_forward_ctx(h, p, p, p, None, 2, p, None, p, need.value,
                                   None) == _lib.DIT_EINVAL
        assert lib.dit_forward_ctx(h, p, p, p, p, 2, p, None, p, need.value - 1,
                                   None) == _lib.DIT_EWORKSPACE
        assert lib.dit_forward_ctx(h, p, p, None, p, 2, p, None, p, need.value,
                                   None) == _lib.DIT_EINVAL        # pooled vector missing
        assert lib.dit_block_forward(h, 0, 2, p, p, p, None, None, p, need.value,
                                     None) == _lib.DIT_EUNSUPPORTED
    finally:
        lib.dit_destroy(h)
    # the ctx entry rejects the other designs
    rc, h = _create(_cfg(), _weights())
    assert rc == _lib.DIT_OK
    need = C.c_size_t()
    assert lib.dit_workspace_size(h, 2, C.byref(need)) == 0
    p = C.c_void_p(0x200000)
    assert lib.dit_forward_ctx(h, p, p, None, p, 2, p, None, p, need.value,
                               None) == _lib.DIT_EINVAL
    lib.dit_destroy(h)


@needs_lib
def test_create_rejects_missing_weights():
    rc, _ = _create(_cfg(), _weights(y_table=1))
    assert rc == _lib.DIT_EINVAL
    rc, _ = _create(_cfg(), _weights(fc2_w=1))
    assert rc == _lib.DIT_EINVAL
    rc, _ = _create(_cfg(cond_dim=4096), _weights(pool_w=1))
    assert rc == _lib.DIT_EINVAL


@needs_lib
def test_forward_validates_before_launch():
    lib = _lib.load()
    rc, h = _create(_cfg(), _weights())
    assert rc == _lib.DIT_OK
    try:
        need = C.c_size_t()
        assert lib.dit_workspace_size(h, 64, C.byref(need)) == 0
        assert need.value > 100 << 20            # ~0.4 GB at this size
        p = C.c_void_p(0x200000)
        # B <= 0, null pointers, missing labels, small workspace: no launch, codes only.
        assert lib.dit_forward(h, p, p, p, None, 0, p, p, need.value, None) == _lib.DIT_EINVAL
        assert lib.dit_forward(h, None, p, p, None, 4, p, p, need.value, None) == _lib.DIT_EINVAL
        assert lib.dit_forward(h, p, p, None, None, 4, p, p, need.value, None) == _lib.DIT_EINVAL
        assert lib.dit_forward(h, p, p, p, None, 64, p, p, need.value - 1, None) == _lib.DIT_EWORKSPACE
        assert lib.dit_forward(h, p, p, p, None, 64, p, None, need.value, None) == _lib.DIT_EWORKSPACE
        assert lib.dit_cfg_forward(h, p, p, p, 32, 1.5, 0, p, p, need.value, None) == _lib.DIT_EINVAL
        assert lib.dit_cfg_forward(h, p, p, p, 32, 1.5, 9, p, p, need.value, None) == _lib.DIT_EINVAL
        assert lib.dit_cfg_forward(h, p, p, p, 32, float("nan"), 4, p, p, need.value, None) == _lib.DIT_EINVAL
        assert lib.dit_cfg_forward(h, p, p, p, 33, 1.5, 4, p, p, need.value, None) == _lib.DIT_EWORKSPACE
        assert lib.dit_block_forward(h, 2, 4, p, p, p, None, None, p, need.value, None) == _lib.DIT_EINVAL
        # the workspace-free forward: the same checks, and 64 rows need more
        # than its static scratch (refused before any HIP call)
        assert lib.dit_forward_noalloc(h, p, p, p, None, 0, p, None) == _lib.DIT_EINVAL
        assert lib.dit_forward_noalloc(h, None, p, p, None, 4, p, None) == _lib.DIT_EINVAL
        assert lib.dit_forward_noalloc(h, p, p, None, None, 4, p, None) == _lib.DIT_EINVAL
        assert lib.dit_forward_noalloc(h, p, p, p, None, 64, p, None) == _lib.DIT_EWORKSPACE
        assert lib.dit_forward_noalloc(None, p, p, p, None, 4, p, None) == _lib.DIT_EINVAL
    finally:
        lib.dit_destroy(h)


@needs_lib
def test_sample_validates_before_launch():
    lib = _lib.load()
    rc, h = _create(_cfg(), _weights())
    assert rc == _lib.DIT_OK
    try:
        sp = _lib.DitSampler(kind=_lib.DIT_SAMPLER_DDPM, num_steps=4, train_steps=1000,
                             beta_start=1e-4, beta_end=0.02)
        st = C.byref(sp)
        need = C.c_size_t()
        assert lib.dit_sample_workspace_size(h, st, 32, 4, C.byref(need)) == 0
        fwd = C.c_size_t()
        assert lib.dit_workspace_size(h, 64, C.byref(fwd)) == 0
        assert need.value > fwd.value   # forward workspace of 2B rows plus the loop's buffers
        assert lib.dit_sample_workspace_size(h, st, 32, 9, C.byref(need)) == _lib.DIT_EINVAL
        assert lib.dit_sample_workspace_size(h, st, 32, 4, C.byref(need)) == 0
        p = C.c_void_p(0x200000)
        n = need.value
        assert lib.dit_sample(h, st, p, p, None, 32, 4.0, 4, None, p, n, None) == _lib.DIT_EINVAL
        assert lib.dit_sample(h, st, None, p, None, 32, 4.0, 4, p, p, n, None) == _lib.DIT_EINVAL
        assert lib.dit_sample(h, st, p, None, None, 32, 4.0, 4, p, p, n, None) == _lib.DIT_EINVAL
        assert lib.dit_sample(h, st, p, p, None, 32, float("inf"), 4, p, p, n, None) == _lib.DIT_EINVAL
        assert lib.dit_sample(h, st, p, p, None, 32, 4.0, 4, p, p, n - 1, None) == _lib.DIT_EWORKSPACE
        assert lib.dit_sample(h, st, p, p, None, 32, 4.0, 4, p, None, n, None) == _lib.DIT_EWORKSPACE
        assert lib.dit_sample(h, st, p, p, None, 0, 4.0, 4, p, p, n, None) == _lib.DIT_EINVAL
        bad = _lib.DitSampler(kind=_lib.DIT_SAMPLER_DDPM, num_steps=4, train_steps=3,
                              beta_start=1e-4, beta_end=0.02)
        assert lib.dit_sample(h, C.byref(bad), p, p, None, 32, 4.0, 4, p, p, n, None) == _lib.DIT_EINVAL
    finally:
        lib.dit_destroy(h)
    # Cout must be C or 2C
    rc, h = _create(_cfg(out_channels=5), _weights())
    assert rc == _lib.DIT_OK
    try:
        rf = _lib.DitSampler(kind=_lib.DIT_SAMPLER_RF_EULER, num_steps=4)
        p = C.c_void_p(0x200000)
        assert lib.dit_sample(h, C.byref(rf), p, p, None, 2, 1.0, 0, None, p, 1 << 40,
                              None) == _lib.DIT_EUNSUPPORTED
    finally:
        lib.dit_destroy(h)


@needs_lib
def test_standalone_steps_validate_before_launch():
    lib = _lib.load()
    p = C.c_void_p(0x200000)
    assert lib.dit_patchify(p, 1, 4, 1, 33, 32, 2, 1, 1, p, None) == _lib.DIT_EINVAL
    assert lib.dit_patchify(None, 1, 4, 1, 32, 32, 2, 1, 1, p, None) == _lib.DIT_EINVAL
    assert lib.dit_unpatchify(p, 1, 8, 3, 32, 32, 2, 2, p, None) == _lib.DIT_EINVAL
    assert lib.dit_timestep_embed(p, 4, 255, p, None) == _lib.DIT_EINVAL
    assert lib.dit_attention(p, 1, 2, 16, 96, 1, p, None) == _lib.DIT_EUNSUPPORTED
    assert lib.dit_attention(None, 1, 2, 16, 64, 1, p, None) == _lib.DIT_EINVAL
    assert lib.dit_attention(p, 1, 2, 16, 72, 1, C.c_void_p(0x200004), None) == _lib.DIT_EINVAL
    assert lib.dit_attention(p, 1, 16, 1 << 18, 72, 1, p, None) == _lib.DIT_EUNSUPPORTED
    assert lib.dit_linear(9, p, p, None, 4, 4, 64, 1, p, None, 0, 1, None) == _lib.DIT_EINVAL
    assert lib.dit_linear(0, p, p, None, 4, 4, 48, 1, p, None, 0, 1, None) == _lib.DIT_EUNSUPPORTED
    assert lib.dit_linear(2, p, p, None, 4, 4, 64, 1, p, None, 0, 1, None) == _lib.DIT_EINVAL
    wg = lib.dit_linear_wgrad
    assert wg(None, 8, p, 8, 8, 8, 64, 1, p, None, None) == _lib.DIT_EINVAL
    assert wg(p, 8, p, 8, 8, 8, 64, 1, None, None, None) == _lib.DIT_EINVAL
    assert wg(p, 8, p, 8, 0, 8, 64, 1, p, None, None) == _lib.DIT_EINVAL
    assert wg(p, 8, p, 8, 8, 8, -1, 1, p, None, None) == _lib.DIT_EINVAL
    assert wg(p, 4, p, 8, 8, 8, 64, 1, p, None, None) == _lib.DIT_EINVAL      # ldy < N
    assert wg(p, 8, p, 4, 8, 8, 64, 1, p, None, None) == _lib.DIT_EINVAL      # ldx < K
    assert wg(p, 8, p, 8, 8, 8, 64, 7, p, None, None) == _lib.DIT_EINVAL
    assert wg(p, 8, p, 8, 8, 8, 1 << 31, 1, p, None, None) == _lib.DIT_EUNSUPPORTED
    assert wg(p, 8, p, 8, 8, 8, 0, 1, p, None, None) == _lib.DIT_OK           # nothing to add
    assert wg(p, 8, p, 8, 6, 8, 64, 1, p, p, None) == _lib.DIT_EUNSUPPORTED  # bf16 bias, N % 8
    assert lib.dit_status_string(_lib.DIT_EWORKSPACE) == b"workspace missing or too small"


@needs_lib
def test_packed_forward_validates_before_launch():
    lib = _lib.load()
    rc, h = _create(_cfg(), _weights())
    assert rc == _lib.DIT_OK
    try:
        fhw = (C.c_int32 * 6)(1, 32, 32, 1, 64, 64)
        need = C.c_size_t()
        assert lib.dit_packed_workspace_size(h, 2, fhw, C.byref(need)) == 0
        one = C.c_size_t()
        assert lib.dit_workspace_size(h, 5, C.byref(one)) == 0
        assert need.value > 0
        p = C.c_void_p(0x200000)
        n = need.value
        bad = (C.c_int32 * 3)(1, 31, 32)          # H not divisible by p
        assert lib.dit_forward_packed(h, 1, bad, p, p, p, None, p, p, n, None) == _lib.DIT_EINVAL
        odd = (C.c_int32 * 3)(1, 10, 10)          # 25 tokens: not a multiple of 32
        assert lib.dit_forward_packed(h, 1, odd, p, p, p, None, p, p, n, None) == _lib.DIT_EUNSUPPORTED
        two_frames = (C.c_int32 * 3)(2, 32, 32)
        assert lib.dit_forward_packed(h, 1, two_frames, p, p, p, None, p, p, n,
                                      None) == _lib.DIT_EINVAL
        assert lib.dit_forward_packed(h, 0, fhw, p, p, p, None, p, p, n, None) == _lib.DIT_EINVAL
        assert lib.dit_forward_packed(h, 65, fhw, p, p, p, None, p, p, n, None) == _lib.DIT_EINVAL
        assert lib.dit_forward_packed(h, 2, fhw, p, p, None, None, p, p, n, None) == _lib.DIT_EINVAL
        assert lib.dit_forward_packed(h, 2, fhw, p, p, p, None, p, p, n - 1,
                                      None) == _lib.DIT_EWORKSPACE
        assert lib.dit_forward_packed(h, 2, None, p, p, p, None, p, p, n, None) == _lib.DIT_EINVAL
    finally:
        lib.dit_destroy(h)
    rc, h = _create(_cfg(conditioning=1), _weights())
    try:
        fhw = (C.c_int32 * 3)(1, 32, 32)
        need = C.c_size_t()
        assert lib.dit_packed_workspace_size(h, 1, fhw, C.byref(need)) == _lib.DIT_EUNSUPPORTED
    finally:
        lib.dit_destroy(h)


@needs_lib
def test_train_layout_and_validation():
    lib = _lib.load()
    rc, h = _create(_cfg(depth=2), _weights())
    assert rc == _lib.DIT_OK
    try:
        n = C.c_size_t()
        assert lib.dit_train_param_count(h, C.byref(n)) == 0
        d, N, hid, kin, kout = 1152, 2, 4608, 16, 32
        ms = (6 * N + 2) * d
        sizes = {0: d * kin, 1: d, 2: d * 256, 3: d, 4: d * d, 5: d, 6: 1001 * d, 9: ms * d,
                 10: ms, 11: N * 3 * d * d, 12: N * 3 * d, 13: N * d * d, 14: N * d,
                 15: N * hid * d, 16: N * hid, 17: N * d * hid, 18: N * d, 19: kout * d,
                 20: kout}
        spans = []
        for f in range(len(_lib.WEIGHT_FIELDS)):
            off, cnt = C.c_size_t(), C.c_size_t()
            assert lib.dit_train_param_layout(h, f, C.byref(off), C.byref(cnt)) == 0
            assert cnt.value == sizes.get(f, 0), f
            if cnt.value:
                assert off.value % 64 == 0
                spans.append((off.value, off.value + cnt.value))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert spans[-1][1] <= n.value
        ws = C.c_size_t()
        assert lib.dit_train_workspace_size(h, 4, C.byref(ws)) == 0 and ws.value > 0
        p = C.c_void_p(0x200000)
        hp = _lib.DitTrainHparams(lr=1e-4, beta1=0.9, beta2=0.999, adam_eps=1e-8,
                                  weight_decay=0.0, ema_decay=0.9999, train_steps=1000,
                                  beta_start=1e-4, beta_end=0.02)
        st = _lib.DitTrainState(master=0x300000, grad=0x300000, m=0x300000, v=0x300000,
                                ema=0x300000)
        step = lambda B, k=1, hpp=hp, sz=ws.value: lib.dit_train_step(
            h, C.byref(hpp), k, C.byref(st), p, p, p, p, B, p, p, sz, None)
        assert step(4, k=0) == _lib.DIT_EINVAL                  # step numbers start at 1
        assert step(4, sz=ws.value - 1) == _lib.DIT_EWORKSPACE
        assert step(5) == _lib.DIT_EWORKSPACE                    # sized for 4 rows
        bad = _lib.DitTrainHparams(**{**{k: getattr(hp, k) for k, _ in hp._fields_}, "beta2": 1.0})
        assert step(4, hpp=bad) == _lib.DIT_EINVAL
        bad = _lib.DitTrainHparams(**{**{k: getattr(hp, k) for k, _ in hp._fields_}, "train_steps": 1})
        assert step(4, hpp=bad) == _lib.DIT_EINVAL
    finally:
        lib.dit_destroy(h)
    # bf16 training needs B * T % 64 == 0 (T = 256 here, so any B works); the
    # other designs are rejected
    rc, h = _create(_cfg(conditioning=1), _weights())
    assert rc == _lib.DIT_OK
    n = C.c_size_t()
    assert lib.dit_train_param_count(h, C.byref(n)) == _lib.DIT_EUNSUPPORTED
    lib.dit_destroy(h)
