"""ctypes view of ``include/dit.h`` (argument marshalling only).

Loads the in-tree ``libdit.so``; raises ImportError with a clear message if it
has not been built.  There is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit.so")

DIT_OK, DIT_EINVAL, DIT_EUNSUPPORTED, DIT_EWORKSPACE, DIT_EHIP = 0, -1, -2, -3, -4
DIT_F32, DIT_BF16 = 0, 1
DIT_EPI_BIAS, DIT_EPI_GELU, DIT_EPI_GATED, DIT_EPI_ACCUM, DIT_EPI_BIAS_DT = 0, 1, 2, 3, 4
DIT_SAMPLER_DDPM, DIT_SAMPLER_DPMPP_2M, DIT_SAMPLER_RF_EULER = 0, 1, 2
DIT_COND_ADALN_ZERO, DIT_COND_IN_CONTEXT, DIT_COND_CROSS_ATTN, DIT_COND_MMDIT = 0, 1, 2, 3
DIT_TIMER_KIND = {"layernorm": 0, "qkv": 1, "attention": 2, "out_proj": 3, "fc1": 4, "fc2": 5}


class DitConfig(C.Structure):
    _fields_ = [(n, C.c_int) for n in (
        "in_channels", "out_channels", "frames", "height", "width", "patch", "patch_t",
        "hidden", "depth", "heads", "mlp_hidden", "num_classes", "cond_dim", "freq_dim",
        "qk_norm", "rope3d", "dtype")] + [("ln_eps", C.c_float)] + [
        (n, C.c_int) for n in ("conditioning", "ctx_len", "ctx_dim")]


WEIGHT_FIELDS = ("pe_w", "pe_b", "t1_w", "t1_b", "t2_w", "t2_b", "y_table", "pool_w", "pool_b",
                 "ada_w", "ada_b", "qkv_w", "qkv_b", "o_w", "o_b", "fc1_w", "fc1_b", "fc2_w",
                 "fc2_b", "out_w", "out_b", "ln_p", "final_ln", "xq_w", "xq_b", "xkv_w",
                 "xkv_b", "xo_w", "xo_b", "ctx_w", "ctx_b", "cada_w", "cada_b", "cqkv_w",
                 "cqkv_b", "co_w", "co_b", "cfc1_w", "cfc1_b", "cfc2_w", "cfc2_b", "qk_rms")


class DitWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS]


class DitTaps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("c", "mod", "x_embed", "x_blocks", "y_final")]


class DitSampler(C.Structure):
    _fields_ = [("kind", C.c_int), ("num_steps", C.c_int),
                ("timesteps", C.POINTER(C.c_int32)), ("times", C.POINTER(C.c_double)),
                ("train_steps", C.c_int), ("beta_start", C.c_double), ("beta_end", C.c_double)]


class DitTrainHparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("adam_eps", C.c_double), ("weight_decay", C.c_double),
                ("ema_decay", C.c_double), ("train_steps", C.c_int),
                ("beta_start", C.c_double), ("beta_end", C.c_double)]


class DitTrainState(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("master", "grad", "m", "v", "ema")]


EXPORTS = {
    "dit_create": (C.c_int, [C.POINTER(DitConfig), C.POINTER(DitWeights), C.POINTER(C.c_void_p)]),
    "dit_destroy": (None, [C.c_void_p]),
    "dit_workspace_size": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_size_t)]),
    "dit_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int,
                              C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "dit_cfg_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int,
                                  C.c_float, C.c_int, C.c_void_p, C.c_void_p, C.c_size_t,
                                  C.c_void_p]),
    "dit_ln_modulate": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_int,
                                  C.c_int, C.c_int, C.c_float, C.c_void_p, C.c_int, C.c_void_p]),
    "dit_forward_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "dit_forward_taps": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_int, C.c_void_p, C.POINTER(DitTaps), C.c_void_p,
                                   C.c_size_t, C.c_void_p]),
    "dit_cfg_forward_taps": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int,
                                       C.c_float, C.c_int, C.c_void_p, C.POINTER(DitTaps),
                                       C.c_void_p, C.c_size_t, C.c_void_p]),
    "dit_forward_ctx": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_int, C.c_void_p, C.POINTER(DitTaps), C.c_void_p,
                                  C.c_size_t, C.c_void_p]),
    "dit_train_param_count": (C.c_int, [C.c_void_p, C.POINTER(C.c_size_t)]),
    "dit_train_param_layout": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_size_t),
                                         C.POINTER(C.c_size_t)]),
    "dit_train_workspace_size": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_size_t)]),
    "dit_train_step": (C.c_int, [C.c_void_p, C.POINTER(DitTrainHparams), C.c_int,
                                 C.POINTER(DitTrainState), C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_size_t,
                                 C.c_void_p]),
    "dit_status_string": (C.c_char_p, [C.c_int]),
    "dit_last_error_message": (C.c_char_p, []),
    "dit_patchify": (C.c_int, [C.c_void_p] + [C.c_int] * 8 + [C.c_void_p, C.c_void_p]),
    "dit_unpatchify": (C.c_int, [C.c_void_p] + [C.c_int] * 7 + [C.c_void_p, C.c_void_p]),
    "dit_timestep_embed": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "dit_attention": (C.c_int, [C.c_void_p] + [C.c_int] * 5 + [C.c_void_p, C.c_void_p]),
    "dit_linear": (C.c_int, [C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                             C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                             C.c_void_p]),
    "dit_linear_wgrad": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_int, C.c_int,
                                   C.c_int64, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dit_block_forward": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                    C.c_void_p]),
    "dit_sampler_coefficients": (C.c_int, [C.POINTER(DitSampler), C.c_int,
                                           C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "dit_sampler_step": (C.c_int, [C.POINTER(DitSampler), C.c_int, C.c_void_p, C.c_void_p,
                                   C.c_int, C.c_int, C.c_int, C.c_int64, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p]),
    "dit_sample_workspace_size": (C.c_int, [C.c_void_p, C.POINTER(DitSampler), C.c_int, C.c_int,
                                            C.POINTER(C.c_size_t)]),
    "dit_sample": (C.c_int, [C.c_void_p, C.POINTER(DitSampler), C.c_void_p, C.c_void_p,
                             C.c_void_p, C.c_int, C.c_float, C.c_int, C.c_void_p, C.c_void_p,
                             C.c_size_t, C.c_void_p]),
    "dit_packed_workspace_size": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_int32),
                                            C.POINTER(C.c_size_t)]),
    "dit_forward_packed": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_int32), C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_size_t, C.c_void_p]),
    "dit_launch_timer_start": (C.c_int, [C.c_uint, C.c_int]),
    "dit_launch_timer_stop": (C.c_int, [C.POINTER(C.c_int), C.POINTER(C.c_float), C.c_int,
                                        C.POINTER(C.c_int)]),
}

_lib = None


def load() -> C.CDLL:
    """Load libdit.so (once).  Raises ImportError if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m diffusion_transformer_denoiser_amd.build` (hipcc, gfx950)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class DitError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def check(code: int) -> None:
    if code != DIT_OK:
        lib = load()
        detail = lib.dit_last_error_message().decode()
        raise DitError(code, f"{lib.dit_status_string(code).decode()}: {detail}")
