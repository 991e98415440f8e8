"""MI355X (gfx950) DiT denoiser forward pass: a C-ABI HIP library
(``libdit.so``, interface in ``include/dit.h``) and its Python binding.

The binding only marshals arguments; every step of the forward pass runs in
the library's kernels.  Importing the package does not load the library;
``DiT(...)`` and the standalone functions do, and fail loudly if it has not
been built.
"""
from ._lib import (DIT_BF16, DIT_EPI_ACCUM, DIT_EPI_BIAS, DIT_EPI_BIAS_DT, DIT_EPI_GATED,  # noqa: F401
                   DIT_EPI_GELU, DIT_F32, DitError, load)
from .model import (DiT, Sampler, attention, config_struct, launch_timer_start,  # noqa: F401
                    launch_timer_stop, linear, linear_wgrad, ln_modulate, patchify,
                    timestep_embed, torch_dtype, unpatchify, upload)
