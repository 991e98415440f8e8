"""Plain fp64 CPU oracle for the DiT denoiser forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library and its Python binding never import, call or load anything here,
and this package imports nothing from them.

Sources (web pages; section names as printed on each page):
  [DiT-wiki]  itwiki "확산 트랜스포머" (Diffusion Transformer)
  [Sora-cvl]  cv-learn.com "Sora / DiT"
  [Sora-obs]  obsidian-dorae222 "Sora: 확산 기반 비디오 생성 모델"
  [DiT-coin]  cointeeth "소라와 안정적 확산 3을 만든 DiT는 무엇인가요?"
  [Goku]      blog.outta.ai "[2025-1] GOKU: Flow Based Video Generative
              Foundation Models" (review)

Pins (what each function is checked against, in tests/test_oracle_*.py):
  patchify / unpatchify      brute-force index loops; exact round trip;
                             torch conv2d(kernel=stride=p) equivalence
  timestep_embedding         closed-form values (t=0, unit-circle pairs,
                             shift invariance of inner products)
  pos_embed_2d               closed-form values (origin, axis separation)
  layer_norm, gelu_tanh,
  silu                       torch fp64 library routines
  attention                  brute-force loops; torch MultiheadAttention;
                             T=1 and equal-key special cases
  qk_layernorm, rope3d       torch layer_norm; rotation invariants
                             (norm, relative position, position 0)
  block                      independent torch.nn fp64 composition of the
                             DiTBlock structure; zero-gate identity
  forward                    independent torch.nn fp64 composition of the
                             whole denoiser at tiny sizes; batch-row
                             independence; token-permutation equivariance
  cfg_combine                s=0 / s=1 / affine-in-s / channel-mask cases
  flops.gmac_per_image       the pages' printed Gflops table
  sampler_oracle             forward process composed step by step (schedule);
                             Gaussian conditioning of (x_s, x_t | x_0) (reverse
                             mean and variance); learned-variance endpoints;
                             closed-form Gaussian-data laws and flow maps
                             (ancestral chain returns the data law, DDIM and
                             Euler first order, DPM-Solver++(2M) second
                             order, point masses hit exactly); DDIM identity
  train_oracle               torch restatement of the forward equals forward;
                             autograd gradients equal central finite
                             differences of the numpy loss (stop-gradient
                             mean frozen); posterior coefficients from the
                             product of Gaussians; KL / NLL against numerical
                             integration; constant-output closed form;
                             AdamW first-step closed form
Full-size forward values: parity unpinned beyond the stage pins above
(the pages print no output tensors and no trained weights exist).
"""
from .dit_oracle import (  # noqa: F401
    patchify, unpatchify, timestep_embedding, pos_embed_2d, layer_norm,
    modulate, silu, gelu_tanh, linear, attention, qk_layernorm, rope3d,
    rope3d_tables, embed_condition, modulation, block, forward, cfg_forward,
    cfg_combine, token_grid, block_in_context, block_cross_attention, cross_attention,
    class_embedding, block_weights, forward_packed, IN_CONTEXT, CROSS_ATTENTION,
    MMDIT, rms_norm, mmdit_block, mmdit_block_weights, mmdit_forward,
)
from . import flops  # noqa: F401
from . import sampler_oracle  # noqa: F401
from . import train_oracle  # noqa: F401
