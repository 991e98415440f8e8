"""Python binding over the C ABI: device memory and streams come from torch;
every step of the forward pass runs in the HIP library.

    model = DiT(cfg, weights)          # uploads weights, dit_create
    eps = model.forward(x_t, t, y)     # dit_forward
    eps = model.cfg_forward(x_t, t, y, scale=1.5, guided=4)   # dit_cfg_forward
    x0 = model.sample(Sampler("ddpm", 250), x_T, y, scale=4.0, guided=4, noise=z)  # dit_sample

``cfg`` is a dict with keys C, Cout, F, H, W, p, pt, d, N, heads, mlp_hidden,
num_classes, cond_dim, freq_dim, qk_norm, rope3d, dtype (0 fp32, 1 bf16),
ln_eps.  ``weights`` maps the names of ``dit_weights`` to arrays in the
layouts of ``include/dit.h``.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib

GEMM_WEIGHTS = ("pe_w", "t1_w", "t2_w", "pool_w", "ada_w", "qkv_w", "o_w", "fc1_w", "fc2_w",
                "out_w", "xq_w", "xkv_w", "xo_w", "ctx_w", "cada_w", "cqkv_w", "co_w", "cfc1_w",
                "cfc2_w")


def torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == _lib.DIT_BF16 else torch.float32


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def config_struct(cfg: dict) -> _lib.DitConfig:
    return _lib.DitConfig(
        in_channels=cfg["C"], out_channels=cfg["Cout"], frames=cfg["F"], height=cfg["H"],
        width=cfg["W"], patch=cfg["p"], patch_t=cfg["pt"], hidden=cfg["d"], depth=cfg["N"],
        heads=cfg["heads"], mlp_hidden=cfg["mlp_hidden"], num_classes=cfg["num_classes"],
        cond_dim=cfg["cond_dim"], freq_dim=cfg["freq_dim"], qk_norm=cfg["qk_norm"],
        rope3d=cfg["rope3d"], dtype=cfg["dtype"], ln_eps=cfg["ln_eps"],
        conditioning=cfg.get("conditioning", _lib.DIT_COND_ADALN_ZERO),
        ctx_len=cfg.get("ctx_len", 0), ctx_dim=cfg.get("ctx_dim", 0))


def upload(a, dtype: torch.dtype, device) -> torch.Tensor:
    """Host array -> contiguous device tensor of ``dtype``."""
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(device)


class Sampler:
    """Host-side description of a sampler (``dit_sampler``).

    kind: "ddpm", "dpmpp_2m" or "rf_euler"; steps: S.  ``timesteps`` (diffusion
    kinds, S ints, decreasing) and ``times`` (RF, S + 1 floats, increasing)
    default to the library's even grids."""
    KINDS = {"ddpm": _lib.DIT_SAMPLER_DDPM, "dpmpp_2m": _lib.DIT_SAMPLER_DPMPP_2M,
             "rf_euler": _lib.DIT_SAMPLER_RF_EULER}

    def __init__(self, kind: str, steps: int, timesteps=None, times=None, train_steps=1000,
                 beta_start=1e-4, beta_end=0.02):
        self.kind, self.steps = kind, int(steps)
        self._ts = None if timesteps is None else (C.c_int32 * len(timesteps))(*map(int, timesteps))
        self._tm = None if times is None else (C.c_double * len(times))(*map(float, times))
        if self._ts is not None and len(self._ts) != self.steps:
            raise ValueError("timesteps needs one entry per step")
        if self._tm is not None and len(self._tm) != self.steps + 1:
            raise ValueError("times needs steps + 1 entries")
        self.struct = _lib.DitSampler(
            kind=self.KINDS[kind], num_steps=self.steps,
            timesteps=C.cast(self._ts, C.POINTER(C.c_int32)) if self._ts is not None else None,
            times=C.cast(self._tm, C.POINTER(C.c_double)) if self._tm is not None else None,
            train_steps=int(train_steps), beta_start=float(beta_start), beta_end=float(beta_end))

    def coefficients(self, k: int):
        """(model time, 8 coefficients) of step k, from the library's host code."""
        lib = _lib.load()
        mt = C.c_double()
        co = (C.c_double * 8)()
        _lib.check(lib.dit_sampler_coefficients(C.byref(self.struct), int(k), C.byref(mt), co))
        return mt.value, list(co)

    def step(self, k: int, x, model_out, z=None, x0_hist=None, out=None):
        """Step k on [B, C, ...] fp32 device tensors (``dit_sampler_step``)."""
        lib = _lib.load()
        B, Cc = x.shape[0], x.shape[1]
        spatial = x[0, 0].numel()
        if out is None:
            out = torch.empty_like(x)
        for name, a in (("x", x), ("model_out", model_out), ("z", z), ("x0_hist", x0_hist),
                        ("out", out)):
            if a is not None and (a.dtype != torch.float32 or not a.is_contiguous()):
                raise TypeError(f"{name} must be a contiguous float32 tensor")
        _lib.check(lib.dit_sampler_step(C.byref(self.struct), int(k), _ptr(x), _ptr(model_out),
                                        B, Cc, model_out.shape[1], spatial, _ptr(z),
                                        _ptr(x0_hist), _ptr(out), _stream(x.device)))
        return out


class DiT:
    def __init__(self, cfg: dict, weights: dict, device="cuda"):
        self.lib = _lib.load()
        self.cfg = dict(cfg)
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.dtype = torch_dtype(cfg["dtype"])
        self.tensors = {}
        for k, a in weights.items():
            dt = self.dtype if k in GEMM_WEIGHTS else torch.float32
            self.tensors[k] = upload(a, dt, self.device)
        self._config = config_struct(cfg)
        self._weights = _lib.DitWeights(**{
            k: (self.tensors[k].data_ptr() if k in self.tensors else None)
            for k in _lib.WEIGHT_FIELDS})
        h = C.c_void_p()
        _lib.check(self.lib.dit_create(C.byref(self._config), C.byref(self._weights), C.byref(h)))
        self.handle = h
        self._ws = None
        self.T = (cfg["F"] // cfg["pt"]) * (cfg["H"] // cfg["p"]) * (cfg["W"] // cfg["p"])
        # tokens per trunk row: the in-context design appends two, MMDiT
        # carries ctx_len text tokens beside the image tokens
        cond = cfg.get("conditioning", 0)
        self.Lc = cfg.get("ctx_len", 0) if cond == _lib.DIT_COND_MMDIT else 0
        self.Tt = self.T + (2 if cond == _lib.DIT_COND_IN_CONTEXT else 0) + self.Lc
        self.Tf = self.T if cond == _lib.DIT_COND_MMDIT else self.Tt   # decoded tokens per row

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self.lib.dit_destroy(h)
            self.handle = None

    # -- memory ---------------------------------------------------------------
    def workspace_bytes(self, rows: int) -> int:
        n = C.c_size_t()
        _lib.check(self.lib.dit_workspace_size(self.handle, rows, C.byref(n)))
        return n.value

    def workspace(self, rows: int) -> torch.Tensor:
        n = self.workspace_bytes(rows)
        if self._ws is None or self._ws.numel() < n:
            self._ws = None
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws

    def out_shape(self, rows: int):
        c = self.cfg
        if c["F"] > 1 or c["rope3d"]:
            return (rows, c["Cout"], c["F"], c["H"], c["W"])
        return (rows, c["Cout"], c["H"], c["W"])

    def make_taps(self, rows: int) -> dict:
        c, M = self.cfg, rows * self.Tt
        kout = c["pt"] * c["p"] * c["p"] * c["Cout"]
        f = dict(device=self.device, dtype=torch.float32)
        return dict(c=torch.empty(rows, c["d"], **f),
                    mod=(torch.empty(rows, (6 * c["N"] + 2) * c["d"], **f)
                         if c.get("conditioning", 0) in (_lib.DIT_COND_ADALN_ZERO,
                                                         _lib.DIT_COND_MMDIT) else None),
                    x_embed=torch.empty(M, c["d"], **f),
                    x_blocks=torch.empty(c["N"], M, c["d"], **f),
                    y_final=torch.empty(rows * self.Tf, kout, **f))

    @staticmethod
    def _taps_struct(taps):
        if taps is None:
            return None
        return C.byref(_lib.DitTaps(**{k: (v.data_ptr() if v is not None else None)
                                        for k, v in taps.items()}))

    # -- forward passes ----------------------------------------------------------
    def forward(self, x_t, t, y=None, pooled=None, out=None, taps=None) -> torch.Tensor:
        B = x_t.shape[0]
        self._check_input(x_t, t, y, pooled, B)
        if out is None:
            out = torch.empty(self.out_shape(B), device=self.device, dtype=torch.float32)
        ws = self.workspace(B)
        if taps is None:
            rc = self.lib.dit_forward(self.handle, _ptr(x_t), _ptr(t), _ptr(y), _ptr(pooled), B,
                                      _ptr(out), _ptr(ws), ws.numel(), _stream(self.device))
        else:
            rc = self.lib.dit_forward_taps(self.handle, _ptr(x_t), _ptr(t), _ptr(y), _ptr(pooled),
                                           B, _ptr(out), self._taps_struct(taps), _ptr(ws),
                                           ws.numel(), _stream(self.device))
        _lib.check(rc)
        return out

    def forward_noalloc(self, x_t, t, y=None, pooled=None, out=None) -> torch.Tensor:
        """``dit_forward_noalloc``: the forward on the library's static scratch
        (no workspace tensor is allocated here either when ``out`` is given)."""
        B = x_t.shape[0]
        self._check_input(x_t, t, y, pooled, B)
        if out is None:
            out = torch.empty(self.out_shape(B), device=self.device, dtype=torch.float32)
        _lib.check(self.lib.dit_forward_noalloc(self.handle, _ptr(x_t), _ptr(t), _ptr(y),
                                                _ptr(pooled), B, _ptr(out),
                                                _stream(self.device)))
        return out

    def forward_ctx(self, x_t, t, pooled, ctx, out=None, taps=None) -> torch.Tensor:
        """MMDiT forward (``dit_forward_ctx``): ctx [B, ctx_len, ctx_dim] text
        embeddings in the model dtype, pooled [B, cond_dim] fp32."""
        B = x_t.shape[0]
        self._check_input(x_t, t, None, pooled, B)
        c = self.cfg
        if (ctx.device != self.device or not ctx.is_contiguous() or ctx.dtype != self.dtype
                or tuple(ctx.shape) != (B, c["ctx_len"], c["ctx_dim"])):
            raise ValueError(f"ctx must be a contiguous {self.dtype} tensor "
                             f"[{B}, {c['ctx_len']}, {c['ctx_dim']}] on {self.device}")
        if out is None:
            out = torch.empty(self.out_shape(B), device=self.device, dtype=torch.float32)
        ws = self.workspace(B)
        _lib.check(self.lib.dit_forward_ctx(self.handle, _ptr(x_t), _ptr(t), _ptr(pooled),
                                            _ptr(ctx), B, _ptr(out), self._taps_struct(taps),
                                            _ptr(ws), ws.numel(), _stream(self.device)))
        return out

    def cfg_forward(self, x_t, t, y, scale: float, guided: int, out=None, taps=None):
        Bh = x_t.shape[0]
        self._check_input(x_t, t, y, None, Bh)
        if out is None:
            out = torch.empty(self.out_shape(Bh), device=self.device, dtype=torch.float32)
        ws = self.workspace(2 * Bh)
        if taps is None:
            rc = self.lib.dit_cfg_forward(self.handle, _ptr(x_t), _ptr(t), _ptr(y), Bh,
                                          float(scale), int(guided), _ptr(out), _ptr(ws),
                                          ws.numel(), _stream(self.device))
        else:
            rc = self.lib.dit_cfg_forward_taps(self.handle, _ptr(x_t), _ptr(t), _ptr(y), Bh,
                                               float(scale), int(guided), _ptr(out),
                                               self._taps_struct(taps), _ptr(ws), ws.numel(),
                                               _stream(self.device))
        _lib.check(rc)
        return out

    def forward_packed(self, xs, t, y=None, pooled=None):
        """Packed sequences (``dit_forward_packed``): xs is a list of latents
        [C, H_i, W_i] (device tensors, model dtype); t [n] fp32, y [n] int32,
        pooled [n, cond_dim].  Returns the list of outputs [Cout, H_i, W_i]."""
        n = len(xs)
        fhw = []
        for a in xs:
            if a.dtype != self.dtype or a.device != self.device:
                raise TypeError(f"latents must be {self.dtype} on {self.device}")
            dims = tuple(a.shape[1:])
            fhw.extend((self.cfg["pt"],) + dims if len(dims) == 2 else dims)
        self._check_input(xs[0], t, y, pooled, n)
        tab = (C.c_int32 * (3 * n))(*fhw)
        x = torch.cat([a.reshape(-1) for a in xs])
        sizes = [self.cfg["Cout"] * a[0].numel() for a in xs]
        out = torch.empty(sum(sizes), device=self.device, dtype=torch.float32)
        nb = C.c_size_t()
        _lib.check(self.lib.dit_packed_workspace_size(self.handle, n, tab, C.byref(nb)))
        if self._ws is None or self._ws.numel() < nb.value:
            self._ws = None
            self._ws = torch.empty(nb.value, dtype=torch.uint8, device=self.device)
        _lib.check(self.lib.dit_forward_packed(self.handle, n, tab, _ptr(x), _ptr(t), _ptr(y),
                                               _ptr(pooled), _ptr(out), _ptr(self._ws),
                                               self._ws.numel(), _stream(self.device)))
        outs, o = [], 0
        for a, sz in zip(xs, sizes):
            outs.append(out[o:o + sz].view((self.cfg["Cout"],) + tuple(a.shape[1:])))
            o += sz
        return outs

    def sample(self, sampler: "Sampler", x, y=None, pooled=None, scale: float = 1.0,
               guided: int = 0, noise=None):
        """Full sampling loop (``dit_sample``) in place on the fp32 state x
        [B, C, (F,) H, W]; returns x.  guided > 0 applies classifier-free
        guidance to that many output channels."""
        B = x.shape[0]
        for name, a in (("x", x), ("y", y), ("pooled", pooled), ("noise", noise)):
            if a is not None and (a.device != self.device or not a.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous tensor on {self.device}")
        if x.dtype != torch.float32 or (noise is not None and noise.dtype != torch.float32):
            raise TypeError("x and noise must be float32")
        if y is not None and (y.dtype != torch.int32 or y.numel() != B):
            raise TypeError("y must be int32 with one entry per row")
        n = C.c_size_t()
        _lib.check(self.lib.dit_sample_workspace_size(self.handle, C.byref(sampler.struct), B,
                                                      int(guided), C.byref(n)))
        if self._ws is None or self._ws.numel() < n.value:
            self._ws = None
            self._ws = torch.empty(n.value, dtype=torch.uint8, device=self.device)
        ws = self._ws
        _lib.check(self.lib.dit_sample(self.handle, C.byref(sampler.struct), _ptr(x), _ptr(y),
                                       _ptr(pooled), B, float(scale), int(guided), _ptr(noise),
                                       _ptr(ws), ws.numel(), _stream(self.device)))
        return x

    # -- training ---------------------------------------------------------------
    def train_init(self):
        """Allocate the fp32 training state (``dit_train_state``): master
        weights copied from the model's current weights, zero Adam moments,
        the EMA equal to the master weights, and the gradient buffer."""
        n = C.c_size_t()
        _lib.check(self.lib.dit_train_param_count(self.handle, C.byref(n)))
        f = dict(device=self.device, dtype=torch.float32)
        self.train_state = {k: torch.zeros(n.value, **f) for k in ("master", "grad", "m", "v", "ema")}
        self.train_fields = {}
        for i, name in enumerate(_lib.WEIGHT_FIELDS):
            off, cnt = C.c_size_t(), C.c_size_t()
            _lib.check(self.lib.dit_train_param_layout(self.handle, i, C.byref(off), C.byref(cnt)))
            if cnt.value:
                self.train_fields[name] = (off.value, cnt.value)
                src = self.tensors[name].reshape(-1).float()
                self.train_state["master"][off.value:off.value + cnt.value] = src
        self.train_state["ema"].copy_(self.train_state["master"])
        self._train_struct = _lib.DitTrainState(**{k: v.data_ptr()
                                                   for k, v in self.train_state.items()})

    def train_view(self, which: str, name: str) -> torch.Tensor:
        """Field ``name`` of state buffer ``which`` ("master", "grad", "m",
        "v", "ema"), shaped like the weight."""
        off, cnt = self.train_fields[name]
        return self.train_state[which][off:off + cnt].view(self.tensors[name].shape)

    def train_step(self, x0, y, t, noise, step: int, lr=1e-4, beta1=0.9, beta2=0.999,
                   adam_eps=1e-8, weight_decay=0.0, ema_decay=0.9999, train_steps=1000,
                   beta_start=1e-4, beta_end=0.02, loss=None) -> torch.Tensor:
        """One optimizer step (``dit_train_step``).  x0, noise: fp32 [B, C, H, W];
        y, t: int32 [B].  Returns the device loss (L_simple, KL term)."""
        B = x0.shape[0]
        for name, a, dt in (("x0", x0, torch.float32), ("noise", noise, torch.float32),
                            ("y", y, torch.int32), ("t", t, torch.int32)):
            if a.device != self.device or not a.is_contiguous() or a.dtype != dt:
                raise ValueError(f"{name} must be a contiguous {dt} tensor on {self.device}")
        if not hasattr(self, "train_state"):
            self.train_init()
        hp = _lib.DitTrainHparams(lr=lr, beta1=beta1, beta2=beta2, adam_eps=adam_eps,
                                  weight_decay=weight_decay, ema_decay=ema_decay,
                                  train_steps=train_steps, beta_start=beta_start,
                                  beta_end=beta_end)
        n = C.c_size_t()
        _lib.check(self.lib.dit_train_workspace_size(self.handle, B, C.byref(n)))
        if self._ws is None or self._ws.numel() < n.value:
            self._ws = None
            self._ws = torch.empty(n.value, dtype=torch.uint8, device=self.device)
        if loss is None:
            loss = torch.empty(2, device=self.device, dtype=torch.float32)
        _lib.check(self.lib.dit_train_step(self.handle, C.byref(hp), int(step),
                                           C.byref(self._train_struct), _ptr(x0), _ptr(y),
                                           _ptr(t), _ptr(noise), B, _ptr(loss), _ptr(self._ws),
                                           self._ws.numel(), _stream(self.device)))
        return loss

    def block_forward(self, layer: int, X, mod, X_out=None, o_branch=None, f_branch=None):
        B = mod.shape[0]
        if X_out is None:
            X_out = torch.empty_like(X)
        ws = self.workspace(B)
        _lib.check(self.lib.dit_block_forward(self.handle, layer, B, _ptr(X), _ptr(mod),
                                              _ptr(X_out), _ptr(o_branch), _ptr(f_branch),
                                              _ptr(ws), ws.numel(), _stream(self.device)))
        return X_out

    def _check_input(self, x_t, t, y, pooled, B):
        for name, a in (("x_t", x_t), ("t", t), ("y", y), ("pooled", pooled)):
            if a is not None and (a.device != self.device or not a.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous tensor on {self.device}")
        if x_t.dtype != self.dtype:
            raise TypeError(f"x_t must be {self.dtype}")
        if t.dtype != torch.float32 or t.numel() != B:
            raise TypeError("t must be float32 with one entry per row")
        if y is not None and (y.dtype != torch.int32 or y.numel() != B):
            raise TypeError("y must be int32 with one entry per row")
        if pooled is not None and pooled.dtype != torch.float32:
            raise TypeError("pooled must be float32")


# ---------------------------------------------------------------------------
# Standalone steps (the same device code as the fused forward pass)

def patchify(x: torch.Tensor, p: int, pt: int = 1) -> torch.Tensor:
    lib = _lib.load()
    x5 = x if x.dim() == 5 else x.unsqueeze(2)
    B, Cc, F, H, W = x5.shape
    code = _lib.DIT_BF16 if x.dtype == torch.bfloat16 else _lib.DIT_F32
    T, K = (F // pt) * (H // p) * (W // p), pt * p * p * Cc
    P = torch.empty(B, T, K, dtype=x.dtype, device=x.device)
    _lib.check(lib.dit_patchify(_ptr(x5.contiguous()), B, Cc, F, H, W, p, pt, code, _ptr(P),
                                _stream(x.device)))
    return P


def unpatchify(Y: torch.Tensor, Cout: int, F: int, H: int, W: int, p: int, pt: int = 1):
    lib = _lib.load()
    B = Y.shape[0]
    out = torch.empty(B, Cout, F, H, W, dtype=torch.float32, device=Y.device)
    _lib.check(lib.dit_unpatchify(_ptr(Y.contiguous()), B, Cout, F, H, W, p, pt, _ptr(out),
                                  _stream(Y.device)))
    return out


def timestep_embed(t: torch.Tensor, dim: int = 256) -> torch.Tensor:
    lib = _lib.load()
    e = torch.empty(t.numel(), dim, dtype=torch.float32, device=t.device)
    _lib.check(lib.dit_timestep_embed(_ptr(t.contiguous()), t.numel(), dim, _ptr(e),
                                      _stream(t.device)))
    return e


def attention(qkv: torch.Tensor, heads: int) -> torch.Tensor:
    """qkv [B, T, 3*heads*dh] packed q | k | v (heads as contiguous slices).
    Returns [B, T, heads*dh]."""
    lib = _lib.load()
    B, T, three_d = qkv.shape
    dh = three_d // (3 * heads)
    code = _lib.DIT_BF16 if qkv.dtype == torch.bfloat16 else _lib.DIT_F32
    o = torch.empty(B, T, heads * dh, dtype=qkv.dtype, device=qkv.device)
    _lib.check(lib.dit_attention(_ptr(qkv.contiguous()), B, heads, T, dh, code, _ptr(o),
                                 _stream(qkv.device)))
    return o


def linear(epilogue: int, A, W, bias, out, gate=None, gate_stride=0, T=1):
    lib = _lib.load()
    M, K = A.shape
    N = W.shape[0]
    code = _lib.DIT_BF16 if A.dtype == torch.bfloat16 else _lib.DIT_F32
    _lib.check(lib.dit_linear(epilogue, _ptr(A), _ptr(W), _ptr(bias), M, N, K, code, _ptr(out),
                              _ptr(gate), gate_stride, T, _stream(A.device)))
    return out


def ln_modulate(X, mod, shift_off, scale_off, T, H, eps=1e-6):
    """H [M, d] = LN(X)(1 + mod[b, scale_off:+d]) + mod[b, shift_off:+d] with
    b = m / T (``dit_ln_modulate``); X [M, d] fp32, mod [rows, stride] fp32,
    H fp32 or bf16."""
    lib = _lib.load()
    M, d = X.shape
    code = _lib.DIT_BF16 if H.dtype == torch.bfloat16 else _lib.DIT_F32
    assert X.dtype == torch.float32 and X.is_contiguous() and H.is_contiguous()
    assert mod.dtype == torch.float32 and mod.is_contiguous()
    _lib.check(lib.dit_ln_modulate(_ptr(X), M, T, d, _ptr(mod), mod.shape[-1], shift_off,
                                   scale_off, eps, _ptr(H), code, _stream(X.device)))
    return H


def linear_wgrad(dY, X, dW, db=None):
    """dW [N, K] fp32 += dY^T X for dY [R, N], X [R, K] (2-D, unit column stride,
    same dtype), and db [N] fp32 += column sums of dY if given: the weight and
    bias gradients of a linear layer."""
    lib = _lib.load()
    R, N = dY.shape
    K = X.shape[1]
    assert X.shape[0] == R and tuple(dW.shape) == (N, K) and dW.dtype == torch.float32
    assert dY.stride(1) == 1 and X.stride(1) == 1 and dW.is_contiguous() and X.dtype == dY.dtype
    code = _lib.DIT_BF16 if dY.dtype == torch.bfloat16 else _lib.DIT_F32
    assert db is None or (db.dtype == torch.float32 and db.numel() == N and db.is_contiguous())
    _lib.check(lib.dit_linear_wgrad(_ptr(dY), dY.stride(0), _ptr(X), X.stride(0), N, K, R, code,
                                    _ptr(dW), _ptr(db), _stream(dY.device)))
    return dW


def launch_timer_start(kinds, capacity: int) -> None:
    """Arm the calling thread's launch timer (``dit_launch_timer_start``): the
    next `capacity` launches of the named block kernels ("layernorm", "qkv",
    "attention", "out_proj", "fc1", "fc2") in this thread's forwards get a HIP
    event pair around them."""
    lib = _lib.load()
    mask = 0
    for k in kinds:
        mask |= 1 << _lib.DIT_TIMER_KIND[k]
    _lib.check(lib.dit_launch_timer_start(mask, capacity))


def launch_timer_stop() -> dict:
    """Wait for the timed launches, release the timer and return
    {kernel name: [ms of each launch, in launch order]}."""
    lib = _lib.load()
    count = C.c_int(0)
    names = {v: k for k, v in _lib.DIT_TIMER_KIND.items()}
    cap = 65536
    kinds = (C.c_int * cap)()
    ms = (C.c_float * cap)()
    _lib.check(lib.dit_launch_timer_stop(kinds, ms, cap, C.byref(count)))
    out = {}
    for i in range(min(count.value, cap)):
        out.setdefault(names[kinds[i]], []).append(float(ms[i]))
    return out

