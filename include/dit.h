/*
 * dit.h - C ABI of the MI355X (gfx950) DiT denoiser forward library.
 *
 * The library computes the Diffusion Transformer (DiT) denoiser forward pass
 * and the classifier-free-guidance combine on one GPU:
 *
 *   patchify of a noisy latent into T = (I/p)^2 tokens, linear embedding and
 *   2-D sine-cosine position embedding
 *     (itwiki "확산 트랜스포머" (Diffusion Transformer), section Structure /
 *      Latent space and patchify; cv-learn "Sora / DiT", Method bullets);
 *   conditioning vector c = timestep embedding + class embedding
 *     (same itwiki page, section adaLN-Zero);
 *   N adaLN-Zero blocks
 *       x <- x + a1 * Attn(LN(x)(1 + g1) + b1)
 *       x <- x + a2 * FFN(LN(x)(1 + g2) + b2),  (b1,g1,a1,b2,g2,a2) = Linear(SiLU(c))
 *     (same page, adaLN-Zero equations and Implementation / adaLN-Zero block);
 *   final LayerNorm + adaLN modulation + linear decoder to p x p x Cout per
 *   token, unpatchify (same page, Latent space and patchify);
 *   guidance  eps_hat = eps(null) + s * (eps(c) - eps(null))
 *     (cv-learn "Sora / DiT", classifier-free guidance bullet), optionally on
 *     the first channels only (itwiki page, ImageNet results notes);
 *   spacetime latents: 3-D patches, full attention with Q-K normalisation and
 *   3-D rotary embedding, pooled-vector conditioning
 *     (blog.outta.ai GOKU review, section 2.2; itwiki page, MMDiT section).
 *
 * Conventions
 *   - Every entry point returns an int status (DIT_OK or a negative code).
 *     All arguments are validated before the first kernel launch; on an error
 *     nothing is launched and nothing is written.  dit_last_error_message()
 *     returns a thread-local description of the last error.
 *   - Device pointers are plain HIP device addresses owned by the caller
 *     (weights, inputs, outputs, workspace).  They must stay valid until the
 *     enqueued work has completed.  The library never allocates or frees
 *     device memory and never changes the current device.
 *   - Work is enqueued on the caller's stream only (a hipStream_t passed as
 *     void*; NULL is the default stream) and never synchronises it.  A device
 *     fault surfaces at the caller's next synchronisation.
 *   - A handle is immutable after dit_create and owns no device resources
 *     (no streams, events or memory); it may be used from several
 *     threads/streams at once if every call has its own workspace.
 *   - No C++ exception crosses this interface.
 *
 * Tensor layouts (row-major, last index fastest)
 *   Linear weights      [out, in]   in the model dtype (fp32 or bf16)
 *   biases, class table fp32
 *   x_t                 [B, C, H, W] (frames == 1) or [B, C, F, H, W], model dtype
 *   t                   [B] fp32 (diffusion step 0..999, or flow time in (0,1))
 *   y                   [B] int32 class ids in [0, num_classes]; num_classes is
 *                       the null label.  Labels are not read on the host: a
 *                       label out of range makes that row's output NaN.
 *   pooled              [B, cond_dim] fp32
 *   out                 [B, Cout, H, W] or [B, Cout, F, H, W] fp32
 *   token order         raster over (frame, row, col) of the patch grid
 *   patch vector order  (frame offset, row offset, col offset, channel), channel
 *                       fastest, for pe_w's input and out_w's output.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DIT_OK            0
#define DIT_EINVAL       -1  /* null pointer, bad size, shape not divisible, ... */
#define DIT_EUNSUPPORTED -2  /* valid but without a kernel (head dim, width, dtype) */
#define DIT_EWORKSPACE   -3  /* workspace pointer null or too small */
#define DIT_EHIP         -4  /* a HIP launch reported an error */

/* dtypes */
#define DIT_F32  0
#define DIT_BF16 1

/* Conditioning designs (itwiki "확산 트랜스포머", Conditioning methods table):
 *   DIT_COND_ADALN_ZERO   adaLN-Zero blocks (regressed shift / scale / gate)
 *   DIT_COND_IN_CONTEXT   the time and class embeddings are two extra tokens
 *                         after the T patch tokens (T + 2 tokens through the
 *                         blocks); standard pre-LN blocks
 *                             x <- x + Attn(LN1(x)),  x <- x + FFN(LN2(x))
 *   DIT_COND_CROSS_ATTN   the two embeddings form a length-2 context that a
 *                         multi-head cross-attention layer after each
 *                         self-attention reads (cointeeth DiT article, block
 *                         description):
 *                             x <- x + Attn(LN1(x)),  x <- x + XAttn(LN2(x), ctx),
 *                             x <- x + FFN(LN3(x))
 * In the last two, every LayerNorm has a learned affine written
 * LN(x)(1 + g) + b, residual adds have no gate, and the final layer is
 * LN (affine) + the linear decoder on the patch tokens.  Both need a class
 * table and no pooled conditioning. */
#define DIT_COND_ADALN_ZERO 0
#define DIT_COND_IN_CONTEXT 1
#define DIT_COND_CROSS_ATTN 2
/* MMDiT (itwiki page, MMDiT section): ctx_len text tokens per row (a
 * Linear(ctx_dim, d) of the given text embeddings) and the image patch tokens
 * are one sequence for attention, but each stream has its own adaLN-Zero
 * modulation, LayerNorms, QKV and output projections and FFN; q and k get a
 * per-head RMSNorm with scale 1 + g (g per stream); the pooled vector and the
 * time embedding enter through the modulations; the final layer reads the
 * image stream.  Needs num_classes == 0, no rope3d, ctx_dim % 64 == 0; runs
 * through dit_forward_ctx. */
#define DIT_COND_MMDIT      3

/* Model configuration.  Supported: hidden % 128 == 0, hidden <= 2048,
 * head dim hidden/heads in {64, 72}, mlp_hidden % 64 == 0, freq_dim even.
 * rope3d needs head dim divisible by 6 with an even third (72 works);
 * without rope3d a 2-D sin-cos position embedding is added and the latent
 * must have frames / patch_t == 1. */
typedef struct dit_config {
  int in_channels;   /* C */
  int out_channels;  /* Cout (2C: noise + diagonal covariance; C for velocity) */
  int frames;        /* F (1 for images) */
  int height;        /* H (= I for square images) */
  int width;         /* W */
  int patch;         /* p */
  int patch_t;       /* temporal patch extent (1 for images) */
  int hidden;        /* d */
  int depth;         /* N blocks */
  int heads;
  int mlp_hidden;    /* FFN hidden width (4d) */
  int num_classes;   /* class table rows - 1 (row num_classes = null label); 0 = no table */
  int cond_dim;      /* pooled conditioning width (0 = none) */
  int freq_dim;      /* timestep sinusoid width (256) */
  int qk_norm;       /* 1: LayerNorm over each head's q and k before attention */
  int rope3d;        /* 1: 3-D rotary embedding on q,k; no additive position embedding */
  int dtype;         /* DIT_F32 or DIT_BF16: GEMM operand / activation dtype */
  float ln_eps;      /* LayerNorm epsilon (1e-6) */
  int conditioning;  /* DIT_COND_* */
  int ctx_len;       /* MMDiT: text tokens per row (0 otherwise) */
  int ctx_dim;       /* MMDiT: width of the text embeddings */
} dit_config;

/* Caller-owned device pointers.  "W" = model dtype, "f32" = float.
 * Shapes with N = depth, d = hidden, Kin = patch_t*patch*patch*C,
 * Kout = patch_t*patch*patch*Cout, hid = mlp_hidden. */
typedef struct dit_weights {
  const void*  pe_w;    /* W   [d, Kin]       patch embedding */
  const float* pe_b;    /* f32 [d] */
  const void*  t1_w;    /* W   [d, freq_dim]  timestep MLP layer 1 */
  const float* t1_b;    /* f32 [d] */
  const void*  t2_w;    /* W   [d, d]         timestep MLP layer 2 */
  const float* t2_b;    /* f32 [d] */
  const float* y_table; /* f32 [num_classes + 1, d] (NULL if num_classes == 0) */
  const void*  pool_w;  /* W   [d, cond_dim]  (NULL if cond_dim == 0) */
  const float* pool_b;  /* f32 [d]            (NULL if cond_dim == 0) */
  const void*  ada_w;   /* W   [(6N + 2) d, d] modulation of all blocks, then final layer;
                           block l rows: b1, g1, a1, b2, g2, a2 (d rows each) at 6 d l;
                           final rows: b_f, g_f at 6 d N */
  const float* ada_b;   /* f32 [(6N + 2) d] */
  const void*  qkv_w;   /* W   [N, 3d, d]  packed q | k | v, heads as contiguous slices */
  const float* qkv_b;   /* f32 [N, 3d] */
  const void*  o_w;     /* W   [N, d, d] */
  const float* o_b;     /* f32 [N, d] */
  const void*  fc1_w;   /* W   [N, hid, d] */
  const float* fc1_b;   /* f32 [N, hid] */
  const void*  fc2_w;   /* W   [N, d, hid] */
  const float* fc2_b;   /* f32 [N, d] */
  const void*  out_w;   /* W   [Kout, d]  linear decoder */
  const float* out_b;   /* f32 [Kout] */
  /* in-context / cross-attention designs only (NULL otherwise; ada_w and
   * ada_b are then NULL): */
  const float* ln_p;     /* f32 [N, nLN, 2, d] (b, g) of each block LayerNorm; nLN = 2
                            in-context, 3 cross-attention (LN1, LN2, LN3) */
  const float* final_ln; /* f32 [2, d] (b, g) of the final LayerNorm */
  /* cross-attention design only: */
  const void*  xq_w;    /* W   [N, d, d]   query projection */
  const float* xq_b;    /* f32 [N, d] */
  const void*  xkv_w;   /* W   [N, 2d, d]  key | value projection of the context tokens */
  const float* xkv_b;   /* f32 [N, 2d] */
  const void*  xo_w;    /* W   [N, d, d]   output projection */
  const float* xo_b;    /* f32 [N, d] */
  /* MMDiT only: the text stream's weights (ada_w / qkv_w / ... above are the
   * image stream's) */
  const void*  ctx_w;   /* W   [d, ctx_dim] text-token embedding */
  const float* ctx_b;   /* f32 [d] */
  const void*  cada_w;  /* W   [6N d, d]   text-stream modulation (block order as ada_w) */
  const float* cada_b;  /* f32 [6N d] */
  const void*  cqkv_w;  /* W   [N, 3d, d] */
  const float* cqkv_b;  /* f32 [N, 3d] */
  const void*  co_w;    /* W   [N, d, d] */
  const float* co_b;    /* f32 [N, d] */
  const void*  cfc1_w;  /* W   [N, hid, d] */
  const float* cfc1_b;  /* f32 [N, hid] */
  const void*  cfc2_w;  /* W   [N, d, hid] */
  const float* cfc2_b;  /* f32 [N, d] */
  const float* qk_rms;  /* f32 [N, 4, dh] g of the image q, image k, text q, text k */
} dit_weights;

typedef struct dit_handle dit_handle;

/* Optional intermediate outputs of the trunk (device pointers, any may be
 * NULL).  M = trunk rows * Tt, Tt = T + 2 for the in-context design, else T. */
typedef struct dit_taps {
  float* c;         /* [rows, d]            conditioning vector (the time embedding in
                                            the in-context / cross-attention designs) */
  float* mod;       /* [rows, (6N + 2) d]   all modulation vectors (adaLN-Zero only) */
  float* x_embed;   /* [M, d]               tokens after patch + position embedding
                                            (and the two conditioning tokens) */
  float* x_blocks;  /* [N, M, d]            residual stream after each block */
  float* y_final;   /* [M, Kout]            decoder output before unpatchify */
} dit_taps;

/* Validate cfg, record the weight pointers and plan the kernels.  Allocates
 * only the host-side handle.  Returns DIT_EINVAL / DIT_EUNSUPPORTED on a bad
 * or unsupported configuration. */
int dit_create(const dit_config* cfg, const dit_weights* w, dit_handle** out);

/* Free the host handle (NULL is ignored). */
void dit_destroy(dit_handle* h);

/* Workspace bytes for a trunk of `rows` rows (dit_forward: rows = B;
 * dit_cfg_forward: rows = 2 * Bh). */
int dit_workspace_size(const dit_handle* h, int rows, size_t* bytes);

/* eps_theta(x_t, t, c) for B rows.  y must be non-NULL iff num_classes > 0,
 * pooled non-NULL iff cond_dim > 0.  out: [B, Cout, (F,) H, W] fp32. */
int dit_forward(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                const float* pooled, int B, float* out, void* ws, size_t ws_bytes,
                void* stream);

/* Guided prediction for Bh rows.  The trunk runs 2 Bh rows: row i < Bh with
 * label y[i], row Bh + i with the null label, both reading x_t[i] and t[i].
 * out[i, ch] = u + s (c - u) for ch < guided_channels (c = conditional row,
 * u = null row), out[i, ch] = c for ch >= guided_channels.
 * Needs num_classes > 0 and 1 <= guided_channels <= Cout. */
int dit_cfg_forward(dit_handle* h, const void* x_t, const float* t, const int32_t* y, int Bh,
                    float s, int guided_channels, float* out, void* ws, size_t ws_bytes,
                    void* stream);

/* MMDiT forward for B rows: ctx [B, ctx_len, ctx_dim] text embeddings in the
 * model dtype; pooled as for dit_forward; out [B, Cout, H, W] fp32.  Taps (may
 * be NULL): x_embed / x_blocks hold the image stream's B*T rows followed by
 * the text stream's B*ctx_len rows. */
int dit_forward_ctx(dit_handle* h, const void* x_t, const float* t, const float* pooled,
                    const void* ctx, int B, float* out, const dit_taps* taps, void* ws,
                    size_t ws_bytes, void* stream);

/* dit_forward / dit_cfg_forward that also write the taps (may be NULL). */
int dit_forward_taps(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                     const float* pooled, int B, float* out, const dit_taps* taps, void* ws,
                     size_t ws_bytes, void* stream);
int dit_cfg_forward_taps(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                         int Bh, float s, int guided_channels, float* out,
                         const dit_taps* taps, void* ws, size_t ws_bytes, void* stream);

/* dit_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It uses a static scratch array of 64 MiB that the
 * library holds on every GPU it is loaded on until the process ends (enough
 * for a DiT-XL/2 256x256 forward of 8 rows).  Calls on one GPU share that
 * array, so calls that overlap on one GPU race.  It calls no allocator.
 * DIT_EWORKSPACE when B needs more scratch than that (nothing is launched);
 * DIT_EUNSUPPORTED for the MMDiT design; otherwise as dit_forward. */
int dit_forward_noalloc(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                        const float* pooled, int B, float* out, void* stream);

const char* dit_status_string(int status);
const char* dit_last_error_message(void);

/* ---- Standalone entry points of single path steps (tests, benchmarks) ----
 * Each runs the same device code as the fused forward. */

/* P[b, tau, k] = x[b, c, f*pt + a, i*p + py, j*p + px], tau = (f*gh + i)*gw + j,
 * k = ((a*p + py)*p + px)*C + c.  x: [B, C, F, H, W]; P: [B, T, pt*p*p*C], both
 * in `dtype` (a bit-exact copy). */
int dit_patchify(const void* x, int B, int C, int F, int H, int W, int p, int pt, int dtype,
                 void* P, void* stream);

/* Inverse index map for Cout channels: out[b, c, f, y, x] = Y[b, tau, k].
 * Y: [B, T, pt*p*p*Cout] fp32; out: [B, Cout, F, H, W] fp32. */
int dit_unpatchify(const float* Y, int B, int Cout, int F, int H, int W, int p, int pt,
                   float* out, void* stream);

/* e[b] = [cos(t_b f_k) | sin(t_b f_k)], f_k = 10000^(-k/(dim/2)), dim even.
 * t: [B] fp32; e: [B, dim] fp32. */
int dit_timestep_embed(const float* t, int B, int dim, float* e, void* stream);

/* Multi-head attention core softmax(q k^T / sqrt(dh)) v for every (b, h)
 * (itwiki "확산 트랜스포머", Implementation: nn.MultiheadAttention(d, heads)).
 * qkv: [B, T, 3*H*dh] packed in-projection output, q | k | v, each with heads as
 * contiguous dh slices (16-byte aligned); o: [B, T, H*dh] (token-major, heads
 * concatenated), same dtype, 8-byte aligned.  dh in {64, 72}; B*H <= 65535;
 * T * 3H * dh * 4 < 2^31.  bf16 with dh 72 and T <= 256 runs whole sequences
 * out of LDS, one persistent workgroup per CU. */
int dit_attention(const void* qkv, int B, int H, int T, int dh, int dtype, void* o, void* stream);

/* Linear layer with one of the fused epilogues of the forward pass,
 * out = epilogue(A W^T + bias): A [M, K] and W [N, K] in `dtype`.
 *   DIT_EPI_BIAS:  out fp32 [M, N] = A W^T + bias
 *   DIT_EPI_GELU:  out dtype [M, N] = GELU_tanh(A W^T + bias)
 *   DIT_EPI_GATED: out fp32 [M, N] += gate[(m / T) * gate_stride + n] * (A W^T + bias)
 * bf16 requires K % 64 == 0.  Uses the kernels and tiles of the forward pass. */
#define DIT_EPI_BIAS  0
#define DIT_EPI_GELU  1
#define DIT_EPI_GATED 2
/*   DIT_EPI_ACCUM: out fp32 [M, N] += A W^T (bias must be NULL): the weight-
 *                  gradient product of a training step when A = dY^T, W = X^T.
 *                  The reduction over K is split into slices whose partial
 *                  sums are added atomically (summation order not fixed). */
#define DIT_EPI_ACCUM 3
/*   DIT_EPI_BIAS_DT: out dtype [M, N] = A W^T + bias, rounded to the model
 *                  dtype (the q | k | v in-projection's epilogue). */
#define DIT_EPI_BIAS_DT 4
int dit_linear(int epilogue, const void* A, const void* W, const float* bias, int M, int N,
               int K, int dtype, void* out, const float* gate, int gate_stride, int T,
               void* stream);

/* LayerNorm and adaLN modulation (itwiki "확산 트랜스포머", adaLN-Zero
 * equations: LN without affine, eps inside the square root, then
 * LN(x)(1 + gamma) + beta):  H[m, :] = LN(X[m, :]) (1 + mod[b, scale_off ..]) +
 * mod[b, shift_off ..] with b = m / T and the row of mod at b * mod_stride
 * (mod_stride 0: one row for every token).  X: [M, d] fp32; mod fp32; H:
 * [M, d] in dtype (rounded to nearest even for bf16).  d a multiple of 128 up
 * to 2048; X, H, mod 16-byte aligned, mod_stride and the offsets multiples of
 * 4.  The kernel the forward runs before the q | k | v and FFN-up products. */
int dit_ln_modulate(const float* X, int M, int T, int d, const float* mod, int mod_stride,
                    int shift_off, int scale_off, float eps, void* H, int dtype, void* stream);

/* One adaLN-Zero block (DIT_EUNSUPPORTED for the other designs),
 * teacher-forced: X_out = block_l(X_in) with the given modulation
 * vectors mod [B, 6d] (b1, g1, a1, b2, g2, a2).  X_in, X_out: [B*T, d] fp32
 * (may alias).  o_branch / f_branch (fp32 [B*T, d], may be NULL) receive the
 * attention and FFN branches before their gates.  ws as for dit_forward with
 * rows = B. */
int dit_block_forward(dit_handle* h, int layer, int B, const float* X_in, const float* mod,
                      float* X_out, float* o_branch, float* f_branch, void* ws,
                      size_t ws_bytes, void* stream);

/* ---- Launch timing (measurement) ----
 * Per-launch durations of the adaLN-Zero block's kernels (itwiki "확산
 * 트랜스포머", adaLN-Zero equations and Implementation / adaLN-Zero block:
 * LayerNorm + modulate, q | k | v, attention, the gated output projection,
 * LayerNorm + modulate, the FFN's two products) inside real forwards, for
 * roofline figures of the kernels as they run there.
 *
 * dit_launch_timer_start arms a timer for the calling thread: it creates
 * 2 * capacity HIP events (host-side runtime objects on the current device;
 * no device memory; timing-only, without the system-scope fence, so an event
 * does not write back or invalidate caches) and, from then on, every forward
 * that thread enqueues
 * (dit_forward, dit_cfg_forward, their _taps and _noalloc forms,
 * dit_forward_packed, dit_sample, dit_block_forward) records one event pair on
 * its stream around each launch of a kernel whose DIT_TIMER_* bit is in
 * kinds_mask, until capacity launches are timed; later launches run untimed.
 * Handles and other threads are not affected.  A timer the thread already
 * had is released first.  Forwards on another device than the one current at
 * start fail with DIT_EHIP while the timer is armed.  Only the blocks of the
 * adaLN-Zero design are timed.
 *   DIT_EINVAL: kinds_mask 0 or with bits beyond DIT_TIMER_KINDS, capacity
 *               outside [1, 65536];  DIT_EHIP: event creation failed (no timer
 *               is left armed).
 *
 * dit_launch_timer_stop waits for the timed launches to finish, writes the
 * first min(count, cap) of them in launch order (kinds[i] a DIT_TIMER_*
 * value, ms[i] the time between the pair's events in milliseconds), sets
 * *count to the number timed, releases the events and disarms the thread.
 * Without an armed timer it sets *count = 0.
 *   DIT_EINVAL: count NULL, cap < 0, or cap > 0 with kinds or ms NULL;
 *   DIT_EHIP: waiting or reading an event failed (the events are still
 *             released). */
#define DIT_TIMER_LN        0   /* LayerNorm + modulate (two per block) */
#define DIT_TIMER_QKV       1   /* q | k | v product */
#define DIT_TIMER_ATTENTION 2
#define DIT_TIMER_OUT_PROJ  3   /* output projection, gated residual epilogue */
#define DIT_TIMER_FC1       4   /* FFN up-projection, GELU epilogue */
#define DIT_TIMER_FC2       5   /* FFN down-projection, gated residual epilogue */
#define DIT_TIMER_KINDS     6
int dit_launch_timer_start(unsigned kinds_mask, int capacity);
int dit_launch_timer_stop(int* kinds, float* ms, int cap, int* count);

/* ---- Sampling around the denoiser ----
 * One reverse step updates the fp32 latent state x [B, C, F, H, W] from the
 * model's prediction.  Kinds:
 *   DIT_SAMPLER_DDPM      ancestral step of the diffusion model whose forward
 *                         process is x_t = sqrt(abar_t) x_0 + sqrt(1 - abar_t) eps
 *                         and whose reverse covariance is learned (cv-learn
 *                         "Sora / DiT", Method, training objective bullet).
 *                         Channels [0, C) are eps; with Cout == 2C channel C + c
 *                         is the raw covariance value v and the variance is
 *                         exp(f log beta + (1 - f) log beta_tilde), f = (v + 1)/2;
 *                         with Cout == C it is beta_tilde.  Adds noise z except
 *                         on the last step, which lands on the clean latent.
 *   DIT_SAMPLER_DPMPP_2M  DPM-Solver++ second-order multistep in data
 *                         prediction, deterministic (the multistep DPM-Solver of
 *                         the itwiki page, inference with diffusers); the first
 *                         step and the last one (into sigma = 0) are first order.
 *   DIT_SAMPLER_RF_EULER  explicit Euler on the predicted rectified-flow
 *                         velocity, x <- x + (t_{k+1} - t_k) v, from t = 0
 *                         (noise) to t = 1 (data) (blog.outta.ai GOKU review,
 *                         section 2.3); channels [0, C) are the velocity.
 * Schedule (the pages give none): beta linear from beta_start to beta_end over
 * train_steps, abar_t = prod_{j <= t} (1 - beta_j); step k evaluates the model
 * at t = tau_k and moves to tau_{k+1} (the clean latent, abar = 1, after the
 * last kept step).  No clipping of the predicted x_0. */
#define DIT_SAMPLER_DDPM      0
#define DIT_SAMPLER_DPMPP_2M  1
#define DIT_SAMPLER_RF_EULER  2

typedef struct dit_sampler {
  int kind;                  /* DIT_SAMPLER_* */
  int num_steps;             /* S >= 1 */
  const int32_t* timesteps;  /* host [S] kept diffusion steps tau_0 > ... > tau_{S-1} in
                                [0, train_steps); NULL: S steps spread evenly over
                                [0, train_steps - 1] (j (train_steps-1)/(S-1), rounded
                                half up), largest first */
  const double* times;       /* host [S + 1] flow times t_0 < ... < t_S (RF); NULL: k / S */
  int train_steps;           /* diffusion kinds: schedule length (1000) */
  double beta_start;         /* 1e-4 */
  double beta_end;           /* 0.02 */
} dit_sampler;

/* Host only (no device work): the model time of step k and the fp64
 * coefficients the step kernel applies (rounded to fp32 there):
 *   DDPM:   x' = c0 x - c1 eps + c4 * exp(0.5 (f c2 + (1 - f) c3)) z;
 *           c0, c1 fold the posterior mean and the x_0 prediction, c2 = log beta,
 *           c3 = log beta_tilde (at the last step the previous step's value; it
 *           is unused there), c4 = 1 if noise is added else 0.
 *   DPM++:  x0 = c0 x - c1 eps,  x' = c2 x + c3 x0 + c4 x0_prev; c5 = 1 if
 *           x0_prev is read (second order) else 0.
 *   RF:     x' = x + c0 v.
 * Unused entries are 0. */
int dit_sampler_coefficients(const dit_sampler* sp, int k, double* model_t, double coef[8]);

/* Step k of `sp` on device buffers: x, x_out [B, C, spatial] fp32 (may alias),
 * model_out [B, Cout, spatial] fp32 (Cout == C or 2C), z [B, C, spatial] fp32
 * (DDPM steps that add noise; else may be NULL), x0_hist [B, C, spatial] fp32
 * (DPM++ only: read as x0 of step k-1 when c5 = 1, overwritten with x0 of
 * step k).  spatial = F * H * W. */
int dit_sampler_step(const dit_sampler* sp, int k, const float* x, const float* model_out,
                     int B, int C, int Cout, int64_t spatial, const float* z, float* x0_hist,
                     float* x_out, void* stream);

/* Workspace bytes of dit_sample (the forward's workspace for its rows plus
 * the model time vector, a model-dtype copy of the state and the DPM++
 * history). */
int dit_sample_workspace_size(const dit_handle* h, const dit_sampler* sp, int B,
                              int guided_channels, size_t* bytes);

/* Full sampling loop of S steps on the caller's stream: each step runs the
 * denoiser on the state (rounded to the model dtype) at the step's model time
 * and applies the update, reading the decoder output directly (no separate
 * unpatchify).  x: [B, C, F, H, W] fp32, in: the starting noise, out: the
 * sample.  guided_channels > 0: classifier-free guidance as dit_cfg_forward
 * (2B trunk rows, scale s, needs num_classes > 0 and no pooled conditioning);
 * 0: the plain forward (y / pooled as for dit_forward).  noise: DDPM with
 * S >= 2: [S, B, C, F, H, W] fp32, slice k is step k's z (the last slice is
 * not read); otherwise may be NULL.  Needs Cout == C or 2C. */
int dit_sample(dit_handle* h, const dit_sampler* sp, float* x, const int32_t* y,
               const float* pooled, int B, float s, int guided_channels, const float* noise,
               void* ws, size_t ws_bytes, void* stream);

/* ---- Packed sequences ----
 * nseq latents of different extents in one call, their tokens packed one
 * sequence after another; attention stays inside each sequence (the Patch n'
 * Pack batching of blog.outta.ai GOKU review, section 2.2).  Each sequence has
 * its own time step, label / pooled vector and 2-D position grid, and the
 * result equals running each sequence on its own.
 *   seq_fhw  host [nseq, 3]: latent extents (F_i, H_i, W_i), F_i = patch_t
 *   x        device: the latents one after another, each [C, F_i, H_i, W_i],
 *            model dtype
 *   t, y, pooled  device, one entry (row) per sequence, as for dit_forward
 *   out      device: the outputs one after another, each [Cout, F_i, H_i, W_i] fp32
 * Needs the adaLN-Zero design with the 2-D position embedding, 1 <= nseq <= 64
 * and (H_i / p)(W_i / p) a multiple of 32 tokens for every sequence. */
int dit_packed_workspace_size(const dit_handle* h, int nseq, const int32_t* seq_fhw,
                              size_t* bytes);
int dit_forward_packed(dit_handle* h, int nseq, const int32_t* seq_fhw, const void* x,
                       const float* t, const int32_t* y, const float* pooled, float* out,
                       void* ws, size_t ws_bytes, void* stream);

/* ---- Training step ----
 * One optimizer step of the adaLN-Zero class-conditional image model
 * (cv-learn.com "Sora / DiT", Method, training-objective bullet; itwiki page,
 * Results: AdamW, constant learning rate, no weight decay, weight EMA).
 *   x_t  = sqrt(abar_t) x0 + sqrt(1 - abar_t) noise   (per row, integer t);
 *   loss = mean over the B C H W latent elements of (eps_theta - noise)^2
 *          + (Cout == 2C) mean over the same elements of the KL term of the
 *          learned covariance: KL(q(x_{t-1} | x_t, x0) || p_theta(x_{t-1} | x_t))
 *          for t > 0, -log N(x0; mu_theta, var_theta) for t = 0, with mu_theta
 *          taken through a stop-gradient (the KL term trains only the
 *          covariance channels); schedule and learned-variance
 *          parameterisation as for the DDPM sampler above;
 *   grad = d loss / d parameters (every field of the flat parameter layout);
 *   AdamW on the fp32 master weights (bias-corrected, decoupled weight
 *   decay), then ema = decay ema + (1 - decay) master, and the handle's
 *   weight buffers receive the new master weights in the model dtype.
 * Label dropout for guidance is the caller's choice of y (the null label
 * num_classes is a valid label); data augmentation is the caller's x0.
 * Needs the adaLN-Zero design, num_classes > 0, cond_dim == 0, no rope3d or
 * qk_norm, frames == patch_t == 1; bf16 models also need B * T % 64 == 0.
 *
 * Flat parameter layout: the trained fields of dit_weights, in struct order
 * (pe_w pe_b t1_w t1_b t2_w t2_b y_table ada_w ada_b qkv_w qkv_b o_w o_b
 * fc1_w fc1_b fc2_w fc2_b out_w out_b), each at a 64-element aligned offset,
 * with the shapes of dit_weights.  dit_train_param_layout gives field f's
 * (offset, count) in elements, f = index of the field in dit_weights (0 =
 * pe_w); count 0 for fields the step does not train. */
typedef struct dit_train_hparams {
  double lr;            /* 1e-4 */
  double beta1, beta2;  /* 0.9, 0.999 */
  double adam_eps;      /* 1e-8 */
  double weight_decay;  /* 0 */
  double ema_decay;     /* 0.9999 */
  int train_steps;      /* diffusion steps of the schedule (1000) */
  double beta_start, beta_end;   /* linear beta line (1e-4, 0.02) */
} dit_train_hparams;

/* Caller-owned fp32 device buffers of dit_train_param_count elements each:
 * master weights (read and updated), gradient (written), Adam moments m, v
 * (read and updated; zero before the first step) and the EMA (read and
 * updated; the initial weights before the first step). */
typedef struct dit_train_state {
  float* master;
  float* grad;
  float* m;
  float* v;
  float* ema;
} dit_train_state;

int dit_train_param_count(const dit_handle* h, size_t* count);
int dit_train_param_layout(const dit_handle* h, int field, size_t* offset, size_t* count);
int dit_train_workspace_size(const dit_handle* h, int B, size_t* bytes);
/* step: 1-based optimizer step number (bias correction).  x0, noise: device
 * [B, C, H, W] fp32; y: device int32 [B] labels in [0, num_classes]; t:
 * device int32 [B] in [0, train_steps) (a t outside makes the loss NaN);
 * loss: device float[2] = (L_simple, KL term).  The handle's weight buffers
 * must be writable device memory (they receive the updated weights).  Calls
 * on one handle must not overlap. */
int dit_train_step(dit_handle* h, const dit_train_hparams* hp, int step,
                   const dit_train_state* st, const float* x0, const int32_t* y, const int32_t* t,
                   const float* noise, int B, float* loss, void* ws, size_t ws_bytes,
                   void* stream);

/* Weight and bias gradients of a linear layer y = x W^T + b over R rows, the
 * product that dominates the backward pass of the step above (cv-learn.com
 * "Sora / DiT", Method, training-objective bullet: the parameters follow the
 * gradient of that loss):  dW[N, K] += dY^T X  =  sum over r of dY[r, n] X[r, k]
 * and, when db is not NULL, db[n] += sum over r of dY[r, n] (device fp32 [N],
 * added to atomically like dW).
 * dY: device [R, N] row-major with row stride ldy >= N; X: device [R, K]
 * row-major with row stride ldx >= K; both in dtype, read as stored (no
 * transposed copies).  dW: device fp32 [N, K] row-major, added to atomically
 * (zero it first for a fresh gradient; the summation order is not fixed).
 * bf16 with N, K, ldy, ldx multiples of 8, R % 64 == 0, R * max(ldy, ldx) <
 * 2^31 and 16-byte aligned dY, X runs on the matrix cores; other shapes and
 * fp32 on the vector ALUs (db then by a column-sum pass; bf16 needs N and
 * ldy multiples of 8 and dY 16-byte aligned for it).  R == 0 adds nothing.
 * DIT_EINVAL for NULL dY, X or dW, N or K not positive, R negative, a short
 * row stride or an unknown dtype; DIT_EUNSUPPORTED for R >= 2^31 or a bias
 * gradient the column-sum pass cannot take. */
int dit_linear_wgrad(const void* dY, int64_t ldy, const void* X, int64_t ldx, int N, int K,
                     int64_t R, int dtype, float* dW, float* db, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DIT_H */
