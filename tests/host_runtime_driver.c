/* Host-runtime driver for the sanitizer build (tests/test_host_sanitizers.py).
 *
 * Calls every entry point of the C ABI that does its work on the host, over
 * the configurations of the workloads the library serves (DiT-S/8 fp32,
 * DiT-B/4, DiT-XL/2 at 256 and 512, the spacetime video model, the in-context,
 * cross-attention and MMDiT designs): handle creation and planning, workspace
 * sizing over many row counts, the training parameter layout, the sampler
 * coefficients, the packed-sequence planner, and the argument checks of the
 * forward, sampling and step entry points that return before any launch.
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
 * of api.cpp and train_api.cpp, it needs no GPU: weight and buffer pointers
 * are stand-ins that the host code records but never dereferences.
 *
 * Prints "host runtime driver: N checks, 0 failed" and exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dit.h"

static int checks = 0, failed = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    ++checks;                                                                    \
    if (!(cond)) {                                                               \
      ++failed;                                                                  \
      fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, #cond, \
              dit_last_error_message());                                         \
    }                                                                            \
  } while (0)

/* Stand-in device addresses: 256-byte aligned, never dereferenced. */
#define FAKE(i) ((void*)(uintptr_t)(0x100000u + 256u * (unsigned)(i)))

static dit_config base_cfg(void) {
  dit_config c;
  memset(&c, 0, sizeof c);
  c.in_channels = 4; c.out_channels = 8; c.frames = 1; c.height = 32; c.width = 32;
  c.patch = 2; c.patch_t = 1; c.hidden = 1152; c.depth = 28; c.heads = 16;
  c.mlp_hidden = 4608; c.num_classes = 1000; c.cond_dim = 0; c.freq_dim = 256;
  c.qk_norm = 0; c.rope3d = 0; c.dtype = DIT_BF16; c.ln_eps = 1e-6f;
  c.conditioning = DIT_COND_ADALN_ZERO;
  return c;
}

/* Every field set: the designs ignore the weights they do not use. */
static dit_weights all_weights(void) {
  dit_weights w;
  const void** f = (const void**)&w;
  for (size_t i = 0; i < sizeof w / sizeof(void*); ++i) f[i] = FAKE(i);
  return w;
}

static dit_handle* create(const dit_config* c, const dit_weights* w) {
  dit_handle* h = NULL;
  const int rc = dit_create(c, w, &h);
  CHECK(rc == DIT_OK && h != NULL);
  return h;
}

/* Workspace sizes: positive, non-decreasing in the row count. */
static void workspace_sweep(dit_handle* h, int max_rows) {
  size_t prev = 0;
  for (int rows = 1; rows <= max_rows; ++rows) {
    size_t n = 0;
    CHECK(dit_workspace_size(h, rows, &n) == DIT_OK);
    CHECK(n > 0 && n >= prev);
    prev = n;
  }
  size_t n = 0;
  CHECK(dit_workspace_size(h, 0, &n) == DIT_EINVAL);
  CHECK(dit_workspace_size(h, -3, &n) == DIT_EINVAL);
  CHECK(dit_workspace_size(h, 4, NULL) == DIT_EINVAL);
  CHECK(dit_workspace_size(NULL, 4, &n) == DIT_EINVAL);
}

/* Forward entry points: each bad argument is refused before any launch. */
static void forward_checks(dit_handle* h, int rows, int has_labels) {
  size_t need = 0;
  CHECK(dit_workspace_size(h, rows, &need) == DIT_OK);
  void* p = FAKE(100);
  const int32_t* y = has_labels ? (const int32_t*)p : NULL;
  const float* pooled = has_labels ? NULL : (const float*)p;
  CHECK(dit_forward(h, p, p, y, pooled, 0, p, p, need, NULL) == DIT_EINVAL);
  CHECK(dit_forward(h, NULL, p, y, pooled, rows, p, p, need, NULL) == DIT_EINVAL);
  CHECK(dit_forward(h, p, NULL, y, pooled, rows, p, p, need, NULL) == DIT_EINVAL);
  CHECK(dit_forward(h, p, p, y, pooled, rows, NULL, p, need, NULL) == DIT_EINVAL);
  CHECK(dit_forward(h, p, p, y, pooled, rows, p, p, need - 1, NULL) == DIT_EWORKSPACE);
  CHECK(dit_forward(h, p, p, y, pooled, rows, p, NULL, need, NULL) == DIT_EWORKSPACE);
  CHECK(dit_forward_taps(h, p, p, y, pooled, rows, p, NULL, p, need - 1, NULL) ==
        DIT_EWORKSPACE);
  if (has_labels && rows % 2 == 0) {
    const int bh = rows / 2;
    CHECK(dit_cfg_forward(h, p, p, y, bh, 1.5f, 0, p, p, need, NULL) == DIT_EINVAL);
    CHECK(dit_cfg_forward(h, p, p, y, bh, NAN, 4, p, p, need, NULL) == DIT_EINVAL);
    CHECK(dit_cfg_forward(h, p, p, y, bh + 1, 1.5f, 4, p, p, need, NULL) == DIT_EWORKSPACE);
    CHECK(dit_cfg_forward(h, p, p, NULL, bh, 1.5f, 4, p, p, need, NULL) == DIT_EINVAL);
  }
  CHECK(dit_forward_noalloc(h, p, p, y, pooled, 0, p, NULL) == DIT_EINVAL);
  CHECK(dit_forward_noalloc(NULL, p, p, y, pooled, rows, p, NULL) == DIT_EINVAL);
}

static void sampler_checks(dit_handle* h, int B, int guided, int has_labels) {
  const int kinds[3] = {DIT_SAMPLER_DDPM, DIT_SAMPLER_DPMPP_2M, DIT_SAMPLER_RF_EULER};
  const int steps[5] = {1, 2, 7, 50, 250};
  for (int a = 0; a < 3; ++a)
    for (int b = 0; b < 5; ++b) {
      dit_sampler sp;
      memset(&sp, 0, sizeof sp);
      sp.kind = kinds[a]; sp.num_steps = steps[b]; sp.train_steps = 1000;
      sp.beta_start = 1e-4; sp.beta_end = 0.02;
      for (int k = 0; k < sp.num_steps; ++k) {
        double t = -1.0, c[8];
        for (int i = 0; i < 8; ++i) c[i] = NAN;
        CHECK(dit_sampler_coefficients(&sp, k, &t, c) == DIT_OK);
        CHECK(isfinite(t));
        for (int i = 0; i < 8; ++i) CHECK(isfinite(c[i]));
      }
      double t, c[8];
      CHECK(dit_sampler_coefficients(&sp, sp.num_steps, &t, c) == DIT_EINVAL);
      CHECK(dit_sampler_coefficients(&sp, -1, &t, c) == DIT_EINVAL);
      size_t n = 0, fwd = 0;
      CHECK(dit_sample_workspace_size(h, &sp, B, guided, &n) == DIT_OK);
      CHECK(dit_workspace_size(h, guided ? 2 * B : B, &fwd) == DIT_OK);
      CHECK(n >= fwd);
      void* p = FAKE(200);
      const int32_t* y = has_labels ? (const int32_t*)p : NULL;
      const float* pooled = has_labels ? NULL : (const float*)p;
      CHECK(dit_sample(h, &sp, p, y, pooled, B, 1.5f, guided, p, p, n - 1, NULL) ==
            DIT_EWORKSPACE);
      CHECK(dit_sample(h, &sp, NULL, y, pooled, B, 1.5f, guided, p, p, n, NULL) == DIT_EINVAL);
    }
  /* explicit, decreasing time steps; a repeated step is refused */
  int32_t ts[4] = {999, 500, 120, 3}, bad[4] = {999, 500, 500, 3};
  dit_sampler sp;
  memset(&sp, 0, sizeof sp);
  sp.kind = DIT_SAMPLER_DDPM; sp.num_steps = 4; sp.timesteps = ts; sp.train_steps = 1000;
  sp.beta_start = 1e-4; sp.beta_end = 0.02;
  double t, c[8];
  CHECK(dit_sampler_coefficients(&sp, 3, &t, c) == DIT_OK && t == 3.0);
  sp.timesteps = bad;
  CHECK(dit_sampler_coefficients(&sp, 0, &t, c) == DIT_EINVAL);
}

static void train_checks(dit_handle* h) {
  size_t total = 0;
  CHECK(dit_train_param_count(h, &total) == DIT_OK && total > 0);
  /* every field of dit_weights: trained ones in struct order, the rest empty */
  const int nfields = (int)(sizeof(dit_weights) / sizeof(void*));
  size_t end = 0;
  for (int f = 0; f < nfields; ++f) {
    size_t off = 0, cnt = 0;
    CHECK(dit_train_param_layout(h, f, &off, &cnt) == DIT_OK);
    if (cnt) {
      CHECK(off % 64 == 0 && off >= end);
      end = off + cnt;
    }
  }
  CHECK(end <= total);
  size_t off, cnt;
  CHECK(dit_train_param_layout(h, nfields, &off, &cnt) == DIT_EINVAL);
  CHECK(dit_train_param_layout(h, -1, &off, &cnt) == DIT_EINVAL);
  for (int B = 1; B <= 256; B *= 2) {
    size_t n = 0;
    CHECK(dit_train_workspace_size(h, B, &n) == DIT_OK && n > 0);
  }
}

static void packed_checks(dit_handle* h) {
  /* mixes of 256-, 1024- and 64-token sequences (multiples of 32 tokens) */
  int32_t fhw[64 * 3];
  for (int n = 1; n <= 64; n = n * 2 + 1) {
    for (int i = 0; i < n; ++i) {
      const int s = (i % 3 == 0) ? 64 : (i % 3 == 1) ? 32 : 16;
      fhw[3 * i] = 1; fhw[3 * i + 1] = s; fhw[3 * i + 2] = s;
    }
    size_t need = 0;
    CHECK(dit_packed_workspace_size(h, n, fhw, &need) == DIT_OK && need > 0);
    void* p = FAKE(300);
    CHECK(dit_forward_packed(h, n, fhw, p, p, p, NULL, p, p, need - 1, NULL) == DIT_EWORKSPACE);
  }
  int32_t odd[3] = {1, 30, 30};   /* 225 tokens: not a multiple of 32 */
  size_t need = 0;
  CHECK(dit_packed_workspace_size(h, 1, odd, &need) != DIT_OK);
  CHECK(dit_packed_workspace_size(h, 0, fhw, &need) == DIT_EINVAL);
}

/* Launch timer: argument checks, and a start without a device either arms
 * (then stop reports no timed launch) or fails with DIT_EHIP, leaving nothing
 * armed. */
static void timer_checks(void) {
  int kinds[4], count = -1;
  float ms[4];
  CHECK(dit_launch_timer_start(0u, 16) == DIT_EINVAL);
  CHECK(dit_launch_timer_start(1u << DIT_TIMER_KINDS, 16) == DIT_EINVAL);
  CHECK(dit_launch_timer_start(1u << DIT_TIMER_FC1, 0) == DIT_EINVAL);
  CHECK(dit_launch_timer_start(1u << DIT_TIMER_FC1, 65537) == DIT_EINVAL);
  CHECK(dit_launch_timer_stop(kinds, ms, 4, NULL) == DIT_EINVAL);
  CHECK(dit_launch_timer_stop(kinds, ms, -1, &count) == DIT_EINVAL);
  CHECK(dit_launch_timer_stop(NULL, ms, 4, &count) == DIT_EINVAL);
  CHECK(dit_launch_timer_stop(kinds, NULL, 4, &count) == DIT_EINVAL);
  CHECK(dit_launch_timer_stop(NULL, NULL, 0, &count) == DIT_OK && count == 0);
  for (int rep = 0; rep < 3; ++rep) {
    const int rc = dit_launch_timer_start((1u << DIT_TIMER_KINDS) - 1u, 8 + rep);
    CHECK(rc == DIT_OK || rc == DIT_EHIP);
    count = -1;
    CHECK(dit_launch_timer_stop(kinds, ms, 4, &count) == DIT_OK && count == 0);
  }
  /* a second start releases the first timer's events */
  const int r1 = dit_launch_timer_start(1u << DIT_TIMER_QKV, 32);
  const int r2 = dit_launch_timer_start(1u << DIT_TIMER_LN, 64);
  CHECK(r1 == r2 && (r1 == DIT_OK || r1 == DIT_EHIP));
  count = -1;
  CHECK(dit_launch_timer_stop(kinds, ms, 4, &count) == DIT_OK && count == 0);
}

int main(void) {
  const dit_weights w = all_weights();
  timer_checks();

  /* DiT-XL/2 at 256 and 512 (class-conditional, guided) */
  for (int res = 32; res <= 64; res *= 2) {
    dit_config c = base_cfg();
    c.height = c.width = res;
    dit_handle* h = create(&c, &w);
    if (!h) continue;
    workspace_sweep(h, 130);
    forward_checks(h, 64, 1);
    forward_checks(h, 3, 1);
    sampler_checks(h, 8, 4, 1);
    sampler_checks(h, 3, 0, 1);
    train_checks(h);
    packed_checks(h);
    dit_destroy(h);
  }
  /* DiT-S/8 fp32 and DiT-B/4 bf16 */
  {
    dit_config c = base_cfg();
    c.patch = 8; c.hidden = 384; c.depth = 12; c.heads = 6; c.mlp_hidden = 1536;
    c.dtype = DIT_F32;
    dit_handle* h = create(&c, &w);
    if (h) { workspace_sweep(h, 40); forward_checks(h, 2, 1); train_checks(h); dit_destroy(h); }
    c.patch = 4; c.hidden = 768; c.heads = 12; c.mlp_hidden = 3072; c.dtype = DIT_BF16;
    h = create(&c, &w);
    if (h) { workspace_sweep(h, 40); forward_checks(h, 32, 1); train_checks(h); dit_destroy(h); }
  }
  /* spacetime video model: 3-D RoPE, q/k LayerNorm, pooled conditioning */
  {
    dit_config c = base_cfg();
    c.in_channels = 16; c.out_channels = 16; c.frames = 16; c.height = 60; c.width = 104;
    c.num_classes = 0; c.cond_dim = 4096; c.qk_norm = 1; c.rope3d = 1;
    dit_handle* h = create(&c, &w);
    if (h) {
      workspace_sweep(h, 4);
      forward_checks(h, 1, 0);
      sampler_checks(h, 1, 0, 0);
      size_t n;
      CHECK(dit_train_workspace_size(h, 1, &n) != DIT_OK);   /* training: images only */
      dit_destroy(h);
    }
  }
  /* in-context and cross-attention designs */
  for (int cond = DIT_COND_IN_CONTEXT; cond <= DIT_COND_CROSS_ATTN; ++cond) {
    dit_config c = base_cfg();
    c.conditioning = cond;
    dit_handle* h = create(&c, &w);
    if (h) { workspace_sweep(h, 70); forward_checks(h, 64, 1); sampler_checks(h, 2, 4, 1); dit_destroy(h); }
  }
  /* MMDiT: text stream of 333 tokens */
  {
    dit_config c = base_cfg();
    c.in_channels = 16; c.out_channels = 16; c.height = 64; c.width = 64; c.hidden = 1536;
    c.depth = 24; c.heads = 24; c.mlp_hidden = 6144; c.num_classes = 0; c.cond_dim = 2048;
    c.conditioning = DIT_COND_MMDIT; c.ctx_len = 333; c.ctx_dim = 4096;
    dit_handle* h = create(&c, &w);
    if (h) {
      workspace_sweep(h, 10);
      size_t need = 0;
      CHECK(dit_workspace_size(h, 8, &need) == DIT_OK);
      void* p = FAKE(400);
      CHECK(dit_forward_ctx(h, p, p, p, p, 8, p, NULL, p, need - 1, NULL) == DIT_EWORKSPACE);
      CHECK(dit_forward_ctx(h, p, p, p, NULL, 8, p, NULL, p, need, NULL) == DIT_EINVAL);
      CHECK(dit_forward_noalloc(h, p, p, NULL, p, 1, p, NULL) == DIT_EUNSUPPORTED);
      dit_destroy(h);
    }
  }
  /* configurations refused at creation leave no handle */
  {
    dit_config c = base_cfg();
    dit_handle* h = FAKE(1);
    c.height = 33;
    CHECK(dit_create(&c, &w, &h) == DIT_EINVAL && h == NULL);
    c = base_cfg(); c.heads = 12;
    CHECK(dit_create(&c, &w, &h) == DIT_EUNSUPPORTED && h == NULL);
    c = base_cfg(); c.depth = 0;
    CHECK(dit_create(&c, &w, &h) == DIT_EINVAL);
    c = base_cfg();
    CHECK(dit_create(NULL, &w, &h) == DIT_EINVAL);
    CHECK(dit_create(&c, NULL, &h) == DIT_EINVAL);
    dit_weights w2 = w;
    w2.fc2_w = NULL;
    CHECK(dit_create(&c, &w2, &h) == DIT_EINVAL);
  }
  /* standalone steps: argument checks */
  {
    void* p = FAKE(500);
    CHECK(dit_patchify(p, 1, 4, 1, 33, 32, 2, 1, DIT_BF16, p, NULL) == DIT_EINVAL);
    CHECK(dit_unpatchify(p, 1, 8, 3, 32, 32, 2, 2, p, NULL) == DIT_EINVAL);
    CHECK(dit_timestep_embed(p, 4, 255, p, NULL) == DIT_EINVAL);
    CHECK(dit_attention(p, 2, 16, 256, 96, DIT_BF16, p, NULL) == DIT_EUNSUPPORTED);
    CHECK(dit_attention(p, 2, 16, 256, 72, DIT_BF16, (char*)p + 4, NULL) == DIT_EINVAL);
    CHECK(dit_linear(DIT_EPI_GATED, p, p, p, 64, 64, 64, DIT_BF16, p, NULL, 0, 1, NULL) ==
          DIT_EINVAL);
    CHECK(dit_linear_wgrad(p, 8, p, 8, 8, 8, -1, DIT_BF16, p, NULL, NULL) == DIT_EINVAL);
    CHECK(dit_linear_wgrad(p, 8, p, 8, 8, 8, (int64_t)1 << 31, DIT_BF16, p, NULL, NULL) ==
          DIT_EUNSUPPORTED);
  }
  /* status strings for every code and a few unknown ones */
  for (int s = -6; s <= 1; ++s) CHECK(dit_status_string(s) != NULL);
  dit_destroy(NULL);

  printf("host runtime driver: %d checks, %d failed\n", checks, failed);
  return failed ? 1 : 0;
}
