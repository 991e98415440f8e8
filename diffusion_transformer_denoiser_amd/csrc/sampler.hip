// Sampler update kernels: one reverse step of the latent state from the
// denoiser's prediction, elementwise over [B, C, F, H, W].
//
//   DDPM ancestral step with a learned diagonal covariance (cv-learn "Sora /
//   DiT", Method: forward process, learned Sigma, noise-and-covariance
//   decoder output);
//   DPM-Solver++ second-order multistep in data prediction (the multistep
//   DPM-Solver of the itwiki page, section on inference with diffusers);
//   explicit Euler on the rectified-flow velocity (blog.outta.ai GOKU
//   review, section 2.3).
//
// The host folds the schedule into a few fp32 coefficients per step (fp64 on
// the host), so each element costs a handful of FMAs; the kernel is bound by
// HBM bandwidth (or launch latency at small batches).  The prediction is read
// either from a plain [B, Cout, F, H, W] tensor or straight from the
// decoder's token-major output [rows, T, Kout], with the guidance combine of
// the conditional row b and the null row b + B applied on the fly, so a
// sampling step needs no separate unpatchify pass.
#include "common.h"

namespace {

template <int KIND, bool FROM_Y, bool BF16_COPY>
__global__ __launch_bounds__(256) void sampler_step_kernel(SamplerStepArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < a.tvec_rows) a.tvec[idx] = a.t_next;
  if (idx >= a.n) return;
  const int64_t sp = idx % a.S;
  const int64_t bc = idx / a.S;
  const int c = (int)(bc % a.C);
  const int b = (int)(bc / a.C);

  // Prediction channel ch of element (b, sp).
  auto fetch = [&](int ch) -> float {
    if constexpr (!FROM_Y) {
      return a.mo[((int64_t)b * a.Cout + ch) * a.S + sp];
    } else {
      const PatchGeom& g = a.g;
      const int xw = (int)(sp % g.W);
      const int64_t r = sp / g.W;
      const int yh = (int)(r % g.H);
      const int f = (int)(r / g.H);
      const int tau = ((f / g.pt) * g.gh + yh / g.p) * g.gw + xw / g.p;
      const int kout = g.pt * g.p * g.p * a.Cout;
      const int k = (((f % g.pt) * g.p + yh % g.p) * g.p + xw % g.p) * a.Cout + ch;
      float v = a.mo[((int64_t)b * g.T + tau) * kout + k];
      if (ch < a.guided) {
        const float u = a.mo[((int64_t)(b + a.null_off) * g.T + tau) * kout + k];
        v = u + a.scale * (v - u);
      }
      return v;
    }
  };

  const float x = a.x[idx];
  float xn;
  if constexpr (KIND == 0) {
    // Posterior mean with the predicted x0 folded in: a_x x - a_e eps.
    const float e = fetch(c);
    xn = fmaf(a.k[0], x, -a.k[1] * e);
    if (a.add_noise) {
      float lv = a.k[3];                              // log beta_tilde
      if (a.learned) {
        const float fr = 0.5f * (fetch(a.C + c) + 1.0f);
        lv = fmaf(fr, a.k[2] - a.k[3], a.k[3]);       // fr log beta + (1 - fr) log beta_tilde
      }
      xn = fmaf(expf(0.5f * lv), a.z[idx], xn);
    }
  } else if constexpr (KIND == 1) {
    const float e = fetch(c);
    const float x0 = fmaf(a.k[0], x, -a.k[1] * e);    // (x - sigma eps) / alpha
    xn = fmaf(a.k[2], x, a.k[3] * x0);
    if (a.has_prev) xn = fmaf(a.k[4], a.hist[idx], xn);
    if (a.hist) a.hist[idx] = x0;
  } else {
    xn = fmaf(a.k[0], fetch(c), x);                   // x + dt v
  }
  a.x_out[idx] = xn;
  if constexpr (BF16_COPY) ((bf16_t*)a.x_model)[idx] = f2bf(xn);
}

// x_model = bf16(x); tvec[0..rows) = t.  Start of a sampling loop.
__global__ __launch_bounds__(256) void sampler_prologue_kernel(const float* __restrict__ x,
                                                               int64_t n, bf16_t* __restrict__ xm,
                                                               float* __restrict__ tvec,
                                                               int rows, float t) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < rows) tvec[idx] = t;
  if (xm && idx < n) xm[idx] = f2bf(x[idx]);
}

template <int KIND, bool FROM_Y>
hipError_t step_dispatch_copy(const SamplerStepArgs& a, int blocks, hipStream_t s) {
  if (a.x_model)
    sampler_step_kernel<KIND, FROM_Y, true><<<blocks, 256, 0, s>>>(a);
  else
    sampler_step_kernel<KIND, FROM_Y, false><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int KIND>
hipError_t step_dispatch(const SamplerStepArgs& a, int blocks, hipStream_t s) {
  return a.from_y ? step_dispatch_copy<KIND, true>(a, blocks, s)
                  : step_dispatch_copy<KIND, false>(a, blocks, s);
}

}  // namespace

hipError_t launch_sampler_step(const SamplerStepArgs& a, hipStream_t s) {
  const int64_t work = a.n > a.tvec_rows ? a.n : a.tvec_rows;
  if (work <= 0) return hipSuccess;
  const int blocks = (int)((work + 255) / 256);
  switch (a.kind) {
    case 0: return step_dispatch<0>(a, blocks, s);
    case 1: return step_dispatch<1>(a, blocks, s);
    case 2: return step_dispatch<2>(a, blocks, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sampler_prologue(const float* x, int64_t n, bf16_t* x_model, float* tvec,
                                   int rows, float t, hipStream_t s) {
  const int64_t work = x_model ? (n > rows ? n : rows) : rows;
  if (work <= 0) return hipSuccess;
  sampler_prologue_kernel<<<(int)((work + 255) / 256), 256, 0, s>>>(x, n, x_model, tvec, rows, t);
  return hipGetLastError();
}
