// Timestep sinusoid, standalone patchify, and unpatchify fused with the
// classifier-free-guidance combine.
#include "common.h"

// e[b, k] = cos(t f_k) (k < dim/2), sin(t f_{k - dim/2}) (k >= dim/2),
// f_k = 10000^(-k/(dim/2)).  Arguments are formed and reduced in fp64 (t can be
// 999, so an fp32 angle would lose ~1e-4 rad); the table is B x dim, tiny.
__global__ void timestep_embed_kernel(const float* __restrict__ t, int rows, int src_rows,
                                      int dim, float* __restrict__ e) {
  int idx = blockIdx.x * blockDim.x + threadIdx.x;
  int half = dim >> 1;
  if (idx >= rows * dim) return;
  int b = idx / dim, k = idx - b * dim;
  int kf = k < half ? k : k - half;
  double f = exp(-9.210340371976184 * (double)kf / (double)half);  // ln(10000)
  double a = (double)t[b % src_rows] * f;
  e[idx] = (float)(k < half ? cos(a) : sin(a));
}

hipError_t launch_timestep_embed(const float* t, int rows, int src_rows, int dim, float* e,
                                 hipStream_t s) {
  int n = rows * dim;
  timestep_embed_kernel<<<(n + 255) / 256, 256, 0, s>>>(t, rows, src_rows, dim, e);
  return hipGetLastError();
}

// P[b, tau, k] = x[b, c, f*pt + a, i*p + py, j*p + px]; one thread per element of
// P, consecutive threads write consecutive k.
template <typename T>
__global__ void patchify_kernel(const T* __restrict__ x, int64_t total, PatchGeom g,
                                T* __restrict__ P) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  int k = (int)(idx % g.K);
  int64_t bt = idx / g.K;
  int tau = (int)(bt % g.T);
  int64_t b = bt / g.T;
  int64_t row = (int64_t)g.C * g.F * g.H * g.W;
  P[idx] = x[b * row + patch_src_offset(g, tau, k)];
}

hipError_t launch_patchify(const void* x, int B, const PatchGeom& g, int dtype, void* P,
                           hipStream_t s) {
  int64_t total = (int64_t)B * g.T * g.K;
  int blocks = (int)((total + 255) / 256);
  if (dtype == 1)
    patchify_kernel<bf16_t><<<blocks, 256, 0, s>>>((const bf16_t*)x, total, g, (bf16_t*)P);
  else
    patchify_kernel<float><<<blocks, 256, 0, s>>>((const float*)x, total, g, (float*)P);
  return hipGetLastError();
}

// out[b, c, f, y, x] = Y[b, tau, k] for the inverse of the patch index map with
// Cout channels.  With guide != 0 the value is combined with the null-label row
// b + Bh_offset: ch < guided -> u + s (v - u), else v.  One thread per output
// element; writes are coalesced along x.
__global__ void unpatchify_kernel(const float* __restrict__ Y, int64_t total, PatchGeom g,
                                  int Cout, int Bh_offset, int guided, float scale, int guide,
                                  float* __restrict__ out) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  int xw = (int)(idx % g.W);
  int64_t r = idx / g.W;
  int yh = (int)(r % g.H); r /= g.H;
  int f = (int)(r % g.F); r /= g.F;
  int c = (int)(r % Cout);
  int64_t b = r / Cout;
  int tau = ((f / g.pt) * g.gh + yh / g.p) * g.gw + xw / g.p;
  int k = (((f % g.pt) * g.p + yh % g.p) * g.p + xw % g.p) * Cout + c;
  int kout = g.pt * g.p * g.p * Cout;
  float v = Y[(b * g.T + tau) * kout + k];
  if (guide && c < guided) {
    float u = Y[((b + Bh_offset) * g.T + tau) * kout + k];
    v = u + scale * (v - u);
  }
  out[idx] = v;
}

hipError_t launch_unpatchify(const float* Y, int Bout, int Bh_offset, const PatchGeom& g,
                             int Cout, int guided, float scale, int guide, float* out,
                             hipStream_t s) {
  int64_t total = (int64_t)Bout * Cout * g.F * g.H * g.W;
  int blocks = (int)((total + 255) / 256);
  unpatchify_kernel<<<blocks, 256, 0, s>>>(Y, total, g, Cout, Bh_offset, guided, scale, guide,
                                           out);
  return hipGetLastError();
}
