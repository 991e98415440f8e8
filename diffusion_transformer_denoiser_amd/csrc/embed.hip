// Timestep sinusoid, position-embedding table, conditioning-vector finish,
// standalone patchify, and unpatchify fused with the classifier-free-guidance
// combine.
#include "common.h"
#include "epilogue.h"

// e[b, k] = cos(t f_k) (k < dim/2), sin(t f_{k - dim/2}) (k >= dim/2),
// f_k = 10000^(-k/(dim/2)).  Arguments are formed and reduced in fp64 (t can be
// 999, so an fp32 angle would lose ~1e-4 rad); the table is B x dim, tiny.
template <typename OT>
__global__ void timestep_embed_kernel(const float* __restrict__ t, int rows, int src_rows,
                                      int dim, OT* __restrict__ e) {
  int idx = blockIdx.x * blockDim.x + threadIdx.x;
  int half = dim >> 1;
  if (idx >= rows * dim) return;
  int b = idx / dim, k = idx - b * dim;
  int kf = k < half ? k : k - half;
  double f = exp(-9.210340371976184 * (double)kf / (double)half);  // ln(10000)
  double a = (double)t[b % src_rows] * f;
  e[idx] = from_f<OT>((float)(k < half ? cos(a) : sin(a)));
}

hipError_t launch_timestep_embed(const float* t, int rows, int src_rows, int dim, float* e,
                                 hipStream_t s) {
  int n = rows * dim;
  timestep_embed_kernel<float><<<(n + 255) / 256, 256, 0, s>>>(t, rows, src_rows, dim, e);
  return hipGetLastError();
}

hipError_t launch_timestep_embed_bf16(const float* t, int rows, int src_rows, int dim, bf16_t* e,
                                      hipStream_t s) {
  int n = rows * dim;
  timestep_embed_kernel<bf16_t><<<(n + 255) / 256, 256, 0, s>>>(t, rows, src_rows, dim, e);
  return hipGetLastError();
}

// Table of the 2-D sin-cos position embedding, pe[tau, n] for tau = i * gw + j.
__global__ void pos_embed_table_kernel(int gh, int gw, int d, float* __restrict__ pe) {
  int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= gh * gw * d) return;
  int tau = idx / d, n = idx - tau * d;
  int i = tau / gw, j = tau - i * gw;
  pe[idx] = pos_embed_2d(i, j, n, d);
}

hipError_t launch_pos_embed_table(int gh, int gw, int d, float* pe, hipStream_t s) {
  int n = gh * gw * d;
  pos_embed_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(gh, gw, d, pe);
  return hipGetLastError();
}

// Conditioning vector: c += class row (+ pooled projection); sc = SiLU(c).
template <typename DT>
__global__ void cond_finish_kernel(float* __restrict__ c, int rows, int d,
                                   const float* __restrict__ table, const int32_t* __restrict__ labels,
                                   int label_rows, int null_from, int ncls,
                                   const float* __restrict__ pooled, DT* __restrict__ sc) {
  int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * d) return;
  int m = idx / d, n = idx - m * d;
  float v = c[idx];
  if (pooled) v += pooled[idx];
  if (table) {
    int lbl = (m >= null_from) ? ncls : labels[m % label_rows];
    if (lbl < 0 || lbl > ncls) v = __builtin_nanf("");
    else v += table[(int64_t)lbl * d + n];
  }
  c[idx] = v;
  sc[idx] = from_f<DT>(silu_f(v));
}

// Conditioning tokens of the in-context and cross-attention designs: token 0
// is the time embedding, token 1 the class row.  One thread per element.
template <typename DT>
__global__ void cond_tokens_kernel(const float* __restrict__ temb, int rows, int d,
                                   const float* __restrict__ table,
                                   const int32_t* __restrict__ labels, int label_rows,
                                   int null_from, int ncls, int mode, void* __restrict__ dst,
                                   int T) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * 2 * d) return;
  const int m = (int)(idx / (2 * d));
  const int rem = (int)(idx - (int64_t)m * 2 * d);
  const int which = rem / d, n = rem - which * d;
  float v;
  if (which == 0) {
    v = temb[(int64_t)m * d + n];
  } else {
    const int lbl = (m >= null_from) ? ncls : labels[m % label_rows];
    v = (lbl < 0 || lbl > ncls) ? __builtin_nanf("") : table[(int64_t)lbl * d + n];
  }
  if (mode == 0)
    ((float*)dst)[((int64_t)m * (T + 2) + T + which) * d + n] = v;
  else
    ((DT*)dst)[((int64_t)m * 2 + which) * d + n] = from_f<DT>(v);
}

hipError_t launch_cond_tokens(const float* temb, int rows, int d, const float* table,
                              const int32_t* labels, int label_rows, int null_from, int ncls,
                              int mode, void* dst, int T, int dtype, hipStream_t s) {
  const int64_t n = (int64_t)rows * 2 * d;
  const int blocks = (int)((n + 255) / 256);
  if (dtype == 1)
    cond_tokens_kernel<bf16_t><<<blocks, 256, 0, s>>>(temb, rows, d, table, labels, label_rows,
                                                      null_from, ncls, mode, dst, T);
  else
    cond_tokens_kernel<float><<<blocks, 256, 0, s>>>(temb, rows, d, table, labels, label_rows,
                                                     null_from, ncls, mode, dst, T);
  return hipGetLastError();
}

hipError_t launch_cond_finish(float* c, int rows, int d, const float* table, const int32_t* labels,
                              int label_rows, int null_from, int ncls, const float* pooled,
                              void* sc, int dtype, hipStream_t s) {
  int n = rows * d;
  if (dtype == 1)
    cond_finish_kernel<bf16_t><<<(n + 255) / 256, 256, 0, s>>>(
        c, rows, d, table, labels, label_rows, null_from, ncls, pooled, (bf16_t*)sc);
  else
    cond_finish_kernel<float><<<(n + 255) / 256, 256, 0, s>>>(
        c, rows, d, table, labels, label_rows, null_from, ncls, pooled, (float*)sc);
  return hipGetLastError();
}

// 16 consecutive elements of a 16-byte aligned row, as floats.
__device__ __forceinline__ void load16(const bf16_t* p, float* f) {
  const uint4 a = ((const uint4*)p)[0], b = ((const uint4*)p)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load16(const float* p, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = ((const float4*)p)[i];
    f[4 * i] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
  }
}

// Patch embedding X[row(m), n] = sum_k P[m, k] W[n, k] + bias[n] (+ pe[m % T, n])
// for token rows m of a [B, C, F, H, W] latent, P the patch vectors (gathered
// from the latent; never stored).  row(m) = m + (m / T) out_skip.  A workgroup
// handles TM tokens: it gathers their patch vectors into LDS; each thread then
// owns 4 consecutive output features, reads their weights 16 k at a time into
// registers once and applies them to all TM tokens (products in order k = 0 ..
// K-1), and stores 16 bytes per token.  K % 16 == 0; W 16-byte aligned.
template <typename AT, int TM>
__global__ __launch_bounds__(256) void patch_embed_kernel(const AT* __restrict__ x, int src_rows,
                                                          PatchGeom g, const AT* __restrict__ W,
                                                          const float* __restrict__ bias,
                                                          const float* __restrict__ pe, int M,
                                                          int d, int out_skip,
                                                          float* __restrict__ X) {
  extern __shared__ float sP[];   // [TM][K]
  const int K = g.K, T = g.T;
  const int m0 = blockIdx.x * TM;
  const int64_t lrow = (int64_t)g.C * g.F * g.H * g.W;
  for (int e = threadIdx.x; e < TM * K; e += blockDim.x) {
    const int r = e / K, k = e - r * K;
    const int m = min(m0 + r, M - 1);
    const int b = m / T, tau = m - b * T;
    sP[e] = to_f<AT>(x[(int64_t)(b % src_rows) * lrow + patch_src_offset(g, tau, k)]);
  }
  __syncthreads();
  for (int grp = threadIdx.x; grp < d / 4; grp += blockDim.x) {
    const int n = grp * 4;
    float acc[TM][4];
#pragma unroll
    for (int r = 0; r < TM; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[r][j] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 16) {
      float w[4][16];
#pragma unroll
      for (int j = 0; j < 4; ++j) load16(W + (int64_t)(n + j) * K + k0, w[j]);
#pragma unroll
      for (int r = 0; r < TM; ++r) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float pv = sP[r * K + k0 + k];
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][j] = fmaf(pv, w[j][k], acc[r][j]);
        }
      }
    }
    const float4 bv = *(const float4*)(bias + n);
#pragma unroll
    for (int r = 0; r < TM; ++r) {
      const int m = m0 + r;
      if (m >= M) break;
      float4 v = make_float4(acc[r][0] + bv.x, acc[r][1] + bv.y, acc[r][2] + bv.z,
                             acc[r][3] + bv.w);
      if (pe) {
        const float4 q = *(const float4*)(pe + (int64_t)(m % T) * d + n);
        v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
      }
      const int64_t row = m + (int64_t)(m / T) * out_skip;
      *(float4*)(X + row * d + n) = v;
    }
  }
}

hipError_t launch_patch_embed(const void* x, int src_rows, const PatchGeom& g, int dtype,
                              const void* W, const float* bias, const float* pe, int M, int d,
                              int out_skip, float* X, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d % 4 || g.K % 16 || ((uintptr_t)W & 15)) return hipErrorInvalidValue;
  constexpr int TM = 8;
  const size_t lds = (size_t)TM * g.K * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const int blocks = (M + TM - 1) / TM;
  if (dtype == 1)
    patch_embed_kernel<bf16_t, TM><<<blocks, 256, lds, s>>>((const bf16_t*)x, src_rows, g,
                                                           (const bf16_t*)W, bias, pe, M, d,
                                                           out_skip, X);
  else
    patch_embed_kernel<float, TM><<<blocks, 256, lds, s>>>((const float*)x, src_rows, g,
                                                          (const float*)W, bias, pe, M, d,
                                                          out_skip, X);
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
