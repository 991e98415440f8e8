// Device kernels of one training step of the adaLN-Zero DiT: the forward
// process, the loss with its gradient at the decoder output, the backward
// pieces that are not matrix products (LayerNorm + modulation, gated
// residuals, attention, bias and modulation reductions, class-table scatter),
// the weight transposes that feed the input-gradient products, and AdamW with
// the weight EMA.
//
// [Sora-cvl] Method / training objective bullet: x_t = sqrt(abar_t) x_0 +
// sqrt(1 - abar_t) eps; L_simple = ||eps_theta(x_t) - eps||^2; the covariance
// is trained with the KL term.  [DiT-wiki] Results: AdamW, constant learning
// rate, no weight decay, EMA of the weights.
#include "common.h"
#include "train.h"

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Per-row constants of the step (one thread per row, fp64 arithmetic).
// abar_t is the product of (1 - beta_j), j <= t, over the linear beta line;
// the reverse step t -> t-1 has beta_t = 1 - abar_t / abar_{t-1}, posterior
// variance beta_tilde_t = beta_t (1 - abar_{t-1}) / (1 - abar_t) and
// posterior-mean weights c_x0 = beta_t sqrt(abar_{t-1}) / (1 - abar_t),
// c_xt = (1 - abar_{t-1}) sqrt(1 - beta_t) / (1 - abar_t).  At t = 0 the
// posterior variance is 0; log beta_tilde of t = 1 takes its place in the
// learned-variance interpolation.  A t outside [0, steps) gives NaN constants.
__global__ void train_schedule_kernel(const int32_t* __restrict__ t, int B, int steps, double b0,
                                      double b1, float* __restrict__ coef, float* __restrict__ tf) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int tt = t[b];
  float* c = coef + (int64_t)b * kCoefStride;
  if (tt < 0 || tt >= steps) {
    for (int i = 0; i < kCoefStride; ++i) c[i] = __builtin_nanf("");
    tf[b] = __builtin_nanf("");
    return;
  }
  auto beta = [&](int j) { return b0 + (b1 - b0) * (double)j / (double)(steps - 1); };
  double a_prev = 1.0, a_t = 1.0;
  for (int j = 0; j <= tt; ++j) {
    a_prev = a_t;
    a_t *= 1.0 - beta(j);
  }
  const double bt = 1.0 - a_t / a_prev;
  double lbt;
  if (tt > 0) {
    lbt = log(bt * (1.0 - a_prev) / (1.0 - a_t));
  } else {
    const double a0 = 1.0 - beta(0), a1 = a0 * (1.0 - beta(1));
    const double bb = 1.0 - a1 / a0;
    lbt = log(bb * (1.0 - a0) / (1.0 - a1));
  }
  c[kSa] = (float)sqrt(a_t);
  c[kSb] = (float)sqrt(1.0 - a_t);
  c[kLogBeta] = (float)log(bt);
  c[kLogBetaTilde] = (float)lbt;
  // mu_q - mu_theta = c_x0 (x_0 - x0_hat) = c_x0 sqrt(1-abar)/sqrt(abar) (eps_theta - eps)
  c[kMeanGap] = (float)(bt * sqrt(a_prev) / (1.0 - a_t) * sqrt(1.0 - a_t) / sqrt(a_t));
  c[kPositive] = tt > 0 ? 1.0f : 0.0f;
  c[6] = 0.0f;
  c[7] = 0.0f;
  tf[b] = (float)tt;
}

// x_t = sqrt(abar_t) x_0 + sqrt(1 - abar_t) eps in the model dtype.
template <typename DT>
__global__ void train_noise_kernel(const float* __restrict__ x0, const float* __restrict__ eps,
                                   const float* __restrict__ coef, int64_t per_row, int64_t n,
                                   DT* __restrict__ xt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float* c = coef + (i / per_row) * kCoefStride;
  xt[i] = from_f<DT>(c[kSa] * x0[i] + c[kSb] * eps[i]);
}

// Xout = Xin + gate[row, n] * v, gate at mod[row * ms + goff + n], row = m / T.
__global__ void gate_residual_kernel(const float* __restrict__ Xin, const float* __restrict__ v,
                                     const float* __restrict__ mod, int ms, int goff, int T, int d,
                                     int64_t nq, float* __restrict__ Xout) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= nq) return;
  const int64_t e = q * 4, m = e / d;
  const int n = (int)(e - m * d);
  const float* g = mod + (m / T) * ms + goff + n;
  const float4 x = ((const float4*)Xin)[q], y = ((const float4*)v)[q];
  ((float4*)Xout)[q] = make_float4(x.x + g[0] * y.x, x.y + g[1] * y.y, x.z + g[2] * y.z,
                                   x.w + g[3] * y.w);
}

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

__global__ void silu_f32_kernel(const float* __restrict__ z, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = z[i] * sigmoid_f(z[i]);
}

// dz = dout * d SiLU(z) / dz = dout * s (1 + z (1 - s)), s = sigmoid(z).
__global__ void silu_bwd_kernel(const float* __restrict__ dout, const float* __restrict__ z,
                                float* __restrict__ dz, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float s = sigmoid_f(z[i]);
  dz[i] = dout[i] * s * (1.0f + z[i] * (1.0f - s));
}

template <typename DT>
__global__ void cast_f32_kernel(const float* __restrict__ in, DT* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = from_f<DT>(in[i]);
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Loss and its gradient at the decoder output.  Y [M, kout] fp32 holds each
// token's patch vector (row offset, column offset, channel; channel fastest).
// Channel c < C of the output is eps_theta: loss term (eps_theta - eps)^2,
// gradient 2 (eps_theta - eps) / n.  Channel C + c is the raw covariance
// value v: log var = f log beta + (1 - f) log beta_tilde, f = (v + 1) / 2;
// the term is KL(N(mu_q, beta_tilde) || N(mu_theta, var)) for t > 0 and
// -log N(x_0; mu_theta, var) for t = 0, with the mean gap mu_q - mu_theta
// (x_0 - mu_theta at t = 0) = c_x0 sqrt(1 - abar)/sqrt(abar) (eps_theta - eps)
// taken through a stop-gradient (it does not depend on v).  n = B C H W; the
// two sums go to acc (fp64) and dY is written in the model dtype.
template <typename DT>
__global__ __launch_bounds__(256) void train_loss_kernel(const float* __restrict__ Y,
                                                         const float* __restrict__ eps,
                                                         const float* __restrict__ coef,
                                                         PatchGeom g, int C, int64_t M, float inv_n,
                                                         DT* __restrict__ dY,
                                                         double* __restrict__ acc) {
  const int kout = g.K;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float ls = 0.0f, lv = 0.0f;
  if (idx < M * kout) {
    const int64_t m = idx / kout;
    const int j = (int)(idx - m * kout);
    const int64_t b = m / g.T;
    const int tau = (int)(m - b * g.T);
    const int i = tau / g.gw, jj = tau - i * g.gw;
    const int c = j % g.C, r = j / g.C;
    const int px = r % g.p, py = r / g.p;
    const int yy = i * g.p + py, xx = jj * g.p + px;
    const float* cf = coef + b * kCoefStride;
    const int cc = c < C ? c : c - C;
    const float e = eps[((b * C + cc) * g.H + yy) * g.W + xx];
    if (c < C) {
      const float dlt = Y[idx] - e;
      ls = dlt * dlt;
      dY[idx] = from_f<DT>(2.0f * dlt * inv_n);
    } else {
      const float v = Y[idx];
      const float e_th = Y[m * kout + r * g.C + cc];
      const float gap = cf[kMeanGap] * (e_th - e);
      const float f = 0.5f * (v + 1.0f);
      const float logv = f * cf[kLogBeta] + (1.0f - f) * cf[kLogBetaTilde];
      const float q = gap * gap * expf(-logv);
      float dlogv;
      if (cf[kPositive] > 0.0f) {
        const float r1 = expf(cf[kLogBetaTilde] - logv);
        lv = 0.5f * (-1.0f + logv - cf[kLogBetaTilde] + r1 + q);
        dlogv = 0.5f * (1.0f - r1 - q);
      } else {
        lv = 0.5f * (1.8378770664093453f + logv + q);
        dlogv = 0.5f * (1.0f - q);
      }
      dY[idx] = from_f<DT>(dlogv * 0.5f * (cf[kLogBeta] - cf[kLogBetaTilde]) * inv_n);
    }
  }
  __shared__ float red[2][4];
  ls = wave_sum(ls);
  lv = wave_sum(lv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][w] = ls;
    red[1][w] = lv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&acc[0], (double)(red[0][0] + red[0][1] + red[0][2] + red[0][3]));
    atomicAdd(&acc[1], (double)(red[1][0] + red[1][1] + red[1][2] + red[1][3]));
  }
}

__global__ void zero_f64_kernel(double* __restrict__ acc) {
  if (threadIdx.x < 2) acc[threadIdx.x] = 0.0;
}

__global__ void loss_finish_kernel(const double* __restrict__ acc, double inv_n,
                                   float* __restrict__ loss) {
  if (threadIdx.x < 2) loss[threadIdx.x] = (float)(acc[threadIdx.x] * inv_n);
}

// ---------------------------------------------------------------------------
// Backward of h = LN(x)(1 + gamma) + beta per token (LN without affine,
// biased variance, eps inside the root), with (beta, gamma) of the token's
// row.  gridDim.y workgroups per batch row: their 4 gridDim.y waves take the
// row's tokens in turn; lane l owns columns l + 64 i.  dX += (g - mean(g) -
// xhat mean(g xhat)) / sigma with g = dH (1 + gamma); d beta = sum over tokens
// of dH, d gamma = sum of dH xhat, added (atomically) to dmod at the offsets of
// beta and gamma, which must start at zero.
template <int NC>
__global__ __launch_bounds__(256) void ln_mod_bwd_kernel(const float* __restrict__ X,
                                                         const float* __restrict__ dH,
                                                         const float* __restrict__ mod, int ms,
                                                         int shoff, int scoff, int T, float eps,
                                                         float* __restrict__ dX,
                                                         float* __restrict__ dmod) {
  constexpr int PER = 2 * NC, D = 128 * NC;
  __shared__ float red[4][2][D];
  const int b = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wg = blockIdx.y * 4 + w, nw = gridDim.y * 4;
  const float* gam = mod + (int64_t)b * ms + scoff;
  float g1[PER], sh[PER], shx[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    g1[i] = 1.0f + gam[lane + 64 * i];
    sh[i] = 0.0f;
    shx[i] = 0.0f;
  }
  for (int t = wg; t < T; t += nw) {
    const int64_t row = ((int64_t)b * T + t) * D;
    float x[PER], dh[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      x[i] = X[row + lane + 64 * i];
      dh[i] = dH[row + lane + 64 * i];
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += x[i];
    const float mu = wave_sum(s) * (1.0f / D);
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) v += (x[i] - mu) * (x[i] - mu);
    const float rs = 1.0f / sqrtf(wave_sum(v) * (1.0f / D) + eps);
    float a = 0.0f, c = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      x[i] = (x[i] - mu) * rs;          // xhat
      const float gx = dh[i] * g1[i];
      a += gx;
      c += gx * x[i];
      sh[i] += dh[i];
      shx[i] += dh[i] * x[i];
    }
    a = wave_sum(a) * (1.0f / D);
    c = wave_sum(c) * (1.0f / D);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t o = row + lane + 64 * i;
      dX[o] += rs * (dh[i] * g1[i] - a - x[i] * c);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    red[w][0][lane + 64 * i] = sh[i];
    red[w][1][lane + 64 * i] = shx[i];
  }
  __syncthreads();
  for (int n = threadIdx.x; n < D; n += 256) {
    unsafeAtomicAdd(&dmod[(int64_t)b * ms + shoff + n],
                    red[0][0][n] + red[1][0][n] + red[2][0][n] + red[3][0][n]);
    unsafeAtomicAdd(&dmod[(int64_t)b * ms + scoff + n],
                    red[0][1][n] + red[1][1][n] + red[2][1][n] + red[3][1][n]);
  }
}

// Backward of Xout = Xin + alpha * v (alpha of the token's row): d alpha =
// sum over the row's tokens of dX v (to dmod at the gate offset), d v =
// alpha dX (model dtype).  dX itself passes through unchanged.
template <int NC, typename DT>
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* __restrict__ dX,
                                                       const float* __restrict__ v,
                                                       const float* __restrict__ mod, int ms,
                                                       int goff, int T, DT* __restrict__ dv,
                                                       float* __restrict__ dmod) {
  constexpr int PER = 2 * NC, D = 128 * NC;
  __shared__ float red[4][D];
  const int b = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* al = mod + (int64_t)b * ms + goff;
  float a[PER], s[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    a[i] = al[lane + 64 * i];
    s[i] = 0.0f;
  }
  for (int t = w; t < T; t += 4) {
    const int64_t row = ((int64_t)b * T + t) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t o = row + lane + 64 * i;
      const float dx = dX[o];
      s[i] += dx * v[o];
      dv[o] = from_f<DT>(a[i] * dx);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) red[w][lane + 64 * i] = s[i];
  __syncthreads();
  for (int n = threadIdx.x; n < D; n += 256)
    dmod[(int64_t)b * ms + goff + n] = red[0][n] + red[1][n] + red[2][n] + red[3][n];
}

// out[c, r] = in[r, c] for r < R, c < Cc; 64 x 64 tiles through LDS.
template <typename IT, typename OT>
__global__ __launch_bounds__(256) void transpose_kernel(const IT* __restrict__ in, int64_t R,
                                                        int64_t Cc, int64_t ldi,
                                                        OT* __restrict__ out, int64_t ldo) {
  __shared__ float tile[64][65];
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < R && c < Cc) ? to_f<IT>(in[r * ldi + c]) : 0.0f;
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int64_t c = c0 + k, r = r0 + tx;
    if (c < Cc && r < R) out[c * ldo + r] = from_f<OT>(tile[tx][k]);
  }
}

// bf16 -> bf16 transpose with 16-byte global accesses (R, Cc, ldi, ldo
// multiples of 8, 16-byte aligned): a 64 x 64 tile is read as 8-element row
// pieces, kept in LDS, and written as 8-element pieces of the output rows.
__global__ __launch_bounds__(256) void transpose16_kernel(const bf16_t* __restrict__ in, int64_t R,
                                                          int64_t Cc, int64_t ldi,
                                                          bf16_t* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int id = tid + 256 * u, row = id >> 3, cc = (id & 7) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + row < R && c0 + cc < Cc) v = *(const uint4*)(in + (r0 + row) * ldi + c0 + cc);
    *(uint4*)&tile[row][cc] = v;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int id = tid + 256 * u, oc = id >> 3, rr = (id & 7) * 8;
    if (c0 + oc < Cc && r0 + rr < R) {
      uint32_t wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wv[i] = (uint32_t)tile[rr + 2 * i][oc] | ((uint32_t)tile[rr + 2 * i + 1][oc] << 16);
      *(uint4*)(out + (c0 + oc) * ldo + r0 + rr) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  }
}

// out[c] += sum over r < rows of in[r * ld + c] for tall matrices: a
// workgroup covers 256 columns (32 lanes of 8 adjacent columns, 16-byte
// loads) of 512 rows, its 8 row lanes taking every 8th row; the row lanes
// combine in LDS and each column's partial sum adds atomically to out
// (calls into one out may overlap).
__global__ __launch_bounds__(256) void colsum_tall_bf16_kernel(const bf16_t* __restrict__ in,
                                                               int64_t rows, int64_t cols,
                                                               int64_t ld, float* __restrict__ out) {
  __shared__ float red[8][257];
  const int cl = threadIdx.x & 31, rl = threadIdx.x >> 5;
  const int64_t c8 = (int64_t)blockIdx.x * 32 + cl;
  const int64_t r0 = (int64_t)blockIdx.y * 512, r1 = min(rows, r0 + 512);
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c8 * 8 < cols) {
    for (int64_t r = r0 + rl; r < r1; r += 8) {
      const uint4 u = *(const uint4*)(in + r * ld + c8 * 8);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[2 * i] += __uint_as_float(wv[i] << 16);
        s[2 * i + 1] += __uint_as_float(wv[i] & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rl][cl * 8 + i] = s[i];
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c < cols) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += red[k][threadIdx.x];
    unsafeAtomicAdd(&out[c], t);
  }
}

// out[c] += sum over r < rows of in[r * ld + c]; one thread per column, the
// column's sum added atomically (calls into one out may overlap).
__global__ void colsum_kernel(const float* __restrict__ in, int rows, int64_t cols, int64_t ld,
                              float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int r = 0; r < rows; ++r) s += in[r * ld + c];
  unsafeAtomicAdd(&out[c], s);
}

// Class-table gradient: row y[b] of the table receives dc[b] (atomically: rows
// can share a label).  Labels outside [0, ncls] are skipped.
__global__ void class_grad_kernel(const float* __restrict__ dc, const int32_t* __restrict__ y,
                                  int B, int d, int ncls, float* __restrict__ gy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * d) return;
  const int b = (int)(i / d), n = (int)(i - (int64_t)b * d);
  const int lbl = y[b];
  if (lbl < 0 || lbl > ncls) return;
  unsafeAtomicAdd(&gy[(int64_t)lbl * d + n], dc[i]);
}

// ---------------------------------------------------------------------------
// Attention backward (vector ALUs, fp32 arithmetic).  P = exp(S - lse) is
// recomputed from q, k and the forward pass's log-sum-exp; with
// D_i = sum_e dO_ie O_ie: dV = P^T dO, dS = P (dO V^T - D), dQ = dS K / sqrt(dh),
// dK = dS^T Q / sqrt(dh).  Four lanes share one key (or query), each owning a
// quarter of the head dimension; dot products combine over the four lanes.

template <int DH, typename DT>
__global__ void attn_bwd_dot_kernel(const DT* __restrict__ O, const DT* __restrict__ dO, int H,
                                    int T, int64_t tokens, float* __restrict__ Dv) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= tokens * H) return;
  const int64_t tok = idx / H;
  const int h = (int)(idx - tok * H);
  const DT* o = O + tok * H * DH + h * DH;
  const DT* g = dO + tok * H * DH + h * DH;
  float s = 0.0f;
  if constexpr (sizeof(DT) == 2) {
#pragma unroll
    for (int c = 0; c < DH / 8; ++c) {
      const uint4 a = ((const uint4*)o)[c], b = ((const uint4*)g)[c];
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s += __uint_as_float(av[i] << 16) * __uint_as_float(bv[i] << 16) +
             __uint_as_float(av[i] & 0xFFFF0000u) * __uint_as_float(bv[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll 8
    for (int e = 0; e < DH; ++e) s += to_f<DT>(o[e]) * to_f<DT>(g[e]);
  }
  const int64_t b = tok / T;
  Dv[(b * H + h) * T + (tok - b * T)] = s;
}

template <int DH, typename DT>
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(const DT* __restrict__ QKV,
                                                          const DT* __restrict__ dO,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ Dv, int H,
                                                          int T, float scale,
                                                          DT* __restrict__ dQKV) {
  constexpr int FPT = DH / 4, QT = 32;
  __shared__ float sQ[QT][DH], sG[QT][DH], sL[QT], sD[QT];
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, part = tid & 3;
  const int j = blockIdx.x * 64 + (tid >> 2);
  const int64_t ld = 3LL * H * DH;
  const DT* base = QKV + (int64_t)b * T * ld + h * DH;
  const DT* gb = dO + (int64_t)b * T * H * DH + h * DH;
  const bool valid = j < T;
  float k[FPT], v[FPT], dk[FPT], dv[FPT];
#pragma unroll
  for (int e = 0; e < FPT; ++e) {
    k[e] = valid ? to_f<DT>(base[(int64_t)j * ld + H * DH + part * FPT + e]) : 0.0f;
    v[e] = valid ? to_f<DT>(base[(int64_t)j * ld + 2 * H * DH + part * FPT + e]) : 0.0f;
    dk[e] = 0.0f;
    dv[e] = 0.0f;
  }
  const float* L = lse + (int64_t)bh * T;
  const float* Dd = Dv + (int64_t)bh * T;
  for (int q0 = 0; q0 < T; q0 += QT) {
    __syncthreads();
    for (int e = tid; e < QT * DH; e += 256) {
      const int r = e / DH, c = e - r * DH, qi = q0 + r;
      const bool ok = qi < T;
      sQ[r][c] = ok ? to_f<DT>(base[(int64_t)qi * ld + c]) : 0.0f;
      sG[r][c] = ok ? to_f<DT>(gb[(int64_t)qi * H * DH + c]) : 0.0f;
    }
    if (tid < QT) {
      const int qi = q0 + tid;
      sL[tid] = qi < T ? L[qi] : 0.0f;
      sD[tid] = qi < T ? Dd[qi] : 0.0f;
    }
    __syncthreads();
    const int nq = min(QT, T - q0);
    for (int r = 0; r < nq; ++r) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        s += sQ[r][part * FPT + e] * k[e];
        dp += sG[r][part * FPT + e] * v[e];
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      dp += __shfl_xor(dp, 1, 64);
      dp += __shfl_xor(dp, 2, 64);
      const float p = expf(s * scale - sL[r]);
      const float ds = p * (dp - sD[r]);
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        dv[e] += p * sG[r][part * FPT + e];
        dk[e] += ds * sQ[r][part * FPT + e];
      }
    }
  }
  if (valid) {
    DT* o = dQKV + ((int64_t)b * T + j) * ld + h * DH + part * FPT;
#pragma unroll
    for (int e = 0; e < FPT; ++e) {
      o[H * DH + e] = from_f<DT>(dk[e] * scale);
      o[2 * H * DH + e] = from_f<DT>(dv[e]);
    }
  }
}

template <int DH, typename DT>
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(const DT* __restrict__ QKV,
                                                         const DT* __restrict__ dO,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ Dv, int H,
                                                         int T, float scale,
                                                         DT* __restrict__ dQKV) {
  constexpr int FPT = DH / 4, KT = 32;
  __shared__ float sK[KT][DH], sV[KT][DH];
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, part = tid & 3;
  const int i = blockIdx.x * 64 + (tid >> 2);
  const int64_t ld = 3LL * H * DH;
  const DT* base = QKV + (int64_t)b * T * ld + h * DH;
  const bool valid = i < T;
  float q[FPT], g[FPT], dq[FPT];
  const DT* grow = dO + ((int64_t)b * T + (valid ? i : 0)) * H * DH + h * DH + part * FPT;
#pragma unroll
  for (int e = 0; e < FPT; ++e) {
    q[e] = valid ? to_f<DT>(base[(int64_t)i * ld + part * FPT + e]) : 0.0f;
    g[e] = valid ? to_f<DT>(grow[e]) : 0.0f;
    dq[e] = 0.0f;
  }
  const float li = valid ? lse[(int64_t)bh * T + i] : 0.0f;
  const float di = valid ? Dv[(int64_t)bh * T + i] : 0.0f;
  for (int k0 = 0; k0 < T; k0 += KT) {
    __syncthreads();
    for (int e = tid; e < KT * DH; e += 256) {
      const int r = e / DH, c = e - r * DH, kj = k0 + r;
      const bool ok = kj < T;
      sK[r][c] = ok ? to_f<DT>(base[(int64_t)kj * ld + H * DH + c]) : 0.0f;
      sV[r][c] = ok ? to_f<DT>(base[(int64_t)kj * ld + 2 * H * DH + c]) : 0.0f;
    }
    __syncthreads();
    const int nk = min(KT, T - k0);
    for (int r = 0; r < nk; ++r) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        s += q[e] * sK[r][part * FPT + e];
        dp += g[e] * sV[r][part * FPT + e];
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      dp += __shfl_xor(dp, 1, 64);
      dp += __shfl_xor(dp, 2, 64);
      const float ds = expf(s * scale - li) * (dp - di);
#pragma unroll
      for (int e = 0; e < FPT; ++e) dq[e] += ds * sK[r][part * FPT + e];
    }
  }
  if (valid) {
    DT* o = dQKV + ((int64_t)b * T + i) * ld + h * DH + part * FPT;
#pragma unroll
    for (int e = 0; e < FPT; ++e) o[e] = from_f<DT>(dq[e] * scale);
  }
}

// ---------------------------------------------------------------------------
// AdamW on the fp32 master weights, then the EMA and the model-dtype copy.
// m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g^2 (the (1 - b) factors come in
// precomputed);
// p -= lr (m bc1 / (sqrt(v bc2) + eps) + wd p), bc = 1 / (1 - b^step);
// ema = decay ema + (1 - decay) p; w = p in the model dtype.
template <typename WT>
__global__ void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                             float* __restrict__ m, float* __restrict__ v, float* __restrict__ ema,
                             int64_t n, AdamArgs a, WT* __restrict__ w) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float gi = g[i];
  const float mi = a.b1 * m[i] + a.omb1 * gi;
  const float vi = a.b2 * v[i] + a.omb2 * gi * gi;
  const float pi = p[i];
  const float pn = pi - a.lr * (mi * a.bc1 / (sqrtf(vi * a.bc2) + a.eps) + a.wd * pi);
  m[i] = mi;
  v[i] = vi;
  p[i] = pn;
  ema[i] = a.ema * ema[i] + a.omema * pn;
  w[i] = from_f<WT>(pn);
}

int blocks_for(int64_t n, int t = 256) { return (int)((n + t - 1) / t); }

}  // namespace

// ---------------------------------------------------------------------------
// Launchers

hipError_t launch_train_schedule(const int32_t* t, int B, int steps, double b0, double b1,
                                 float* coef, float* tf, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (steps < 2) return hipErrorInvalidValue;
  train_schedule_kernel<<<blocks_for(B, 64), 64, 0, s>>>(t, B, steps, b0, b1, coef, tf);
  return hipGetLastError();
}

hipError_t launch_train_noise(const float* x0, const float* eps, const float* coef,
                              int64_t per_row, int64_t n, int dtype, void* xt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 1)
    train_noise_kernel<bf16_t><<<blocks_for(n), 256, 0, s>>>(x0, eps, coef, per_row, n, (bf16_t*)xt);
  else
    train_noise_kernel<float><<<blocks_for(n), 256, 0, s>>>(x0, eps, coef, per_row, n, (float*)xt);
  return hipGetLastError();
}

hipError_t launch_gate_residual(const float* Xin, const float* v, const float* mod, int ms,
                                int goff, int T, int d, int64_t M, float* Xout, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d % 4) return hipErrorInvalidValue;
  const int64_t nq = M * d / 4;
  gate_residual_kernel<<<blocks_for(nq), 256, 0, s>>>(Xin, v, mod, ms, goff, T, d, nq, Xout);
  return hipGetLastError();
}

hipError_t launch_silu_f32(const float* z, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  silu_f32_kernel<<<blocks_for(n), 256, 0, s>>>(z, out, n);
  return hipGetLastError();
}

hipError_t launch_silu_bwd(const float* dout, const float* z, float* dz, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  silu_bwd_kernel<<<blocks_for(n), 256, 0, s>>>(dout, z, dz, n);
  return hipGetLastError();
}

hipError_t launch_cast_f32(const float* in, void* out, int64_t n, int dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 1)
    cast_f32_kernel<bf16_t><<<blocks_for(n), 256, 0, s>>>(in, (bf16_t*)out, n);
  else
    cast_f32_kernel<float><<<blocks_for(n), 256, 0, s>>>(in, (float*)out, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_f32_kernel<<<blocks_for(n), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_train_loss(const float* Y, const float* eps, const float* coef,
                             const PatchGeom& gout, int C, int64_t M, int dtype, void* dY,
                             double* acc, float* loss, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (gout.F != 1 || gout.pt != 1) return hipErrorInvalidValue;
  const int64_t n_lat = M / gout.T * C * gout.H * gout.W;
  const float inv_n = (float)(1.0 / (double)n_lat);
  zero_f64_kernel<<<1, 64, 0, s>>>(acc);
  const int64_t total = M * gout.K;
  if (dtype == 1)
    train_loss_kernel<bf16_t><<<blocks_for(total), 256, 0, s>>>(Y, eps, coef, gout, C, M, inv_n,
                                                                (bf16_t*)dY, acc);
  else
    train_loss_kernel<float><<<blocks_for(total), 256, 0, s>>>(Y, eps, coef, gout, C, M, inv_n,
                                                               (float*)dY, acc);
  loss_finish_kernel<<<1, 64, 0, s>>>(acc, 1.0 / (double)n_lat, loss);
  return hipGetLastError();
}

hipError_t launch_ln_mod_bwd(const float* X, const float* dH, const float* mod, int ms, int shoff,
                             int scoff, int B, int T, int d, float eps, float* dX, float* dmod,
                             hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (d % 128 || d > 2048) return hipErrorInvalidValue;
  // about 1024 workgroups, each with at least one token per wave
  int split = (1024 + B - 1) / B;
  split = split > (T + 3) / 4 ? (T + 3) / 4 : split;
  split = split < 1 ? 1 : (split > 16 ? 16 : split);
#define DIT_LNB(NC)                                                                         \
  case NC:                                                                                  \
    ln_mod_bwd_kernel<NC><<<dim3(B, split), 256, 0, s>>>(X, dH, mod, ms, shoff, scoff, T, eps, \
                                                        dX, dmod);                             \
    break;
  switch (d / 128) {
    DIT_LNB(1) DIT_LNB(2) DIT_LNB(3) DIT_LNB(4) DIT_LNB(5) DIT_LNB(6) DIT_LNB(7) DIT_LNB(8)
    DIT_LNB(9) DIT_LNB(10) DIT_LNB(11) DIT_LNB(12) DIT_LNB(13) DIT_LNB(14) DIT_LNB(15)
    DIT_LNB(16)
    default: return hipErrorInvalidValue;
  }
#undef DIT_LNB
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const float* dX, const float* v, const float* mod, int ms, int goff,
                           int B, int T, int d, int dtype, void* dv, float* dmod, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (d % 128 || d > 2048) return hipErrorInvalidValue;
#define DIT_GB(NC)                                                                             \
  case NC:                                                                                     \
    if (dtype == 1)                                                                            \
      gate_bwd_kernel<NC, bf16_t><<<B, 256, 0, s>>>(dX, v, mod, ms, goff, T, (bf16_t*)dv, dmod); \
    else                                                                                       \
      gate_bwd_kernel<NC, float><<<B, 256, 0, s>>>(dX, v, mod, ms, goff, T, (float*)dv, dmod);   \
    break;
  switch (d / 128) {
    DIT_GB(1) DIT_GB(2) DIT_GB(3) DIT_GB(4) DIT_GB(5) DIT_GB(6) DIT_GB(7) DIT_GB(8)
    DIT_GB(9) DIT_GB(10) DIT_GB(11) DIT_GB(12) DIT_GB(13) DIT_GB(14) DIT_GB(15) DIT_GB(16)
    default: return hipErrorInvalidValue;
  }
#undef DIT_GB
  return hipGetLastError();
}

hipError_t launch_transpose(const void* in, int in_dtype, int64_t R, int64_t Cc, int64_t ldi,
                            void* out, int out_dtype, int64_t ldo, hipStream_t s) {
  if (R <= 0 || Cc <= 0) return hipSuccess;
  if ((Cc + 63) / 64 > INT32_MAX || (R + 63) / 64 > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((Cc + 63) / 64), (unsigned)((R + 63) / 64));
  if (in_dtype == 1 && out_dtype == 1 && R % 8 == 0 && Cc % 8 == 0 && ldi % 8 == 0 &&
      ldo % 8 == 0 && ((uintptr_t)in & 15) == 0 && ((uintptr_t)out & 15) == 0) {
    transpose16_kernel<<<grid, 256, 0, s>>>((const bf16_t*)in, R, Cc, ldi, (bf16_t*)out, ldo);
    return hipGetLastError();
  }
#define DIT_TR(IT, OT) \
  transpose_kernel<IT, OT><<<grid, 256, 0, s>>>((const IT*)in, R, Cc, ldi, (OT*)out, ldo);
  if (in_dtype == 1 && out_dtype == 1) { DIT_TR(bf16_t, bf16_t) }
  else if (in_dtype == 1) { DIT_TR(bf16_t, float) }
  else if (out_dtype == 1) { DIT_TR(float, bf16_t) }
  else { DIT_TR(float, float) }
#undef DIT_TR
  return hipGetLastError();
}

hipError_t launch_colsum_tall_bf16(const void* in, int64_t rows, int64_t cols, int64_t ld,
                                  float* out, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 8 || ld % 8 || ((uintptr_t)in & 15) || rows > kColsumTallMaxRows)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols + 255) / 256), (unsigned)((rows + 511) / 512));
  colsum_tall_bf16_kernel<<<grid, 256, 0, s>>>((const bf16_t*)in, rows, cols, ld, out);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* in, int rows, int64_t cols, int64_t ld, float* out,
                         hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  colsum_kernel<<<blocks_for(cols), 256, 0, s>>>(in, rows, cols, ld, out);
  return hipGetLastError();
}

hipError_t launch_class_grad(const float* dc, const int32_t* y, int B, int d, int ncls, float* gy,
                             hipStream_t s) {
  if (B <= 0) return hipSuccess;
  class_grad_kernel<<<blocks_for((int64_t)B * d), 256, 0, s>>>(dc, y, B, d, ncls, gy);
  return hipGetLastError();
}

hipError_t launch_attention_bwd(const void* qkv, const void* O, const void* dO, const float* lse,
                                float* Dv, int B, int heads, int T, int dh, int dtype, void* dqkv,
                                hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  if (dh != 64 && dh != 72) return hipErrorInvalidValue;
  if ((int64_t)B * heads > 65535) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)dh);
  const int64_t tokens = (int64_t)B * T;
  const dim3 grid((T + 63) / 64, B * heads);
#define DIT_AB(DH, DT)                                                                        \
  attn_bwd_dot_kernel<DH, DT><<<blocks_for(tokens * heads), 256, 0, s>>>(                     \
      (const DT*)O, (const DT*)dO, heads, T, tokens, Dv);                                     \
  attn_bwd_kv_kernel<DH, DT><<<grid, 256, 0, s>>>((const DT*)qkv, (const DT*)dO, lse, Dv, heads, \
                                                  T, scale, (DT*)dqkv);                       \
  attn_bwd_q_kernel<DH, DT><<<grid, 256, 0, s>>>((const DT*)qkv, (const DT*)dO, lse, Dv, heads,  \
                                                 T, scale, (DT*)dqkv);
  if (dtype == 1) {
    if (dh == 64)
      attn_bwd_dot_kernel<64, bf16_t><<<blocks_for(tokens * heads), 256, 0, s>>>(
          (const bf16_t*)O, (const bf16_t*)dO, heads, T, tokens, Dv);
    else
      attn_bwd_dot_kernel<72, bf16_t><<<blocks_for(tokens * heads), 256, 0, s>>>(
          (const bf16_t*)O, (const bf16_t*)dO, heads, T, tokens, Dv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attention_bwd_mfma(qkv, dO, lse, Dv, B, heads, T, dh, dqkv, s);
  } else {
    if (dh == 64) { DIT_AB(64, float) } else { DIT_AB(72, float) }
  }
#undef DIT_AB
  return hipGetLastError();
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, float* ema, int64_t n,
                        const AdamArgs& a, void* w, int w_dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (w_dtype == 1)
    adamw_kernel<bf16_t><<<blocks_for(n), 256, 0, s>>>(p, g, m, v, ema, n, a, (bf16_t*)w);
  else
    adamw_kernel<float><<<blocks_for(n), 256, 0, s>>>(p, g, m, v, ema, n, a, (float*)w);
  return hipGetLastError();
}
