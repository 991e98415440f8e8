// LayerNorm (no affine) fused with adaLN modulation, and the per-head Q-K
// LayerNorm + 3-D rotary embedding of spacetime attention.
#include "common.h"

#define DIT_LOG2_1E4 13.287712379549449f

// H[m, :] = LN(X[m, :]) * (1 + scale[b, :]) + shift[b, :],  b = m / T.
// One wave per R consecutive rows.  d = 256 N4 + 128 N2: each lane holds N4
// float4 and N2 float2 of every row (16-byte loads where the width allows),
// so a row is read from HBM once and both moments come from registers.  The
// loads of all R rows are issued before the first reduction, which keeps R
// rows of memory traffic in flight per wave; the R rows share one read of
// the shift and scale vectors when they belong to one batch row.
template <int N4, int N2, typename DT, int R>
__global__ __launch_bounds__(256) void ln_modulate_kernel(const float* __restrict__ X, int M,
                                                          int T, const float* __restrict__ mod,
                                                          int mod_stride, int shift_off,
                                                          int scale_off, float eps,
                                                          DT* __restrict__ H,
                                                          const int* __restrict__ tok_seg) {
  constexpr int D = 256 * N4 + 128 * N2;
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  const int lane = threadIdx.x & 63;
  if (row0 >= M) return;
  float4 v4[R][N4 ? N4 : 1];
  float2 v2[R][N2 ? N2 : 1];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* x = X + (int64_t)min(row0 + r, M - 1) * D;
#pragma unroll
    for (int i = 0; i < N4; ++i) v4[r][i] = ((const float4*)x)[lane + 64 * i];
#pragma unroll
    for (int i = 0; i < N2; ++i) v2[r][i] = ((const float2*)(x + 256 * N4))[lane + 64 * i];
  }
  // shift / scale of a batch row, in the same register layout as a row of X
  float4 sh4[N4 ? N4 : 1], sc4[N4 ? N4 : 1];
  float2 sh2[N2 ? N2 : 1], sc2[N2 ? N2 : 1];
  auto load_mod = [&](int b) {
    const float* sh = mod + (int64_t)b * mod_stride + shift_off;
    const float* sc = mod + (int64_t)b * mod_stride + scale_off;
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      sh4[i] = ((const float4*)sh)[lane + 64 * i];
      sc4[i] = ((const float4*)sc)[lane + 64 * i];
    }
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      sh2[i] = ((const float2*)(sh + 256 * N4))[lane + 64 * i];
      sc2[i] = ((const float2*)(sc + 256 * N4))[lane + 64 * i];
    }
  };
  auto brow = [&](int row) { return tok_seg ? tok_seg[row] : row / T; };
  const int rlast = min(row0 + R, M) - 1;
  const bool shared = !tok_seg && row0 / T == rlast / T;
  if (shared) load_mod(row0 / T);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    if (row >= M) break;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < N4; ++i) s += (v4[r][i].x + v4[r][i].y) + (v4[r][i].z + v4[r][i].w);
#pragma unroll
    for (int i = 0; i < N2; ++i) s += v2[r][i].x + v2[r][i].y;
    const float mean = wave_sum(s) * (1.0f / D);
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      const float a = v4[r][i].x - mean, b = v4[r][i].y - mean;
      const float c = v4[r][i].z - mean, e = v4[r][i].w - mean;
      q += (a * a + b * b) + (c * c + e * e);
    }
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      const float a = v2[r][i].x - mean, b = v2[r][i].y - mean;
      q += a * a + b * b;
    }
    const float var = wave_sum(q) * (1.0f / D);
    const float rstd = 1.0f / sqrtf(var + eps);
    if (!shared) load_mod(brow(row));
    DT* h = H + (int64_t)row * D;
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      const float4 x = v4[r][i], g = sc4[i], t = sh4[i];
      const float h0 = (x.x - mean) * rstd * (1.0f + g.x) + t.x;
      const float h1 = (x.y - mean) * rstd * (1.0f + g.y) + t.y;
      const float h2 = (x.z - mean) * rstd * (1.0f + g.z) + t.z;
      const float h3 = (x.w - mean) * rstd * (1.0f + g.w) + t.w;
      if constexpr (sizeof(DT) == 2)
        ((uint2*)h)[lane + 64 * i] = make_uint2(f2bf2(h0, h1), f2bf2(h2, h3));
      else
        ((float4*)h)[lane + 64 * i] = make_float4(h0, h1, h2, h3);
    }
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      const float2 x = v2[r][i], g = sc2[i], t = sh2[i];
      const float h0 = (x.x - mean) * rstd * (1.0f + g.x) + t.x;
      const float h1 = (x.y - mean) * rstd * (1.0f + g.y) + t.y;
      if constexpr (sizeof(DT) == 2)
        ((uint32_t*)(h + 256 * N4))[lane + 64 * i] = f2bf2(h0, h1);
      else
        ((float2*)(h + 256 * N4))[lane + 64 * i] = make_float2(h0, h1);
    }
  }
}

#ifndef DIT_LN_ROWS
#define DIT_LN_ROWS 2
#endif
template <typename DT>
static hipError_t ln_dispatch(const float* X, int M, int T, int d, const float* mod,
                              int mod_stride, int shift_off, int scale_off, float eps, DT* H,
                              const int* tok_seg, hipStream_t s) {
  constexpr int R = DIT_LN_ROWS;
  dim3 grid((M + 4 * R - 1) / (4 * R));
#define DIT_LN_CASE(N4, N2)                                                                    \
  if (d == 256 * N4 + 128 * N2) {                                                              \
    ln_modulate_kernel<N4, N2, DT, R><<<grid, 256, 0, s>>>(X, M, T, mod, mod_stride, shift_off, \
                                                           scale_off, eps, H, tok_seg);       \
    return hipGetLastError();                                                                  \
  }
  DIT_LN_CASE(0, 1) DIT_LN_CASE(1, 0) DIT_LN_CASE(1, 1) DIT_LN_CASE(2, 0) DIT_LN_CASE(2, 1)
  DIT_LN_CASE(3, 0) DIT_LN_CASE(3, 1) DIT_LN_CASE(4, 0) DIT_LN_CASE(4, 1) DIT_LN_CASE(5, 0)
  DIT_LN_CASE(5, 1) DIT_LN_CASE(6, 0) DIT_LN_CASE(6, 1) DIT_LN_CASE(7, 0) DIT_LN_CASE(7, 1)
  DIT_LN_CASE(8, 0)
#undef DIT_LN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_ln_modulate(const float* X, int M, int T, int d, const float* mod,
                              int mod_stride, int shift_off, int scale_off, float eps, void* H,
                              int dtype, hipStream_t s, const int* tok_seg) {
  if (M <= 0) return hipSuccess;
  if (d % 128 || d > 2048) return hipErrorInvalidValue;
  if (dtype == 1)
    return ln_dispatch<bf16_t>(X, M, T, d, mod, mod_stride, shift_off, scale_off, eps,
                               (bf16_t*)H, tok_seg, s);
  return ln_dispatch<float>(X, M, T, d, mod, mod_stride, shift_off, scale_off, eps, (float*)H,
                            tok_seg, s);
}

// Per-head q/k post-processing for spacetime attention, in place on the packed
// in-projection output qkv [B*T, 3 H DH]: LayerNorm over each head's DH
// features (no affine), then the 3-D rotary embedding: DH splits into
// (frame, row, col) thirds of da = DH/3; pair (x_2k, x_2k+1) of a third rotates
// by pos * 10000^(-2k/da).  One thread per (q or k, token, head).
template <int DH, typename DT>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(DT* __restrict__ qkv, int64_t rows,
                                                           int heads, int T, int qk_norm,
                                                           float eps, int rope, int gh, int gw,
                                                           const float* __restrict__ rms_g,
                                                           int L) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 2 * rows) return;
  const int which = idx >= rows;                 // 0: q, 1: k
  const int64_t r = idx - which * rows;           // (token, head)
  const int64_t bt = r / heads;
  const int h = (int)(r - bt * heads);
  DT* p = qkv + bt * 3 * heads * DH + (int64_t)which * heads * DH + h * DH;
  float x[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) x[e] = to_f<DT>(p[e]);
  if (qk_norm == 2) {
    // RMSNorm with scale 1 + g; g of q or k of the text stream for the first
    // L tokens of a row, of the image stream for the rest (rms_g [4, DH]:
    // image q, image k, text q, text k)
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < DH; ++e) ss += x[e] * x[e];
    const float rr = 1.0f / sqrtf(ss * (1.0f / DH) + eps);
    const int t = (int)(bt % T);
    const float* g = rms_g + ((t < L ? 2 : 0) + which) * DH;
#pragma unroll
    for (int e = 0; e < DH; ++e) x[e] = x[e] * rr * (1.0f + g[e]);
  } else if (qk_norm) {
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < DH; ++e) s += x[e];
    float mean = s * (1.0f / DH), v = 0.0f;
#pragma unroll
    for (int e = 0; e < DH; ++e) v += (x[e] - mean) * (x[e] - mean);
    float rstd = 1.0f / sqrtf(v * (1.0f / DH) + eps);
#pragma unroll
    for (int e = 0; e < DH; ++e) x[e] = (x[e] - mean) * rstd;
  }
  if constexpr (DH % 6 == 0) {
    if (rope) {
      constexpr int DA = DH / 3;
      int t = (int)(bt % T);
      int pos[3] = {t / (gh * gw), (t / gw) % gh, t % gw};
#pragma unroll
      for (int a = 0; a < 3; ++a) {
#pragma unroll
        for (int kk = 0; kk < DA / 2; ++kk) {
          float theta = exp2f(-2.0f * kk / DA * DIT_LOG2_1E4);
          float sn, cs;
          sincosf((float)pos[a] * theta, &sn, &cs);
          float x0 = x[a * DA + 2 * kk], x1 = x[a * DA + 2 * kk + 1];
          x[a * DA + 2 * kk] = x0 * cs - x1 * sn;
          x[a * DA + 2 * kk + 1] = x0 * sn + x1 * cs;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < DH; ++e) p[e] = from_f<DT>(x[e]);
}

hipError_t launch_qk_norm_rope(void* qkv, int B, int heads, int T, int dh, int dtype,
                               int qk_norm, float eps, int rope, int gh, int gw, hipStream_t s) {
  int64_t rows = (int64_t)B * T * heads;
  if (rows <= 0) return hipSuccess;
  int blocks = (int)((2 * rows + 255) / 256);
  if (dh == 72) {
    if (dtype == 1)
      qk_norm_rope_kernel<72, bf16_t><<<blocks, 256, 0, s>>>((bf16_t*)qkv, rows, heads, T,
                                                             qk_norm, eps, rope, gh, gw, nullptr, 0);
    else
      qk_norm_rope_kernel<72, float><<<blocks, 256, 0, s>>>((float*)qkv, rows, heads, T, qk_norm,
                                                            eps, rope, gh, gw, nullptr, 0);
  } else if (dh == 64) {
    if (rope) return hipErrorInvalidValue;
    if (dtype == 1)
      qk_norm_rope_kernel<64, bf16_t><<<blocks, 256, 0, s>>>((bf16_t*)qkv, rows, heads, T,
                                                             qk_norm, eps, 0, gh, gw, nullptr, 0);
    else
      qk_norm_rope_kernel<64, float><<<blocks, 256, 0, s>>>((float*)qkv, rows, heads, T, qk_norm,
                                                            eps, 0, gh, gw, nullptr, 0);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qk_rms(void* qkv, int B, int heads, int T, int L, int dh, int dtype, float eps,
                         const float* g4, hipStream_t s) {
  const int64_t rows = (int64_t)B * T * heads;
  if (rows <= 0) return hipSuccess;
  const int blocks = (int)((2 * rows + 255) / 256);
  if (dh == 64) {
    if (dtype == 1)
      qk_norm_rope_kernel<64, bf16_t><<<blocks, 256, 0, s>>>((bf16_t*)qkv, rows, heads, T, 2, eps,
                                                             0, 1, 1, g4, L);
    else
      qk_norm_rope_kernel<64, float><<<blocks, 256, 0, s>>>((float*)qkv, rows, heads, T, 2, eps, 0,
                                                            1, 1, g4, L);
  } else if (dh == 72) {
    if (dtype == 1)
      qk_norm_rope_kernel<72, bf16_t><<<blocks, 256, 0, s>>>((bf16_t*)qkv, rows, heads, T, 2, eps,
                                                             0, 1, 1, g4, L);
    else
      qk_norm_rope_kernel<72, float><<<blocks, 256, 0, s>>>((float*)qkv, rows, heads, T, 2, eps, 0,
                                                            1, 1, g4, L);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
