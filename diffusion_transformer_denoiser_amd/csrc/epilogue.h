// GEMM epilogues fused into the producing kernels (bias, SiLU, conditioning
// sum, alpha-gated residual, tanh-GELU, patch position term).
#pragma once
#include "common.h"

// log2(10000)
#define DIT_LOG2_1E4 13.287712379549449f

// 2-D sine-cosine position embedding of token (i, j), feature n of d:
// d/4 frequencies w_k = 10000^(-k/(d/4)); [sin(i w) | cos(i w) | sin(j w) | cos(j w)].
__device__ __forceinline__ float pos_embed_2d(int i, int j, int n, int d) {
  int dq = d >> 2;
  int seg = n / dq, kk = n - seg * dq;
  float w = exp2f(-(float)kk / (float)dq * DIT_LOG2_1E4);
  float ang = (float)(seg < 2 ? i : j) * w;
  return (seg & 1) ? cosf(ang) : sinf(ang);
}

template <int EPI, typename DT>
__device__ __forceinline__ void epi_apply(const EpiParams& ep, int m, int n, float acc) {
  float v = acc + (ep.bias ? ep.bias[n] : 0.0f);
  if constexpr (EPI == EPI_BIAS_F32) {
    ((float*)ep.out)[(int64_t)m * ep.ldo + n] = v;
  } else if constexpr (EPI == EPI_BIAS_SILU) {
    ((float*)ep.out)[(int64_t)m * ep.ldo + n] = silu_f(v);
  } else if constexpr (EPI == EPI_COND) {
    float* c = (float*)ep.out;
    int64_t o = (int64_t)m * ep.ldo + n;
    if (ep.add_prev) v += c[o];
    if (ep.table) {
      int lbl = (m >= ep.null_from) ? ep.ncls : ep.labels[m % ep.label_rows];
      if (lbl < 0 || lbl > ep.ncls) v = __builtin_nanf("");
      else v += ep.table[(int64_t)lbl * ep.ldo + n];
    }
    c[o] = v;
    ((DT*)ep.silu_out)[o] = from_f<DT>(silu_f(v));
  } else if constexpr (EPI == EPI_BIAS_DT) {
    ((DT*)ep.out)[row_map(m, ep.o_seg, ep.o_skip, ep.o_off) * ep.ldo + n] = from_f<DT>(v);
  } else if constexpr (EPI == EPI_GATED) {
    int b = ep.tok_seg ? ep.tok_seg[m] : m / ep.T;
    float g = ep.mod ? ep.mod[(int64_t)b * ep.mod_stride + ep.gate_off + n] : 1.0f;
    float* X = (float*)ep.out;
    int64_t o = (int64_t)m * ep.ldo + n;
    X[o] = X[o] + g * v;
  } else if constexpr (EPI == EPI_GELU) {
    ((DT*)ep.out)[(int64_t)m * ep.ldo + n] = from_f<DT>(gelu_tanh_f(v));
  } else if constexpr (EPI == EPI_PATCH) {
    if (ep.pe_tab) v += ep.pe_tab[(int64_t)(m % ep.T) * ep.ldo + n];
    const int64_t orow = m + (int64_t)(m / ep.T) * ep.out_skip;
    ((float*)ep.out)[orow * ep.ldo + n] = v;
  } else if constexpr (EPI == EPI_SILU_DT) {
    ((DT*)ep.out)[(int64_t)m * ep.ldo + n] = from_f<DT>(silu_f(v));
  } else if constexpr (EPI == EPI_ATOMIC_F32) {
    unsafeAtomicAdd(&((float*)ep.out)[(int64_t)m * ep.ldo + n], v);
  } else if constexpr (EPI == EPI_GELU2) {
    ((DT*)ep.out)[(int64_t)m * ep.ldo + n] = from_f<DT>(gelu_tanh_f(v));
    ((DT*)ep.aux)[(int64_t)m * ep.ldo + n] = from_f<DT>(v);
  } else if constexpr (EPI == EPI_DGELU) {
    const float z = to_f<DT>(((const DT*)ep.aux)[(int64_t)m * ep.ldo + n]);
    ((DT*)ep.out)[(int64_t)m * ep.ldo + n] = from_f<DT>(v * gelu_tanh_grad_f(z));
  }
}
