// fp32-arithmetic tiled GEMM C = A W^T on the vector ALUs.
//
// Serves the small products of the forward pass (timestep MLP, pooled
// projection, patch embedding with its patchify gather, linear decoder) and
// every product of the fp32 model path.  64x64 tile, BK = 16, 256 threads,
// 4x4 outputs per thread, sequential fp32 accumulation over k (deterministic).
#include "common.h"
#include "epilogue.h"

namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <int ASRC, typename AT>
__device__ __forceinline__ float load_a(const ALoad& a, int m, int k) {
  if constexpr (ASRC == A_PATCH) {
    int b = m / a.g.T, tau = m - b * a.g.T;
    int64_t row = (int64_t)a.g.C * a.g.F * a.g.H * a.g.W;
    return to_f<AT>(((const AT*)a.ptr)[(int64_t)(b % a.src_rows) * row +
                                       patch_src_offset(a.g, tau, k)]);
  } else {
    const int64_t row = row_map(m % a.src_rows, a.seg, a.skip, a.off);
    if (a.trans) return to_f<AT>(((const AT*)a.ptr)[(int64_t)k * a.lda + row]);
    return to_f<AT>(((const AT*)a.ptr)[row * a.lda + k]);
  }
}

template <int EPI, int ASRC, typename AT, typename WT, typename DT>
__global__ __launch_bounds__(256) void gemm_valu_kernel(ALoad a, const WT* __restrict__ W, int M,
                                                         int N, int K, EpiParams ep) {
  __shared__ __attribute__((aligned(16))) float As[BK][BM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[BK][BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  // split-K: grid layer z reduces over [kbeg, kend)
  const int64_t ldw = ep.ldw ? ep.ldw : K;
  const int kbeg = ep.ksplit ? blockIdx.z * ep.ksplit : 0;
  const int kend = ep.ksplit ? min(K, kbeg + ep.ksplit) : K;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const int m = m0 + lr, n = n0 + lr;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int k = k0 + lk + u;
      As[lk + u][lr] = (m < M && k < kend) ? load_a<ASRC, AT>(a, m, k) : 0.0f;
      Bs[lk + u][lr] = (n < N && k < kend)
                           ? to_f<WT>(ep.w_trans ? W[(int64_t)k * ldw + n] : W[(int64_t)n * ldw + k])
                           : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float4 av = *(const float4*)&As[kk][ty * 4];
      float4 bv = *(const float4*)&Bs[kk][tx * 4];
      float ar[4] = {av.x, av.y, av.z, av.w};
      float br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int n = n0 + tx * 4 + j;
      if (n < N) epi_apply<EPI, DT>(ep, m, n, acc[i][j]);
    }
  }
}

template <int EPI, int ASRC, typename AT, typename WT, typename DT>
hipError_t run(const ALoad& a, const void* W, int M, int N, int K, const EpiParams& ep,
               hipStream_t s) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, ep.ksplit ? (K + ep.ksplit - 1) / ep.ksplit : 1);
  gemm_valu_kernel<EPI, ASRC, AT, WT, DT><<<grid, 256, 0, s>>>(a, (const WT*)W, M, N, K, ep);
  return hipGetLastError();
}

// The model dtype fixes the weight dtype and the dtype of dtype-valued outputs
// (SiLU(c), q/k/v, GELU).  The A operand is fp32 (embedding tables, pooled
// vectors) or the model dtype (activations, latent).
template <int EPI, int ASRC, typename DT>
hipError_t dispatch_a(const ALoad& a, const void* W, int M, int N, int K, const EpiParams& ep,
                      hipStream_t s) {
  if (a.a_dtype == 1) return run<EPI, ASRC, bf16_t, DT, DT>(a, W, M, N, K, ep, s);
  return run<EPI, ASRC, float, DT, DT>(a, W, M, N, K, ep, s);
}

template <int EPI, typename DT>
hipError_t dispatch_src(int asrc, const ALoad& a, const void* W, int M, int N, int K,
                        const EpiParams& ep, hipStream_t s) {
  if (asrc == A_PATCH) return dispatch_a<EPI, A_PATCH, DT>(a, W, M, N, K, ep, s);
  return dispatch_a<EPI, A_PLAIN, DT>(a, W, M, N, K, ep, s);
}

template <typename DT>
hipError_t dispatch_epi(int epi, int asrc, const ALoad& a, const void* W, int M, int N, int K,
                        const EpiParams& ep, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS_F32: return dispatch_src<EPI_BIAS_F32, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_BIAS_SILU: return dispatch_src<EPI_BIAS_SILU, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_COND: return dispatch_src<EPI_COND, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_BIAS_DT: return dispatch_src<EPI_BIAS_DT, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_GATED: return dispatch_src<EPI_GATED, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_GELU: return dispatch_src<EPI_GELU, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_PATCH: return dispatch_src<EPI_PATCH, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_ATOMIC_F32: return dispatch_src<EPI_ATOMIC_F32, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_GELU2: return dispatch_src<EPI_GELU2, DT>(asrc, a, W, M, N, K, ep, s);
    case EPI_DGELU: return dispatch_src<EPI_DGELU, DT>(asrc, a, W, M, N, K, ep, s);
  }
  return hipErrorInvalidValue;
}

// Products of at most GV_ROWS fp32 rows with bf16 weights, bias epilogue (the
// pooled-vector projection of one to a few rows): the 64 x 64 tile kernel
// would run N / 64 workgroups, each reading its weight rows 32 bytes at a time
// for one useful row.  Here one wave owns one output column: its lanes read the
// column's weight row 16 bytes at a time (lane l takes k = 8 l .. 8 l + 7 of
// every 512) with the matching A values, accumulate in fp32, and combine their
// partial sums by a fixed xor-shuffle tree, so the result is deterministic.
constexpr int GV_ROWS = 8;

template <int MR>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(ALoad a, const bf16_t* __restrict__ W,
                                                        int M, int N, int K, EpiParams ep) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int64_t ldw = ep.ldw ? ep.ldw : K;
  const bf16_t* wr = W + (int64_t)n * ldw;
  const float* arow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m)
    arow[m] = (const float*)a.ptr + row_map(min(m, M - 1) % a.src_rows, a.seg, a.skip, a.off) * a.lda;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  for (int k0 = 8 * lane; k0 < K; k0 += 512) {
    const uint4 wv = *(const uint4*)(wr + k0);
    const uint32_t wp[4] = {wv.x, wv.y, wv.z, wv.w};
    float w[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = __uint_as_float(wp[i] << 16);
      w[2 * i + 1] = __uint_as_float(wp[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float4 a0 = *(const float4*)(arow[m] + k0), a1 = *(const float4*)(arow[m] + k0 + 4);
      acc[m] = fmaf(a0.x, w[0], acc[m]);
      acc[m] = fmaf(a0.y, w[1], acc[m]);
      acc[m] = fmaf(a0.z, w[2], acc[m]);
      acc[m] = fmaf(a0.w, w[3], acc[m]);
      acc[m] = fmaf(a1.x, w[4], acc[m]);
      acc[m] = fmaf(a1.y, w[5], acc[m]);
      acc[m] = fmaf(a1.z, w[6], acc[m]);
      acc[m] = fmaf(a1.w, w[7], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = acc[m];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0 && m < M) epi_apply<EPI_BIAS_F32, bf16_t>(ep, m, n, v);
  }
}

template <int MR>
hipError_t run_gemv(const ALoad& a, const void* W, int M, int N, int K, const EpiParams& ep,
                    hipStream_t s) {
  gemv_bf16_kernel<MR><<<(N + 3) / 4, 256, 0, s>>>(a, (const bf16_t*)W, M, N, K, ep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_valu(int epi, int asrc, const ALoad& a, const void* W, int w_dtype,
                            int M, int N, int K, const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (ep.ksplit < 0 || (ep.ksplit % BK) || (ep.ksplit && epi != EPI_ATOMIC_F32) ||
      (epi == EPI_ATOMIC_F32 && ep.bias))
    return hipErrorInvalidValue;
  const int64_t ldw = ep.ldw ? ep.ldw : K;
  if (epi == EPI_BIAS_F32 && asrc == A_PLAIN && w_dtype == 1 && a.a_dtype == 0 && !a.trans &&
      !ep.w_trans && !ep.ksplit && M <= GV_ROWS && K % 8 == 0 && ldw % 8 == 0 && a.lda % 4 == 0 &&
      ((uintptr_t)W & 15) == 0 && ((uintptr_t)a.ptr & 15) == 0) {
    if (M <= 1) return run_gemv<1>(a, W, M, N, K, ep, s);
    if (M <= 2) return run_gemv<2>(a, W, M, N, K, ep, s);
    if (M <= 4) return run_gemv<4>(a, W, M, N, K, ep, s);
    return run_gemv<8>(a, W, M, N, K, ep, s);
  }
  if (w_dtype == 1) return dispatch_epi<bf16_t>(epi, asrc, a, W, M, N, K, ep, s);
  return dispatch_epi<float>(epi, asrc, a, W, M, N, K, ep, s);
}
