// bf16 GEMM C = A W^T on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation, fused epilogues.
//
// A [M, K] and W [N, K] are both K-contiguous (row-major activations,
// [out, in] weights).  A BM x BN block tile is split over 4 waves (2 x 2); each
// wave owns (BM/2) x (BN/2) outputs as 32x32 MFMA blocks.  K is staged through
// LDS in 64-wide slices, double-buffered: the next slice is fetched from HBM
// into registers while the current one feeds the MFMAs.  LDS rows are 128 B
// (64 bf16); the 16-byte chunk c of row r is stored at chunk c ^ (r & 7), so
// the 32 rows read by one MFMA operand fetch spread over all banks.
#include "common.h"
#include "epilogue.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

namespace {

constexpr int BK = 64;

template <int EPI, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(const bf16_t* __restrict__ A, int lda,
                                                         const bf16_t* __restrict__ W, int M,
                                                         int N, int K, EpiParams ep) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int CA = BM * BK / 8 / 256;  // 16-byte chunks per thread per slice
  constexpr int CB = BN * BK / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  uint4 ra[CA], rb[CB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int idx = tid + i * 256, row = idx >> 3, ch = idx & 7;
      int m = m0 + row;
      ra[i] = (m < M) ? *(const uint4*)(A + (int64_t)m * lda + k0 + ch * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      int idx = tid + i * 256, row = idx >> 3, ch = idx & 7;
      int n = n0 + row;
      rb[i] = (n < N) ? *(const uint4*)(W + (int64_t)n * K + k0 + ch * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int idx = tid + i * 256, row = idx >> 3, ch = idx & 7;
      *(uint4*)&sA[buf][row * BK + ((ch ^ (row & 7)) << 3)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      int idx = tid + i * 256, row = idx >> 3, ch = idx & 7;
      *(uint4*)&sB[buf][row * BK + ((ch ^ (row & 7)) << 3)] = rb[i];
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      // lane supplies row (lane % 32), k = kk*16 + 8*(lane/32) .. +8
      const int ch = kk * 2 + (lane >> 5);
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int row = wm * WM + i * 32 + (lane & 31);
        af[i] = *(const bf16x8_t*)&sA[buf][row * BK + ((ch ^ (row & 7)) << 3)];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int row = wn * WN + j * 32 + (lane & 31);
        bfr[j] = *(const bf16x8_t*)&sB[buf][row * BK + ((ch ^ (row & 7)) << 3)];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column (lane % 32); register r holds
  // row 8*(r/4) + 4*(lane/32) + (r % 4).
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        int col = n0 + wn * WN + j * 32 + (lane & 31);
        if (row < M && col < N) epi_apply<EPI, bf16_t>(ep, row, col, acc[i][j][r]);
      }
}

template <int EPI, int BM, int BN>
hipError_t run(const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
               const EpiParams& ep, hipStream_t s) {
  int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  gemm_mfma_kernel<EPI, BM, BN><<<tiles, 256, 0, s>>>(A, lda, W, M, N, K, ep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N,
                            int K, const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % BK) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_BIAS_F32: return run<EPI_BIAS_F32, 128, 128>(A, lda, W, M, N, K, ep, s);
    case EPI_QKV: return run<EPI_QKV, 128, 128>(A, lda, W, M, N, K, ep, s);
    case EPI_GATED: return run<EPI_GATED, 128, 128>(A, lda, W, M, N, K, ep, s);
    case EPI_GELU: return run<EPI_GELU, 128, 128>(A, lda, W, M, N, K, ep, s);
  }
  return hipErrorInvalidValue;
}
