// bf16 GEMM C = A W^T on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation, fused epilogues.
//
// A [M, K] (row stride lda) and W [N, K] are both K-contiguous (row-major
// activations, [out, in] weights).  A BM x BN block tile is split over 4 waves
// (2 x 2); each wave owns (BM/2) x (BN/2) outputs as 32x32 MFMA blocks.
//
// K is consumed in 64-wide slices through a ring of STAGES LDS buffers filled
// by direct global->LDS loads (global_load_lds_dwordx4: each lane moves 16 bytes
// straight into LDS at base + 16*lane), so the next STAGES-1 slices are in
// flight while the current one feeds the MFMAs and no registers stage the
// copy.  LDS rows are 128 B (64 bf16); the 16-byte chunk c of row r sits at
// chunk c ^ ((r >> 1) & 7), which spreads the rows of one MFMA operand fetch
// over all 64 banks; each lane therefore fetches the global chunk that belongs
// in its LDS slot.  Rows past M or N read a clamped (valid) row and are never stored.
// Within a slice the operand fragments of the next 16-wide k step are read
// from LDS while the current step's MFMAs run.
#include <type_traits>

#include "common.h"
#include "epilogue.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((address_space(3))) void lds_void;

namespace {

constexpr int KSTEP = 64;   // K must be a multiple of this (every slice width used divides it)

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `left` slices of this wave's copies are in flight
// (left < STAGES - 1; each slice is L copies).
template <int L, int STAGES>
__device__ __forceinline__ void wait_slices(int left) {
  if constexpr (STAGES >= 4) {
    if (left >= 2) { wait_vmcnt<2 * L>(); return; }
  }
  if constexpr (STAGES >= 3) {
    if (left >= 1) { wait_vmcnt<L>(); return; }
  }
  wait_vmcnt<0>();
}

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs (each with
// its own L2): with SWZ, workgroup b runs logical tile (b % 8) * (n / 8) + b / 8,
// so each XCD walks a contiguous range of logical tiles, and logical tiles are
// ordered in groups of G row-tiles (column-major inside a group) so the tiles
// resident on one XCD at a time share A and W tiles.  Needs n % 8 == 0.
template <int SWZ>
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  if constexpr (SWZ) {
    const int n = tiles_m * tiles_n;
    const int logical = (b & 7) * (n >> 3) + (b >> 3);
    constexpr int G = 8;
    const int per_group = G * tiles_n;
    const int grp = logical / per_group, in = logical - grp * per_group;
    const int rows = min(G, tiles_m - grp * G);
    tm = grp * G + in % rows;
    tn = in / rows;
  } else {
    tm = b / tiles_n;
    tn = b - tm * tiles_n;
  }
}

// LDS rows are BK bf16 = BK/8 chunks of 16 B; chunk c of row r is stored at
// c ^ key(r).  The key makes the 16 rows read together by one 16-lane phase of
// ds_read_b128 (64 four-byte banks = 256 B per phase) land on distinct banks:
// BK = 64 (128-B rows, rows alternate bank halves): key = (r >> 1) & 7;
// BK = 32 (64-B rows, rows cycle through bank quarters): key = (r >> 2) & 3.
template <int BK>
__device__ __forceinline__ int row_key(int r) {
  if constexpr (BK == 64) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// s_waitcnt with only the LDS/scalar counter constrained to 0.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

template <int EPI, int BM, int BN, int BK, int STAGES, int MINWG, int SWZ, int FP = 0>
__global__ __launch_bounds__(256, MINWG) void gemm_bf16_kernel(const bf16_t* __restrict__ A, int lda,
                                                                const bf16_t* __restrict__ W, int M,
                                                                int N, int K, EpiParams ep) {
  static_assert(BK == 32 || BK == 64, "slice width");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  constexpr int CPR = BK / 8;                    // 16-byte chunks per LDS row
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NA = BM * CPR / 256, NB = BN * CPR / 256;   // 1 KB copies per wave per slice
  constexpr int L = NA + NB;
  constexpr int ROWB = BK * 2;                   // LDS row bytes
  constexpr int A_BYTES = BM * ROWB, STAGE_BYTES = (BM + BN) * ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  tile_coords<SWZ>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Per-lane source of each direct LDS copy: slot s of the tile is row s / CPR,
  // stored chunk s % CPR = logical chunk (s % CPR) ^ key(row).
  const bf16_t* pa[NA];
  const bf16_t* pb[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    int s = (w * NA + i) * 64 + lane, r = s / CPR, c = (s % CPR) ^ row_key<BK>(r);
    int m = min(m0 + r, M - 1);
    pa[i] = A + (int64_t)m * lda + c * 8;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    int s = (w * NB + i) * 64 + lane, r = s / CPR, c = (s % CPR) ^ row_key<BK>(r);
    int n = min(n0 + r, N - 1);
    pb[i] = W + (int64_t)n * K + c * 8;
  }
  auto issue = [&](int kt) {
    char* st = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(pa[i] + kt * BK),
                                       (lds_void*)(st + (w * NA + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(pb[i] + kt * BK),
                                       (lds_void*)(st + A_BYTES + (w * NB + i) * 1024), 16, 0, 0);
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // LDS byte offsets of this lane's operand rows (fixed over the loop); every
  // fragment row is a multiple of 32 plus (lane & 31), so its key depends on
  // the lane only.
  int offa[TM], offb[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) offa[i] = (wm * WM + i * 32 + (lane & 31)) * ROWB;
#pragma unroll
  for (int j = 0; j < TN; ++j) offb[j] = A_BYTES + (wn * WN + j * 32 + (lane & 31)) * ROWB;
  const int key = row_key<BK>(lane & 31);
  const int half = lane >> 5;

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);

  if constexpr (FP == 0) {
    for (int kt = 0; kt < nk; ++kt) {
      // Slice kt has landed in LDS once this wave's copies of it are done (later
      // slices may stay in flight) and every wave has passed the barrier.  A bare
      // s_barrier is used: __syncthreads() would add a release fence that drains
      // all outstanding copies.  The stage refilled below was last read in
      // iteration kt-1; those LDS reads completed before their MFMAs, which each
      // wave issued before reaching this barrier.
      wait_slices<L, STAGES>(min(STAGES - 2, nk - 1 - kt));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
      const char* st = smem + (kt % STAGES) * STAGE_BYTES;

      bf16x8_t fa[2][TM], fb[2][TN];
      auto fetch = [&](int buf, int kk) {
        const int ch = ((kk * 2 + half) ^ key) << 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[buf][i] = *(const bf16x8_t*)(st + offa[i] + ch);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[buf][j] = *(const bf16x8_t*)(st + offb[j] + ch);
      };
      fetch(0, 0);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        if (kk + 1 < BK / 16) fetch((kk + 1) & 1, kk + 1);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j],
                                                                acc[i][j], 0, 0, 0);
      }
    }
  } else {
    // Slice-ahead operand prefetch: iteration kt reads all fragments of slice
    // kt+1 from LDS while the MFMAs of slice kt run on fragments read one
    // iteration earlier.  Needs STAGES >= 3: the stage refilled in iteration kt
    // holds slice kt-1, whose fragments every wave finished reading (and waited
    // for) before this iteration's barrier.
    static_assert(STAGES >= 3, "slice-ahead prefetch needs 3 stages");
    constexpr int KK = BK / 16;
    bf16x8_t fa[2][KK][TM], fb[2][KK][TN];
    auto fetch_slice = [&](int buf, int kt) {
      const char* st = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int ch = ((kk * 2 + half) ^ key) << 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[buf][kk][i] = *(const bf16x8_t*)(st + offa[i] + ch);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[buf][kk][j] = *(const bf16x8_t*)(st + offb[j] + ch);
      }
    };
    wait_slices<L, STAGES>(min(STAGES - 2, nk - 1));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    fetch_slice(0, 0);
    // One step per slice; the register buffer index must be a compile-time
    // constant (a runtime index would turn the fragment arrays into memory), so
    // the loop runs two slices per trip with the buffers swapped.
    auto step = [&](auto cur_c, int kt) {
      constexpr int cur = decltype(cur_c)::value;
      if (kt + 1 < nk) {
        // the fragments of slice kt are in registers; slice kt+1 must be in LDS
        wait_lgkm0();
        wait_slices<L, STAGES>(min(STAGES - 3, nk - 2 - kt));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
        fetch_slice(cur ^ 1, kt + 1);
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][kk][i], fb[cur][kk][j],
                                                                acc[i][j], 0, 0, 0);
    };
    for (int kt = 0; kt < nk; kt += 2) {
      step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
    }
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane % 32);
  // register r holds row 8*(r/4) + 4*(lane/32) + (r % 4).  Per-column values
  // (bias, and the gate when the tile lies in one batch row) are loaded once.
  const int col0 = n0 + wn * WN + (lane & 31);
  const int row0 = m0 + wm * WM + 4 * half;
  float bcol[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int col = col0 + j * 32;
    bcol[j] = (ep.bias && col < N) ? ep.bias[col] : 0.0f;
  }
  if constexpr (EPI == EPI_GATED) {
    const int mlast = min(m0 + BM, M) - 1;
    const bool one_b = (m0 / ep.T) == (mlast / ep.T);
    float gcol[TN];
    if (one_b) {
      const float* g = ep.mod + (int64_t)(m0 / ep.T) * ep.mod_stride + ep.gate_off;
#pragma unroll
      for (int j = 0; j < TN; ++j) gcol[j] = (col0 + j * 32 < N) ? g[col0 + j * 32] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= M) continue;
        float* xr = (float*)ep.out + (int64_t)row * ep.ldo;
        const float* g = ep.mod + (int64_t)(row / ep.T) * ep.mod_stride + ep.gate_off;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = col0 + j * 32;
          if (col < N) {
            const float gv = one_b ? gcol[j] : g[col];
            xr[col] = xr[col] + gv * (acc[i][j][r] + bcol[j]);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = col0 + j * 32;
          if (col >= N) continue;
          float v = acc[i][j][r] + bcol[j];
          const int64_t o = (int64_t)row * ep.ldo + col;
          if constexpr (EPI == EPI_BIAS_F32) ((float*)ep.out)[o] = v;
          else if constexpr (EPI == EPI_BIAS_DT) ((bf16_t*)ep.out)[o] = f2bf(v);
          else if constexpr (EPI == EPI_GELU) ((bf16_t*)ep.out)[o] = f2bf(gelu_tanh_f(v));
          else static_assert(EPI == EPI_BIAS_F32, "epilogue");
        }
      }
  }
}

template <int EPI, int BM, int BN, int BK, int STAGES, int MINWG>
hipError_t run(const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
               const EpiParams& ep, hipStream_t s) {
  int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles % 8 == 0)
    gemm_bf16_kernel<EPI, BM, BN, BK, STAGES, MINWG, 1><<<tiles, 256, 0, s>>>(A, lda, W, M, N, K, ep);
  else
    gemm_bf16_kernel<EPI, BM, BN, BK, STAGES, MINWG, 0><<<tiles, 256, 0, s>>>(A, lda, W, M, N, K, ep);
  return hipGetLastError();
}

template <int EPI>
hipError_t pick(const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
                const EpiParams& ep, hipStream_t s) {
  // 128x192 tiles, 32-wide K slices, 2 LDS stages (40 KB): three workgroups fit
  // on a CU, and M = 16384 with N in {1152, 3456, 4608} gives 1, 3 and 4 full
  // rounds of 768 resident workgroups on 256 CUs.
  if (N % 192 == 0) return run<EPI, 128, 192, 32, 2, 3>(A, lda, W, M, N, K, ep, s);
  return run<EPI, 128, 128, 32, 2, 3>(A, lda, W, M, N, K, ep, s);
}

}  // namespace

hipError_t launch_gemm_mfma(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N,
                            int K, const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % KSTEP || lda % 8) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_BIAS_F32: return pick<EPI_BIAS_F32>(A, lda, W, M, N, K, ep, s);
    case EPI_BIAS_DT: return pick<EPI_BIAS_DT>(A, lda, W, M, N, K, ep, s);
    case EPI_GATED: return pick<EPI_GATED>(A, lda, W, M, N, K, ep, s);
    case EPI_GELU: return pick<EPI_GELU>(A, lda, W, M, N, K, ep, s);
  }
  return hipErrorInvalidValue;
}
