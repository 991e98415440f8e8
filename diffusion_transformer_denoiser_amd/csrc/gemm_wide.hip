// Wide-tile bf16 GEMM C = A W^T for the large products of the adaLN-Zero
// blocks (q | k | v in-projection, output projection, FFN up and down
// projections; itwiki "확산 트랜스포머", Implementation / adaLN-Zero block),
// on the CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation,
// fused epilogues.
//
// A [M, K] (row stride lda) and W [N, K] (row stride ldw) are K-contiguous.
// One workgroup of 8 waves owns a 256 x BN output tile (BN = 288 or 256), one
// workgroup per CU; the waves form a 4 x 2 grid of 64 x BN/2 wave tiles, i.e.
// 4 x BN/32 blocks of 16 x 16 per wave.  A 256 x 288 tile moves
// (256 + 288) x 2 bytes per k over 256 x 288 x 2 FLOP: 7.4 mB per FLOP, 43%
// less global->LDS traffic than a 128 x 192 tile, and at M = 16384 the four
// block products (N = 3456, 1152, 4608, 1152) fill whole waves of 256 tiles.
//
// K is consumed in 64-wide slices through two LDS stages filled by
// buffer->LDS copies (each lane moves 16 bytes straight into LDS at
// base + 16 * lane).  An LDS row holds 64 bf16 of one operand row; 16-byte
// chunk c of row r sits at chunk c ^ ((r >> 1) & 7), which puts the 16 rows
// one ds_read_b128 phase reads on distinct banks.  Each lane therefore copies
// the global chunk that belongs in its LDS slot.  Rows past M read row M - 1
// and are never stored.
//
// Schedule per slice: two 32-wide k steps of 4 x BN/32 MFMAs each, column
// block by column block.  The B fragment of column block j + 2 is read while
// block j's MFMAs run (a ring of fragments), the A fragments of the next k
// step during the current one.  The one barrier per slice follows the last
// LDS read of the slice; after it the first fragments of the next slice are
// read and the copies of slice kt + 2 refill the stage of slice kt, spread
// over the MFMAs that remain.
#include <type_traits>

#include "common.h"
#include "mfma_util.h"


namespace {

constexpr int WBM = 256;   // tile rows
constexpr int WBK = 64;    // K slice
constexpr int kWideSlots = 256;   // resident workgroups: one per CU of the MI355X

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs (each
// with its own L2): XCD x = b % 8 runs workgroups b = x, x + 8, ..., and takes
// one contiguous range of logical tiles, walked in groups of 8 row tiles
// (column-major inside a group), so the tiles resident on one XCD at a time
// share A row tiles and W column tiles.
__device__ __forceinline__ void wide_tile(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int n = tiles_m * tiles_n;
  const int q = n >> 3, r = n & 7, x = b & 7;
  const int logical = x * q + min(x, r) + (b >> 3);
  constexpr int G = 8;
  const int per_group = G * tiles_n;
  const int grp = logical / per_group, in = logical - grp * per_group;
  const int rows = min(G, tiles_m - grp * G);
  tm = grp * G + in % rows;
  tn = in / rows;
}

__device__ __forceinline__ float dpp_swap_pair(float v) {
  // quad_perm [1, 0, 3, 2]: the value of the neighbouring lane
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <int EPI, int BN>
__global__ __launch_bounds__(512) void gemm_wide_kernel(const bf16_t* __restrict__ A, int lda,
                                                        const bf16_t* __restrict__ W, int M,
                                                        int N, int K, EpiParams ep) {
  constexpr int BM = WBM, BK = WBK, ROWB = BK * 2;
  constexpr int WN = BN / 2, NJ = WN / 16, NI = 4;
  constexpr int ROWS = BM + BN, STAGE = ROWS * ROWB;
  constexpr int NCOPY = ROWS / 8;       // 1 KB copies (8 LDS rows each) per stage
  constexpr int CPW = (NCOPY + 7) / 8;  // copies per wave (the last one on the first waves only)
  constexpr int NA = BM / 64;           // the first NA copies of every wave are A rows
  constexpr int RING = (2 * NJ) % 3 == 0 ? 3 : 4;   // B fragments in flight (divides 2 NJ)
  static_assert(BN % 32 == 0 && (2 * NJ) % RING == 0, "tile width");
  static_assert(2 * STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int c16 = lane & 15, g = lane >> 4;
  const int tiles_n = N / BN, tiles_m = (M + BM - 1) / BM, ntiles = tiles_m * tiles_n;
  const int64_t ldw = ep.ldw ? ep.ldw : K;
  const int nk = K / BK;

  // Copy u of this wave fills LDS rows 8 (w + 8 u) .. + 7 of a stage; lane l
  // fills row 8 (w + 8 u) + l / 8, stored chunk l % 8.
  int voff[CPW];
  auto set_tile = [&](int m0, int n0) {
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int c = min(w + 8 * u, NCOPY - 1);
      const int r = c * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ ((r >> 1) & 7);
      if (u < NA)
        voff[u] = (int)(((int64_t)min(m0 + r, M - 1) * lda + lc * 8) * 2);
      else
        voff[u] = (int)(((int64_t)(n0 + r - BM) * ldw + lc * 8) * 2);
    }
  };
  const bool full_copies = w + 8 * (CPW - 1) < NCOPY;   // this wave issues CPW copies per slice
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, (short)0, (int)(((int64_t)(M - 1) * lda + K) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)W, (short)0, (int)(((int64_t)(N - 1) * ldw + K) * 2), 0x00020000);
  auto copy = [&](int kt, int u) {
    if (u < CPW - 1 || full_copies) {
      char* dst = smem + (kt & 1) * STAGE + (w + 8 * u) * 1024;
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(u < NA ? ars : wrs, (lds_void*)dst, 16, voff[u],
                                               kt * ROWB, 0, 0);
#endif
    }
  };
  auto copies = [&](int kt) {
#pragma unroll
    for (int u = 0; u < CPW; ++u) copy(kt, u);
  };

  // Fragment reads: lane l supplies row (or column) l % 16 of a 16-row block,
  // k = 8 (l / 16) .. + 7 of the 32-wide step, i.e. logical chunk 4 s + l / 16
  // of the LDS row; the row's key depends on l % 16 only.
  const int key = (c16 >> 1) & 7;
  const int xs0 = ((0 + g) ^ key) << 4, xs1 = ((4 + g) ^ key) << 4;
  const int arow = (wm * 64 + c16) * ROWB, brow = (BM + wn * WN + c16) * ROWB;
  auto rdA = [&](int kt, int s, int i) {
    return *(const bf16x8_t*)(smem + (kt & 1) * STAGE + arow + i * 16 * ROWB + (s ? xs1 : xs0));
  };
  auto rdB = [&](int kt, int s, int j) {
    return *(const bf16x8_t*)(smem + (kt & 1) * STAGE + brow + j * 16 * ROWB + (s ? xs1 : xs0));
  };

  // Persistent: workgroup b runs tiles b, b + gridDim.x, ...; the first two
  // slices of the next tile are copied while the current tile's epilogue runs.
  int t = blockIdx.x;
  if (t >= ntiles) return;
  int tm, tn;
  wide_tile(t, tiles_m, tiles_n, tm, tn);
  int m0 = tm * BM, n0 = tn * BN;
  set_tile(m0, n0);
  copies(0);
  if (nk > 1) copies(1);
  bool relaxed = false;
  static_assert(2 * NI * NJ + CPW >= 63, "every whole-tile epilogue issues >= 63 - CPW memory ops");

  for (;;) {
    // Accumulators start at the bias.  acc[i][j][r] is output row
    // m0 + 64 wm + 16 i + 4 g + r, column n0 + WN wn + 16 j + c16.
    floatx4 acc[NI][NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float b = ep.bias ? ep.bias[n0 + wn * WN + 16 * j + c16] : 0.0f;
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[i][j] = floatx4{b, b, b, b};
    }
    // Slice 0 has landed once at most the ops issued after its copies are
    // outstanding: slice 1's copies and, after an epilogue of a whole tile
    // (at least 63 - CPW stores or loads, issued after the copies), up to 63
    // (the counter's limit), so the epilogue's stores keep draining.
    if (nk == 1) wait_vmcnt<0>();
    else if (relaxed) wait_vmcnt<63>();
    else if (full_copies) wait_vmcnt<CPW>();
    else wait_vmcnt<CPW - 1>();
    bare_barrier();
    bf16x8_t af[2][NI];
    bf16x8_t bfr[RING];
#pragma unroll
    for (int i = 0; i < NI; ++i) af[0][i] = rdA(0, 0, i);
    bfr[0] = rdB(0, 0, 0);
    bfr[1] = rdB(0, 0, 1);

    // One slice; MORE: slice kt + 1 exists, DMA: slice kt + 2 exists.  The
    // MFMA slots after the barrier (step 1, block NJ - 2, i = 1) carry the
    // next slice's first fragment reads and the copies of slice kt + 2.
    auto slice = [&](int kt, auto more_c, auto dma_c) {
      constexpr bool MORE = decltype(more_c)::value, DMA = decltype(dma_c)::value;
      constexpr int AFTER = 2 + NI;   // (NJ - 2, 2), (NJ - 2, 3), (NJ - 1, 0..3)
      constexpr int PER = (CPW + AFTER - 1) / AFTER;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int bq = s * NJ + j;
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][i], bfr[bq % RING],
                                                                acc[i][j], 0, 0, 0);
            if (i == 0 && bq + 2 < 2 * NJ) {
              const int nq = bq + 2;
              bfr[nq % RING] = rdB(kt, nq / NJ, nq % NJ);
            }
            if (s == 0 && i == 2 && j < NI) af[1][j] = rdA(kt, 1, j);
            if constexpr (MORE) {
              if (s == 1 && j == NJ - 2 && i == 1) {
                // every read of this slice has returned; slice kt + 1 has landed
                // once this wave's copies of it are done and all waves pass
                wait_lgkm0();
                wait_vmcnt<0>();
                bare_barrier();
              }
              if (s == 1 && (j == NJ - 2 && i >= 2 || j == NJ - 1)) {
                const int slot = j == NJ - 2 ? i - 2 : 2 + i;   // 0 .. AFTER - 1
                if (slot < NI) af[0][slot] = rdA(kt + 1, 0, slot);
                if (slot == 1) bfr[0] = rdB(kt + 1, 0, 0);
                if (slot == 3) bfr[1] = rdB(kt + 1, 0, 1);
                if constexpr (DMA) {
#pragma unroll
                  for (int v = 0; v < PER; ++v)
                    if (slot * PER + v < CPW) copy(kt + 2, slot * PER + v);
                }
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    int kt = 0;
    for (; kt + 2 < nk; ++kt) slice(kt, T_{}, T_{});
    if (kt + 1 < nk) slice(kt++, T_{}, F_{});
    slice(kt, F_{}, F_{});

    // The next tile's first two slices are copied while this tile's epilogue
    // runs (after a barrier: every wave has finished reading the stages).
    const int tnext = t + gridDim.x;
    const bool more_tiles = tnext < ntiles;
    const int em0 = m0, en0 = n0;
    if (more_tiles) {
      wide_tile(tnext, tiles_m, tiles_n, tm, tn);
      m0 = tm * BM;
      n0 = tn * BN;
      wait_lgkm0();
      bare_barrier();
      set_tile(m0, n0);
      copies(0);
      if (nk > 1) copies(1);
    }

    // Epilogues.
    const int rbase = em0 + wm * 64 + 4 * g;        // + 16 i + r
    const int cbase = en0 + wn * WN + c16;          // + 16 j
    const bool full = em0 + BM <= M;
    if constexpr (EPI == EPI_BIAS_DT || EPI == EPI_GELU) {
      // bf16 column pairs: lanes c16 and c16 ^ 1 trade two values each, so the
      // even lane stores rows 0 and 2 of the pair of columns, the odd lane
      // rows 1 and 3, as 4-byte words.
      bf16_t* out = (bf16_t*)ep.out;
      const bool even = (c16 & 1) == 0;
      const int col0 = en0 + wn * WN + (c16 & ~1);
      const int rodd = even ? 0 : 1;
      auto value = [&](int i, int j, int r) {
        const float x = acc[i][j][r];
        if constexpr (EPI == EPI_GELU) return gelu_tanh_f(x);
        else return x;
      };
      if (full && (int64_t)M * ep.ldo * 2 < (1LL << 31)) {
        // Whole tile: each lane packs its own rows (0, 1) and (2, 3) to bf16
        // pairs, takes the neighbour's pairs by one DPP move each and keeps
        // one half of each with a byte permute (even lane: own low half, then
        // the neighbour's low half; odd lane: the neighbour's high half, then
        // its own).  Stores through buffer addressing: one lane offset, the
        // row offsets in scalar registers, the column block as the immediate.
        const int ldb = ep.ldo * 2;
        const __amdgpu_buffer_rsrc_t ors =
            __builtin_amdgcn_make_buffer_rsrc(out, (short)0, M * ldb, 0x00020000);
        const int oo = (rbase + rodd) * ldb + col0 * 2;
        const uint32_t sel = even ? 0x05040100u : 0x03020706u;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const uint32_t p01 = f2bf2(value(i, j, 0), value(i, j, 1));
            const uint32_t p23 = f2bf2(value(i, j, 2), value(i, j, 3));
            const uint32_t q01 =
                (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p01, 0xB1, 0xF, 0xF, false);
            const uint32_t q23 =
                (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p23, 0xB1, 0xF, 0xF, false);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_amdgcn_perm(q01, p01, sel), ors,
                                                  oo + 32 * j, (16 * i) * ldb, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_amdgcn_perm(q23, p23, sel), ors,
                                                  oo + 32 * j, (16 * i + 2) * ldb, 0);
          }
      } else {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v[r] = acc[i][j][r];
            if constexpr (EPI == EPI_GELU) v[r] = gelu_tanh_f(v[r]);
          }
          const float r0 = dpp_swap_pair(even ? v[1] : v[0]);
          const float r1 = dpp_swap_pair(even ? v[3] : v[2]);
          const uint32_t w0 = even ? f2bf2(v[0], r0) : f2bf2(r0, v[1]);
          const uint32_t w1 = even ? f2bf2(v[2], r1) : f2bf2(r1, v[3]);
          const int row = rbase + 16 * i + rodd;
          bf16_t* o = out + (int64_t)row * ep.ldo + col0 + 16 * j;
          if (full || row < M) *(uint32_t*)o = w0;
          if (full || row + 2 < M) *(uint32_t*)(o + 2 * (int64_t)ep.ldo) = w1;
        }
      }
    } else if constexpr (EPI == EPI_BIAS_F32) {
      float* out = (float*)ep.out;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + 16 * i + r;
          if (!full && row >= M) continue;
#pragma unroll
          for (int j = 0; j < NJ; ++j) out[(int64_t)row * ep.ldo + cbase + 16 * j] = acc[i][j][r];
        }
    } else {
      static_assert(EPI == EPI_GATED, "epilogue");
      // X += gate * C, in place on the fp32 residual.  Each 16-row block lies in
      // one batch row (T % 16 == 0).  One column block at a time, the next
      // block's residual values loaded before the current block is stored.
      float* X = (float*)ep.out;
      if (full) {
        // Buffer addressing: one lane offset, the row offsets of (i, r) in
        // scalar registers, the column block as the immediate.  Three column
        // blocks of residual and gate loads are in flight; block j is stored
        // before the loads of block j + 3 are issued.  Without a gate the
        // loads read X and the gate is 1.
        constexpr int D = 3;
        const int ldb = ep.ldo * 4;
        const __amdgpu_buffer_rsrc_t xrs =
            __builtin_amdgcn_make_buffer_rsrc(X, (short)0, M * ldb, 0x00020000);
        const int xo = rbase * ldb + cbase * 4;
        const bool gated = ep.mod != nullptr;
        const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
            gated ? (void*)ep.mod : (void*)X, (short)0,
            gated ? ((M - 1) / ep.T + 1) * ep.mod_stride * 4 : M * ldb, 0x00020000);
        const int go = gated ? (ep.gate_off + cbase) * 4 : xo;
        // scalar offsets: the wave index is uniform, which the compiler cannot see
        const int wrow = __builtin_amdgcn_readfirstlane(em0 + wm * 64);
        int gso[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
          gso[i] = gated ? (min(wrow + 16 * i, M - 1) / ep.T) * ep.mod_stride * 4 : 0;
        // the gate word is masked rather than selected, so that the loads stay
        // unconditional and in issue order (no branch around them)
        const uint32_t gmask = gated ? ~0u : 0u, gone = gated ? 0u : 0x3F800000u;
        float xv[D][NI][4];
        uint32_t gv[D][NI];
        auto load = [&](int j) {
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            gv[j % D][i] = __builtin_amdgcn_raw_buffer_load_b32(grs, go + 64 * j, gso[i], 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              xv[j % D][i][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                  xrs, xo + 64 * j, (16 * i + r) * ldb, 0));
          }
          __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll
        for (int j = 0; j < D; ++j) load(j);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const float gt = __uint_as_float((gv[j % D][i] & gmask) | gone);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              __builtin_amdgcn_raw_buffer_store_b32(
                  __float_as_uint(__builtin_fmaf(gt, acc[i][j][r], xv[j % D][i][r])), xrs,
                  xo + 64 * j, (16 * i + r) * ldb, 0);
          }
          if (j + D < NJ) load(j + D);
        }
      } else {
        const float* gp[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int brow = min(rbase - 4 * g + 16 * i, M - 1) / ep.T;
          gp[i] = ep.mod ? ep.mod + (int64_t)brow * ep.mod_stride + ep.gate_off + cbase : nullptr;
        }
        auto xaddr = [&](int i, int r, int j) {
          return X + (int64_t)(rbase + 16 * i + r) * ep.ldo + cbase + 16 * j;
        };
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (rbase + 16 * i + r >= M) continue;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              float* p = xaddr(i, r, j);
              *p = *p + (gp[i] ? gp[i][16 * j] : 1.0f) * acc[i][j][r];
            }
          }
      }
    }
    if (!more_tiles) break;
    t = tnext;
    relaxed = full;
    // recompute the copy offsets here rather than keeping them live through
    // the epilogue (the register file is the binding limit)
    asm volatile("" : "+s"(m0), "+s"(n0));
    set_tile(m0, n0);
  }
}

template <int EPI, int BN>
hipError_t run_wide(const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
                    const EpiParams& ep, hipStream_t s) {
  const int tiles = ((M + WBM - 1) / WBM) * (N / BN);
  // one workgroup per CU (the LDS stages take 128-136 KB), persistent
  const int grid = tiles < kWideSlots ? tiles : kWideSlots;
  gemm_wide_kernel<EPI, BN><<<grid, 512, 0, s>>>(A, lda, W, M, N, K, ep);
  return hipGetLastError();
}

template <int BN>
hipError_t pick_wide(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
                     const EpiParams& ep, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS_DT: return run_wide<EPI_BIAS_DT, BN>(A, lda, W, M, N, K, ep, s);
    case EPI_GELU: return run_wide<EPI_GELU, BN>(A, lda, W, M, N, K, ep, s);
    case EPI_GATED: return run_wide<EPI_GATED, BN>(A, lda, W, M, N, K, ep, s);
    case EPI_BIAS_F32: return run_wide<EPI_BIAS_F32, BN>(A, lda, W, M, N, K, ep, s);
  }
  return hipErrorNotSupported;
}

}  // namespace

bool gemm_wide_supported(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
                         const EpiParams& ep) {
  if (epi != EPI_BIAS_DT && epi != EPI_GELU && epi != EPI_GATED && epi != EPI_BIAS_F32)
    return false;
  if (M < WBM || K <= 0 || K % WBK || lda % 8 || lda < K) return false;
  if (N % 288 && N % 256) return false;
  if (ep.ksplit || ep.a_seg || ep.o_seg || ep.tok_seg || ep.aux) return false;
  const int64_t ldw = ep.ldw ? ep.ldw : K;
  if (ldw % 8 || ldw < K) return false;
  if (((uintptr_t)A & 15) || ((uintptr_t)W & 15)) return false;
  if (((int64_t)(M - 1) * lda + K) * 2 >= (1LL << 31) || ((int64_t)(N - 1) * ldw + K) * 2 >= (1LL << 31))
    return false;   // buffer descriptors with 32-bit byte offsets
  if ((epi == EPI_BIAS_DT || epi == EPI_GELU) && (((uintptr_t)ep.out & 3) || ep.ldo % 2))
    return false;   // bf16 outputs stored as 4-byte column pairs
  if (epi == EPI_GATED && ep.mod && (ep.T <= 0 || ep.T % 16)) return false;
  if (epi == EPI_GATED) {   // residual and gates through buffer descriptors
    if (ep.ldo < N || (int64_t)M * ep.ldo * 4 >= (1LL << 31)) return false;
    if (ep.mod && (int64_t)((M - 1) / ep.T + 1) * ep.mod_stride * 4 >= (1LL << 31)) return false;
  }
  return true;
}

hipError_t launch_gemm_wide(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N,
                            int K, const EpiParams& ep, hipStream_t s) {
  if (!gemm_wide_supported(epi, A, lda, W, M, N, K, ep)) return hipErrorNotSupported;
  if (N % 288 == 0) return pick_wide<288>(epi, A, lda, W, M, N, K, ep, s);
  return pick_wide<256>(epi, A, lda, W, M, N, K, ep, s);
}
