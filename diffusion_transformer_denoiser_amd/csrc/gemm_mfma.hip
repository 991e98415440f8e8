// bf16 GEMM C = A W^T on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation, fused epilogues.
//
// A [M, K] (row stride lda) and W [N, K] are both K-contiguous (row-major
// activations, [out, in] weights).  A BM x BN block tile is split over 4 waves
// (2 x 2); each wave owns (BM/2) x (BN/2) outputs as 32x32 MFMA blocks, in
// which a lane holds one output column and 16 rows, so each store instruction
// of the epilogue covers whole 128-byte row segments.
//
// K is consumed in BK-wide slices through two LDS buffers filled by direct
// global->LDS loads (global_load_lds_dwordx4: each lane moves 16 bytes straight
// into LDS at base + 16*lane), so no registers stage the copy.  LDS rows are
// BK bf16; 16-byte chunk c of row r sits at chunk c ^ key(r), which spreads the
// rows of one operand fetch over all 64 banks; each lane therefore fetches the
// global chunk that belongs in its LDS slot.  Rows past M or N read a clamped
// (valid) row and are never stored.
//
// Schedule (one flat sequence of 16-wide k steps): the operand fragments of
// step s+1 are read from LDS while the MFMAs of step s run.  The one barrier
// per slice sits before the slice's last step: by then every fragment of the
// slice is in registers, so after it (a) the first fragments of the next slice
// can be read under the last step's MFMAs and (b) the copies of slice kt+2 can
// refill the buffer of slice kt, interleaved with those MFMAs.
#include <type_traits>

#include "common.h"
#include "mfma_util.h"

namespace {

constexpr int KSTEP = 64;   // K must be a multiple of this (every slice width used divides it)

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs (each with
// its own L2): with SWZ, XCD x = b % 8 runs workgroups b = x, x + 8, ..., and
// they take one contiguous range of logical tiles (the first n % 8 XCDs one
// tile more than the others), so each XCD walks its own range.  Logical tiles
// are ordered in groups of G row-tiles (column-major inside a group, the
// column index rotated per XCD) so the tiles resident on one XCD at a time
// share A and W tiles.
template <int SWZ>
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  if constexpr (SWZ) {
    const int n = tiles_m * tiles_n;
    const int q = n >> 3, r = n & 7, x = b & 7;
    const int logical = x * q + min(x, r) + (b >> 3);
    constexpr int G = 8;
    const int per_group = G * tiles_n;
    const int grp = logical / per_group, in = logical - grp * per_group;
    const int rows = min(G, tiles_m - grp * G);
    tm = grp * G + in % rows;
    // The column walk of a group starts 1/8 of the way further along for each
    // XCD (the XCD of the group's first tile, so all tiles of a group share
    // one rotation and the map stays one-to-one): at any moment the XCDs fetch
    // different W columns, so a weight tile comes from HBM once and later XCDs
    // find it in the Infinity Cache (-8% per launch when the weights are not
    // cached yet, as in a forward).
    const int l0 = grp * per_group;   // the group's first tile, and the XCD whose range holds it
    const int xg = l0 < r * (q + 1) ? l0 / (q + 1) : r + (l0 - r * (q + 1)) / max(q, 1);
    tn = (in / rows + (xg & 7) * tiles_n / 8) % tiles_n;
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

// vec: the output is 4-byte aligned with an even row stride (bf16 column pairs
// may be stored as words).  BUF: the copies address A and W through buffer
// descriptors (scalar base + 32-bit lane offset), which takes less of the
// address unit than 64-bit lane addresses; needs both operands under 2 GiB.
template <int EPI, int BM, int BN, int BK, int MINWG, int SWZ, int ILV, int BUF>
__global__ __launch_bounds__(256, MINWG) void gemm_bf16_kernel(const bf16_t* __restrict__ A, int lda,
                                                                const bf16_t* __restrict__ W, int M,
                                                                int N, int K, EpiParams ep, int vec) {
  static_assert(BK == 32 || BK == 64, "slice width");
  constexpr int CPR = BK / 8;                    // 16-byte chunks per LDS row
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NA = BM * CPR / 256, NB = BN * CPR / 256;   // 1 KB copies per wave per slice
  constexpr int L = NA + NB;
  constexpr int KK = BK / 16;                    // MFMA k steps per slice (even)
  constexpr int NF = TM + TN;                    // fragments per step
  constexpr int NMF = TM * TN;                   // MFMAs per step
  constexpr int ROWB = BK * 2;                   // LDS row bytes
  constexpr int A_BYTES = BM * ROWB, STAGE_BYTES = (BM + BN) * ROWB;
  static_assert((L + NMF - 1) / NMF <= 4, "interleave shape");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  tile_coords<SWZ>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int half = lane >> 5;
  const int64_t ldw = ep.ldw ? ep.ldw : K;
  if (gridDim.y > 1) {   // split-K: this grid layer's slice of the reduction
    const int kb = blockIdx.y * ep.ksplit;
    A += kb;
    W += kb;
    K = min(ep.ksplit, K - kb);
  }

  // Accumulators start at the bias.  acc[i][j][r] is output column
  // ncol + 32 j, row mrow + 32 i + 8 (r / 4) + (r % 4).
  const int ncol = n0 + wn * WN + (lane & 31);
  const int mrow = m0 + wm * WM + 4 * half;
  floatx16 acc[TM][TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = ncol + j * 32;
    const float b = ep.bias && blockIdx.y == 0 ? (col < N ? 1.0f : 0.0f) * ep.bias[min(col, N - 1)]
                                               : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = b;
  }

  // Per-lane source of each direct LDS copy: slot s of the tile is row s / CPR,
  // stored chunk s % CPR = logical chunk (s % CPR) ^ key(row).
  const bf16_t* src[L];
#pragma unroll
  for (int c = 0; c < L; ++c) {
    const bool is_a = c < NA;
    const int s = (w * (is_a ? NA : NB) + (is_a ? c : c - NA)) * 64 + lane;
    const int r = s / CPR, ch = (s % CPR) ^ row_key<BK>(r);
    src[c] = is_a ? A + row_map(min(m0 + r, M - 1), ep.a_seg, ep.a_skip, ep.a_off) * lda + ch * 8
                  : W + (int64_t)min(n0 + r, N - 1) * ldw + ch * 8;
  }
  int boff[L];
#pragma unroll
  for (int c = 0; c < L; ++c)
    boff[c] = (int)((const char*)src[c] - (c < NA ? (const char*)A : (const char*)W));
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, (short)0,
      (int)((row_map(M - 1, ep.a_seg, ep.a_skip, ep.a_off) * lda + K) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)(((int64_t)(N - 1) * ldw + K) * 2),
                                        0x00020000);
  auto copy = [&](int kt, int c) {
    char* st = smem + (kt & 1) * STAGE_BYTES +
               (c < NA ? (w * NA + c) * 1024 : A_BYTES + (w * NB + c - NA) * 1024);
    if constexpr (BUF) {
      // The buffer->LDS builtin exists only for the device; the host pass keeps
      // just the launch stub of this kernel.
#if defined(__HIP_DEVICE_COMPILE__)
      if (c < NA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)st, 16, boff[c], kt * BK * 2, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void*)st, 16, boff[c], kt * BK * 2, 0, 0);
#endif
    } else {
      __builtin_amdgcn_global_load_lds((const void*)(src[c] + kt * BK), (lds_void*)st, 16, 0, 0);
    }
  };

  // LDS byte offsets of this lane's operand rows (fixed over the loop); every
  // fragment row is a multiple of 32 plus (lane & 31), so its key depends on
  // the lane only.
  int off[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
    off[f] = f < TM ? (wm * WM + f * 32 + (lane & 31)) * ROWB
                    : A_BYTES + (wn * WN + (f - TM) * 32 + (lane & 31)) * ROWB;
  const int key = row_key<BK>(lane & 31);

  // Fragment slots are read in the order of their first use by the MFMAs of a
  // step (A0, B0 .. B(TN-1), A1 .. A(TM-1)), so each MFMA waits only for the
  // reads it needs.
  bf16x8_t frag[2][NF];
  auto slot = [](int q) { return q == 0 ? 0 : (q <= TN ? TM + q - 1 : q - TN); };
  auto fetch = [&](int buf, int kt, int kk, int q) {
    const int f = slot(q);
    const char* st = smem + (kt & 1) * STAGE_BYTES;
    frag[buf][f] = *(const bf16x8_t*)(st + off[f] + ((((kk * 2 + half) ^ key)) << 4));
  };

  const int nk = K / BK;
#pragma unroll
  for (int c = 0; c < L; ++c) copy(0, c);
  if (nk > 1) {
#pragma unroll
    for (int c = 0; c < L; ++c) copy(1, c);
    wait_vmcnt<L>();
  } else {
    wait_vmcnt<0>();
  }
  bare_barrier();
#pragma unroll
  for (int q = 0; q < NF; ++q) fetch(0, 0, 0, q);

  // One slice; MORE: slice kt+1 exists, DMA: slice kt+2 exists.
  auto slice = [&](int kt, auto more_c, auto dma_c) {
    constexpr bool MORE = decltype(more_c)::value, DMA = decltype(dma_c)::value;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;   // KK is even: step parity = kk parity
      const bool last = kk == KK - 1;
      if (last && MORE) {
        // Every fragment of slice kt is in registers once this wave's reads
        // are done; slice kt+1 has landed once this wave's copies of it (the
        // only ones in flight) are done and all waves pass the barrier.
        wait_lgkm0();
        wait_vmcnt<0>();
        bare_barrier();
      }
      const bool nfetch = !last || MORE;
      const int fkt = last ? kt + 1 : kt, fkk = last ? 0 : kk + 1;
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        const int i = q / TN, j = q % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[cur][i], frag[cur][TM + j],
                                                            acc[i][j], 0, 0, 0);
        if (nfetch) {
          // one fragment per MFMA; a step with more fragments than MFMAs
          // (a single 32-row block per wave) reads the rest after its last MFMA
          if (q < NF) fetch(nxt, fkt, fkk, q);
          if (q == NMF - 1)
#pragma unroll
            for (int qq = NMF; qq < NF; ++qq) fetch(nxt, fkt, fkk, qq);
        }
        if (last && DMA) {
          constexpr int PER = (L + NMF - 1) / NMF;
#pragma unroll
          for (int u = 0; u < PER; ++u)
            if (q * PER + u < L) copy(kt + 2, q * PER + u);
        }
        if constexpr (ILV) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0;
  for (; kt + 2 < nk; ++kt) slice(kt, T_{}, T_{});
  if (kt + 1 < nk) slice(kt++, T_{}, F_{});
  slice(kt, F_{}, F_{});

  // Epilogue.
  const bool full = m0 + BM <= M && n0 + BN <= N;
  if constexpr (EPI == EPI_GATED) {
    // In-place read-modify-write of the fp32 residual.  The compiler must
    // assume the stores alias later loads, and one counter tracks both, so
    // loads interleaved with stores would each wait a full round trip.  Whole
    // tiles whose 32-row blocks each lie in one batch row (T % 32 == 0), or
    // that have no gate (plain residual add), run a two-deep pipeline over
    // batches of 4 rows x TN columns per lane instead: batch q+1 is loaded
    // before batch q is stored.
    if (full && !ep.o_seg && (!ep.mod || ep.tok_seg || ep.T % 32 == 0)) {
      float gv[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int grow = ep.tok_seg ? ep.tok_seg[mrow + i * 32] : (mrow + i * 32) / ep.T;
        const float* g = ep.mod ? ep.mod + (int64_t)grow * ep.mod_stride + ep.gate_off : nullptr;
#pragma unroll
        for (int j = 0; j < TN; ++j) gv[i][j] = g ? g[ncol + j * 32] : 1.0f;
      }
      float* xt = (float*)ep.out + (int64_t)mrow * ep.ldo + ncol;
      constexpr int NQ = TM * 4;   // batch q: block q / 4, register group q % 4
      auto xaddr = [&](int q, int r4, int j) {
        return xt + (int64_t)((q >> 2) * 32 + 8 * (q & 3) + r4) * ep.ldo + j * 32;
      };
      float xv[2][4][TN];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int j = 0; j < TN; ++j) xv[0][r4][j] = *xaddr(0, r4, j);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q + 1 < NQ) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
            for (int j = 0; j < TN; ++j) xv[(q + 1) & 1][r4][j] = *xaddr(q + 1, r4, j);
        }
        const int i = q >> 2;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            *xaddr(q, r4, j) = xv[q & 1][r4][j] + gv[i][j] * acc[i][j][(q & 3) * 4 + r4];
      }
      return;
    }
  } else if constexpr (EPI == EPI_BIAS_F32) {
    if (full && !ep.o_seg) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* o = (float*)ep.out + (int64_t)(mrow + i * 32 + 8 * (r >> 2) + (r & 3)) * ep.ldo + ncol;
#pragma unroll
          for (int j = 0; j < TN; ++j) o[j * 32] = acc[i][j][r];
        }
      return;
    }
  } else if constexpr (EPI == EPI_ATOMIC_F32) {
    // split-K partial sums: element by element below
  } else {
    // bf16 outputs: each lane packs rows r, r+1 of its column; neighbouring
    // lanes (columns 2c, 2c+1) exchange those words (one DPP move) and each
    // keeps one row of the column pair, stored as a 4-byte word.
    if (full && vec) {
      const bool odd = lane & 1;
      const uint32_t sel = odd ? 0x03020706u : 0x05040100u;   // (q.hi, p.hi) : (p.lo, q.lo)
      bf16_t* ot = (bf16_t*)ep.out + (int64_t)(mrow + odd) * ep.ldo + (ncol & ~1);
      bf16_t* oc = (bf16_t*)ep.out + (ncol & ~1);   // row-mapped outputs
      // EPI_GELU2 also stores the pre-activation; EPI_DGELU reads it first
      // (all loads before the stores: one counter tracks both)
      bf16_t* ot2 = nullptr;
      if constexpr (EPI == EPI_GELU2) ot2 = (bf16_t*)ep.aux + (int64_t)(mrow + odd) * ep.ldo + (ncol & ~1);
      [[maybe_unused]] uint32_t pk[TM][TN][8];
      if constexpr (EPI == EPI_DGELU) {
        const uint16_t* pa = (const uint16_t*)ep.aux + (int64_t)mrow * ep.ldo + ncol;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              const int r = (p >> 1) * 4 + (p & 1) * 2;
              const int rr = i * 32 + 8 * (r >> 2) + (r & 3);
              pk[i][j][p] = (uint32_t)pa[(int64_t)rr * ep.ldo + j * 32] |
                            ((uint32_t)pa[(int64_t)(rr + 1) * ep.ldo + j * 32] << 16);
            }
      }
      // SEG: rows go through the output row map (only the q | k | v epilogue
      // has one); the choice is made once, outside the store loop
      auto emit = [&](auto seg_tag) {
        constexpr bool SEG = decltype(seg_tag)::value;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const int r = (p >> 1) * 4 + (p & 1) * 2;     // rows r, r+1 of a register group
            float v0 = acc[i][j][r], v1 = acc[i][j][r + 1];
            if constexpr (EPI == EPI_GELU) {
              v0 = gelu_tanh_f(v0);
              v1 = gelu_tanh_f(v1);
            } else if constexpr (EPI == EPI_SILU_DT) {
              v0 = silu_f(v0);
              v1 = silu_f(v1);
            } else if constexpr (EPI == EPI_DGELU) {
              v0 *= gelu_tanh_grad_f(__uint_as_float(pk[i][j][p] << 16));
              v1 *= gelu_tanh_grad_f(__uint_as_float(pk[i][j][p] & 0xFFFF0000u));
            } else if constexpr (EPI == EPI_GELU2) {
              const uint32_t mp = f2bf2(v0, v1);
              const uint32_t op = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mp, 0xB1, 0xF,
                                                                        0xF, false);
              const int rr2 = i * 32 + 8 * (r >> 2) + (r & 3);
              *(uint32_t*)(ot2 + (int64_t)rr2 * ep.ldo + j * 32) = __builtin_amdgcn_perm(op, mp, sel);
              v0 = gelu_tanh_f(v0);
              v1 = gelu_tanh_f(v1);
            } else {
              static_assert(EPI == EPI_BIAS_DT, "epilogue");
            }
            const uint32_t mine = f2bf2(v0, v1);
            // quad_perm [1, 0, 3, 2]: the neighbouring lane's word
            const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xB1, 0xF,
                                                                         0xF, false);
            const uint32_t word = __builtin_amdgcn_perm(other, mine, sel);
            const int rr = i * 32 + 8 * (r >> 2) + (r & 3);
            if constexpr (SEG)
              *(uint32_t*)(oc + row_map(mrow + odd + rr, ep.o_seg, ep.o_skip, ep.o_off) * ep.ldo +
                           j * 32) = word;
            else
              *(uint32_t*)(ot + (int64_t)rr * ep.ldo + j * 32) = word;
          }
      };
      if constexpr (EPI == EPI_BIAS_DT) {
        if (ep.o_seg) emit(std::true_type{});
        else emit(std::false_type{});
      } else {
        emit(std::false_type{});
      }
      return;
    }
  }
  // Ragged or unaligned tiles: element by element with bounds checks (the
  // output row map, used by the q | k | v epilogue only, chosen once).
  auto ragged = [&](auto seg_tag) {
    constexpr bool SEG = decltype(seg_tag)::value;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mrow + i * 32 + 8 * (r >> 2) + (r & 3);
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = ncol + j * 32;
        if (n >= N) continue;
        const float v = acc[i][j][r];
        const int64_t o = (SEG ? row_map(m, ep.o_seg, ep.o_skip, ep.o_off) : (int64_t)m) * ep.ldo + n;
        if constexpr (EPI == EPI_BIAS_F32) {
          ((float*)ep.out)[o] = v;
        } else if constexpr (EPI == EPI_BIAS_DT) {
          ((bf16_t*)ep.out)[o] = f2bf(v);
        } else if constexpr (EPI == EPI_GELU) {
          ((bf16_t*)ep.out)[o] = f2bf(gelu_tanh_f(v));
        } else if constexpr (EPI == EPI_SILU_DT) {
          ((bf16_t*)ep.out)[o] = f2bf(silu_f(v));
        } else if constexpr (EPI == EPI_ATOMIC_F32) {
          unsafeAtomicAdd(&((float*)ep.out)[o], v);
        } else if constexpr (EPI == EPI_GELU2) {
          ((bf16_t*)ep.out)[o] = f2bf(gelu_tanh_f(v));
          ((bf16_t*)ep.aux)[o] = f2bf(v);
        } else if constexpr (EPI == EPI_DGELU) {
          const float z = __uint_as_float((uint32_t)((const uint16_t*)ep.aux)[o] << 16);
          ((bf16_t*)ep.out)[o] = f2bf(v * gelu_tanh_grad_f(z));
        } else {
          static_assert(EPI == EPI_GATED, "epilogue");
          const int grow = ep.tok_seg ? ep.tok_seg[m] : m / ep.T;
          const float g = ep.mod ? ep.mod[(int64_t)grow * ep.mod_stride + ep.gate_off + n] : 1.0f;
          float* X = (float*)ep.out;
          X[o] = X[o] + g * v;
        }
      }
    }
  };
  if constexpr (EPI == EPI_BIAS_DT) {
    if (ep.o_seg) ragged(std::true_type{});
    else ragged(std::false_type{});
  } else {
    ragged(std::false_type{});
  }
}

template <int EPI, int BM, int BN, int BK, int MINWG>
hipError_t run(const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
               const EpiParams& ep, hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  // bf16 outputs are stored as 4-byte column pairs
  const int vec = ((uintptr_t)ep.out & 3) == 0 && ep.ldo % 2 == 0;
  const int64_t ldw = ep.ldw ? ep.ldw : K;
  const bool buf = (row_map(M - 1, ep.a_seg, ep.a_skip, ep.a_off) * lda + K) * 2 < (1LL << 31) &&
                   ((int64_t)(N - 1) * ldw + K) * 2 < (1LL << 31);
  const dim3 grid(tiles, ep.ksplit ? (K + ep.ksplit - 1) / ep.ksplit : 1);
#define DIT_GEMM_LAUNCH(SWZ, BUF)                                                                 \
  gemm_bf16_kernel<EPI, BM, BN, BK, MINWG, SWZ, 1, BUF><<<grid, 256, 0, s>>>(A, lda, W, M, N, K,  \
                                                                           ep, vec)
  if (buf) DIT_GEMM_LAUNCH(1, 1);
  else DIT_GEMM_LAUNCH(1, 0);
#undef DIT_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

int64_t mfma_tiles_128(int64_t M, int64_t N) {
  return ((M + 127) / 128) * (N % 192 ? (N + 127) / 128 : N / 192);
}

namespace {

template <int EPI>
hipError_t pick(const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
                const EpiParams& ep, hipStream_t s) {
  // 128x192 tiles, 64-wide K slices, two LDS buffers (80 KB): two workgroups
  // per CU.  At most 64 rows (the per-row conditioning products) take 64-row
  // tiles, so no MFMA work or LDS traffic goes to padding rows; so do products
  // with at most half as many 128-row tiles as CUs, which doubles their
  // workgroups.  Both tile heights accumulate every output in the same k order
  // with the same MFMA, so the choice does not change a result bit.
  if (M <= 64 || mfma_tiles_128(M, N) <= 128) {
    if (N % 192 == 0) return run<EPI, 64, 192, 64, 2>(A, lda, W, M, N, K, ep, s);
    return run<EPI, 64, 128, 64, 2>(A, lda, W, M, N, K, ep, s);
  }
  if (N % 192 == 0) return run<EPI, 128, 192, 64, 2>(A, lda, W, M, N, K, ep, s);
  return run<EPI, 128, 128, 64, 2>(A, lda, W, M, N, K, ep, s);
}

// ---------------------------------------------------------------------------
// Weight-gradient product C[i, j] += sum_r A[r, i] B[r, j] ("TN": both
// operands stored with the reduction index r as the row, i.e. row-major
// activations and output gradients of a layer, with no transposed copy).
// 128 x 192 tiles over 4 waves (2 x 2, each 64 x 96 as 2 x 3 blocks of
// v_mfma_f32_32x32x16_bf16), r consumed in 64-row slices through two LDS
// stages filled by direct global->LDS copies.  A stage holds each operand as
// 64 rows (r) of its tile width (A 128 bf16 = 16 chunks of 16 B, B 192 = 24
// chunks); chunk c of row r sits at (c + 4 (r % 4)) mod chunks, so the 4
// consecutive rows that one transposing read touches start in 4 different
// 64-byte quarters of the banks.  The MFMA operands (8 consecutive r of one
// column per lane) come from pairs of ds_read_b64_tr_b16.  The grid's second
// dimension splits r (ksplit rows per layer, a multiple of 64) and every layer
// adds its partial sums atomically.
// BUF: the copies go through buffer descriptors over the layer's slab of r
// (32-bit byte offsets), which the compiler leaves to the explicit waits of
// the loop; the plain global->LDS form makes it drain every copy in flight,
// the next slice's included, before the first LDS read of each slice.
template <bool BUF>
__global__ __launch_bounds__(256, 2) void gemm_tn_kernel(const bf16_t* __restrict__ A, int lda,
                                                         const bf16_t* __restrict__ B, int ldb,
                                                         int Mi, int Nj, int R, int ksplit,
                                                         float* __restrict__ out, int ldo,
                                                         float* __restrict__ asum) {
  constexpr int BM = 128, BN = 192, BK = 64, TM = 2, TN = 3;
  constexpr int CA = BM / 8, CB = BN / 8;                     // chunks per row
  constexpr int OPA = BK * BM * 2, OPB = BK * BN * 2;         // bytes per operand tile
  constexpr int STAGE = OPA + OPB;
  constexpr int NCA = OPA / 1024 / 4, NCB = OPB / 1024 / 4;   // 1 KB copies per wave (4, 6)
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  typedef short v4i16 __attribute__((ext_vector_type(4)));

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int tiles_n = (Nj + BN - 1) / BN, tiles_m = (Mi + BM - 1) / BM;
  // Workgroups are dispatched round-robin over the 8 XCDs (workgroup b, in
  // x-fastest order, on XCD b % 8), each with its own L2.  When the counts
  // allow, XCD x takes one contiguous eighth of the tiles, cut across the
  // wider operand, for every layer in turn: the tiles it runs together then
  // share all of the narrow operand's columns and one eighth of the wide
  // one's, and each reduction slab is fetched into that L2 once.
  const int ntile = tiles_m * tiles_n;
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  int tm, tn, layer;
  if ((ntile & 7) == 0) {
    const int per = ntile >> 3, q = lin >> 3;
    const int tl = (lin & 7) * per + q % per;
    layer = q / per;
    if (Nj >= Mi) {
      tn = tl / tiles_m;
      tm = tl - tn * tiles_m;
    } else {
      tm = tl / tiles_n;
      tn = tl - tm * tiles_n;
    }
  } else {
    tile_coords<1>(blockIdx.x, tiles_m, tiles_n, tm, tn);
    layer = blockIdx.y;
  }
  const int i0 = tm * BM, j0 = tn * BN;
  // this layer's slice of the reduction
  const int rb = layer * ksplit;
  const int Rl = min(ksplit, R - rb);
  A += (int64_t)rb * lda;
  B += (int64_t)rb * ldb;

  // Copy slot sl of an operand tile with C chunks per row: LDS row sl / C,
  // stored chunk p = sl % C, which holds logical chunk (p - 4 (row % 4)) mod C
  // of global row r0 + row.  Columns past the operand's width read a clamped
  // (valid) chunk; their outputs are never stored.
  int aoff[NCA], boff[NCB];
#pragma unroll
  for (int c = 0; c < NCA; ++c) {
    const int sl = (w * NCA + c) * 64 + lane, row = sl / CA;
    const int lc = (sl % CA - 4 * (row & 3) + 4 * CA) % CA;
    aoff[c] = row * lda + min(i0 + lc * 8, Mi - 8);
  }
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int sl = (w * NCB + c) * 64 + lane, row = sl / CB;
    const int lc = (sl % CB - 4 * (row & 3) + 4 * CB) % CB;
    boff[c] = row * ldb + min(j0 + lc * 8, Nj - 8);
  }
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t ars =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, BUF ? Rl * lda * 2 : 0, 0x00020000);
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t brs =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, BUF ? Rl * ldb * 2 : 0, 0x00020000);
  auto copy = [&](int kt) {
    char* st = smem + (kt & 1) * STAGE;
    if constexpr (BUF) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
      for (int c = 0; c < NCA; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)(st + (w * NCA + c) * 1024), 16,
                                                 aoff[c] * 2, kt * BK * lda * 2, 0, 0);
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void*)(st + OPA + (w * NCB + c) * 1024),
                                                 16, boff[c] * 2, kt * BK * ldb * 2, 0, 0);
#endif
    } else {
      const int64_t ra = (int64_t)kt * BK * lda, rbb = (int64_t)kt * BK * ldb;
#pragma unroll
      for (int c = 0; c < NCA; ++c)
        __builtin_amdgcn_global_load_lds((const void*)(A + ra + aoff[c]),
                                         (lds_void*)(st + (w * NCA + c) * 1024), 16, 0, 0);
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        __builtin_amdgcn_global_load_lds((const void*)(B + rbb + boff[c]),
                                         (lds_void*)(st + OPA + (w * NCB + c) * 1024), 16, 0, 0);
    }
  };

  // Transposing reads: lane s of 16-lane group G reads row 16 kk + 8 (G / 2) +
  // s / 4 (+ 4 for the second read), columns col + 16 (G % 2) + 4 (s % 4) ..
  // + 3, and receives column col + 16 (G % 2) + s of the 4 rows: the MFMA
  // operand layout (lane l: column l % 32, rows 8 (l / 32) .. + 7).
  const int G = lane >> 4, sx = lane & 15;
  auto frag = [&](const char* op, int C, int col, int kk) {
    const int c = col + 16 * (G & 1) + 4 * (sx & 3);
    const int r0 = 16 * kk + 8 * (G >> 1) + (sx >> 2), r1 = r0 + 4;
    const char* p0 = op + r0 * C * 16 + ((((c >> 3) + 4 * (r0 & 3)) % C) << 4) + (c & 7) * 2;
    const char* p1 = op + r1 * C * 16 + ((((c >> 3) + 4 * (r1 & 3)) % C) << 4) + (c & 7) * 2;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
    return __builtin_bit_cast(bf16x8_t, (__attribute__((ext_vector_type(8))) short){
                                            lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Column sums of A (the bias gradient), taken by the waves with wn == 0 of
  // the tiles in the first column (tn == 0) from the A fragments they already
  // hold: per k step lane l adds 8 r of column l % 32; lanes l and l + 32
  // (the other 8 r) combine at the end.
  const bool csum = asum != nullptr && tn == 0 && wn == 0;
  float cs[TM] = {};
  auto colsum = [&](const bf16x8_t& f, float& acc) {
    const uint4 u = __builtin_bit_cast(uint4, f);
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc += __uint_as_float(wv[e] << 16) + __uint_as_float(wv[e] & 0xFFFF0000u);
  };

  const int nk = Rl / BK;
  copy(0);
  if (nk > 1) {
    copy(1);
    wait_vmcnt<NCA + NCB>();
  } else {
    wait_vmcnt<0>();
  }
  bare_barrier();
  // Per slice: every fragment of the slice is read first; one barrier (the
  // stage is read by every wave, slice kt + 1 has landed for every wave); the
  // copies of slice kt + 2 refill the stage; then the MFMAs, from registers.
  // The compiler makes each slice's first transposing read wait for all
  // copies in flight, so those copies get one slice of MFMAs to land.
  for (int kt = 0; kt < nk; ++kt) {
    const char* st = smem + (kt & 1) * STAGE;
    bf16x8_t fa[BK / 16][TM], fb[BK / 16][TN];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[kk][i] = frag(st, CA, wm * 64 + i * 32, kk);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[kk][j] = frag(st + OPA, CB, wn * 96 + j * 32, kk);
    }
    wait_lgkm0();
    wait_vmcnt<0>();
    bare_barrier();
    if (kt + 2 < nk) copy(kt + 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0,
                                                              0, 0);
      if (csum)
#pragma unroll
        for (int i = 0; i < TM; ++i) colsum(fa[kk][i], cs[i]);
    }
  }

  if (csum) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const float v = cs[i] + __shfl_xor(cs[i], 32, 64);
      const int col = i0 + wm * 64 + i * 32 + lane;
      if (lane < 32 && col < Mi) unsafeAtomicAdd(&asum[col], v);
    }
  }

  // lane: column j0 + wn 96 + 32 j + lane % 32, rows i0 + wm 64 + 32 i + 4 (lane / 32) + 8 (r / 4) + r % 4
  const int ncol = j0 + wn * 96 + (lane & 31);
  const int mrow = i0 + wm * 64 + 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mrow + i * 32 + 8 * (r >> 2) + (r & 3);
      if (m >= Mi) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = ncol + j * 32;
        if (n < Nj) unsafeAtomicAdd(&out[(int64_t)m * ldo + n], acc[i][j][r]);
      }
    }
}

}  // namespace

#ifndef DIT_WIDE_MIN_TILES
#define DIT_WIDE_MIN_TILES 256
#endif

hipError_t launch_gemm_mfma(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N,
                            int K, const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // The wide-tile kernel runs one persistent workgroup per CU, so it pays only
  // when its tiles fill its rounds of 256 workgroups: to 95% for the gated
  // residual epilogue, whose read-modify-write the 128 x 192 kernel below (two
  // workgroups per CU) overlaps with the other workgroup's products, and to
  // 85% for the others (measured at M = 16,512 and 24,960 token rows).
  if (gemm_wide_supported(epi, A, lda, W, M, N, K, ep)) {
    const int64_t wt = (int64_t)((M + 255) / 256) * (N % 288 == 0 ? N / 288 : N / 256);
    const int64_t slots = (wt + 255) / 256 * 256;
    const int64_t fill20 = epi == EPI_GATED ? 19 : 17;   // twentieths
    if (wt >= DIT_WIDE_MIN_TILES && wt * 20 >= slots * fill20)
      return launch_gemm_wide(epi, A, lda, W, M, N, K, ep, s);
  }
  if (K % KSTEP || lda % 8 || (ep.ldw && (ep.ldw % 8 || ep.ldw < K))) return hipErrorInvalidValue;
  if (ep.ksplit < 0 || ep.ksplit % KSTEP || (ep.ksplit && epi != EPI_ATOMIC_F32) ||
      (epi == EPI_ATOMIC_F32 && ep.bias))
    return hipErrorInvalidValue;
  switch (epi) {
    case EPI_BIAS_F32: return pick<EPI_BIAS_F32>(A, lda, W, M, N, K, ep, s);
    case EPI_BIAS_DT: return pick<EPI_BIAS_DT>(A, lda, W, M, N, K, ep, s);
    case EPI_GATED: return pick<EPI_GATED>(A, lda, W, M, N, K, ep, s);
    case EPI_GELU: return pick<EPI_GELU>(A, lda, W, M, N, K, ep, s);
    case EPI_SILU_DT: return pick<EPI_SILU_DT>(A, lda, W, M, N, K, ep, s);
    case EPI_ATOMIC_F32: return pick<EPI_ATOMIC_F32>(A, lda, W, M, N, K, ep, s);
    case EPI_GELU2: return pick<EPI_GELU2>(A, lda, W, M, N, K, ep, s);
    case EPI_DGELU: return pick<EPI_DGELU>(A, lda, W, M, N, K, ep, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_tn(const bf16_t* A, int lda, const bf16_t* B, int ldb, int Mi, int Nj,
                          int R, float* out, int ldo, float* asum, hipStream_t s) {
  if (Mi <= 0 || Nj <= 0 || R <= 0) return hipSuccess;
  if (Mi % 8 || Nj % 8 || R % 64 || lda % 8 || ldb % 8 || lda < Mi || ldb < Nj ||
      ((uintptr_t)A & 15) || ((uintptr_t)B & 15))
    return hipErrorInvalidValue;
  if ((int64_t)(R - 1) * lda + lda > INT32_MAX || (int64_t)(R - 1) * ldb + ldb > INT32_MAX)
    return hipErrorInvalidValue;   // 32-bit element offsets inside the kernel
  const int tiles = ((Mi + 127) / 128) * ((Nj + 191) / 192);
  // fewest reduction layers whose grid fills whole waves of 512 resident
  // workgroups (two per CU) to 92% or more
  int best = 1;
  double best_fill = 0.0;
  for (int sp = 1; sp <= R / 64 && sp <= 256; ++sp) {
    const int64_t wg = (int64_t)tiles * sp, waves = (wg + 511) / 512;
    const double fill = (double)wg / (double)(waves * 512);
    if (fill > best_fill + 0.02) {
      best_fill = fill;
      best = sp;
    }
    if (fill >= 0.92) break;
  }
  int ks = (R + best - 1) / best;
  ks = (ks + 63) / 64 * 64;
  const dim3 grid(tiles, (R + ks - 1) / ks);
  if ((int64_t)ks * lda * 2 < (1LL << 31) && (int64_t)ks * ldb * 2 < (1LL << 31))
    gemm_tn_kernel<true><<<grid, 256, 0, s>>>(A, lda, B, ldb, Mi, Nj, R, ks, out, ldo, asum);
  else
    gemm_tn_kernel<false><<<grid, 256, 0, s>>>(A, lda, B, ldb, Mi, Nj, R, ks, out, ldo, asum);
  return hipGetLastError();
}
