// Attention backward on the matrix cores (bf16 operands, fp32 accumulation),
// dh in {64, 72}.
//
// With S = Q K^T, P = exp(S / sqrt(dh) - lse) (lse: the forward pass's
// log-sum-exp per query) and D_q = sum_e dO_qe O_qe:
//   dV = P^T dO,  dS = P (dO V^T - D),  dK = dS^T Q / sqrt(dh),  dQ = dS K / sqrt(dh).
// Two kernels, each a loop over the other side's tiles:
//   kv: a workgroup owns 64 keys of one (row, head), 16 per wave, and streams
//       32-query tiles; per tile S and dO V^T (queries x keys) come out of
//       v_mfma_f32_16x16x32_bf16 with each lane holding 4 queries of one key,
//       which, for two 16-query blocks, is the B operand of dV^T = dO^T P and
//       dK^T = Q^T dS once the queries inside each 32-query step are taken in
//       the same order on the A side (two transposing LDS reads of the
//       row-major tile);
//   q:  a workgroup owns 64 queries, 16 per wave, and streams 32-key tiles;
//       S^T and V dO^T (keys x queries) give the B operand of dQ^T = K^T dS^T.
// P never leaves registers.  dh = 72 runs its third 32-wide k step with lanes
// past dh 72 holding zeros.
#include "common.h"
#include "train.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

// Tiles of the streamed side are NB x 32 rows (with the next tile prefetched,
// both kernels measured fastest at NB = 1), stored row-major with stride RLD
// and 16 elements of padding (transposing reads past dh 72 of the last row).
constexpr int RLD = 72;           // row-major tile stride (elements)
template <int NB>
struct Tile {
  static constexpr int TQ = 32 * NB;
  static constexpr int SZ = TQ * RLD + 16;
};

template <int DH>
struct Shape {
  static constexpr int NCH = (DH + 31) / 32;    // 32-wide k steps over dh
  static constexpr int NDB = (DH + 15) / 16;    // 16-row blocks of a dh x 16 accumulator
};

__device__ __forceinline__ bf16x8_t ld8(const bf16_t* p) { return *(const bf16x8_t*)p; }

// A/B operand of dh chunk ch of row `row` of a row-major tile (stride RLD):
// lane group g covers dh 32 ch + 8 g .. + 7; past dh the operand is zero.
template <int DH>
__device__ __forceinline__ bf16x8_t row_chunk(const bf16_t* tile, int row, int ch, int g) {
  const int e = 32 * ch + 8 * g;
  if (e >= DH) return bf16x8_t{};
  return ld8(tile + row * RLD + e);
}

// A operand over dh rows 16 db .. 16 db + 15 (lane c16: dh 16 db + c16) and
// the 8 tile rows 4g .. 4g+3, 16 + 4g .. 16 + 4g + 3 of a row-major tile, by
// two transposing LDS reads: lane c16 of group g addresses row 4g + c16 / 4,
// columns 16 db + 4 (c16 % 4) .. + 3, and receives column 16 db + c16 of the
// group's 4 rows.  Lanes past dh 72 read finite neighbouring data that only
// reaches accumulator rows past dh, which are never stored.
__device__ __forceinline__ bf16x8_t tr_operand(const bf16_t* tile, int db, int g, int c16) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const bf16_t* p = tile + (4 * g + (c16 >> 2)) * RLD + 16 * db + 4 * (c16 & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
  const v4i16 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 16 * RLD));
  return __builtin_bit_cast(bf16x8_t, (__attribute__((ext_vector_type(8))) short){
                                          lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

__device__ __forceinline__ bf16x8_t pack8(const floatx4& a, const floatx4& b) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(f2bf2(a[0], a[1]), f2bf2(a[2], a[3]),
                                                 f2bf2(b[0], b[1]), f2bf2(b[2], b[3])));
}

// Staging of TQ rows (row0 ..) of the dh slice at `src` (row stride ld
// elements) into a row-major tile, in two halves so the next tile's global
// loads are in flight while the current one is consumed: load() fills this
// thread's registers (rows at or past T read as zeros), store() writes them.
template <int DH, int TQ>
struct Stager {
  static constexpr int CPR = DH / 8;                 // 16-byte chunks per row
  static constexpr int PER = (TQ * CPR + 255) / 256;  // chunks per thread
  uint4 v[PER];
  __device__ __forceinline__ void load(const bf16_t* src, int64_t ld, int row0, int T, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u, r = c / CPR, e = (c - r * CPR) * 8;
      v[u] = make_uint4(0, 0, 0, 0);
      if (c < TQ * CPR && row0 + r < T) v[u] = *(const uint4*)(src + (int64_t)(row0 + r) * ld + e);
    }
  }
  __device__ __forceinline__ void store(bf16_t* tile, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u, r = c / CPR, e = (c - r * CPR) * 8;
      if (c < TQ * CPR) *(uint4*)(tile + r * RLD + e) = v[u];
    }
  }
};


template <int DH, int NB>
__global__ __launch_bounds__(256) void attn_bwd_kv_mfma(const bf16_t* __restrict__ QKV,
                                                        const bf16_t* __restrict__ dO,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ Dv, int H, int T,
                                                        float sl2, bf16_t* __restrict__ dQKV) {
  using S = Shape<DH>;
  constexpr int TQ = Tile<NB>::TQ;
  __shared__ __attribute__((aligned(16))) bf16_t sQb[2][Tile<NB>::SZ], sGb[2][Tile<NB>::SZ];
  __shared__ float sLb[2][TQ], sDb[2][TQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int64_t ld = 3LL * H * DH, ldo = (int64_t)H * DH;
  const bf16_t* Qb = QKV + (int64_t)b * T * ld + h * DH;
  const bf16_t* Gb = dO + (int64_t)b * T * ldo + h * DH;
  const int key = blockIdx.x * 64 + wave * 16 + c16;   // this lane's key (B-operand column)
  const bool kval = key < T;

  // This wave's K and V rows as B operands (zero past T and past dh).
  bf16x8_t kf[S::NCH], vf[S::NCH];
#pragma unroll
  for (int ch = 0; ch < S::NCH; ++ch) {
    const int e = 32 * ch + 8 * g;
    const bool ok = kval && e < DH;
    kf[ch] = ok ? ld8(Qb + (int64_t)key * ld + ldo + e) : bf16x8_t{};
    vf[ch] = ok ? ld8(Qb + (int64_t)key * ld + 2 * ldo + e) : bf16x8_t{};
  }
  floatx4 dk[S::NDB], dv[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) {
    dk[db] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    dv[db] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  if (tid < 16) {   // the pad after each tile: finite values
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sQb[bb][TQ * RLD + tid] = f2bf(0.0f);
      sGb[bb][TQ * RLD + tid] = f2bf(0.0f);
    }
  }
  const float* L = lse + (int64_t)bh * T;
  const float* Dd = Dv + (int64_t)bh * T;
  const float LOG2E = 1.4426950408889634f;
  Stager<DH, TQ> stq, stg;
  float lv = 0.0f, dv_ = 0.0f;
  // per-query constants of tile rows: exp2(. - inf) = 0 for missing queries
  auto load_consts = [&](int q0) {
    if (tid < TQ) {
      const int q = q0 + tid;
      lv = q < T ? L[q] * LOG2E : INFINITY;
      dv_ = q < T ? Dd[q] : 0.0f;
    }
  };
  auto store_consts = [&](int bb) {
    if (tid < TQ) {
      sLb[bb][tid] = lv;
      sDb[bb][tid] = dv_;
    }
  };
  stq.load(Qb, ld, 0, T, tid);
  stg.load(Gb, ldo, 0, T, tid);
  load_consts(0);
  stq.store(sQb[0], tid);
  stg.store(sGb[0], tid);
  store_consts(0);
  __syncthreads();

  for (int it = 0, q0 = 0; q0 < T; ++it, q0 += TQ) {
    const int bb = it & 1;
    const bool more = q0 + TQ < T;
    if (more) {   // next tile's loads in flight during this one
      stq.load(Qb, ld, q0 + TQ, T, tid);
      stg.load(Gb, ldo, q0 + TQ, T, tid);
      load_consts(q0 + TQ);
    }
    const bf16_t* sQ = sQb[bb];
    const bf16_t* sG = sGb[bb];
    const float* sL = sLb[bb];
    const float* sD = sDb[bb];

    // S, dP (queries x this wave's keys): lane holds queries 16 qb + 4 g + r.
    floatx4 s[2 * NB], dp[2 * NB];
#pragma unroll
    for (int qb = 0; qb < 2 * NB; ++qb) {
      s[qb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      dp[qb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ch = 0; ch < S::NCH; ++ch) {
        s[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_chunk<DH>(sQ, 16 * qb + c16, ch, g),
                                                         kf[ch], s[qb], 0, 0, 0);
        dp[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_chunk<DH>(sG, 16 * qb + c16, ch, g),
                                                          vf[ch], dp[qb], 0, 0, 0);
      }
    }
    floatx4 p[2 * NB], ds[2 * NB];
#pragma unroll
    for (int qb = 0; qb < 2 * NB; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = 16 * qb + 4 * g + r;
        const float pv = __builtin_amdgcn_exp2f(s[qb][r] * sl2 - sL[qi]);
        p[qb][r] = pv;
        ds[qb][r] = pv * (dp[qb][r] - sD[qi]);
      }
#pragma unroll
    for (int j = 0; j < NB; ++j) {   // 32-query step j: blocks 2j, 2j + 1
      const bf16x8_t pf = pack8(p[2 * j], p[2 * j + 1]);
      const bf16x8_t dsf = pack8(ds[2 * j], ds[2 * j + 1]);
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_operand(sG + 32 * j * RLD, db, g, c16),
                                                          pf, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_operand(sQ + 32 * j * RLD, db, g, c16),
                                                          dsf, dk[db], 0, 0, 0);
      }
    }
    // the other buffer was last read in the previous iteration, before its barrier
    if (more) {
      stq.store(sQb[bb ^ 1], tid);
      stg.store(sGb[bb ^ 1], tid);
      store_consts(bb ^ 1);
    }
    __syncthreads();
  }

  // lane holds dh 16 db + 4 g + r of `key`
  if (kval) {
    const float scale = sl2 / LOG2E;
    bf16_t* o = dQKV + ((int64_t)b * T + key) * ld + h * DH;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
      const int e = 16 * db + 4 * g;
      if (e < DH) {
        *(uint2*)(o + ldo + e) = make_uint2(f2bf2(dk[db][0] * scale, dk[db][1] * scale),
                                            f2bf2(dk[db][2] * scale, dk[db][3] * scale));
        *(uint2*)(o + 2 * ldo + e) = make_uint2(f2bf2(dv[db][0], dv[db][1]),
                                                f2bf2(dv[db][2], dv[db][3]));
      }
    }
  }
}

template <int DH, int NB>
__global__ __launch_bounds__(256) void attn_bwd_q_mfma(const bf16_t* __restrict__ QKV,
                                                       const bf16_t* __restrict__ dO,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ Dv, int H, int T,
                                                       float sl2, bf16_t* __restrict__ dQKV) {
  using S = Shape<DH>;
  constexpr int TQ = Tile<NB>::TQ;
  __shared__ __attribute__((aligned(16))) bf16_t sKb[2][Tile<NB>::SZ], sVb[2][Tile<NB>::SZ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int64_t ld = 3LL * H * DH, ldo = (int64_t)H * DH;
  const bf16_t* Qb = QKV + (int64_t)b * T * ld + h * DH;
  const bf16_t* Gb = dO + (int64_t)b * T * ldo + h * DH;
  const int q = blockIdx.x * 64 + wave * 16 + c16;      // this lane's query (B-operand column)
  const bool qval = q < T;
  const float LOG2E = 1.4426950408889634f;

  bf16x8_t qf[S::NCH], gf[S::NCH];
#pragma unroll
  for (int ch = 0; ch < S::NCH; ++ch) {
    const int e = 32 * ch + 8 * g;
    const bool ok = qval && e < DH;
    qf[ch] = ok ? ld8(Qb + (int64_t)q * ld + e) : bf16x8_t{};
    gf[ch] = ok ? ld8(Gb + (int64_t)q * ldo + e) : bf16x8_t{};
  }
  const float lq = qval ? lse[(int64_t)bh * T + q] * LOG2E : INFINITY;
  const float dq_ = qval ? Dv[(int64_t)bh * T + q] : 0.0f;
  floatx4 dq[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) dq[db] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  if (tid < 16) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sKb[bb][TQ * RLD + tid] = f2bf(0.0f);
      sVb[bb][TQ * RLD + tid] = f2bf(0.0f);
    }
  }
  Stager<DH, TQ> stk, stv;
  stk.load(Qb + ldo, ld, 0, T, tid);
  stv.load(Qb + 2 * ldo, ld, 0, T, tid);
  stk.store(sKb[0], tid);
  stv.store(sVb[0], tid);
  __syncthreads();

  for (int it = 0, k0 = 0; k0 < T; ++it, k0 += TQ) {
    const int bb = it & 1;
    const bool more = k0 + TQ < T;
    if (more) {
      stk.load(Qb + ldo, ld, k0 + TQ, T, tid);
      stv.load(Qb + 2 * ldo, ld, k0 + TQ, T, tid);
    }
    const bf16_t* sK = sKb[bb];
    const bf16_t* sV = sVb[bb];

    // S^T, dP^T (keys x this wave's queries): lane holds keys 16 kb + 4 g + r.
    floatx4 st[2 * NB], dpt[2 * NB];
#pragma unroll
    for (int kb = 0; kb < 2 * NB; ++kb) {
      st[kb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      dpt[kb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ch = 0; ch < S::NCH; ++ch) {
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_chunk<DH>(sK, 16 * kb + c16, ch, g),
                                                          qf[ch], st[kb], 0, 0, 0);
        dpt[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_chunk<DH>(sV, 16 * kb + c16, ch, g),
                                                           gf[ch], dpt[kb], 0, 0, 0);
      }
    }
    floatx4 dst[2 * NB];
#pragma unroll
    for (int kb = 0; kb < 2 * NB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kj = k0 + 16 * kb + 4 * g + r;
        const float pv = kj < T ? __builtin_amdgcn_exp2f(st[kb][r] * sl2 - lq) : 0.0f;
        dst[kb][r] = pv * (dpt[kb][r] - dq_);
      }
#pragma unroll
    for (int j = 0; j < NB; ++j) {   // 32-key step j
      const bf16x8_t dsf = pack8(dst[2 * j], dst[2 * j + 1]);
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
        dq[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_operand(sK + 32 * j * RLD, db, g, c16),
                                                          dsf, dq[db], 0, 0, 0);
    }
    if (more) {
      stk.store(sKb[bb ^ 1], tid);
      stv.store(sVb[bb ^ 1], tid);
    }
    __syncthreads();
  }

  if (qval) {
    const float scale = sl2 / LOG2E;
    bf16_t* o = dQKV + ((int64_t)b * T + q) * ld + h * DH;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
      const int e = 16 * db + 4 * g;
      if (e < DH)
        *(uint2*)(o + e) = make_uint2(f2bf2(dq[db][0] * scale, dq[db][1] * scale),
                                      f2bf2(dq[db][2] * scale, dq[db][3] * scale));
    }
  }
}

}  // namespace

hipError_t launch_attention_bwd_mfma(const void* qkv, const void* dO, const float* lse,
                                     const float* Dv, int B, int heads, int T, int dh,
                                     void* dqkv, hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  if ((dh != 64 && dh != 72) || (int64_t)B * heads > 65535) return hipErrorInvalidValue;
  const float sl2 = 1.4426950408889634f / sqrtf((float)dh);
  const dim3 grid((T + 63) / 64, B * heads);
  if (dh == 64) {
    attn_bwd_kv_mfma<64, 1><<<grid, 256, 0, s>>>((const bf16_t*)qkv, (const bf16_t*)dO, lse, Dv,
                                              heads, T, sl2, (bf16_t*)dqkv);
    attn_bwd_q_mfma<64, 1><<<grid, 256, 0, s>>>((const bf16_t*)qkv, (const bf16_t*)dO, lse, Dv,
                                             heads, T, sl2, (bf16_t*)dqkv);
  } else {
    attn_bwd_kv_mfma<72, 1><<<grid, 256, 0, s>>>((const bf16_t*)qkv, (const bf16_t*)dO, lse, Dv,
                                              heads, T, sl2, (bf16_t*)dqkv);
    attn_bwd_q_mfma<72, 1><<<grid, 256, 0, s>>>((const bf16_t*)qkv, (const bf16_t*)dO, lse, Dv,
                                             heads, T, sl2, (bf16_t*)dqkv);
  }
  return hipGetLastError();
}
