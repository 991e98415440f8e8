// Multi-head attention core O = softmax(Q K^T / sqrt(dh)) V, flash style:
// keys are streamed in tiles with an online softmax, so memory is O(T).
//
// bf16 path (MFMA, dh in {64, 72}).  A workgroup of 4 waves owns 128 queries of
// one (batch, head); each wave 32 queries.  Per 64-key tile, staged in LDS:
//   S^T[key, q] = K Q^T  with v_mfma_f32_16x16x32_bf16 (dh 64..71 of dh = 72 by
//                        a third 16x16x32 step whose lanes past dh 72 hold zeros,
//                        so every S accumulation is one chain of the same
//                        instruction, accumulated in place),
//   online softmax per query column in the exp2 domain,
//   O^T[dh, q] += V^T P^T with v_mfma_f32_16x16x32_bf16.
// Computing S transposed leaves each lane holding keys 4g..4g+3 of four 16-key
// blocks for one query, which is exactly a B operand of the P V^T product once
// the key order inside each 32-key step is permuted the same way for V (the
// contraction is a sum, so any consistent key order is correct).  P therefore
// never leaves registers; V is stored transposed (keys fastest) so its operand
// is two 8-byte LDS reads.
//
// fp32 path: one thread per query, keys streamed through LDS (small shapes).
#include "common.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

template <int DH>
__global__ __launch_bounds__(256) void attn_bf16_kernel(const bf16_t* __restrict__ Q,
                                                        const bf16_t* __restrict__ K,
                                                        const bf16_t* __restrict__ Vt,
                                                        bf16_t* __restrict__ O, int H, int T,
                                                        int ldv, float sl2) {
  constexpr int KV = 64;                 // keys per tile
  constexpr int KLD = 72;                // K tile row stride (elements), 144 B
  constexpr int VLD = KV + 4;            // V^T tile row stride (elements), 136 B
  constexpr int NDB = (DH + 15) / 16;    // 16-row blocks of the O^T accumulator
  constexpr bool TAIL = (DH % 32) != 0;  // dh = 72: columns 64..71
  static_assert(DH == 64 || DH == 72, "head dim");
  __shared__ __attribute__((aligned(16))) bf16_t sK[KV * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[DH * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int q0 = blockIdx.x * 128 + wave * 32;
  const bf16_t* Qb = Q + (int64_t)bh * T * DH;
  const bf16_t* Kb = K + (int64_t)bh * T * DH;
  const bf16_t* Vb = Vt + (int64_t)bh * DH * ldv;

  const bf16x8_t z8 = {};
  bf16x8_t qf[2][2];
  bf16x8_t qt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int q = q0 + 16 * qb + c16;
    bool ok = q < T;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      qf[qb][c] = ok ? *(const bf16x8_t*)(Qb + (int64_t)q * DH + 32 * c + 8 * g) : z8;
    qt[qb] = z8;   // dh 64..71 in lanes g == 0, zeros elsewhere
    if constexpr (TAIL)
      if (ok && g == 0) qt[qb] = *(const bf16x8_t*)(Qb + (int64_t)q * DH + 64);
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
  floatx4 oacc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kv0 = 0; kv0 < T; kv0 += KV) {
    __syncthreads();
    // K tile: KV rows of DH, contiguous in HBM.
    constexpr int KCH = KV * DH / 8;
    for (int idx = tid; idx < KCH; idx += 256) {
      int row = idx / (DH / 8), col = (idx - row * (DH / 8)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kv0 + row < T) v = *(const uint4*)(Kb + (int64_t)(kv0 + row) * DH + col);
      *(uint4*)&sK[row * KLD + col] = v;
    }
    // V^T tile: DH rows of KV keys (row stride ldv in HBM).
    constexpr int VCH = DH * KV / 8;
    for (int idx = tid; idx < VCH; idx += 256) {
      int row = idx / (KV / 8), col = (idx - row * (KV / 8)) * 8;
      int kv = kv0 + col;
      const bf16_t* src = Vb + (int64_t)row * ldv + kv;
      uint4 v;
      if (kv + 8 <= T) {
        v = *(const uint4*)src;
      } else {
        uint16_t e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = (kv + u < T) ? src[u] : (uint16_t)0;
        v.x = e[0] | ((uint32_t)e[1] << 16);
        v.y = e[2] | ((uint32_t)e[3] << 16);
        v.z = e[4] | ((uint32_t)e[5] << 16);
        v.w = e[6] | ((uint32_t)e[7] << 16);
      }
      uint2* dst = (uint2*)&sV[row * VLD + col];
      dst[0] = make_uint2(v.x, v.y);
      dst[1] = make_uint2(v.z, v.w);
    }
    __syncthreads();

    // S^T blocks: 4 key blocks x 2 query blocks of 16x16.
    floatx4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16_t* kr = &sK[(16 * kb + c16) * KLD];
      bf16x8_t k0 = *(const bf16x8_t*)(kr + 8 * g);
      bf16x8_t k1 = *(const bf16x8_t*)(kr + 32 + 8 * g);
      bf16x8_t kt = z8;
      if constexpr (TAIL)
        if (g == 0) kt = *(const bf16x8_t*)(kr + 64);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        floatx4 a = {0.0f, 0.0f, 0.0f, 0.0f};
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[qb][0], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[qb][1], a, 0, 0, 0);
        if constexpr (TAIL) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, qt[qb], a, 0, 0, 0);
        s[kb][qb] = a;
      }
    }

    // Online softmax (log2 domain).  Lane holds query column c16 of block qb and
    // keys 16 kb + 4 g + r; the 4 lanes sharing c16 are combined by xor 16, 32.
    bf16x8_t pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int kv = kv0 + 16 * kb + 4 * g + r;
          float v = s[kb][qb][r] * sl2;
          v = kv < T ? v : -INFINITY;
          s[kb][qb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[qb], mx);
      const float alpha = exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      l_run[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][qb][r] *= alpha;
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bf16_t pb = f2bf(exp2f(s[kb][qb][r] - m_new));
          ls += bf2f(pb);
          pf[qb][kb >> 1][(kb & 1) * 4 + r] = __builtin_bit_cast(__bf16, pb);
        }
      l_run[qb] += ls;
    }

    // O^T[dh, q] += V^T[dh, key] P^T[key, q]; key order within each 32-key step:
    // 4g..4g+3 of the even 16-block, then 4g..4g+3 of the odd one.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dr = 16 * db + c16;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t vf = z8;
        if (dr < DH) {
          uint2 lo = *(const uint2*)&sV[dr * VLD + 32 * j + 4 * g];
          uint2 hi = *(const uint2*)&sV[dr * VLD + 32 * j + 16 + 4 * g];
          uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
          vf = __builtin_bit_cast(bf16x8_t, u);
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb][j], oacc[db][qb], 0, 0, 0);
      }
    }
  }

  // Normalise and store O[b, q, h*DH + dh] (token-major, heads concatenated).
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int q = q0 + 16 * qb + c16;
    if (q >= T) continue;
    bf16_t* orow = O + ((int64_t)b * T + q) * H * DH + h * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      int d0 = 16 * db + 4 * g;
      if (d0 + 3 < DH) {
        uint32_t lo = (uint32_t)f2bf(oacc[db][qb][0] * inv) | ((uint32_t)f2bf(oacc[db][qb][1] * inv) << 16);
        uint32_t hi = (uint32_t)f2bf(oacc[db][qb][2] * inv) | ((uint32_t)f2bf(oacc[db][qb][3] * inv) << 16);
        *(uint2*)(orow + d0) = make_uint2(lo, hi);
      }
    }
  }
}

template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      float* __restrict__ O, int H, int T,
                                                      float scale) {
  constexpr int KT = 32;
  __shared__ float sK[KT][DH], sV[KT][DH];
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const float* Qb = Q + (int64_t)bh * T * DH;
  const float* Kb = K + (int64_t)bh * T * DH;
  const float* Vb = V + (int64_t)bh * T * DH;
  float qv[DH], acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    qv[e] = qi < T ? Qb[(int64_t)qi * DH + e] : 0.0f;
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int kv0 = 0; kv0 < T; kv0 += KT) {
    __syncthreads();
    for (int e = threadIdx.x; e < KT * DH; e += 64) {
      int r = e / DH, c = e - r * DH;
      bool ok = kv0 + r < T;
      sK[r][c] = ok ? Kb[(int64_t)(kv0 + r) * DH + c] : 0.0f;
      sV[r][c] = ok ? Vb[(int64_t)(kv0 + r) * DH + c] : 0.0f;
    }
    __syncthreads();
    const int nv = min(KT, T - kv0);
    for (int j = 0; j < nv; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < DH; ++e) s = fmaf(qv[e], sK[j][e], s);
      s *= scale;
      float mn = fmaxf(m, s);
      float corr = expf(m - mn), p = expf(s - mn);
      l = l * corr + p;
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] = fmaf(p, sV[j][e], acc[e] * corr);
      m = mn;
    }
  }
  if (qi < T) {
    float* orow = O + ((int64_t)b * T + qi) * H * DH + h * DH;
    float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DH; ++e) orow[e] = acc[e] * inv;
  }
}

}  // namespace

hipError_t launch_attention(const void* q, const void* k, const void* v, int B, int heads,
                            int T, int dh, int dtype, void* o, hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  if (dtype == 1) {
    const float sl2 = 1.4426950408889634f / sqrtf((float)dh);
    dim3 grid((T + 127) / 128, B * heads);
    int ldv = round_up(T, 64);
    if (dh == 64)
      attn_bf16_kernel<64><<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)k,
                                                (const bf16_t*)v, (bf16_t*)o, heads, T, ldv, sl2);
    else if (dh == 72)
      attn_bf16_kernel<72><<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)k,
                                                (const bf16_t*)v, (bf16_t*)o, heads, T, ldv, sl2);
    else
      return hipErrorInvalidValue;
  } else {
    const float scale = 1.0f / sqrtf((float)dh);
    dim3 grid((T + 63) / 64, B * heads);
    if (dh == 64)
      attn_f32_kernel<64><<<grid, 64, 0, s>>>((const float*)q, (const float*)k, (const float*)v,
                                              (float*)o, heads, T, scale);
    else if (dh == 72)
      attn_f32_kernel<72><<<grid, 64, 0, s>>>((const float*)q, (const float*)k, (const float*)v,
                                              (float*)o, heads, T, scale);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
