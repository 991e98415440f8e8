// Multi-head attention core O = softmax(Q K^T / sqrt(dh)) V, flash style:
// keys are streamed in tiles with an online softmax, so memory is O(T).
//
// bf16 path (MFMA, dh in {64, 72}).  A workgroup of NWV waves owns 32 NWV queries of
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
// never leaves registers.  The V tile is transposed while it is staged into
// LDS (4 keys x 4 features per thread, transposed in registers) so its operand
// is two 8-byte LDS reads.
//
// Input: the packed in-projection output qkv [B, T, 3 H dh] (q | k | v, heads as
// contiguous dh slices), read with its row stride; output o [B, T, H dh].
//
// fp32 path: one thread per query, keys streamed through LDS (small shapes).
#include <type_traits>

#include "common.h"
#include "mfma_util.h"


namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

// 8 bf16 query features times the exp2-domain score scale, rounded to bf16
// once (round to nearest even): scores then come out of the MFMA already in
// the exp2 domain.
__device__ __forceinline__ bf16x8_t scale_bf16x8(bf16x8_t v, float sc) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  auto two = [&](uint32_t w) {
    return f2bf2(__uint_as_float(w << 16) * sc, __uint_as_float(w & 0xFFFF0000u) * sc);
  };
  return __builtin_bit_cast(bf16x8_t, make_uint4(two(u.x), two(u.y), two(u.z), two(u.w)));
}

// PK: packed sequences.  The grid is (query blocks of all sequences, heads);
// a block finds its sequence in the by-value table and attends over that
// sequence's tokens only.
template <int DH, int NWV, bool PK = false>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void attn_bf16_kernel(const bf16_t* __restrict__ QKV,
                                                           bf16_t* __restrict__ O, int H,
                                                           int T_rows, float sl2, SeqTable seqs,
                                                           float* __restrict__ lse) {
  constexpr int KV = 64;                  // keys per tile
  // K tile row stride (elements), 160 B: the fragment reads of 16 rows x 2
  // chunks that the LDS serves together land on distinct banks (144-byte
  // rows put two of them on one bank)
  constexpr int KLD = 80;
  constexpr int VLD = KV + 4;             // V^T tile row stride (elements), 136 B
  constexpr int NDB = (DH + 15) / 16;     // 16-row blocks of the O^T accumulator
  constexpr bool TAIL = (DH % 32) != 0;   // dh = 72: columns 64..71
  constexpr int KCH = KV * DH / 8;        // 16-byte chunks of a K tile
  constexpr int NTH = 64 * NWV;           // threads of the workgroup
  constexpr int QPB = 32 * NWV;           // queries per workgroup
  constexpr int KPT = (KCH + NTH - 1) / NTH;  // ... per thread
  constexpr int VB = (KV / 4) * (DH / 4); // 4x4 (key x feature) items of a V tile
  constexpr int VPT = (VB + NTH - 1) / NTH;   // ... per thread
  constexpr float RESCALE_SLACK = 8.0f;   // log2 headroom before the running max is raised
  static_assert(DH == 64 || DH == 72, "head dim");
  // dh = 72: K and V tiles are copied into LDS as they are (dense [key][72]
  // rows) by buffer->LDS loads, and the V^T operand of the P V product is read
  // with transposing LDS reads.  dh = 64: registers stage the tiles and V is
  // transposed on the way into LDS.
  constexpr bool DMA = DH == 72;
  // dh 72: V rows of 80 in LDS; columns 72..79 hold (1, 0, .., 0), so row 72
  // of O^T = V^T P^T is the sum of the tile's (bf16) weights: the softmax
  // normaliser comes out of the same products as the numerator.
  constexpr int VS = 80;
  constexpr int VSZ = DMA ? KV * VS : DH * VLD;
  // K tiles carry 24 zero elements after their last row: the dh 64..95 operand
  // reads of the last rows reach into them (see the score products)
  constexpr int KPAD = 24;
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KV * KLD + KPAD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][VSZ];
  // 16 zero bytes: operand lanes past dh read here instead of taking a branch
  __shared__ __attribute__((aligned(16))) uint4 zslot;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform as far as the compiler can see (a lane-derived index would
  // turn the per-wave choice of copy source into a loop over lanes)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  // Workgroups are dispatched round-robin over the 8 XCDs; when their count
  // allows, workgroup i runs logical block (i % 8) * (n / 8) + i / 8, so the
  // query blocks of one (row, head) run on one XCD and share its L2 copy of K, V.
  const int nwg = gridDim.x * gridDim.y;
  int lin = blockIdx.y * gridDim.x + blockIdx.x;
  if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
  const int bh = lin / gridDim.x;
  const int b = bh / H, h = bh - b * H;
  int qblk = lin - bh * gridDim.x;
  int T = T_rows;                      // tokens of this block's row / sequence
  int64_t tok0 = (int64_t)b * T_rows;  // its first token in the packed rows
  if constexpr (PK) {
    int j = 0;
    while (j + 1 < seqs.n && seqs.blk[j + 1] <= qblk) ++j;
    qblk -= seqs.blk[j];
    tok0 = seqs.tok[j];
    T = seqs.tok[j + 1] - seqs.tok[j];
  }
  const int q0 = qblk * QPB + wave * 32;
  const int64_t ld = 3LL * H * DH;                       // packed row stride
  const bf16_t* Qb = QKV + tok0 * ld + h * DH;           // + t * ld
  const bf16_t* Kb = Qb + (int64_t)H * DH;
  const bf16_t* Vb = Qb + 2LL * H * DH;

  const bf16x8_t z8 = {};
  bf16x8_t qf[2][2];
  bf16x8_t qt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int q = q0 + 16 * qb + c16;
    bool ok = q < T;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      qf[qb][c] = ok ? scale_bf16x8(*(const bf16x8_t*)(Qb + q * ld + 32 * c + 8 * g), sl2) : z8;
    qt[qb] = z8;   // dh 64..71 in lanes g == 0, zeros elsewhere
    if constexpr (TAIL)
      if (ok && g == 0) qt[qb] = scale_bf16x8(*(const bf16x8_t*)(Qb + q * ld + 64), sl2);
  }

  // Tile staging: global -> registers (issued one tile ahead) -> LDS.  Loads
  // are raw buffer loads on this (batch row)'s slice of qkv: keys at or past T
  // lie outside the buffer range and read as zeros, so the loop carries no
  // bounds tests.  Each thread's byte offsets inside a tile are fixed; a tile
  // adds kv0 * row stride.
  const int nrec = (int)((int64_t)T * ld * 2);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Kb, (short)0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vb, (short)0, nrec, 0x00020000);
  int koff[KPT], voff[VPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int idx = min(tid + u * NTH, KCH - 1);
    const int row = idx / (DH / 8), col = (idx - row * (DH / 8)) * 8;
    koff[u] = (int)((row * ld + col) * 2);
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int idx = min(tid + u * NTH, VB - 1);
    const int kb4 = idx / (DH / 4), d4 = (idx - kb4 * (DH / 4)) * 4;
    voff[u] = (int)((4 * kb4 * ld + d4) * 2);
  }
  const int ldb = (int)(ld * 2);
  uint4 kreg[KPT];
  uint2 vreg[VPT][4];
  auto gload = [&](int kv0) {
    const int t0 = kv0 * ldb;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      kreg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, koff[u] + t0, 0, 0));
#pragma unroll
    for (int u = 0; u < VPT; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        vreg[u][q] = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(vrs, voff[u] + t0 + q * ldb, 0, 0));
  };
  // DMA staging (dh = 72): direct global->LDS copies of 64 lanes x 16 bytes,
  // lane l of a copy landing at its LDS base + 16 l.  A K tile and a V tile
  // are 10 copies each (slot c: row c / 10, 16-byte column c % 10), whose
  // lanes on column 9, the pad (zeros in K, (1, 0, .., 0) in V), stay
  // inactive and leave it as written at the start.  Copy u of wave w is
  // number w + NWV u.  Byte offsets inside a tile are fixed per lane; the
  // tile's row offset rides in the scalar offset.  The rows of a ragged last
  // tile past T read row T - 1: finite data whose weights are 0.
  constexpr int NCK = KV * KLD / 512, NCV = KV * VS / 512, NCP = NCK + NCV;
  constexpr int CPW = (NCP + NWV - 1) / NWV;
  int drow[CPW], doff[CPW];
  uint32_t dpad = 0;                       // bit u: copy u's lane is a K or V pad slot
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int ii = wave + NWV * u;
    const bool isv = ii >= NCK;
    const int c = (isv ? ii - NCK : ii) * 64 + lane;
    const int per = isv ? VS / 8 : KLD / 8;
    const int row = c / per, col = c - row * per;
    drow[u] = row;
    doff[u] = (int)(((int64_t)row * ld + (col < DH / 8 ? col : 0) * 8) * 2);
    if (col == DH / 8) dpad |= 1u << u;
  }
  auto dma = [&](int kv0, int buf, auto rag_c) {
    constexpr bool ragged = decltype(rag_c)::value;   // the tile reaches past T
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int ii = wave + NWV * u;                // wave-uniform
      if (ii < NCP) {
        const bool isv = ii >= NCK;
        char* dst = (isv ? (char*)sV[buf] : (char*)sK[buf]) + (isv ? ii - NCK : ii) * 1024;
        int voff_ = doff[u], soff = kv0 * ldb;
        if constexpr (ragged) {
          voff_ += (min(kv0 + drow[u], T - 1) - drow[u]) * ldb;
          soff = 0;
        }
        // buffer form: ordered by the explicit waits and barriers of the loop
        if (!(dpad >> u & 1)) {
#if defined(__HIP_DEVICE_COMPILE__)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vrs : krs, (lds_void*)dst, 16, voff_, soff, 0,
                                                   0);
#endif
        }
      }
    }
  };

  // K rows as they are; V transposed into sV[dh][key]: vreg[u][q] holds features
  // d4..d4+3 of key 4*kb4+q, column e is (vreg[u][0].e, .., vreg[u][3].e).
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int idx = tid + u * NTH;
      if (idx < KCH) {
        const int row = idx / (DH / 8), col = (idx - row * (DH / 8)) * 8;
        *(uint4*)&sK[buf][row * KLD + col] = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int idx = tid + u * NTH;
      if (idx < VB) {
        const int kb4 = idx / (DH / 4), d4 = (idx - kb4 * (DH / 4)) * 4;
        const uint2* r = vreg[u];
        // pairs of features packed per key: x = (f0, f1), y = (f2, f3)
        uint32_t lo01 = __builtin_amdgcn_perm(r[1].x, r[0].x, 0x05040100u);  // f0 of keys 0,1
        uint32_t hi01 = __builtin_amdgcn_perm(r[3].x, r[2].x, 0x05040100u);  // f0 of keys 2,3
        uint32_t lo11 = __builtin_amdgcn_perm(r[1].x, r[0].x, 0x07060302u);  // f1 of keys 0,1
        uint32_t hi11 = __builtin_amdgcn_perm(r[3].x, r[2].x, 0x07060302u);  // f1 of keys 2,3
        uint32_t lo02 = __builtin_amdgcn_perm(r[1].y, r[0].y, 0x05040100u);  // f2
        uint32_t hi02 = __builtin_amdgcn_perm(r[3].y, r[2].y, 0x05040100u);
        uint32_t lo13 = __builtin_amdgcn_perm(r[1].y, r[0].y, 0x07060302u);  // f3
        uint32_t hi13 = __builtin_amdgcn_perm(r[3].y, r[2].y, 0x07060302u);
        bf16_t* base = &sV[buf][d4 * VLD + 4 * kb4];
        *(uint2*)(base + 0 * VLD) = make_uint2(lo01, hi01);
        *(uint2*)(base + 1 * VLD) = make_uint2(lo11, hi11);
        *(uint2*)(base + 2 * VLD) = make_uint2(lo02, hi02);
        *(uint2*)(base + 3 * VLD) = make_uint2(lo13, hi13);
      }
    }
  };

  // Reference maximum of the exp2-domain scores per query column; the first
  // tile sets it, later tiles only raise it.
  float m_run[2] = {0.0f, 0.0f}, l_run[2] = {0.0f, 0.0f};
  floatx4 ainit[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};   // -m_run
  // ds_bpermute byte addresses of lanes xor 16 and xor 32
  const int bp16 = (lane ^ 16) << 2, bp32 = (lane ^ 32) << 2;
  floatx4 oacc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int ntiles = (T + KV - 1) / KV;
  if (tid == 0) zslot = make_uint4(0, 0, 0, 0);
  if (tid < 2 * KPAD / 8) *(uint4*)&sK[tid / (KPAD / 8)][KV * KLD + 8 * (tid % (KPAD / 8))] = make_uint4(0, 0, 0, 0);
  if constexpr (DMA) {
    // The (1, 0, .., 0) column chunk of every V row and the zero column chunk
    // of every K row of both buffers, once.
    for (int i = tid; i < 2 * KV; i += NTH) {
      *(uint4*)&sV[i / KV][(i % KV) * VS + DH] = make_uint4(0x3F80u, 0, 0, 0);
      *(uint4*)&sK[i / KV][(i % KV) * KLD + DH] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    if (ntiles == 1 && T % KV) dma(0, 0, std::true_type{});
    else dma(0, 0, std::false_type{});
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies have landed
  } else {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  // One 64-key tile; RAG: the last tile of a length that is not a multiple
  // of 64 (keys >= T masked).  For dh 72 only that one tile carries the
  // masking code; dh 64 tests at run time.
  auto tile = [&](int it, auto rag_c, auto next_rag_c) {
    constexpr bool RAG = decltype(rag_c)::value;
    const int buf = it & 1, kv0 = it * KV;
    if (it + 1 < ntiles) {                   // next tile in flight during this one
      if constexpr (DMA) dma(kv0 + KV, buf ^ 1, next_rag_c);
      else gload(kv0 + KV);
    }

    // S^T blocks: 4 key blocks x 2 query blocks of 16x16, in the exp2 domain
    // relative to the reference maximum: K (sl2 Q)^T - m_run (the
    // accumulators start at -m_run).
    floatx4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16_t* kr = &sK[buf][(16 * kb + c16) * KLD];
      bf16x8_t k0 = *(const bf16x8_t*)(kr + 8 * g);
      bf16x8_t k1 = *(const bf16x8_t*)(kr + 32 + 8 * g);
      // dh 64..95: lanes g > 0 read past dh 72 (the row's zero pad column, the
      // next row, or the zero pad after the last one); the query operand is
      // zero there, so the products only need those values finite
      bf16x8_t kt = z8;
      if constexpr (TAIL) kt = *(const bf16x8_t*)(kr + 64 + 8 * g);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        floatx4 a = ainit[qb];
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[qb][0], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[qb][1], a, 0, 0, 0);
        if constexpr (TAIL) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, qt[qb], a, 0, 0, 0);
        s[kb][qb] = a;
      }
    }
    if (RAG || (!DMA && kv0 + KV > T)) {     // ragged last tile: drop keys >= T
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kv0 + 16 * kb + 4 * g + r >= T) {
            s[kb][0][r] = -INFINITY;
            s[kb][1][r] = -INFINITY;
          }
    }

    // Online softmax in the exp2 domain.  Lane holds query column c16 of block
    // qb and keys 16 kb + 4 g + r; the 4 lanes sharing c16 combine by xor 16, 32.
    // The first tile sets the reference maximum m_run; later it is raised only
    // when some query's tile maximum exceeds it by RESCALE_SLACK, so P stays
    // <= 2^RESCALE_SLACK and O, l are rescaled rarely; l and O always share
    // the same reference.  The scores, relative to m_run, follow it.
    bf16x8_t pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      // the test needs each lane's own maximum only; the query column's (over
      // the 4 lanes sharing c16) is formed when the reference moves
      if (__any(it == 0 || mx > RESCALE_SLACK)) {
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(bp16, __float_as_int(mx))));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(bp32, __float_as_int(mx))));
        // key 0 lies in the first tile, so its maximum is finite
        const float delta = it == 0 ? mx : fmaxf(mx, 0.0f);
        m_run[qb] += delta;
        ainit[qb] = floatx4{-m_run[qb], -m_run[qb], -m_run[qb], -m_run[qb]};
        if (it > 0) {
          const float alpha = __builtin_amdgcn_exp2f(-delta);
          if constexpr (!DMA) l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[db][qb][r] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][qb][r] -= delta;
      }
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; kb += 2) {
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(s[kb][qb][r]);
          p[4 + r] = __builtin_amdgcn_exp2f(s[kb + 1][qb][r]);
        }
        if constexpr (!DMA)
#pragma unroll
          for (int r = 0; r < 8; ++r) ls += p[r];
        uint4 u = make_uint4(f2bf2(p[0], p[1]), f2bf2(p[2], p[3]), f2bf2(p[4], p[5]),
                             f2bf2(p[6], p[7]));
        pf[qb][kb >> 1] = __builtin_bit_cast(bf16x8_t, u);
      }
      if constexpr (!DMA) l_run[qb] += ls;
    }

    // O^T[dh, q] += V^T[dh, key] P^T[key, q]; key order within each 32-key step:
    // 4g..4g+3 of the even 16-block, then 4g..4g+3 of the odd one.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dr = 16 * db + c16;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t vf;
        if constexpr (DMA) {
          // Transposing reads: lane s of 16-lane group g points at
          // V[key 32 j + 4 g + s / 4 (+16)][d 16 db + 4 (s % 4)]; lane s then
          // holds d 16 db + s of keys 32 j + 4 g .. +3 (and 16 + those).
          const bf16_t* vb = &sV[buf][(32 * j + 4 * g + (c16 >> 2)) * VS + 16 * db + 4 * (c16 & 3)];
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)vb);
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(vb + 16 * VS));
          vf = __builtin_bit_cast(bf16x8_t, (__attribute__((ext_vector_type(8))) short){
                                                lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        } else {
          const bool in = dr < DH;
          const uint2 lo = *(const uint2*)(in ? &sV[buf][dr * VLD + 32 * j + 4 * g] : (const bf16_t*)&zslot);
          const uint2 hi = *(const uint2*)(in ? &sV[buf][dr * VLD + 32 * j + 16 + 4 * g] : (const bf16_t*)&zslot);
          vf = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb][j], oacc[db][qb], 0, 0, 0);
      }
    }

    // Stage the prefetched tile into the other buffer (last read in iteration it-1,
    // which every wave finished before the previous barrier).
    if constexpr (DMA) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next tile's copies have landed
    } else {
      if (it + 1 < ntiles) sstore(buf ^ 1);
    }
    __syncthreads();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (T % KV == 0 || !DMA) {           // (dh 64 keeps one loop body: registers)
    for (int it = 0; it < ntiles; ++it) tile(it, F_{}, F_{});
  } else {
    // only the copy of the ragged last tile clamps its rows, only that tile masks
    for (int it = 0; it + 2 < ntiles; ++it) tile(it, F_{}, F_{});
    if (ntiles >= 2) tile(ntiles - 2, F_{}, T_{});
    tile(ntiles - 1, T_{}, F_{});
  }

  // Normalise and store O[b, q, h*DH + dh] (token-major, heads concatenated).
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l;
    if constexpr (DMA) {
      l = __shfl(oacc[4][qb][0], 32 + c16, 64);   // O^T row 72: lane group 2, element 0
    } else {
      l = l_run[qb];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
    }
    const float inv = 1.0f / l;
    const int q = q0 + 16 * qb + c16;
    if (q >= T) continue;
    // natural-log log-sum-exp of the query's scaled scores: sum exp = 2^m_run l
    if (lse && g == 0) lse[(int64_t)bh * T_rows + q] = (m_run[qb] + log2f(l)) * 0.6931471805599453f;
    bf16_t* orow = O + (tok0 + q) * H * DH + h * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      int d0 = 16 * db + 4 * g;
      if (d0 + 3 < DH)
        *(uint2*)(orow + d0) = make_uint2(f2bf2(oacc[db][qb][0] * inv, oacc[db][qb][1] * inv),
                                          f2bf2(oacc[db][qb][2] * inv, oacc[db][qb][3] * inv));
    }
  }
}

// Short sequences (T <= 256, dh = 72): one workgroup of 8 waves owns every
// query of one (row, head), 32 per wave, with the sequence's K and V resident
// in LDS.  Workgroups are persistent over the (row, head) pairs; the next
// pair's K, V and this wave's next queries are loaded into registers while
// the current pair computes and are written to LDS between two barriers.
// Per 64-key tile: S^T = K Q^T (24 MFMAs), exp2-domain weights, O^T += V^T
// P^T (20 MFMAs).  V sits in LDS with a row stride of 80 whose column 72 is 1
// and 73..79 are 0, so O^T row 72 is the sum of the (bf16) weights
// themselves: the normaliser comes out of the same products as the
// numerator.

// NT = ceil(T / 64) key tiles; RAG: T is not a multiple of 64 (mask keys >= T)
template <int NT, bool RAG>
__global__ __launch_bounds__(512) void attn_short_kernel(const bf16_t* __restrict__ QKV,
                                                         bf16_t* __restrict__ O, int H, int T,
                                                         int npairs, float sl2) {
  constexpr int DH = 72, NWV = 8, KS = 80, VS = 80, NDB = 5;
  constexpr int NCH = 256 * (DH / 8);               // 16-byte chunks of K (or V) per pair
  constexpr int CPT = (NCH + 64 * NWV - 1) / (64 * NWV);
  // 24 zero elements after K's last row: the dh 64..95 operand reads of the
  // last rows reach into them (see s_tile)
  __shared__ __attribute__((aligned(16))) bf16_t sK[256 * KS + 24];
  __shared__ __attribute__((aligned(16))) bf16_t sV[256 * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t ld = 3LL * H * DH;                  // packed row stride
  const int q0 = 32 * wave;
  const bf16x8_t z8 = {};

  // K / V chunk u of this thread: chunk c = tid + 512 u is row c / 9, 16-byte
  // column c % 9 (rows past T read row T - 1: finite data whose weights are 0)
  // In LDS, K and V chunk c sit at element 8 (c + c / 9): rows of 80, one
  // pad chunk per row (zeros in K, so that the 16 rows x 2 chunks of a
  // fragment read fall on distinct banks; (1, 0, .., 0) in V).  Offsets are
  // recomputed at each use rather than held in registers across the pair.
  const int ldb = (int)(ld * 2);
  static_assert(KS == DH + 8 && VS == DH + 8, "LDS row strides");
  const int nrec = (int)(((int64_t)(T - 1) * ld + DH) * 2);
  uint4 kreg[CPT], vreg[CPT];
  auto gload = [&](int p) {
    const int b = p / H, h = p - b * H;
    const bf16_t* Kb = QKV + (int64_t)b * T * ld + (int64_t)(H + h) * DH;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kb, (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kb + (int64_t)H * DH), (short)0, nrec, 0x00020000);
    int t0 = tid;
    asm volatile("" : "+v"(t0));
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = min(t0 + 64 * NWV * u, NCH - 1);
      const int row = c / (DH / 8), col = c - row * (DH / 8);
      const int off = min(row, T - 1) * ldb + col * 16;
      kreg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
      vreg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
    }
  };
  auto sstore = [&]() {
    int t0 = tid;
    asm volatile("" : "+v"(t0));       // keep the address arithmetic here (not hoisted and spilled)
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      if (t0 + 64 * NWV * u < NCH) {
        const int c = t0 + 64 * NWV * u;
        *(uint4*)&sK[8 * (c + c / (DH / 8))] = kreg[u];
        *(uint4*)&sV[8 * (c + c / (DH / 8))] = vreg[u];
      }
  };
  // This wave's 32 queries as MFMA B operands: dh 0..63 in qf, dh 64..71 in
  // qt.  The loads are unconditional (row clamped to T - 1; lanes g > 0 of
  // the tail read dh 72..95, inside the packed row); the selects that zero
  // queries >= T and tail lanes g > 0 run when the pair starts.
  auto load_q = [&](int p, bf16x8_t (&qf)[2][2], bf16x8_t (&qt)[2]) {
    const int b = p / H, h = p - b * H;
    const bf16_t* Qb = QKV + (int64_t)b * T * ld + h * DH;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const bf16_t* qr = Qb + (int64_t)min(q0 + 16 * qb + c16, T - 1) * ld;
#pragma unroll
      for (int c = 0; c < 2; ++c) qf[qb][c] = *(const bf16x8_t*)(qr + 32 * c + 8 * g);
      qt[qb] = *(const bf16x8_t*)(qr + 64 + 8 * g);
    }
  };

  // Workgroup w runs on XCD w % 8 (round-robin dispatch).  With a grid that
  // is a multiple of 8, XCD x takes the logical slots x G/8 .. (x+1) G/8 - 1,
  // so the pairs it runs together are consecutive heads of the same rows:
  // the cache lines that neighbouring heads' 144-byte slices share are
  // fetched (and written) once, through that XCD's L2.
  const int G = gridDim.x;
  int pair = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  if (pair >= npairs) return;
  if (tid < 256) {
    *(uint4*)&sV[tid * VS + DH] = make_uint4(0x3F80u, 0, 0, 0);   // (1, 0, .., 0)
    *(uint4*)&sK[tid * KS + DH] = make_uint4(0, 0, 0, 0);
  }
  if (tid < 3) *(uint4*)&sK[256 * KS + 8 * tid] = make_uint4(0, 0, 0, 0);
  bf16x8_t qn[2][2], qtn[2];
  load_q(pair, qn, qtn);
  gload(pair);
  sstore();
  __syncthreads();

  for (;;) {
    const int next = pair + G;
    bf16x8_t qf[2][2], qt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const bool ok = q0 + 16 * qb + c16 < T;
      qf[qb][0] = ok ? qn[qb][0] : z8;
      qf[qb][1] = ok ? qn[qb][1] : z8;
      qt[qb] = ok && g == 0 ? qtn[qb] : z8;
    }
    if (next < npairs) gload(next);    // in flight while this pair computes

    floatx4 oacc[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // S^T[key, q] of 64-key tile t: 4 key blocks x 2 query blocks of 16 x 16
    auto s_tile = [&](int t, floatx4 (&sa)[4][2]) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16_t* kr = sK + (64 * t + 16 * kb + c16) * KS;
        const bf16x8_t k0 = *(const bf16x8_t*)(kr + 8 * g);
        const bf16x8_t k1 = *(const bf16x8_t*)(kr + 32 + 8 * g);
        // dh 64..95: lanes g > 0 read past dh 72 (the row's zero pad column,
        // the next row, or the zero pad after the last one); their query
        // operand is zero, so the products only need those values finite
        const bf16x8_t kt = *(const bf16x8_t*)(kr + 64 + 8 * g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[qb][0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[qb][1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, qt[qb], acc, 0, 0, 0);
          sa[kb][qb] = acc;
        }
      }
      if (RAG && t == NT - 1) {        // keys >= T of the ragged last tile
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool out = 64 * t + 16 * kb + 4 * g + r >= T;
            sa[kb][0][r] = out ? -INFINITY : sa[kb][0][r];
            sa[kb][1][r] = out ? -INFINITY : sa[kb][1][r];
          }
      }
    };
    // O^T[d, q] += V^T[d, key] P^T[key, q] for tile t.  Key order inside a
    // 32-key block j follows the weights: lane group g holds keys 4 g .. + 3
    // and 16 + those.  Transposing reads: lane s of group g points at
    // V[key 32 j + 4 g + s / 4 (+16)][d 16 db + 4 (s % 4)] and receives d
    // 16 db + s of those 4 keys.
    auto pv_tile = [&](int t, const bf16x8_t (&pw)[2][2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16_t* vb = sV + (64 * t + 32 * j + 4 * g + (c16 >> 2)) * VS + 4 * (c16 & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(vb + 16 * db));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(vb + 16 * VS + 16 * db));
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, (__attribute__((ext_vector_type(8))) short){lo[0], lo[1], lo[2], lo[3],
                                                                    hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pw[qb][j], oacc[db][qb],
                                                                   0, 0, 0);
        }
      }
    };
    // scaled (exp2-domain) maximum of a tile's scores for query block qb
    auto tile_max = [&](const floatx4 (&sa)[4][2], int qb) {
      float mx = sa[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sa[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      return mx * sl2;
    };

    // Software pipeline over the tiles: the MFMAs of PV(t-1) are issued among
    // the maxima of tile t and those of S(t+1) among its weights, so that one
    // wave keeps the matrix cores and the VALU busy together.  Weights are
    // exp2(s sl2 - m_ref) against a reference maximum that is raised (and the
    // output rescaled) only when a tile's maximum exceeds it by more than
    // 2^RESCALE_SLACK, which keeps the weights finite and rarely branches.
    constexpr float RESCALE_SLACK = 8.0f;
    float m_ref[2];
    floatx4 sc[4][2], sn[4][2];
    bf16x8_t pw[2][2];
    s_tile(0, sc);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t > 0) pv_tile(t - 1, pw);
      const float mx0 = tile_max(sc, 0), mx1 = tile_max(sc, 1);
      if (t == 0) {
        m_ref[0] = mx0;
        m_ref[1] = mx1;
      } else if (__any(mx0 > m_ref[0] + RESCALE_SLACK || mx1 > m_ref[1] + RESCALE_SLACK)) {
        const float mx[2] = {mx0, mx1};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = fmaxf(m_ref[qb], mx[qb]);
          const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
          m_ref[qb] = m_new;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[db][qb][r] *= alpha;
        }
      }
      if (t + 1 < NT) s_tile(t + 1, sn);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mneg = -m_ref[qb];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float pv[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pv[r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * j][qb][r], sl2, mneg));
            pv[4 + r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * j + 1][qb][r], sl2, mneg));
          }
          const uint4 u = make_uint4(f2bf2(pv[0], pv[1]), f2bf2(pv[2], pv[3]),
                                     f2bf2(pv[4], pv[5]), f2bf2(pv[6], pv[7]));
          pw[qb][j] = __builtin_bit_cast(bf16x8_t, u);
        }
      }
      if (t + 1 < NT) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          sc[kb][0] = sn[kb][0];
          sc[kb][1] = sn[kb][1];
        }
      }
    }
    // the next queries are loaded once the scores are dead (fewer live
    // registers); the last products, the stores and the barriers cover them
    if (next < npairs) load_q(next, qn, qtn);
    pv_tile(NT - 1, pw);

    // O^T row 72 (block 4, lane group 2, element 0) is the sum of the weights
    // of query c16: divide and store O[b, q, h*DH + d]
    {
      const int b = pair / H, h = pair - b * H;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float l = __shfl(oacc[4][qb][0], 32 + c16, 64);
        const float inv = 1.0f / l;
        const int q = q0 + 16 * qb + c16;
        if (q >= T) continue;
        bf16_t* orow = O + ((int64_t)b * T + q) * H * DH + h * DH;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d0 = 16 * db + 4 * g;
          if (d0 + 3 < DH)
            *(uint2*)(orow + d0) = make_uint2(f2bf2(oacc[db][qb][0] * inv, oacc[db][qb][1] * inv),
                                              f2bf2(oacc[db][qb][2] * inv, oacc[db][qb][3] * inv));
        }
      }
    }
    if (next >= npairs) break;
    __syncthreads();                   // every wave is done with this pair's K and V
    sstore();
    __syncthreads();
    pair = next;
  }
}

template <int DH, bool PK = false>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ QKV,
                                                      float* __restrict__ O, int H, int T_rows,
                                                      float scale, SeqTable seqs,
                                                      float* __restrict__ lse) {
  constexpr int KT = 32;
  __shared__ float sK[KT][DH], sV[KT][DH];
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  int qblk = blockIdx.x;
  int T = T_rows;
  int64_t tok0 = (int64_t)b * T_rows;
  if constexpr (PK) {   // grid (query blocks of all sequences, heads)
    int j = 0;
    while (j + 1 < seqs.n && seqs.blk[j + 1] <= qblk) ++j;
    qblk -= seqs.blk[j];
    tok0 = seqs.tok[j];
    T = seqs.tok[j + 1] - seqs.tok[j];
  }
  const int qi = qblk * 64 + threadIdx.x;
  const int64_t ld = 3LL * H * DH;
  const float* Qb = QKV + tok0 * ld + h * DH;
  const float* Kb = Qb + (int64_t)H * DH;
  const float* Vb = Qb + 2LL * H * DH;
  float qv[DH], acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    qv[e] = qi < T ? Qb[qi * ld + e] : 0.0f;
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int kv0 = 0; kv0 < T; kv0 += KT) {
    __syncthreads();
    for (int e = threadIdx.x; e < KT * DH; e += 64) {
      int r = e / DH, c = e - r * DH;
      bool ok = kv0 + r < T;
      sK[r][c] = ok ? Kb[(kv0 + r) * ld + c] : 0.0f;
      sV[r][c] = ok ? Vb[(kv0 + r) * ld + c] : 0.0f;
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
    if (lse) lse[(int64_t)bh * T_rows + qi] = m + logf(l);
    float* orow = O + (tok0 + qi) * H * DH + h * DH;
    float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DH; ++e) orow[e] = acc[e] * inv;
  }
}

}  // namespace

// one resident workgroup of the short-sequence kernel per CU (8 waves of up
// to 256 VGPRs fill a CU's register file)
constexpr int kShortSlots = 256;

hipError_t launch_attention(const void* qkv, int B, int heads, int T, int dh, int dtype, void* o,
                            hipStream_t s, float* lse) {
  if (B <= 0 || T <= 0) return hipSuccess;
  if (dtype == 1) {
    const float sl2 = 1.4426950408889634f / sqrtf((float)dh);
    // 4 waves (128 queries) per workgroup (8 waves of 256 queries measured
    // slower at every length).  When T leaves a mostly empty last block of
    // 128 queries (T = 258 with two conditioning tokens), 3 or 2 waves per
    // workgroup waste fewer query slots: pick the fewest wasted, then the most
    // waves.
    int nwv = 4;
    int64_t best = (T + 127) / 128 * 128 - T;
    for (int c : {3, 2}) {
      const int64_t waste = (T + 32 * c - 1) / (32 * c) * (32 * c) - T;
      if (waste < best) { best = waste; nwv = c; }
    }
    if (dh != 64 && dh != 72) return hipErrorInvalidValue;
    if (dh == 72 && T <= 256 && !lse) {
      // whole sequences resident in LDS, persistent over the (row, head) pairs
      const int npairs = B * heads;
      const int grid = npairs < kShortSlots ? npairs : kShortSlots;
#define DIT_SHORT(NT, RAG)                                                                    \
  attn_short_kernel<NT, RAG><<<grid, 512, 0, s>>>((const bf16_t*)qkv, (bf16_t*)o, heads, T, npairs, sl2)
      const bool rag = T % 64 != 0;
      switch ((T + 63) / 64) {
        case 1: if (rag) DIT_SHORT(1, true); else DIT_SHORT(1, false); break;
        case 2: if (rag) DIT_SHORT(2, true); else DIT_SHORT(2, false); break;
        case 3: if (rag) DIT_SHORT(3, true); else DIT_SHORT(3, false); break;
        default: if (rag) DIT_SHORT(4, true); else DIT_SHORT(4, false); break;
      }
#undef DIT_SHORT
      return hipGetLastError();
    }
    SeqTable none;
    none.n = 0;
#define DIT_ATTN_LAUNCH(NWV)                                                                  \
  {                                                                                           \
    dim3 grid((T + 32 * NWV - 1) / (32 * NWV), B * heads);                                    \
    if (dh == 64)                                                                             \
      attn_bf16_kernel<64, NWV><<<grid, 64 * NWV, 0, s>>>((const bf16_t*)qkv, (bf16_t*)o,     \
                                                          heads, T, sl2, none, lse);          \
    else                                                                                      \
      attn_bf16_kernel<72, NWV><<<grid, 64 * NWV, 0, s>>>((const bf16_t*)qkv, (bf16_t*)o,     \
                                                          heads, T, sl2, none, lse);          \
  }
    if (nwv == 4) DIT_ATTN_LAUNCH(4)
    else if (nwv == 3) DIT_ATTN_LAUNCH(3)
    else DIT_ATTN_LAUNCH(2)
#undef DIT_ATTN_LAUNCH
  } else {
    const float scale = 1.0f / sqrtf((float)dh);
    dim3 grid((T + 63) / 64, B * heads);
    SeqTable none;
    none.n = 0;
    if (dh == 64)
      attn_f32_kernel<64><<<grid, 64, 0, s>>>((const float*)qkv, (float*)o, heads, T, scale, none,
                                              lse);
    else if (dh == 72)
      attn_f32_kernel<72><<<grid, 64, 0, s>>>((const float*)qkv, (float*)o, heads, T, scale, none,
                                              lse);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_packed(const void* qkv, const SeqTable& seqs_in, int heads, int dh,
                                   int dtype, void* o, hipStream_t s) {
  if (seqs_in.n <= 0 || seqs_in.n > kMaxSeq) return hipErrorInvalidValue;
  if (dh != 64 && dh != 72) return hipErrorInvalidValue;
  SeqTable seqs = seqs_in;
  const int QPB = dtype == 1 ? 128 : 64;   // queries per workgroup
  seqs.blk[0] = 0;
  for (int j = 0; j < seqs.n; ++j)
    seqs.blk[j + 1] = seqs.blk[j] + (seqs.tok[j + 1] - seqs.tok[j] + QPB - 1) / QPB;
  if (dtype != 1) {
    const float scale = 1.0f / sqrtf((float)dh);
    dim3 grid(seqs.blk[seqs.n], heads);
    if (dh == 64)
      attn_f32_kernel<64, true><<<grid, 64, 0, s>>>((const float*)qkv, (float*)o, heads, 0,
                                                    scale, seqs, nullptr);
    else
      attn_f32_kernel<72, true><<<grid, 64, 0, s>>>((const float*)qkv, (float*)o, heads, 0,
                                                    scale, seqs, nullptr);
    return hipGetLastError();
  }
  constexpr int NWV = 4;
  const float sl2 = 1.4426950408889634f / sqrtf((float)dh);
  dim3 grid(seqs.blk[seqs.n], heads);
  if (dh == 64)
    attn_bf16_kernel<64, NWV, true><<<grid, 64 * NWV, 0, s>>>((const bf16_t*)qkv, (bf16_t*)o,
                                                              heads, 0, sl2, seqs, nullptr);
  else
    attn_bf16_kernel<72, NWV, true><<<grid, 64 * NWV, 0, s>>>((const bf16_t*)qkv, (bf16_t*)o,
                                                              heads, 0, sl2, seqs, nullptr);
  return hipGetLastError();
}

namespace {
__global__ void fill_int_kernel(int* __restrict__ out, int64_t n, int v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = v;
}
}  // namespace

hipError_t launch_fill_int(int* out, int64_t n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_int_kernel<<<(int)((n + 255) / 256), 256, 0, s>>>(out, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cross-attention of every token over the two context tokens of its row (the
// cross-attention conditioning design): per head, softmax over two scores.
// One thread per (token, head), 16-byte loads and stores; fp32 arithmetic.
namespace {
// 16 bytes of DT as floats: 8 bf16 or 4 fp32.
template <typename DT> struct Vec16;
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* f) {
    const uint4 u = *(const uint4*)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* f) {
    uint4 u;
    u.x = f2bf2(f[0], f[1]); u.y = f2bf2(f[2], f[3]);
    u.z = f2bf2(f[4], f[5]); u.w = f2bf2(f[6], f[7]);
    *(uint4*)p = u;
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* f) {
    const float4 v = *(const float4*)p;
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* f) {
    *(float4*)p = make_float4(f[0], f[1], f[2], f[3]);
  }
};

template <typename DT, int DH>
__global__ __launch_bounds__(256) void cross_attn2_kernel(const DT* __restrict__ q,
                                                          const DT* __restrict__ kv,
                                                          int64_t kv_stride, int64_t n, int T,
                                                          int heads, DT* __restrict__ o) {
  using V = Vec16<DT>;
  constexpr int NC = DH / V::N;
  static_assert(DH % V::N == 0, "head dim");
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int h = (int)(idx % heads);
  const int64_t m = idx / heads;
  const int64_t b = m / T;
  const int D = heads * DH;
  const DT* qp = q + m * D + h * DH;
  const DT* k0 = kv + (b * 2) * kv_stride + h * DH;
  const DT* k1 = k0 + kv_stride;
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float a[V::N], x0[V::N], x1[V::N];
    V::load(qp + c * V::N, a);
    V::load(k0 + c * V::N, x0);
    V::load(k1 + c * V::N, x1);
#pragma unroll
    for (int i = 0; i < V::N; ++i) {
      s0 = fmaf(a[i], x0[i], s0);
      s1 = fmaf(a[i], x1[i], s1);
    }
  }
  const float scale = 1.0f / sqrtf((float)DH);
  s0 *= scale;
  s1 *= scale;
  const float mx = fmaxf(s0, s1);
  const float e0 = expf(s0 - mx), e1 = expf(s1 - mx);
  const float inv = 1.0f / (e0 + e1);
  const float p0 = e0 * inv, p1 = e1 * inv;
  DT* op = o + m * D + h * DH;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float v0[V::N], v1[V::N], r[V::N];
    V::load(k0 + D + c * V::N, v0);
    V::load(k1 + D + c * V::N, v1);
#pragma unroll
    for (int i = 0; i < V::N; ++i) r[i] = fmaf(p0, v0[i], p1 * v1[i]);
    V::store(op + c * V::N, r);
  }
}

template <typename DT>
hipError_t cross2_dispatch(const void* q, const void* kv, int64_t kv_stride, int rows, int T,
                           int heads, int dh, void* o, hipStream_t s) {
  const int64_t n = (int64_t)rows * T * heads;
  const int blocks = (int)((n + 255) / 256);
  if (dh == 72)
    cross_attn2_kernel<DT, 72><<<blocks, 256, 0, s>>>((const DT*)q, (const DT*)kv, kv_stride, n,
                                                     T, heads, (DT*)o);
  else if (dh == 64)
    cross_attn2_kernel<DT, 64><<<blocks, 256, 0, s>>>((const DT*)q, (const DT*)kv, kv_stride, n,
                                                     T, heads, (DT*)o);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
}  // namespace

hipError_t launch_cross_attention2(const void* q, const void* kv, int64_t kv_stride, int rows,
                                   int T, int heads, int dh, int dtype, void* o, hipStream_t s) {
  if (rows <= 0 || T <= 0) return hipSuccess;
  return dtype == 1 ? cross2_dispatch<bf16_t>(q, kv, kv_stride, rows, T, heads, dh, o, s)
                    : cross2_dispatch<float>(q, kv, kv_stride, rows, T, heads, dh, o, s);
}
