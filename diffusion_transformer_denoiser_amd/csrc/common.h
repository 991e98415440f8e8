// Shared device helpers and launcher declarations for the DiT forward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bfloat16 bits

// bf16 <-> fp32.  fp32 -> bf16 rounds to nearest even (gfx950's
// v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// exp2 and reciprocal on the hardware units (v_exp_f32, v_rcp_f32: ~1 ulp).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float silu_f(float z) {
  return z * fast_rcp(1.0f + fast_exp2(-1.4426950408889634f * z));
}
// tanh-approximate GELU: 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated through the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)).
// d/dz of the tanh-GELU: with s = sigmoid(2u) = (1 + tanh u) / 2,
// u = sqrt(2/pi)(z + 0.044715 z^3): s + 2 z s (1 - s) du/dz.
__device__ __forceinline__ float gelu_tanh_grad_f(float z);

__device__ __forceinline__ float gelu_tanh_f(float z) {
  const float k2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float k3 = k2 * 0.044715f;
  const float u2 = z * fmaf(z * z, k3, k2);                             // -2u log2(e)
  return z * fast_rcp(1.0f + fast_exp2(u2));
}

__device__ __forceinline__ float gelu_tanh_grad_f(float z) {
  const float k = 0.7978845608028654f;
  const float k2 = -2.0f * k * 1.4426950408889634f;
  const float sg = fast_rcp(1.0f + fast_exp2(z * fmaf(z * z, k2 * 0.044715f, k2)));
  return sg + 2.0f * z * sg * (1.0f - sg) * k * fmaf(3.0f * 0.044715f, z * z, 1.0f);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Patch index maps (shared by the gather prologue of the patch embedding, the
// standalone patchify kernel and the unpatchify kernel).
struct PatchGeom {
  int C, F, H, W, p, pt;  // latent extents and patch sizes
  int gh, gw, T, K;       // token grid rows/cols, tokens per row, patch vector length
};

// Offset into a [.., C, F, H, W] latent row for token tau and patch element k.
__device__ __forceinline__ int64_t patch_src_offset(const PatchGeom& g, int tau, int k) {
  int ghw = g.gh * g.gw;
  int f = tau / ghw, rem = tau - f * ghw;
  int i = rem / g.gw, j = rem - i * g.gw;
  int c = k % g.C, r = k / g.C;
  int px = r % g.p; r /= g.p;
  int py = r % g.p; int a = r / g.p;
  return (((int64_t)c * g.F + (f * g.pt + a)) * g.H + (i * g.p + py)) * g.W + (j * g.p + px);
}

// ---------------------------------------------------------------------------
// GEMM epilogues.  C = A W^T computed in fp32; the epilogue consumes C[m, n].
enum EpiKind {
  EPI_BIAS_F32 = 0,     // out_f32[m, n] = C + bias[n]
  EPI_BIAS_SILU = 1,    // out_f32[m, n] = SiLU(C + bias[n])                   (timestep MLP)
  EPI_COND = 2,         // c = C + bias (+ c_prev) (+ table[label]); writes c and SiLU(c) (dtype)
  EPI_BIAS_DT = 3,      // out_dtype[m, n] = C + bias[n]            (packed q | k | v)
  EPI_GATED = 4,        // X[m, n] += gate[b, n] * (C + bias[n]) (fp32 residual; gate 1 if mod null)
  EPI_GELU = 5,         // out_dtype[m, n] = GELU_tanh(C + bias[n])
  EPI_PATCH = 6,        // X[m + (m / T) out_skip, n] = C + bias[n] (+ pe_tab[m % T, n])
  EPI_SILU_DT = 7,      // out_dtype[m, n] = SiLU(C + bias[n])                  (timestep MLP)
  EPI_ATOMIC_F32 = 8,   // out_f32[m, n] += C, atomically (split-K partial sums; bias null)
  EPI_GELU2 = 9,        // out_dtype[m, n] = GELU_tanh(C + bias[n]); aux_dtype[m, n] = C + bias[n]
  EPI_DGELU = 10,       // out_dtype[m, n] = (C + bias[n]) GELU_tanh'(aux_dtype[m, n])
};

struct EpiParams {
  const float* bias;
  void* out;            // output (type depends on the epilogue)
  int ldo;              // leading dimension of out (elements)
  // gated residual: gate = mod + (m / T) * mod_stride + gate_off
  const float* mod;
  int mod_stride;
  int gate_off;
  int T;                // tokens per row (rows of A per batch row)
  // conditioning
  const float* table;   // class table [ncls + 1, d] or null
  const int32_t* labels;
  int label_rows;       // rows of `labels` (source rows); row b reads labels[b % label_rows]
  int null_from;        // rows b >= null_from use the null label
  int ncls;
  int add_prev;         // 1: add the current content of out (pooled projection)
  void* silu_out;       // SiLU(c) in the GEMM operand dtype
  // patch embedding position term: table [T, ldo] of the 2-D sin-cos embedding
  const float* pe_tab;
  // patch embedding: rows of out skipped after every T rows (extra tokens of a row)
  int out_skip;
  // gated residual of packed sequences: the gate row of output row m is
  // tok_seg[m] (sequences start at multiples of 32 rows); else m / T
  const int* tok_seg;
  // Row maps (0 = identity): GEMM row m reads A row a_map(m) and the bias /
  // bf16 epilogues write out row o_map(m), with
  // map(m) = m + (m / seg) * skip + off.  They interleave two token streams
  // of a row (MMDiT: text tokens, then image tokens) in one buffer.
  int a_seg, a_skip, a_off;
  int o_seg, o_skip, o_off;
  // Row stride of W in elements (0: K).  Split-K: with ksplit > 0 the
  // reduction is cut into slices of ksplit (the last one shorter), one grid
  // layer each, whose partial sums the EPI_ATOMIC_F32 epilogue adds up.
  int ldw;
  int ksplit;
  // EPI_GELU2: the pre-activation output; EPI_DGELU: the pre-activation input
  // (model dtype, row stride ldo)
  void* aux;
  // VALU kernel only: W element (n, k) at W[k * ldw + n] (stored transposed)
  int w_trans;
};

// (m < 2^31 and seg > 0: 32-bit unsigned division)
__device__ __host__ __forceinline__ int64_t row_map(int64_t m, int seg, int skip, int off) {
  return seg ? m + (int64_t)((uint32_t)m / (uint32_t)seg) * skip + off : m;
}

// ---------------------------------------------------------------------------
// Launchers (each returns hipGetLastError() after the launch).
hipError_t launch_timestep_embed(const float* t, int rows, int src_rows, int dim, float* e,
                                 hipStream_t s);
// Same sinusoid rounded to bf16 (operand of the bf16 timestep MLP).
hipError_t launch_timestep_embed_bf16(const float* t, int rows, int src_rows, int dim, bf16_t* e,
                                      hipStream_t s);
// pe[tau, n] = 2-D sin-cos position embedding of token tau of a gh x gw grid, d wide.
hipError_t launch_pos_embed_table(int gh, int gw, int d, float* pe, hipStream_t s);
// c[m, :] += table[label(m), :] (+ pooled[m, :]); sc = SiLU(c) in dtype.  label(m) is
// the null label ncls for m >= null_from, else labels[m % label_rows]; a label
// outside [0, ncls] makes the row NaN.
hipError_t launch_cond_finish(float* c, int rows, int d, const float* table, const int32_t* labels,
                              int label_rows, int null_from, int ncls, const float* pooled,
                              void* sc, int dtype, hipStream_t s);
hipError_t launch_patchify(const void* x, int B, const PatchGeom& g, int dtype, void* P,
                           hipStream_t s);
// X[m + (m / T) out_skip, :] = patch vector of token m (gathered from the
// latent x of src_rows rows; row b of the tokens reads latent row b % src_rows)
// times W^T + bias (+ pe[m % T, :]).  W [d, g.K] and x in `dtype`; X fp32.
hipError_t launch_patch_embed(const void* x, int src_rows, const PatchGeom& g, int dtype,
                              const void* W, const float* bias, const float* pe, int M, int d,
                              int out_skip, float* X, hipStream_t s);
// Conditioning tokens of the in-context and cross-attention designs: for trunk
// row r, the time embedding temb[r] and the class embedding table[label(r)]
// (label(r) as in launch_cond_finish; a label out of range gives NaN).
// mode 0: X[r, T, :] = temb[r], X[r, T + 1, :] = class row (fp32 residual
// stream, rows of T + 2 tokens); mode 1: ctx[r, 0, :], ctx[r, 1, :] in dtype.
hipError_t launch_cond_tokens(const float* temb, int rows, int d, const float* table,
                              const int32_t* labels, int label_rows, int null_from, int ncls,
                              int mode, void* dst, int T, int dtype, hipStream_t s);
// Cross-attention over two context tokens per row: q [rows * T, H * dh] and
// o [rows * T, H * dh] in dtype; context token j of row b has its keys at
// kv + (2 b + j) * kv_stride and its values H * dh elements further on
// (kv_stride in elements, a multiple of 8; all offsets 16-byte aligned).
hipError_t launch_cross_attention2(const void* q, const void* kv, int64_t kv_stride, int rows,
                                   int T, int heads, int dh, int dtype, void* o, hipStream_t s);
hipError_t launch_unpatchify(const float* Y, int Bout, int Bh_offset, const PatchGeom& g,
                             int Cout, int guided, float scale, int guide, float* out,
                             hipStream_t s);

// A-operand sources of the VALU GEMM.
enum ASrc { A_PLAIN = 0, A_PATCH = 1 };
struct ALoad {
  const void* ptr;      // A matrix (or latent for A_PATCH)
  int lda;
  int a_dtype;          // 0 fp32, 1 bf16
  int src_rows;         // A_PLAIN: row r reads row r % src_rows; A_PATCH: latent rows
  PatchGeom g;          // A_PATCH only
  int seg, skip, off;   // A_PLAIN: row map of the source row (see EpiParams), 0 = identity
  int trans;            // A_PLAIN: element (m, k) at ptr[k * lda + m] (the operand stored transposed)
};
// out[i, j] += sum_r A[r, i] B[r, j] (fp32, atomically): A [R, Mi] and B [R, Nj]
// bf16, row strides lda, ldb; Mi, Nj multiples of 8, R a multiple of 64,
// 16-byte aligned.  The weight gradient of a layer from its row-major input
// and output gradient.  asum (optional): asum[i] += sum_r A[r, i], the bias
// gradient, also atomically.
hipError_t launch_gemm_tn(const bf16_t* A, int lda, const bf16_t* B, int ldb, int Mi, int Nj,
                          int R, float* out, int ldo, float* asum, hipStream_t s);
hipError_t launch_gemm_valu(int epi, int asrc, const ALoad& a, const void* W, int w_dtype,
                            int M, int N, int K, const EpiParams& ep, hipStream_t s);
// 128-row tiles of an M x N product on the 128 x 192 (or 128 x 128) MFMA kernel.
int64_t mfma_tiles_128(int64_t M, int64_t N);
hipError_t launch_gemm_mfma(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N,
                            int K, const EpiParams& ep, hipStream_t s);
// The wide-tile kernel (256-row tiles, one workgroup per CU) for the large
// block products; launch_gemm_mfma picks it when the shape fills the chip.
bool gemm_wide_supported(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N, int K,
                         const EpiParams& ep);
hipError_t launch_gemm_wide(int epi, const bf16_t* A, int lda, const bf16_t* W, int M, int N,
                            int K, const EpiParams& ep, hipStream_t s);

// Row m's modulation row is tok_seg[m] when tok_seg is given (packed
// sequences), else m / T.
hipError_t launch_ln_modulate(const float* X, int M, int T, int d, const float* mod,
                              int mod_stride, int shift_off, int scale_off, float eps,
                              void* H, int dtype, hipStream_t s, const int* tok_seg = nullptr);
hipError_t launch_qk_norm_rope(void* qkv, int B, int heads, int T, int dh, int dtype,
                               int qk_norm, float eps, int rope, int gh, int gw, hipStream_t s);
// lse (optional, [B heads T]): natural-log log-sum-exp of each query's scaled
// scores, for the backward pass.
hipError_t launch_attention(const void* qkv, int B, int heads, int T, int dh, int dtype, void* o,
                            hipStream_t s, float* lse = nullptr);
// RMSNorm with scale 1 + g of every head's q and k in the packed qkv [B*T, 3
// H dh], in place: tokens t < L of a row use g4[2], g4[3] (q, k), the others
// g4[0], g4[1] (g4 [4, dh]).
hipError_t launch_qk_rms(void* qkv, int B, int heads, int T, int L, int dh, int dtype, float eps,
                         const float* g4, hipStream_t s);

// Packed sequences: sequence j owns tokens [tok[j], tok[j + 1]) of the packed
// rows; attention stays inside each sequence (block-diagonal).  At most
// kMaxSeq sequences; the table travels by value in the kernel arguments.
constexpr int kMaxSeq = 64;
struct SeqTable {
  int n;
  int tok[kMaxSeq + 1];   // token offsets, tok[0] = 0
  int blk[kMaxSeq + 1];   // query-block offsets (filled by the attention launcher)
};
hipError_t launch_attention_packed(const void* qkv, const SeqTable& seqs, int heads, int dh,
                                   int dtype, void* o, hipStream_t s);
// out[i] = v for i in [0, n)
hipError_t launch_fill_int(int* out, int64_t n, int v, hipStream_t s);

static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// Sampler update (sampler.hip).  kind 0: DDPM ancestral step
//   x' = k0 x - k1 eps [+ exp(0.5 lv) z],  lv = fr k2 + (1 - fr) k3,
//   fr = (v + 1) / 2 from the covariance channel C + c when `learned`, else lv = k3;
// kind 1: DPM-Solver++ step  x0 = k0 x - k1 eps,  x' = k2 x + k3 x0 [+ k4 hist],
//   hist <- x0;
// kind 2: rectified-flow Euler  x' = x + k0 v.
// The prediction comes from `mo` as [B, Cout, S] (from_y == 0) or from the
// decoder output [rows, T, Kout] (from_y == 1) with the guidance combine of
// rows b and b + null_off on channels < guided.
struct SamplerStepArgs {
  int kind;
  int from_y;
  const float* x;       // [B, C, S] state
  float* x_out;         // [B, C, S] (may alias x)
  void* x_model;        // bf16 copy of x_out, or null
  const float* mo;      // prediction
  const float* z;       // [B, C, S] noise (kind 0 with add_noise)
  float* hist;          // [B, C, S] x0 history (kind 1), or null
  float* tvec;          // tvec[0..tvec_rows) = t_next (next model time), or null
  int tvec_rows;
  float t_next;
  int64_t n;            // B * C * S
  int64_t S;            // F * H * W
  int C, Cout;
  PatchGeom g;          // decoder geometry (from_y)
  int null_off, guided;
  float scale;
  int add_noise, learned, has_prev;
  float k[5];
};
hipError_t launch_sampler_step(const SamplerStepArgs& a, hipStream_t s);
// x_model = bf16(x) over n elements (skipped when x_model is null); tvec[0..rows) = t.
hipError_t launch_sampler_prologue(const float* x, int64_t n, bf16_t* x_model, float* tvec,
                                   int rows, float t, hipStream_t s);
