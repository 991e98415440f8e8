// Host side of the C ABI: configuration checks, workspace layout and the launch
// sequence of the DiT forward pass.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "dit.h"
#include "common.h"
#include "internal.h"
#include "train.h"

namespace dit_host {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DIT_OK;
}


size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace dit_host

using namespace dit_host;




namespace {

// Launch timer of the calling thread (dit_launch_timer_start / _stop): event
// pair i brackets the i-th timed launch; kinds[i] is its DIT_TIMER_* value.
struct LaunchTimer {
  unsigned mask = 0;
  int cap = 0, used = 0;
  bool open = false;           // pair `used` has its first event recorded
  hipEvent_t* ev = nullptr;    // 2 * cap
  int* kinds = nullptr;        // cap
};
thread_local LaunchTimer tl_timer;

void timer_release(LaunchTimer& t) {
  if (t.ev)
    for (int i = 0; i < 2 * t.cap; ++i)
      if (t.ev[i]) (void)hipEventDestroy(t.ev[i]);
  delete[] t.ev;
  delete[] t.kinds;
  t = LaunchTimer{};
}

hipError_t timer_begin(int kind, hipStream_t s) {
  LaunchTimer& t = tl_timer;
  if (!((t.mask >> kind) & 1u) || t.used >= t.cap) return hipSuccess;
  const hipError_t e = hipEventRecord(t.ev[2 * t.used], s);
  t.open = e == hipSuccess;
  return e;
}

hipError_t timer_end(int kind, hipStream_t s) {
  LaunchTimer& t = tl_timer;
  if (!t.open || !((t.mask >> kind) & 1u)) return hipSuccess;
  t.open = false;
  const hipError_t e = hipEventRecord(t.ev[2 * t.used + 1], s);
  if (e == hipSuccess) t.kinds[t.used++] = kind;
  return e;
}

// A launch of one of the block's kernels, bracketed by the thread's timer
// events when that kernel is being timed.
#define DIT_TIMED(kind, s, call)        \
  do {                                  \
    DIT_HIP(timer_begin((kind), (s)));  \
    DIT_HIP(call);                      \
    DIT_HIP(timer_end((kind), (s)));    \
  } while (0)

struct WsLayout {
  size_t e, th, c, sc, pp, pe, mod, cmod, ctx, kv, X, H, qkv, o, G, Y, seg, total;
};

// rows: conditioning rows; M: token rows of the trunk; packed: M tokens of
// packed sequences (position table and token -> sequence map for all of them).
WsLayout ws_layout_m(const dit_handle* h, int rows, size_t M, bool packed) {
  WsLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t es = h->es, R = (size_t)rows;
  L.e = take(R * h->freq * 4);
  L.th = take(R * h->d * 4);
  L.c = take(R * h->d * 4);
  L.sc = take(R * h->d * es);
  L.pp = take(h->cond_dim > 0 ? R * h->d * 4 : 0);          // pooled projection
  L.pe = take(h->cfg.rope3d ? 0 : (packed ? M : (size_t)h->T) * h->d * 4);  // 2-D position table
  L.mod = take(R * h->mod_stride * 4);                        // 0 without adaLN
  L.cmod = take(h->cond == DIT_COND_MMDIT ? R * 6 * h->N * h->d * 4 : 0);   // text stream
  L.ctx = take(h->cond == DIT_COND_CROSS_ATTN ? R * 2 * h->d * es : 0);      // context tokens
  // k | v of the context tokens for every block: [rows, 2, N, 2d]
  L.kv = take(h->cond == DIT_COND_CROSS_ATTN ? R * 2 * h->N * 2 * h->d * es : 0);
  L.X = take(M * h->d * 4);
  L.H = take(M * h->d * es);
  L.qkv = take(M * 3 * h->d * es);
  L.o = take(M * h->d * es);
  L.G = take(M * h->hid * es);
  L.Y = take(M * h->kout * 4);
  L.seg = take(packed ? M * 4 : 0);
  L.total = off;
  return L;
}

WsLayout ws_layout(const dit_handle* h, int rows) {
  return ws_layout_m(h, rows, (size_t)rows * h->Tt, false);
}

}  // namespace

namespace dit_host {
int splitk_slice(bool mfma, int64_t M, int64_t N, int64_t K) {
  // the MFMA kernel takes 64-row tiles for M <= 64 and when its 128-row
  // tiles would number at most half the CUs
  const int64_t t128 = mfma_tiles_128(M, N), ncol = t128 / ((M + 127) / 128);
  const int64_t tiles = mfma ? (M <= 64 || t128 <= 128 ? (M + 63) / 64 * ncol : t128)
                             : ((M + 63) / 64) * ((N + 63) / 64);
  const int kstep = mfma ? 64 : 16;
  // Workgroups resident at once: 256 CUs x 2 (the MFMA kernel's LDS allows
  // two per CU); the VALU kernel fits more.  Take the fewest slices whose
  // grid fills its last wave of resident workgroups to 92% or more (more
  // slices only add atomic traffic), else the best fill found.
  const int64_t slots = mfma ? 512 : 1024;
  const int64_t max_s = K / kstep < 256 ? K / kstep : 256;
  int64_t best = 1;
  double best_fill = 0.0;
  for (int64_t sp = 1; sp <= max_s; ++sp) {
    const int64_t wg = tiles * sp, waves = (wg + slots - 1) / slots;
    const double fill = (double)wg / (double)(waves * slots);
    if (fill > best_fill + 0.02) {
      best_fill = fill;
      best = sp;
    }
    if (fill >= 0.92) break;
  }
  int64_t ks = (K + best - 1) / best;
  ks = (ks + kstep - 1) / kstep * kstep;
  return ks >= K ? 0 : (int)ks;
}

hipError_t linear_wgrad(const void* dY, int64_t ldy, const void* X, int64_t ldx, int N, int K,
                        int64_t R, int dtype, float* dW, int lddw, float* db, hipStream_t s) {
  if (N <= 0 || K <= 0 || R <= 0) return hipSuccess;
  if (dtype == DIT_BF16 && N % 8 == 0 && K % 8 == 0 && R % 64 == 0 && ldy % 8 == 0 &&
      ldx % 8 == 0 && ((uintptr_t)dY & 15) == 0 && ((uintptr_t)X & 15) == 0 &&
      R * (ldy > ldx ? ldy : ldx) <= INT32_MAX)
    return launch_gemm_tn((const bf16_t*)dY, (int)ldy, (const bf16_t*)X, (int)ldx, N, K, (int)R,
                          dW, lddw, db, s);
  if (R > INT32_MAX || ldy > INT32_MAX || ldx > INT32_MAX) return hipErrorInvalidValue;
  // the bias-gradient pass's limits are checked before dW is touched
  if (db && dtype == DIT_BF16 &&
      (N % 8 || ldy % 8 || ((uintptr_t)dY & 15) || R > kColsumTallMaxRows))
    return hipErrorInvalidValue;
  ALoad a;
  memset(&a, 0, sizeof a);
  a.ptr = dY; a.lda = (int)ldy; a.a_dtype = dtype == DIT_BF16 ? 1 : 0; a.src_rows = N; a.trans = 1;
  EpiParams ep;
  memset(&ep, 0, sizeof ep);
  ep.out = dW; ep.ldo = lddw; ep.ldw = (int)ldx; ep.w_trans = 1;
  ep.ksplit = splitk_slice(false, N, K, R);
  hipError_t e = launch_gemm_valu(EPI_ATOMIC_F32, A_PLAIN, a, X, dtype == DIT_BF16 ? 1 : 0, N, K,
                                  (int)R, ep, s);
  if (e != hipSuccess || !db) return e;
  if (dtype != DIT_BF16) return launch_colsum((const float*)dY, (int)R, N, ldy, db, s);
  return launch_colsum_tall_bf16(dY, R, N, ldy, db, s);
}

EpiParams epi0() {
  EpiParams ep;
  memset(&ep, 0, sizeof ep);
  return ep;
}

// One linear layer: MFMA for bf16, VALU for fp32.
hipError_t linear(const dit_handle* h, int epi, const void* A, int lda, const void* W, int M,
                  int N, int K, const EpiParams& ep, hipStream_t s) {
  if (h->dtype == DIT_BF16)
    return launch_gemm_mfma(epi, (const bf16_t*)A, lda, (const bf16_t*)W, M, N, K, ep, s);
  ALoad a;
  memset(&a, 0, sizeof a);
  a.ptr = A;
  a.lda = lda;
  a.a_dtype = 0;
  a.src_rows = M;
  a.seg = ep.a_seg; a.skip = ep.a_skip; a.off = ep.a_off;
  return launch_gemm_valu(epi, A_PLAIN, a, W, 0, M, N, K, ep, s);
}
}  // namespace dit_host

namespace {

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

const void* woff(const void* base, size_t elems, int es) {
  return (const char*)base + elems * es;
}


// Patch embedding of M tokens (see launch_patch_embed); patch vectors whose
// length is not a multiple of 16 go through the VALU GEMM with the patch
// gather as its A loader.
hipError_t patch_embed(const dit_handle* h, const void* x, int src_rows, const PatchGeom& g,
                       const float* pe, int M, int out_skip, float* X, hipStream_t s) {
  if (h->kin % 16 == 0 && ((uintptr_t)h->w.pe_w & 15) == 0)
    return launch_patch_embed(x, src_rows, g, h->dtype, h->w.pe_w, h->w.pe_b, pe, M, h->d,
                              out_skip, X, s);
  ALoad a;
  memset(&a, 0, sizeof a);
  a.ptr = x; a.a_dtype = h->dtype; a.src_rows = src_rows; a.g = g;
  EpiParams ep = epi0();
  ep.bias = h->w.pe_b; ep.out = X; ep.ldo = h->d; ep.T = g.T; ep.out_skip = out_skip;
  ep.pe_tab = pe;
  return launch_gemm_valu(EPI_PATCH, A_PATCH, a, h->w.pe_w, h->dtype, M, h->d, h->kin, ep, s);
}

// Packed sequences: token rows, token -> sequence map (the modulation row of
// each token) and the sequence table for block-diagonal attention.
struct Packed {
  int M;
  const int* tok_seg;
  SeqTable seqs;
};

// One adaLN-Zero block on the residual stream X [rows*T, d] (fp32, in place).
// mod + base points at this block's (b1, g1, a1, b2, g2, a2) in rows of mod_stride.
int run_block(const dit_handle* h, int l, int rows, float* X, const float* mod, int mod_stride,
              int base, void* ws, const WsLayout& L, float* o_branch, float* f_branch,
              hipStream_t s, const Packed* pk = nullptr) {
  const int d = h->d, T = h->T, M = pk ? pk->M : rows * T, es = h->es;
  const int* ts = pk ? pk->tok_seg : nullptr;
  void* Hb = at<void>(ws, L.H);
  void* O = at<void>(ws, L.o);
  void* G = at<void>(ws, L.G);
  void* qkv = at<void>(ws, L.qkv);

  DIT_TIMED(DIT_TIMER_LN, s, launch_ln_modulate(X, M, T, d, mod, mod_stride, base, base + d,
                                                h->eps, Hb, h->dtype, s, ts));

  // Packed in-projection q | k | v [M, 3d] (heads as contiguous dh slices).
  EpiParams ep = epi0();
  ep.bias = h->w.qkv_b + (size_t)l * 3 * d;
  ep.out = qkv; ep.ldo = 3 * d;
  const void* qw = woff(h->w.qkv_w, (size_t)l * 3 * d * d, es);
  DIT_TIMED(DIT_TIMER_QKV, s, linear(h, EPI_BIAS_DT, Hb, d, qw, M, 3 * d, d, ep, s));

  if (pk) {
    if (h->cfg.qk_norm)   // per-token LayerNorm of q and k (no rotary embedding when packed)
      DIT_HIP(launch_qk_norm_rope(qkv, 1, h->heads, M, h->dh, h->dtype, 1, h->eps, 0, h->gh,
                                  h->gw, s));
    DIT_TIMED(DIT_TIMER_ATTENTION, s,
              launch_attention_packed(qkv, pk->seqs, h->heads, h->dh, h->dtype, O, s));
  } else {
    if (h->cfg.qk_norm || h->cfg.rope3d)
      DIT_HIP(launch_qk_norm_rope(qkv, rows, h->heads, T, h->dh, h->dtype, h->cfg.qk_norm, h->eps,
                                  h->cfg.rope3d, h->gh, h->gw, s));
    DIT_TIMED(DIT_TIMER_ATTENTION, s,
              launch_attention(qkv, rows, h->heads, T, h->dh, h->dtype, O, s));
  }

  const void* ow = woff(h->w.o_w, (size_t)l * d * d, es);
  if (o_branch) {
    EpiParams eb = epi0();
    eb.bias = h->w.o_b + (size_t)l * d;
    eb.out = o_branch; eb.ldo = d;
    DIT_HIP(linear(h, EPI_BIAS_F32, O, d, ow, M, d, d, eb, s));
  }
  ep = epi0();
  ep.bias = h->w.o_b + (size_t)l * d;
  ep.out = X; ep.ldo = d;
  ep.mod = mod; ep.mod_stride = mod_stride; ep.gate_off = base + 2 * d; ep.T = T;
  ep.tok_seg = ts;
  DIT_TIMED(DIT_TIMER_OUT_PROJ, s, linear(h, EPI_GATED, O, d, ow, M, d, d, ep, s));

  DIT_TIMED(DIT_TIMER_LN, s, launch_ln_modulate(X, M, T, d, mod, mod_stride, base + 3 * d,
                                                base + 4 * d, h->eps, Hb, h->dtype, s, ts));
  ep = epi0();
  ep.bias = h->w.fc1_b + (size_t)l * h->hid;
  ep.out = G; ep.ldo = h->hid;
  const void* w1 = woff(h->w.fc1_w, (size_t)l * h->hid * d, es);
  DIT_TIMED(DIT_TIMER_FC1, s, linear(h, EPI_GELU, Hb, d, w1, M, h->hid, d, ep, s));

  const void* w2 = woff(h->w.fc2_w, (size_t)l * d * h->hid, es);
  if (f_branch) {
    EpiParams eb = epi0();
    eb.bias = h->w.fc2_b + (size_t)l * d;
    eb.out = f_branch; eb.ldo = d;
    DIT_HIP(linear(h, EPI_BIAS_F32, G, h->hid, w2, M, d, h->hid, eb, s));
  }
  ep = epi0();
  ep.bias = h->w.fc2_b + (size_t)l * d;
  ep.out = X; ep.ldo = d;
  ep.mod = mod; ep.mod_stride = mod_stride; ep.gate_off = base + 5 * d; ep.T = T;
  ep.tok_seg = ts;
  DIT_TIMED(DIT_TIMER_FC2, s, linear(h, EPI_GATED, G, h->hid, w2, M, d, h->hid, ep, s));
  return DIT_OK;
}

// One block of the in-context or cross-attention design on X [rows * Tt, d]
// (fp32, in place).  Each LayerNorm's affine (b, g) is applied as a modulation
// that is the same for every row (row stride 0); residual adds have no gate.
// kv: block l's context keys | values of this row group's first row, rows of
// stride N * 2d elements (cross-attention).
int run_block_variant(const dit_handle* h, int l, int rows, float* X, const void* kv, void* ws,
                      const WsLayout& L, hipStream_t s) {
  const int d = h->d, Tt = h->Tt, M = rows * Tt, es = h->es;
  void* Hb = at<void>(ws, L.H);
  void* O = at<void>(ws, L.o);
  void* G = at<void>(ws, L.G);
  void* qkv = at<void>(ws, L.qkv);
  const float* lnp = h->w.ln_p + (size_t)l * h->nln * 2 * d;

  DIT_HIP(launch_ln_modulate(X, M, Tt, d, lnp, 0, 0, d, h->eps, Hb, h->dtype, s));
  EpiParams ep = epi0();
  ep.bias = h->w.qkv_b + (size_t)l * 3 * d;
  ep.out = qkv; ep.ldo = 3 * d;
  DIT_HIP(linear(h, EPI_BIAS_DT, Hb, d, woff(h->w.qkv_w, (size_t)l * 3 * d * d, es), M, 3 * d, d,
                 ep, s));
  DIT_HIP(launch_attention(qkv, rows, h->heads, Tt, h->dh, h->dtype, O, s));
  ep = epi0();
  ep.bias = h->w.o_b + (size_t)l * d;
  ep.out = X; ep.ldo = d; ep.T = Tt;
  DIT_HIP(linear(h, EPI_GATED, O, d, woff(h->w.o_w, (size_t)l * d * d, es), M, d, d, ep, s));

  int li = 1;
  if (h->cond == DIT_COND_CROSS_ATTN) {
    DIT_HIP(launch_ln_modulate(X, M, Tt, d, lnp, 0, 2 * d, 3 * d, h->eps, Hb, h->dtype, s));
    ep = epi0();
    ep.bias = h->w.xq_b + (size_t)l * d;
    ep.out = qkv; ep.ldo = d;
    DIT_HIP(linear(h, EPI_BIAS_DT, Hb, d, woff(h->w.xq_w, (size_t)l * d * d, es), M, d, d, ep, s));
    DIT_HIP(launch_cross_attention2(qkv, kv, (int64_t)h->N * 2 * d, rows, Tt, h->heads, h->dh,
                                    h->dtype, O, s));
    ep = epi0();
    ep.bias = h->w.xo_b + (size_t)l * d;
    ep.out = X; ep.ldo = d; ep.T = Tt;
    DIT_HIP(linear(h, EPI_GATED, O, d, woff(h->w.xo_w, (size_t)l * d * d, es), M, d, d, ep, s));
    li = 2;
  }

  DIT_HIP(launch_ln_modulate(X, M, Tt, d, lnp, 0, 2 * d * li, 2 * d * li + d, h->eps, Hb, h->dtype,
                             s));
  ep = epi0();
  ep.bias = h->w.fc1_b + (size_t)l * h->hid;
  ep.out = G; ep.ldo = h->hid;
  DIT_HIP(linear(h, EPI_GELU, Hb, d, woff(h->w.fc1_w, (size_t)l * h->hid * d, es), M, h->hid, d,
                 ep, s));
  ep = epi0();
  ep.bias = h->w.fc2_b + (size_t)l * d;
  ep.out = X; ep.ldo = d; ep.T = Tt;
  DIT_HIP(linear(h, EPI_GATED, G, h->hid, woff(h->w.fc2_w, (size_t)l * d * h->hid, es), M, d,
                 h->hid, ep, s));
  return DIT_OK;
}

// Trunk of `rows` rows.  Row r reads latent/time/pooled row r % src_rows; rows
// r >= null_from take the null label.  Leaves the decoder output in ws Y.
// One MMDiT block for `rows` rows: image stream Xi [rows * T, d], text stream
// Xc [rows * Lc, d] (fp32, in place), modulations modi (rows of mod_stride)
// and modc (rows of 6 N d).  The two streams' q | k | v land in one joint
// buffer [rows, Lc + T, 3d] (text tokens first) through the GEMM output row
// map, attention runs over the joint rows, and each stream's output
// projection reads its own rows of the joint output through the A row map.
int run_block_mmdit(const dit_handle* h, int l, int rows, float* Xi, float* Xc, const float* modi,
                    const float* modc, void* ws, const WsLayout& L, hipStream_t s) {
  const int d = h->d, T = h->T, Lc = h->Lc, J = T + Lc, es = h->es;
  const int cms = 6 * h->N * d, base = 6 * d * l;
  void* Hb = at<void>(ws, L.H);
  void* O = at<void>(ws, L.o);
  void* G = at<void>(ws, L.G);
  void* qkv = at<void>(ws, L.qkv);
  struct Stream {
    float* X; const float* mod; int ms; int n; const void *qkv_w, *o_w, *fc1_w, *fc2_w;
    const float *qkv_b, *o_b, *fc1_b, *fc2_b; int seg, skip, off;
  };
  const Stream st[2] = {
      {Xc, modc, cms, Lc, h->w.cqkv_w, h->w.co_w, h->w.cfc1_w, h->w.cfc2_w, h->w.cqkv_b,
       h->w.co_b, h->w.cfc1_b, h->w.cfc2_b, Lc, T, 0},
      {Xi, modi, h->mod_stride, T, h->w.qkv_w, h->w.o_w, h->w.fc1_w, h->w.fc2_w, h->w.qkv_b,
       h->w.o_b, h->w.fc1_b, h->w.fc2_b, T, Lc, Lc}};
  for (const Stream& q : st) {
    const int M = rows * q.n;
    DIT_HIP(launch_ln_modulate(q.X, M, q.n, d, q.mod, q.ms, base, base + d, h->eps, Hb, h->dtype,
                               s));
    EpiParams ep = epi0();
    ep.bias = q.qkv_b + (size_t)l * 3 * d;
    ep.out = qkv; ep.ldo = 3 * d;
    ep.o_seg = q.seg; ep.o_skip = q.skip; ep.o_off = q.off;
    DIT_HIP(linear(h, EPI_BIAS_DT, Hb, d, woff(q.qkv_w, (size_t)l * 3 * d * d, es), M, 3 * d, d,
                   ep, s));
  }
  DIT_HIP(launch_qk_rms(qkv, rows, h->heads, J, Lc, h->dh, h->dtype, h->eps,
                        h->w.qk_rms + (size_t)l * 4 * h->dh, s));
  DIT_HIP(launch_attention(qkv, rows, h->heads, J, h->dh, h->dtype, O, s));
  for (const Stream& q : st) {
    const int M = rows * q.n;
    EpiParams ep = epi0();
    ep.bias = q.o_b + (size_t)l * d;
    ep.out = q.X; ep.ldo = d;
    ep.mod = q.mod; ep.mod_stride = q.ms; ep.gate_off = base + 2 * d; ep.T = q.n;
    ep.a_seg = q.seg; ep.a_skip = q.skip; ep.a_off = q.off;
    DIT_HIP(linear(h, EPI_GATED, O, d, woff(q.o_w, (size_t)l * d * d, es), M, d, d, ep, s));
    DIT_HIP(launch_ln_modulate(q.X, M, q.n, d, q.mod, q.ms, base + 3 * d, base + 4 * d, h->eps, Hb,
                               h->dtype, s));
    ep = epi0();
    ep.bias = q.fc1_b + (size_t)l * h->hid;
    ep.out = G; ep.ldo = h->hid;
    DIT_HIP(linear(h, EPI_GELU, Hb, d, woff(q.fc1_w, (size_t)l * h->hid * d, es), M, h->hid, d,
                   ep, s));
    ep = epi0();
    ep.bias = q.fc2_b + (size_t)l * d;
    ep.out = q.X; ep.ldo = d;
    ep.mod = q.mod; ep.mod_stride = q.ms; ep.gate_off = base + 5 * d; ep.T = q.n;
    DIT_HIP(linear(h, EPI_GATED, G, h->hid, woff(q.fc2_w, (size_t)l * d * h->hid, es), M, d,
                   h->hid, ep, s));
  }
  return DIT_OK;
}

// Conditioning of `rows` rows: c (time embedding, + class row, + pooled
// projection), SiLU(c) and all modulation vectors for adaLN-Zero; the two
// conditioning tokens (and the context keys / values) for the other designs.
// Row r reads time / pooled row r % src_rows; rows r >= null_from take the
// null label.
int run_conditioning(const dit_handle* h, const float* t, const int32_t* y, const float* pooled,
                     int rows, int src_rows, int null_from, void* ws, const WsLayout& L,
                     hipStream_t s) {
  const int d = h->d, T = h->T;
  const bool ada = h->cond == DIT_COND_ADALN_ZERO || h->cond == DIT_COND_MMDIT;
  float* e = at<float>(ws, L.e);
  float* th = at<float>(ws, L.th);
  float* c = at<float>(ws, L.c);
  void* sc = at<void>(ws, L.sc);
  float* mod = at<float>(ws, L.mod);
  float* X = at<float>(ws, L.X);

  // c = t_emb (+ pooled projection) (+ class row); sc = SiLU(c) in the GEMM dtype.
  ALoad a;
  memset(&a, 0, sizeof a);
  EpiParams ep = epi0();
  if (h->dtype == DIT_BF16 && h->freq % 64 == 0) {
    // bf16: the sinusoid and SiLU(hidden) are bf16 GEMM operands on the MFMA
    // path; the class row and the pooled projection are added afterwards.
    bf16_t* eb = at<bf16_t>(ws, L.e);
    bf16_t* thb = at<bf16_t>(ws, L.th);
    DIT_HIP(launch_timestep_embed_bf16(t, rows, src_rows, h->freq, eb, s));
    ep.bias = h->w.t1_b; ep.out = thb; ep.ldo = d;
    DIT_HIP(linear(h, EPI_SILU_DT, eb, h->freq, h->w.t1_w, rows, d, h->freq, ep, s));
    ep = epi0();
    ep.bias = h->w.t2_b; ep.out = c; ep.ldo = d;
    DIT_HIP(linear(h, EPI_BIAS_F32, thb, d, h->w.t2_w, rows, d, d, ep, s));
    float* pp = nullptr;
    if (h->cond_dim > 0) {
      pp = at<float>(ws, L.pp);
      a.ptr = pooled; a.lda = h->cond_dim; a.a_dtype = 0; a.src_rows = src_rows;
      ep = epi0();
      ep.bias = h->w.pool_b; ep.out = pp; ep.ldo = d;
      DIT_HIP(launch_gemm_valu(EPI_BIAS_F32, A_PLAIN, a, h->w.pool_w, h->dtype, rows, d,
                               h->cond_dim, ep, s));
    }
    if (ada)
      DIT_HIP(launch_cond_finish(c, rows, d, h->ncls > 0 ? h->w.y_table : nullptr, y, src_rows,
                                 null_from, h->ncls, pp, sc, h->dtype, s));
  } else if (!ada) {
    // time embedding alone (the class row becomes a token of its own)
    DIT_HIP(launch_timestep_embed(t, rows, src_rows, h->freq, e, s));
    a.ptr = e; a.lda = h->freq; a.a_dtype = 0; a.src_rows = rows;
    ep = epi0();
    ep.bias = h->w.t1_b; ep.out = th; ep.ldo = d;
    DIT_HIP(launch_gemm_valu(EPI_BIAS_SILU, A_PLAIN, a, h->w.t1_w, h->dtype, rows, d, h->freq,
                             ep, s));
    a.ptr = th; a.lda = d;
    ep = epi0();
    ep.bias = h->w.t2_b; ep.out = c; ep.ldo = d;
    DIT_HIP(launch_gemm_valu(EPI_BIAS_F32, A_PLAIN, a, h->w.t2_w, h->dtype, rows, d, d, ep, s));
  } else {
    DIT_HIP(launch_timestep_embed(t, rows, src_rows, h->freq, e, s));
    if (h->cond_dim > 0) {
      a.ptr = pooled; a.lda = h->cond_dim; a.a_dtype = 0; a.src_rows = src_rows;
      ep.bias = h->w.pool_b; ep.out = c; ep.ldo = d;
      DIT_HIP(launch_gemm_valu(EPI_BIAS_F32, A_PLAIN, a, h->w.pool_w, h->dtype, rows, d,
                               h->cond_dim, ep, s));
    }
    a.ptr = e; a.lda = h->freq; a.a_dtype = 0; a.src_rows = rows;
    ep = epi0();
    ep.bias = h->w.t1_b; ep.out = th; ep.ldo = d;
    DIT_HIP(launch_gemm_valu(EPI_BIAS_SILU, A_PLAIN, a, h->w.t1_w, h->dtype, rows, d, h->freq,
                             ep, s));
    a.ptr = th; a.lda = d;
    ep = epi0();
    ep.bias = h->w.t2_b; ep.out = c; ep.ldo = d; ep.silu_out = sc;
    ep.add_prev = h->cond_dim > 0;
    if (h->ncls > 0) {
      ep.table = h->w.y_table; ep.labels = y; ep.label_rows = src_rows;
      ep.null_from = null_from; ep.ncls = h->ncls;
    }
    DIT_HIP(launch_gemm_valu(EPI_COND, A_PLAIN, a, h->w.t2_w, h->dtype, rows, d, d, ep, s));
  }

  if (ada) {
    // All modulation vectors (every block and the final layer) in one GEMM.
    ep = epi0();
    ep.bias = h->w.ada_b; ep.out = mod; ep.ldo = h->mod_stride;
    DIT_HIP(linear(h, EPI_BIAS_F32, sc, d, h->w.ada_w, rows, h->mod_stride, d, ep, s));
    if (h->cond == DIT_COND_MMDIT) {
      // the text stream's modulation vectors of every block
      ep = epi0();
      ep.bias = h->w.cada_b; ep.out = at<float>(ws, L.cmod); ep.ldo = 6 * h->N * d;
      DIT_HIP(linear(h, EPI_BIAS_F32, sc, d, h->w.cada_w, rows, 6 * h->N * d, d, ep, s));
    }
  } else {
    // The time and class embeddings as two tokens after each row's patch
    // tokens (in-context) or as each row's two context tokens.
    const bool in_ctx = h->cond == DIT_COND_IN_CONTEXT;
    DIT_HIP(launch_cond_tokens(c, rows, d, h->w.y_table, y, src_rows, null_from, h->ncls,
                               in_ctx ? 0 : 1, in_ctx ? (void*)X : at<void>(ws, L.ctx), T,
                               h->dtype, s));
    if (!in_ctx) {
      // keys | values of the context tokens for all blocks in one GEMM (they
      // depend on the conditioning only): [rows * 2, N * 2d]
      ep = epi0();
      ep.bias = h->w.xkv_b; ep.out = at<void>(ws, L.kv); ep.ldo = h->N * 2 * d;
      DIT_HIP(linear(h, EPI_BIAS_DT, at<void>(ws, L.ctx), d, h->w.xkv_w, 2 * rows, h->N * 2 * d, d,
                     ep, s));
    }
  }

  return DIT_OK;
}

int run_trunk(const dit_handle* h, const void* x_t, const float* t, const int32_t* y,
              const float* pooled, const void* ctx, int rows, int src_rows, int null_from,
              void* ws, const WsLayout& L, const dit_taps* taps, hipStream_t s) {
  const int d = h->d, T = h->T, Tt = h->Tt, Tf = h->Tf, M = rows * Tt;
  const bool mm = h->cond == DIT_COND_MMDIT;
  const bool ada = h->cond == DIT_COND_ADALN_ZERO || mm;
  // MMDiT: the image stream's rows * T tokens, then the text stream's rows * Lc
  const float* cmod = at<float>(ws, L.cmod);
  float* Xtext = at<float>(ws, L.X) + (size_t)rows * T * d;
  float* c = at<float>(ws, L.c);
  float* mod = at<float>(ws, L.mod);
  float* X = at<float>(ws, L.X);
  void* Hb = at<void>(ws, L.H);
  float* Y = at<float>(ws, L.Y);
  {
    int rc = run_conditioning(h, t, y, pooled, rows, src_rows, null_from, ws, L, s);
    if (rc) return rc;
  }
  // Patchify gather + patch embedding + bias + 2-D position embedding (from a
  // table of the T x d embedding, computed once per call).
  float* pe = nullptr;
  if (!h->cfg.rope3d) {
    pe = at<float>(ws, L.pe);
    DIT_HIP(launch_pos_embed_table(h->gh, h->gw, d, pe, s));
  }
  DIT_HIP(patch_embed(h, x_t, src_rows, h->gin, pe, rows * T, Tf - T, X, s));
  if (mm) {
    // text embeddings [rows * Lc, ctx_dim] -> the text stream
    EpiParams ec = epi0();
    ec.bias = h->w.ctx_b; ec.out = Xtext; ec.ldo = d;
    DIT_HIP(linear(h, EPI_BIAS_F32, ctx, h->cfg.ctx_dim, h->w.ctx_w, rows * h->Lc, d,
                   h->cfg.ctx_dim, ec, s));
  }

  if (taps) {
    if (taps->c) DIT_HIP(hipMemcpyAsync(taps->c, c, (size_t)rows * d * 4, hipMemcpyDeviceToDevice, s));
    if (taps->mod && ada)
      DIT_HIP(hipMemcpyAsync(taps->mod, mod, (size_t)rows * h->mod_stride * 4,
                             hipMemcpyDeviceToDevice, s));
    if (taps->x_embed)
      DIT_HIP(hipMemcpyAsync(taps->x_embed, X, (size_t)M * d * 4, hipMemcpyDeviceToDevice, s));
  }

  // Blocks and the final layer (LN + modulation (b_f, g_f), linear decoder),
  // all rows at once on the caller's stream: at the image configurations
  // every block product then fills whole waves of the wide-tile GEMM.
  const int fb = 6 * d * h->N;
  const char* kv_base = at<char>(ws, L.kv);
  // Final layer: LN + (adaLN modulation or the learned affine) + decoder.
  auto final_layer = [&](float* Xg, const float* modg, int Mg, void* Hg, float* Yg,
                         hipStream_t st) -> int {
    if (ada)
      DIT_HIP(launch_ln_modulate(Xg, Mg, Tf, d, modg, h->mod_stride, fb, fb + d, h->eps, Hg,
                                 h->dtype, st));
    else
      DIT_HIP(launch_ln_modulate(Xg, Mg, Tf, d, h->w.final_ln, 0, 0, d, h->eps, Hg, h->dtype, st));
    EpiParams ef = epi0();
    ef.bias = h->w.out_b; ef.out = Yg; ef.ldo = h->kout;
    DIT_HIP(linear(h, EPI_BIAS_F32, Hg, d, h->w.out_w, Mg, h->kout, d, ef, st));
    return DIT_OK;
  };
  auto one_block = [&](int l, int r0, int nr, float* Xg, const float* modg, const WsLayout& Lg,
                       hipStream_t st) -> int {
    if (mm)
      return run_block_mmdit(h, l, nr, Xg, Xtext + (size_t)r0 * h->Lc * d, modg,
                             cmod + (size_t)r0 * 6 * h->N * d, ws, Lg, st);
    if (ada) return run_block(h, l, nr, Xg, modg, h->mod_stride, 6 * d * l, ws, Lg, nullptr,
                              nullptr, st);
    const size_t es = h->es;
    return run_block_variant(h, l, nr, Xg,
                             kv_base + ((size_t)r0 * 2 * h->N * 2 * d + (size_t)l * 2 * d) * es,
                             ws, Lg, st);
  };
  for (int l = 0; l < h->N; ++l) {
    int rc = one_block(l, 0, rows, X, mod, L, s);
    if (rc) return rc;
    if (taps && taps->x_blocks)
      DIT_HIP(hipMemcpyAsync(taps->x_blocks + (size_t)l * M * d, X, (size_t)M * d * 4,
                             hipMemcpyDeviceToDevice, s));
  }
  {
    int rc = final_layer(X, mod, rows * Tf, Hb, Y, s);
    if (rc) return rc;
  }
  if (taps && taps->y_final)
    DIT_HIP(hipMemcpyAsync(taps->y_final, Y, (size_t)rows * Tf * h->kout * 4,
                           hipMemcpyDeviceToDevice, s));
  return DIT_OK;
}

int check_rows(const dit_handle* h, int rows) {
  if ((int64_t)rows * h->Tt > (1LL << 30)) return fail(DIT_EINVAL, "rows * T too large");
  if ((int64_t)rows * h->heads > 65535)
    return fail(DIT_EUNSUPPORTED, "rows * heads > 65535 (attention grid limit)");
  return DIT_OK;
}

int check_ws_bytes(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(DIT_EWORKSPACE, "workspace pointer is NULL");
  if (ws_bytes < need)
    return fail(DIT_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws & 255) return fail(DIT_EWORKSPACE, "workspace must be 256-byte aligned");
  return DIT_OK;
}

int check_ws(const dit_handle* h, int rows, const void* ws, size_t ws_bytes, WsLayout* L) {
  int rc = check_rows(h, rows);
  if (rc) return rc;
  *L = ws_layout(h, rows);
  return check_ws_bytes(ws, ws_bytes, L->total);
}

int forward_impl(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                 const float* pooled, const void* ctx, int B, float* out, const dit_taps* taps,
                 void* ws, size_t ws_bytes, void* stream) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (!x_t || !t || !out) return fail(DIT_EINVAL, "x_t, t and out must be non-NULL");
  if (h->cond == DIT_COND_MMDIT && !ctx)
    return fail(DIT_EINVAL, "the MMDiT design needs text embeddings (dit_forward_ctx)");
  if (h->cond != DIT_COND_MMDIT && ctx)
    return fail(DIT_EINVAL, "text embeddings are only taken by the MMDiT design");
  if (ctx && ((uintptr_t)ctx & 15)) return fail(DIT_EINVAL, "ctx must be 16-byte aligned");
  if (B <= 0) return fail(DIT_EINVAL, "B must be positive (got %d)", B);
  if (h->ncls > 0 && !y) return fail(DIT_EINVAL, "class labels y are required");
  if (h->cond_dim > 0 && !pooled) return fail(DIT_EINVAL, "pooled conditioning is required");
  WsLayout L;
  int rc = check_ws(h, B, ws, ws_bytes, &L);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  rc = run_trunk(h, x_t, t, y, pooled, ctx, B, B, B, ws, L, taps, s);
  if (rc) return rc;
  DIT_HIP(launch_unpatchify(at<float>(ws, L.Y), B, 0, h->gouty, h->cfg.out_channels, 0, 0.0f, 0,
                            out, s));
  return ok();
}

int cfg_forward_impl(dit_handle* h, const void* x_t, const float* t, const int32_t* y, int Bh,
                     float scale, int guided, float* out, const dit_taps* taps, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (!x_t || !t || !y || !out) return fail(DIT_EINVAL, "x_t, t, y and out must be non-NULL");
  if (Bh <= 0 || Bh > (1 << 29)) return fail(DIT_EINVAL, "Bh must be positive (got %d)", Bh);
  if (h->ncls <= 0) return fail(DIT_EINVAL, "guidance needs a class table with a null label");
  if (h->cond_dim > 0) return fail(DIT_EUNSUPPORTED, "guidance with pooled conditioning");
  if (h->cond == DIT_COND_MMDIT) return fail(DIT_EUNSUPPORTED, "guidance with the MMDiT design");
  if (guided < 1 || guided > h->cfg.out_channels)
    return fail(DIT_EINVAL, "guided_channels must be in [1, %d]", h->cfg.out_channels);
  if (!std::isfinite(scale)) return fail(DIT_EINVAL, "guidance scale must be finite");
  WsLayout L;
  int rc = check_ws(h, 2 * Bh, ws, ws_bytes, &L);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  rc = run_trunk(h, x_t, t, y, nullptr, nullptr, 2 * Bh, Bh, Bh, ws, L, taps, s);
  if (rc) return rc;
  DIT_HIP(launch_unpatchify(at<float>(ws, L.Y), Bh, Bh, h->gouty, h->cfg.out_channels, guided,
                            scale, 1, out, s));
  return ok();
}

PatchGeom make_geom(int C, int F, int H, int W, int p, int pt) {
  PatchGeom g;
  g.C = C; g.F = F; g.H = H; g.W = W; g.p = p; g.pt = pt;
  g.gh = H / p; g.gw = W / p;
  g.T = (F / pt) * g.gh * g.gw;
  g.K = pt * p * p * C;
  return g;
}

int check_geom(int B, int C, int F, int H, int W, int p, int pt) {
  if (B <= 0 || C <= 0 || F <= 0 || H <= 0 || W <= 0 || p <= 0 || pt <= 0)
    return fail(DIT_EINVAL, "sizes must be positive");
  if (H % p || W % p || F % pt)
    return fail(DIT_EINVAL, "latent extents (%d, %d, %d) not divisible by patch (%d, %d, %d)", F,
                H, W, pt, p, p);
  if ((int64_t)B * C * F * H * W > (1LL << 40)) return fail(DIT_EINVAL, "latent too large");
  return DIT_OK;
}


// ---------------------------------------------------------------------------
// Sampler schedule (host, fp64).  Sources: the forward process and the learned
// reverse covariance (cv-learn "Sora / DiT", Method, training objective
// bullet), the multistep DPM-Solver used for inference (itwiki page, inference
// with diffusers), the rectified-flow interpolation and velocity target
// (blog.outta.ai GOKU review, section 2.3).  Readings where the pages stop:
// beta linear from beta_start to beta_end over train_steps, abar the running
// product of (1 - beta); kept steps tau_0 > ... > tau_{S-1}, step k going to
// tau_{k+1} and the last one to the clean latent (abar = 1); learned variance
// exp(f log beta + (1 - f) log beta_tilde), f = (v + 1) / 2; no x0 clipping.

struct StepCoef {
  double model_t;
  double c[8];
};

int check_sampler(const dit_sampler* sp) {
  if (!sp) return fail(DIT_EINVAL, "sampler is NULL");
  const int S = sp->num_steps;
  if (S < 1 || S > 1000000) return fail(DIT_EINVAL, "num_steps must be in [1, 1e6] (got %d)", S);
  if (sp->kind == DIT_SAMPLER_DDPM || sp->kind == DIT_SAMPLER_DPMPP_2M) {
    const int Tn = sp->train_steps;
    if (Tn < 1 || Tn > 1000000) return fail(DIT_EINVAL, "train_steps must be in [1, 1e6]");
    if (!(sp->beta_start > 0.0 && sp->beta_start < 1.0 && sp->beta_end > 0.0 &&
          sp->beta_end < 1.0))
      return fail(DIT_EINVAL, "betas must lie in (0, 1)");
    if (sp->timesteps) {
      for (int k = 0; k < S; ++k) {
        const int t = sp->timesteps[k];
        if (t < 0 || t >= Tn) return fail(DIT_EINVAL, "timesteps[%d] = %d outside [0, %d)", k, t, Tn);
        if (k && t >= sp->timesteps[k - 1])
          return fail(DIT_EINVAL, "timesteps must be strictly decreasing (index %d)", k);
      }
    } else if (S > Tn) {
      return fail(DIT_EINVAL, "num_steps %d > train_steps %d", S, Tn);
    }
  } else if (sp->kind == DIT_SAMPLER_RF_EULER) {
    if (sp->times) {
      for (int k = 0; k <= S; ++k) {
        if (!std::isfinite(sp->times[k])) return fail(DIT_EINVAL, "times[%d] not finite", k);
        if (k && !(sp->times[k] > sp->times[k - 1]))
          return fail(DIT_EINVAL, "times must be strictly increasing (index %d)", k);
      }
    }
  } else {
    return fail(DIT_EINVAL, "unknown sampler kind %d", sp->kind);
  }
  return DIT_OK;
}

// abar_t = prod_{j <= t} (1 - beta_j), beta on a straight line.
std::vector<double> abar_table(const dit_sampler* sp) {
  const int Tn = sp->train_steps;
  std::vector<double> ab(Tn);
  double prod = 1.0;
  for (int j = 0; j < Tn; ++j) {
    const double beta =
        Tn == 1 ? sp->beta_start
                : (j == Tn - 1 ? sp->beta_end
                               : sp->beta_start + j * ((sp->beta_end - sp->beta_start) / (Tn - 1)));
    prod *= 1.0 - beta;
    ab[j] = prod;
  }
  return ab;
}

// Kept step k: the given list, or S steps spread evenly over [0, train_steps),
// rounded half up, largest first.
int kept_step(const dit_sampler* sp, int k) {
  if (sp->timesteps) return sp->timesteps[k];
  const int S = sp->num_steps, Tn = sp->train_steps;
  if (S == 1) return Tn - 1;
  const int j = S - 1 - k;
  return (int)std::floor((double)j * (Tn - 1) / (S - 1) + 0.5);
}

double flow_time(const dit_sampler* sp, int k) {
  return sp->times ? sp->times[k] : (double)k / sp->num_steps;
}

// log(alpha / sigma) of a VP level; +inf at abar = 1.
double half_log_snr(double ab) {
  return ab >= 1.0 ? INFINITY : 0.5 * std::log(ab) - 0.5 * std::log1p(-ab);
}

void step_coef(const dit_sampler* sp, const std::vector<double>& ab, int k, StepCoef* o) {
  const int S = sp->num_steps;
  for (double& v : o->c) v = 0.0;
  if (sp->kind == DIT_SAMPLER_RF_EULER) {
    o->model_t = flow_time(sp, k);
    o->c[0] = flow_time(sp, k + 1) - flow_time(sp, k);
    return;
  }
  const int tk = kept_step(sp, k);
  o->model_t = tk;
  const double at = ab[tk];
  const double as = k + 1 < S ? ab[kept_step(sp, k + 1)] : 1.0;
  if (sp->kind == DIT_SAMPLER_DDPM) {
    const double beta = 1.0 - at / as;
    const double c_x0 = beta * std::sqrt(as) / (1.0 - at);
    const double c_xt = (1.0 - as) * std::sqrt(1.0 - beta) / (1.0 - at);
    // mean = c_x0 x0 + c_xt x with x0 = (x - sqrt(1 - abar_t) eps) / sqrt(abar_t)
    o->c[0] = c_x0 / std::sqrt(at) + c_xt;
    o->c[1] = c_x0 * std::sqrt(1.0 - at) / std::sqrt(at);
    o->c[2] = std::log(beta);
    if (as < 1.0) {
      o->c[3] = std::log(beta * (1.0 - as) / (1.0 - at));
      o->c[4] = 1.0;
    } else if (S >= 2) {
      // last step: beta_tilde is 0 there; take the previous step's (no noise is added)
      const double a0 = ab[kept_step(sp, S - 2)], a1 = ab[kept_step(sp, S - 1)];
      const double b1 = 1.0 - a0 / a1;
      o->c[3] = std::log(b1 * (1.0 - a1) / (1.0 - a0));
    } else {
      o->c[3] = o->c[2];
    }
    return;
  }
  // DPM-Solver++ in data prediction: alpha = sqrt(abar), sigma = sqrt(1 - abar).
  const double al_t = std::sqrt(at), sg_t = std::sqrt(1.0 - at);
  o->c[0] = 1.0 / al_t;
  o->c[1] = sg_t / al_t;
  if (as >= 1.0) {          // into sigma = 0: x' = x0 (first order)
    o->c[3] = 1.0;
    return;
  }
  const double al_s = std::sqrt(as), sg_s = std::sqrt(1.0 - as);
  const double h = half_log_snr(as) - half_log_snr(at);
  const double b = al_s * -std::expm1(-h);
  o->c[2] = sg_s / sg_t;
  if (k >= 1) {
    const double ap = ab[kept_step(sp, k - 1)];
    const double r = (half_log_snr(at) - half_log_snr(ap)) / h;
    o->c[3] = b * (1.0 + 0.5 / r);
    o->c[4] = b * (-0.5 / r);
    o->c[5] = 1.0;
  } else {
    o->c[3] = b;
  }
}

void fill_step_args(SamplerStepArgs* a, int kind, const StepCoef& sc) {
  a->kind = kind;
  for (int i = 0; i < 5; ++i) a->k[i] = (float)sc.c[i];
  if (kind == DIT_SAMPLER_DDPM) {
    a->add_noise = sc.c[4] != 0.0;
  } else if (kind == DIT_SAMPLER_DPMPP_2M) {
    a->has_prev = sc.c[5] != 0.0;
  }
}

struct SampleLayout {
  WsLayout L;
  size_t tvec, xm, hist, total;
};

SampleLayout sample_layout(const dit_handle* h, int kind, int B, int rows) {
  SampleLayout S;
  S.L = ws_layout(h, rows);
  size_t off = S.L.total;
  const size_t n = (size_t)B * h->cfg.in_channels * h->gin.F * h->gin.H * h->gin.W;
  S.tvec = off; off += align256((size_t)B * 4);
  S.xm = off; off += align256(h->dtype == DIT_BF16 ? n * 2 : 0);
  S.hist = off; off += align256(kind == DIT_SAMPLER_DPMPP_2M ? n * 4 : 0);
  S.total = off;
  return S;
}

int check_sample_model(int C, int Cout) {
  if (Cout != C && Cout != 2 * C)
    return fail(DIT_EUNSUPPORTED, "sampler needs Cout == C or 2C (got C = %d, Cout = %d)", C, Cout);
  return DIT_OK;
}
int sample_rows(const dit_handle* h, int B, int guided, int* rows) {
  if (B <= 0 || B > (1 << 29)) return fail(DIT_EINVAL, "B must be positive (got %d)", B);
  if (guided < 0 || guided > h->cfg.out_channels)
    return fail(DIT_EINVAL, "guided_channels must be in [0, %d]", h->cfg.out_channels);
  if (guided > 0) {
    if (h->ncls <= 0) return fail(DIT_EINVAL, "guidance needs a class table with a null label");
    if (h->cond_dim > 0) return fail(DIT_EUNSUPPORTED, "guidance with pooled conditioning");
  }
  *rows = guided > 0 ? 2 * B : B;
  return DIT_OK;
}

// Packed sequences: validation and token offsets.  seq_fhw: host [nseq, 3].
int check_packed(const dit_handle* h, int nseq, const int32_t* seq_fhw, SeqTable* st,
                 int64_t* x_elems, int64_t* out_elems) {
  if (!seq_fhw) return fail(DIT_EINVAL, "seq_fhw must be non-NULL");
  if (nseq < 1 || nseq > kMaxSeq) return fail(DIT_EINVAL, "nseq must be in [1, %d]", kMaxSeq);
  if (h->cond != DIT_COND_ADALN_ZERO)
    return fail(DIT_EUNSUPPORTED, "packed sequences need the adaLN-Zero design");
  if (h->cfg.rope3d) return fail(DIT_EUNSUPPORTED, "packed sequences need 2-D position embedding");
  const dit_config& c = h->cfg;
  st->n = nseq;
  st->tok[0] = 0;
  int64_t xe = 0, oe = 0;
  for (int j = 0; j < nseq; ++j) {
    const int F = seq_fhw[3 * j], H = seq_fhw[3 * j + 1], W = seq_fhw[3 * j + 2];
    if (F != c.patch_t || H <= 0 || W <= 0 || H % c.patch || W % c.patch)
      return fail(DIT_EINVAL, "sequence %d: extents (%d, %d, %d) need F = %d and H, W divisible by %d",
                  j, F, H, W, c.patch_t, c.patch);
    const int64_t T = (int64_t)(H / c.patch) * (W / c.patch);
    if (T % 32) return fail(DIT_EUNSUPPORTED, "sequence %d: %lld tokens, not a multiple of 32", j,
                            (long long)T);
    if (st->tok[j] + T > (1 << 26)) return fail(DIT_EINVAL, "too many packed tokens");
    st->tok[j + 1] = (int)(st->tok[j] + T);
    xe += (int64_t)c.in_channels * F * H * W;
    oe += (int64_t)c.out_channels * F * H * W;
  }
  if ((int64_t)st->tok[nseq] * h->heads > (1LL << 31)) return fail(DIT_EINVAL, "too many tokens");
  *x_elems = xe;
  *out_elems = oe;
  return DIT_OK;
}

}  // namespace

extern "C" {

const char* dit_status_string(int status) {
  switch (status) {
    case DIT_OK: return "ok";
    case DIT_EINVAL: return "invalid argument";
    case DIT_EUNSUPPORTED: return "unsupported configuration";
    case DIT_EWORKSPACE: return "workspace missing or too small";
    case DIT_EHIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* dit_last_error_message(void) { return g_err.c_str(); }

int dit_create(const dit_config* cfg, const dit_weights* w, dit_handle** out) {
  if (!cfg || !w || !out) return fail(DIT_EINVAL, "cfg, w and out must be non-NULL");
  *out = nullptr;
  const dit_config& c = *cfg;
  if (c.in_channels <= 0 || c.out_channels <= 0 || c.frames <= 0 || c.height <= 0 ||
      c.width <= 0 || c.patch <= 0 || c.patch_t <= 0 || c.hidden <= 0 || c.depth <= 0 ||
      c.heads <= 0 || c.mlp_hidden <= 0 || c.freq_dim <= 0 || c.num_classes < 0 ||
      c.cond_dim < 0)
    return fail(DIT_EINVAL, "config sizes must be positive");
  if (c.freq_dim % 2) return fail(DIT_EINVAL, "freq_dim must be even");
  if (c.dtype != DIT_F32 && c.dtype != DIT_BF16) return fail(DIT_EINVAL, "dtype must be F32 or BF16");
  if (!(c.ln_eps > 0.0f) || !std::isfinite(c.ln_eps)) return fail(DIT_EINVAL, "ln_eps must be > 0");
  if (c.height % c.patch || c.width % c.patch || c.frames % c.patch_t)
    return fail(DIT_EINVAL, "latent extents not divisible by the patch size");
  if (c.hidden % c.heads) return fail(DIT_EINVAL, "hidden %% heads != 0");
  const int dh = c.hidden / c.heads;
  if (dh != 64 && dh != 72) return fail(DIT_EUNSUPPORTED, "head dim %d (supported: 64, 72)", dh);
  if (c.hidden % 128 || c.hidden > 2048)
    return fail(DIT_EUNSUPPORTED, "hidden %d (supported: multiple of 128, <= 2048)", c.hidden);
  if (c.mlp_hidden % 64) return fail(DIT_EUNSUPPORTED, "mlp_hidden must be a multiple of 64");
  const int gf = c.frames / c.patch_t;
  if (!c.rope3d && gf != 1)
    return fail(DIT_EUNSUPPORTED, "2-D position embedding needs frames / patch_t == 1");
  if (c.rope3d && (dh % 6 || (dh / 3) % 2))
    return fail(DIT_EUNSUPPORTED, "3-D RoPE needs head dim divisible by 6 with even thirds");
  if (c.qk_norm != 0 && c.qk_norm != 1) return fail(DIT_EINVAL, "qk_norm must be 0 or 1");
  if (c.rope3d != 0 && c.rope3d != 1) return fail(DIT_EINVAL, "rope3d must be 0 or 1");
  if (c.conditioning < DIT_COND_ADALN_ZERO || c.conditioning > DIT_COND_MMDIT)
    return fail(DIT_EINVAL, "unknown conditioning design %d", c.conditioning);
  const bool mm = c.conditioning == DIT_COND_MMDIT;
  const bool ada = c.conditioning == DIT_COND_ADALN_ZERO || mm;
  const bool xattn = c.conditioning == DIT_COND_CROSS_ATTN;
  if (mm) {
    if (c.num_classes != 0 || c.cond_dim <= 0)
      return fail(DIT_EUNSUPPORTED, "the MMDiT design takes a pooled vector and no class table");
    if (c.ctx_len <= 0 || c.ctx_dim <= 0 || c.ctx_dim % 64)
      return fail(DIT_EUNSUPPORTED, "MMDiT needs ctx_len > 0 and ctx_dim a positive multiple of 64");
    if (c.rope3d || c.qk_norm || gf != 1)
      return fail(DIT_EUNSUPPORTED, "MMDiT takes images (frames / patch_t == 1), no RoPE or qk_norm");
    if (!w->ctx_w || !w->ctx_b || !w->cada_w || !w->cada_b || !w->cqkv_w || !w->cqkv_b ||
        !w->co_w || !w->co_b || !w->cfc1_w || !w->cfc1_b || !w->cfc2_w || !w->cfc2_b ||
        !w->qk_rms)
      return fail(DIT_EINVAL, "an MMDiT weight pointer is NULL");
    const void* mp[] = {w->ctx_w, w->cada_w, w->cqkv_w, w->co_w, w->cfc1_w, w->cfc2_w};
    for (const void* p : mp)
      if ((uintptr_t)p & 15) return fail(DIT_EINVAL, "GEMM weights must be 16-byte aligned");
  } else if (c.ctx_len != 0 || c.ctx_dim != 0) {
    return fail(DIT_EINVAL, "ctx_len / ctx_dim are for the MMDiT design only (set them to 0)");
  }
  if (!ada && (c.num_classes <= 0 || c.cond_dim > 0))
    return fail(DIT_EUNSUPPORTED,
                "the in-context and cross-attention designs need a class table and no pooled "
                "conditioning");
  if (!w->pe_w || !w->pe_b || !w->t1_w || !w->t1_b || !w->t2_w || !w->t2_b || !w->qkv_w ||
      !w->qkv_b || !w->o_w || !w->o_b || !w->fc1_w || !w->fc1_b || !w->fc2_w || !w->fc2_b ||
      !w->out_w || !w->out_b)
    return fail(DIT_EINVAL, "a required weight pointer is NULL");
  if (ada && (!w->ada_w || !w->ada_b)) return fail(DIT_EINVAL, "ada_w/ada_b NULL");
  if (!ada && (!w->ln_p || !w->final_ln)) return fail(DIT_EINVAL, "ln_p/final_ln NULL");
  if (xattn && (!w->xq_w || !w->xq_b || !w->xkv_w || !w->xkv_b || !w->xo_w || !w->xo_b))
    return fail(DIT_EINVAL, "a cross-attention weight pointer is NULL");
  if (c.num_classes > 0 && !w->y_table) return fail(DIT_EINVAL, "y_table is NULL");
  if (c.cond_dim > 0 && (!w->pool_w || !w->pool_b)) return fail(DIT_EINVAL, "pool_w/pool_b NULL");
  const void* ptrs[] = {w->qkv_w, w->o_w, w->fc1_w, w->fc2_w, w->ada_w, w->xq_w, w->xkv_w,
                        w->xo_w};
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return fail(DIT_EINVAL, "GEMM weights must be 16-byte aligned");
  const int64_t T = (int64_t)gf * (c.height / c.patch) * (c.width / c.patch);
  if (T + (mm ? c.ctx_len : 0) > (1 << 26)) return fail(DIT_EINVAL, "too many tokens");

  dit_handle* h = new (std::nothrow) dit_handle;
  if (!h) return fail(DIT_EINVAL, "out of host memory");
  h->cfg = c;
  h->w = *w;
  h->d = c.hidden; h->N = c.depth; h->heads = c.heads; h->dh = dh; h->hid = c.mlp_hidden;
  h->ncls = c.num_classes; h->cond_dim = c.cond_dim; h->freq = c.freq_dim; h->dtype = c.dtype;
  h->es = c.dtype == DIT_BF16 ? 2 : 4;
  h->eps = c.ln_eps;
  h->gf = gf; h->gh = c.height / c.patch; h->gw = c.width / c.patch;
  h->T = (int)T;
  h->kin = c.patch_t * c.patch * c.patch * c.in_channels;
  h->kout = c.patch_t * c.patch * c.patch * c.out_channels;
  h->cond = c.conditioning;
  h->Lc = mm ? c.ctx_len : 0;
  h->Tt = h->T + (c.conditioning == DIT_COND_IN_CONTEXT ? 2 : 0) + h->Lc;
  h->Tf = mm ? h->T : h->Tt;
  h->nln = xattn ? 3 : 2;
  h->mod_stride = ada ? (6 * c.depth + 2) * c.hidden : 0;
  h->gin = make_geom(c.in_channels, c.frames, c.height, c.width, c.patch, c.patch_t);
  h->gout = make_geom(c.out_channels, c.frames, c.height, c.width, c.patch, c.patch_t);
  h->gouty = h->gout;
  h->gouty.T = h->Tf;
  *out = h;
  return ok();
}

void dit_destroy(dit_handle* h) { delete h; }

int dit_workspace_size(const dit_handle* h, int rows, size_t* bytes) {
  if (!h || !bytes) return fail(DIT_EINVAL, "handle and bytes must be non-NULL");
  if (rows <= 0) return fail(DIT_EINVAL, "rows must be positive");
  *bytes = ws_layout(h, rows).total;
  return ok();
}

int dit_forward(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                const float* pooled, int B, float* out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(h, x_t, t, y, pooled, nullptr, B, out, nullptr, ws, ws_bytes, stream);
}

int dit_forward_taps(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                     const float* pooled, int B, float* out, const dit_taps* taps, void* ws,
                     size_t ws_bytes, void* stream) {
  return forward_impl(h, x_t, t, y, pooled, nullptr, B, out, taps, ws, ws_bytes, stream);
}

int dit_forward_ctx(dit_handle* h, const void* x_t, const float* t, const float* pooled,
                    const void* ctx, int B, float* out, const dit_taps* taps, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DIT_EINVAL, "ctx must be non-NULL");
  return forward_impl(h, x_t, t, nullptr, pooled, ctx, B, out, taps, ws, ws_bytes, stream);
}

int dit_cfg_forward(dit_handle* h, const void* x_t, const float* t, const int32_t* y, int Bh,
                    float s, int guided_channels, float* out, void* ws, size_t ws_bytes,
                    void* stream) {
  return cfg_forward_impl(h, x_t, t, y, Bh, s, guided_channels, out, nullptr, ws, ws_bytes,
                          stream);
}

int dit_cfg_forward_taps(dit_handle* h, const void* x_t, const float* t, const int32_t* y,
                         int Bh, float s, int guided_channels, float* out,
                         const dit_taps* taps, void* ws, size_t ws_bytes, void* stream) {
  return cfg_forward_impl(h, x_t, t, y, Bh, s, guided_channels, out, taps, ws, ws_bytes, stream);
}

int dit_patchify(const void* x, int B, int C, int F, int H, int W, int p, int pt, int dtype,
                 void* P, void* stream) {
  if (!x || !P) return fail(DIT_EINVAL, "x and P must be non-NULL");
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EINVAL, "dtype");
  int rc = check_geom(B, C, F, H, W, p, pt);
  if (rc) return rc;
  DIT_HIP(launch_patchify(x, B, make_geom(C, F, H, W, p, pt), dtype, P, (hipStream_t)stream));
  return ok();
}

int dit_unpatchify(const float* Y, int B, int Cout, int F, int H, int W, int p, int pt,
                   float* out, void* stream) {
  if (!Y || !out) return fail(DIT_EINVAL, "Y and out must be non-NULL");
  int rc = check_geom(B, Cout, F, H, W, p, pt);
  if (rc) return rc;
  DIT_HIP(launch_unpatchify(Y, B, 0, make_geom(Cout, F, H, W, p, pt), Cout, 0, 0.0f, 0, out,
                            (hipStream_t)stream));
  return ok();
}

int dit_timestep_embed(const float* t, int B, int dim, float* e, void* stream) {
  if (!t || !e) return fail(DIT_EINVAL, "t and e must be non-NULL");
  if (B <= 0 || dim <= 0 || dim % 2) return fail(DIT_EINVAL, "B > 0 and even dim > 0 required");
  DIT_HIP(launch_timestep_embed(t, B, B, dim, e, (hipStream_t)stream));
  return ok();
}

int dit_attention(const void* qkv, int B, int H, int T, int dh, int dtype, void* o,
                  void* stream) {
  if (!qkv || !o) return fail(DIT_EINVAL, "qkv and o must be non-NULL");
  if (B <= 0 || H <= 0 || T <= 0) return fail(DIT_EINVAL, "B, H, T must be positive");
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EINVAL, "dtype");
  if (dh != 64 && dh != 72) return fail(DIT_EUNSUPPORTED, "head dim %d", dh);
  if ((int64_t)B * H > 65535) return fail(DIT_EUNSUPPORTED, "B * H > 65535");
  if ((uintptr_t)qkv & 15) return fail(DIT_EINVAL, "qkv must be 16-byte aligned");
  if ((uintptr_t)o & 7) return fail(DIT_EINVAL, "o must be 8-byte aligned");
  // one (row, head) slice is addressed with 32-bit byte offsets
  if ((int64_t)T * 3 * H * dh * 4 >= (int64_t)1 << 31)
    return fail(DIT_EUNSUPPORTED, "T * 3 H dh too large for one row");
  DIT_HIP(launch_attention(qkv, B, H, T, dh, dtype, o, (hipStream_t)stream));
  return ok();
}

int dit_linear(int epilogue, const void* A, const void* W, const float* bias, int M, int N,
               int K, int dtype, void* out, const float* gate, int gate_stride, int T,
               void* stream) {
  if (!A || !W || !out) return fail(DIT_EINVAL, "A, W and out must be non-NULL");
  if (M <= 0 || N <= 0 || K <= 0) return fail(DIT_EINVAL, "M, N, K must be positive");
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EINVAL, "dtype");
  int epi;
  switch (epilogue) {
    case DIT_EPI_BIAS: epi = EPI_BIAS_F32; break;
    case DIT_EPI_GELU: epi = EPI_GELU; break;
    case DIT_EPI_GATED: epi = EPI_GATED; break;
    case DIT_EPI_ACCUM: epi = EPI_ATOMIC_F32; break;
    case DIT_EPI_BIAS_DT: epi = EPI_BIAS_DT; break;
    default: return fail(DIT_EINVAL, "unknown epilogue %d", epilogue);
  }
  if (epilogue == DIT_EPI_ACCUM && bias)
    return fail(DIT_EINVAL, "the accumulating epilogue takes no bias");
  if (epilogue == DIT_EPI_GATED && (!gate || T <= 0 || gate_stride < N))
    return fail(DIT_EINVAL, "gated epilogue needs gate, T > 0 and gate_stride >= N");
  if (dtype == DIT_BF16 && (K % 64 || ((uintptr_t)A & 15) || ((uintptr_t)W & 15)))
    return fail(DIT_EUNSUPPORTED, "bf16 linear needs K %% 64 == 0 and 16-byte aligned A, W");
  EpiParams ep = epi0();
  ep.bias = bias; ep.out = out; ep.ldo = N;
  ep.mod = gate; ep.mod_stride = gate_stride; ep.gate_off = 0; ep.T = T > 0 ? T : 1;
  if (epilogue == DIT_EPI_ACCUM) ep.ksplit = splitk_slice(dtype == DIT_BF16, M, N, K);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == DIT_BF16) {
    DIT_HIP(launch_gemm_mfma(epi, (const bf16_t*)A, K, (const bf16_t*)W, M, N, K, ep, s));
  } else {
    ALoad a;
    memset(&a, 0, sizeof a);
    a.ptr = A; a.lda = K; a.a_dtype = 0; a.src_rows = M;
    DIT_HIP(launch_gemm_valu(epi, A_PLAIN, a, W, 0, M, N, K, ep, s));
  }
  return ok();
}

int dit_ln_modulate(const float* X, int M, int T, int d, const float* mod, int mod_stride,
                    int shift_off, int scale_off, float eps, void* H, int dtype, void* stream) {
  if (!X || !mod || !H) return fail(DIT_EINVAL, "X, mod and H must be non-NULL");
  if (M <= 0 || T <= 0 || d <= 0) return fail(DIT_EINVAL, "M, T, d must be positive");
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EINVAL, "dtype");
  if (mod_stride < 0 || shift_off < 0 || scale_off < 0 ||
      (mod_stride > 0 && (shift_off + d > mod_stride || scale_off + d > mod_stride)))
    return fail(DIT_EINVAL, "the shift / scale vectors must lie inside a modulation row");
  if (d % 128 || d > 2048 || !(eps > 0.0f))
    return fail(DIT_EUNSUPPORTED, "LayerNorm width must be a multiple of 128 up to 2048, eps > 0");
  if (((uintptr_t)X & 15) || ((uintptr_t)H & 15) || ((uintptr_t)mod & 15) || mod_stride % 4 ||
      shift_off % 4 || scale_off % 4)
    return fail(DIT_EINVAL, "X, H and mod must be 16-byte aligned, mod_stride and the offsets "
                            "multiples of 4");
  DIT_HIP(launch_ln_modulate(X, M, T, d, mod, mod_stride, shift_off, scale_off, eps, H, dtype,
                             (hipStream_t)stream));
  return ok();
}

int dit_linear_wgrad(const void* dY, int64_t ldy, const void* X, int64_t ldx, int N, int K,
                     int64_t R, int dtype, float* dW, float* db, void* stream) {
  if (!dY || !X || !dW) return fail(DIT_EINVAL, "dY, X and dW must be non-NULL");
  if (N <= 0 || K <= 0 || R < 0) return fail(DIT_EINVAL, "N, K must be positive and R >= 0");
  if (ldy < N || ldx < K) return fail(DIT_EINVAL, "row strides ldy >= N and ldx >= K");
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EINVAL, "dtype");
  if (R > INT32_MAX || ldy > INT32_MAX || ldx > INT32_MAX)
    return fail(DIT_EUNSUPPORTED, "R and the row strides must be below 2^31");
  const bool tn = dtype == DIT_BF16 && N % 8 == 0 && K % 8 == 0 && R % 64 == 0 && ldy % 8 == 0 &&
                  ldx % 8 == 0 && ((uintptr_t)dY & 15) == 0 && ((uintptr_t)X & 15) == 0 &&
                  R * (ldy > ldx ? ldy : ldx) <= INT32_MAX;
  if (db && dtype == DIT_BF16 && !tn && (N % 8 || ldy % 8 || ((uintptr_t)dY & 15)))
    return fail(DIT_EUNSUPPORTED, "bf16 bias gradient needs N, ldy multiples of 8 and aligned dY");
  if (db && dtype == DIT_BF16 && !tn && R > kColsumTallMaxRows)
    return fail(DIT_EUNSUPPORTED, "bf16 bias gradient of more than %lld rows",
                (long long)kColsumTallMaxRows);
  DIT_HIP(linear_wgrad(dY, ldy, X, ldx, N, K, R, dtype, dW, K, db, (hipStream_t)stream));
  return ok();
}

int dit_block_forward(dit_handle* h, int layer, int B, const float* X_in, const float* mod,
                      float* X_out, float* o_branch, float* f_branch, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (!X_in || !mod || !X_out) return fail(DIT_EINVAL, "X_in, mod and X_out must be non-NULL");
  if (layer < 0 || layer >= h->N) return fail(DIT_EINVAL, "layer %d out of range", layer);
  if (B <= 0) return fail(DIT_EINVAL, "B must be positive");
  if (h->cond != DIT_COND_ADALN_ZERO)
    return fail(DIT_EUNSUPPORTED, "dit_block_forward runs adaLN-Zero blocks only");
  WsLayout L;
  int rc = check_ws(h, B, ws, ws_bytes, &L);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (X_out != X_in)
    DIT_HIP(hipMemcpyAsync(X_out, X_in, (size_t)B * h->T * h->d * 4, hipMemcpyDeviceToDevice, s));
  rc = run_block(h, layer, B, X_out, mod, 6 * h->d, 0, ws, L, o_branch, f_branch, s);
  if (rc) return rc;
  return ok();
}

int dit_launch_timer_start(unsigned kinds_mask, int capacity) {
  if (kinds_mask == 0 || (kinds_mask >> DIT_TIMER_KINDS) != 0)
    return fail(DIT_EINVAL, "kinds_mask 0x%x: needs a DIT_TIMER_* bit and no other", kinds_mask);
  if (capacity < 1 || capacity > 65536)
    return fail(DIT_EINVAL, "capacity %d outside [1, 65536]", capacity);
  timer_release(tl_timer);
  LaunchTimer t;
  t.ev = new (std::nothrow) hipEvent_t[2 * (size_t)capacity]();
  t.kinds = new (std::nothrow) int[capacity]();
  t.cap = capacity;
  if (!t.ev || !t.kinds) {
    timer_release(t);
    return fail(DIT_EHIP, "launch timer: no host memory for %d event pairs", capacity);
  }
  // Timing-only events: no system-scope fence (cache writeback and
  // invalidation) at each record, which would slow the launches after it.
  for (int i = 0; i < 2 * capacity; ++i) {
    const hipError_t e = hipEventCreateWithFlags(&t.ev[i], hipEventDisableSystemFence);
    if (e != hipSuccess) {
      t.ev[i] = nullptr;
      timer_release(t);
      return fail(DIT_EHIP, "launch timer: hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  t.mask = kinds_mask;
  tl_timer = t;
  return ok();
}

int dit_launch_timer_stop(int* kinds, float* ms, int cap, int* count) {
  if (!count) return fail(DIT_EINVAL, "count must be non-NULL");
  if (cap < 0 || (cap > 0 && (!kinds || !ms)))
    return fail(DIT_EINVAL, "cap %d needs kinds and ms of that length", cap);
  *count = 0;
  LaunchTimer& t = tl_timer;
  if (!t.ev) return ok();
  const int n = t.used;
  hipError_t err = hipSuccess;
  // every recorded event completes before the events are released
  for (int i = 0; i < 2 * n + (t.open ? 1 : 0) && err == hipSuccess; ++i)
    err = hipEventSynchronize(t.ev[i]);
  for (int i = 0; i < n && i < cap && err == hipSuccess; ++i) {
    err = hipEventElapsedTime(&ms[i], t.ev[2 * i], t.ev[2 * i + 1]);
    kinds[i] = t.kinds[i];
  }
  timer_release(t);
  if (err != hipSuccess) return fail(DIT_EHIP, "launch timer: %s", hipGetErrorString(err));
  *count = n;
  return ok();
}


int dit_sampler_coefficients(const dit_sampler* sp, int k, double* model_t, double coef[8]) {
  int rc = check_sampler(sp);
  if (rc) return rc;
  if (k < 0 || k >= sp->num_steps) return fail(DIT_EINVAL, "step %d outside [0, %d)", k, sp->num_steps);
  if (!model_t || !coef) return fail(DIT_EINVAL, "model_t and coef must be non-NULL");
  std::vector<double> ab;
  if (sp->kind != DIT_SAMPLER_RF_EULER) ab = abar_table(sp);
  StepCoef sc;
  step_coef(sp, ab, k, &sc);
  *model_t = sc.model_t;
  for (int i = 0; i < 8; ++i) coef[i] = sc.c[i];
  return ok();
}

int dit_sampler_step(const dit_sampler* sp, int k, const float* x, const float* model_out, int B,
                     int C, int Cout, int64_t spatial, const float* z, float* x0_hist,
                     float* x_out, void* stream) {
  int rc = check_sampler(sp);
  if (rc) return rc;
  if (k < 0 || k >= sp->num_steps) return fail(DIT_EINVAL, "step %d outside [0, %d)", k, sp->num_steps);
  if (!x || !model_out || !x_out) return fail(DIT_EINVAL, "x, model_out and x_out must be non-NULL");
  if (B <= 0 || C <= 0 || spatial <= 0) return fail(DIT_EINVAL, "B, C and spatial must be positive");
  rc = check_sample_model(C, Cout);
  if (rc) return rc;
  const int64_t n = (int64_t)B * C * spatial;
  if (n > (1LL << 38)) return fail(DIT_EINVAL, "state too large");
  std::vector<double> ab;
  if (sp->kind != DIT_SAMPLER_RF_EULER) ab = abar_table(sp);
  StepCoef sc;
  step_coef(sp, ab, k, &sc);
  SamplerStepArgs a;
  memset(&a, 0, sizeof a);
  fill_step_args(&a, sp->kind, sc);
  if (a.add_noise && !z) return fail(DIT_EINVAL, "this DDPM step needs noise z");
  if (sp->kind == DIT_SAMPLER_DPMPP_2M && !x0_hist)
    return fail(DIT_EINVAL, "DPM-Solver++ needs the x0 history buffer");
  a.x = x; a.x_out = x_out; a.mo = model_out; a.z = z;
  a.hist = sp->kind == DIT_SAMPLER_DPMPP_2M ? x0_hist : nullptr;
  a.n = n; a.S = spatial; a.C = C; a.Cout = Cout;
  a.learned = Cout == 2 * C;
  DIT_HIP(launch_sampler_step(a, (hipStream_t)stream));
  return ok();
}


int dit_sample_workspace_size(const dit_handle* h, const dit_sampler* sp, int B,
                              int guided_channels, size_t* bytes) {
  if (!h || !bytes) return fail(DIT_EINVAL, "handle and bytes must be non-NULL");
  int rc = check_sampler(sp);
  if (rc) return rc;
  int rows;
  rc = sample_rows(h, B, guided_channels, &rows);
  if (rc) return rc;
  rc = check_rows(h, rows);
  if (rc) return rc;
  *bytes = sample_layout(h, sp->kind, B, rows).total;
  return ok();
}

int dit_sample(dit_handle* h, const dit_sampler* sp, float* x, const int32_t* y,
               const float* pooled, int B, float scale, int guided_channels, const float* noise,
               void* ws, size_t ws_bytes, void* stream) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  int rc = check_sampler(sp);
  if (rc) return rc;
  if (!x) return fail(DIT_EINVAL, "x must be non-NULL");
  if (h->cond == DIT_COND_MMDIT)
    return fail(DIT_EUNSUPPORTED, "the sampling loop does not take text embeddings (MMDiT)");
  const int C = h->cfg.in_channels, Cout = h->cfg.out_channels, S = sp->num_steps;
  rc = check_sample_model(C, Cout);
  if (rc) return rc;
  int rows;
  rc = sample_rows(h, B, guided_channels, &rows);
  if (rc) return rc;
  if (h->ncls > 0 && !y) return fail(DIT_EINVAL, "class labels y are required");
  if (guided_channels == 0 && h->cond_dim > 0 && !pooled)
    return fail(DIT_EINVAL, "pooled conditioning is required");
  if (guided_channels > 0 && !std::isfinite(scale))
    return fail(DIT_EINVAL, "guidance scale must be finite");
  if (sp->kind == DIT_SAMPLER_DDPM && S >= 2 && !noise)
    return fail(DIT_EINVAL, "DDPM sampling needs noise [S, B, C, F, H, W]");
  rc = check_rows(h, rows);
  if (rc) return rc;
  const SampleLayout SL = sample_layout(h, sp->kind, B, rows);
  rc = check_ws_bytes(ws, ws_bytes, SL.total);
  if (rc) return rc;
  const WsLayout& L = SL.L;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)B * C * h->gin.F * h->gin.H * h->gin.W;
  std::vector<double> ab;
  if (sp->kind != DIT_SAMPLER_RF_EULER) ab = abar_table(sp);
  std::vector<StepCoef> co(S);
  for (int k = 0; k < S; ++k) step_coef(sp, ab, k, &co[k]);

  float* tvec = at<float>(ws, SL.tvec);
  bf16_t* xm = h->dtype == DIT_BF16 ? at<bf16_t>(ws, SL.xm) : nullptr;
  float* hist = sp->kind == DIT_SAMPLER_DPMPP_2M ? at<float>(ws, SL.hist) : nullptr;
  DIT_HIP(launch_sampler_prologue(x, n, xm, tvec, B, (float)co[0].model_t, s));
  const void* x_in = xm ? (const void*)xm : (const void*)x;
  for (int k = 0; k < S; ++k) {
    if (guided_channels > 0)
      rc = run_trunk(h, x_in, tvec, y, nullptr, nullptr, rows, B, B, ws, L, nullptr, s);
    else
      rc = run_trunk(h, x_in, tvec, y, pooled, nullptr, B, B, B, ws, L, nullptr, s);
    if (rc) return rc;
    SamplerStepArgs a;
    memset(&a, 0, sizeof a);
    fill_step_args(&a, sp->kind, co[k]);
    const bool more = k + 1 < S;
    a.from_y = 1;
    a.x = x; a.x_out = x;
    a.x_model = more ? xm : nullptr;
    a.mo = at<float>(ws, L.Y);
    a.z = a.add_noise ? noise + (size_t)k * n : nullptr;
    a.hist = hist;
    a.tvec = more ? tvec : nullptr;
    a.tvec_rows = more ? B : 0;
    a.t_next = more ? (float)co[k + 1].model_t : 0.0f;
    a.n = n; a.S = (int64_t)h->gin.F * h->gin.H * h->gin.W;
    a.C = C; a.Cout = Cout; a.g = h->gouty;
    a.null_off = B; a.guided = guided_channels; a.scale = scale;
    a.learned = Cout == 2 * C;
    DIT_HIP(launch_sampler_step(a, s));
  }
  return ok();
}


int dit_packed_workspace_size(const dit_handle* h, int nseq, const int32_t* seq_fhw,
                              size_t* bytes) {
  if (!h || !bytes) return fail(DIT_EINVAL, "handle and bytes must be non-NULL");
  SeqTable st;
  int64_t xe, oe;
  int rc = check_packed(h, nseq, seq_fhw, &st, &xe, &oe);
  if (rc) return rc;
  *bytes = ws_layout_m(h, nseq, (size_t)st.tok[nseq], true).total;
  return ok();
}

int dit_forward_packed(dit_handle* h, int nseq, const int32_t* seq_fhw, const void* x,
                       const float* t, const int32_t* y, const float* pooled, float* out,
                       void* ws, size_t ws_bytes, void* stream) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (!x || !t || !out) return fail(DIT_EINVAL, "x, t and out must be non-NULL");
  if (h->ncls > 0 && !y) return fail(DIT_EINVAL, "class labels y are required");
  if (h->cond_dim > 0 && !pooled) return fail(DIT_EINVAL, "pooled conditioning is required");
  Packed pk;
  int64_t xe, oe;
  int rc = check_packed(h, nseq, seq_fhw, &pk.seqs, &xe, &oe);
  if (rc) return rc;
  pk.M = pk.seqs.tok[nseq];
  const WsLayout L = ws_layout_m(h, nseq, (size_t)pk.M, true);
  rc = check_ws_bytes(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int d = h->d, C = h->cfg.in_channels, Cout = h->cfg.out_channels;
  const int p = h->cfg.patch, pt = h->cfg.patch_t;
  float* X = at<float>(ws, L.X);
  float* Y = at<float>(ws, L.Y);
  float* pe = at<float>(ws, L.pe);
  int* seg = at<int>(ws, L.seg);
  pk.tok_seg = seg;

  rc = run_conditioning(h, t, y, pooled, nseq, nseq, nseq, ws, L, s);
  if (rc) return rc;
  // Per sequence: its token -> sequence map, its position table and its patch
  // embedding (the patch gather reads its own latent extents).
  int64_t xoff = 0;
  for (int j = 0; j < nseq; ++j) {
    const int F = seq_fhw[3 * j], H = seq_fhw[3 * j + 1], W = seq_fhw[3 * j + 2];
    const int t0 = pk.seqs.tok[j], Tj = pk.seqs.tok[j + 1] - t0;
    DIT_HIP(launch_fill_int(seg + t0, Tj, j, s));
    DIT_HIP(launch_pos_embed_table(H / p, W / p, d, pe + (size_t)t0 * d, s));
    DIT_HIP(patch_embed(h, (const char*)x + xoff * h->es, 1, make_geom(C, F, H, W, p, pt),
                        pe + (size_t)t0 * d, Tj, 0, X + (size_t)t0 * d, s));
    xoff += (int64_t)C * F * H * W;
  }
  const float* mod = at<float>(ws, L.mod);
  const int fb = 6 * d * h->N;
  // Blocks and the final layer of the sequences [j0, j1): their tokens are a
  // contiguous range, so every workspace region is offset by its first token.
  auto group = [&](int j0, int j1, hipStream_t st) -> int {
    Packed g;
    const int tok0 = pk.seqs.tok[j0];
    g.seqs.n = j1 - j0;
    for (int j = j0; j <= j1; ++j) g.seqs.tok[j - j0] = pk.seqs.tok[j] - tok0;
    g.M = g.seqs.tok[g.seqs.n];
    g.tok_seg = seg + tok0;
    const size_t m0 = tok0, es = h->es;
    WsLayout Lg = L;
    Lg.H += m0 * d * es;
    Lg.qkv += m0 * 3 * d * es;
    Lg.o += m0 * d * es;
    Lg.G += m0 * h->hid * es;
    float* Xg = X + m0 * d;
    for (int l = 0; l < h->N; ++l) {
      int r = run_block(h, l, g.seqs.n, Xg, mod, h->mod_stride, 6 * d * l, ws, Lg, nullptr,
                        nullptr, st, &g);
      if (r) return r;
    }
    void* Hg = at<void>(ws, Lg.H);
    DIT_HIP(launch_ln_modulate(Xg, g.M, h->T, d, mod, h->mod_stride, fb, fb + d, h->eps, Hg,
                               h->dtype, st, g.tok_seg));
    EpiParams ef = epi0();
    ef.bias = h->w.out_b; ef.out = Y + m0 * h->kout; ef.ldo = h->kout;
    DIT_HIP(linear(h, EPI_BIAS_F32, Hg, d, h->w.out_w, g.M, h->kout, d, ef, st));
    return DIT_OK;
  };
  rc = group(0, nseq, s);
  if (rc) return rc;
  int64_t ooff = 0;
  for (int j = 0; j < nseq; ++j) {
    const int F = seq_fhw[3 * j], H = seq_fhw[3 * j + 1], W = seq_fhw[3 * j + 2];
    const PatchGeom g = make_geom(Cout, F, H, W, p, pt);
    DIT_HIP(launch_unpatchify(Y + (size_t)pk.seqs.tok[j] * h->kout, 1, 0, g, Cout, 0, 0.0f, 0,
                              out + ooff, s));
    ooff += (int64_t)Cout * F * H * W;
  }
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Forward without a caller workspace, for callers that cannot allocate device
// memory: code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation.  The workspace is a file-scope device array of
// kNoallocScratchBytes; every GPU the library is loaded on holds its own copy
// until the process ends.  The host uses only the address that
// hipGetSymbolAddress returns for the current device (taken at the first call
// on that device), never the array's name.  Calls on one GPU share the array:
// calls that overlap on one GPU race.  The forward writes every workspace
// region before reading it, so nothing needs clearing between calls.
namespace {
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DIT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DIT_EUNSUPPORTED, "device ordinal %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DIT_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DIT_OK;
}
}  // namespace

extern "C" int dit_forward_noalloc(dit_handle* h, const void* x_t, const float* t,
                                   const int32_t* y, const float* pooled, int B, float* out,
                                   void* stream) {
  // Everything dit_forward checks, and the size limit, before any HIP call.
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (!x_t || !t || !out) return fail(DIT_EINVAL, "x_t, t and out must be non-NULL");
  if (h->cond == DIT_COND_MMDIT)
    return fail(DIT_EUNSUPPORTED, "the MMDiT design has no workspace-free forward");
  if (B <= 0) return fail(DIT_EINVAL, "B must be positive (got %d)", B);
  if (h->ncls > 0 && !y) return fail(DIT_EINVAL, "class labels y are required");
  if (h->cond_dim > 0 && !pooled) return fail(DIT_EINVAL, "pooled conditioning is required");
  int rc = check_rows(h, B);
  if (rc) return rc;
  const size_t need = ws_layout(h, B).total;
  if (need > kNoallocScratchBytes)
    return fail(DIT_EWORKSPACE,
                "B = %d needs %zu bytes of scratch; the static scratch holds %zu (use "
                "dit_forward with a workspace)", B, need, kNoallocScratchBytes);
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  return forward_impl(h, x_t, t, y, pooled, nullptr, B, out, nullptr, ws, kNoallocScratchBytes,
                      stream);
}
