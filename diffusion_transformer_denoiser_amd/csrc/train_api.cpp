// Host side of dit_train_step: parameter layout, workspace layout and the
// launch sequence of one optimizer step (forward with saved activations, loss,
// backward, AdamW).  No device memory is allocated here.
//
// Input gradients reuse the forward GEMM kernels, which compute C = A W^T with
// both operands K-contiguous: dA[M, K] = dC[M, N] W[N, K] takes A = dC and the
// W-operand W^T [K, N], so the weights are transposed once per step.  Weight
// gradients dW[N, K] += dC^T A read dC and A row-major as saved (a transposing
// matrix-core kernel for bf16, transposed addressing for fp32); they reduce
// over all B T tokens, split along that reduction, and the slices add their
// partial sums atomically into the zeroed gradient buffer.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "common.h"
#include "dit.h"
#include "internal.h"
#include "train.h"

using namespace dit_host;

// Propagates a non-zero status of a host helper.
#define DIT_RC(call)         \
  do {                       \
    const int rc_ = (call);  \
    if (rc_) return rc_;     \
  } while (0)

namespace {

constexpr int kNumFields = 42;   // pointers in dit_weights
constexpr int kTrained[] = {0, 1, 2, 3, 4, 5, 6, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20};
enum {
  F_PE_W = 0, F_PE_B = 1, F_T1_W = 2, F_T1_B = 3, F_T2_W = 4, F_T2_B = 5, F_Y = 6, F_ADA_W = 9,
  F_ADA_B = 10, F_QKV_W = 11, F_QKV_B = 12, F_O_W = 13, F_O_B = 14, F_FC1_W = 15, F_FC1_B = 16,
  F_FC2_W = 17, F_FC2_B = 18, F_OUT_W = 19, F_OUT_B = 20
};

bool is_gemm_weight(int f) {
  return f == F_PE_W || f == F_T1_W || f == F_T2_W || f == F_ADA_W || f == F_QKV_W ||
         f == F_O_W || f == F_FC1_W || f == F_FC2_W || f == F_OUT_W;
}

size_t field_count(const dit_handle* h, int f) {
  const size_t d = h->d, N = h->N, hid = h->hid;
  switch (f) {
    case F_PE_W: return d * h->kin;
    case F_PE_B: return d;
    case F_T1_W: return d * h->freq;
    case F_T1_B: return d;
    case F_T2_W: return d * d;
    case F_T2_B: return d;
    case F_Y: return (size_t)(h->ncls + 1) * d;
    case F_ADA_W: return (size_t)h->mod_stride * d;
    case F_ADA_B: return h->mod_stride;
    case F_QKV_W: return N * 3 * d * d;
    case F_QKV_B: return N * 3 * d;
    case F_O_W: return N * d * d;
    case F_O_B: return N * d;
    case F_FC1_W: return N * hid * d;
    case F_FC1_B: return N * hid;
    case F_FC2_W: return N * d * hid;
    case F_FC2_B: return N * d;
    case F_OUT_W: return (size_t)h->kout * d;
    case F_OUT_B: return h->kout;
  }
  return 0;
}

struct ParamLayout {
  size_t off[kNumFields], cnt[kNumFields], total;
};

ParamLayout param_layout(const dit_handle* h) {
  ParamLayout P;
  memset(&P, 0, sizeof P);
  size_t o = 0;
  for (int f : kTrained) {
    P.off[f] = o;
    P.cnt[f] = field_count(h, f);
    o += (P.cnt[f] + 63) / 64 * 64;
  }
  P.total = o;
  return P;
}

// Field f of the handle's weights (dit_weights read as an array of pointers).
void* weight_ptr(const dit_handle* h, int f) {
  const void* p;
  memcpy(&p, (const char*)&h->w + (size_t)f * sizeof(void*), sizeof p);
  return const_cast<void*>(p);
}

int check_train(const dit_handle* h) {
  if (h->cond != DIT_COND_ADALN_ZERO)
    return fail(DIT_EUNSUPPORTED, "training supports the adaLN-Zero design");
  if (h->ncls <= 0 || h->cond_dim > 0)
    return fail(DIT_EUNSUPPORTED, "training supports class-conditional models without pooled "
                                  "conditioning");
  if (h->cfg.rope3d || h->cfg.qk_norm || h->cfg.frames != 1 || h->cfg.patch_t != 1)
    return fail(DIT_EUNSUPPORTED, "training supports single-frame models without RoPE / qk_norm");
  return DIT_OK;
}

struct TrainLayout {
  size_t coef, tf, acc, xt, P, e, t1pre, th, c, sc, mod, dmod, pe;
  size_t Xs, Xmid, H1, qkv, O, lse, o, H2, pre, f, G, Hf, Y;
  size_t dY, dX, dH, dBr, dpre, dO, Dv, dqkv;
  size_t wqkv, wo, wfc1, wfc2, wout, wada, wt2;
  size_t dmod_dt, dsc, dc, dth, dt1;
  size_t total;
};

TrainLayout train_layout(const dit_handle* h, int B) {
  TrainLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t es = h->es, Bz = (size_t)B, T = h->T, M = Bz * T, d = h->d, N = h->N;
  const size_t hid = h->hid, ms = h->mod_stride, kout = h->kout, kin = h->kin;
  const size_t lat = Bz * h->cfg.in_channels * h->cfg.height * h->cfg.width;
  L.coef = take(Bz * kCoefStride * 4);
  L.tf = take(Bz * 4);
  L.acc = take(16);
  L.xt = take(lat * es);
  L.P = take(M * kin * es);
  L.e = take(Bz * h->freq * 4);
  L.t1pre = take(Bz * d * 4);
  L.th = take(Bz * d * 4);
  L.c = take(Bz * d * 4);
  L.sc = take(Bz * d * es);
  L.mod = take(Bz * ms * 4);
  L.dmod = take(Bz * ms * 4);
  L.pe = take(T * d * 4);
  // saved activations
  L.Xs = take((N + 1) * M * d * 4);
  L.Xmid = take(N * M * d * 4);
  L.H1 = take(N * M * d * es);
  L.qkv = take(N * M * 3 * d * es);
  L.O = take(N * M * d * es);
  L.lse = take(N * Bz * h->heads * T * 4);
  L.o = take(N * M * d * 4);
  L.H2 = take(N * M * d * es);
  L.pre = take(N * M * hid * es);
  L.f = take(N * M * d * 4);
  L.G = take(N * M * hid * es);   // GELU(pre) of every block (weight gradients of fc2)
  L.Hf = take(M * d * es);
  L.Y = take(M * kout * 4);
  // backward scratch
  L.dY = take(M * kout * es);
  L.dX = take(M * d * 4);
  L.dH = take(M * d * 4);
  L.dBr = take(M * d * es);
  L.dpre = take(M * hid * es);
  L.dO = take(M * d * es);
  L.Dv = take(Bz * h->heads * T * 4);
  L.dqkv = take(M * 3 * d * es);
  // transposed weights (model dtype)
  L.wqkv = take(N * d * 3 * d * es);
  L.wo = take(N * d * d * es);
  L.wfc1 = take(N * d * hid * es);
  L.wfc2 = take(N * hid * d * es);
  L.wout = take(d * kout * es);
  L.wada = take(d * ms * es);
  L.wt2 = take(d * d * 4);
  // conditioning backward
  L.dmod_dt = take(Bz * ms * es);
  L.dsc = take(Bz * d * 4);
  L.dc = take(Bz * d * 4);
  L.dth = take(Bz * d * 4);
  L.dt1 = take(Bz * d * 4);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// C = A W^T with A [M, K] (row stride lda, dtype adt) and W [N, K] (row stride
// ldw, dtype wdt): the MFMA kernel when both operands are bf16 and the shapes
// fit it, else the VALU kernel.  EPI_ATOMIC_F32 splits the reduction so the
// grid has about 1024 workgroups.
hipError_t gemm_any(int epi, const void* A, int adt, int64_t lda, const void* W, int wdt,
                    int64_t ldw, int M, int N, int K, EpiParams ep, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  ep.ldw = (int)ldw;
  const bool mfma = adt == 1 && wdt == 1 && K % 64 == 0 && lda % 8 == 0 && ldw % 8 == 0 &&
                    aligned16(A) && aligned16(W);
  if (epi == EPI_ATOMIC_F32) ep.ksplit = splitk_slice(mfma, M, N, K);
  if (mfma) return launch_gemm_mfma(epi, (const bf16_t*)A, (int)lda, (const bf16_t*)W, M, N, K, ep, s);
  ALoad a;
  memset(&a, 0, sizeof a);
  a.ptr = A;
  a.lda = (int)lda;
  a.a_dtype = adt;
  a.src_rows = M;
  return launch_gemm_valu(epi, A_PLAIN, a, W, wdt, M, N, K, ep, s);
}

// Gradients of a linear layer from its row-major output gradient dC [R, N]
// (row stride ldc) and input X [R, K] (row stride ldx), both in dtype dt:
// weight gW [N, K] += dC^T X and, if gb, bias gb [N] += column sums of dC
// (both fp32, zeroed beforehand).
int layer_grads(int dt, const void* dC, int64_t ldc, const void* X, int64_t ldx, int N, int K,
                int64_t R, float* gW, float* gb, hipStream_t s) {
  DIT_HIP(linear_wgrad(dC, ldc, X, ldx, N, K, R, dt, gW, K, gb, s));
  return DIT_OK;
}

}  // namespace

extern "C" {

int dit_train_param_count(const dit_handle* h, size_t* count) {
  if (!h || !count) return fail(DIT_EINVAL, "handle and count must be non-NULL");
  int rc = check_train(h);
  if (rc) return rc;
  *count = param_layout(h).total;
  return ok();
}

int dit_train_param_layout(const dit_handle* h, int field, size_t* offset, size_t* count) {
  if (!h || !offset || !count) return fail(DIT_EINVAL, "handle, offset and count must be non-NULL");
  if (field < 0 || field >= kNumFields) return fail(DIT_EINVAL, "field %d out of range", field);
  int rc = check_train(h);
  if (rc) return rc;
  const ParamLayout P = param_layout(h);
  *offset = P.off[field];
  *count = P.cnt[field];
  return ok();
}

int dit_train_workspace_size(const dit_handle* h, int B, size_t* bytes) {
  if (!h || !bytes) return fail(DIT_EINVAL, "handle and bytes must be non-NULL");
  if (B <= 0) return fail(DIT_EINVAL, "B must be positive");
  int rc = check_train(h);
  if (rc) return rc;
  *bytes = train_layout(h, B).total;
  return ok();
}

int dit_train_step(dit_handle* h, const dit_train_hparams* hp, int step,
                   const dit_train_state* st, const float* x0, const int32_t* y, const int32_t* t,
                   const float* noise, int B, float* loss, void* ws, size_t ws_bytes,
                   void* stream) {
  if (!h || !hp || !st) return fail(DIT_EINVAL, "handle, hparams and state must be non-NULL");
  if (!st->master || !st->grad || !st->m || !st->v || !st->ema)
    return fail(DIT_EINVAL, "a training-state buffer is NULL");
  if (!x0 || !y || !t || !noise || !loss) return fail(DIT_EINVAL, "x0, y, t, noise and loss must be non-NULL");
  if (B <= 0) return fail(DIT_EINVAL, "B must be positive");
  if (step < 1) return fail(DIT_EINVAL, "step must be >= 1");
  int rc = check_train(h);
  if (rc) return rc;
  if (hp->train_steps < 2 || !(hp->beta_start > 0.0) || !(hp->beta_end < 1.0) ||
      !(hp->beta_start <= hp->beta_end))
    return fail(DIT_EINVAL, "schedule needs train_steps >= 2 and 0 < beta_start <= beta_end < 1");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) ||
      !(hp->adam_eps > 0.0) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay) ||
      !(hp->ema_decay >= 0.0 && hp->ema_decay <= 1.0))
    return fail(DIT_EINVAL, "invalid AdamW / EMA hyper-parameters");
  const int64_t T = h->T, M = (int64_t)B * T;
  if ((int64_t)B * h->heads > 65535) return fail(DIT_EUNSUPPORTED, "B * heads > 65535");
  if (M * h->hid > (1LL << 31) || (M + 63) / 64 > 65535)
    return fail(DIT_EUNSUPPORTED, "B * T too large for one step");
  if (h->dtype == DIT_BF16 && M % 64)
    return fail(DIT_EUNSUPPORTED, "bf16 training needs B * T to be a multiple of 64 (got %lld)",
                (long long)M);
  const TrainLayout L = train_layout(h, B);
  if (!ws) return fail(DIT_EWORKSPACE, "workspace pointer is NULL");
  if (ws_bytes < L.total)
    return fail(DIT_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  if ((uintptr_t)ws & 255) return fail(DIT_EWORKSPACE, "workspace must be 256-byte aligned");
  for (int f : kTrained)
    if (!weight_ptr(h, f)) return fail(DIT_EINVAL, "weight field %d is NULL", f);

  hipStream_t s = (hipStream_t)stream;
  const ParamLayout P = param_layout(h);
  const int d = h->d, N = h->N, hid = h->hid, ms = h->mod_stride, es = h->es, dt = h->dtype;
  const int heads = h->heads, kout = h->kout, kin = h->kin, C = h->cfg.in_channels;
  float* grad = st->grad;
  auto G_ = [&](int f) { return grad + P.off[f]; };
  auto W_ = [&](int f) { return weight_ptr(h, f); };
  auto wl = [&](int f, size_t l, size_t per) { return (const char*)W_(f) + l * per * es; };
  float* mod = at<float>(ws, L.mod);
  float* dmod = at<float>(ws, L.dmod);
  const float* coef = at<float>(ws, L.coef);

  // ---- schedule, x_t, transposed weights, zeroed gradient --------------------------------
  DIT_HIP(launch_train_schedule(t, B, hp->train_steps, hp->beta_start, hp->beta_end,
                                at<float>(ws, L.coef), at<float>(ws, L.tf), s));
  const int64_t per_row = (int64_t)C * h->cfg.height * h->cfg.width;
  DIT_HIP(launch_train_noise(x0, noise, coef, per_row, per_row * B, dt, at<void>(ws, L.xt), s));
  DIT_HIP(launch_fill_f32(grad, (int64_t)P.total, 0.0f, s));
  DIT_HIP(launch_fill_f32(dmod, (int64_t)B * ms, 0.0f, s));   // LN backward adds into it
  for (int l = 0; l < N; ++l) {
    DIT_HIP(launch_transpose(wl(F_QKV_W, l, (size_t)3 * d * d), dt, 3 * d, d, d,
                             at<char>(ws, L.wqkv) + (size_t)l * d * 3 * d * es, dt, 3 * d, s));
    DIT_HIP(launch_transpose(wl(F_O_W, l, (size_t)d * d), dt, d, d, d,
                             at<char>(ws, L.wo) + (size_t)l * d * d * es, dt, d, s));
    DIT_HIP(launch_transpose(wl(F_FC1_W, l, (size_t)hid * d), dt, hid, d, d,
                             at<char>(ws, L.wfc1) + (size_t)l * d * hid * es, dt, hid, s));
    DIT_HIP(launch_transpose(wl(F_FC2_W, l, (size_t)d * hid), dt, d, hid, hid,
                             at<char>(ws, L.wfc2) + (size_t)l * hid * d * es, dt, d, s));
  }
  DIT_HIP(launch_transpose(W_(F_OUT_W), dt, kout, d, d, at<void>(ws, L.wout), dt, kout, s));
  DIT_HIP(launch_transpose(W_(F_ADA_W), dt, ms, d, d, at<void>(ws, L.wada), dt, ms, s));
  DIT_HIP(launch_transpose(W_(F_T2_W), dt, d, d, d, at<void>(ws, L.wt2), 0, d, s));

  // ---- conditioning: c = t-MLP(e(t)) + y_table[y]; mod = Linear(SiLU(c)) ----------------
  float* e = at<float>(ws, L.e);
  float* t1pre = at<float>(ws, L.t1pre);
  float* th = at<float>(ws, L.th);
  float* c = at<float>(ws, L.c);
  void* sc = at<void>(ws, L.sc);
  DIT_HIP(launch_timestep_embed(at<float>(ws, L.tf), B, B, h->freq, e, s));
  {
    EpiParams ep = epi0();
    ep.bias = (const float*)W_(F_T1_B); ep.out = t1pre; ep.ldo = d;
    DIT_HIP(gemm_any(EPI_BIAS_F32, e, 0, h->freq, W_(F_T1_W), dt, h->freq, B, d, h->freq, ep, s));
    DIT_HIP(launch_silu_f32(t1pre, th, (int64_t)B * d, s));
    ep = epi0();
    ep.bias = (const float*)W_(F_T2_B); ep.out = c; ep.ldo = d; ep.silu_out = sc;
    ep.table = (const float*)W_(F_Y); ep.labels = y; ep.label_rows = B; ep.null_from = B;
    ep.ncls = h->ncls;
    ALoad a;
    memset(&a, 0, sizeof a);
    a.ptr = th; a.lda = d; a.a_dtype = 0; a.src_rows = B;
    DIT_HIP(launch_gemm_valu(EPI_COND, A_PLAIN, a, W_(F_T2_W), dt, B, d, d, ep, s));
    ep = epi0();
    ep.bias = (const float*)W_(F_ADA_B); ep.out = mod; ep.ldo = ms;
    DIT_HIP(linear(h, EPI_BIAS_F32, sc, d, W_(F_ADA_W), B, ms, d, ep, s));
  }

  // ---- forward with saved activations ---------------------------------------------------
  const size_t Md = (size_t)M * d;
  float* Xs = at<float>(ws, L.Xs);
  float* pe = at<float>(ws, L.pe);
  DIT_HIP(launch_pos_embed_table(h->gh, h->gw, d, pe, s));
  if (kin % 16 == 0 && aligned16(W_(F_PE_W))) {
    DIT_HIP(launch_patch_embed(at<void>(ws, L.xt), B, h->gin, dt, W_(F_PE_W),
                               (const float*)W_(F_PE_B), pe, (int)M, d, 0, Xs, s));
  } else {
    ALoad a;
    memset(&a, 0, sizeof a);
    a.ptr = at<void>(ws, L.xt); a.a_dtype = dt; a.src_rows = B; a.g = h->gin;
    EpiParams ep = epi0();
    ep.bias = (const float*)W_(F_PE_B); ep.out = Xs; ep.ldo = d; ep.T = (int)T; ep.pe_tab = pe;
    DIT_HIP(launch_gemm_valu(EPI_PATCH, A_PATCH, a, W_(F_PE_W), dt, (int)M, d, kin, ep, s));
  }
  auto Xl = [&](int l) { return Xs + (size_t)l * Md; };
  auto Xm = [&](int l) { return at<float>(ws, L.Xmid) + (size_t)l * Md; };
  auto H1 = [&](int l) { return at<char>(ws, L.H1) + (size_t)l * Md * es; };
  auto QKV = [&](int l) { return at<char>(ws, L.qkv) + (size_t)l * Md * 3 * es; };
  auto Ob = [&](int l) { return at<char>(ws, L.O) + (size_t)l * Md * es; };
  auto LSE = [&](int l) { return at<float>(ws, L.lse) + (size_t)l * B * heads * T; };
  auto ob = [&](int l) { return at<float>(ws, L.o) + (size_t)l * Md; };
  auto H2 = [&](int l) { return at<char>(ws, L.H2) + (size_t)l * Md * es; };
  auto PRE = [&](int l) { return at<char>(ws, L.pre) + (size_t)l * M * hid * es; };
  auto fb_ = [&](int l) { return at<float>(ws, L.f) + (size_t)l * Md; };
  auto Gl = [&](int l) { return at<char>(ws, L.G) + (size_t)l * M * hid * es; };
  for (int l = 0; l < N; ++l) {
    const int base = 6 * d * l;
    DIT_HIP(launch_ln_modulate(Xl(l), (int)M, (int)T, d, mod, ms, base, base + d, h->eps, H1(l),
                               dt, s));
    EpiParams ep = epi0();
    ep.bias = (const float*)W_(F_QKV_B) + (size_t)l * 3 * d; ep.out = QKV(l); ep.ldo = 3 * d;
    DIT_HIP(linear(h, EPI_BIAS_DT, H1(l), d, wl(F_QKV_W, l, (size_t)3 * d * d), (int)M, 3 * d, d,
                   ep, s));
    DIT_HIP(launch_attention(QKV(l), B, heads, (int)T, h->dh, dt, Ob(l), s, LSE(l)));
    ep = epi0();
    ep.bias = (const float*)W_(F_O_B) + (size_t)l * d; ep.out = ob(l); ep.ldo = d;
    DIT_HIP(linear(h, EPI_BIAS_F32, Ob(l), d, wl(F_O_W, l, (size_t)d * d), (int)M, d, d, ep, s));
    DIT_HIP(launch_gate_residual(Xl(l), ob(l), mod, ms, base + 2 * d, (int)T, d, M, Xm(l), s));
    DIT_HIP(launch_ln_modulate(Xm(l), (int)M, (int)T, d, mod, ms, base + 3 * d, base + 4 * d,
                               h->eps, H2(l), dt, s));
    ep = epi0();
    ep.bias = (const float*)W_(F_FC1_B) + (size_t)l * hid; ep.out = Gl(l); ep.aux = PRE(l);
    ep.ldo = hid;
    DIT_HIP(linear(h, EPI_GELU2, H2(l), d, wl(F_FC1_W, l, (size_t)hid * d), (int)M, hid, d, ep,
                   s));
    ep = epi0();
    ep.bias = (const float*)W_(F_FC2_B) + (size_t)l * d; ep.out = fb_(l); ep.ldo = d;
    DIT_HIP(linear(h, EPI_BIAS_F32, Gl(l), hid, wl(F_FC2_W, l, (size_t)d * hid), (int)M, d, hid,
                   ep, s));
    DIT_HIP(launch_gate_residual(Xm(l), fb_(l), mod, ms, base + 5 * d, (int)T, d, M, Xl(l + 1), s));
  }
  const int fbo = 6 * d * N;
  void* Hf = at<void>(ws, L.Hf);
  float* Y = at<float>(ws, L.Y);
  DIT_HIP(launch_ln_modulate(Xl(N), (int)M, (int)T, d, mod, ms, fbo, fbo + d, h->eps, Hf, dt, s));
  {
    EpiParams ep = epi0();
    ep.bias = (const float*)W_(F_OUT_B); ep.out = Y; ep.ldo = kout;
    DIT_HIP(gemm_any(EPI_BIAS_F32, Hf, dt, d, W_(F_OUT_W), dt, d, (int)M, kout, d, ep, s));
  }

  // ---- loss and dY ---------------------------------------------------------------------
  void* dY = at<void>(ws, L.dY);
  DIT_HIP(launch_train_loss(Y, noise, coef, h->gout, C, M, dt, dY, at<double>(ws, L.acc), loss, s));

  // ---- final layer backward --------------------------------------------------------------
  float* dX = at<float>(ws, L.dX);
  float* dH = at<float>(ws, L.dH);
  {
    DIT_RC(layer_grads(dt, dY, kout, Hf, d, kout, d, M, G_(F_OUT_W), G_(F_OUT_B), s));
    EpiParams ep = epi0();
    ep.out = dH; ep.ldo = d;
    DIT_HIP(gemm_any(EPI_BIAS_F32, dY, dt, kout, at<void>(ws, L.wout), dt, kout, (int)M, d, kout,
                     ep, s));
    DIT_HIP(launch_fill_f32(dX, (int64_t)Md, 0.0f, s));
    DIT_HIP(launch_ln_mod_bwd(Xl(N), dH, mod, ms, fbo, fbo + d, B, (int)T, d, h->eps, dX, dmod, s));
  }

  // ---- blocks, last to first -------------------------------------------------------------
  void* dBr = at<void>(ws, L.dBr);
  void* dpre = at<void>(ws, L.dpre);
  void* dO = at<void>(ws, L.dO);
  void* dqkv = at<void>(ws, L.dqkv);
  for (int l = N - 1; l >= 0; --l) {
    const int base = 6 * d * l;
    // FFN branch: X_{l+1} = X_mid + a2 f, f = GELU(pre) W2^T + b2
    DIT_HIP(launch_gate_bwd(dX, fb_(l), mod, ms, base + 5 * d, B, (int)T, d, dt, dBr, dmod, s));
    DIT_RC(layer_grads(dt, dBr, d, Gl(l), hid, d, hid, M, G_(F_FC2_W) + (size_t)l * d * hid,
                        G_(F_FC2_B) + (size_t)l * d, s));
    EpiParams ep = epi0();
    ep.out = dpre; ep.aux = PRE(l); ep.ldo = hid;   // d pre = (df W2) GELU'(pre)
    DIT_HIP(gemm_any(EPI_DGELU, dBr, dt, d, at<char>(ws, L.wfc2) + (size_t)l * hid * d * es, dt,
                     d, (int)M, hid, d, ep, s));
    DIT_RC(layer_grads(dt, dpre, hid, H2(l), d, hid, d, M, G_(F_FC1_W) + (size_t)l * hid * d,
                        G_(F_FC1_B) + (size_t)l * hid, s));
    ep = epi0();
    ep.out = dH; ep.ldo = d;
    DIT_HIP(gemm_any(EPI_BIAS_F32, dpre, dt, hid, at<char>(ws, L.wfc1) + (size_t)l * d * hid * es,
                     dt, hid, (int)M, d, hid, ep, s));
    DIT_HIP(launch_ln_mod_bwd(Xm(l), dH, mod, ms, base + 3 * d, base + 4 * d, B, (int)T, d, h->eps,
                              dX, dmod, s));
    // attention branch: X_mid = X_l + a1 o, o = O Wo^T + bo
    DIT_HIP(launch_gate_bwd(dX, ob(l), mod, ms, base + 2 * d, B, (int)T, d, dt, dBr, dmod, s));
    DIT_RC(layer_grads(dt, dBr, d, Ob(l), d, d, d, M, G_(F_O_W) + (size_t)l * d * d,
                        G_(F_O_B) + (size_t)l * d, s));
    ep = epi0();
    ep.out = dO; ep.ldo = d;
    DIT_HIP(gemm_any(EPI_BIAS_DT, dBr, dt, d, at<char>(ws, L.wo) + (size_t)l * d * d * es, dt, d,
                     (int)M, d, d, ep, s));
    DIT_HIP(launch_attention_bwd(QKV(l), Ob(l), dO, LSE(l), at<float>(ws, L.Dv), B, heads, (int)T,
                                 h->dh, dt, dqkv, s));
    DIT_RC(layer_grads(dt, dqkv, 3 * d, H1(l), d, 3 * d, d, M,
                        G_(F_QKV_W) + (size_t)l * 3 * d * d, G_(F_QKV_B) + (size_t)l * 3 * d, s));
    ep = epi0();
    ep.out = dH; ep.ldo = d;
    DIT_HIP(gemm_any(EPI_BIAS_F32, dqkv, dt, 3 * d, at<char>(ws, L.wqkv) + (size_t)l * d * 3 * d * es,
                     dt, 3 * d, (int)M, d, 3 * d, ep, s));
    DIT_HIP(launch_ln_mod_bwd(Xl(l), dH, mod, ms, base, base + d, B, (int)T, d, h->eps, dX, dmod,
                              s));
  }

  // ---- patch embedding: X_0 = patches W_pe^T + b_pe (+ fixed PE) ---------------------
  {
    DIT_HIP(launch_cast_f32(dX, dBr, (int64_t)Md, dt, s));
    DIT_HIP(launch_patchify(at<void>(ws, L.xt), B, h->gin, dt, at<void>(ws, L.P), s));
    DIT_RC(layer_grads(dt, dBr, d, at<void>(ws, L.P), kin, d, kin, M, G_(F_PE_W), G_(F_PE_B), s));
  }

  // ---- conditioning backward ---------------------------------------------------------
  {
    // mod = SiLU(c) ada_w^T + ada_b
    DIT_HIP(launch_cast_f32(dmod, at<void>(ws, L.dmod_dt), (int64_t)B * ms, dt, s));
    DIT_RC(layer_grads(dt, at<void>(ws, L.dmod_dt), ms, sc, d, ms, d, B, G_(F_ADA_W), nullptr, s));
    DIT_HIP(launch_colsum(dmod, B, ms, ms, G_(F_ADA_B), s));
    float* dsc = at<float>(ws, L.dsc);
    DIT_HIP(launch_fill_f32(dsc, (int64_t)B * d, 0.0f, s));
    EpiParams ep = epi0();
    ep.out = dsc; ep.ldo = d;
    DIT_HIP(gemm_any(EPI_ATOMIC_F32, at<void>(ws, L.dmod_dt), dt, ms, at<void>(ws, L.wada), dt, ms,
                     B, d, ms, ep, s));
    // c = t2(th) + t2_b + y_table[y]
    float* dc = at<float>(ws, L.dc);
    DIT_HIP(launch_silu_bwd(dsc, c, dc, (int64_t)B * d, s));
    DIT_HIP(launch_class_grad(dc, y, B, d, h->ncls, G_(F_Y), s));
    DIT_RC(layer_grads(0, dc, d, th, d, d, d, B, G_(F_T2_W), G_(F_T2_B), s));
    float* dth = at<float>(ws, L.dth);
    ep = epi0();
    ep.out = dth; ep.ldo = d;
    DIT_HIP(gemm_any(EPI_BIAS_F32, dc, 0, d, at<void>(ws, L.wt2), 0, d, B, d, d, ep, s));
    // th = SiLU(e t1_w^T + t1_b)
    float* dt1 = at<float>(ws, L.dt1);
    DIT_HIP(launch_silu_bwd(dth, t1pre, dt1, (int64_t)B * d, s));
    DIT_RC(layer_grads(0, dt1, d, e, h->freq, d, h->freq, B, G_(F_T1_W), G_(F_T1_B), s));
  }

  // ---- AdamW, EMA, model-dtype weights ---------------------------------------------
  {
    AdamArgs a;
    a.lr = (float)hp->lr;
    a.b1 = (float)hp->beta1;
    a.omb1 = (float)(1.0 - hp->beta1);
    a.b2 = (float)hp->beta2;
    a.omb2 = (float)(1.0 - hp->beta2);
    a.eps = (float)hp->adam_eps;
    a.wd = (float)hp->weight_decay;
    a.ema = (float)hp->ema_decay;
    a.omema = (float)(1.0 - hp->ema_decay);
    a.bc1 = (float)(1.0 / (1.0 - std::pow(hp->beta1, step)));
    a.bc2 = (float)(1.0 / (1.0 - std::pow(hp->beta2, step)));
    for (int f : kTrained) {
      const size_t o = P.off[f];
      DIT_HIP(launch_adamw(st->master + o, grad + o, st->m + o, st->v + o, st->ema + o,
                           (int64_t)P.cnt[f], a, W_(f), is_gemm_weight(f) ? dt : 0, s));
    }
  }
  return ok();
}

}  // extern "C"
