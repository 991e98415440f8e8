// Launchers of the training-step kernels (train.hip).  Each returns
// hipGetLastError() after its launches.
#pragma once
#include "common.h"

// Per-row constants written by launch_train_schedule: coef[b * kCoefStride + k].
constexpr int kCoefStride = 8;
constexpr int kSa = 0;            // sqrt(abar_t)
constexpr int kSb = 1;            // sqrt(1 - abar_t)
constexpr int kLogBeta = 2;       // log beta_t
constexpr int kLogBetaTilde = 3;  // log beta_tilde_t (t = 0: that of t = 1)
constexpr int kMeanGap = 4;       // c_x0 sqrt(1 - abar_t) / sqrt(abar_t)
constexpr int kPositive = 5;      // 1 for t > 0

// Factors of the AdamW / EMA update, each rounded to fp32 from its fp64 value
// (1 - beta and 1 - decay are formed in fp64: 1 - (float)0.999 is off by 1e-5).
struct AdamArgs {
  float lr, b1, omb1, b2, omb2, eps, wd, bc1, bc2, ema, omema;
};

hipError_t launch_train_schedule(const int32_t* t, int B, int steps, double b0, double b1,
                                 float* coef, float* tf, hipStream_t s);
// xt = sqrt(abar) x0 + sqrt(1 - abar) eps, per_row elements per row, in dtype.
hipError_t launch_train_noise(const float* x0, const float* eps, const float* coef,
                              int64_t per_row, int64_t n, int dtype, void* xt, hipStream_t s);
// Xout = Xin + mod[m / T, goff + n] * v (fp32, [M, d]).
hipError_t launch_gate_residual(const float* Xin, const float* v, const float* mod, int ms,
                                int goff, int T, int d, int64_t M, float* Xout, hipStream_t s);
hipError_t launch_silu_f32(const float* z, float* out, int64_t n, hipStream_t s);
hipError_t launch_silu_bwd(const float* dout, const float* z, float* dz, int64_t n, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
// out = in converted to dtype (0 fp32, 1 bf16).
hipError_t launch_cast_f32(const float* in, void* out, int64_t n, int dtype, hipStream_t s);
// Loss sums (loss[0] = L_simple, loss[1] = KL term; device floats) and dY
// [M, kout] in dtype from the decoder output Y [M, kout].  gout: output patch
// geometry (C = output channels, K = kout); C: latent channels; acc: 2 doubles
// of scratch.
hipError_t launch_train_loss(const float* Y, const float* eps, const float* coef,
                             const PatchGeom& gout, int C, int64_t M, int dtype, void* dY,
                             double* acc, float* loss, hipStream_t s);
// d beta / d gamma are added into dmod (zero it first).
hipError_t launch_ln_mod_bwd(const float* X, const float* dH, const float* mod, int ms, int shoff,
                             int scoff, int B, int T, int d, float eps, float* dX, float* dmod,
                             hipStream_t s);
hipError_t launch_gate_bwd(const float* dX, const float* v, const float* mod, int ms, int goff,
                           int B, int T, int d, int dtype, void* dv, float* dmod, hipStream_t s);
// out[c, r] = in[r, c]; dtypes 0 fp32, 1 bf16.
hipError_t launch_transpose(const void* in, int in_dtype, int64_t R, int64_t Cc, int64_t ldi,
                            void* out, int out_dtype, int64_t ldo, hipStream_t s);
// out[c] += column sums of in [rows, cols] (row stride ld), fp32, atomically.
hipError_t launch_colsum(const float* in, int rows, int64_t cols, int64_t ld, float* out,
                         hipStream_t s);
// out[c] += column sums of a tall bf16 matrix (cols, ld multiples of 8),
// atomically; at most kColsumTallMaxRows rows (the grid's second dimension).
constexpr int64_t kColsumTallMaxRows = 65535LL * 512;
hipError_t launch_colsum_tall_bf16(const void* in, int64_t rows, int64_t cols, int64_t ld,
                                  float* out, hipStream_t s);
hipError_t launch_class_grad(const float* dc, const int32_t* y, int B, int d, int ncls, float* gy,
                             hipStream_t s);
// dqkv [B T, 3 H dh] from qkv, O, dO (dtype) and the forward's log-sum-exp
// lse [B H T]; Dv: B H T floats of scratch.
hipError_t launch_attention_bwd(const void* qkv, const void* O, const void* dO, const float* lse,
                                float* Dv, int B, int heads, int T, int dh, int dtype, void* dqkv,
                                hipStream_t s);
// The same on the matrix cores for bf16 (attention_bwd.hip), given Dv.
hipError_t launch_attention_bwd_mfma(const void* qkv, const void* dO, const float* lse,
                                     const float* Dv, int B, int heads, int T, int dh,
                                     void* dqkv, hipStream_t s);
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, float* ema, int64_t n,
                        const AdamArgs& a, void* w, int w_dtype, hipStream_t s);
