// Host-side internals shared by the C-ABI sources: the handle and the
// helpers every entry point uses (status strings, the dtype-dispatching
// linear layer).  Not part of the public interface.
#pragma once
#include <hip/hip_runtime.h>

#include "common.h"
#include "dit.h"

struct dit_handle {
  dit_config cfg;
  dit_weights w;
  int d, N, heads, dh, hid, ncls, cond_dim, freq, dtype, es;
  float eps;
  int gf, gh, gw, T, kin, kout, mod_stride;
  // conditioning design; tokens per trunk row (T + 2 in-context, else T);
  // LayerNorms per block of the in-context / cross-attention designs
  int cond, Tt, nln;
  int Lc;            // MMDiT: text tokens per row (0 otherwise)
  int Tf;            // tokens per row of the stream the final layer decodes
  PatchGeom gin, gout;
  PatchGeom gouty;   // gout with T = Tf: the decoder output's row stride
};

namespace dit_host {
// Records the message for dit_last_error_message and returns code.
int fail(int code, const char* fmt, ...);
// Clears the message; returns DIT_OK.
int ok();
size_t align256(size_t b);
// Zero-initialised epilogue parameters.
EpiParams epi0();
// Split-K slice length for an EPI_ATOMIC_F32 product of M x N outputs over K
// (0: no split): about 1024 workgroups, slices a multiple of the kernel's k
// step (64 on the matrix cores, 16 on the VALU path).
int splitk_slice(bool mfma, int64_t M, int64_t N, int64_t K);
// Weight gradient dW [N, K] += dY^T X (fp32, atomically) from the row-major
// output gradient dY [R, N] (row stride ldy) and input X [R, K] (row stride
// ldx), both in dtype: the TN matrix-core kernel for bf16 when the shapes fit
// it, else the VALU kernel reading both operands transposed.  db (optional):
// db[n] += sum_r dY[r, n], the bias gradient (inside the TN kernel, else a
// column-sum kernel; bf16 then needs N, ldy multiples of 8 and dY 16-byte
// aligned).
hipError_t linear_wgrad(const void* dY, int64_t ldy, const void* X, int64_t ldx, int N, int K,
                        int64_t R, int dtype, float* dW, int lddw, float* db, hipStream_t s);
// One linear layer C = A W^T with the epilogue: MFMA for bf16 models, VALU
// for fp32 ones.
hipError_t linear(const dit_handle* h, int epi, const void* A, int lda, const void* W, int M,
                  int N, int K, const EpiParams& ep, hipStream_t s);
}  // namespace dit_host

#define DIT_HIP(call)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess)                                                                \
      return dit_host::fail(DIT_EHIP, "%s: %s", #call, hipGetErrorString(e_));           \
  } while (0)
