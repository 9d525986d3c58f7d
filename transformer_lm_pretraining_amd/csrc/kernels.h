// Internal launchers of the gfx950 kernels (host side).  Every launcher
// checks nothing beyond what its kernel needs to stay in bounds; argument
// validation against the public contract happens in the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gpt2mi.h"  // GPT2_IGNORE_TARGET

// ---- GEMM (k_gemm.hip) -----------------------------------------------------
// out[M,N] = A[M,K] . B[N,K]^T (+bias[N]) (+res[M,N]); K % 64 == 0.
hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                          const float* bias, const uint16_t* res, int64_t ldr, uint16_t* out, int64_t ldo,
                          hipStream_t s);
// pre = bf16(A . B^T + bias); gprime = GELU'(pre), g = GELU(pre).
hipError_t launch_gemm_nt_gelu(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                               const float* bias, uint16_t* gprime, uint16_t* g, int64_t ldo, hipStream_t s);
// out = (A . B^T) * gprime, all bf16 [M, N] with leading dim ldo.
hipError_t launch_gemm_nt_dgelu(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                                const uint16_t* gprime, uint16_t* out, int64_t ldo, hipStream_t s);
// dW[N,K] += sum_m dY[m,n] X[m,k]; dbias[n] += sum_m dY[m,n] if dbias != null.
// M % 64 == 0, N % 8 == 0, K % 8 == 0.
hipError_t launch_gemm_tn_acc(const uint16_t* dY, int64_t ldy, const uint16_t* X, int64_t ldx, int M, int N, int K,
                              float* dW, float* dbias, float* partial, int64_t partial_elems, hipStream_t s);
// One weight-gradient product dW[N][K] (+)= dY^T X over M tokens (dY [M][N] row
// stride ldy, X [M][K] row stride ldx), db[N] (+)= column sums of dY (may be null).
struct TnJobDesc {
    const uint16_t* dY;
    int64_t ldy;
    const uint16_t* X;
    int64_t ldx;
    int N, K;
    float* dW;
    float* db;
};
// Up to 48 products over the same M tokens in one launch (+ one reduce when split;
// a mostly idle last pass is avoided by running the smallest products as a second,
// token-split launch).
constexpr int TN_GROUP_MAX = 48;
hipError_t launch_gemm_tn_group(const TnJobDesc* jobs, int n, int M, float* partial, int64_t partial_elems,
                                hipStream_t s);
int64_t gemm_tn_group_partial_elems(const TnJobDesc* jobs, int n, int M);
int64_t gemm_tn_partial_elems(int M, int N, int K);

// ---- LayerNorm / elementwise / loss (k_norm.hip, k_misc.hip) ----------------
bool layernorm_supports(int C);
hipError_t launch_layernorm_fwd(const uint16_t* x, const float* w, const float* b, uint16_t* y, float* mean,
                                float* rstd, int64_t rows, int C, hipStream_t s);
int64_t layernorm_bwd_partial_elems(int64_t rows, int C);
// With dw == nullptr the LayerNorm backward leaves its column partials in
// `partial` (layernorm_bwd_partial_elems floats); launch_layernorm_fold then
// adds slots 0..nslots-1 (slot_elems apart) into dw[i], db[i] (two launches, a
// fixed order of additions; the slots are overwritten).
constexpr int LN_FOLD_MAX = 64;
hipError_t launch_layernorm_fold(float* partial, int64_t slot_elems, int nslots, float* const* dw,
                                 float* const* db, int64_t rows, int C, hipStream_t s);
// dres = (accumulate ? dres_in : 0) + dx; dres_in may equal dres (in place)
hipError_t launch_layernorm_bwd(const uint16_t* x, const uint16_t* dy, const float* w, const float* mean,
                                const float* rstd, const uint16_t* dres_in, uint16_t* dres, int accumulate,
                                float* dw, float* db, float* partial, int64_t rows, int C, hipStream_t s);
int64_t colsum_partial_elems(int64_t rows, int N);
hipError_t launch_bias_gelu_fwd(const uint16_t* u, const float* b, uint16_t* pre, uint16_t* g, int64_t rows, int N,
                                hipStream_t s);
hipError_t launch_bias_gelu_bwd(const uint16_t* pre, const uint16_t* dg, uint16_t* dpre, float* db, float* partial,
                                int64_t rows, int N, hipStream_t s);
hipError_t launch_bias_grad(const uint16_t* dY, int64_t ldy, float* db, float* partial, int64_t rows, int N,
                            hipStream_t s);
hipError_t launch_xent(uint16_t* logits, const int32_t* tgt, float* loss_rows, int64_t rows, int V, int Vp,
                       float dloss, int write_grad, int32_t* flag, hipStream_t s);
// out[0] = mean of x over the rows whose target is not GPT2_IGNORE_TARGET (tgt may be null: all rows).
hipError_t launch_mean(const float* x, const int32_t* tgt, int64_t n, float* out, hipStream_t s);
hipError_t launch_embedding_fwd(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, uint16_t* x, int B,
                                int T, int C, int V, int32_t* flag, hipStream_t s);
// work: embedding_bwd_work_elems(B*T, V, C) int32 scratch, 16-byte aligned (radix sort of the
// rows by token, bucket ends, and the pieces of runs that cross summation windows)
int64_t embedding_bwd_work_elems(int64_t rows, int V, int C);
hipError_t launch_embedding_bwd(const int32_t* tok, const uint16_t* dx, float* dwte, float* dwpe, int B, int T,
                                int C, int V, int32_t* work, int64_t work_elems, hipStream_t s);

// ---- attention (k_attention.hip) ---------------------------------------------
hipError_t launch_attention_fwd(const uint16_t* qkv, uint16_t* out, float* lse, int B, int T, int H, int C,
                                hipStream_t s);
hipError_t launch_attention_bwd(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse,
                                uint16_t* dqkv, float* dvec, int B, int T, int H, int C, hipStream_t s);

// ---- optimizer / init (k_optim.hip) -------------------------------------------
int64_t adamw_partial_elems(int64_t n);  // doubles
struct AdamwHostArgs {
    float lr, beta1, beta2, eps, wd, max_norm;
    float inv_bc1, inv_bc2;  // 1/(1-beta1^t), 1/(1-beta2^t)
};
hipError_t launch_clip_adamw(float* p, float* g, float* m, float* v, uint16_t* shadow, int64_t n, int64_t n_decay,
                             const AdamwHostArgs& a, float* norm_dev, double* partial, float* scale_dev,
                             hipStream_t s);
// The same with the gradient taken as g[0] + ... + g[ng-1] (1 <= ng <= 4, added in that
// order); every g[j] is zeroed.
hipError_t launch_clip_adamw(float* p, float* const* g, int ng, float* m, float* v, uint16_t* shadow, int64_t n,
                             int64_t n_decay, const AdamwHostArgs& a, float* norm_dev, double* partial,
                             float* scale_dev, hipStream_t s);
hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
// dst[c][r] = src[r][c] for a bf16 [R, Cc] matrix.
hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int R, int Cc, hipStream_t s);
// n transposes dst[j] = src[j]^T (R[j] x Cc[j] row-major in, Cc[j] x R[j] out) in as few launches as possible
hipError_t launch_transpose_bf16_batch(const uint16_t* const* src, uint16_t* const* dst, const int* R,
                                       const int* Cc, int n, hipStream_t s);
hipError_t launch_fill_f32(float* dst, float val, int64_t n, hipStream_t s);
// dst[e] = float32(std * N(0,1) draw (seed, tensor, e)) for e in [0, n); rows >= zero_from_row (of
// width cols) are set to 0.
hipError_t launch_init_normal(float* dst, int64_t n, uint64_t seed, int tensor, double stdv, int64_t zero_from,
                              hipStream_t s);
