/*
 * gpt2mi_kernels.h -- kernel-level C ABI of libgpt2mi (same library as gpt2mi.h).
 *
 * Each entry point runs one hot-path kernel (or its fixed kernel sequence) on
 * caller-owned device buffers, asynchronously on `stream`.  They exist for
 * kernel-level parity tests and microbenchmarks at the shapes of one card's
 * micro-batch; gpt2_forward / gpt2_backward / gpt2_clip_adamw call the same
 * kernels.  Conventions as in gpt2mi.h: bf16 as uint16_t bit patterns,
 * row-major arrays, 256-byte aligned device pointers, status codes
 * GPT2_OK / GPT2_E_*.  Sources are cited as in gpt2mi.h (PDS, GLM =
 * "Was ein Sprachmodell vorhersagt", activity table).
 * Empty inputs: the row-wise calls (xent, layernorm_*, bias_gelu_*, bias_grad)
 * accept rows == 0 and then launch nothing, write nothing and return GPT2_OK;
 * the GEMM, attention and embedding calls need at least one row (B, T, M >= 1)
 * and return GPT2_E_INVALID otherwise, before any device work.
 */
#ifndef GPT2MI_KERNELS_H
#define GPT2MI_KERNELS_H

#include "gpt2mi.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Fused masked softmax cross-entropy (PDS model text: softmax over the V real
 * tokens; padding columns get no probability and no gradient).  logits: bf16
 * [rows, Vp], overwritten in place when write_grad != 0 by
 * (softmax_j - [j == tgt]) * dloss for j < V and exactly 0 for j >= V.
 * loss_rows: fp32 [rows] = logsumexp_{j<V} z - z_tgt.  A target equal to
 * GPT2_IGNORE_TARGET gives loss 0 and an all-zero gradient row; other ids
 * outside [0, V) set *flag (int32, device, may be NULL) to 1 and are clamped.
 * Requires Vp % 128 == 0, 1 <= V <= Vp, Vp <= 65536.
 */
int gpt2k_xent(uint16_t* logits, const int32_t* tgt, float* loss_rows, int64_t rows, int32_t V, int32_t Vp,
               float dloss, int32_t write_grad, int32_t* flag, hipStream_t stream);

/*
 * LayerNorm forward (PDS model text: normalisation before attention and
 * before the feed-forward part; statistics in fp32): y = w (x - mean) rstd + b,
 * rstd = 1/sqrt(var + 1e-5), biased variance.  x, y: bf16 [rows, C];
 * w, b: fp32 [C]; mean, rstd: fp32 [rows].  C % 128 == 0, C <= 4096.
 */
int gpt2k_layernorm_fwd(const uint16_t* x, const float* w, const float* b, uint16_t* y, float* mean, float* rstd,
                        int64_t rows, int32_t C, hipStream_t stream);

/*
 * LayerNorm backward.  dx = rstd (w dy - mean(w dy) - xhat mean(w dy xhat));
 * dres (bf16 [rows, C]) <- dx if accumulate == 0, else dres + dx (the
 * residual-stream gradient).  dw += sum_rows dy xhat; db += sum_rows dy
 * (fp32 [C], accumulated; the sums have a fixed order, so the same inputs give
 * the same bits).  scratch: at least gpt2k_scratch_bytes(1, rows, C, 0).
 */
int gpt2k_layernorm_bwd(const uint16_t* x, const uint16_t* dy, const float* w, const float* mean,
                        const float* rstd, uint16_t* dres, int32_t accumulate, float* dw, float* db, void* scratch,
                        int64_t scratch_bytes, int64_t rows, int32_t C, hipStream_t stream);

/*
 * Bias + GELU forward (GPT-2's tanh form): pre = u + b (bf16 [rows, N]),
 * g = 0.5 pre (1 + tanh(sqrt(2/pi) (pre + 0.044715 pre^3))) (bf16).
 * pre may alias u.  N % 8 == 0.
 */
int gpt2k_bias_gelu_fwd(const uint16_t* u, const float* b, uint16_t* pre, uint16_t* g, int64_t rows, int32_t N,
                        hipStream_t stream);

/*
 * Bias + GELU backward: dpre = dg * GELU'(pre) (bf16 [rows, N], may alias dg);
 * db += sum_rows dpre (fp32 [N]).  scratch: gpt2k_scratch_bytes(2, rows, N, 0).
 */
int gpt2k_bias_gelu_bwd(const uint16_t* pre, const uint16_t* dg, uint16_t* dpre, float* db, void* scratch,
                        int64_t scratch_bytes, int64_t rows, int32_t N, hipStream_t stream);

/*
 * Linear-layer GEMMs on bf16 MFMA with fp32 accumulation.
 *  gpt2k_gemm_nt: out[M, N] = A[M, K] . B[N, K]^T (+ bias[N]) (+ res[M, N]),
 *    bf16 out/res, fp32 bias; bias/res may be NULL.  K % 64 == 0.
 *  gpt2k_gemm_nt_gelu: with pre = A . B^T + bias rounded to bf16, writes
 *    g = GELU(pre) and gprime = GELU'(pre), both bf16 [M, N] (the backward
 *    needs only the derivative of the pre-activation, so it is stored instead).
 *  gpt2k_gemm_nt_dgelu: out = (A . B^T) * gprime (bf16 gprime, out [M, N]):
 *    the input gradient of the MLP projection taken through the GELU.
 *  gpt2k_gemm_tn_acc: dW[N, K] += sum_m dY[m, n] X[m, k] (fp32 dW, bf16
 *    dY [M, N] and X [M, K]) and, if db != NULL, db[n] += sum_m dY[m, n]
 *    (fp32, the bias gradient); M % 64 == 0.  scratch: gpt2k_scratch_bytes(3,
 *    M, N, K) (split-K partials and their bias column sums, added in split
 *    order: the same inputs give the same bits).
 */
int gpt2k_gemm_nt(const uint16_t* A, const uint16_t* B, const float* bias, const uint16_t* res, uint16_t* out,
                  int64_t M, int64_t N, int64_t K, hipStream_t stream);
int gpt2k_gemm_nt_gelu(const uint16_t* A, const uint16_t* B, const float* bias, uint16_t* gprime, uint16_t* g,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);
int gpt2k_gemm_nt_dgelu(const uint16_t* A, const uint16_t* B, const uint16_t* gprime, uint16_t* out, int64_t M,
                        int64_t N, int64_t K, hipStream_t stream);
int gpt2k_gemm_tn_acc(const uint16_t* dY, const uint16_t* X, float* dW, float* db, void* scratch,
                      int64_t scratch_bytes, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Column sums: db[n] += sum_m dY[m, n] (bf16 dY [M, N], fp32 db).
 * scratch: gpt2k_scratch_bytes(2, M, N, 0).
 */
int gpt2k_bias_grad(const uint16_t* dY, float* db, void* scratch, int64_t scratch_bytes, int64_t M, int32_t N,
                    hipStream_t stream);

/*
 * Causal multi-head attention (GLM activity 5: softmax(Q K^T / sqrt(d)) V with
 * a causal mask; position t sees positions <= t).  qkv: bf16 [B*T, 3C]
 * (row = b*T + t; Q | K | V thirds; head h at columns h*d .. h*d+d-1 of each
 * third), out: bf16 [B*T, C], lse: fp32 [B, H, T] natural-log log-sum-exp of
 * the scaled scores.  d = C/H in {32, 64}; T % 64 == 0.
 */
int gpt2k_attention_fwd(const uint16_t* qkv, uint16_t* out, float* lse, int32_t B, int32_t T, int32_t H,
                        int32_t C, hipStream_t stream);

/*
 * Attention backward: dqkv (bf16 [B*T, 3C]) = gradients of the forward above
 * given dout (bf16 [B*T, C]), the saved out and lse.  dvec: fp32 [B, H, T]
 * workspace (rowsum(dout * out)).
 */
int gpt2k_attention_bwd(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse,
                        uint16_t* dqkv, float* dvec, int32_t B, int32_t T, int32_t H, int32_t C,
                        hipStream_t stream);

/*
 * Global-norm clip + AdamW on flat fp32 arrays (semantics of
 * gpt2_clip_adamw): decay on elements [0, n_decay); shadow (bf16 [n_decay],
 * may be NULL) <- round(p) there; g zeroed.  n % 4 == 0, n_decay % 4 == 0.
 * scratch: gpt2k_scratch_bytes(4, n, 0, 0).  norm_dev (fp32, may be NULL) <- ||g||.
 */
int gpt2k_clip_adamw(float* p, float* g, float* m, float* v, uint16_t* shadow, int64_t n, int64_t n_decay,
                     const gpt2_adamw_args* args, float* norm_dev, void* scratch, int64_t scratch_bytes,
                     hipStream_t stream);

/*
 * gpt2k_clip_adamw without a scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight training loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics and results as
 * gpt2k_clip_adamw; it allocates nothing.  Its scratch (the clip scale and
 * the fp64 partial sums of the squared gradient) is a fixed 16 KiB device
 * array inside the library, one copy per GPU, kept until the process ends;
 * sizes whose scratch would not fit return GPT2_E_SHAPE (at present every n
 * fits: the partial-sum count does not grow with n).  All calls on one GPU
 * share that GPU's copy: calls that overlap on one GPU race.  Errors:
 * GPT2_E_INVALID (as gpt2k_clip_adamw), GPT2_E_SHAPE, GPT2_E_HIP.
 */
int gpt2k_clip_adamw_noalloc(float* p, float* g, float* m, float* v, uint16_t* shadow, int64_t n, int64_t n_decay,
                             const gpt2_adamw_args* args, float* norm_dev, hipStream_t stream);

/*
 * Token + position embedding: x[r] = wte[tok[r]] + wpe[r % T] (bf16 tables,
 * bf16 out [B*T, C]).  Ids outside [0, V) set *flag and are clamped.
 */
int gpt2k_embedding_fwd(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, uint16_t* x, int32_t B,
                        int32_t T, int32_t C, int32_t V, int32_t* flag, hipStream_t stream);

/*
 * Embedding backward: dwte[tok[r]] += dx[r]; dwpe[t] += sum_b dx[b*T + t]
 * (fp32 tables, bf16 dx).  Ids outside [0, V) are skipped.  scratch: device
 * bytes, 16-byte aligned, at least gpt2k_scratch_bytes(5, B*T, V, C) (the rows
 * are counting-sorted by token there); too small -> GPT2_E_SHAPE.  The rows of
 * a token are added in increasing row order, in windows of 32 whose partial
 * sums are then added in window order: the result is the same bits every run.
 */
int gpt2k_embedding_bwd(const int32_t* tok, const uint16_t* dx, float* dwte, float* dwpe, int32_t B, int32_t T,
                        int32_t C, int32_t V, void* scratch, int64_t scratch_bytes, hipStream_t stream);

/*
 * Scratch bytes needed by the kernel-level calls, written to *out:
 * kind 1 = layernorm_bwd (a = rows, b = C); kind 2 = bias_gelu_bwd or
 * bias_grad (a = rows, b = N); kind 3 = gemm_tn_acc (a = M, b = N, c = K);
 * kind 4 = clip_adamw (a = n); kind 5 = embedding_bwd (a = B*T, b = V, c = C).
 * Unused arguments are ignored.
 */
int gpt2k_scratch_bytes(int32_t kind, int64_t a, int64_t b, int64_t c, int64_t* out);

#ifdef __cplusplus
}
#endif
#endif /* GPT2MI_KERNELS_H */
