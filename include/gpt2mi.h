/*
 * gpt2mi.h -- C ABI of the GPT-2 training-step library for MI355X (gfx950).
 *
 * One optimizer step of a GPT-2 style decoder-only model: forward, backward,
 * global-norm clipping and AdamW, with the recipe of
 *   PDS = "Pretraining and adapting a language model on a dependency-free
 *          stack" (arXiv HTML): model text around Fig. 1 (12 blocks, 12 heads,
 *          768 channels, context 1,024, tied input/output embeddings, pre-LN
 *          blocks with residuals; vocabulary padded 50,257 -> 50,304 with the
 *          softmax over the real tokens only; N(0, 0.02) init with residual
 *          projections scaled by 1/sqrt(2L)); §4 optimisation paragraph
 *          (AdamW 0.9/0.95/1e-8, decay 0.1 on 2-D weights, clip 1.0, warmup
 *          700 to 6e-4 then cosine to zero over 18,865 steps, seed 1,337);
 *          §4 precision paragraph (bf16 activations; fp32 master weights,
 *          gradients, optimizer state, normalisation statistics and loss);
 *          §4.4 batch (19 sequences x 1,024 tokens x 9 accumulation steps
 *          per card).
 *
 * Ownership: the caller allocates every device buffer (sizes from
 * gpt2_sizes) and owns the stream.  The library keeps only a small host-side
 * handle; it allocates no device memory and keeps no global state.  Every
 * device pointer must be 256-byte aligned.  A handle is not thread-safe and
 * serves one stream at a time.
 *
 * Asynchrony: gpt2_init, gpt2_forward, gpt2_backward and gpt2_clip_adamw
 * only enqueue work on the given stream and return at once.  gpt2_eval_loss
 * and gpt2_sync_status synchronise the stream.  Bad token / target ids are
 * detected on the device; they set a sticky flag that only gpt2_sync_status
 * and gpt2_eval_loss report (GPT2_E_DATA).  Such ids are clamped into range
 * so every kernel stays in bounds.
 *
 * Reproducibility: every sum in the step has a fixed order (no floating-point
 * atomics whose order depends on scheduling), so the same weights, moments,
 * batch and arguments give the same bits on every run of a given build and
 * device; a run restored from its saved state continues exactly.
 *
 * Data types: bf16 values are passed as uint16_t bit patterns (round to
 * nearest even).  Token and target ids are int32.
 */
#ifndef GPT2MI_H
#define GPT2MI_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (every call returns one). */
#define GPT2_OK 0
#define GPT2_E_INVALID 1       /* null/misaligned pointer, inconsistent config or argument */
#define GPT2_E_SHAPE 2         /* sizes that the workspace or the kernels do not support */
#define GPT2_E_STATE 3         /* call order violated (e.g. backward without a forward with targets) */
#define GPT2_E_HIP 4           /* a HIP runtime call failed; see gpt2_last_hip_error */
#define GPT2_E_DATA 5          /* a token or target id was outside [0, V) (sticky, device-detected) */
#define GPT2_E_UNSUPPORTED 6   /* no GPU of the supported architecture */

/* Model + batch configuration.  Requirements: C % H == 0, head dim C/H in
 * {32, 64}; C % 128 == 0; Vp % 128 == 0 and V <= Vp; 1 <= T <= Tmax;
 * T % 64 == 0; B >= 1. */
typedef struct gpt2_config {
    int32_t L;     /* blocks */
    int32_t H;     /* heads */
    int32_t C;     /* channels */
    int32_t V;     /* real vocabulary (softmax support) */
    int32_t Vp;    /* padded vocabulary (rows of the token table) */
    int32_t Tmax;  /* context length = rows of the position table */
    int32_t B;     /* sequences per micro-step */
    int32_t T;     /* tokens per sequence in a micro-step */
} gpt2_config;

/* Sizes of the caller-owned buffers. */
typedef struct gpt2_sizes_t {
    int64_t n_params;       /* fp32 elements of params, grads, m, v (padded vocabulary) */
    int64_t n_params_real;  /* parameters excluding the padding rows of wte */
    int64_t n_decay;        /* elements of the leading 2-D (weight-decayed) segment = bf16 shadow length */
    int64_t n_shadow_t;     /* bf16 elements of the transposed shadow (wte and the 4 matrices per block) */
    int64_t n_tensors;      /* 12 L + 4 */
    int64_t acts_bytes;     /* activation workspace for B x T */
    int64_t scratch_bytes;  /* scratch workspace (partials, flags) */
} gpt2_sizes_t;

/* One parameter tensor in the flat layout. */
typedef struct gpt2_tensor_info_t {
    char name[48];      /* HF-style name, e.g. "h.10.ln_2.weight" */
    int64_t offset;     /* element offset in params/grads/m/v */
    int64_t rows;       /* rows (1 for 1-D tensors) */
    int64_t cols;       /* columns ([out, in] for matrices; length for 1-D tensors) */
    int32_t decayed;    /* 1 for 2-D tensors (weight decay, bf16 shadow), else 0 */
    int64_t shadow_t_offset; /* element offset of the transposed bf16 copy, -1 if none */
} gpt2_tensor_info_t;

/* Caller-owned device buffers (all 256-byte aligned). */
typedef struct gpt2_buffers {
    float* params;        /* fp32 [n_params] master weights, flat layout below */
    float* grads;         /* fp32 [n_params] accumulated gradients */
    float* m;             /* fp32 [n_params] AdamW first moment */
    float* v;             /* fp32 [n_params] AdamW second moment */
    uint16_t* shadow;     /* bf16 [n_decay]  copy of the 2-D weights used by the GEMMs */
    uint16_t* shadow_t;   /* bf16 [n_shadow_t] transposed copies ([in, out]) for the backward GEMMs */
    void* acts;           /* [acts_bytes] saved activations */
    void* scratch;        /* [scratch_bytes] */
} gpt2_buffers;

/* AdamW + clipping arguments (PDS §4 optimisation paragraph). */
typedef struct gpt2_adamw_args {
    float lr;             /* learning rate of this step (host computes the schedule) */
    float beta1;          /* 0.9 */
    float beta2;          /* 0.95 */
    float eps;            /* 1e-8 */
    float weight_decay;   /* 0.1, applied to the 2-D segment only */
    float max_norm;       /* 1.0: grads scaled by min(1, max_norm / ||g||_2) */
    int32_t t;            /* 1-based optimizer step (bias correction) */
} gpt2_adamw_args;

typedef struct gpt2_handle gpt2_handle;

/*
 * Flat parameter layout (element offsets in params/grads/m/v):
 *   decayed 2-D segment: wte [Vp, C] (rows >= V are padding: zero, no
 *   gradient), wpe [Tmax, C], then per block l: h.l.attn.c_attn.weight
 *   [3C, C], h.l.attn.c_proj.weight [C, C], h.l.mlp.c_fc.weight [4C, C],
 *   h.l.mlp.c_proj.weight [C, 4C];
 *   1-D segment: per block h.l.ln_1.weight, h.l.ln_1.bias [C],
 *   h.l.attn.c_attn.bias [3C], h.l.attn.c_proj.bias [C], h.l.ln_2.weight,
 *   h.l.ln_2.bias [C], h.l.mlp.c_fc.bias [4C], h.l.mlp.c_proj.bias [C]; then
 *   ln_f.weight, ln_f.bias [C].
 * Matrices are row-major [out, in] (y = x W^T + b).  In c_attn the rows are
 * [Q | K | V] and head h owns rows h*d .. h*d+d-1 of each third.
 */

/* Pure host function: validates cfg and fills *out.  No GPU access. */
int gpt2_sizes(const gpt2_config* cfg, gpt2_sizes_t* out);

/* Pure host function: describes tensor `index` (0 .. n_tensors-1) of the flat layout. */
int gpt2_tensor_info(const gpt2_config* cfg, int32_t index, gpt2_tensor_info_t* out);

/*
 * Creates a handle bound to `bufs` and enqueues the init on `stream`:
 * params <- host_init (fp32 [n_params], copied) if non-NULL, otherwise the
 * seeded init (PDS model text around Fig. 1): every 2-D weight ~ N(0, 0.02),
 * attn.c_proj and mlp.c_proj ~ N(0, 0.02 / sqrt(2L)), wte padding rows 0,
 * biases 0, LayerNorm gains 1.  The normal draws come from SplitMix64
 * (Steele, Lea & Flood 2014) used as a counter-based hash -- output x for
 * seed s is mix64(s + (x+1) * 0x9E3779B97F4A7C15) -- with counters
 * x1 = tensor_index * 2^40 + 2 * element, x2 = x1 + 1, uniforms
 * ((out >> 11) + 0.5) * 2^-53, and Box-Muller sqrt(-2 ln u1) cos(2 pi u2)
 * in double, rounded to fp32 after scaling by the standard deviation.
 * Then writes the bf16 shadow and its transposes and zeroes grads, m, v.
 * Errors: GPT2_E_INVALID (bad cfg, null/misaligned buffer), GPT2_E_HIP.
 */
int gpt2_init(const gpt2_config* cfg, uint64_t seed, const float* host_init, const gpt2_buffers* bufs,
              hipStream_t stream, gpt2_handle** out);

/*
 * Target id of a position whose loss is not taken (answer-only loss in the
 * PDS clinical-adaptation paragraph): its row loss and logit gradient are 0,
 * and it is left out of the mean loss.
 */
#define GPT2_IGNORE_TARGET (-100)

/*
 * Forward pass on device-resident ids tok, tgt (int32 [B, T], row-major).
 * Saves the activations needed by gpt2_backward.  With tgt != NULL it runs
 * the masked softmax cross-entropy over the V real columns (PDS model text:
 * padding columns get no probability), leaves the bf16 logit gradient
 * (softmax - onehot) * dloss_scale in the logits buffer for gpt2_backward
 * (exactly 0 on the padding columns), and writes the mean loss over the rows
 * whose target is not GPT2_IGNORE_TARGET (0 if there are none) to loss_dev[0]
 * (fp32, device) if loss_dev != NULL.  Ignored rows get loss 0 and a zero
 * logit gradient.  dloss_scale is the weight of one row's loss in the
 * optimised objective: 1/(kept rows over the n_micro micro-steps) for the
 * mean over an accumulated step (1/(B*T*n_micro) when nothing is ignored).  With tgt == NULL only the bf16
 * logits [B*T, Vp] are produced (read them with gpt2_logits_ptr).
 * Errors: GPT2_E_INVALID (null tok), GPT2_E_HIP.
 */
int gpt2_forward(gpt2_handle* h, const int32_t* tok, const int32_t* tgt, float dloss_scale, float* loss_dev,
                 hipStream_t stream);

/*
 * Backward pass for the last gpt2_forward with targets.  ACCUMULATES the
 * fp32 parameter gradients into bufs->grads (they are zeroed by
 * gpt2_init and by gpt2_clip_adamw), so n_micro forward/backward pairs
 * followed by one gpt2_clip_adamw form one accumulated optimizer step
 * (PDS §4.4).  Errors: GPT2_E_STATE (no forward with targets since the last
 * backward), GPT2_E_HIP.
 */
int gpt2_backward(gpt2_handle* h, hipStream_t stream);

/*
 * Lanes: micro-steps in flight at once.  The n_micro forward/backward pairs
 * of one accumulated optimizer step (PDS §4.4) depend on each other only
 * through the gradient sum, so they can run on several streams when each
 * stream has its own activations and its own gradient accumulator.
 * gpt2_lane_init creates such a lane of model h: a handle that reads h's
 * parameters and bf16 shadows (bufs->params, shadow, shadow_t of h) and
 * writes only `grads` (fp32 [n_params], zeroed here on `stream`), `acts`
 * (acts_bytes) and `scratch` (scratch_bytes), all caller-owned and 256-byte
 * aligned.  gpt2_forward / gpt2_backward / gpt2_eval_loss / gpt2_sync_status
 * and the timing calls take a lane like a model handle; gpt2_clip_adamw does
 * not (GPT2_E_STATE): it is called on h and takes the gradient as h's
 * accumulator plus those of its lanes in creation order, then zeroes them all.
 * Ordering across streams is the caller's: every lane's backward must be
 * complete before gpt2_clip_adamw(h) starts, and no lane's forward may start
 * before that call has finished.  At most GPT2_MAX_LANES lanes per model;
 * a lane cannot have lanes.  Destroy lanes before their model (destroying
 * the model first detaches them: they keep their buffers but no clip counts
 * their gradients).  Errors: GPT2_E_INVALID (null/misaligned pointer, h is a
 * lane, a buffer overlapping another of the lane's or any buffer of h or of its
 * lanes), GPT2_E_STATE (GPT2_MAX_LANES lanes exist), GPT2_E_HIP.
 */
#define GPT2_MAX_LANES 3
int gpt2_lane_init(gpt2_handle* h, float* grads, void* acts, void* scratch, hipStream_t stream,
                   gpt2_handle** lane);

/*
 * Global-norm clip + AdamW over all parameters (PDS §4 optimisation):
 * n = ||grads||_2 (fp32 partial sums, fp64 across blocks); s = min(1,
 * max_norm / n); g = s * grads; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
 * p -= lr * (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd * p), with wd only on
 * the first n_decay elements.  grads is the sum of h's accumulator and
 * those of h's lanes (see gpt2_lane_init), added in that order.  Then
 * refreshes the bf16 shadow (and its transposes) from p and zeroes every
 * accumulator.  Writes n to grad_norm_dev[0] if non-NULL.
 * Errors: GPT2_E_INVALID (t < 1, null args), GPT2_E_STATE (h is a lane),
 * GPT2_E_HIP.
 */
int gpt2_clip_adamw(gpt2_handle* h, const gpt2_adamw_args* args, float* grad_norm_dev, hipStream_t stream);

/*
 * Held-out loss: forward + masked cross-entropy (no gradient written),
 * synchronises the stream and returns the mean loss over the rows whose
 * target is not GPT2_IGNORE_TARGET in *loss_host.  Errors: GPT2_E_INVALID, GPT2_E_DATA (bad ids seen since the
 * last status read), GPT2_E_HIP.
 */
int gpt2_eval_loss(gpt2_handle* h, const int32_t* tok, const int32_t* tgt, float* loss_host, hipStream_t stream);

/* Synchronises the stream and reports (and clears) the sticky device data flag. */
int gpt2_sync_status(gpt2_handle* h, hipStream_t stream);

/* Device pointer to the bf16 logits [B*T, Vp] of the last forward (gradients after a forward with targets). */
const uint16_t* gpt2_logits_ptr(const gpt2_handle* h);

/* Device pointer to the fp32 per-row losses [B*T] of the last forward with targets. */
const float* gpt2_row_loss_ptr(const gpt2_handle* h);

/* Device pointer to the bf16 residual stream entering block l ([B*T, C]); l == L gives the last block's output. */
const uint16_t* gpt2_residual_ptr(const gpt2_handle* h, int32_t l);

/* hipError_t of the last failed HIP call in this handle (0 if none). */
int gpt2_last_hip_error(const gpt2_handle* h);

/* Frees the host-side handle (device buffers stay owned by the caller). */
void gpt2_destroy(gpt2_handle* h);

/* Static description of a status code. */
const char* gpt2_strerror(int status);

/*
 * Kernel timing.  gpt2_prof_enable(h, kclass) starts recording: every launch
 * issued by this handle's gpt2_forward / gpt2_backward / gpt2_clip_adamw /
 * gpt2_eval_loss whose kernel class equals kclass (-1: every class; 0: stop)
 * gets a pair of HIP events that the launch itself records at the kernel's
 * own start and end (the six launches of the token-table gradient share one
 * pair recorded on their stream before and after them), and the previous
 * records are dropped.  A class id names exactly one compiled kernel; its
 * name is gpt2_prof_class_name(kclass) (NULL for an unknown id), ids run
 * from 1 to 26.  gpt2_prof_read synchronises the stream and sums, over the
 * recorded launches of class kclass (-1: all), the event-measured duration
 * (ms), the launch count and the algorithmic work (FLOP for the MFMA kernels
 * gemm_* and attn_fwd/dkdv/dq, bytes moved for the others).  At most 65,536
 * launches are recorded after an enable.  Errors: GPT2_E_INVALID, GPT2_E_HIP.
 */
int gpt2_prof_enable(gpt2_handle* h, int32_t kclass);
int gpt2_prof_read(gpt2_handle* h, hipStream_t stream, int32_t kclass, double* total_ms, int64_t* launches,
                   double* work);
const char* gpt2_prof_class_name(int32_t kclass);
#ifdef __cplusplus
}
#endif
#endif /* GPT2MI_H */
