// Optional per-launch kernel timing.  While a handle has timing enabled, the
// C-ABI layer installs a thread-local sink; every launcher brackets its
// hipLaunchKernelGGL with begin/end so one class id always names exactly one
// compiled kernel (the ids are listed in include/gpt2mi.h).
#pragma once

#include <hip/hip_runtime.h>

struct ProfSink {
    virtual void begin(int cls, double work, hipStream_t s) = 0;
    virtual void end(int cls, hipStream_t s) = 0;
    virtual ~ProfSink() {}
};

extern thread_local ProfSink* g_prof_sink;

#define PROF_LAUNCH(cls, work, stream, ...)                                   \
    do {                                                                      \
        ProfSink* ps_ = g_prof_sink;                                          \
        if (ps_) ps_->begin((cls), (work), (stream));                         \
        __VA_ARGS__;                                                          \
        if (ps_) ps_->end((cls), (stream));                                   \
    } while (0)

// Kernel class ids (one compiled kernel each).
enum KernelClass {
    KC_GEMM_NT = 1,        // NT GEMM (gemm_nt_w8_kernel; gemm_kernel below 128 tiles), bf16 epilogue (bias / residual)
    KC_GEMM_NT_GELU = 2,   // NT GEMM, bias + GELU epilogue
    KC_GEMM_TN_ACC = 3,    // TN GEMM (gemm_tn_w8_kernel; gemm_kernel for small shapes), fp32 += epilogue
    KC_GEMM_TN_SPLIT = 4,  // TN GEMM, fp32 split-K partials
    KC_SPLITK_REDUCE = 5,
    KC_ATTN_FWD = 6,
    KC_ATTN_DVEC = 7,      // reserved: D = rowsum(dO * O) is taken inside the dQ kernel
    KC_ATTN_DKDV = 8,
    KC_ATTN_DQ = 9,
    KC_XENT = 10,
    KC_LN_FWD = 11,
    KC_LN_BWD = 12,
    KC_FOLD = 13,          // fold of per-block partial column sums
    KC_GELU_BWD = 14,
    KC_COLSUM = 15,
    KC_EMB_FWD = 16,
    KC_EMB_BWD_WTE = 17,
    KC_EMB_BWD_WPE = 18,
    KC_SUMSQ = 19,
    KC_NORM_FINAL = 20,
    KC_ADAMW = 21,
    KC_TRANSPOSE = 22,
    KC_MEAN = 23,
    KC_BIAS_GELU_FWD = 24,
    KC_GEMM_NT_DGELU = 25, // NT GEMM, output times GELU'(pre) epilogue
    KC_OTHER = 26,
    KC_COUNT = 27
};
