// Optional per-launch kernel timing.  While a handle has timing enabled, the
// C-ABI layer installs a thread-local sink; every launcher wraps its launch in
// PROF_LAUNCH so one class id always names exactly one compiled kernel (the
// ids are listed in include/gpt2mi.h).
//
// Inside PROF_LAUNCH a kernel goes out through prof_launch: when the sink has
// selected the launch it hands over a start/stop event pair, and the launch
// extension of the HIP runtime records them at that kernel's own start and
// end, so the measured time excludes the host's dispatch and any gap in front
// of the kernel on its stream.  PROF_SPAN times a group of launches with
// events recorded on the stream before the first and after the last.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

struct ProfSink {
    // multi: the span holds several launches (stream-recorded events); else the
    // sink may leave an event pair in pend0/pend1 for the span's prof_launch
    virtual void begin(int cls, double work, hipStream_t s, bool multi) = 0;
    virtual void end(int cls, hipStream_t s) = 0;
    virtual ~ProfSink() {}
    hipEvent_t pend0 = nullptr, pend1 = nullptr;
};

extern thread_local ProfSink* g_prof_sink;

namespace prof_detail {
template <class Tup, size_t... I>
inline void arg_ptrs(Tup& t, void** out, std::index_sequence<I...>) {
    ((out[I] = (void*)&std::get<I>(t)), ...);
}
}  // namespace prof_detail

// Launches kernel(args...) on stream s; arguments are converted to the
// kernel's parameter types as a triple-chevron launch would convert them.  As
// with that launch, a failure is read back with hipGetLastError.
template <typename... Formal, typename... Actual>
inline void prof_launch(void (*kernel)(Formal...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                              Actual&&... args) {
    static_assert(sizeof...(Formal) == sizeof...(Actual), "kernel argument count");
    std::tuple<Formal...> vals{static_cast<Formal>(std::forward<Actual>(args))...};
    void* argv[sizeof...(Formal) + 1];
    prof_detail::arg_ptrs(vals, argv, std::index_sequence_for<Formal...>{});
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (ProfSink* ps = g_prof_sink) {
        e0 = ps->pend0;
        e1 = ps->pend1;
        ps->pend0 = ps->pend1 = nullptr;
    }
    if (e0)
        (void)hipExtLaunchKernel((const void*)kernel, grid, block, argv, shmem, s, e0, e1, 0);
    else
        (void)hipLaunchKernel((const void*)kernel, grid, block, argv, shmem, s);
}

#define PROF_TIMED_(multi, cls, work, stream, ...)                            \
    do {                                                                      \
        ProfSink* ps_ = g_prof_sink;                                          \
        if (ps_) ps_->begin((cls), (work), (stream), (multi));                \
        __VA_ARGS__;                                                          \
        if (ps_) ps_->end((cls), (stream));                                   \
    } while (0)

#define PROF_LAUNCH(cls, work, stream, ...) PROF_TIMED_(false, cls, work, stream, __VA_ARGS__)
#define PROF_SPAN(cls, work, stream, ...) PROF_TIMED_(true, cls, work, stream, __VA_ARGS__)

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
