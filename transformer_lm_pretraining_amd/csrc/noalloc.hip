// Allocation-free variant of the kernel-level global-norm clip + AdamW.
//
// For callers that cannot allocate device memory: code under HIP graph
// capture, tight training loops, harnesses that forbid hipMalloc.  The scratch
// of the clip + AdamW sequence -- the clip scale and the fp64 per-block partial
// sums of the squared gradient -- lives in the file-scope device array
// `scratch` below instead of a caller buffer.  Each GPU that runs this entry
// point holds its own copy of the array until the process ends.  Host code
// never uses the array's name as an address: once per device, with that device
// current, it asks hipGetSymbolAddress for that device's copy and passes the
// returned pointer to the kernels.
//
// Every call on a GPU shares that GPU's array, which keeps the last call's
// contents: calls that overlap on one GPU (two streams, two host threads)
// race.  Nothing in it has to start at zero: each call writes every partial
// sum and the scale before it reads them.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "../../include/gpt2mi.h"
#include "../../include/gpt2mi_kernels.h"
#include "kernels.h"

namespace {

constexpr int64_t SCRATCH_BYTES = 16384;   // the whole array: 16 KiB per GPU
constexpr int64_t PARTIALS_AT = 256;       // byte 0: the clip scale (fp32); from byte 256: fp64 partials
constexpr int MAX_DEVICES = 64;

}  // namespace

static __device__ __align__(256) char scratch[SCRATCH_BYTES];

namespace {

std::mutex g_lock;
void* g_scratch[MAX_DEVICES];  // device address of each GPU's copy, once looked up

// The address of the current device's copy of `scratch`, looked up on the first
// call on that device (with it current) and kept for the rest of the process.
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GPT2_E_HIP;
    if (dev < 0 || dev >= MAX_DEVICES) return GPT2_E_UNSUPPORTED;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GPT2_E_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GPT2_OK;
}

}  // namespace

extern "C" int gpt2k_clip_adamw_noalloc(float* p, float* g, float* m, float* v, uint16_t* shadow, int64_t n,
                                        int64_t n_decay, const gpt2_adamw_args* a, float* norm_dev, hipStream_t s) {
    if (!p || !g || !m || !v || !a || n < 4 || n % 4 || n_decay < 0 || n_decay > n || n_decay % 4 || a->t < 1 ||
        !(a->max_norm > 0.0f))
        return GPT2_E_INVALID;
    // The sequence needs adamw_partial_elems(n) fp64 partials behind the scale.
    if (PARTIALS_AT + adamw_partial_elems(n) * 8 > SCRATCH_BYTES) return GPT2_E_SHAPE;
    void* sc = nullptr;
    const int st = scratch_of_current_device(&sc);
    if (st != GPT2_OK) return st;
    const AdamwHostArgs ha{a->lr, a->beta1, a->beta2, a->eps, a->weight_decay, a->max_norm,
                           (float)(1.0 / (1.0 - std::pow((double)a->beta1, (double)a->t))),
                           (float)(1.0 / (1.0 - std::pow((double)a->beta2, (double)a->t)))};
    const hipError_t e = launch_clip_adamw(p, g, m, v, shadow, n, n_decay, ha, norm_dev,
                                           (double*)((char*)sc + PARTIALS_AT), (float*)sc, s);
    if (e == hipErrorInvalidValue) return GPT2_E_SHAPE;
    return e == hipSuccess ? GPT2_OK : GPT2_E_HIP;
}
