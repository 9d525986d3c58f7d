// Global-norm clipping + AdamW (PDS §4 optimisation paragraph: AdamW with
// betas (0.9, 0.95), eps 1e-8, weight decay 0.1 on two-dimensional weights
// only, clipping to global norm 1.0; §4 precision: fp32 master weights,
// gradients and optimizer state), plus the seeded init and bf16 shadow
// maintenance.  All HBM-bound: float4 vectors, grid-stride loops.
#include <algorithm>
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace {

constexpr int NORM_BLOCKS = 1024;
constexpr int OPT_THREADS = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt(const float4* p) {
    const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(float4* p, float4 v) {
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, (f32x4*)p);
}

// The gradient is the sum of NG accumulators (the model's and its lanes'),
// added in accumulator order; element i of it as a vector.
template <int NG>
struct GradSum {
    float4* g[NG];
    __device__ __forceinline__ float4 at(int64_t i) const {
        float4 v = ld_nt(g[0] + i);
#pragma unroll
        for (int j = 1; j < NG; ++j) {
            const float4 w = ld_nt(g[j] + i);
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
        }
        return v;
    }
    __device__ __forceinline__ void zero(int64_t i) const {
#pragma unroll
        for (int j = 0; j < NG; ++j) st_nt(g[j] + i, make_float4(0.f, 0.f, 0.f, 0.f));
    }
};

// Per-block sum of squares of g (fp32 per thread, fp64 across the block).
template <int NG>
__global__ __launch_bounds__(OPT_THREADS) void sumsq_kernel(GradSum<NG> G, int64_t n4, double* __restrict__ partial) {
    __shared__ double red[OPT_THREADS / 64];
    // four vectors per thread in flight, each in its own accumulator (a fixed order:
    // the same inputs give the same bits)
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    const int64_t step = (int64_t)gridDim.x * OPT_THREADS;
    int64_t i = blockIdx.x * (int64_t)OPT_THREADS + threadIdx.x;
    for (; i + 3 * step < n4; i += 4 * step) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = G.at(i + u * step);
#pragma unroll
        for (int u = 0; u < 4; ++u) s4[u] += v[u].x * v[u].x + v[u].y * v[u].y + v[u].z * v[u].z + v[u].w * v[u].w;
    }
    for (; i < n4; i += step) {
        const float4 v = G.at(i);
        s4[0] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    double d = wave_sum_d((double)s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = d;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < OPT_THREADS / 64; ++w) t += red[w];
        partial[blockIdx.x] = t;
    }
}

// norm = sqrt(sum of partials) (fp64); scale = min(1, max_norm / norm).
__global__ __launch_bounds__(OPT_THREADS) void norm_finalize_kernel(const double* __restrict__ partial, int nparts,
                                                                    float max_norm, float* __restrict__ scale_out,
                                                                    float* __restrict__ norm_out) {
    __shared__ double red[OPT_THREADS / 64];
    double s = 0.0;
    for (int i = threadIdx.x; i < nparts; i += OPT_THREADS) s += partial[i];
    s = wave_sum_d(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < OPT_THREADS / 64; ++w) t += red[w];
        double norm = sqrt(t);
        double sc = (norm > (double)max_norm) ? (double)max_norm / norm : 1.0;
        scale_out[0] = (float)sc;
        if (norm_out) norm_out[0] = (float)norm;
    }
}

struct AdamwDev {
    float lr, beta1, beta2, eps, wd, inv_bc1, inv_bc2;
};

__device__ __forceinline__ float adam_one(float& p, float g, float& m, float& v, float wd, const AdamwDev& a) {
    m = a.beta1 * m + (1.0f - a.beta1) * g;
    v = a.beta2 * v + (1.0f - a.beta2) * g * g;
    const float mhat = m * a.inv_bc1;
    const float vhat = v * a.inv_bc2;
    p = p - a.lr * (mhat / (sqrtf(vhat) + a.eps) + wd * p);
    return p;
}


template <int NG>
__global__ __launch_bounds__(OPT_THREADS) void adamw_kernel(float4* __restrict__ p, GradSum<NG> G,
                                                            float4* __restrict__ m, float4* __restrict__ v,
                                                            uint2* __restrict__ shadow, int64_t n4,
                                                            int64_t n_decay4, AdamwDev a,
                                                            const float* __restrict__ scale_ptr) {
    const float sc = scale_ptr[0];
    // streaming: each element is touched once per step, so the loads and stores
    // carry the non-temporal hint.  Two vectors per thread per pass, all loads
    // issued before the arithmetic, keep more bytes in flight per thread.
    auto update = [&](int64_t i, float4 pp, float4 gg, float4 mm, float4 vv) {
        const bool dec = i < n_decay4;
        const float wd = dec ? a.wd : 0.0f;
        adam_one(pp.x, gg.x * sc, mm.x, vv.x, wd, a);
        adam_one(pp.y, gg.y * sc, mm.y, vv.y, wd, a);
        adam_one(pp.z, gg.z * sc, mm.z, vv.z, wd, a);
        adam_one(pp.w, gg.w * sc, mm.w, vv.w, wd, a);
        st_nt(p + i, pp);
        st_nt(m + i, mm);
        st_nt(v + i, vv);
        G.zero(i);
        if (dec && shadow) shadow[i] = make_uint2(pack_bf2(pp.x, pp.y), pack_bf2(pp.z, pp.w));
    };
    const int64_t step = (int64_t)gridDim.x * OPT_THREADS;
    int64_t i = blockIdx.x * (int64_t)OPT_THREADS + threadIdx.x;
    for (; i + step < n4; i += 2 * step) {
        const int64_t k = i + step;
        const float4 p0 = ld_nt(p + i), g0 = G.at(i), m0 = ld_nt(m + i), v0 = ld_nt(v + i);
        const float4 p1 = ld_nt(p + k), g1 = G.at(k), m1 = ld_nt(m + k), v1 = ld_nt(v + k);
        update(i, p0, g0, m0, v0);
        update(k, p1, g1, m1, v1);
    }
    if (i < n4) update(i, ld_nt(p + i), G.at(i), ld_nt(m + i), ld_nt(v + i));
}

__global__ __launch_bounds__(OPT_THREADS) void cast_bf16_kernel(const float4* __restrict__ src,
                                                                uint2* __restrict__ dst, int64_t n4) {
    for (int64_t i = blockIdx.x * (int64_t)OPT_THREADS + threadIdx.x; i < n4; i += (int64_t)gridDim.x * OPT_THREADS) {
        float4 x = src[i];
        dst[i] = make_uint2(pack_bf2(x.x, x.y), pack_bf2(x.z, x.w));
    }
}

// 64x64 tiles through LDS: dst[c][r] = src[r][c].
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst, int R, int Cc) {
    __shared__ uint16_t tile[64][65];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    for (int k = threadIdx.x; k < 64 * 64; k += 256) {
        int rr = k / 64, cc = k % 64;
        int r = r0 + rr, c = c0 + cc;
        tile[rr][cc] = (r < R && c < Cc) ? src[(int64_t)r * Cc + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int k = threadIdx.x; k < 64 * 64; k += 256) {
        int cc = k / 64, rr = k % 64;
        int r = r0 + rr, c = c0 + cc;
        if (r < R && c < Cc) dst[(int64_t)c * R + r] = tile[rr][cc];
    }
}

// Several transposes in one launch, 64x64 tiles through LDS in 16-byte vectors:
// dst_j[c][r] = src_j[r][c] for every job j (R_j and C_j multiples of 8).  Thread t
// reads 8 consecutive columns of rows t/8 and t/8 + 32 and, after the barrier,
// writes 8 consecutive rows of columns t/8 and t/8 + 32 of the transposed tile.
constexpr int TR_MAX_JOBS = 64;
struct TransposeJobs {
    const uint16_t* src[TR_MAX_JOBS];
    uint16_t* dst[TR_MAX_JOBS];
    int R[TR_MAX_JOBS], C[TR_MAX_JOBS];
    int tile_start[TR_MAX_JOBS + 1];  // prefix sums of the jobs' 64x64 tile counts
    int n;
};

__global__ __launch_bounds__(256) void transpose_batch_kernel(TransposeJobs J) {
    __shared__ uint16_t tile[64][64 + 2];
    const int b = blockIdx.x;
    int j = 0;
    while (j + 1 < J.n && b >= J.tile_start[j + 1]) ++j;
    const int R = J.R[j], C = J.C[j], tc = (C + 63) / 64;
    const int t = b - J.tile_start[j], r0 = (t / tc) * 64, c0 = (t % tc) * 64;
    const int tid = threadIdx.x, v = tid & 7, q = tid >> 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rr = q + 32 * h, r = r0 + rr, c = c0 + 8 * v;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (r < R && c < C) w = *(const u32x4*)(J.src[j] + (int64_t)r * C + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[rr][8 * v + 2 * e] = (uint16_t)(w[e] & 0xffffu);
            tile[rr][8 * v + 2 * e + 1] = (uint16_t)(w[e] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int cc = q + 32 * h, c = c0 + cc, r = r0 + 8 * v;
        if (c >= C || r >= R) continue;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)tile[8 * v + 2 * e][cc] | ((uint32_t)tile[8 * v + 2 * e + 1][cc] << 16);
        *(u32x4*)(J.dst[j] + (int64_t)c * R + r) = w;
    }
}

__global__ void fill_f32_kernel(float* __restrict__ dst, float val, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = val;
}

// SplitMix64 (Steele, Lea & Flood 2014) as a counter-based hash.
__device__ __forceinline__ uint64_t splitmix_at(uint64_t seed, uint64_t counter) {
    uint64_t z = seed + (counter + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Box-Muller normal for element e of tensor `tensor`, scaled and rounded to fp32.
__global__ void init_normal_kernel(float* __restrict__ dst, int64_t n, uint64_t seed, uint64_t tensor_base,
                                   double stdv, int64_t zero_from) {
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        if (e >= zero_from) {
            dst[e] = 0.0f;
            continue;
        }
        const uint64_t x1 = tensor_base + 2ull * (uint64_t)e;
        const double u1 = ((double)(splitmix_at(seed, x1) >> 11) + 0.5) * 0x1.0p-53;
        const double u2 = ((double)(splitmix_at(seed, x1 + 1ull) >> 11) + 0.5) * 0x1.0p-53;
        const double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        dst[e] = (float)(stdv * z);
    }
}

int grid_for(int64_t n, int cap = 4096) { return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, 256), cap)); }

}  // namespace

int64_t adamw_partial_elems(int64_t) { return NORM_BLOCKS; }

namespace {
template <int NG>
hipError_t clip_adamw_ng(float* p, float* const* g, float* m, float* v, uint16_t* shadow, int64_t n, int64_t n_decay,
                         const AdamwHostArgs& a, float* norm_dev, double* partial, float* scale_dev, hipStream_t s) {
    const int64_t n4 = n / 4;
    GradSum<NG> G;
    for (int j = 0; j < NG; ++j) G.g[j] = (float4*)g[j];
    PROF_LAUNCH(KC_SUMSQ, 4.0 * NG * n, s, prof_launch(sumsq_kernel<NG>, dim3(NORM_BLOCKS), dim3(OPT_THREADS), 0, s, G, n4, partial));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PROF_LAUNCH(KC_NORM_FINAL, 8.0 * NORM_BLOCKS, s, prof_launch(norm_finalize_kernel, dim3(1), dim3(OPT_THREADS), 0, s, partial, NORM_BLOCKS, a.max_norm,
                       scale_dev, norm_dev));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    AdamwDev d{a.lr, a.beta1, a.beta2, a.eps, a.wd, a.inv_bc1, a.inv_bc2};
    PROF_LAUNCH(KC_ADAMW, (24.0 + 8.0 * NG) * n + 2.0 * n_decay, s, prof_launch(adamw_kernel<NG>, dim3(grid_for(n4, 8192)), dim3(OPT_THREADS), 0, s, (float4*)p, G,
                       (float4*)m, (float4*)v, (uint2*)shadow, n4, n_decay / 4, d, (const float*)scale_dev));
    return hipGetLastError();
}
}  // namespace

hipError_t launch_clip_adamw(float* p, float* const* g, int ng, float* m, float* v, uint16_t* shadow, int64_t n,
                             int64_t n_decay, const AdamwHostArgs& a, float* norm_dev, double* partial,
                             float* scale_dev, hipStream_t s) {
    switch (ng) {
        case 1: return clip_adamw_ng<1>(p, g, m, v, shadow, n, n_decay, a, norm_dev, partial, scale_dev, s);
        case 2: return clip_adamw_ng<2>(p, g, m, v, shadow, n, n_decay, a, norm_dev, partial, scale_dev, s);
        case 3: return clip_adamw_ng<3>(p, g, m, v, shadow, n, n_decay, a, norm_dev, partial, scale_dev, s);
        case 4: return clip_adamw_ng<4>(p, g, m, v, shadow, n, n_decay, a, norm_dev, partial, scale_dev, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_clip_adamw(float* p, float* g, float* m, float* v, uint16_t* shadow, int64_t n, int64_t n_decay,
                             const AdamwHostArgs& a, float* norm_dev, double* partial, float* scale_dev,
                             hipStream_t s) {
    float* gs[1] = {g};
    return launch_clip_adamw(p, gs, 1, m, v, shadow, n, n_decay, a, norm_dev, partial, scale_dev, s);
}

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
    PROF_LAUNCH(KC_OTHER, 6.0 * n, s, prof_launch(cast_bf16_kernel, dim3(grid_for(n / 4)), dim3(OPT_THREADS), 0, s, (const float4*)src,
                       (uint2*)dst, n / 4));
    return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int R, int Cc, hipStream_t s) {
    dim3 grid((unsigned)cdiv(Cc, 64), (unsigned)cdiv(R, 64));
    PROF_LAUNCH(KC_TRANSPOSE, 4.0 * R * Cc, s, prof_launch(transpose_bf16_kernel, grid, dim3(256), 0, s, src, dst, R, Cc));
    return hipGetLastError();
}

hipError_t launch_transpose_bf16_batch(const uint16_t* const* src, uint16_t* const* dst, const int* R,
                                       const int* Cc, int n, hipStream_t s) {
    for (int j0 = 0; j0 < n; j0 += TR_MAX_JOBS) {
        const int m = std::min(TR_MAX_JOBS, n - j0);
        bool vec = true;
        for (int j = j0; j < j0 + m; ++j) vec = vec && R[j] % 8 == 0 && Cc[j] % 8 == 0;
        if (!vec) {  // odd shapes: one scalar transpose each
            for (int j = j0; j < j0 + m; ++j) {
                hipError_t e = launch_transpose_bf16(src[j], dst[j], R[j], Cc[j], s);
                if (e != hipSuccess) return e;
            }
            continue;
        }
        TransposeJobs J{};
        J.n = m;
        int64_t tiles = 0;
        double bytes = 0;
        for (int i = 0; i < m; ++i) {
            J.src[i] = src[j0 + i];
            J.dst[i] = dst[j0 + i];
            J.R[i] = R[j0 + i];
            J.C[i] = Cc[j0 + i];
            J.tile_start[i] = (int)tiles;
            tiles += cdiv(R[j0 + i], 64) * cdiv(Cc[j0 + i], 64);
            bytes += 4.0 * R[j0 + i] * Cc[j0 + i];
        }
        J.tile_start[m] = (int)tiles;
        if (tiles == 0) continue;
        if (tiles > INT32_MAX) return hipErrorInvalidValue;
        PROF_LAUNCH(KC_TRANSPOSE, bytes, s,
                    prof_launch(transpose_batch_kernel, dim3((unsigned)tiles), dim3(256), 0, s, J));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_fill_f32(float* dst, float val, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    PROF_LAUNCH(KC_OTHER, 4.0 * n, s, prof_launch(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, dst, val, n));
    return hipGetLastError();
}

hipError_t launch_init_normal(float* dst, int64_t n, uint64_t seed, int tensor, double stdv, int64_t zero_from,
                              hipStream_t s) {
    if (n <= 0) return hipSuccess;
    PROF_LAUNCH(KC_OTHER, 4.0 * n, s, prof_launch(init_normal_kernel, dim3(grid_for(n)), dim3(256), 0, s, dst, n, seed,
                       (uint64_t)tensor << 40, stdv, zero_from));
    return hipGetLastError();
}
