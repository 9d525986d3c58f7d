// Memory-bound kernels of the step: bias + GELU forward/backward, bias
// gradients (column sums), the fused masked softmax cross-entropy, the
// embedding lookup and its scatter-add backward.  All move 16-byte vectors
// (8 bf16) per lane and keep fp32 arithmetic (PDS §4 precision paragraph).
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace {

// ---------------------------------------------------------------- bias + GELU

__global__ __launch_bounds__(256) void bias_gelu_fwd_kernel(const u32x4* __restrict__ u, const float* __restrict__ b,
                                                            u32x4* __restrict__ pre, u32x4* __restrict__ g,
                                                            int64_t nvec, int nvec_row) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * blockDim.x) {
        const int c0 = (int)(i % nvec_row) * 8;
        u32x4 w = u[i];
        float x[8], y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bflo(w[e]) + b[c0 + 2 * e];
            x[2 * e + 1] = bfhi(w[e]) + b[c0 + 2 * e + 1];
        }
        u32x4 po, go;
        // GELU of the stored (bf16) pre-activation, the value the backward differentiates at
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = gelu_f(bf2f(f2bf(x[e])));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            po[e] = pack_bf2(x[2 * e], x[2 * e + 1]);
            go[e] = pack_bf2(y[2 * e], y[2 * e + 1]);
        }
        pre[i] = po;
        g[i] = go;
    }
}

// Column-sum layout: block b handles rows [b*rpb, (b+1)*rpb); thread t owns the
// 8-wide column vectors t, t+256, ... and keeps their sums in registers.
constexpr int CS_THREADS = 256;
constexpr int CS_MAXV = 4;  // N <= 8 * 256 * 4 = 8192

int colsum_blocks(int64_t rows) { return (int)std::min<int64_t>(256, cdiv(rows, 16)); }

template <bool GELU_BWD>
__global__ __launch_bounds__(CS_THREADS) void colsum_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                            const uint16_t* __restrict__ pre,
                                                            uint16_t* __restrict__ dst, float* __restrict__ partial,
                                                            int64_t rows, int N) {
    const int nv = N / 8;
    const int64_t rpb = cdiv(rows, gridDim.x);
    const int64_t r0 = blockIdx.x * rpb;
    const int64_t r1 = std::min<int64_t>(rows, r0 + rpb);
    float acc[CS_MAXV][8];
#pragma unroll
    for (int q = 0; q < CS_MAXV; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
    for (int64_t r = r0; r < r1; ++r) {
#pragma unroll
        for (int q = 0; q < CS_MAXV; ++q) {
            const int cv = threadIdx.x + CS_THREADS * q;
            if (cv >= nv) break;
            u32x4 w = *(const u32x4*)(src + r * lds + cv * 8);
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bflo(w[e]);
                x[2 * e + 1] = bfhi(w[e]);
            }
            if constexpr (GELU_BWD) {
                u32x4 pw = *(const u32x4*)(pre + r * (int64_t)N + cv * 8);
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] *= gelu_grad_f(bflo(pw[e]));
                    x[2 * e + 1] *= gelu_grad_f(bfhi(pw[e]));
                    o[e] = pack_bf2(x[2 * e], x[2 * e + 1]);
                }
                *(u32x4*)(dst + r * (int64_t)N + cv * 8) = o;
                // the bias gradient is the sum of the stored (bf16) dpre
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = bflo(o[e]);
                    x[2 * e + 1] = bfhi(o[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] += x[e];
        }
    }
#pragma unroll
    for (int q = 0; q < CS_MAXV; ++q) {
        const int cv = threadIdx.x + CS_THREADS * q;
        if (cv >= nv) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) partial[(int64_t)blockIdx.x * N + cv * 8 + e] = acc[q][e];
    }
}

__global__ void fold_colsum_kernel(const float* __restrict__ partial, int nblocks, int N, float* __restrict__ out) {
    int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= N) return;
    float s = 0.f;
    for (int b = 0; b < nblocks; ++b) s += partial[(int64_t)b * N + c];
    out[c] += s;
}

// ---------------------------------------------------------------- cross-entropy

constexpr int XE_THREADS = 512;

template <int NV>
__global__ __launch_bounds__(XE_THREADS) void xent_kernel(uint16_t* __restrict__ logits,
                                                          const int32_t* __restrict__ tgt,
                                                          float* __restrict__ loss_rows, int V, int Vp, float dloss,
                                                          int write_grad, int32_t* __restrict__ flag) {
    __shared__ float red[XE_THREADS / 64];
    const int64_t row = blockIdx.x;
    u32x4* z = (u32x4*)(logits + row * (int64_t)Vp);
    const int nvec = Vp / 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    u32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int vid = tid + XE_THREADS * i;
        v[i] = vid < nvec ? z[vid] : u32x4{0, 0, 0, 0};
    }
    // pass 1: row max over the real columns
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int j0 = (tid + XE_THREADS * i) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = (e & 1) ? bfhi(v[i][e >> 1]) : bflo(v[i][e >> 1]);
            if (j0 + e < V) mx = fmaxf(mx, x);
        }
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < XE_THREADS / 64; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();
    // pass 2: sum of exp over the real columns
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int j0 = (tid + XE_THREADS * i) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = (e & 1) ? bfhi(v[i][e >> 1]) : bflo(v[i][e >> 1]);
            if (j0 + e < V) sum += __expf(x - mx);
        }
    }
    sum = wave_sum(sum);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = 0.f;
#pragma unroll
    for (int w = 0; w < XE_THREADS / 64; ++w) sum += red[w];
    int t = tgt[row];
    if (t < 0 || t >= V) {
        if (tid == 0 && flag) atomicOr(flag, 1);
        t = t < 0 ? 0 : V - 1;
    }
    if (tid == 0) loss_rows[row] = mx + logf(sum) - bf2f(logits[row * (int64_t)Vp + t]);
    if (!write_grad) return;
    __syncthreads();  // the target logit is read before any thread overwrites the row
    const float inv = 1.0f / sum;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int vid = tid + XE_THREADS * i;
        if (vid >= nvec) break;
        int j0 = vid * 8;
        u32x4 o;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            float d[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                int j = j0 + 2 * e2 + h;
                float x = h ? bfhi(v[i][e2]) : bflo(v[i][e2]);
                float p = __expf(x - mx) * inv;
                d[h] = j < V ? (p - (j == t ? 1.0f : 0.0f)) * dloss : 0.0f;
            }
            o[e2] = pack_bf2(d[0], d[1]);
        }
        z[vid] = o;
    }
}

__global__ __launch_bounds__(1024) void mean_kernel(const float* __restrict__ x, int64_t n, float* __restrict__ out) {
    __shared__ double red[16];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += x[i];
    s = wave_sum_d(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
        out[0] = (float)(t / (double)n);
    }
}

// ---------------------------------------------------------------- embedding

__global__ __launch_bounds__(256) void embedding_fwd_kernel(const int32_t* __restrict__ tok,
                                                            const uint16_t* __restrict__ wte,
                                                            const uint16_t* __restrict__ wpe,
                                                            uint16_t* __restrict__ x, int64_t rows, int T, int C,
                                                            int V, int32_t* __restrict__ flag) {
    const int nv = C / 8;
    const int64_t total = rows * nv;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nv;
        const int cv = (int)(i % nv);
        int id = tok[r];
        if (id < 0 || id >= V) {
            if (flag) atomicOr(flag, 1);
            id = id < 0 ? 0 : V - 1;
        }
        const int t = (int)(r % T);
        u32x4 a = *(const u32x4*)(wte + (int64_t)id * C + cv * 8);
        u32x4 p = *(const u32x4*)(wpe + (int64_t)t * C + cv * 8);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf2(bflo(a[e]) + bflo(p[e]), bfhi(a[e]) + bfhi(p[e]));
        *(u32x4*)(x + r * C + cv * 8) = o;
    }
}

__global__ __launch_bounds__(256) void embedding_bwd_wte_kernel(const int32_t* __restrict__ tok,
                                                                const uint16_t* __restrict__ dx,
                                                                float* __restrict__ dwte, int64_t rows, int C,
                                                                int V) {
    const int nv = C / 8;
    const int64_t total = rows * nv;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nv;
        const int cv = (int)(i % nv);
        const int id = tok[r];
        if (id < 0 || id >= V) continue;
        u32x4 g = *(const u32x4*)(dx + r * C + cv * 8);
        float* d = dwte + (int64_t)id * C + cv * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            unsafeAtomicAdd(d + 2 * e, bflo(g[e]));
            unsafeAtomicAdd(d + 2 * e + 1, bfhi(g[e]));
        }
    }
}

__global__ __launch_bounds__(256) void embedding_bwd_wpe_kernel(const uint16_t* __restrict__ dx,
                                                                float* __restrict__ dwpe, int B, int T, int C) {
    const int64_t total = (int64_t)T * C;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int b = 0; b < B; ++b) s += bf2f(dx[(int64_t)b * total + i]);
        dwpe[i] += s;
    }
}

int grid_for(int64_t n, int per_block = 256, int cap = 8192) {
    return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per_block), cap));
}

}  // namespace

hipError_t launch_bias_gelu_fwd(const uint16_t* u, const float* b, uint16_t* pre, uint16_t* g, int64_t rows, int N,
                                hipStream_t s) {
    int64_t nvec = rows * (N / 8);
    if (nvec <= 0) return hipSuccess;
    PROF_LAUNCH(KC_BIAS_GELU_FWD, 48.0 * nvec, s, hipLaunchKernelGGL(bias_gelu_fwd_kernel, dim3(grid_for(nvec)), dim3(256), 0, s, (const u32x4*)u, b, (u32x4*)pre,
                       (u32x4*)g, nvec, N / 8));
    return hipGetLastError();
}

int64_t colsum_partial_elems(int64_t rows, int N) { return (int64_t)colsum_blocks(rows) * N; }

hipError_t launch_bias_gelu_bwd(const uint16_t* pre, const uint16_t* dg, uint16_t* dpre, float* db, float* partial,
                                int64_t rows, int N, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (N % 8 || N > 8 * CS_THREADS * CS_MAXV) return hipErrorInvalidValue;
    int blocks = colsum_blocks(rows);
    PROF_LAUNCH(KC_GELU_BWD, 6.0 * rows * N, s, hipLaunchKernelGGL(colsum_kernel<true>, dim3(blocks), dim3(CS_THREADS), 0, s, dg, (int64_t)N, pre, dpre, partial,
                       rows, N));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PROF_LAUNCH(KC_FOLD, 4.0 * blocks * N, s, hipLaunchKernelGGL(fold_colsum_kernel, dim3(cdiv(N, 256)), dim3(256), 0, s, partial, blocks, N, db));
    return hipGetLastError();
}

hipError_t launch_bias_grad(const uint16_t* dY, int64_t ldy, float* db, float* partial, int64_t rows, int N,
                            hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (N % 8 || N > 8 * CS_THREADS * CS_MAXV) return hipErrorInvalidValue;
    int blocks = colsum_blocks(rows);
    PROF_LAUNCH(KC_COLSUM, 2.0 * rows * N, s, hipLaunchKernelGGL(colsum_kernel<false>, dim3(blocks), dim3(CS_THREADS), 0, s, dY, ldy, (const uint16_t*)nullptr,
                       (uint16_t*)nullptr, partial, rows, N));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fold_colsum_kernel, dim3(cdiv(N, 256)), dim3(256), 0, s, partial, blocks, N, db);
    return hipGetLastError();
}

hipError_t launch_xent(uint16_t* logits, const int32_t* tgt, float* loss_rows, int64_t rows, int V, int Vp,
                       float dloss, int write_grad, int32_t* flag, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int nv = (int)cdiv(Vp / 8, XE_THREADS);
    dim3 grid((unsigned)rows), block(XE_THREADS);
    switch (nv) {
#define XE(n) \
    case n: PROF_LAUNCH(KC_XENT, 2.0 * rows * Vp * (write_grad ? 2 : 1), s, hipLaunchKernelGGL(xent_kernel<n>, grid, block, 0, s, logits, tgt, loss_rows, V, Vp, dloss, write_grad, flag)); break;
        XE(1) XE(2) XE(3) XE(4) XE(5) XE(6) XE(7) XE(8) XE(9) XE(10) XE(11) XE(12) XE(13) XE(14) XE(15) XE(16)
#undef XE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mean(const float* x, int64_t n, float* out, hipStream_t s) {
    PROF_LAUNCH(KC_MEAN, 4.0 * n, s, hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, x, n, out));
    return hipGetLastError();
}

hipError_t launch_embedding_fwd(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, uint16_t* x, int B,
                                int T, int C, int V, int32_t* flag, hipStream_t s) {
    int64_t rows = (int64_t)B * T;
    PROF_LAUNCH(KC_EMB_FWD, 6.0 * rows * C, s, hipLaunchKernelGGL(embedding_fwd_kernel, dim3(grid_for(rows * (C / 8))), dim3(256), 0, s, tok, wte, wpe, x, rows,
                       T, C, V, flag));
    return hipGetLastError();
}

hipError_t launch_embedding_bwd(const int32_t* tok, const uint16_t* dx, float* dwte, float* dwpe, int B, int T,
                                int C, int V, hipStream_t s) {
    int64_t rows = (int64_t)B * T;
    PROF_LAUNCH(KC_EMB_BWD_WTE, 10.0 * rows * C, s, hipLaunchKernelGGL(embedding_bwd_wte_kernel, dim3(grid_for(rows * (C / 8))), dim3(256), 0, s, tok, dx, dwte, rows,
                       C, V));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PROF_LAUNCH(KC_EMB_BWD_WPE, 2.0 * rows * C + 8.0 * T * C, s, hipLaunchKernelGGL(embedding_bwd_wpe_kernel, dim3(grid_for((int64_t)T * C)), dim3(256), 0, s, dx, dwpe, B, T, C));
    return hipGetLastError();
}
