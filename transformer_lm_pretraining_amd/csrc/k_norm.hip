// LayerNorm forward / backward (PDS model text around Fig. 1: normalisation
// before attention and before the feed-forward part; §4 precision paragraph:
// statistics in fp32).  One wavefront per row: each lane keeps C/64 values in
// registers, so a row is read once; statistics are wavefront reductions.
// The backward also adds the row's input gradient to the residual-stream
// gradient (read from one buffer, written to another or the same one) and produces per-block fp32 partial column sums of dy*xhat and dy,
// which a second small kernel folds into dw, db.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace {

constexpr float LN_EPS = 1e-5f;
constexpr int ROWS_PER_BLOCK = 4;  // one wave per row, 4 waves per block

// Lane element mapping: element (j*64 + lane)*VEC + v, j < NV, v < VEC.
template <int VEC>
struct Vec;
template <>
struct Vec<2> {
    typedef uint32_t T;
    __device__ static void unpack(T w, float* f) { f[0] = bflo(w); f[1] = bfhi(w); }
    __device__ static T pack(const float* f) { return pack_bf2(f[0], f[1]); }
};
template <>
struct Vec<4> {
    typedef u32x2 T;
    __device__ static void unpack(T w, float* f) { f[0] = bflo(w.x); f[1] = bfhi(w.x); f[2] = bflo(w.y); f[3] = bfhi(w.y); }
    __device__ static T pack(const float* f) { return T{pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3])}; }
};

// Each wave walks rows with a grid stride, with w and b in registers and the
// next row's load in flight while the current row is normalised.
template <int VEC, int NV>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ b, uint16_t* __restrict__ y,
                                                     float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                     int64_t rows) {
    constexpr int C = NV * 64 * VEC;
    typedef typename Vec<VEC>::T VT;
    const int lane = threadIdx.x & 63;
    float wv[NV][VEC], bv[NV][VEC];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            wv[j][e] = w[(j * 64 + lane) * VEC + e];
            bv[j][e] = b[(j * 64 + lane) * VEC + e];
        }
    auto load = [&](int64_t row, VT* xv) {
        const VT* xr = (const VT*)(x + row * C);
#pragma unroll
        for (int j = 0; j < NV; ++j) xv[j] = xr[j * 64 + lane];
    };
    auto compute = [&](int64_t row, const VT* xv) {
        float v[NV][VEC];
#pragma unroll
        for (int j = 0; j < NV; ++j) Vec<VEC>::unpack(xv[j], v[j]);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) s += v[j][e];
        const float mean = wave_sum(s) * (1.0f / C);
        float q = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float d = v[j][e] - mean;
                q += d * d;
            }
        const float var = wave_sum(q) * (1.0f / C);
        const float rstd = 1.0f / sqrtf(var + LN_EPS);
        VT* yr = (VT*)(y + row * C);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = (v[j][e] - mean) * rstd * wv[j][e] + bv[j][e];
            yr[j * 64 + lane] = Vec<VEC>::pack(o);
        }
        if (lane == 0) {
            mean_out[row] = mean;
            rstd_out[row] = rstd;
        }
    };
    const int64_t stride = (int64_t)gridDim.x * ROWS_PER_BLOCK;
    int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
    VT xa[NV], xb[NV];
    if (row < rows) load(row, xa);
    while (row < rows) {
        const int64_t r1 = row + stride;
        if (r1 < rows) load(r1, xb);
        compute(row, xa);
        if (r1 >= rows) break;
        const int64_t r2 = r1 + stride;
        if (r2 < rows) load(r2, xa);
        compute(r1, xb);
        row = r2;
    }
}

// Rows of C = 256 NV elements: each half-wave takes one row with 16-byte loads
// (lane l of the half covers elements (j*32 + l)*8 .. +7), so a wave normalises
// two rows at a time; sums are taken over the 32 lanes of the half.  Rows walk
// with a grid stride and the next pair's loads are in flight during the current.
template <int NV>
__global__ __launch_bounds__(256) void ln_fwd16_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                       const float* __restrict__ b, uint16_t* __restrict__ y,
                                                       float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                       int64_t rows) {
    constexpr int C = NV * 256;
    const int lane = threadIdx.x & 63, hl = lane & 31;
    float wv[NV][8], bv[NV][8];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const float4* wp = (const float4*)(w + (j * 32 + hl) * 8);
        const float4* bp = (const float4*)(b + (j * 32 + hl) * 8);
        const float4 w0 = wp[0], w1 = wp[1], b0 = bp[0], b1 = bp[1];
        wv[j][0] = w0.x; wv[j][1] = w0.y; wv[j][2] = w0.z; wv[j][3] = w0.w;
        wv[j][4] = w1.x; wv[j][5] = w1.y; wv[j][6] = w1.z; wv[j][7] = w1.w;
        bv[j][0] = b0.x; bv[j][1] = b0.y; bv[j][2] = b0.z; bv[j][3] = b0.w;
        bv[j][4] = b1.x; bv[j][5] = b1.y; bv[j][6] = b1.z; bv[j][7] = b1.w;
    }
    auto half_sum = [](float v) {
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
        return v;
    };
    auto load = [&](int64_t row, u32x4* xv) {
        const u32x4* xr = (const u32x4*)(x + row * C);
#pragma unroll
        for (int j = 0; j < NV; ++j) xv[j] = xr[j * 32 + hl];
    };
    auto compute = [&](int64_t row, const u32x4* xv) {
        float v[NV][8];
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[j][2 * e] = bflo(xv[j][e]);
                v[j][2 * e + 1] = bfhi(xv[j][e]);
            }
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) s += v[j][e];
        const float mean = half_sum(s) * (1.0f / C);
        float q = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = v[j][e] - mean;
                q += d * d;
            }
        const float var = half_sum(q) * (1.0f / C);
        const float rstd = 1.0f / sqrtf(var + LN_EPS);
        u32x4* yr = (u32x4*)(y + row * C);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf2((v[j][2 * e] - mean) * rstd * wv[j][2 * e] + bv[j][2 * e],
                                (v[j][2 * e + 1] - mean) * rstd * wv[j][2 * e + 1] + bv[j][2 * e + 1]);
            yr[j * 32 + hl] = o;
        }
        if (hl == 0) {
            mean_out[row] = mean;
            rstd_out[row] = rstd;
        }
    };
    const int64_t stride = (int64_t)gridDim.x * (2 * ROWS_PER_BLOCK);
    int64_t row = (int64_t)blockIdx.x * (2 * ROWS_PER_BLOCK) + (threadIdx.x >> 5);
    u32x4 xa[NV], xb[NV];
    if (row < rows) load(row, xa);
    while (row < rows) {
        const int64_t r1 = row + stride;
        if (r1 < rows) load(r1, xb);
        compute(row, xa);
        if (r1 >= rows) break;
        const int64_t r2 = r1 + stride;
        if (r2 < rows) load(r2, xa);
        compute(r1, xb);
        row = r2;
    }
}

// Each wave walks rows with a grid stride and keeps the next row's loads (x,
// dy and, when accumulating, the residual gradient) in flight while it
// computes the current one.
template <int VEC, int NV>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dy,
                                                     const float* __restrict__ w, const float* __restrict__ mean,
                                                     const float* __restrict__ rstd, const uint16_t* dres_in,
                                                     uint16_t* dres, int accumulate, float* __restrict__ partial,
                                                     int64_t rows) {
    constexpr int C = NV * 64 * VEC;
    typedef typename Vec<VEC>::T VT;
    __shared__ float red[ROWS_PER_BLOCK][2][C];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float wv[NV][VEC], dw_acc[NV][VEC], db_acc[NV][VEC];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            wv[j][e] = w[(j * 64 + lane) * VEC + e];
            dw_acc[j][e] = 0.f;
            db_acc[j][e] = 0.f;
        }
    struct RowIn {
        VT xv[NV], gv[NV], rv[NV];
        float mu, rs;
    };
    auto load = [&](int64_t row, RowIn& in) {
        const VT* xr = (const VT*)(x + row * C);
        const VT* dyr = (const VT*)(dy + row * C);
        const VT* dr = (const VT*)(dres_in + row * C);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            in.xv[j] = xr[j * 64 + lane];
            in.gv[j] = dyr[j * 64 + lane];
            if (accumulate) in.rv[j] = dr[j * 64 + lane];
        }
        in.mu = mean[row];
        in.rs = rstd[row];
    };
    auto compute = [&](int64_t row, const RowIn& in) {
        float xh[NV][VEC], g[NV][VEC], wdy[NV][VEC];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            Vec<VEC>::unpack(in.xv[j], xh[j]);
            Vec<VEC>::unpack(in.gv[j], g[j]);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                xh[j][e] = (xh[j][e] - in.mu) * in.rs;
                wdy[j][e] = wv[j][e] * g[j][e];
                s1 += wdy[j][e];
                s2 += wdy[j][e] * xh[j][e];
                dw_acc[j][e] += g[j][e] * xh[j][e];
                db_acc[j][e] += g[j][e];
            }
        }
        s1 = wave_sum(s1) * (1.0f / C);
        s2 = wave_sum(s2) * (1.0f / C);
        VT* dr = (VT*)(dres + row * C);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float o[VEC], prev[VEC];
            if (accumulate) Vec<VEC>::unpack(in.rv[j], prev);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                o[e] = (wdy[j][e] - s1 - xh[j][e] * s2) * in.rs;
                if (accumulate) o[e] += prev[e];
            }
            dr[j * 64 + lane] = Vec<VEC>::pack(o);
        }
    };
    const int64_t stride = (int64_t)gridDim.x * ROWS_PER_BLOCK;
    int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + wave;
    RowIn a, b;
    if (row < rows) load(row, a);
    while (row < rows) {
        const int64_t r1 = row + stride;
        if (r1 < rows) load(r1, b);
        compute(row, a);
        if (r1 >= rows) break;
        const int64_t r2 = r1 + stride;
        if (r2 < rows) load(r2, a);
        compute(r1, b);
        row = r2;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            red[wave][0][(j * 64 + lane) * VEC + e] = dw_acc[j][e];
            red[wave][1][(j * 64 + lane) * VEC + e] = db_acc[j][e];
        }
    __syncthreads();
    for (int c = threadIdx.x; c < 2 * C; c += blockDim.x) {
        int k = c / C, cc = c % C;
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < ROWS_PER_BLOCK; ++r) s += red[r][k][cc];
        partial[(int64_t)blockIdx.x * 2 * C + c] = s;
    }
}

// Fold of the per-block column partials into dw (rows [0, C)) and db (rows
// [C, 2C)), in two launches whose additions happen in a fixed order, so the
// parameter gradients are the same bits on every run.  Stage 1: block (x, y, z)
// sums partial rows y, y + FOLD_SEGS, ... of slot z for 256 columns (coalesced
// loads, 8 independent accumulators) and stores the segment sum in row y, the
// first row it read (no other block reads those columns of that row).  Stage 2
// adds the min(FOLD_SEGS, nblocks) segment sums of a column in segment order.
constexpr int FOLD_SEGS = 16;
struct LnFoldSet {
    float* dw[LN_FOLD_MAX];
    float* db[LN_FOLD_MAX];
};
__global__ __launch_bounds__(256) void fold_segments_kernel(float* __restrict__ partial, int64_t slot_elems,
                                                            int nblocks, int C) {
    float* part = partial + (int64_t)blockIdx.z * slot_elems;
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int y = blockIdx.y;
    if (c >= 2 * C || y >= nblocks) return;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int b = y;
    for (; b + 7 * FOLD_SEGS < nblocks; b += 8 * FOLD_SEGS) {
#pragma unroll
        for (int u = 0; u < 8; ++u) s[u] += part[(int64_t)(b + u * FOLD_SEGS) * 2 * C + c];
    }
    for (; b < nblocks; b += FOLD_SEGS) s[0] += part[(int64_t)b * 2 * C + c];
    part[(int64_t)y * 2 * C + c] = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}
__global__ __launch_bounds__(256) void fold_finish_kernel(const float* __restrict__ partial, int64_t slot_elems,
                                                          int nblocks, int C, LnFoldSet set) {
    const float* part = partial + (int64_t)blockIdx.y * slot_elems;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= 2 * C) return;
    const int nseg = min(FOLD_SEGS, nblocks);
    float t = 0.f;
    for (int y = 0; y < nseg; ++y) t += part[(int64_t)y * 2 * C + c];
    if (c < C)
        set.dw[blockIdx.y][c] += t;
    else
        set.db[blockIdx.y][c - C] += t;
}

hipError_t fold_slots(float* partial, int64_t slot_elems, int nslots, int nblocks, int C, const LnFoldSet& set,
                      hipStream_t s) {
    PROF_LAUNCH(KC_FOLD, 8.0 * nblocks * C * nslots, s,
                prof_launch(fold_segments_kernel, dim3(cdiv(2 * C, 256), FOLD_SEGS, nslots), dim3(256), 0, s,
                                   partial, slot_elems, nblocks, C));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PROF_LAUNCH(KC_FOLD, 8.0 * std::min(FOLD_SEGS, nblocks) * C * nslots, s,
                prof_launch(fold_finish_kernel, dim3(cdiv(2 * C, 256), nslots), dim3(256), 0, s, partial,
                                   slot_elems, nblocks, C, set));
    return hipGetLastError();
}

int ln_blocks(int64_t rows) { return (int)std::min<int64_t>(768, cdiv(rows, ROWS_PER_BLOCK)); }

template <int VEC, int NV>
hipError_t ln_fwd_t(const uint16_t* x, const float* w, const float* b, uint16_t* y, float* mean, float* rstd,
                    int64_t rows, hipStream_t s) {
    constexpr int C = NV * 64 * VEC;
    if constexpr (C % 256 == 0) {
        // half-wave rows with 16-byte loads: eight rows per block of four waves
        const int blocks = (int)std::min<int64_t>(768, cdiv(rows, 2 * ROWS_PER_BLOCK));
        PROF_LAUNCH(KC_LN_FWD, 4.0 * rows * C, s,
                    prof_launch((ln_fwd16_kernel<C / 256>), dim3(blocks), dim3(256), 0, s, x, w, b, y, mean,
                                       rstd, rows));
    } else {
        PROF_LAUNCH(KC_LN_FWD, 4.0 * rows * C, s,
                    prof_launch((ln_fwd_kernel<VEC, NV>), dim3(ln_blocks(rows)), dim3(256), 0, s, x, w, b, y,
                                       mean, rstd, rows));
    }
    return hipGetLastError();
}

template <int VEC, int NV>
hipError_t ln_bwd_t(const uint16_t* x, const uint16_t* dy, const float* w, const float* mean, const float* rstd,
                    const uint16_t* dres_in, uint16_t* dres, int accumulate, float* dw, float* db, float* partial,
                    int64_t rows,
                    hipStream_t s) {
    constexpr int C = NV * 64 * VEC;
    int blocks = ln_blocks(rows);
    PROF_LAUNCH(KC_LN_BWD, 2.0 * rows * C * (accumulate ? 4 : 3), s, prof_launch((ln_bwd_kernel<VEC, NV>), dim3(blocks), dim3(256), 0, s, x, dy, w, mean, rstd, dres_in, dres,
                       accumulate, partial, rows));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || dw == nullptr) return e;  // no dw: the partials are folded later
    LnFoldSet set{};
    set.dw[0] = dw;
    set.db[0] = db;
    return fold_slots(partial, (int64_t)blocks * 2 * C, 1, blocks, C, set, s);
}

}  // namespace

#define LN_CASES(X)  \
    X(128, 2, 1)     \
    X(256, 4, 1)     \
    X(384, 2, 3)     \
    X(512, 4, 2)     \
    X(768, 4, 3)     \
    X(1024, 4, 4)    \
    X(1536, 4, 6)    \
    X(2048, 4, 8)    \
    X(3072, 4, 12)

hipError_t launch_layernorm_fwd(const uint16_t* x, const float* w, const float* b, uint16_t* y, float* mean,
                                float* rstd, int64_t rows, int C, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    switch (C) {
#define X(c, vec, nv) \
    case c: return ln_fwd_t<vec, nv>(x, w, b, y, mean, rstd, rows, s);
        LN_CASES(X)
#undef X
    }
    return hipErrorInvalidValue;
}

int64_t layernorm_bwd_partial_elems(int64_t rows, int C) { return (int64_t)ln_blocks(rows) * 2 * C; }

hipError_t launch_layernorm_bwd(const uint16_t* x, const uint16_t* dy, const float* w, const float* mean,
                                const float* rstd, const uint16_t* dres_in, uint16_t* dres, int accumulate,
                                float* dw, float* db,
                                float* partial, int64_t rows, int C, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    switch (C) {
#define X(c, vec, nv) \
    case c: return ln_bwd_t<vec, nv>(x, dy, w, mean, rstd, dres_in, dres, accumulate, dw, db, partial, rows, s);
        LN_CASES(X)
#undef X
    }
    return hipErrorInvalidValue;
}

hipError_t launch_layernorm_fold(float* partial, int64_t slot_elems, int nslots, float* const* dw, float* const* db,
                                 int64_t rows, int C, hipStream_t s) {
    if (nslots < 1 || nslots > LN_FOLD_MAX || rows <= 0) return nslots == 0 ? hipSuccess : hipErrorInvalidValue;
    LnFoldSet set{};
    for (int i = 0; i < nslots; ++i) {
        set.dw[i] = dw[i];
        set.db[i] = db[i];
    }
    return fold_slots(partial, slot_elems, nslots, ln_blocks(rows), C, set, s);
}

bool layernorm_supports(int C) {
    switch (C) {
#define X(c, vec, nv) \
    case c: return true;
        LN_CASES(X)
#undef X
    }
    return false;
}
