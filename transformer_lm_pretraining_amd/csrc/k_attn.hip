// Causal multi-head attention forward and backward on gfx950 MFMA.
//
// GLM activity 5/6 (scaled dot-product attention softmax(Q K^T / sqrt(d)) V
// with a causal mask, heads as parallel projections); PDS model text around
// Fig. 1 (GPT-2 124M: 12 heads of 64).  Flash-attention style: scores never
// reach HBM; the forward keeps a running max / sum per query (online softmax)
// and saves the natural-log log-sum-exp of each query's scaled scores; the
// backward recomputes probabilities from it.
//
// Layout trick: the forward and the dQ kernel compute transposed score tiles
// S^T = K Q^T with the 32x32x16 MFMA, so each lane owns one query (its
// column) and 16 keys of a 32-key tile.  The per-query softmax state then
// lives in one lane (plus its partner lane l^32), and the probabilities in
// registers are directly the B operand of O^T = V^T P^T.  V^T comes from an
// LDS tile that is transposed (8x8 bf16 blocks in registers) on the way in.
// The dK/dV kernel uses untransposed S = Q K^T (lane = key) for the same
// reason, with Q^T and dO^T tiles in LDS.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace {

constexpr int QB = 128;     // queries per workgroup (4 waves x 32)
constexpr int KVB = 64;     // keys per inner step
constexpr int TLD = KVB + 4;  // row stride (bf16) of transposed [d][64] tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Row-major [64][D] tile of a qkv third into LDS (stride D+8).
template <int D>
__device__ __forceinline__ void load_rows(uint16_t* s, const uint16_t* g, int64_t ld, int row0, int tid) {
    constexpr int NV = KVB * D / 8;
#pragma unroll
    for (int v = tid; v < NV; v += 256) {
        int r = v / (D / 8), c = v % (D / 8);
        *(u32x4*)(s + r * (D + 8) + c * 8) = *(const u32x4*)(g + (int64_t)(row0 + r) * ld + c * 8);
    }
}

// Transposed tile: s[d][r] = g[row0 + r][d] for r < 64, d < D (stride TLD).
template <int D>
__device__ __forceinline__ void load_rows_t(uint16_t* s, const uint16_t* g, int64_t ld, int row0, int tid) {
    constexpr int NB = (KVB / 8) * (D / 8);
    for (int blk = tid; blk < NB; blk += 256) {
        int sc = blk % (KVB / 8), dc = blk / (KVB / 8);
        u32x4 in[8], o[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) in[rr] = *(const u32x4*)(g + (int64_t)(row0 + sc * 8 + rr) * ld + dc * 8);
        transpose8x8(in, o);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x2* dst = (u32x2*)(s + (dc * 8 + c) * TLD + sc * 8);
            dst[0] = u32x2{o[c].x, o[c].y};
            dst[1] = u32x2{o[c].z, o[c].w};
        }
    }
}

// A-operand fragment from a transposed tile for MFMA k-step ks (16 keys):
// lane (row = base_row + lane%32, group g) takes columns 16ks+4g..+3 and 16ks+8+4g..+3,
// matching the key order of the score accumulator's registers 8*(ks%2) .. +7.
__device__ __forceinline__ bf16x8 frag_t(const uint16_t* s, int row, int ks, int g) {
    const uint16_t* p = s + row * TLD + 16 * ks + 4 * g;
    u32x2 lo = *(const u32x2*)p;
    u32x2 hi = *(const u32x2*)(p + 8);
    return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// ---------------------------------------------------------------- forward

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ out,
                                                       float* __restrict__ lse, int T, int H, int C,
                                                       float scale_log2) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[KVB * (D + 8)];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D * TLD];
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int q0 = (gridDim.x - 1 - blockIdx.x) * QB;  // heaviest blocks first
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* Qg = qkv + (int64_t)b * T * ld + h * D;
    const uint16_t* Kg = Qg + C;
    const uint16_t* Vg = Qg + 2 * C;

    const int qw = q0 + wave * 32;
    const int qi = qw + (lane & 31);
    const bool qvalid = qi < T;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = qvalid ? *(const bf16x8*)(Qg + (int64_t)qi * ld + kk * 16 + g * 8) : bf16x8{};
    floatx16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int q_last = min(q0 + QB - 1, T - 1);
    const int nkv = q_last / KVB + 1;
    const int q_last_w = min(qw + 31, T - 1);
    for (int kb = 0; kb < nkv; ++kb) {
        const int s0 = kb * KVB;
        __syncthreads();
        load_rows<D>(sK, Kg, ld, s0, tid);
        load_rows_t<D>(sVt, Vg, ld, s0, tid);
        __syncthreads();
        if (qw >= T || s0 > q_last_w) continue;
        floatx16 sacc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[st][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                bf16x8 kf = *(const bf16x8*)(sK + (st * 32 + (lane & 31)) * (D + 8) + kk * 16 + g * 8);
                sacc[st] = mfma32(kf, qf[kk], sacc[st]);
            }
        }
        const bool diag = s0 + KVB - 1 > qw;  // some key of this block is after some query of this wave
        float mloc = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = sacc[st][r] * scale_log2;
                if (diag && s0 + st * 32 + acc_row(r, lane) > qi) x = -INFINITY;
                sacc[st][r] = x;
                mloc = fmaxf(mloc, x);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, WAVE));
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = exp2f(m_run - m_new);
        float lsum = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = exp2f(sacc[st][r] - m_new);
                sacc[st][r] = p;
                lsum += p;
            }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
#pragma unroll
        for (int ks = 0; ks < KVB / 16; ++ks) {
            const int st = ks >> 1, half = ks & 1;
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = sacc[st][8 * half + e];
            bf16x8 pf = pack8(pv);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mfma32(frag_t(sVt, dt * 32 + (lane & 31), ks, g), pf, acc[dt]);
        }
    }
    if (!qvalid) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32, WAVE);
    const float inv = 1.0f / l_tot;
    uint16_t* orow = out + ((int64_t)b * T + qi) * C + h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d0 = dt * 32 + 8 * rg + 4 * g;
            u32x2 w{pack_bf2(acc[dt][4 * rg] * inv, acc[dt][4 * rg + 1] * inv),
                    pack_bf2(acc[dt][4 * rg + 2] * inv, acc[dt][4 * rg + 3] * inv)};
            *(u32x2*)(orow + d0) = w;
        }
    if (g == 0) lse[((int64_t)b * H + h) * T + qi] = (m_run + log2f(l_tot)) * LN2;
}

// ---------------------------------------------------------------- backward

// dvec[b,h,i] = sum_d dO[i, h*D + d] * O[i, h*D + d]
template <int D>
__global__ __launch_bounds__(256) void attn_dvec_kernel(const uint16_t* __restrict__ out,
                                                        const uint16_t* __restrict__ dout, float* __restrict__ dvec,
                                                        int B, int T, int H, int C) {
    const int64_t n = (int64_t)B * T * H;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = idx / H;
        const int h = (int)(idx % H);
        const u32x4* o = (const u32x4*)(out + row * C + h * D);
        const u32x4* d = (const u32x4*)(dout + row * C + h * D);
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < D / 8; ++v) {
            u32x4 a = o[v], c = d[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) s += bflo(a[e]) * bflo(c[e]) + bfhi(a[e]) * bfhi(c[e]);
        }
        const int64_t b = row / T, t = row % T;
        dvec[(b * H + h) * T + t] = s;
    }
}

// dK, dV for 128 keys per workgroup (lane = key), looping over 64-query blocks.
template <int D>
__global__ __launch_bounds__(256) void attn_dkdv_kernel(const uint16_t* __restrict__ qkv,
                                                        const uint16_t* __restrict__ dout,
                                                        const float* __restrict__ lse, const float* __restrict__ dvec,
                                                        uint16_t* __restrict__ dqkv, int T, int H, int C,
                                                        float scale_log2, float scale) {
    __shared__ __attribute__((aligned(16))) uint16_t sQ[KVB * (D + 8)];
    __shared__ __attribute__((aligned(16))) uint16_t sdO[KVB * (D + 8)];
    __shared__ __attribute__((aligned(16))) uint16_t sQt[D * TLD];
    __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * TLD];
    __shared__ float sL[KVB], sDv[KVB];
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int k0 = blockIdx.x * QB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* Qg = qkv + (int64_t)b * T * ld + h * D;
    const uint16_t* Kg = Qg + C;
    const uint16_t* Vg = Qg + 2 * C;
    const uint16_t* dOg = dout + (int64_t)b * T * C + h * D;
    const float* lse_bh = lse + ((int64_t)b * H + h) * T;
    const float* dv_bh = dvec + ((int64_t)b * H + h) * T;

    const int kw = k0 + wave * 32;  // first key of this wave
    const int sk = kw + (lane & 31);
    const bool kvalid = sk < T;
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        kf[kk] = kvalid ? *(const bf16x8*)(Kg + (int64_t)sk * ld + kk * 16 + g * 8) : bf16x8{};
        vf[kk] = kvalid ? *(const bf16x8*)(Vg + (int64_t)sk * ld + kk * 16 + g * 8) : bf16x8{};
    }
    floatx16 adk[D / 32], adv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            adk[dt][r] = 0.f;
            adv[dt][r] = 0.f;
        }

    for (int i0 = (k0 / KVB) * KVB; i0 < T; i0 += KVB) {
        __syncthreads();
        load_rows<D>(sQ, Qg, ld, i0, tid);
        load_rows<D>(sdO, dOg, C, i0, tid);
        load_rows_t<D>(sQt, Qg, ld, i0, tid);
        load_rows_t<D>(sdOt, dOg, C, i0, tid);
        if (tid < KVB) {
            sL[tid] = lse_bh[i0 + tid] * LOG2E;
            sDv[tid] = dv_bh[i0 + tid];
        }
        __syncthreads();
        if (kw >= T || kw > i0 + KVB - 1) continue;  // every key of this wave is after every query
        floatx16 sacc[2], dpacc[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[it][r] = 0.f;
                dpacc[it][r] = 0.f;
            }
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const int off = (it * 32 + (lane & 31)) * (D + 8) + kk * 16 + g * 8;
                sacc[it] = mfma32(*(const bf16x8*)(sQ + off), kf[kk], sacc[it]);
                dpacc[it] = mfma32(*(const bf16x8*)(sdO + off), vf[kk], dpacc[it]);
            }
        }
        // P and dS; rows = queries i0 + it*32 + acc_row(r), column = key sk
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ii = it * 32 + acc_row(r, lane);
                float p = exp2f(sacc[it][r] * scale_log2 - sL[ii]);
                if (sk > i0 + ii) p = 0.f;
                sacc[it][r] = p;
                dpacc[it][r] = p * (dpacc[it][r] - sDv[ii]);
            }
#pragma unroll
        for (int ks = 0; ks < KVB / 16; ++ks) {
            const int it = ks >> 1, half = ks & 1;
            float pv[8], dsv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = sacc[it][8 * half + e];
                dsv[e] = dpacc[it][8 * half + e];
            }
            bf16x8 pf = pack8(pv), dsf = pack8(dsv);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                adv[dt] = mfma32(frag_t(sdOt, dt * 32 + (lane & 31), ks, g), pf, adv[dt]);
                adk[dt] = mfma32(frag_t(sQt, dt * 32 + (lane & 31), ks, g), dsf, adk[dt]);
            }
        }
    }
    if (!kvalid) return;
    uint16_t* krow = dqkv + ((int64_t)b * T + sk) * ld + C + h * D;
    uint16_t* vrow = krow + C;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d0 = dt * 32 + 8 * rg + 4 * g;
            *(u32x2*)(krow + d0) = u32x2{pack_bf2(adk[dt][4 * rg] * scale, adk[dt][4 * rg + 1] * scale),
                                         pack_bf2(adk[dt][4 * rg + 2] * scale, adk[dt][4 * rg + 3] * scale)};
            *(u32x2*)(vrow + d0) = u32x2{pack_bf2(adv[dt][4 * rg], adv[dt][4 * rg + 1]),
                                         pack_bf2(adv[dt][4 * rg + 2], adv[dt][4 * rg + 3])};
        }
}

// dQ for 128 queries per workgroup (lane = query), looping over 64-key blocks.
template <int D>
__global__ __launch_bounds__(256) void attn_dq_kernel(const uint16_t* __restrict__ qkv,
                                                      const uint16_t* __restrict__ dout,
                                                      const float* __restrict__ lse, const float* __restrict__ dvec,
                                                      uint16_t* __restrict__ dqkv, int T, int H, int C,
                                                      float scale_log2, float scale) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[KVB * (D + 8)];
    __shared__ __attribute__((aligned(16))) uint16_t sV[KVB * (D + 8)];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[D * TLD];
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int q0 = (gridDim.x - 1 - blockIdx.x) * QB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* Qg = qkv + (int64_t)b * T * ld + h * D;
    const uint16_t* Kg = Qg + C;
    const uint16_t* Vg = Qg + 2 * C;
    const uint16_t* dOg = dout + (int64_t)b * T * C + h * D;

    const int qw = q0 + wave * 32;
    const int qi = qw + (lane & 31);
    const bool qvalid = qi < T;
    bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        qf[kk] = qvalid ? *(const bf16x8*)(Qg + (int64_t)qi * ld + kk * 16 + g * 8) : bf16x8{};
        df[kk] = qvalid ? *(const bf16x8*)(dOg + (int64_t)qi * C + kk * 16 + g * 8) : bf16x8{};
    }
    const float lse2 = qvalid ? lse[((int64_t)b * H + h) * T + qi] * LOG2E : 0.f;
    const float dvi = qvalid ? dvec[((int64_t)b * H + h) * T + qi] : 0.f;
    floatx16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

    const int q_last = min(q0 + QB - 1, T - 1);
    const int nkv = q_last / KVB + 1;
    const int q_last_w = min(qw + 31, T - 1);
    for (int kb = 0; kb < nkv; ++kb) {
        const int s0 = kb * KVB;
        __syncthreads();
        load_rows<D>(sK, Kg, ld, s0, tid);
        load_rows<D>(sV, Vg, ld, s0, tid);
        load_rows_t<D>(sKt, Kg, ld, s0, tid);
        __syncthreads();
        if (qw >= T || s0 > q_last_w) continue;
        floatx16 sacc[2], dpacc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[st][r] = 0.f;
                dpacc[st][r] = 0.f;
            }
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const int off = (st * 32 + (lane & 31)) * (D + 8) + kk * 16 + g * 8;
                sacc[st] = mfma32(*(const bf16x8*)(sK + off), qf[kk], sacc[st]);
                dpacc[st] = mfma32(*(const bf16x8*)(sV + off), df[kk], dpacc[st]);
            }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = exp2f(sacc[st][r] * scale_log2 - lse2);
                if (s0 + st * 32 + acc_row(r, lane) > qi) p = 0.f;
                dpacc[st][r] = p * (dpacc[st][r] - dvi);
            }
#pragma unroll
        for (int ks = 0; ks < KVB / 16; ++ks) {
            const int st = ks >> 1, half = ks & 1;
            float dsv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) dsv[e] = dpacc[st][8 * half + e];
            bf16x8 dsf = pack8(dsv);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mfma32(frag_t(sKt, dt * 32 + (lane & 31), ks, g), dsf, acc[dt]);
        }
    }
    if (!qvalid) return;
    uint16_t* qrow = dqkv + ((int64_t)b * T + qi) * ld + h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d0 = dt * 32 + 8 * rg + 4 * g;
            *(u32x2*)(qrow + d0) = u32x2{pack_bf2(acc[dt][4 * rg] * scale, acc[dt][4 * rg + 1] * scale),
                                         pack_bf2(acc[dt][4 * rg + 2] * scale, acc[dt][4 * rg + 3] * scale)};
        }
}

// MFMA work executed over the causal pairs (t, s <= t): `matmuls` products of 2*D FLOP per pair.
double attn_work(int B, int T, int H, int D, int matmuls) {
    return (double)B * H * ((double)T * (T + 1) / 2.0) * 2.0 * D * matmuls;
}

template <int D>
hipError_t fwd_t(const uint16_t* qkv, uint16_t* out, float* lse, int B, int T, int H, int C, hipStream_t s) {
    const float scale_log2 = LOG2E / sqrtf((float)D);
    dim3 grid((unsigned)cdiv(T, QB), (unsigned)(B * H));
    PROF_LAUNCH(KC_ATTN_FWD, attn_work(B, T, H, D, 2), s, hipLaunchKernelGGL(attn_fwd_kernel<D>, grid, dim3(256), 0, s, qkv, out, lse, T, H, C, scale_log2));
    return hipGetLastError();
}

template <int D>
hipError_t bwd_t(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse, uint16_t* dqkv,
                 float* dvec, int B, int T, int H, int C, hipStream_t s) {
    const float scale = 1.0f / sqrtf((float)D);
    const float scale_log2 = LOG2E * scale;
    int64_t n = (int64_t)B * T * H;
    PROF_LAUNCH(KC_ATTN_DVEC, 4.0 * (double)n * D, s, hipLaunchKernelGGL(attn_dvec_kernel<D>, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 8192)), dim3(256), 0, s,
                       out, dout, dvec, B, T, H, C));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)cdiv(T, QB), (unsigned)(B * H));
    PROF_LAUNCH(KC_ATTN_DKDV, attn_work(B, T, H, D, 4), s, hipLaunchKernelGGL(attn_dkdv_kernel<D>, grid, dim3(256), 0, s, qkv, dout, lse, dvec, dqkv, T, H, C, scale_log2,
                       scale));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    PROF_LAUNCH(KC_ATTN_DQ, attn_work(B, T, H, D, 3), s, hipLaunchKernelGGL(attn_dq_kernel<D>, grid, dim3(256), 0, s, qkv, dout, lse, dvec, dqkv, T, H, C, scale_log2,
                       scale));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fwd(const uint16_t* qkv, uint16_t* out, float* lse, int B, int T, int H, int C,
                                hipStream_t s) {
    if (T % KVB) return hipErrorInvalidValue;
    switch (C / H) {
        case 64: return fwd_t<64>(qkv, out, lse, B, T, H, C, s);
        case 32: return fwd_t<32>(qkv, out, lse, B, T, H, C, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attention_bwd(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse,
                                uint16_t* dqkv, float* dvec, int B, int T, int H, int C, hipStream_t s) {
    if (T % KVB) return hipErrorInvalidValue;
    switch (C / H) {
        case 64: return bwd_t<64>(qkv, out, dout, lse, dqkv, dvec, B, T, H, C, s);
        case 32: return bwd_t<32>(qkv, out, dout, lse, dqkv, dvec, B, T, H, C, s);
    }
    return hipErrorInvalidValue;
}
