// Causal multi-head attention forward and backward on gfx950 MFMA.
//
// GLM activity 5/6 (scaled dot-product attention softmax(Q K^T / sqrt(d)) V
// with a causal mask, heads as parallel projections); PDS model text around
// Fig. 1 (GPT-2 124M: 12 heads of 64).  Flash-attention style: scores never
// reach HBM; the forward keeps a running max / sum per query (online softmax)
// and saves the natural-log log-sum-exp of each query's scaled scores; the
// backward recomputes probabilities from it.
//
// Layouts.  The forward and the dQ kernel compute transposed score tiles
// S^T = K Q^T with the 32x32x16 MFMA, so each lane owns one query (its
// column) and 16 keys of a 32-key tile: the per-query softmax state lives in
// one lane and its partner l^32, and the probabilities in registers are
// directly the B operand of O^T = V^T P^T.  The dK/dV kernel uses S = Q K^T
// (lane = key) for the same reason.  Operands that are needed transposed
// (V^T, K^T, Q^T, dO^T) are read from the row-major LDS tiles with
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8-byte chunks addressed by lanes i/4, 4+i/4, 8+i/4 and 12+i/4, so two
// such reads assemble an MFMA A operand whose key order matches the score
// accumulator's registers.
//
// Pipelining.  Each workgroup stages the next 64-row block of its streamed
// operands in registers while it multiplies the current one, then writes it
// to the other LDS buffer: one barrier per block.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace {

constexpr int QB = 128;     // rows owned per workgroup (4 waves x 32)
constexpr int KVB = 64;     // streamed rows per step
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_LOG2 = 8.0f;  // forward: largest probability 2^8 before a rescale

typedef short v4s __attribute__((ext_vector_type(4)));

// Work unit of a workgroup: head bh and row-block rank (0 = the heaviest).
// Workgroups reach the eight XCDs round-robin by linear index (XCD = index mod
// 8), and each XCD has its own L2.  Head bh goes to XCD bh mod 8, so every row
// block of a head reads that head's operands through one L2; within an XCD the
// units run in rank order, the heaviest row block of each of its heads first, so
// every XCD receives an equal share of each causal work level and the row blocks
// of one head that run at the same time share their streamed blocks in L2.  The
// grid holds 8 * ceil(BH / 8) * nunits workgroups; the spare ones of XCDs with a
// head fewer return false (before any memory access or barrier).
__device__ __forceinline__ bool attn_unit(int BH, int nunits, int& bh, int& rank) {
    const int x = (int)(blockIdx.x & 7u), j = (int)(blockIdx.x >> 3);
    const int nx = (BH - x + 7) >> 3;  // heads x, x + 8, ... below BH
    if (j >= nx * nunits) return false;
    rank = j / nx;
    bh = x + 8 * (j - rank * nx);
    return true;
}

inline unsigned attn_grid(int BH, int T) { return (unsigned)(8 * cdiv(BH, 8) * cdiv(T, QB)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A operand X^T (rows = features col0..col0+31, k = 16 streamed rows of step ks) from a
// row-major LDS tile X[row][feature] with row stride ld: element e of lane (f, g) is
// X[16 ks + 8 (e/4) + 4 g + e%4][col0 + f].
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* tile, int ld, int ks, int col0, int lane) {
    const int grp = lane >> 4, j = lane & 15, g = lane >> 5;
    const uint16_t* p = tile + (16 * ks + 4 * g + (j >> 2)) * ld + col0 + 16 * (grp & 1) + 4 * (j & 3);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 8 * ld));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand X (rows row0 + lane%32, k = d 16 kk .. +15) from a row-major tile.
__device__ __forceinline__ const bf16x8& frag_rows(const uint16_t* tile, int ld, int row0, int kk, int lane) {
    return *(const bf16x8*)(tile + (row0 + (lane & 31)) * ld + kk * 16 + (lane >> 5) * 8);
}

// Register staging of a 64 x D block of one qkv/dout third through buffer loads.
// The resource holds the operand's base for this sequence and head; each
// thread's byte offsets within a block are fixed and a block's first row enters
// as the scalar offset, so a block costs no per-thread address arithmetic.
constexpr int BUF_DWORD3 = 0x00020000;  // buffer resource word 3 for gfx9-family raw loads

template <int D>
struct Stage {
    static constexpr int NV = KVB * D / 8 / 256;
    static_assert(NV >= 1, "at least one vector per thread");
    u32x4 v[NV];
    int voff[NV];
    int row_bytes;
    __amdgpu_buffer_rsrc_t rs;
    // base: element (row 0, column 0) of the operand; ld: row stride in elements;
    // rows: rows addressable from base (every block lies inside them)
    __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int rows, int tid) {
        row_bytes = (int)ld * 2;
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (rows - 1) * row_bytes + D * 2, BUF_DWORD3);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int vid = tid + 256 * i, r = vid / (D / 8), c = vid % (D / 8);
            voff[i] = r * row_bytes + c * 16;
        }
    }
    __device__ __forceinline__ void load(int row0) {
        const int so = row0 * row_bytes;
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], so, 0);
    }
    __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int vid = tid + 256 * i, r = vid / (D / 8), c = vid % (D / 8);
            *(u32x4*)(s + r * (D + 8) + c * 8) = v[i];
        }
    }
};


// ---------------------------------------------------------------- forward

// Each workgroup iteration: per 32-key half the wave reads its 4 K fragments
// and issues the S^T MFMAs; after the softmax it reads the V^T fragments one
// 16-key step at a time, just ahead of that step's O^T MFMAs.  Holding no
// more fragments than that keeps the kernel at 128 VGPRs (four waves per
// SIMD), and the other waves cover the LDS latency.  Scores stay in raw units: the max is taken
// on raw scores and exp2(s * scale*log2e - m * scale*log2e) is one FMA + exp.
// Masks are applied only on blocks that straddle the diagonal; the reference
// max (and with it O and l) is moved only when a block max exceeds it by more
// than a factor 2^RESCALE_LOG2 in probability.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const uint16_t* __restrict__ qkv,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse,
                                                          int T, int H, int C, int BH, float sl) {
    constexpr int LD = D + 8;
    constexpr int KK = D / 16, DT = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][KVB * LD];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][KVB * LD];
    const int nqb = (int)cdiv(T, QB);
    int bh, rank;
    if (!attn_unit(BH, nqb, bh, rank)) return;
    const int q0 = (nqb - 1 - rank) * QB;  // heaviest blocks first
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: causal tests are scalar branches
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* Qg = qkv + (int64_t)b * T * ld + h * D;
    const uint16_t* Kg = Qg + C;
    const uint16_t* Vg = Qg + 2 * C;

    const int qw = q0 + wave * 32;
    const int qi = qw + (lane & 31);
    const bool qvalid = qi < T;
    bf16x8 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = qvalid ? *(const bf16x8*)(Qg + (int64_t)qi * ld + kk * 16 + g * 8) : bf16x8{};
    floatx16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int q_last = min(q0 + QB - 1, T - 1);
    const int nkv = q_last / KVB + 1;
    const int q_last_w = min(qw + 31, T - 1);
    Stage<D> stk, stv;
    stk.init(Kg, ld, T, tid);
    stv.init(Vg, ld, T, tid);
    stk.load(0);
    stv.load(0);
    stk.store(sK[0], tid);
    stv.store(sV[0], tid);
    __syncthreads();
    for (int kb = 0; kb < nkv; ++kb) {
        const int buf = kb & 1;
        const int s0 = kb * KVB;
        if (kb + 1 < nkv) {
            stk.load(s0 + KVB);
            stv.load(s0 + KVB);
        }
        if (qw < T && s0 <= q_last_w) {
            floatx16 sacc[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 kfr[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) kfr[kk] = frag_rows(sK[buf], LD, st * 32, kk, lane);
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[st][r] = 0.f;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) sacc[st] = mfma32(kfr[kk], qf[kk], sacc[st]);
            }
            if (s0 + KVB - 1 > qw) {  // block straddles the diagonal for this wave
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (s0 + st * 32 + acc_row(r, lane) > qi) sacc[st][r] = -INFINITY;
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[st][r]);
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, WAVE));
            // The reference m_run moves only when some query's block max exceeds it
            // by more than RESCALE_LOG2 (log2 units), so probabilities stay below
            // 2^RESCALE_LOG2 and the O / l rescale is rare; numerator and denominator
            // share the reference, so the result is unchanged.  The first block
            // always sets it (m_run = -inf; key 0 is visible to every query).
            if (__any((mloc - m_run) * sl > RESCALE_LOG2)) {
                const float m_new = fmaxf(m_run, mloc);
                const float alpha = fast_exp2((m_run - m_new) * sl);
                l_run *= alpha;
                m_run = m_new;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
            }
            const float mb = m_run * sl;
            bf16x8 pf[KVB / 16];
            float ls[KVB / 16];
#pragma unroll
            for (int ks = 0; ks < KVB / 16; ++ks) {
                const int st = ks >> 1, half = ks & 1;
                float pv[8];
                ls[ks] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = fast_exp2(fmaf(sacc[st][8 * half + e], sl, -mb));
                    ls[ks] += pv[e];
                }
                pf[ks] = pack8(pv);
            }
            l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
            for (int ks = 0; ks < KVB / 16; ++ks) {
                bf16x8 vfr[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vfr[dt] = frag_tr(sV[buf], LD, ks, dt * 32, lane);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(vfr[dt], pf[ks], acc[dt]);
            }
        }
        if (kb + 1 < nkv) {
            // buffer buf^1 was last read in step kb-1, before the previous barrier
            stk.store(sK[buf ^ 1], tid);
            stv.store(sV[buf ^ 1], tid);
        }
        __syncthreads();
    }
    if (!qvalid) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32, WAVE);
    const float inv = 1.0f / l_tot;
    uint16_t* orow = out + ((int64_t)b * T + qi) * C + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d0 = dt * 32 + 8 * rg + 4 * g;
            u32x2 w{pack_bf2(acc[dt][4 * rg] * inv, acc[dt][4 * rg + 1] * inv),
                    pack_bf2(acc[dt][4 * rg + 2] * inv, acc[dt][4 * rg + 3] * inv)};
            *(u32x2*)(orow + d0) = w;
        }
    if (g == 0) lse[((int64_t)b * H + h) * T + qi] = (m_run * sl + log2f(l_tot)) * LN2;
}

// ---------------------------------------------------------------- backward

// dK, dV for 128 keys per workgroup (lane = key), looping over 64-query blocks;
// each block is processed as two 32-query halves (it).  Per half: Q and dO
// fragments -> S and dP MFMAs; Q^T and dO^T fragments are read while the
// probabilities P = exp2(S sl - lse2) and dS = P (dP - D) are formed; then the
// dV += dO^T P and dK += Q^T dS MFMAs.  LSE and D of the half's rows are read
// as float4 (4 consecutive query rows per accumulator register group).
template <int D>
__global__ __launch_bounds__(256, 2) void attn_dkdv_kernel(const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ dvec,
                                                           uint16_t* __restrict__ dqkv, int T, int H, int C,
                                                           int BH, float sl, float scale) {
    constexpr int LD = D + 8;
    constexpr int KK = D / 16, DT = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[2][KVB * LD];
    __shared__ __attribute__((aligned(16))) uint16_t sdO[2][KVB * LD];
    __shared__ __attribute__((aligned(16))) float sL[2][KVB];
    __shared__ __attribute__((aligned(16))) float sDv[2][KVB];
    int bh, rank;
    if (!attn_unit(BH, (int)cdiv(T, QB), bh, rank)) return;
    const int k0 = rank * QB;  // the first key blocks see the most queries
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: causal tests are scalar branches
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
    bf16x8 kf[KK], vf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        kf[kk] = kvalid ? *(const bf16x8*)(Kg + (int64_t)sk * ld + kk * 16 + g * 8) : bf16x8{};
        vf[kk] = kvalid ? *(const bf16x8*)(Vg + (int64_t)sk * ld + kk * 16 + g * 8) : bf16x8{};
    }
    floatx16 adk[DT], adv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            adk[dt][r] = 0.f;
            adv[dt][r] = 0.f;
        }

    const int i_first = k0;  // k0 is a multiple of 128 below T
    const int nqb = (T - i_first) / KVB;
    Stage<D> stq, sto;
    stq.init(Qg, ld, T, tid);
    sto.init(dOg, C, T, tid);
    float rl = 0.f, rd = 0.f;
    auto load_block = [&](int i0) {
        stq.load(i0);
        sto.load(i0);
        if (tid < KVB) {  // consumed by store_block only, so the loads stay in flight through the block
            rl = lse_bh[i0 + tid];
            rd = dv_bh[i0 + tid];
        }
    };
    auto store_block = [&](int buf) {
        stq.store(sQ[buf], tid);
        sto.store(sdO[buf], tid);
        if (tid < KVB) {
            sL[buf][tid] = rl * LOG2E;
            sDv[buf][tid] = rd;
        }
    };
    load_block(i_first);
    store_block(0);
    __syncthreads();
    for (int qb = 0; qb < nqb; ++qb) {
        const int buf = qb & 1;
        const int i0 = i_first + qb * KVB;
        if (qb + 1 < nqb) load_block(i0 + KVB);
        if (kw < T && kw <= i0 + KVB - 1) {  // some query of this block sees some key of this wave
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                if (kw > i0 + it * 32 + 31) continue;  // every key after every query of this half
                bf16x8 qa[KK], oa[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    qa[kk] = frag_rows(sQ[buf], LD, it * 32, kk, lane);
                    oa[kk] = frag_rows(sdO[buf], LD, it * 32, kk, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
                floatx16 sacc, dpacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[r] = 0.f;
                    dpacc[r] = 0.f;
                }
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    sacc = mfma32(qa[kk], kf[kk], sacc);
                    dpacc = mfma32(oa[kk], vf[kk], dpacc);
                }
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 qt[2][DT], ot[2][DT];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        qt[hh][dt] = frag_tr(sQ[buf], LD, 2 * it + hh, dt * 32, lane);
                        ot[hh][dt] = frag_tr(sdO[buf], LD, 2 * it + hh, dt * 32, lane);
                    }
                float4 l4[4], d4[4];
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    l4[qd] = *(const float4*)(&sL[buf][it * 32 + 8 * qd + 4 * g]);
                    d4[qd] = *(const float4*)(&sDv[buf][it * 32 + 8 * qd + 4 * g]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const float lv[4] = {l4[qd].x, l4[qd].y, l4[qd].z, l4[qd].w};
                    const float dv[4] = {d4[qd].x, d4[qd].y, d4[qd].z, d4[qd].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float pr = fast_exp2(fmaf(sacc[4 * qd + e], sl, -lv[e]));
                        sacc[4 * qd + e] = pr;
                        dpacc[4 * qd + e] = pr * (dpacc[4 * qd + e] - dv[e]);
                    }
                }
                if (kw + 31 > i0 + it * 32) {  // half straddles the diagonal: zero s > i
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (sk > i0 + it * 32 + acc_row(r, lane)) {
                            sacc[r] = 0.f;
                            dpacc[r] = 0.f;
                        }
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float pv[8], dsv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        pv[e] = sacc[8 * hh + e];
                        dsv[e] = dpacc[8 * hh + e];
                    }
                    const bf16x8 pf = pack8(pv), dsf = pack8(dsv);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        adv[dt] = mfma32(ot[hh][dt], pf, adv[dt]);
                        adk[dt] = mfma32(qt[hh][dt], dsf, adk[dt]);
                    }
                }
            }
        }
        if (qb + 1 < nqb) store_block(buf ^ 1);
        __syncthreads();
    }
    if (!kvalid) return;
    uint16_t* krow = dqkv + ((int64_t)b * T + sk) * ld + C + h * D;
    uint16_t* vrow = krow + C;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d0 = dt * 32 + 8 * rg + 4 * g;
            *(u32x2*)(krow + d0) = u32x2{pack_bf2(adk[dt][4 * rg] * scale, adk[dt][4 * rg + 1] * scale),
                                         pack_bf2(adk[dt][4 * rg + 2] * scale, adk[dt][4 * rg + 3] * scale)};
            *(u32x2*)(vrow + d0) = u32x2{pack_bf2(adv[dt][4 * rg], adv[dt][4 * rg + 1]),
                                         pack_bf2(adv[dt][4 * rg + 2], adv[dt][4 * rg + 3])};
        }
}

// dQ for 128 queries per workgroup (lane = query), looping over 64-key blocks:
// K and V fragments -> S^T and dP^T MFMAs; K^T fragments are read while
// dS^T = P^T (dP^T - D) is formed; then dQ^T += K^T dS^T.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(const uint16_t* __restrict__ qkv,
                                                         const uint16_t* __restrict__ out,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         float* __restrict__ dvec,
                                                         uint16_t* __restrict__ dqkv, int T, int H, int C,
                                                         int BH, float sl, float scale) {
    constexpr int LD = D + 8;
    constexpr int KK = D / 16, DT = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][KVB * LD];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][KVB * LD];
    const int nqb = (int)cdiv(T, QB);
    int bh, rank;
    if (!attn_unit(BH, nqb, bh, rank)) return;
    const int q0 = (nqb - 1 - rank) * QB;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: causal tests are scalar branches
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* Qg = qkv + (int64_t)b * T * ld + h * D;
    const uint16_t* Kg = Qg + C;
    const uint16_t* Vg = Qg + 2 * C;
    const uint16_t* dOg = dout + (int64_t)b * T * C + h * D;

    const int qw = q0 + wave * 32;
    const int qi = qw + (lane & 31);
    const bool qvalid = qi < T;
    bf16x8 qf[KK], df[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = qvalid ? *(const bf16x8*)(Qg + (int64_t)qi * ld + kk * 16 + g * 8) : bf16x8{};
        df[kk] = qvalid ? *(const bf16x8*)(dOg + (int64_t)qi * C + kk * 16 + g * 8) : bf16x8{};
    }
    const float lse2 = qvalid ? lse[((int64_t)b * H + h) * T + qi] * LOG2E : 0.f;
    // D = rowsum(dO * O) of this lane's query: the lane pair (g = 0, 1) holds
    // complementary halves of the dO row, the matching O halves are read with it.
    // The sum is taken once the first K/V block's loads are in flight; the dK/dV
    // kernel, launched after this one, reads D from dvec.
    bf16x8 of[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        of[kk] = qvalid ? *(const bf16x8*)(out + ((int64_t)b * T + qi) * C + h * D + kk * 16 + g * 8) : bf16x8{};
    floatx16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

    const int q_last = min(q0 + QB - 1, T - 1);
    const int nkv = q_last / KVB + 1;
    const int q_last_w = min(qw + 31, T - 1);
    Stage<D> stk, stv;
    stk.init(Kg, ld, T, tid);
    stv.init(Vg, ld, T, tid);
    stk.load(0);
    stv.load(0);
    float dvi = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const u32x4 o = __builtin_bit_cast(u32x4, of[kk]);
        const u32x4 d = __builtin_bit_cast(u32x4, df[kk]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dvi += bflo(o[e]) * bflo(d[e]) + bfhi(o[e]) * bfhi(d[e]);
    }
    dvi += __shfl_xor(dvi, 32, WAVE);
    if (qvalid && g == 0) dvec[((int64_t)b * H + h) * T + qi] = dvi;
    stk.store(sK[0], tid);
    stv.store(sV[0], tid);
    __syncthreads();
    for (int kb = 0; kb < nkv; ++kb) {
        const int buf = kb & 1;
        const int s0 = kb * KVB;
        if (kb + 1 < nkv) {
            stk.load(s0 + KVB);
            stv.load(s0 + KVB);
        }
        if (qw < T && s0 <= q_last_w) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                if (s0 + st * 32 > q_last_w) continue;  // every key of this half after every query
                bf16x8 ka[KK], va[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    ka[kk] = frag_rows(sK[buf], LD, st * 32, kk, lane);
                    va[kk] = frag_rows(sV[buf], LD, st * 32, kk, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
                floatx16 sacc, dpacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[r] = 0.f;
                    dpacc[r] = 0.f;
                }
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    sacc = mfma32(ka[kk], qf[kk], sacc);
                    dpacc = mfma32(va[kk], df[kk], dpacc);
                }
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 kt[2][DT];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) kt[hh][dt] = frag_tr(sK[buf], LD, 2 * st + hh, dt * 32, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = fast_exp2(fmaf(sacc[r], sl, -lse2));
                    dpacc[r] = pr * (dpacc[r] - dvi);
                }
                if (s0 + st * 32 + 31 > qw) {  // half straddles the diagonal
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (s0 + st * 32 + acc_row(r, lane) > qi) dpacc[r] = 0.f;
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float dsv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) dsv[e] = dpacc[8 * hh + e];
                    const bf16x8 dsf = pack8(dsv);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(kt[hh][dt], dsf, acc[dt]);
                }
            }
        }
        if (kb + 1 < nkv) {
            stk.store(sK[buf ^ 1], tid);
            stv.store(sV[buf ^ 1], tid);
        }
        __syncthreads();
    }
    if (!qvalid) return;
    uint16_t* qrow = dqkv + ((int64_t)b * T + qi) * ld + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
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
    const float sl = LOG2E / sqrtf((float)D);
    dim3 grid(attn_grid(B * H, T));
    PROF_LAUNCH(KC_ATTN_FWD, attn_work(B, T, H, D, 2), s,
                prof_launch(attn_fwd_kernel<D>, grid, dim3(256), 0, s, qkv, out, lse, T, H, C, B * H, sl));
    return hipGetLastError();
}

template <int D>
hipError_t bwd_t(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse, uint16_t* dqkv,
                 float* dvec, int B, int T, int H, int C, hipStream_t s) {
    const float scale = 1.0f / sqrtf((float)D);
    const float scale_log2 = LOG2E * scale;
    dim3 grid(attn_grid(B * H, T));
    PROF_LAUNCH(KC_ATTN_DQ, attn_work(B, T, H, D, 3), s,
                prof_launch(attn_dq_kernel<D>, grid, dim3(256), 0, s, qkv, out, dout, lse, dvec, dqkv, T, H, C,
                                   B * H, scale_log2, scale));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PROF_LAUNCH(KC_ATTN_DKDV, attn_work(B, T, H, D, 4), s,
                prof_launch(attn_dkdv_kernel<D>, grid, dim3(256), 0, s, qkv, dout, lse, dvec, dqkv, T, H, C,
                                   B * H, scale_log2, scale));
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
