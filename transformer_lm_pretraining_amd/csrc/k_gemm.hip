// bf16 GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// The linear layers of the GPT-2 block and the tied lm_head (PDS model text
// around Fig. 1) run three products:
//   forward / input gradient ("NT"): C[M,N] = A[M,K] . B[N,K]^T, both operands
//     contiguous along the reduction.  The input-gradient GEMMs use the
//     transposed bf16 weight copy so they are NT products too;
//   weight gradient ("TN"): dW[N,K] += sum_m dY[m,n] X[m,k], reduction over
//     tokens, operands contiguous along the output dims.  Their tiles are
//     transposed in registers (8x8 bf16 blocks) on the way into LDS, so the
//     MFMA loop is identical for both.  The bias gradient (column sums of dY)
//     is folded into the same pass: the workgroups of the first output column
//     tile sum the dY tiles they load anyway.
// Tiles: BM x BN per workgroup of WGM x WGN waves, K step 64, LDS double
// buffered (one barrier per K step) with register prefetch of the next tile;
// LDS rows padded to 72 bf16 (144 B) so the 16-byte fragment reads of 32
// consecutive rows hit distinct banks.  Workgroups are renumbered so each of
// the 8 XCDs (own L2 each) walks a contiguous run of the grouped tile order.
// Weight-gradient GEMMs split the token reduction (uneven splits allowed) to
// fill the 256 CUs; the fp32 partials are summed into dW by a second kernel.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;
constexpr int NUM_CU = 256;

enum Epi { EPI_BF16 = 0, EPI_GELU = 1, EPI_DGELU = 2, EPI_F32_ACC = 3, EPI_F32_STORE = 4 };

struct GemmParams {
    const uint16_t* A;
    const uint16_t* B;
    int64_t lda, ldb;
    int M, N;          // output rows / cols
    int nk_total;      // reduction length / BK
    int splits;
    int tiles_m, tiles_n;
    const float* bias;
    const uint16_t* res;   // residual (EPI_BF16) or pre-activation (EPI_DGELU)
    int64_t ldr;
    uint16_t* out;
    uint16_t* out2;
    int64_t ldo;
    float* outf;
    int64_t ldf;
    int64_t split_stride;
    float* dbias;      // TN: bias gradient (column sums of A's source), may be null
};

// Tile loader for an operand stored contiguous along the reduction:
// element (row, k) at base[row * ld + k].
template <int R, int NT>
struct LoaderK {
    static constexpr int NV = R * (BK / 8) / NT;
    static_assert(NV * NT == R * (BK / 8), "tile vectors divide evenly");
    u32x4 v[NV];
    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int row0, int rows, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int vid = tid + NT * i;
            int r = vid >> 3, kv = vid & 7;
            if (row0 + r < rows)
                v[i] = *(const u32x4*)(base + (int64_t)(row0 + r) * ld + k0 + kv * 8);
            else
                v[i] = u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint16_t* s, int tid, bool) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int vid = tid + NT * i;
            int r = vid >> 3, kv = vid & 7;
            *(u32x4*)(s + r * LDK + kv * 8) = v[i];
        }
    }
    __device__ __forceinline__ void bias_reduce(float*, float*, int, int, int, int) {}
};

// Tile loader for an operand stored contiguous along the output dim:
// element (row, k) at base[k * ld + row].  A thread owns 8(k) x 8(row)
// blocks: it loads 8 row-vectors and writes 8 transposed k-vectors.
template <int R, int NT>
struct LoaderT {
    static constexpr int NB = R;  // (R/8) row chunks x (BK/8) k chunks
    static constexpr int PER = (NB + NT - 1) / NT;
    u32x4 v[PER][8];
    float bsum[PER][8];
    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int row0, int rows, int k0, int tid) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int blk = tid + NT * q;
            if (blk >= NB) break;
            int rc = blk % (R / 8), kc = blk / (R / 8);
            int row = row0 + rc * 8;
            bool ok = row < rows;  // rows % 8 == 0
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                v[q][kk] = ok ? *(const u32x4*)(base + (int64_t)(k0 + kc * 8 + kk) * ld + row) : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint16_t* s, int tid, bool sum_rows) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int blk = tid + NT * q;
            if (blk >= NB) break;
            int rc = blk % (R / 8), kc = blk / (R / 8);
            u32x4 w[8];
            transpose8x8(v[q], w);
#pragma unroll
            for (int c = 0; c < 8; ++c) *(u32x4*)(s + (rc * 8 + c) * LDK + kc * 8) = w[c];
            if (sum_rows) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    float t = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) t += bflo(w[c][e]) + bfhi(w[c][e]);
                    bsum[q][c] += t;
                }
            }
        }
    }
    // Sum the per-thread partial row sums over the 8 k chunks and add them to dbias.
    __device__ __forceinline__ void bias_reduce(float* red, float* dbias, int row0, int rows, int tid, int) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int blk = tid + NT * q;
            if (blk >= NB) break;
            int rc = blk % (R / 8), kc = blk / (R / 8);
#pragma unroll
            for (int c = 0; c < 8; ++c) red[kc * R + rc * 8 + c] = bsum[q][c];
        }
        __syncthreads();
        for (int r = tid; r < R; r += NT) {
            float t = 0.f;
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) t += red[kc * R + r];
            if (row0 + r < rows) unsafeAtomicAdd(dbias + row0 + r, t);
        }
    }
};

template <int BM, int BN, int WGM, int WGN, bool A_T, bool B_T, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_kernel(GemmParams p) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int STAGE = (BM + BN) * LDK;  // stage s: A tile at smem + s*STAGE, B tile after it
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // XCD-contiguous renumbering, then (split, tile); grouped tile order for L2 reuse
    const int ntiles = p.tiles_m * p.tiles_n;
    const int total = ntiles * p.splits;
    int lin = blockIdx.x;
    if ((total % NUM_XCD) == 0) lin = (lin % NUM_XCD) * (total / NUM_XCD) + lin / NUM_XCD;
    const int split = lin / ntiles;
    const int pid = lin % ntiles;
    const int in_group = GROUP_M * p.tiles_n;
    const int first_m = (pid / in_group) * GROUP_M;
    const int gsize = min(p.tiles_m - first_m, GROUP_M);
    const int tm = first_m + (pid % in_group) % gsize;
    const int tn = (pid % in_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;
    const int q = p.nk_total / p.splits, rr = p.nk_total % p.splits;
    const int it0 = split * q + min(split, rr);
    const int nk = q + (split < rr ? 1 : 0);
    const int kbeg = it0 * BK;
    const bool sum_rows = A_T && p.dbias != nullptr && tn == 0;

    typename std::conditional<A_T, LoaderT<BM, NT>, LoaderK<BM, NT>>::type la;
    typename std::conditional<B_T, LoaderT<BN, NT>, LoaderK<BN, NT>>::type lb;
    if constexpr (A_T) {
#pragma unroll
        for (int a = 0; a < LoaderT<BM, NT>::PER; ++a)
#pragma unroll
            for (int c = 0; c < 8; ++c) la.bsum[a][c] = 0.f;
    }

    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        la.load(p.A, p.lda, m0, p.M, kbeg, tid);
        lb.load(p.B, p.ldb, n0, p.N, kbeg, tid);
        la.store(smem, tid, sum_rows);
        lb.store(smem + BM * LDK, tid, false);
    }
    __syncthreads();

    const int frow = lane & 31;
    const int fk = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            la.load(p.A, p.lda, m0, p.M, kbeg + (kt + 1) * BK, tid);
            lb.load(p.B, p.ldb, n0, p.N, kbeg + (kt + 1) * BK, tid);
        }
        const uint16_t* a_s = smem + cur * STAGE + (wm * WTM + frow) * LDK + fk;
        const uint16_t* b_s = smem + cur * STAGE + BM * LDK + (wn * WTN + frow) * LDK + fk;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8*)(a_s + i * 32 * LDK + kk * 16);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[j] = *(const bf16x8*)(b_s + j * 32 * LDK + kk * 16);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < nk) {
            la.store(smem + (cur ^ 1) * STAGE, tid, sum_rows);
            lb.store(smem + (cur ^ 1) * STAGE + BM * LDK, tid, false);
        }
        __syncthreads();
    }

    if (sum_rows) la.bias_reduce((float*)smem, p.dbias, m0, p.M, tid, 0);

    // epilogue: lane holds column (lane & 31) of each 32x32 tile, rows acc_row(r, lane)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + j * 32 + (lane & 31);
            if (col >= p.N) continue;
            float bcol = 0.0f;
            if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU) {
                if (p.bias) bcol = p.bias[col];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WTM + i * 32 + acc_row(r, lane);
                if (row >= p.M) continue;
                float x = acc[i][j][r];
                if constexpr (EPI == EPI_BF16) {
                    x += bcol;
                    if (p.res) x += bf2f(p.res[(int64_t)row * p.ldr + col]);
                    p.out[(int64_t)row * p.ldo + col] = f2bf(x);
                } else if constexpr (EPI == EPI_GELU) {
                    const uint16_t pre = f2bf(x + bcol);
                    p.out[(int64_t)row * p.ldo + col] = pre;
                    p.out2[(int64_t)row * p.ldo + col] = f2bf(gelu_f(bf2f(pre)));
                } else if constexpr (EPI == EPI_DGELU) {
                    x *= gelu_grad_f(bf2f(p.res[(int64_t)row * p.ldr + col]));
                    p.out[(int64_t)row * p.ldo + col] = f2bf(x);
                } else if constexpr (EPI == EPI_F32_ACC) {
                    p.outf[(int64_t)row * p.ldf + col] += x;
                } else {
                    p.outf[split * p.split_stride + (int64_t)row * p.ldf + col] = x;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large NT tiles: 256x256 per workgroup, four 128x128 wave tiles.  Operands go
// global -> LDS with global_load_lds_dwordx4 (no register staging): each wave
// instruction fills 1 KB = 8 rows of 64 bf16.  Rows are unpadded (128 B) and
// the 16-byte vector kv of row r sits at slot kv ^ ((r >> 1) & 7), which
// makes the fragment reads of 16 consecutive rows hit 16 distinct bank
// groups.  The MFMA takes B as its first operand, so a lane's accumulator
// holds 4 consecutive output columns of one output row; the epilogue stages
// the bf16 tile in LDS (16-byte chunks XOR-swizzled by row) and writes it
// back in coalesced 16-byte row segments, applying bias / residual / GELU.
constexpr int BIG = 256;
constexpr int BIG_STAGE = 2 * BIG * BK;  // A and B tiles of one stage, bf16 elements

__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* dst_wave_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst_wave_base, 16, 0, 0);
}

__device__ __forceinline__ int big_slot(int row, int kv) { return row * BK + ((kv ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ const bf16x8& big_frag(const uint16_t* tile, int row, int kv) {
    return *(const bf16x8*)(tile + big_slot(row, kv));
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_nt_big_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BIG_STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    const int ntiles = p.tiles_m * p.tiles_n;
    int pid = blockIdx.x;
    if ((ntiles % NUM_XCD) == 0) pid = (pid % NUM_XCD) * (ntiles / NUM_XCD) + pid / NUM_XCD;
    const int in_group = GROUP_M * p.tiles_n;
    const int first_m = (pid / in_group) * GROUP_M;
    const int gsize = min(p.tiles_m - first_m, GROUP_M);
    const int m0 = (first_m + (pid % in_group) % gsize) * BIG;
    const int n0 = ((pid % in_group) / gsize) * BIG;
    const int nk = p.nk_total;

    // Lane source of this wave's chunk i (rows 64*wave + 8*i + lane/8): the row is
    // clamped into range (rows past M / N load valid memory whose products are
    // never stored) and the vector slot is un-swizzled.  Offsets are 32-bit
    // (the host checks M*lda and N*ldb < 2^31).
    const int lrow = lane >> 3, pv = lane & 7;
    const int kv_even = (pv ^ (lrow >> 1)) << 3;        // chunks i even: (row >> 1) & 7 == lrow >> 1
    const int kv_odd = (pv ^ ((lrow >> 1) + 4)) << 3;   // chunks i odd: 4 + lrow >> 1
    const int rowA = m0 + wave * 64 + lrow, rowB = n0 + wave * 64 + lrow;
    const int lda = (int)p.lda, ldb = (int)p.ldb;
    auto issue = [&](int stage, int k0) {
        uint16_t* sa = smem + stage * BIG_STAGE;
        uint16_t* sb = sa + BIG * BK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kv = (i & 1) ? kv_odd : kv_even;
            lds_dma16(p.A + (uint32_t)(min(rowA + 8 * i, p.M - 1) * lda + k0 + kv), sa + (wave * 8 + i) * 512);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kv = (i & 1) ? kv_odd : kv_even;
            lds_dma16(p.B + (uint32_t)(min(rowB + 8 * i, p.N - 1) * ldb + k0 + kv), sb + (wave * 8 + i) * 512);
        }
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int fr = lane & 31;
    // fragment rows are fixed per lane: precompute the LDS element offsets of the
    // 4 A and 4 B fragment rows (swizzle term included) for both K halves g
    const int ra = wm * 128 + fr, rb = wn * 128 + fr;
    bf16x8 af[2][4], bfr[2][4];
    auto load_frags = [&](const uint16_t* sa, const uint16_t* sb, int kk, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) af[buf][i] = big_frag(sa, ra + i * 32, 2 * kk + g);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[buf][j] = big_frag(sb, rb + j * 32, 2 * kk + g);
    };
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) issue(cur ^ 1, (kt + 1) * BK);
        const uint16_t* sa = smem + cur * BIG_STAGE;
        const uint16_t* sb = sa + BIG * BK;
        load_frags(sa, sb, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cb = kk & 1, nb = cb ^ 1;
            // next step's A fragments (4 reads), then half of this step's MFMAs
            if (kk + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) af[nb][i] = big_frag(sa, ra + i * 32, 2 * (kk + 1) + g);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(bfr[cb][j], af[cb][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
            // next step's B fragments, then the other half
            if (kk + 1 < BK / 16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) bfr[nb][j] = big_frag(sb, rb + j * 32, 2 * (kk + 1) + g);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 2; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(bfr[cb][j], af[cb][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // stage 1: acc (+bias) -> bf16 tile [256][256] in LDS.  acc[i][j][4*rg + e] is
    // C[m0 + wm*128 + i*32 + (lane&31)][n0 + wn*128 + j*32 + 8*rg + 4*g + e].
    uint16_t* so = smem;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + fr;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int col = wn * 128 + j * 32 + 8 * rg + 4 * g;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * rg + e];
                if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU) {
                    if (p.bias && n0 + col < p.N) {
                        const float4 b4 = *(const float4*)(p.bias + n0 + col);
                        v[0] += b4.x; v[1] += b4.y; v[2] += b4.z; v[3] += b4.w;
                    }
                }
                const int chunk = (col >> 3) ^ (row & 31);
                *(u32x2*)(so + row * BIG + chunk * 8 + (col & 7)) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
            }
    }
    __syncthreads();
    // stage 2: coalesced 16-byte row segments
#pragma unroll 4
    for (int it = 0; it < BIG * BIG / 8 / 256; ++it) {
        const int idx = it * 256 + tid;
        const int row = idx >> 5, chunk = idx & 31;
        const int grow = m0 + row, gcol = n0 + chunk * 8;
        if (grow >= p.M || gcol >= p.N) continue;
        u32x4 w = *(const u32x4*)(so + row * BIG + ((chunk ^ (row & 31)) << 3));
        const int64_t o = (int64_t)grow * p.ldo + gcol;
        if constexpr (EPI == EPI_BF16) {
            if (p.res) {
                const u32x4 r = *(const u32x4*)(p.res + (int64_t)grow * p.ldr + gcol);
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = pack_bf2(bflo(w[e]) + bflo(r[e]), bfhi(w[e]) + bfhi(r[e]));
            }
            *(u32x4*)(p.out + o) = w;
        } else if constexpr (EPI == EPI_GELU) {
            u32x4 gv;
#pragma unroll
            for (int e = 0; e < 4; ++e) gv[e] = pack_bf2(gelu_f(bflo(w[e])), gelu_f(bfhi(w[e])));
            *(u32x4*)(p.out + o) = w;
            *(u32x4*)(p.out2 + o) = gv;
        } else {  // EPI_DGELU
            const u32x4 pr = *(const u32x4*)(p.res + (int64_t)grow * p.ldr + gcol);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = pack_bf2(bflo(w[e]) * gelu_grad_f(bflo(pr[e])), bfhi(w[e]) * gelu_grad_f(bfhi(pr[e])));
            *(u32x4*)(p.out + o) = w;
        }
    }
}

// ---------------------------------------------------------------------------
// Large TN tiles (weight gradients): dW[n][k] (+)= sum_m dY[m][n] X[m][k] over
// one split's token range, 256x256 output tile, four 128x128 wave tiles.  Both
// operands are stored token-major, so each thread loads an 8 (tokens) x 8
// (features) block of each (8 row vectors), transposes it in registers and
// writes 8 token vectors into the swizzled LDS layout used by the NT kernel.
// Loads are issued one K step ahead into registers (two LDS stages).  The
// workgroups of output column tile 0 also sum the dY blocks they transpose
// (the bias gradient, added atomically).  Lane l of wave tile (wm, wn) holds
// output rows wm*128 + 32i + (l&31) and 4 consecutive columns per register
// group, written as float4.
template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_tn_big_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BIG_STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    const int ntiles = p.tiles_m * p.tiles_n;
    const int total = ntiles * p.splits;
    int lin = blockIdx.x;
    if ((total % NUM_XCD) == 0) lin = (lin % NUM_XCD) * (total / NUM_XCD) + lin / NUM_XCD;
    const int split = lin / ntiles;
    const int pid = lin % ntiles;
    const int in_group = GROUP_M * p.tiles_n;
    const int first_m = (pid / in_group) * GROUP_M;
    const int gsize = min(p.tiles_m - first_m, GROUP_M);
    const int tm = first_m + (pid % in_group) % gsize;
    const int tn = (pid % in_group) / gsize;
    const int m0 = tm * BIG, n0 = tn * BIG;
    const int q = p.nk_total / p.splits, rr = p.nk_total % p.splits;
    const int nk = q + (split < rr ? 1 : 0);
    const int kbeg = (split * q + min(split, rr)) * BK;
    const bool sum_rows = p.dbias != nullptr && tn == 0;

    // thread t owns feature chunk fc = t >> 3 (8 features) and token chunk tc = t & 7
    // (8 tokens) of each 256 x 64 operand tile
    const int fc = tid >> 3, tc = tid & 7;
    const int fa = min(m0 + fc * 8, p.M - 8), fb = min(n0 + fc * 8, p.N - 8);  // clamped (M, N % 8 == 0)
    u32x4 va[8], vb[8];
    float bs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto gload = [&](int k0) {
        const int tok = kbeg + k0 + tc * 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) va[r] = *(const u32x4*)(p.A + (int64_t)(tok + r) * p.lda + fa);
#pragma unroll
        for (int r = 0; r < 8; ++r) vb[r] = *(const u32x4*)(p.B + (int64_t)(tok + r) * p.ldb + fb);
    };
    auto lstore = [&](int stage) {
        uint16_t* sa = smem + stage * BIG_STAGE;
        uint16_t* sb = sa + BIG * BK;
        u32x4 w[8];
        transpose8x8(va, w);
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(sa + big_slot(fc * 8 + c, tc)) = w[c];
        if (sum_rows) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float t = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) t += bflo(w[c][e]) + bfhi(w[c][e]);
                bs[c] += t;
            }
        }
        transpose8x8(vb, w);
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(sb + big_slot(fc * 8 + c, tc)) = w[c];
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        gload(0);
        lstore(0);
        if (nk > 1) gload(BK);
    }
    __syncthreads();
    const int fr = lane & 31;
    const int ra = wm * 128 + fr, rb = wn * 128 + fr;
    bf16x8 af[2][4], bfr[2][4];
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const uint16_t* sa = smem + cur * BIG_STAGE;
        const uint16_t* sb = sa + BIG * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[0][i] = big_frag(sa, ra + i * 32, g);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[0][j] = big_frag(sb, rb + j * 32, g);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cb = kk & 1, nb = cb ^ 1;
            if (kk + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) af[nb][i] = big_frag(sa, ra + i * 32, 2 * (kk + 1) + g);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(bfr[cb][j], af[cb][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (kk + 1 < BK / 16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) bfr[nb][j] = big_frag(sb, rb + j * 32, 2 * (kk + 1) + g);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 2; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(bfr[cb][j], af[cb][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // every wave is done with the other stage since the previous barrier: fill it
        // with K step kt+1 (in registers) and start the loads of step kt+2
        if (kt + 1 < nk) {
            lstore(cur ^ 1);
            if (kt + 2 < nk) gload((kt + 2) * BK);
        }
        __syncthreads();
    }

    if (sum_rows) {
        // sum the 8 token chunks of each feature row, add to the bias gradient
        float* red = (float*)smem;
#pragma unroll
        for (int c = 0; c < 8; ++c) red[tc * BIG + fc * 8 + c] = bs[c];
        __syncthreads();
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) t += red[k * BIG + tid];
        if (m0 + tid < p.M) unsafeAtomicAdd(p.dbias + m0 + tid, t);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 128 + i * 32 + fr;
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int col = n0 + wn * 128 + j * 32 + 8 * rg + 4 * g;
                if (col >= p.N) continue;
                float4 v = make_float4(acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2],
                                       acc[i][j][4 * rg + 3]);
                if constexpr (EPI == EPI_F32_ACC) {
                    float4* o = (float4*)(p.outf + (int64_t)row * p.ldf + col);
                    float4 a = *o;
                    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
                    *o = a;
                } else {
                    *(float4*)(p.outf + split * p.split_stride + (int64_t)row * p.ldf + col) = v;
                }
            }
    }
}

// dW += sum over splits of the partials (float4 vectors).
__global__ void splitk_reduce_kernel(const float4* __restrict__ part, float4* __restrict__ dw, int64_t n4,
                                     int splits, int64_t stride4) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        float4 a = dw[i];
        for (int s = 0; s < splits; ++s) {
            float4 b = part[s * stride4 + i];
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        dw[i] = a;
    }
}

constexpr int gemm_class(bool a_t, int epi) {
    return !a_t ? (epi == EPI_GELU ? KC_GEMM_NT_GELU : (epi == EPI_DGELU ? KC_GEMM_NT_DGELU : KC_GEMM_NT))
                : (epi == EPI_F32_STORE ? KC_GEMM_TN_SPLIT : KC_GEMM_TN_ACC);
}

template <int BM, int BN, int WGM, int WGN, bool A_T, bool B_T, int EPI>
hipError_t run(GemmParams p, hipStream_t s) {
    p.tiles_m = (int)cdiv(p.M, BM);
    p.tiles_n = (int)cdiv(p.N, BN);
    dim3 grid(p.tiles_m * p.tiles_n * p.splits);
    const double work = 2.0 * p.M * p.N * (double)p.nk_total * BK;
    PROF_LAUNCH(gemm_class(A_T, EPI), work, s,
                hipLaunchKernelGGL((gemm_kernel<BM, BN, WGM, WGN, A_T, B_T, EPI>), grid, dim3(64 * WGM * WGN), 0,
                                   s, p));
    return hipGetLastError();
}

// Forward / input-gradient products: 256x256 tiles (four 128x128 wave tiles)
// when the problem has enough of them, else 128x128.
template <int EPI>
hipError_t run_nt(GemmParams p, hipStream_t s) {
    p.splits = 1;
    if ((int64_t)cdiv(p.M, BIG) * cdiv(p.N, BIG) >= NUM_CU / 2 && p.N % 8 == 0 && p.lda % 8 == 0 &&
        p.ldb % 8 == 0 && p.ldo % 8 == 0 && (p.res == nullptr || p.ldr % 8 == 0) &&
        (int64_t)p.M * p.lda < (1ll << 31) && (int64_t)p.N * p.ldb < (1ll << 31)) {
        p.tiles_m = (int)cdiv(p.M, BIG);
        p.tiles_n = (int)cdiv(p.N, BIG);
        const double work = 2.0 * p.M * p.N * (double)p.nk_total * BK;
        PROF_LAUNCH(gemm_class(false, EPI), work, s,
                    hipLaunchKernelGGL(gemm_nt_big_kernel<EPI>, dim3(p.tiles_m * p.tiles_n), dim3(256), 0, s, p));
        return hipGetLastError();
    }
    return run<128, 128, 2, 2, false, false, EPI>(p, s);
}

template <int EPI>
hipError_t run_tn_big(GemmParams p, hipStream_t s) {
    p.tiles_m = (int)cdiv(p.M, BIG);
    p.tiles_n = (int)cdiv(p.N, BIG);
    const double work = 2.0 * p.M * p.N * (double)p.nk_total * BK;
    PROF_LAUNCH(gemm_class(true, EPI), work, s,
                hipLaunchKernelGGL(gemm_tn_big_kernel<EPI>, dim3(p.tiles_m * p.tiles_n * p.splits), dim3(256), 0,
                                   s, p));
    return hipGetLastError();
}

// Weight-gradient split: a multiple of the tile count close to a whole number of
// passes over the 256 CUs, each split keeping >= 4 K-steps.
struct TnPlan {
    int splits;
    bool big;  // 256x256 tiles
};
TnPlan tn_plan(int M, int N, int K) {
    const int nk = M / BK;
    const bool big = (int64_t)cdiv(N, 256) * cdiv(K, 256) >= 8;
    const int64_t tiles = big ? cdiv(N, 256) * cdiv(K, 256) : cdiv(N, 128) * cdiv(K, 128);
    if (tiles >= NUM_CU) return {1, big};
    int best = 1;
    double best_eff = 0.0;
    for (int s = 1; s <= 64 && nk / s >= 4; ++s) {
        const int64_t wg = tiles * s;
        const double waves = (double)wg / NUM_CU;
        const double eff = waves / std::ceil(waves);
        if (eff > best_eff + 0.02) {
            best_eff = eff;
            best = s;
        }
    }
    return {best, big};
}

}  // namespace

hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                          const float* bias, const uint16_t* res, int64_t ldr, uint16_t* out, int64_t ldo,
                          hipStream_t s) {
    GemmParams p{};
    p.A = A; p.B = B; p.lda = lda; p.ldb = ldb; p.M = M; p.N = N; p.nk_total = K / BK;
    p.bias = bias; p.res = res; p.ldr = ldr; p.out = out; p.ldo = ldo;
    return run_nt<EPI_BF16>(p, s);
}

hipError_t launch_gemm_nt_gelu(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                               const float* bias, uint16_t* pre, uint16_t* g, int64_t ldo, hipStream_t s) {
    GemmParams p{};
    p.A = A; p.B = B; p.lda = lda; p.ldb = ldb; p.M = M; p.N = N; p.nk_total = K / BK;
    p.bias = bias; p.out = pre; p.out2 = g; p.ldo = ldo;
    return run_nt<EPI_GELU>(p, s);
}

hipError_t launch_gemm_nt_dgelu(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                                const uint16_t* pre, uint16_t* out, int64_t ldo, hipStream_t s) {
    GemmParams p{};
    p.A = A; p.B = B; p.lda = lda; p.ldb = ldb; p.M = M; p.N = N; p.nk_total = K / BK;
    p.res = pre; p.ldr = ldo; p.out = out; p.ldo = ldo;
    return run_nt<EPI_DGELU>(p, s);
}

int64_t gemm_tn_partial_elems(int M, int N, int K) {
    TnPlan t = tn_plan(M, N, K);
    return t.splits > 1 ? (int64_t)t.splits * N * K : 0;
}

hipError_t launch_gemm_tn_acc(const uint16_t* dY, int64_t ldy, const uint16_t* X, int64_t ldx, int M, int N, int K,
                              float* dW, float* dbias, float* partial, int64_t partial_elems, hipStream_t s) {
    // output rows = N (features of dY), output cols = K (features of X), reduction = M tokens
    TnPlan t = tn_plan(M, N, K);
    if (t.splits > 1 && (partial == nullptr || partial_elems < (int64_t)t.splits * N * K)) t.splits = 1;
    GemmParams p{};
    p.A = dY; p.B = X; p.lda = ldy; p.ldb = ldx; p.M = N; p.N = K; p.nk_total = M / BK; p.splits = t.splits;
    p.dbias = dbias;
    if (t.splits == 1) {
        p.outf = dW; p.ldf = K;
        return t.big ? run_tn_big<EPI_F32_ACC>(p, s) : run<128, 128, 2, 2, true, true, EPI_F32_ACC>(p, s);
    }
    p.outf = partial; p.ldf = K; p.split_stride = (int64_t)N * K;
    hipError_t e = t.big ? run_tn_big<EPI_F32_STORE>(p, s) : run<128, 128, 2, 2, true, true, EPI_F32_STORE>(p, s);
    if (e != hipSuccess) return e;
    const int64_t n4 = (int64_t)N * K / 4;
    const int blocks = (int)std::min<int64_t>(cdiv(n4, 256), 4096);
    PROF_LAUNCH(KC_SPLITK_REDUCE, 4.0 * n4 * 4 * (t.splits + 2), s,
                hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, (const float4*)partial,
                                   (float4*)dW, n4, t.splits, n4));
    return hipGetLastError();
}
