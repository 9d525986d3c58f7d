// bf16 GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// The linear layers of the GPT-2 block and the tied lm_head (PDS model text
// around Fig. 1) run three products:
//   forward / input gradient ("NT"): C[M,N] = A[M,K] . B[N,K]^T, both operands
//     contiguous along the reduction.  The input-gradient GEMMs use the
//     transposed bf16 weight copy so they are NT products too;
//   weight gradient ("TN"): dW[N,K] += sum_m dY[m,n] X[m,k], reduction over
//     tokens, operands contiguous along the output dims.  Their MFMA fragments
//     are read transposed out of LDS (ds_read_b64_tr_b16).  The bias gradient
//     (column sums of dY) is folded into the same pass: the workgroups of the
//     first output column tile sum the dY fragments they read anyway.
// Large problems run 256x256 tiles (gemm_nt_w8_kernel, gemm_tn_w8_kernel):
// operands go global -> LDS without register staging, several stages in
// flight.  Small ones run the generic BM x BN kernel (gemm_kernel: register
// prefetch, LDS double buffer, rows padded to 72 bf16).  Workgroups are
// renumbered so each of the 8 XCDs (own L2 each) walks a contiguous run of the
// grouped tile order.  Weight-gradient GEMMs split the token reduction (uneven
// splits allowed) to fill the 256 CUs; the fp32 partials are summed into dW by
// a second kernel.
#include <algorithm>
#include "common.h"
#include <type_traits>
#include "kernels.h"
#include "prof.h"

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int GROUP_M = 8;
// weight-gradient tiles: a group of 4 output-row tiles per X column block (measured against 2, 8, 16)
constexpr int TN_GROUP_M = 4;
constexpr int NUM_XCD = 8;
constexpr int NUM_CU = 256;

// EPI_BF16R: bias + residual (large-tile kernel only; the generic kernel handles p.res under EPI_BF16)
enum Epi { EPI_BF16 = 0, EPI_GELU = 1, EPI_DGELU = 2, EPI_F32_ACC = 3, EPI_F32_STORE = 4, EPI_BF16R = 5 };

struct GemmParams {
    const uint16_t* A;
    const uint16_t* B;
    int64_t lda, ldb;
    int M, N;          // output rows / cols
    int nk_total;      // reduction length / BK
    int splits;
    int tiles_m, tiles_n;
    int band;          // tile order: row tiles per band, 0 = round-robin bands of GROUP_M (see nt_tile)
    const float* bias;
    const uint16_t* res;   // residual (EPI_BF16 / EPI_BF16R) or GELU'(pre-activation) (EPI_DGELU)
    int64_t ldr;
    uint16_t* out;
    uint16_t* out2;
    int64_t ldo;
    float* outf;
    int64_t ldf;
    int64_t split_stride;
    float* dbias;      // TN: bias gradient (column sums of A's source), may be null
};

// Workgroup ids go round-robin over the XCDs.  Renumbered so that each XCD holds
// one contiguous run of tiles (XCD x takes total/8 ids, one more when x < total % 8),
// tiles that share operand slices meet in that XCD's L2 at any tile count.
__device__ __forceinline__ int xcd_contiguous(int lin, int total) {
    const int q = total / NUM_XCD, r = total % NUM_XCD, x = lin % NUM_XCD;
    return x * q + min(x, r) + lin / NUM_XCD;
}

// Output tile of work-group `lin` among tiles_m x tiles_n.  Work-groups reach
// the 8 XCDs round-robin by linear index.  With band > 0 each XCD is given one
// contiguous share of the tile sequence (the first ntiles % 8 XCDs one tile
// more), and the sequence walks bands of `band` row tiles, row tile fastest:
// with band = ceil(tiles_m / 8) each XCD keeps its own rows of A and streams
// B about once (wide outputs such as the vocabulary projection).  With
// band = 0 the sequence is dealt round-robin (split into 8 contiguous shares
// when ntiles is a multiple of 8) over bands of GROUP_M row tiles; for outputs
// a few tiles wide that keeps every column tile of a row tile on one XCD.
__device__ __forceinline__ void nt_tile(int lin, int tiles_m, int tiles_n, int band, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    int pid;
    if (band > 0) {
        pid = xcd_contiguous(lin, ntiles);
    } else {
        band = GROUP_M;
        pid = (ntiles % NUM_XCD) == 0 ? (lin % NUM_XCD) * (ntiles / NUM_XCD) + lin / NUM_XCD : lin;
    }
    const int in_group = band * tiles_n;
    const int first_m = (pid / in_group) * band;
    const int gsize = min(tiles_m - first_m, band);
    tm = first_m + (pid % in_group) % gsize;
    tn = (pid % in_group) / gsize;
}

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
                    float g, gp;
                    gelu_and_grad_f(bf2f(f2bf(x + bcol)), g, gp);
                    p.out[(int64_t)row * p.ldo + col] = f2bf(gp);
                    p.out2[(int64_t)row * p.ldo + col] = f2bf(g);
                } else if constexpr (EPI == EPI_DGELU) {
                    x *= bf2f(p.res[(int64_t)row * p.ldr + col]);
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
// 256x256 tiles (one per workgroup of four waves) load their operands global ->
// LDS with global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS at
// M0 + 16 * lane, so the swizzle of a tile is chosen by which global vector each
// lane fetches.
constexpr int BIG = 256;

__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* dst_wave_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst_wave_base, 16, 0, 0);
}

// ---------------------------------------------------------------------------
// Shared pieces of the pipelined 256x256 kernels.  Stage depth and count are
// fixed: NT runs 2 stages of 64 reduction columns, TN 4 stages of 32 tokens.
constexpr int NT_STAGES = 2;
constexpr int NT_KD = 64;
constexpr int TN_STAGES = 4;
constexpr int TN_TD = 32;

// Read one accumulator element out of its AGPR where it is needed, so the
// epilogue never asks for all 256 accumulators in VGPRs at once (which makes
// the register allocator spill them around the main loop).
__device__ __forceinline__ float acc_read(float x) {
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
    return r;
}

// s_waitcnt immediate waiting for vmcnt <= n (expcnt and lgkmcnt left alone):
// vmcnt[3:0] | expcnt[6:4] = 7 | lgkmcnt[11:8] = 15 | vmcnt[5:4] at [15:14].
constexpr int vm_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Wait until at most n stage groups of G loads per wave are still in flight.
template <int G>
__device__ __forceinline__ void wait_stage_groups(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(vm_imm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(vm_imm(G)); break;
        case 2: __builtin_amdgcn_s_waitcnt(vm_imm(2 * G)); break;
        case 3: __builtin_amdgcn_s_waitcnt(vm_imm(3 * G)); break;
        default: __builtin_amdgcn_s_waitcnt(vm_imm(4 * G)); break;
    }
}

// ---------------------------------------------------------------------------
// NT tiles with eight waves: 256x256 per workgroup of 512 threads, wave grid
// 2 (rows) x 4 (columns) of 128x64 wave tiles (128 accumulators per lane, two
// waves per SIMD).  Each wave sustains only ~10-12 GB/s of loads into LDS, so
// eight issuing waves are needed to feed 256x256 tiles; the second wave on each
// SIMD also hides the other's barrier and LDS waits.  A stage holds KD
// reduction columns (rows of 2*KD bytes; 128-byte rows make every L2 request
// a full line), NS stages in LDS.  The 16-byte vector c of a row r sits at
// slot c ^ swz(r) so the fragment reads of 16 consecutive rows hit distinct
// bank groups.  At the end of each stage every wave waits for its own loads of
// the next stage, one barrier makes all of them visible, and the buffer just
// read takes the stage after next; the epilogue stages the bf16 tile through
// LDS and stores 16-byte row segments.
template <int KD>
struct NtStage {
    static constexpr int CPR = KD / 8;                // 16-byte vectors per row
    static constexpr int RPI = 64 / CPR;              // rows per 1 KB load instruction
    static constexpr int ELEMS = 2 * BIG * KD;        // A and B tiles, bf16 elements
    static constexpr int KS = KD / 16;                // MFMA k-steps per stage
    __device__ static int swz(int r) { return CPR == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
};

template <int EPI, int NS, int KD>
__global__ __launch_bounds__(512, 1) void gemm_nt_w8_kernel(GemmParams p) {
    typedef NtStage<KD> St;
    static_assert(NS * St::ELEMS >= BIG * BIG, "the epilogue reuses 128 KB of stage buffers");
    static_assert(NS * St::ELEMS * 2 <= 160 * 1024, "LDS");
    constexpr int IPO = BIG / St::RPI / 8;            // load instructions per wave per operand
    __shared__ __attribute__((aligned(16))) uint16_t smem[NS * St::ELEMS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;

    int tm, tn;
    nt_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.band, tm, tn);
    const int m0 = tm * BIG, n0 = tn * BIG;
    const int nk = p.nk_total * (BK / KD);

    // Lane q of load instruction i covers row (wave*IPO + i)*RPI + q/CPR at
    // physical slot q%CPR, i.e. logical vector (q%CPR) ^ swz(row).  Rows past
    // M / N are clamped (their products are never stored).  Offsets are 32-bit
    // elements (the host checks M*lda and N*ldb < 2^31).
    uint32_t offA[IPO], offB[IPO];
#pragma unroll
    for (int i = 0; i < IPO; ++i) {
        const int row = (wave * IPO + i) * St::RPI + lane / St::CPR;
        const int lv = ((lane % St::CPR) ^ St::swz(row)) << 3;
        offA[i] = (uint32_t)min(m0 + row, p.M - 1) * (uint32_t)p.lda + lv;
        offB[i] = (uint32_t)min(n0 + row, p.N - 1) * (uint32_t)p.ldb + lv;
    }
    auto issue = [&](int t) {
        uint16_t* sa = smem + (t % NS) * St::ELEMS;
        uint16_t* sb = sa + BIG * KD;
        const uint32_t k0 = (uint32_t)t * KD;
#pragma unroll
        for (int i = 0; i < IPO; ++i) lds_dma16(p.A + (offA[i] + k0), sa + (wave * IPO + i) * 512);
#pragma unroll
        for (int i = 0; i < IPO; ++i) lds_dma16(p.B + (offB[i] + k0), sb + (wave * IPO + i) * 512);
    };

    // prologue: all NS stage buffers in flight (nk >= 1: the host requires K >= 64)
#pragma unroll
    for (int t = 0; t < NS; ++t)
        if (t < nk) issue(t);
    __builtin_amdgcn_sched_barrier(0);
    // bias of this lane's 8 column groups (zero past N; N % 8 == 0 keeps a group whole)
    float4 b4[2][4];
    if ((EPI == EPI_BF16 || EPI == EPI_BF16R || EPI == EPI_GELU) && p.bias != nullptr) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
                b4[j][rg] = *(const float4*)(p.bias + min(n0 + wn * 64 + j * 32 + 8 * rg + 4 * g, p.N - 4));
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const bool in = n0 + wn * 64 + j * 32 + 8 * rg + 4 * g < p.N;
                b4[j][rg].x = in ? b4[j][rg].x : 0.f;
                b4[j][rg].y = in ? b4[j][rg].y : 0.f;
                b4[j][rg].z = in ? b4[j][rg].z : 0.f;
                b4[j][rg].w = in ? b4[j][rg].w : 0.f;
            }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) b4[j][rg] = float4{0.f, 0.f, 0.f, 0.f};
    }

    // acc[i][j][4*rg + e] is C[m0 + wm*128 + i*32 + (lane&31)][n0 + wn*64 + j*32 + 8*rg + 4*g + e].
    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                acc[i][j][4 * rg + 0] = b4[j][rg].x;
                acc[i][j][4 * rg + 1] = b4[j][rg].y;
                acc[i][j][4 * rg + 2] = b4[j][rg].z;
                acc[i][j][4 * rg + 3] = b4[j][rg].w;
            }
    wait_stage_groups<2 * IPO>(min(NS, nk) - 1);
    __syncthreads();

    // fragment rows are fixed per lane (32-aligned + lane&31); k-step kk reads vector 2*kk + g
    const int fr = lane & 31;
    const int sw = St::swz(fr);
    const int ra = (wm * 128 + fr) * KD, rb = BIG * KD + (wn * 64 + fr) * KD;
    auto cvec = [&](int kk) { return ((2 * kk + g) ^ sw) << 3; };
    bf16x8 af[2][4], bfr[2][2];
    auto read = [&](const uint16_t* st, int kk, int b) {
        const int cv = cvec(kk);
#pragma unroll
        for (int i = 0; i < 4; ++i) af[b][i] = *(const bf16x8*)(st + ra + i * 32 * KD + cv);
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[b][j] = *(const bf16x8*)(st + rb + j * 32 * KD + cv);
    };
    auto mma = [&](int b, int i0) {
#pragma unroll
        for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(bfr[b][j], af[b][i], acc[i][j]);
    };
    // second epilogue input for the whole tile: thread tid covers 16-byte chunk
    // (tid & 31) of rows 16*it + tid/32.  The first PIN_EARLY chunks are read at the
    // top of the last stage, so their latency hides behind its products.
    constexpr int EIT = BIG * BIG / 8 / 512;
    constexpr bool HAS_IN = EPI == EPI_DGELU || EPI == EPI_BF16R;
    constexpr int PIN_EARLY = HAS_IN ? 8 : 0;
    u32x4 pin[HAS_IN ? EIT : 1];
    auto load_pin = [&](int it) {
        const int grow = m0 + it * 16 + (tid >> 5), gcol = n0 + (tid & 31) * 8;
        pin[it] = (grow < p.M && gcol < p.N) ? *(const u32x4*)(p.res + (int64_t)grow * p.ldr + gcol) : u32x4{0u, 0u, 0u, 0u};
    };
    read(smem, 0, 0);
    int s = 0;
    do {
        const uint16_t* st = smem + (s % NS) * St::ELEMS;
        if constexpr (HAS_IN) {
            if (s == nk - 1) {
#pragma unroll
                for (int it = 0; it < PIN_EARLY; ++it) load_pin(it);
            }
        }
#pragma unroll
        for (int kk = 0; kk < St::KS; ++kk) {
            const int b = kk & 1;
            if (kk + 1 < St::KS) {
                mma(b, 0);
                read(st, kk + 1, b ^ 1);
                mma(b, 2);
                // the next k-step's 6 reads spread over all 8 products
#pragma unroll
                for (int q = 0; q < 6; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_barrier(0);
                continue;
            }
            mma(b, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < nk) {
                // stage s+1 has landed once only the stages issued after it remain in flight
                wait_stage_groups<2 * IPO>(min(s + NS - 1, nk - 1) - (s + 1));
                __syncthreads();
                // every wave has read all of stage s (its last fragments are in
                // registers): its buffer takes stage s+NS
                if (s + NS < nk) issue(s + NS);
                read(smem + ((s + 1) % NS) * St::ELEMS, 0, b ^ 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            mma(b, 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    } while (++s < nk);
    __syncthreads();
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // the rest of the second epilogue input, read now so its latency overlaps the staging
    if constexpr (HAS_IN) {
#pragma unroll
        for (int it = PIN_EARLY; it < EIT; ++it) load_pin(it);
    }

    // stage 1: acc -> bf16 tile [256][256] in LDS (16-byte chunks XOR-swizzled by row)
    uint16_t* so = smem;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + fr;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int col = wn * 64 + j * 32 + 8 * rg + 4 * g;
                const int chunk = (col >> 3) ^ (row & 31);
                *(u32x2*)(so + row * BIG + chunk * 8 + (col & 7)) =
                    u32x2{pack_bf2(acc_read(acc[i][j][4 * rg]), acc_read(acc[i][j][4 * rg + 1])),
                          pack_bf2(acc_read(acc[i][j][4 * rg + 2]), acc_read(acc[i][j][4 * rg + 3]))};
            }
    }
    __syncthreads();
    // stage 2: coalesced 16-byte row segments
    auto out_chunk = [&](int it) {
        const int row = it * 16 + (tid >> 5), chunk = tid & 31;
        const int grow = m0 + row, gcol = n0 + chunk * 8;
        if (grow >= p.M || gcol >= p.N) return;
        u32x4 w = *(const u32x4*)(so + row * BIG + ((chunk ^ (row & 31)) << 3));
        const int64_t o = (int64_t)grow * p.ldo + gcol;
        if constexpr (EPI == EPI_BF16) {
            *(u32x4*)(p.out + o) = w;
        } else if constexpr (EPI == EPI_BF16R) {
            const u32x4 r = pin[it];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf2(bflo(w[e]) + bflo(r[e]), bfhi(w[e]) + bfhi(r[e]));
            *(u32x4*)(p.out + o) = w;
        } else if constexpr (EPI == EPI_GELU) {
            // w holds the bf16 pre-activation: GELU goes to out2, GELU' to out
            u32x4 gv, gd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float g0, d0, g1, d1;
                gelu_and_grad_f(bflo(w[e]), g0, d0);
                gelu_and_grad_f(bfhi(w[e]), g1, d1);
                gv[e] = pack_bf2(g0, g1);
                gd[e] = pack_bf2(d0, d1);
            }
            *(u32x4*)(p.out + o) = gd;
            *(u32x4*)(p.out2 + o) = gv;
        } else {  // EPI_DGELU: times the stored GELU'
            const u32x4 pr = pin[it];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = pack_bf2(bflo(w[e]) * bflo(pr[e]), bfhi(w[e]) * bfhi(pr[e]));
            *(u32x4*)(p.out + o) = w;
        }
    };
    if constexpr (HAS_IN) {
#pragma unroll
        for (int it = 0; it < EIT; ++it) out_chunk(it);
    } else {
#pragma unroll 4
        for (int it = 0; it < EIT; ++it) out_chunk(it);
    }
}

// ---------------------------------------------------------------------------
// Pipelined TN tiles (weight gradients): dW[r][c] (+)= sum_t dY[t][r] X[t][c]
// over one split's token range, 256x256 output tile per workgroup of eight
// waves (wave grid 2 x 4 of 128x64 wave tiles, as for NT).  Both operands are
// token-major, so a stage holds TD tokens x 256 features of each, loaded
// straight into LDS (global_load_lds_dwordx4: 1 KB = 2 token rows of 512 B
// per wave instruction) with the 16-byte vector v of row t at
// slot v ^ ((t & 7) << 2).  The MFMA fragments are the transposes of those
// tiles, read with ds_read_b64_tr_b16 (8 consecutive tokens of one feature
// per lane); the XOR spreads the 8 token rows one read touches over the banks.
// Pipeline, waits and barrier placement are those of the NT kernel (the loads
// are issued through inline asm, see lds_dma16_asm).  The
// workgroups of output column tile 0 also sum the dY fragments they read (the
// bias gradient).  The fp32 epilogue goes through a per-wave LDS buffer so
// each row segment is written (or read-modified-written) in 512-byte runs.

// LDS element offset of (token t, feature f) within a token-major stage tile.
__device__ __forceinline__ int tn_off(int t, int f) { return t * BIG + (((f >> 3) ^ ((t & 7) << 2)) << 3) + (f & 7); }

typedef short tn_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 tn_frag(const uint16_t* p) {
    // two transposed 4-element reads 8 token rows apart: tokens 16ks + 4g + 0..3, then + 8
    const tn_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tn_v4s*)p);
    const tn_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tn_v4s*)(p + 8 * BIG));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// lds_dma16 written as inline asm.  With the builtin, the compiler treats every
// in-flight load-to-LDS as possibly aliasing a ds_read_b64_tr_b16 (which carries
// no memory operand) and drains all outstanding loads before each one, which
// leaves a single stage in flight.  Completion of these loads is tracked by the
// explicit vmcnt waits and barriers around the stage buffers instead.
__device__ __forceinline__ void lds_dma16_asm(const uint16_t* src, uint16_t* dst_wave_base) {
    const uint32_t lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)dst_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}

// One weight-gradient product of a grouped launch.
constexpr int TN_MAX_JOBS = 48;
struct TnJob {
    const uint16_t* A;  // dY [tokens][M] (row stride lda)
    const uint16_t* B;  // X  [tokens][N] (row stride ldb)
    int lda, ldb, M, N, tiles_m, tiles_n;
    float* out;         // dW [M][N] (EPI_F32_ACC) or split partials, split s at out + s * M * N
    float* dbias;       // += column sums of dY (may be null)
};
struct TnGroup {
    TnJob job[TN_MAX_JOBS];
    int tile_start[TN_MAX_JOBS + 1];  // prefix sums of the jobs' tile counts
    int njobs, splits, nk_total;      // nk_total = tokens / 64
    // split launches (EPI_F32_STORE): split s of job j leaves its bias column sums at
    // bpart + splits * (M_0 + ... + M_{j-1}) + s * M_j, added in split order by the reduce
    float* bpart;
};

template <int EPI, int NS, int TD>
__global__ __launch_bounds__(512, 1) void gemm_tn_w8_kernel(TnGroup G) {
    // a stage holds TD tokens of both operands; each wave issues IPO 1 KB loads per operand
    constexpr int SE = 2 * TD * BIG, IPO = TD / 16, KS = TD / 16;
    static_assert(NS >= 2 && NS * SE * 2 <= 160 * 1024 && NS * SE >= 8 * 32 * 64 * 2, "stage count");
    __shared__ __attribute__((aligned(16))) uint16_t smem[NS * SE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;

    const int ntiles = G.tile_start[G.njobs];
    const int total = ntiles * G.splits;
    const int lin = xcd_contiguous(blockIdx.x, total);
    const int split = lin / ntiles;
    int pid = lin % ntiles, jb = 0;
    while (jb + 1 < G.njobs && pid >= G.tile_start[jb + 1]) ++jb;
    pid -= G.tile_start[jb];
    const TnJob p = G.job[jb];
    const int in_group = TN_GROUP_M * p.tiles_n;
    const int first_m = (pid / in_group) * TN_GROUP_M;
    const int gsize = min(p.tiles_m - first_m, TN_GROUP_M);
    const int tm = first_m + (pid % in_group) % gsize;
    const int tn = (pid % in_group) / gsize;
    const int m0 = tm * BIG, n0 = tn * BIG;  // dY feature (output row) and X feature (output column) origins
    const int steps = G.nk_total * (BK / TD);
    const int q = steps / G.splits, rr = steps % G.splits;
    const int nk = q + (split < rr ? 1 : 0);                 // >= 1: the host keeps splits <= steps
    const int tok0 = (split * q + min(split, rr)) * TD;
    // bias column sums: in the tiles of the first X column block, the four waves of a
    // wave row read the same dY fragments; wave wn sums fragment group i = wn
    const bool sum_rows = p.dbias != nullptr && tn == 0;
    const int bw = __builtin_amdgcn_readfirstlane(wn);

    // Load instruction i of this wave covers token rows 2*(wave*IPO + i) + (lane>>5)
    // of the stage, physical vector lane&31, i.e. logical vector (lane&31) ^ ((row&7)<<2).
    // Features past M / N are clamped (their products are never stored).
    uint32_t offA[IPO], offB[IPO];
#pragma unroll
    for (int i = 0; i < IPO; ++i) {
        const int row = 2 * (wave * IPO + i) + g;
        const int lv = (lane & 31) ^ ((row & 7) << 2);
        offA[i] = (uint32_t)(tok0 + row) * (uint32_t)p.lda + (uint32_t)min(m0 + lv * 8, p.M - 8);
        offB[i] = (uint32_t)(tok0 + row) * (uint32_t)p.ldb + (uint32_t)min(n0 + lv * 8, p.N - 8);
    }
    const uint32_t stepA = (uint32_t)TD * (uint32_t)p.lda, stepB = (uint32_t)TD * (uint32_t)p.ldb;
    // Every stage boundary issues one group of loads, so the number in flight is the
    // same at every wait (one immediate s_waitcnt, no run-time switch): stage t goes
    // to buffer t % NS, and past the last stage the last stage's data is loaded
    // again into the buffer just released, which is never read.
    auto issue = [&](int t) {
        uint16_t* sa = smem + (t % NS) * SE;
        uint16_t* sb = sa + TD * BIG;
        const uint32_t ts = (uint32_t)min(t, nk - 1);
#pragma unroll
        for (int i = 0; i < IPO; ++i)
            lds_dma16_asm(p.A + (offA[i] + ts * stepA), sa + 2 * (wave * IPO + i) * BIG);
#pragma unroll
        for (int i = 0; i < IPO; ++i)
            lds_dma16_asm(p.B + (offB[i] + ts * stepB), sb + 2 * (wave * IPO + i) * BIG);
    };

#pragma unroll
    for (int t = 0; t < NS; ++t) issue(t);
    __builtin_amdgcn_sched_barrier(0);

    // acc[i][j][4*rg + e] is dW[m0 + wm*128 + i*32 + (lane&31)][n0 + wn*64 + j*32 + 8*rg + 4*g + e]
    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    float bsum = 0.f;
    __builtin_amdgcn_s_waitcnt(vm_imm((NS - 1) * 2 * IPO));  // stage 0 has landed
    __syncthreads();

    // per-lane fragment addresses within a stage tile (token row 4g + (lane&15)/4,
    // features col0 + 16*((lane>>4)&1) + 4*(lane&3), col0 = 32-column subtile)
    int fa[4], fb[2];
    {
        const int t = 4 * g + ((lane & 15) >> 2);
        const int f = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = tn_off(t, wm * 128 + i * 32 + f);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = TD * BIG + tn_off(t, wn * 64 + j * 32 + f);
    }
    bf16x8 dyf[2][4], xf[2][2];
    auto read_frags = [&](const uint16_t* st, int ks, int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dyf[b][i] = tn_frag(st + fa[i] + ks * 16 * BIG);
#pragma unroll
        for (int j = 0; j < 2; ++j) xf[b][j] = tn_frag(st + fb[j] + ks * 16 * BIG);
    };
    auto add_bias = [&](int b, auto fi) {
        const u32x4 w = __builtin_bit_cast(u32x4, dyf[b][decltype(fi)::value]);
#pragma unroll
        for (int e = 0; e < 4; ++e) bsum += bflo(w[e]) + bfhi(w[e]);
    };
    auto mma = [&](int b, int i0) {
#pragma unroll
        for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(xf[b][j], dyf[b][i], acc[i][j]);
    };
    // two copies of the main loop: tiles without bias sums carry no bias code at all
    auto main_loop = [&](auto bias_frag) {
        read_frags(smem, 0, 0);
        int s = 0;
        do {
            const uint16_t* st = smem + (s % NS) * SE;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int b = kk & 1;
                mma(b, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (kk + 1 < KS) {
                    read_frags(st, kk + 1, b ^ 1);
                    mma(b, 2);
                    // 12 transposed reads spread over the 4 products
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (decltype(bias_frag)::value >= 0) add_bias(b, bias_frag);
                    __builtin_amdgcn_sched_barrier(0);
                    continue;
                } else if (s + 1 < nk) {
                    // stage s+1 has landed once only the NS-2 groups issued after it remain
                    __builtin_amdgcn_s_waitcnt(vm_imm((NS - 2) * 2 * IPO));
                    __syncthreads();
                    // all of stage s is in registers: its buffer takes stage s+NS
                    issue(s + NS);
                    read_frags(smem + ((s + 1) % NS) * SE, 0, b ^ 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                mma(b, 2);
                if constexpr (decltype(bias_frag)::value >= 0) add_bias(b, bias_frag);
                __builtin_amdgcn_sched_barrier(0);
            }
        } while (++s < nk);
    };
    if (!sum_rows)
        main_loop(std::integral_constant<int, -1>{});
    else if (bw == 0)
        main_loop(std::integral_constant<int, 0>{});
    else if (bw == 1)
        main_loop(std::integral_constant<int, 1>{});
    else if (bw == 2)
        main_loop(std::integral_constant<int, 2>{});
    else
        main_loop(std::integral_constant<int, 3>{});
    __builtin_amdgcn_s_waitcnt(vm_imm(0));  // the loads past the last stage have landed before the LDS is reused
    __syncthreads();
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    if (sum_rows) {
        // the two lane halves hold different tokens of the same feature rows
        {
            const float t = bsum + __shfl_xor(bsum, 32, WAVE);
            const int row = m0 + wm * 128 + bw * 32 + (lane & 31);
            if constexpr (EPI == EPI_F32_STORE) {
                // several splits per row: each leaves its sum for the ordered reduce
                if (g == 0 && row < p.M) {
                    int64_t off = 0;
                    for (int j = 0; j < jb; ++j) off += G.job[j].M;
                    G.bpart[off * G.splits + (int64_t)split * p.M + row] = t;
                }
            } else {
                if (g == 0 && row < p.M) unsafeAtomicAdd(p.dbias + row, t);  // one writer per row
            }
        }
    }

    // Epilogue through a per-wave 32 x 64 fp32 buffer (8 KB), one 32-row group i
    // at a time: 16-byte vector v of buffer row r sits at slot v ^ (r & 15).
    float* buf = (float*)smem + wave * (32 * 64);
    const int fr = lane & 31;
    float* outp = EPI == EPI_F32_ACC ? p.out : p.out + (int64_t)split * p.M * p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int v = 8 * j + 2 * rg + g;  // 16-byte vector index within the 64-column row
                *(float4*)(buf + fr * 64 + ((v ^ (fr & 15)) << 2)) =
                    make_float4(acc_read(acc[i][j][4 * rg]), acc_read(acc[i][j][4 * rg + 1]),
                                acc_read(acc[i][j][4 * rg + 2]), acc_read(acc[i][j][4 * rg + 3]));
            }
        // read back row-contiguous: lane covers vector lane&15 of rows 4*it + lane/16
#pragma unroll 4
        for (int it = 0; it < 8; ++it) {
            const int r = 4 * it + (lane >> 4), v = lane & 15;
            const float4 a = *(const float4*)(buf + r * 64 + ((v ^ (r & 15)) << 2));
            const int row = m0 + wm * 128 + i * 32 + r, col = n0 + wn * 64 + v * 4;
            if (row < p.M && col < p.N) {
                float4* o = (float4*)(outp + (int64_t)row * p.N + col);
                if constexpr (EPI == EPI_F32_ACC) {
                    float4 c = *o;
                    c.x += a.x; c.y += a.y; c.z += a.z; c.w += a.w;
                    *o = c;
                } else {
                    *o = a;
                }
            }
        }
    }
}

// dW_j += sum over splits of job j's partials, all jobs of a group in one launch
// (float4 vectors; job j owns vectors [start4[j], start4[j+1]) of the index space).
struct TnReduce {
    const float4* part[TN_MAX_JOBS];
    float4* dw[TN_MAX_JOBS];
    const float* bpart[TN_MAX_JOBS];
    float* db[TN_MAX_JOBS];
    int64_t start4[TN_MAX_JOBS + 1];
    int bstart[TN_MAX_JOBS + 1];
    int njobs, splits;
};
// dW_j += the splits' partials of job j (float4 vectors [start4[j], start4[j+1]) of
// one index space) and db_j += the splits' bias column sums (rows [bstart[j],
// bstart[j+1]) of a second one), all jobs of a group in one launch, splits in order.
__global__ void splitk_reduce_group_kernel(TnReduce R) {
    const int64_t n4 = R.start4[R.njobs];
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        int j = 0;
        while (j + 1 < R.njobs && i >= R.start4[j + 1]) ++j;
        const int64_t e = i - R.start4[j], stride4 = R.start4[j + 1] - R.start4[j];
        float4 a = R.dw[j][e];
        for (int sp = 0; sp < R.splits; ++sp) {
            const float4 b = R.part[j][sp * stride4 + e];
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        R.dw[j][e] = a;
    }
    const int nb = R.bstart[R.njobs];
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nb; i += gridDim.x * blockDim.x) {
        int j = 0;
        while (j + 1 < R.njobs && i >= R.bstart[j + 1]) ++j;
        if (R.db[j] == nullptr) continue;
        const int r = i - R.bstart[j], rows = R.bstart[j + 1] - R.bstart[j];
        float a = R.db[j][r];
        for (int sp = 0; sp < R.splits; ++sp) a += R.bpart[j][(int64_t)sp * rows + r];
        R.db[j][r] = a;
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
                prof_launch((gemm_kernel<BM, BN, WGM, WGN, A_T, B_T, EPI>), grid, dim3(64 * WGM * WGN), 0,
                                   s, p));
    return hipGetLastError();
}

// Forward / input-gradient products: 256x256 tiles (eight 128x64 wave tiles)
// when the problem has enough of them, else 128x128.
template <int EPI>
hipError_t run_nt(GemmParams p, hipStream_t s) {
    p.splits = 1;
    if ((int64_t)cdiv(p.M, BIG) * cdiv(p.N, BIG) >= NUM_CU / 2 && p.N % 8 == 0 && p.lda % 8 == 0 &&
        p.ldb % 8 == 0 && p.ldo % 8 == 0 && (p.res == nullptr || p.ldr % 8 == 0) &&
        (int64_t)p.M * p.lda < (1ll << 31) && (int64_t)p.N * p.ldb < (1ll << 31)) {
        p.tiles_m = (int)cdiv(p.M, BIG);
        p.tiles_n = (int)cdiv(p.N, BIG);
        p.band = p.tiles_n >= 16 ? (int)std::max<int64_t>(1, cdiv(p.tiles_m, NUM_XCD)) : 0;
        const double work = 2.0 * p.M * p.N * (double)p.nk_total * BK;
        if (EPI == EPI_BF16 && p.res != nullptr)
            PROF_LAUNCH(gemm_class(false, EPI), work, s,
                        prof_launch((gemm_nt_w8_kernel<EPI_BF16R, NT_STAGES, NT_KD>), dim3(p.tiles_m * p.tiles_n),
                                           dim3(512), 0, s, p));
        else
            PROF_LAUNCH(gemm_class(false, EPI), work, s,
                        prof_launch((gemm_nt_w8_kernel<EPI, NT_STAGES, NT_KD>), dim3(p.tiles_m * p.tiles_n),
                                           dim3(512), 0, s, p));
        return hipGetLastError();
    }
    return run<128, 128, 2, 2, false, false, EPI>(p, s);
}

// Splits for a group of weight-gradient products with `tiles` 256x256 output
// tiles in all: the fewest that fill at least 80% of the last pass over the 256
// CUs (fewer splits, less partial traffic), else the best filling count; each
// split keeps >= 4 K-steps of 64 tokens.
int tn_group_splits(int64_t tiles, int nk) {
    if (tiles >= NUM_CU) return 1;
    int best = 1;
    double best_eff = 0.0;
    for (int sp = 1; sp <= 64 && nk / sp >= 4; ++sp) {
        const double waves = (double)(tiles * sp) / NUM_CU;
        const double eff = waves / std::ceil(waves);
        if (eff >= 0.8) return sp;
        if (eff > best_eff + 0.02) {
            best_eff = eff;
            best = sp;
        }
    }
    return best;
}

// A group of products whose tiles fill whole passes over the CUs except for a
// mostly idle last pass: the smallest products that cover that remainder run
// as a second launch split over tokens (with fp32 partials and a reduce), the
// rest as full passes.  head / tail receive job indices in their given order.
bool tn_group_tail_plan(const TnJobDesc* jobs, int n, int nk, int* head, int* nh, int* tail, int* nt,
                        int* tail_splits) {
    if (n < 2) return false;
    int64_t t[TN_MAX_JOBS], T = 0;
    for (int j = 0; j < n; ++j) {
        t[j] = cdiv(jobs[j].N, BIG) * cdiv(jobs[j].K, BIG);
        T += t[j];
    }
    const int64_t r = T % NUM_CU;
    if (T < NUM_CU || r == 0 || r * 5 >= NUM_CU * 4) return false;
    int order[TN_MAX_JOBS];
    for (int j = 0; j < n; ++j) order[j] = j;
    std::stable_sort(order, order + n, [&](int a, int b) { return t[a] < t[b]; });
    int64_t st = 0;
    int k = 0;
    while (k < n && st < r) st += t[order[k++]];
    if (k >= n) return false;
    const int sp = tn_group_splits(st, nk);
    if (sp < 2) return false;
    const double passes = std::ceil((double)(T - st) / NUM_CU) + std::ceil((double)(st * sp) / NUM_CU) / sp;
    if (passes >= std::ceil((double)T / NUM_CU) - 0.25) return false;
    bool in_tail[TN_MAX_JOBS] = {};
    for (int i = 0; i < k; ++i) in_tail[order[i]] = true;
    *nh = *nt = 0;
    for (int j = 0; j < n; ++j) (in_tail[j] ? tail[(*nt)++] : head[(*nh)++]) = j;
    *tail_splits = sp;
    return true;
}

bool tn_pipe_ok(int M, int64_t ldy, int64_t ldx, int N, int K) {
    // 32-bit element offsets, 16-byte vectors, 256x256 tiles worth running
    return ldy % 8 == 0 && ldx % 8 == 0 && N % 8 == 0 && K % 8 == 0 && (int64_t)M * ldy < (1ll << 31) &&
           (int64_t)M * ldx < (1ll << 31);
}

// A single product with more tiles than CUs whose last pass would run mostly
// idle: the output rows that fill whole passes run unsplit and the remaining
// rows run as a second product split over tokens, so the last pass is short
// instead of mostly empty.  Returns the split row and the tail's split count.
bool tn_tail_plan(int N, int K, int nk, int* full_rows, int* tail_splits) {
    const int64_t tm = cdiv(N, BIG), tn = cdiv(K, BIG), tiles = tm * tn;
    if (tiles < NUM_CU || (tiles % NUM_CU) * 5 >= NUM_CU * 4 || tiles % NUM_CU == 0) return false;
    const int64_t full_m = (tiles / NUM_CU) * NUM_CU / tn;
    if (full_m <= 0 || full_m >= tm) return false;
    const int sp = tn_group_splits((tm - full_m) * tn, nk);
    if (sp < 2) return false;
    const double passes_split = std::ceil((double)(full_m * tn) / NUM_CU) +
                                std::ceil((double)((tm - full_m) * tn * sp) / NUM_CU) / sp;
    if (passes_split >= std::ceil((double)tiles / NUM_CU) - 0.25) return false;
    *full_rows = (int)(full_m * BIG);
    *tail_splits = sp;
    return true;
}

// Bias column sums of a split launch: one row per output row of each product and split.
int64_t tn_bias_partial_elems(const TnJobDesc* jobs, int n, int splits) {
    int64_t e = 0;
    for (int j = 0; j < n; ++j) e += (int64_t)splits * jobs[j].N;
    return e;
}

// Runs jobs [0, n) of equal token count M as one grouped 256x256-tile launch
// (plus one reduce launch when split).
hipError_t run_tn_group(const TnJobDesc* jobs, int n, int M, float* partial, int64_t partial_elems, hipStream_t s) {
    TnGroup G{};
    G.njobs = n;
    G.nk_total = M / BK;
    int64_t tiles = 0, elems = 0;
    double work = 0.0;
    for (int j = 0; j < n; ++j) {
        const TnJobDesc& d = jobs[j];
        TnJob& t = G.job[j];
        t.A = d.dY; t.B = d.X; t.lda = (int)d.ldy; t.ldb = (int)d.ldx; t.M = d.N; t.N = d.K;
        t.tiles_m = (int)cdiv(d.N, BIG); t.tiles_n = (int)cdiv(d.K, BIG);
        t.dbias = d.db;
        G.tile_start[j] = (int)tiles;
        tiles += (int64_t)t.tiles_m * t.tiles_n;
        elems += (int64_t)d.N * d.K;
        work += 2.0 * d.N * d.K * (double)M;
    }
    G.tile_start[n] = (int)tiles;
    int sp = tn_group_splits(tiles, G.nk_total);
    if (sp > 1 && (partial == nullptr || partial_elems < sp * elems + tn_bias_partial_elems(jobs, n, sp))) sp = 1;
    G.splits = sp;
    if (sp == 1) {
        for (int j = 0; j < n; ++j) G.job[j].out = jobs[j].dW;
        PROF_LAUNCH(KC_GEMM_TN_ACC, work, s,
                    prof_launch((gemm_tn_w8_kernel<EPI_F32_ACC, TN_STAGES, TN_TD>), dim3(tiles), dim3(512),
                                       0, s, G));
        return hipGetLastError();
    }
    TnReduce R{};
    R.njobs = n;
    R.splits = sp;
    int64_t off = 0;
    for (int j = 0; j < n; ++j) {
        const int64_t e = (int64_t)jobs[j].N * jobs[j].K;
        G.job[j].out = partial + off;
        R.part[j] = (const float4*)(partial + off);
        R.dw[j] = (float4*)jobs[j].dW;
        R.start4[j + 1] = R.start4[j] + e / 4;
        off += sp * e;
    }
    G.bpart = partial + off;  // then the splits' bias column sums, sp * N floats per job
    for (int j = 0; j < n; ++j) {
        R.bpart[j] = partial + off;
        R.db[j] = jobs[j].db;
        R.bstart[j + 1] = R.bstart[j] + jobs[j].N;
        off += (int64_t)sp * jobs[j].N;
    }
    PROF_LAUNCH(KC_GEMM_TN_SPLIT, work, s,
                prof_launch((gemm_tn_w8_kernel<EPI_F32_STORE, TN_STAGES, TN_TD>), dim3(tiles * sp),
                                   dim3(512), 0, s, G));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = std::max<int64_t>(R.start4[n], R.bstart[n]);
    const int blocks = (int)std::min<int64_t>(cdiv(n4, 256), 4096);
    PROF_LAUNCH(KC_SPLITK_REDUCE, 16.0 * n4 * (sp + 2), s,
                prof_launch(splitk_reduce_group_kernel, dim3(blocks), dim3(256), 0, s, R));
    return hipGetLastError();
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
                               const float* bias, uint16_t* gprime, uint16_t* g, int64_t ldo, hipStream_t s) {
    GemmParams p{};
    p.A = A; p.B = B; p.lda = lda; p.ldb = ldb; p.M = M; p.N = N; p.nk_total = K / BK;
    p.bias = bias; p.out = gprime; p.out2 = g; p.ldo = ldo;
    return run_nt<EPI_GELU>(p, s);
}

hipError_t launch_gemm_nt_dgelu(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                                const uint16_t* gprime, uint16_t* out, int64_t ldo, hipStream_t s) {
    GemmParams p{};
    p.A = A; p.B = B; p.lda = lda; p.ldb = ldb; p.M = M; p.N = N; p.nk_total = K / BK;
    p.res = gprime; p.ldr = ldo; p.out = out; p.ldo = ldo;
    return run_nt<EPI_DGELU>(p, s);
}

int64_t gemm_tn_partial_elems(int M, int N, int K) {
    const TnJobDesc d{nullptr, K, nullptr, K, N, K, nullptr, nullptr};
    return gemm_tn_group_partial_elems(&d, 1, M);
}

hipError_t launch_gemm_tn_acc(const uint16_t* dY, int64_t ldy, const uint16_t* X, int64_t ldx, int M, int N, int K,
                              float* dW, float* dbias, float* partial, int64_t partial_elems, hipStream_t s) {
    // output rows = N (features of dY), output cols = K (features of X), reduction = M tokens
    const TnJobDesc d{dY, ldy, X, ldx, N, K, dW, dbias};
    return launch_gemm_tn_group(&d, 1, M, partial, partial_elems, s);
}

hipError_t launch_gemm_tn_group(const TnJobDesc* jobs, int n, int M, float* partial, int64_t partial_elems,
                                hipStream_t s) {
    if (n < 1 || n > TN_MAX_JOBS || M < BK || M % BK) return hipErrorInvalidValue;
    int64_t tiles = 0;
    bool pipe = true;
    for (int j = 0; j < n; ++j) {
        pipe = pipe && tn_pipe_ok(M, jobs[j].ldy, jobs[j].ldx, jobs[j].N, jobs[j].K);
        tiles += cdiv(jobs[j].N, BIG) * cdiv(jobs[j].K, BIG);
    }
    int full_rows = 0, tail_sp = 1;
    if (pipe && n == 1 && tn_tail_plan(jobs[0].N, jobs[0].K, M / BK, &full_rows, &tail_sp)) {
        const TnJobDesc& d = jobs[0];
        const TnJobDesc head{d.dY, d.ldy, d.X, d.ldx, full_rows, d.K, d.dW, d.db};
        const TnJobDesc tail{d.dY + full_rows, d.ldy, d.X, d.ldx, d.N - full_rows, d.K,
                             d.dW + (int64_t)full_rows * d.K, d.db ? d.db + full_rows : nullptr};
        hipError_t e = run_tn_group(&head, 1, M, nullptr, 0, s);
        return e != hipSuccess ? e : run_tn_group(&tail, 1, M, partial, partial_elems, s);
    }
    int hi[TN_MAX_JOBS], ti[TN_MAX_JOBS], nh = 0, nt = 0;
    if (pipe && tn_group_tail_plan(jobs, n, M / BK, hi, &nh, ti, &nt, &tail_sp)) {
        TnJobDesc hj[TN_MAX_JOBS], tj[TN_MAX_JOBS];
        for (int i = 0; i < nh; ++i) hj[i] = jobs[hi[i]];
        for (int i = 0; i < nt; ++i) tj[i] = jobs[ti[i]];
        hipError_t e = run_tn_group(hj, nh, M, nullptr, 0, s);
        return e != hipSuccess ? e : run_tn_group(tj, nt, M, partial, partial_elems, s);
    }
    if (pipe && tiles >= 8) return run_tn_group(jobs, n, M, partial, partial_elems, s);
    // small or unaligned products: the generic 128x128 kernel, one job at a time
    for (int j = 0; j < n; ++j) {
        const TnJobDesc& d = jobs[j];
        GemmParams p{};
        p.A = d.dY; p.B = d.X; p.lda = d.ldy; p.ldb = d.ldx; p.M = d.N; p.N = d.K; p.nk_total = M / BK;
        p.splits = 1; p.dbias = d.db; p.outf = d.dW; p.ldf = d.K;
        hipError_t e = run<128, 128, 2, 2, true, true, EPI_F32_ACC>(p, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Split partials of a launch: splits x (N x K dW partials + N bias column sums) per product.
int64_t gemm_tn_group_partial_elems(const TnJobDesc* jobs, int n, int M) {
    int full_rows = 0, tail_sp = 1;
    if (n == 1 && tn_tail_plan(jobs[0].N, jobs[0].K, M / BK, &full_rows, &tail_sp))
        return (int64_t)tail_sp * (jobs[0].N - full_rows) * (jobs[0].K + 1);
    int hi[TN_MAX_JOBS], ti[TN_MAX_JOBS], nh = 0, nt = 0;
    if (n <= TN_MAX_JOBS && tn_group_tail_plan(jobs, n, M / BK, hi, &nh, ti, &nt, &tail_sp)) {
        int64_t e = 0;
        for (int i = 0; i < nt; ++i) e += (int64_t)jobs[ti[i]].N * (jobs[ti[i]].K + 1);
        return tail_sp * e;
    }
    int64_t tiles = 0, elems = 0;
    for (int j = 0; j < n; ++j) {
        tiles += cdiv(jobs[j].N, BIG) * cdiv(jobs[j].K, BIG);
        elems += (int64_t)jobs[j].N * jobs[j].K;
    }
    const int sp = tn_group_splits(tiles, M / BK);
    return sp > 1 ? sp * elems + tn_bias_partial_elems(jobs, n, sp) : 0;
}
