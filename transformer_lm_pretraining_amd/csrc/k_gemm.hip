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
//     MFMA loop is identical for both.
// Tiles: BM x BN per 256-thread workgroup (4 waves), K step 64, LDS double
// buffered (one barrier per K step) with register prefetch of the next
// tile; rows padded to 72 bf16 (144 B) so the 16-byte fragment reads of 32
// consecutive rows hit distinct banks.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int NTHREADS = 256;
constexpr int GROUP_M = 8;

enum Epi { EPI_BF16 = 0, EPI_GELU = 1, EPI_F32_ACC = 2, EPI_F32_STORE = 3 };

struct GemmParams {
    const uint16_t* A;
    const uint16_t* B;
    int64_t lda, ldb;
    int M, N;          // output rows / cols
    int k_len;         // reduction length handled by one split
    int tiles_m, tiles_n;
    const float* bias;
    const uint16_t* res;
    int64_t ldr;
    uint16_t* out;
    uint16_t* out2;
    int64_t ldo;
    float* outf;
    int64_t ldf;
    int64_t split_stride;
};

// Tile loader for an operand stored contiguous along the reduction:
// element (row, k) at base[row * ld + k].
template <int R>
struct LoaderK {
    static constexpr int NV = R * (BK / 8) / NTHREADS;
    u32x4 v[NV];
    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int row0, int rows, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int vid = tid + NTHREADS * i;
            int r = vid >> 3, kv = vid & 7;
            if (row0 + r < rows)
                v[i] = *(const u32x4*)(base + (int64_t)(row0 + r) * ld + k0 + kv * 8);
            else
                v[i] = u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int vid = tid + NTHREADS * i;
            int r = vid >> 3, kv = vid & 7;
            *(u32x4*)(s + r * LDK + kv * 8) = v[i];
        }
    }
};

// Tile loader for an operand stored contiguous along the output dim:
// element (row, k) at base[k * ld + row].  Each active thread loads an 8(k) x
// 8(row) block and writes it transposed.
template <int R>
struct LoaderT {
    static constexpr int NB = R;  // (R/8) row chunks x (BK/8) k chunks
    static_assert(NB <= NTHREADS, "one 8x8 block per thread");
    u32x4 v[8];
    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int row0, int rows, int k0, int tid) {
        if (tid >= NB) return;
        int rc = tid % (R / 8), kc = tid / (R / 8);
        int row = row0 + rc * 8;
        bool ok = row < rows;  // rows % 8 == 0
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            v[kk] = ok ? *(const u32x4*)(base + (int64_t)(k0 + kc * 8 + kk) * ld + row) : u32x4{0, 0, 0, 0};
    }
    __device__ __forceinline__ void store(uint16_t* s, int tid) const {
        if (tid >= NB) return;
        int rc = tid % (R / 8), kc = tid / (R / 8);
        u32x4 w[8];
        transpose8x8(v, w);
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(s + (rc * 8 + c) * LDK + kc * 8) = w[c];
    }
};

template <int BM, int BN, int WGM, int WGN, bool A_T, bool B_T, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(GemmParams p) {
    static_assert(WGM * WGN == 4, "4 waves");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * LDK];
    constexpr int STAGE = (BM + BN) * LDK;  // stage s: A tile at smem + s*STAGE, B tile after it

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // grouped tile order: GROUP_M row tiles share each column sweep (L2 reuse)
    int pid = blockIdx.x;
    int in_group = GROUP_M * p.tiles_n;
    int first_m = (pid / in_group) * GROUP_M;
    int gsize = min(p.tiles_m - first_m, GROUP_M);
    int tm = first_m + (pid % in_group) % gsize;
    int tn = (pid % in_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kbeg = split * p.k_len;
    const int nk = p.k_len / BK;

    typename std::conditional<A_T, LoaderT<BM>, LoaderK<BM>>::type la;
    typename std::conditional<B_T, LoaderT<BN>, LoaderK<BN>>::type lb;

    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    la.load(p.A, p.lda, m0, p.M, kbeg, tid);
    lb.load(p.B, p.ldb, n0, p.N, kbeg, tid);
    la.store(smem, tid);
    lb.store(smem + BM * LDK, tid);
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
            la.store(smem + (cur ^ 1) * STAGE, tid);
            lb.store(smem + (cur ^ 1) * STAGE + BM * LDK, tid);
        }
        __syncthreads();
    }

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
                } else if constexpr (EPI == EPI_F32_ACC) {
                    p.outf[(int64_t)row * p.ldf + col] += x;
                } else {
                    p.outf[split * p.split_stride + (int64_t)row * p.ldf + col] = x;
                }
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
    return !a_t ? (epi == EPI_GELU ? KC_GEMM_NT_GELU : KC_GEMM_NT)
                : (epi == EPI_F32_STORE ? KC_GEMM_TN_SPLIT : KC_GEMM_TN_ACC);
}

template <int BM, int BN, int WGM, int WGN, bool A_T, bool B_T, int EPI>
hipError_t run(GemmParams p, int splits, hipStream_t s) {
    p.tiles_m = (int)cdiv(p.M, BM);
    p.tiles_n = (int)cdiv(p.N, BN);
    dim3 grid(p.tiles_m * p.tiles_n, splits);
    PROF_LAUNCH(gemm_class(A_T, EPI), 2.0 * p.M * p.N * (double)p.k_len * splits, s, hipLaunchKernelGGL((gemm_kernel<BM, BN, WGM, WGN, A_T, B_T, EPI>), grid, dim3(NTHREADS), 0, s, p));
    return hipGetLastError();
}

// Split count for the weight-gradient GEMM: enough workgroups to cover the
// chip (256 CUs) while each split keeps a reduction of >= 512 tokens.
int tn_splits(int M, int N, int K) {
    int64_t tiles = cdiv(N, 128) * cdiv(K, 128);
    int splits = 1;
    while (tiles * splits < 256 && (M / (splits * 2)) >= 512 && (M % (splits * 2 * BK)) == 0) splits *= 2;
    return splits;
}

}  // namespace

hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                          const float* bias, const uint16_t* res, int64_t ldr, uint16_t* out, int64_t ldo,
                          hipStream_t s) {
    GemmParams p{};
    p.A = A; p.B = B; p.lda = lda; p.ldb = ldb; p.M = M; p.N = N; p.k_len = K;
    p.bias = bias; p.res = res; p.ldr = ldr; p.out = out; p.ldo = ldo;
    return run<128, 128, 2, 2, false, false, EPI_BF16>(p, 1, s);
}

hipError_t launch_gemm_nt_gelu(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N, int K,
                               const float* bias, uint16_t* pre, uint16_t* g, int64_t ldo, hipStream_t s) {
    GemmParams p{};
    p.A = A; p.B = B; p.lda = lda; p.ldb = ldb; p.M = M; p.N = N; p.k_len = K;
    p.bias = bias; p.out = pre; p.out2 = g; p.ldo = ldo;
    return run<128, 128, 2, 2, false, false, EPI_GELU>(p, 1, s);
}

int64_t gemm_tn_partial_elems(int M, int N, int K) {
    int splits = tn_splits(M, N, K);
    return splits > 1 ? (int64_t)splits * N * K : 0;
}

hipError_t launch_gemm_tn_acc(const uint16_t* dY, int64_t ldy, const uint16_t* X, int64_t ldx, int M, int N, int K,
                              float* dW, float* partial, int64_t partial_elems, hipStream_t s) {
    // output rows = N (features of dY), output cols = K (features of X), reduction = M tokens
    int splits = tn_splits(M, N, K);
    if (splits > 1 && (partial == nullptr || partial_elems < (int64_t)splits * N * K)) splits = 1;
    GemmParams p{};
    p.A = dY; p.B = X; p.lda = ldy; p.ldb = ldx; p.M = N; p.N = K; p.k_len = M / splits;
    if (splits == 1) {
        p.outf = dW; p.ldf = K;
        return run<128, 128, 2, 2, true, true, EPI_F32_ACC>(p, 1, s);
    }
    p.outf = partial; p.ldf = K; p.split_stride = (int64_t)N * K;
    hipError_t e = run<128, 128, 2, 2, true, true, EPI_F32_STORE>(p, splits, s);
    if (e != hipSuccess) return e;
    int64_t n4 = (int64_t)N * K / 4;
    int blocks = (int)std::min<int64_t>(cdiv(n4, 256), 4096);
    PROF_LAUNCH(KC_SPLITK_REDUCE, 4.0 * n4 * 4 * (splits + 2), s, hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, (const float4*)partial, (float4*)dW, n4,
                       splits, n4));
    return hipGetLastError();
}
