// Memory-bound kernels of the step: bias + GELU forward/backward, bias
// gradients (column sums), the fused masked softmax cross-entropy, the
// embedding lookup and its scatter-add backward.  All move 16-byte vectors
// (8 bf16) per lane and keep fp32 arithmetic (PDS §4 precision paragraph).
#include <type_traits>

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
// 8-wide column vector t (a block has one thread per vector of a row, rounded up
// to whole waves) and keeps its sums in registers.  Four rows are loaded before
// any of them is used, and several blocks run per CU, so enough loads are in
// flight to stream HBM.  Each block leaves one partial row of column sums;
// fold_colsum_kernel adds the partial rows in a fixed order.
constexpr int CS_MAX_THREADS = 1024;  // N <= 8 * 1024 = 8192
constexpr int CS_ROWS = 4;            // rows in flight per thread

int colsum_blocks(int64_t rows) { return (int)std::min<int64_t>(1024, cdiv(rows, 16)); }
int colsum_threads(int N) { return (int)std::min<int64_t>(CS_MAX_THREADS, cdiv(N / 8, 64) * 64); }

template <bool GELU_BWD>
__global__ __launch_bounds__(CS_MAX_THREADS) void colsum_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                const uint16_t* __restrict__ pre,
                                                                uint16_t* __restrict__ dst,
                                                                float* __restrict__ partial, int64_t rows, int N) {
    const int cv = threadIdx.x;
    if (cv >= N / 8) return;  // no barrier below
    const int64_t rpb = cdiv(rows, gridDim.x);
    const int64_t r0 = blockIdx.x * rpb;
    const int64_t r1 = std::min<int64_t>(rows, r0 + rpb);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    // rows r .. r+n-1: loads first, then the sums in row order
    auto rows_at = [&](int64_t r, int n) {
        u32x4 w[CS_ROWS], pw[CS_ROWS];
#pragma unroll
        for (int u = 0; u < CS_ROWS; ++u)
            if (u < n) {
                w[u] = *(const u32x4*)(src + (r + u) * lds + cv * 8);
                if constexpr (GELU_BWD) pw[u] = *(const u32x4*)(pre + (r + u) * (int64_t)N + cv * 8);
            }
#pragma unroll
        for (int u = 0; u < CS_ROWS; ++u) {
            if (u >= n) break;
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bflo(w[u][e]);
                x[2 * e + 1] = bfhi(w[u][e]);
            }
            if constexpr (GELU_BWD) {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] *= gelu_grad_f(bflo(pw[u][e]));
                    x[2 * e + 1] *= gelu_grad_f(bfhi(pw[u][e]));
                    o[e] = pack_bf2(x[2 * e], x[2 * e + 1]);
                }
                *(u32x4*)(dst + (r + u) * (int64_t)N + cv * 8) = o;
                // the bias gradient is the sum of the stored (bf16) dpre
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = bflo(o[e]);
                    x[2 * e + 1] = bfhi(o[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += x[e];
        }
    };
    int64_t r = r0;
    for (; r + CS_ROWS <= r1; r += CS_ROWS) rows_at(r, CS_ROWS);
    if (r < r1) rows_at(r, (int)(r1 - r));
#pragma unroll
    for (int e = 0; e < 8; ++e) partial[(int64_t)blockIdx.x * N + cv * 8 + e] = acc[e];
}

// out[c] += sum over the nblocks partial rows of column c.  A block takes 32
// columns; its 32 phases of 32 threads each sum every 32nd partial row (phase ph:
// rows ph, ph+32, ...), then the 32 phase sums are added in phase order.
constexpr int FOLD_COLS = 32, FOLD_PHASES = 32;
__global__ __launch_bounds__(FOLD_COLS * FOLD_PHASES) void fold_colsum_kernel(const float* __restrict__ partial,
                                                                              int nblocks, int N,
                                                                              float* __restrict__ out) {
    __shared__ float red[FOLD_PHASES][FOLD_COLS];
    const int cl = threadIdx.x % FOLD_COLS, ph = threadIdx.x / FOLD_COLS;
    const int c = blockIdx.x * FOLD_COLS + cl;
    float s = 0.f;
    if (c < N) {
        int b = ph;
        for (; b + 3 * FOLD_PHASES < nblocks; b += 4 * FOLD_PHASES) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = partial[(int64_t)(b + u * FOLD_PHASES) * N + c];
#pragma unroll
            for (int u = 0; u < 4; ++u) s += v[u];
        }
        for (; b < nblocks; b += FOLD_PHASES) s += partial[(int64_t)b * N + c];
    }
    red[ph][cl] = s;
    __syncthreads();
    if (ph == 0 && c < N) {
        float t = red[0][cl];
#pragma unroll
        for (int p = 1; p < FOLD_PHASES; ++p) t += red[p][cl];
        out[c] += t;
    }
}

// ---------------------------------------------------------------- cross-entropy

constexpr int XE_THREADS = 512;

// One row per workgroup, held in registers (NV 16-byte vectors per thread).
// Three register passes: max, sum of exp, gradient.  Only the vector that
// straddles V takes per-column bounds tests; whole vectors past V are padding
// (gradient 0).  exp(x - m) is evaluated as 2^(x log2e - m log2e) (one FMA and
// the hardware exp2).  The gradient pass writes p_j * dloss for every real
// column; the owner of the target column then subtracts dloss there.
template <int NV>
__global__ __launch_bounds__(XE_THREADS) void xent_kernel(uint16_t* __restrict__ logits,
                                                          const int32_t* __restrict__ tgt,
                                                          float* __restrict__ loss_rows, int V, int Vp, float dloss,
                                                          int write_grad, int32_t* __restrict__ flag) {
    __shared__ float red[XE_THREADS / 64];
    constexpr float L2E = 1.4426950408889634f;
    const int64_t row = blockIdx.x;
    u32x4* z = (u32x4*)(logits + row * (int64_t)Vp);
    const int nvec = Vp / 8, nfull = V / 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int t = tgt[row];
    if (t == GPT2_IGNORE_TARGET) {  // loss not taken here: zero loss, zero gradient row
        if (tid == 0) loss_rows[row] = 0.f;
        if (write_grad)
            for (int vid = tid; vid < nvec; vid += XE_THREADS) z[vid] = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    u32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vid = tid + XE_THREADS * i;
        // the row is read once and its gradient written once: non-temporal hints
        v[i] = vid < nvec ? __builtin_nontemporal_load(z + vid) : u32x4{0, 0, 0, 0};
    }
    auto elem = [&](int i, int e) { return (e & 1) ? bfhi(v[i][e >> 1]) : bflo(v[i][e >> 1]); };
    // pass 1: row max over the real columns
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vid = tid + XE_THREADS * i;
        if (vid < nfull) {
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, elem(i, e));
        } else if (vid * 8 < V) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (vid * 8 + e < V) mx = fmaxf(mx, elem(i, e));
        }
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < XE_THREADS / 64; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();
    const float mb = mx * L2E;
    // pass 2: sum of exp over the real columns
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vid = tid + XE_THREADS * i;
        if (vid < nfull) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += __builtin_amdgcn_exp2f(fmaf(elem(i, e), L2E, -mb));
        } else if (vid * 8 < V) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (vid * 8 + e < V) sum += __builtin_amdgcn_exp2f(fmaf(elem(i, e), L2E, -mb));
        }
    }
    sum = wave_sum(sum);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = 0.f;
#pragma unroll
    for (int w = 0; w < XE_THREADS / 64; ++w) sum += red[w];
    if (t < 0 || t >= V) {
        if (tid == 0 && flag) atomicOr(flag, 1);
        t = t < 0 ? 0 : V - 1;
    }
    if (tid == 0) loss_rows[row] = mx + logf(sum) - bf2f(logits[row * (int64_t)Vp + t]);
    if (!write_grad) return;
    __syncthreads();  // the target logit is read before any thread overwrites the row
    const float sc = dloss / sum;
    const int tvid = t >> 3;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vid = tid + XE_THREADS * i;
        if (vid >= nvec) break;
        float d[8];
        if (vid < nfull) {
#pragma unroll
            for (int e = 0; e < 8; ++e) d[e] = __builtin_amdgcn_exp2f(fmaf(elem(i, e), L2E, -mb)) * sc;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                d[e] = vid * 8 + e < V ? __builtin_amdgcn_exp2f(fmaf(elem(i, e), L2E, -mb)) * sc : 0.0f;
        }
        if (vid == tvid) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e == (t & 7)) d[e] -= dloss;
        }
        __builtin_nontemporal_store(u32x4{pack_bf2(d[0], d[1]), pack_bf2(d[2], d[3]), pack_bf2(d[4], d[5]), pack_bf2(d[6], d[7])}, z + vid);
    }
}

__global__ __launch_bounds__(1024) void mean_kernel(const float* __restrict__ x, const int32_t* __restrict__ tgt,
                                                     int64_t n, float* __restrict__ out) {
    __shared__ double red[16];
    __shared__ double cnt[16];
    double s = 0.0, c = 0.0;
    // thread j adds rows j, j + 1024, j + 2048, ... in that order, eight loads in flight
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 8 * (int64_t)blockDim.x) {
        float xv[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = i0 + u * (int64_t)blockDim.x;
            ok[u] = i < n && (!tgt || tgt[i] != GPT2_IGNORE_TARGET);
            xv[u] = i < n ? x[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (ok[u]) {
                s += xv[u];
                c += 1.0;
            }
    }
    s = wave_sum_d(s);
    c = wave_sum_d(c);
    if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x >> 6] = s;
        cnt[threadIdx.x >> 6] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0, k = 0.0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
            t += red[w];
            k += cnt[w];
        }
        out[0] = k > 0.0 ? (float)(t / k) : 0.0f;
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

// Token-table gradient, with every addition in a fixed order (the same bits on
// every run).  (1) The rows with a valid id are sorted by token with a stable
// two-pass LSD radix sort (8 bits of the 16-bit id per pass), so the rows of
// each token come out in increasing row order.  (2) Each wave sums a window of
// EMB_WIN sorted rows run by run, for a chunk of columns.  A run inside one
// window is the only writer of its table row and read-modify-writes it; the
// pieces of a run that crosses window edges go to per-window scratch (H: the
// window's first run, T: its last run).  (3) One pass adds each crossing run's
// pieces, window by window, into its table row.  A token occurring N times
// (Zipf: the most frequent id covers ~14% of a batch) costs about N / EMB_WIN
// additions to its table row.  Ids outside [0, V) are left out.
constexpr int EMB_WIN = 32;

// Radix sort: EMB_SORT_ROWS consecutive input positions per workgroup (one per
// thread).  Pass P orders by bits [8P, 8P + 8) of the id.  hist[d * nb + b]
// holds how many keys of block b have digit d, so its exclusive scan in that
// order is where block b's keys of digit d start.
constexpr int EMB_SORT_ROWS = 1024;
constexpr int EMB_SORT_WAVES = EMB_SORT_ROWS / 64;

// Input position i of pass P: pass 0 reads row i of the token ids (valid when
// the id is in [0, V)); pass 1 reads position i of pass 0's output (valid below
// the number of valid rows).
template <int P>
__device__ __forceinline__ bool emb_key(const int32_t* __restrict__ tok, int n, int V,
                                        const int32_t* __restrict__ in_key, int nv, int i, int& key) {
    key = 0;
    if (P == 0) {
        if (i >= n) return false;
        const int t = tok[i];
        if (t < 0 || t >= V) return false;
        key = t;
        return true;
    }
    if (i >= nv) return false;
    key = in_key[i];
    return true;
}

// The lanes of this wave that hold a valid key with the same 8-bit digit (one
// ballot per digit bit); rank = how many of them sit in lower lanes.
__device__ __forceinline__ uint64_t emb_digit_match(int dig, bool valid, int lane, int& rank) {
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const bool bit = (dig >> k) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    rank = __popcll(m & ((1ull << lane) - 1ull));
    return m;
}

template <int P>
__global__ __launch_bounds__(EMB_SORT_ROWS) void emb_hist_kernel(const int32_t* __restrict__ tok, int n, int V,
                                                                 const int32_t* __restrict__ in_key,
                                                                 const int32_t* __restrict__ nvalid,
                                                                 int32_t* __restrict__ hist, int nb) {
    __shared__ int h[256];
    const int tid = threadIdx.x, lane = tid & 63, b = blockIdx.x;
    if (tid < 256) h[tid] = 0;
    __syncthreads();
    int key;
    const bool valid = emb_key<P>(tok, n, V, in_key, P == 0 ? 0 : *nvalid, b * EMB_SORT_ROWS + tid, key);
    const int dig = (key >> (8 * P)) & 255;
    int rank;
    const uint64_t m = emb_digit_match(dig, valid, lane, rank);
    if (valid && rank == 0) atomicAdd(&h[dig], (int)__popcll(m));  // one add per digit and wave
    __syncthreads();
    if (tid < 256) hist[tid * nb + b] = h[tid];
}

// Stable scatter of pass P: a key's place is where its digit starts for this
// block (scan of hist), plus the keys of that digit in lower waves of the block,
// plus those in lower lanes of its wave.  Pass 0 also records the number of
// valid rows; pass 1 writes the sorted tokens and row ids.
template <int P>
__global__ __launch_bounds__(EMB_SORT_ROWS) void emb_scatter_kernel(const int32_t* __restrict__ tok, int n, int V,
                                                                    const int32_t* __restrict__ hist, int nb,
                                                                    const int32_t* __restrict__ in_key,
                                                                    const int32_t* __restrict__ in_row,
                                                                    int32_t* __restrict__ out_key,
                                                                    int32_t* __restrict__ out_row,
                                                                    int32_t* __restrict__ nvalid) {
    __shared__ int off[256];
    __shared__ int wpre[EMB_SORT_WAVES][256];
    __shared__ int wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
    for (int i = tid; i < EMB_SORT_WAVES * 256; i += EMB_SORT_ROWS) (&wpre[0][0])[i] = 0;
    const int nv = P == 0 ? 0 : *nvalid;
    int before = 0, total = 0, incl = 0;
    if (tid < 256) {  // digit tid: keys in lower blocks, keys in all blocks, inclusive scan over digits
        const int32_t* hd = hist + (int64_t)tid * nb;
        for (int j = 0; j < nb; ++j) {
            const int c = hd[j];
            total += c;
            before += j < b ? c : 0;
        }
        incl = total;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, WAVE);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
    }
    int key;
    const int i = b * EMB_SORT_ROWS + tid;
    const bool valid = emb_key<P>(tok, n, V, in_key, nv, i, key);
    const int dig = (key >> (8 * P)) & 255;
    int rank;
    const uint64_t m = emb_digit_match(dig, valid, lane, rank);
    __syncthreads();
    if (tid < 256) {
        int lower = 0;
        for (int w = 0; w < wave; ++w) lower += wsum[w];
        off[tid] = lower + incl - total + before;
    }
    if (P == 0 && b == 0 && tid == 0) *nvalid = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (valid && rank == 0) wpre[wave][dig] = (int)__popcll(m);
    __syncthreads();
    if (tid < 256) {  // exclusive scan over the waves, digit tid
        int run = 0;
        for (int w = 0; w < EMB_SORT_WAVES; ++w) {
            const int c = wpre[w][tid];
            wpre[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    if (!valid) return;
    const int pos = off[dig] + wpre[wave][dig] + rank;
    out_key[pos] = key;
    out_row[pos] = P == 0 ? i : in_row[i];
}

// One wave per (window of EMB_WIN sorted rows, chunk of 256 columns); each lane
// owns 4 columns.  part: [window][2][C] floats (H, then T).  The column-chunk 0
// wave also records, for each run that ends in its window, the end position
// (one past its last sorted row) in bend[token].
__global__ __launch_bounds__(256) void emb_segsum_kernel(const int32_t* __restrict__ order,
                                                         const int32_t* __restrict__ stok,
                                                         const int32_t* __restrict__ nvalid,
                                                         const uint16_t* __restrict__ dx, int C,
                                                         float* __restrict__ dwte, float* __restrict__ part,
                                                         int32_t* __restrict__ bend) {
    const int n = *nvalid;
    const int nch = (C / 4 + 63) / 64;
    const int wid = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * 256 + threadIdx.x) >> 6));
    const int wv = wid / nch, ch = wid % nch;
    const int lane = threadIdx.x & 63;
    const int p0 = wv * EMB_WIN;
    if (p0 >= n) return;
    const int p1 = min(p0 + EMB_WIN, n);
    const bool head_shared = p0 > 0 && stok[p0 - 1] == stok[p0];
    const bool tail_shared = p1 < n && stok[p1] == stok[p1 - 1];
    if (ch == 0 && lane < p1 - p0) {  // lane q: does the run at sorted position p0 + q end there?
        const int p = p0 + lane, t = stok[p];
        if (p + 1 >= n || stok[p + 1] != t) bend[t] = p + 1;
    }
    const int c4 = ch * 64 + lane;
    if (c4 >= C / 4) return;
    u32x2 gv[EMB_WIN];
#pragma unroll
    for (int q = 0; q < EMB_WIN; ++q)
        if (p0 + q < p1) gv[q] = *(const u32x2*)(dx + (int64_t)order[p0 + q] * C + c4 * 4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int cur = stok[p0];
    bool first = true;
    // a run piece goes to H (first run, continuing from the previous window), to T
    // (last run, continuing into the next window) or, whole, into its table row
    auto flush = [&](bool last) {
        if (first && head_shared) {
            *(float4*)(part + (int64_t)(2 * wv) * C + c4 * 4) = acc;
        } else if (last && tail_shared) {
            *(float4*)(part + (int64_t)(2 * wv + 1) * C + c4 * 4) = acc;
        } else {
            float* d = dwte + (int64_t)cur * C + c4 * 4;
            float4 o = *(float4*)d;
            o.x += acc.x; o.y += acc.y; o.z += acc.z; o.w += acc.w;
            *(float4*)d = o;
        }
    };
#pragma unroll
    for (int q = 0; q < EMB_WIN; ++q) {
        if (p0 + q >= p1) break;
        const int t = stok[p0 + q];
        if (t != cur) {
            flush(false);
            acc = make_float4(0.f, 0.f, 0.f, 0.f);
            cur = t;
            first = false;
        }
        acc.x += bflo(gv[q].x);
        acc.y += bfhi(gv[q].x);
        acc.z += bflo(gv[q].y);
        acc.w += bfhi(gv[q].y);
    }
    flush(true);
}

// A run that crosses window edges, from the window where it starts: its piece
// there (T), the whole windows it spans and its piece in the window where it
// ends (H; that window holds the bucket's last row), added in window order, then
// into its table row.  Block (w, y): window w, 64 column vectors of 4.
__global__ __launch_bounds__(64) void emb_combine_kernel(const int32_t* __restrict__ stok,
                                                         const int32_t* __restrict__ bend,
                                                         const int32_t* __restrict__ nvalid, int C,
                                                         const float* __restrict__ part, float* __restrict__ dwte) {
    const int n = *nvalid;
    const int w = blockIdx.x;
    const int p0 = w * EMB_WIN, p1 = min(p0 + EMB_WIN, n);
    if (p0 >= n) return;
    if (!(p1 < n && stok[p1] == stok[p1 - 1])) return;                           // last run ends here
    if (p0 > 0 && stok[p0 - 1] == stok[p0] && stok[p0] == stok[p1 - 1]) return;  // it started earlier
    const int c4 = blockIdx.y * 64 + threadIdx.x;
    if (c4 >= C / 4) return;
    const int t = stok[p1 - 1];
    const int wlast = (bend[t] - 1) / EMB_WIN;
    float4 acc = *(const float4*)(part + (int64_t)(2 * w + 1) * C + c4 * 4);
    int w2 = w + 1;
    for (; w2 + 8 <= wlast + 1; w2 += 8) {  // eight loads in flight, added in window order
        float4 h[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) h[u] = *(const float4*)(part + (int64_t)(2 * (w2 + u)) * C + c4 * 4);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc.x += h[u].x; acc.y += h[u].y; acc.z += h[u].z; acc.w += h[u].w;
        }
    }
    for (; w2 <= wlast; ++w2) {
        const float4 h = *(const float4*)(part + (int64_t)(2 * w2) * C + c4 * 4);
        acc.x += h.x; acc.y += h.y; acc.z += h.z; acc.w += h.w;
    }
    float* d = dwte + (int64_t)t * C + c4 * 4;
    float4 o = *(float4*)d;
    o.x += acc.x; o.y += acc.y; o.z += acc.z; o.w += acc.w;
    *(float4*)d = o;
}

// Position-table gradient: each thread owns VEC consecutive entries of the T x C
// table and adds the batch's B rows of them in batch order (16- or 8-byte loads).
template <int VEC>
__global__ __launch_bounds__(256) void embedding_bwd_wpe_kernel(const uint16_t* __restrict__ dx,
                                                                float* __restrict__ dwpe, int B, int T, int C) {
    using LoadT = std::conditional_t<VEC == 8, u32x4, u32x2>;
    const int64_t total = (int64_t)T * C, nvec = total / VEC;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * blockDim.x) {
        float s[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] = 0.f;
        const uint16_t* src = dx + v * VEC;
#pragma unroll 4
        for (int b = 0; b < B; ++b) {
            const LoadT w = *(const LoadT*)(src + (int64_t)b * total);
#pragma unroll
            for (int e = 0; e < VEC / 2; ++e) {
                s[2 * e] += bflo(w[e]);
                s[2 * e + 1] += bfhi(w[e]);
            }
        }
        float* d = dwpe + v * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            float4 o = *(float4*)(d + e);
            o.x += s[e]; o.y += s[e + 1]; o.z += s[e + 2]; o.w += s[e + 3];
            *(float4*)(d + e) = o;
        }
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
    PROF_LAUNCH(KC_BIAS_GELU_FWD, 48.0 * nvec, s, prof_launch(bias_gelu_fwd_kernel, dim3(grid_for(nvec)), dim3(256), 0, s, (const u32x4*)u, b, (u32x4*)pre,
                       (u32x4*)g, nvec, N / 8));
    return hipGetLastError();
}

int64_t colsum_partial_elems(int64_t rows, int N) { return (int64_t)colsum_blocks(rows) * N; }

hipError_t launch_bias_gelu_bwd(const uint16_t* pre, const uint16_t* dg, uint16_t* dpre, float* db, float* partial,
                                int64_t rows, int N, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (N % 8 || N > 8 * CS_MAX_THREADS) return hipErrorInvalidValue;
    int blocks = colsum_blocks(rows);
    PROF_LAUNCH(KC_GELU_BWD, 6.0 * rows * N, s, prof_launch(colsum_kernel<true>, dim3(blocks), dim3(colsum_threads(N)), 0, s, dg, (int64_t)N, pre, dpre, partial,
                       rows, N));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PROF_LAUNCH(KC_FOLD, 4.0 * blocks * N, s, prof_launch(fold_colsum_kernel, dim3(cdiv(N, FOLD_COLS)), dim3(FOLD_COLS * FOLD_PHASES), 0, s, partial, blocks, N, db));
    return hipGetLastError();
}

hipError_t launch_bias_grad(const uint16_t* dY, int64_t ldy, float* db, float* partial, int64_t rows, int N,
                            hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (N % 8 || N > 8 * CS_MAX_THREADS) return hipErrorInvalidValue;
    int blocks = colsum_blocks(rows);
    PROF_LAUNCH(KC_COLSUM, 2.0 * rows * N, s, prof_launch(colsum_kernel<false>, dim3(blocks), dim3(colsum_threads(N)), 0, s, dY, ldy, (const uint16_t*)nullptr,
                       (uint16_t*)nullptr, partial, rows, N));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fold_colsum_kernel, dim3(cdiv(N, FOLD_COLS)), dim3(FOLD_COLS * FOLD_PHASES), 0, s, partial, blocks, N, db);
    return hipGetLastError();
}

hipError_t launch_xent(uint16_t* logits, const int32_t* tgt, float* loss_rows, int64_t rows, int V, int Vp,
                       float dloss, int write_grad, int32_t* flag, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int nv = (int)cdiv(Vp / 8, XE_THREADS);
    dim3 grid((unsigned)rows), block(XE_THREADS);
    switch (nv) {
#define XE(n) \
    case n: PROF_LAUNCH(KC_XENT, 2.0 * rows * Vp * (write_grad ? 2 : 1), s, prof_launch(xent_kernel<n>, grid, block, 0, s, logits, tgt, loss_rows, V, Vp, dloss, write_grad, flag)); break;
        XE(1) XE(2) XE(3) XE(4) XE(5) XE(6) XE(7) XE(8) XE(9) XE(10) XE(11) XE(12) XE(13) XE(14) XE(15) XE(16)
#undef XE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mean(const float* x, const int32_t* tgt, int64_t n, float* out, hipStream_t s) {
    PROF_LAUNCH(KC_MEAN, 8.0 * n, s, prof_launch(mean_kernel, dim3(1), dim3(1024), 0, s, x, tgt, n, out));
    return hipGetLastError();
}

hipError_t launch_embedding_fwd(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, uint16_t* x, int B,
                                int T, int C, int V, int32_t* flag, hipStream_t s) {
    int64_t rows = (int64_t)B * T;
    PROF_LAUNCH(KC_EMB_FWD, 6.0 * rows * C, s, prof_launch(embedding_fwd_kernel, dim3(grid_for(rows * (C / 8))), dim3(256), 0, s, tok, wte, wpe, x, rows,
                       T, C, V, flag));
    return hipGetLastError();
}

namespace {
constexpr int64_t EMB_CHUNK = 65535;  // rows per chunk; larger batches go in several
// work (int32): nvalid (+ 3 pad), the two histograms (256 x blocks each), pass 0's
// keys and rows, the sorted tokens and rows (nmax each), bucket ends (V), then
// the window pieces (floats) from the next 16-byte boundary
int64_t emb_part_offset(int64_t nmax, int V) {
    return (4 + 2 * 256 * cdiv(nmax, EMB_SORT_ROWS) + 4 * nmax + V + 3) / 4 * 4;
}
}  // namespace

int64_t embedding_bwd_work_elems(int64_t rows, int V, int C) {
    const int64_t nmax = std::min(rows, EMB_CHUNK);
    return emb_part_offset(nmax, V) + 2 * cdiv(nmax, EMB_WIN) * C;
}

hipError_t launch_embedding_bwd(const int32_t* tok, const uint16_t* dx, float* dwte, float* dwpe, int B, int T,
                                int C, int V, int32_t* work, int64_t work_elems, hipStream_t s) {
    const int64_t rows = (int64_t)B * T;
    if (C % 4 || V > 65536 || work == nullptr || work_elems < embedding_bwd_work_elems(rows, V, C) ||
        rows > INT32_MAX)
        return hipErrorInvalidValue;
    const int64_t nmax = std::min(rows, EMB_CHUNK);
    const int64_t nbmax = cdiv(nmax, EMB_SORT_ROWS);
    int32_t* nvalid = work;
    int32_t* hist0 = work + 4;
    int32_t* hist1 = hist0 + 256 * nbmax;
    int32_t* key0 = hist1 + 256 * nbmax;
    int32_t* row0 = key0 + nmax;
    int32_t* stok = row0 + nmax;
    int32_t* order = stok + nmax;
    int32_t* bend = order + nmax;
    float* part = (float*)(work + emb_part_offset(nmax, V));
    for (int64_t r0 = 0; r0 < rows; r0 += EMB_CHUNK) {
        const int n = (int)std::min(EMB_CHUNK, rows - r0);
        const int nb = (int)cdiv(n, EMB_SORT_ROWS);
        const int64_t nwin = cdiv(n, EMB_WIN);
        const int64_t nwaves = nwin * cdiv(C / 4, 64);
        const int32_t* tk = tok + r0;
        PROF_SPAN(KC_EMB_BWD_WTE, 4.0 * n * C + 8.0 * n * C, s, {
            hipLaunchKernelGGL(emb_hist_kernel<0>, dim3(nb), dim3(EMB_SORT_ROWS), 0, s, tk, n, V, nullptr, nvalid,
                               hist0, nb);
            hipLaunchKernelGGL(emb_scatter_kernel<0>, dim3(nb), dim3(EMB_SORT_ROWS), 0, s, tk, n, V, hist0, nb,
                               nullptr, nullptr, key0, row0, nvalid);
            hipLaunchKernelGGL(emb_hist_kernel<1>, dim3(nb), dim3(EMB_SORT_ROWS), 0, s, tk, n, V, key0, nvalid,
                               hist1, nb);
            hipLaunchKernelGGL(emb_scatter_kernel<1>, dim3(nb), dim3(EMB_SORT_ROWS), 0, s, tk, n, V, hist1, nb,
                               key0, row0, stok, order, nvalid);
            hipLaunchKernelGGL(emb_segsum_kernel, dim3((unsigned)cdiv(nwaves, 4)), dim3(256), 0, s, order, stok,
                               nvalid, dx + r0 * C, C, dwte, part, bend);
            hipLaunchKernelGGL(emb_combine_kernel, dim3((unsigned)nwin, (unsigned)cdiv(C / 4, 64)), dim3(64), 0, s,
                               stok, bend, nvalid, C, part, dwte);
        });
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (((int64_t)T * C) % 8 == 0)
        PROF_LAUNCH(KC_EMB_BWD_WPE, 2.0 * rows * C + 8.0 * T * C, s,
                    prof_launch(embedding_bwd_wpe_kernel<8>, dim3(grid_for((int64_t)T * C / 8)), dim3(256), 0,
                                       s, dx, dwpe, B, T, C));
    else  // C % 4 == 0
        PROF_LAUNCH(KC_EMB_BWD_WPE, 2.0 * rows * C + 8.0 * T * C, s,
                    prof_launch(embedding_bwd_wpe_kernel<4>, dim3(grid_for((int64_t)T * C / 4)), dim3(256), 0,
                                       s, dx, dwpe, B, T, C));
    return hipGetLastError();
}
