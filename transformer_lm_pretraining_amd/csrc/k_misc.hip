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
    int64_t r = r0;
    if constexpr (!GELU_BWD) {
        // four rows' loads in flight, added in row order
        for (; r + 4 <= r1; r += 4) {
#pragma unroll
            for (int q = 0; q < CS_MAXV; ++q) {
                const int cv = threadIdx.x + CS_THREADS * q;
                if (cv >= nv) break;
                u32x4 w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) w[u] = *(const u32x4*)(src + (r + u) * lds + cv * 8);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[q][2 * e] += bflo(w[u][e]);
                        acc[q][2 * e + 1] += bfhi(w[u][e]);
                    }
            }
        }
    }
    for (; r < r1; ++r) {
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
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        if (tgt && tgt[i] == GPT2_IGNORE_TARGET) continue;
        s += x[i];
        c += 1.0;
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
// every run).  (1) The rows are counting-sorted by token id in one workgroup
// (count, scan and scatter in LDS); the scan also leaves each token's bucket
// start in global memory.  (2) Within each bucket the rows are put in
// increasing row order (a row's place is the number of smaller row ids in its
// bucket).  (3) Each wave sums a window of EMB_WIN sorted rows run by run, for a
// chunk of columns.  A run inside one window is the only writer of its table
// row and read-modify-writes it; the pieces of a run that crosses window edges
// go to per-window scratch (H: the window's first run, T: its last run).
// (4) One pass adds each crossing run's pieces, window by window, into its
// table row.  A token occurring N times (Zipf: the most frequent id covers ~14%
// of a batch) costs about N / EMB_WIN additions to its table row.  Ids outside
// [0, V) are left out.
constexpr int EMB_WIN = 32;

// Counting sort of the row ids by token in one workgroup, all in LDS: 16-bit
// counts packed two per word (a chunk has fewer than 65,536 rows), counted with
// LDS atomics, scanned in place into start offsets (also written to bstart[0..V],
// bstart[V] = number of valid rows), then advanced by the scatter.  Writes
// order[] / stok[] (row index and token of each sorted position; the order
// within a bucket is not yet fixed) and the valid row count to *nvalid.
constexpr int EMB_SORT_THREADS = 1024;
__global__ __launch_bounds__(EMB_SORT_THREADS) void emb_sort_kernel(const int32_t* __restrict__ tok, int rows, int V,
                                                                    int32_t* __restrict__ order,
                                                                    int32_t* __restrict__ stok,
                                                                    int32_t* __restrict__ bstart,
                                                                    int32_t* __restrict__ nvalid) {
    __shared__ uint32_t cnt[32768];  // counts of token t in half (t & 1) of word t >> 1
    __shared__ int wtot[EMB_SORT_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int words = (V + 1) >> 1;
    for (int i = tid; i < words; i += EMB_SORT_THREADS) cnt[i] = 0u;
    __syncthreads();
    for (int i = tid; i < rows; i += EMB_SORT_THREADS) {
        const int t = tok[i];
        if (t >= 0 && t < V) atomicAdd(&cnt[t >> 1], 1u << ((t & 1) * 16));
    }
    __syncthreads();
    // exclusive scan over the counts: thread tid owns words [tid*per, (tid+1)*per)
    const int per = (words + EMB_SORT_THREADS - 1) / EMB_SORT_THREADS;
    const int w0 = min(tid * per, words), w1 = min(w0 + per, words);
    int local = 0;
    for (int w = w0; w < w1; ++w) local += (int)(cnt[w] & 0xffffu) + (int)(cnt[w] >> 16);
    int x = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    int run = before + x - local;
    for (int w = w0; w < w1; ++w) {
        const uint32_t c = cnt[w];
        const uint32_t lo = (uint32_t)run, hi = (uint32_t)(run + (int)(c & 0xffffu));
        run = (int)hi + (int)(c >> 16);
        cnt[w] = lo | (hi << 16);
    }
    if (tid == EMB_SORT_THREADS - 1) {
        *nvalid = run;
        bstart[V] = run;
    }
    __syncthreads();
    for (int t = tid; t < V; t += EMB_SORT_THREADS) bstart[t] = (int)((cnt[t >> 1] >> ((t & 1) * 16)) & 0xffffu);
    __syncthreads();
    for (int i = tid; i < rows; i += EMB_SORT_THREADS) {
        const int t = tok[i];
        if (t < 0 || t >= V) continue;
        const int sh = (t & 1) * 16;
        const int pos = (int)((atomicAdd(&cnt[t >> 1], 1u << sh) >> sh) & 0xffffu);
        order[pos] = i;
        stok[pos] = t;
    }
}

// Sorted position p of bucket [s, e) takes the row whose id has rank p - s among
// the bucket's ids (ids in a bucket are distinct), from the scatter's order.  A
// block of 256 positions copies the ids of every bucket it touches into LDS
// (EMB_RANK_TILE at a time, all loads in flight); each thread counts the smaller
// ids inside its own bucket, four per LDS read where the range allows.
constexpr int EMB_RANK_TILE = 8192;
__global__ __launch_bounds__(256) void emb_rank_kernel(const int32_t* __restrict__ scattered,
                                                       const int32_t* __restrict__ stok,
                                                       const int32_t* __restrict__ bstart,
                                                       const int32_t* __restrict__ nvalid,
                                                       int32_t* __restrict__ order) {
    __shared__ int4 ids4[EMB_RANK_TILE / 4];
    const int* ids = (const int*)ids4;
    const int n = *nvalid;
    const int b0 = blockIdx.x * 256;
    if (b0 >= n) return;
    const int b1 = min(b0 + 256, n);
    const int p = b0 + threadIdx.x;
    const bool live = p < n;
    const int t = stok[live ? p : b0];
    const int s = bstart[t], e = bstart[t + 1];
    const int my = live ? scattered[p] : 0;
    const int u0 = bstart[stok[b0]], u1 = bstart[stok[b1 - 1] + 1];  // the buckets this block touches
    int rank = 0;
    for (int q0 = u0; q0 < u1; q0 += EMB_RANK_TILE) {
        const int m = min(EMB_RANK_TILE, u1 - q0);
        __syncthreads();
        for (int i = threadIdx.x; i < m; i += 256) ((int*)ids4)[i] = scattered[q0 + i];
        __syncthreads();
        int k = max(s - q0, 0);
        const int k1 = min(e - q0, m);
        for (; k < k1 && (k & 3); ++k) rank += ids[k] < my ? 1 : 0;
#pragma unroll 8
        for (; k + 4 <= k1; k += 4) {
            const int4 v = ids4[k >> 2];
            rank += (v.x < my ? 1 : 0) + (v.y < my ? 1 : 0) + (v.z < my ? 1 : 0) + (v.w < my ? 1 : 0);
        }
        for (; k < k1; ++k) rank += ids[k] < my ? 1 : 0;
    }
    if (live) order[s + rank] = my;
}

// One wave per (window of EMB_WIN sorted rows, chunk of 256 columns); each lane
// owns 4 columns.  part: [window][2][C] floats (H, then T).
__global__ __launch_bounds__(256) void emb_segsum_kernel(const int32_t* __restrict__ order,
                                                         const int32_t* __restrict__ stok,
                                                         const int32_t* __restrict__ nvalid,
                                                         const uint16_t* __restrict__ dx, int C,
                                                         float* __restrict__ dwte, float* __restrict__ part) {
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
                                                         const int32_t* __restrict__ bstart,
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
    const int wlast = (bstart[t + 1] - 1) / EMB_WIN;
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

hipError_t launch_mean(const float* x, const int32_t* tgt, int64_t n, float* out, hipStream_t s) {
    PROF_LAUNCH(KC_MEAN, 8.0 * n, s, hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, x, tgt, n, out));
    return hipGetLastError();
}

hipError_t launch_embedding_fwd(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, uint16_t* x, int B,
                                int T, int C, int V, int32_t* flag, hipStream_t s) {
    int64_t rows = (int64_t)B * T;
    PROF_LAUNCH(KC_EMB_FWD, 6.0 * rows * C, s, hipLaunchKernelGGL(embedding_fwd_kernel, dim3(grid_for(rows * (C / 8))), dim3(256), 0, s, tok, wte, wpe, x, rows,
                       T, C, V, flag));
    return hipGetLastError();
}

namespace {
constexpr int64_t EMB_CHUNK = 65535;  // the sort keeps 16-bit offsets: larger batches go in chunks
// work: nvalid (+ 3 pad), scattered ids, sorted ids, sorted tokens (nmax each), bucket starts
// (V + 1), then the window pieces (floats) from the next 16-byte boundary
int64_t emb_part_offset(int64_t nmax, int V) { return (4 + 3 * nmax + V + 1 + 3) / 4 * 4; }
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
    int32_t* nvalid = work;
    int32_t* scattered = work + 4;
    int32_t* order = scattered + nmax;
    int32_t* stok = order + nmax;
    int32_t* bstart = stok + nmax;
    float* part = (float*)(work + emb_part_offset(nmax, V));
    for (int64_t r0 = 0; r0 < rows; r0 += EMB_CHUNK) {
        const int64_t n = std::min(EMB_CHUNK, rows - r0);
        const int64_t nwin = cdiv(n, EMB_WIN);
        const int64_t nwaves = nwin * cdiv(C / 4, 64);
        PROF_LAUNCH(KC_EMB_BWD_WTE, 4.0 * n * C + 8.0 * n * C, s, {
            hipLaunchKernelGGL(emb_sort_kernel, dim3(1), dim3(EMB_SORT_THREADS), 0, s, tok + r0, (int)n, V, scattered,
                               stok, bstart, nvalid);
            hipLaunchKernelGGL(emb_rank_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, scattered, stok, bstart,
                               nvalid, order);
            hipLaunchKernelGGL(emb_segsum_kernel, dim3((unsigned)cdiv(nwaves, 4)), dim3(256), 0, s, order, stok,
                               nvalid, dx + r0 * C, C, dwte, part);
            hipLaunchKernelGGL(emb_combine_kernel, dim3((unsigned)nwin, (unsigned)cdiv(C / 4, 64)), dim3(64), 0, s,
                               stok, bstart, nvalid, C, part, dwte);
        });
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    PROF_LAUNCH(KC_EMB_BWD_WPE, 2.0 * rows * C + 8.0 * T * C, s, hipLaunchKernelGGL(embedding_bwd_wpe_kernel, dim3(grid_for((int64_t)T * C)), dim3(256), 0, s, dx, dwpe, B, T, C));
    return hipGetLastError();
}
