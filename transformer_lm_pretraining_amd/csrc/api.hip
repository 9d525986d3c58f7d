// C ABI of libgpt2mi: configuration checks, buffer planning, and the launch
// sequences of the GPT-2 training step (forward, backward, clip + AdamW).
// The model and recipe are those of PDS (see include/gpt2mi.h): pre-LN
// blocks with residuals, causal multi-head attention, GELU MLP, tied and
// padded token table, bf16 activations with fp32 master weights, gradients,
// optimizer state, statistics and loss.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gpt2mi.h"
#include "../../include/gpt2mi_kernels.h"
#include "kernels.h"
#include "prof.h"

namespace {

constexpr int64_t ALIGN = 256;
int64_t align_up(int64_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
bool aligned(const void* p) { return ((uintptr_t)p % ALIGN) == 0; }

struct Tensor {
    std::string name;
    int64_t off, rows, cols;
    bool decayed;
    int64_t toff;  // transposed shadow offset or -1
};

bool config_ok(const gpt2_config* c) {
    if (!c) return false;
    if (c->L < 1 || c->H < 1 || c->C < 128 || c->V < 2 || c->Vp < c->V || c->Tmax < 1 || c->B < 1 || c->T < 1)
        return false;
    if (c->C % c->H) return false;
    const int d = c->C / c->H;
    if (d != 32 && d != 64) return false;
    if (c->C % 128 || c->Vp % 128 || c->Vp > 65536) return false;
    if (c->T > c->Tmax || c->T % 64) return false;
    if (!layernorm_supports(c->C) || 4 * c->C > 8192) return false;
    if ((int64_t)c->B * c->T > (1ll << 30)) return false;
    return true;
}

// Flat layout: decayed 2-D segment first, then the 1-D segment (see gpt2mi.h).
std::vector<Tensor> tensors_of(const gpt2_config& c) {
    std::vector<Tensor> t;
    int64_t off = 0, toff = 0;
    const int64_t C = c.C;
    auto add2 = [&](const std::string& n, int64_t r, int64_t cols, bool transposed) {
        t.push_back({n, off, r, cols, true, transposed ? toff : -1});
        off += r * cols;
        if (transposed) toff += r * cols;
    };
    add2("wte", c.Vp, C, true);
    add2("wpe", c.Tmax, C, false);
    for (int l = 0; l < c.L; ++l) {
        std::string p = "h." + std::to_string(l) + ".";
        add2(p + "attn.c_attn.weight", 3 * C, C, true);
        add2(p + "attn.c_proj.weight", C, C, true);
        add2(p + "mlp.c_fc.weight", 4 * C, C, true);
        add2(p + "mlp.c_proj.weight", C, 4 * C, true);
    }
    auto add1 = [&](const std::string& n, int64_t len) {
        t.push_back({n, off, 1, len, false, -1});
        off += len;
    };
    for (int l = 0; l < c.L; ++l) {
        std::string p = "h." + std::to_string(l) + ".";
        add1(p + "ln_1.weight", C);
        add1(p + "ln_1.bias", C);
        add1(p + "attn.c_attn.bias", 3 * C);
        add1(p + "attn.c_proj.bias", C);
        add1(p + "ln_2.weight", C);
        add1(p + "ln_2.bias", C);
        add1(p + "mlp.c_fc.bias", 4 * C);
        add1(p + "mlp.c_proj.bias", C);
    }
    add1("ln_f.weight", C);
    add1("ln_f.bias", C);
    return t;
}

// Byte offsets of the saved activations and backward temporaries in `acts`.
struct LayerActs {
    int64_t x, ln1, mean1, rstd1, qkv, att, lse, xmid, ln2, mean2, rstd2, gprime, gel;
};
struct ActsPlan {
    std::vector<LayerActs> layer;
    int64_t xfinal, lnf, meanf, rstdf, logits, loss_rows;
    // backward temporaries; each block keeps the gradients its weight-gradient
    // products read (output and x_mid residual gradients, dpre, dqkv) until the
    // products of all blocks run together after the last block
    std::vector<int64_t> d_out, d_mid, d_big, d_qkv;
    int64_t d_in0, d_ln, d_att;
    int64_t total;
};
struct ScratchPlan {
    int64_t flag, loss, scale, norm;  // header slots (256 B)
    int64_t norm_partial, col_partial, splitk, dvec, emb_work, ln_partial;
    int64_t col_partial_elems, splitk_elems, emb_work_elems, ln_slot_elems;
    int64_t total;
};

ActsPlan plan_acts(const gpt2_config& c) {
    ActsPlan a;
    int64_t off = 0;
    const int64_t BT = (int64_t)c.B * c.T, C = c.C;
    auto take = [&](int64_t bytes) {
        int64_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    for (int l = 0; l < c.L; ++l) {
        LayerActs la;
        la.x = take(BT * C * 2);
        la.ln1 = take(BT * C * 2);
        la.mean1 = take(BT * 4);
        la.rstd1 = take(BT * 4);
        la.qkv = take(BT * 3 * C * 2);
        la.att = take(BT * C * 2);
        la.lse = take((int64_t)c.B * c.H * c.T * 4);
        la.xmid = take(BT * C * 2);
        la.ln2 = take(BT * C * 2);
        la.mean2 = take(BT * 4);
        la.rstd2 = take(BT * 4);
        la.gprime = take(BT * 4 * C * 2);  // GELU'(pre), what the FC-proj backward needs of pre
        la.gel = take(BT * 4 * C * 2);
        a.layer.push_back(la);
    }
    a.xfinal = take(BT * C * 2);
    a.lnf = take(BT * C * 2);
    a.meanf = take(BT * 4);
    a.rstdf = take(BT * 4);
    a.logits = take(BT * (int64_t)c.Vp * 2);
    a.loss_rows = take(BT * 4);
    for (int l = 0; l < c.L; ++l) {
        a.d_out.push_back(take(BT * C * 2));
        a.d_mid.push_back(take(BT * C * 2));
        a.d_big.push_back(take(BT * 4 * C * 2));
        a.d_qkv.push_back(take(BT * 3 * C * 2));
    }
    a.d_in0 = take(BT * C * 2);
    a.d_ln = take(BT * C * 2);
    a.d_att = take(BT * C * 2);
    a.total = off;
    return a;
}

// Blocks whose weight-gradient products go out in one grouped call.
constexpr int DW_GROUP_BLOCKS = TN_GROUP_MAX / 4;

// The four weight-gradient products of one block, shapes only.
void block_dw_shapes(const gpt2_config& c, TnJobDesc* jobs) {
    const int C = c.C;
    jobs[0] = {nullptr, C, nullptr, 4 * C, C, 4 * C, nullptr, nullptr};
    jobs[1] = {nullptr, 4 * C, nullptr, C, 4 * C, C, nullptr, nullptr};
    jobs[2] = {nullptr, C, nullptr, C, C, C, nullptr, nullptr};
    jobs[3] = {nullptr, 3 * C, nullptr, C, 3 * C, C, nullptr, nullptr};
}

ScratchPlan plan_scratch(const gpt2_config& c) {
    ScratchPlan s;
    const int64_t BT = (int64_t)c.B * c.T, C = c.C;
    s.flag = 0;
    s.loss = 4;
    s.scale = 8;
    s.norm = 12;
    int64_t off = 256;
    s.norm_partial = off;
    off = align_up(off + adamw_partial_elems(0) * 8);
    s.col_partial_elems = std::max({layernorm_bwd_partial_elems(BT, c.C), colsum_partial_elems(BT, 4 * c.C),
                                    colsum_partial_elems(BT, 3 * c.C)});
    s.col_partial = off;
    off = align_up(off + s.col_partial_elems * 4);
    // column partials of every LayerNorm backward of a step (folded once at its end)
    s.ln_slot_elems = layernorm_bwd_partial_elems(BT, c.C);
    s.ln_partial = off;
    off = align_up(off + s.ln_slot_elems * (2 * c.L + 1) * 4);
    {
        // the blocks' grouped weight-gradient products (chunks of DW_GROUP_BLOCKS
        // blocks, the last one possibly shorter), and the lm_head's
        TnJobDesc blk[4 * DW_GROUP_BLOCKS];
        int64_t part = 0;
        for (int l0 = 0; l0 < c.L; l0 += DW_GROUP_BLOCKS) {
            const int nb = std::min(DW_GROUP_BLOCKS, c.L - l0);
            for (int k = 0; k < nb; ++k) block_dw_shapes(c, blk + 4 * k);
            part = std::max(part, gemm_tn_group_partial_elems(blk, 4 * nb, (int)BT));
        }
        s.splitk_elems = std::max(part,
                                  gemm_tn_partial_elems((int)BT, c.Vp, (int)C));
    }
    s.splitk = off;
    off = align_up(off + s.splitk_elems * 4);
    s.dvec = off;
    off = align_up(off + (int64_t)c.B * c.H * c.T * 4);
    s.emb_work_elems = embedding_bwd_work_elems(BT, c.V, c.C);
    s.emb_work = off;
    off = align_up(off + s.emb_work_elems * 4);
    s.total = off;
    return s;
}

constexpr int PROF_MAX = 65536;

}  // namespace

thread_local ProfSink* g_prof_sink = nullptr;

struct gpt2_handle {
    gpt2_config cfg;
    gpt2_buffers bufs;
    std::vector<Tensor> tens;
    ActsPlan acts;
    ScratchPlan scr;
    int64_t n_params, n_decay;
    // lanes: a lane reads its model's parameters and shadows and owns its grads, acts and scratch
    bool is_lane = false;
    gpt2_handle* parent = nullptr;  // null once the model is destroyed
    std::vector<gpt2_handle*> lanes;
    int last_hip = 0;
    bool grad_ready = false;
    const int32_t* last_tok = nullptr;
    // kernel timing: class filter (0 off, -1 all), event pairs and records
    struct Rec {
        int cls;
        double work;
    };
    struct Sink : ProfSink {
        gpt2_handle* h = nullptr;
        bool active = false, multi = false;
        void begin(int cls, double work, hipStream_t s, bool many) override {
            active = false;
            pend0 = pend1 = nullptr;
            if ((h->prof_class != -1 && h->prof_class != cls) || (int)h->recs.size() >= PROF_MAX) return;
            const size_t n = h->recs.size();
            multi = many;
            if (multi) {
                if (hipEventRecord(h->ev0[n], s) != hipSuccess) return;
            } else {  // recorded by the launch itself at the kernel's start and end
                pend0 = h->ev0[n];
                pend1 = h->ev1[n];
            }
            h->recs.push_back({cls, work});
            active = true;
        }
        void end(int, hipStream_t s) override {
            if (active) {
                if (multi)
                    (void)hipEventRecord(h->ev1[h->recs.size() - 1], s);  // a failed record only loses a timing
                else if (pend0)
                    h->recs.pop_back();  // nothing was launched
            }
            pend0 = pend1 = nullptr;
            active = false;
        }
    } sink;
    int prof_class = 0;
    std::vector<Rec> recs;
    std::vector<hipEvent_t> ev0, ev1;

    char* A() const { return (char*)bufs.acts; }
    char* S() const { return (char*)bufs.scratch; }
    template <class T>
    T* act(int64_t off) const { return (T*)(A() + off); }
    const Tensor& t(int i) const { return tens[i]; }
    // tensor index helpers (flat-layout order)
    int i_wte() const { return 0; }
    int i_wpe() const { return 1; }
    int i_mat(int l, int k) const { return 2 + 4 * l + k; }  // k: 0 qkv, 1 proj, 2 fc, 3 fcproj
    int i_vec(int l, int k) const { return 2 + 4 * cfg.L + 8 * l + k; }  // ln1w ln1b bqkv bproj ln2w ln2b bfc bfp
    int i_lnf(int k) const { return 2 + 12 * cfg.L + k; }
    float* P(int i) const { return bufs.params + tens[i].off; }
    float* G(int i) const { return bufs.grads + tens[i].off; }
    uint16_t* W(int i) const { return bufs.shadow + tens[i].off; }
    uint16_t* WT(int i) const { return bufs.shadow_t + tens[i].toff; }
};

namespace {

// Installs the handle's timing sink for the duration of one API call.
struct SinkGuard {
    ProfSink* prev;
    explicit SinkGuard(gpt2_handle* h) : prev(g_prof_sink) { g_prof_sink = h->prof_class ? &h->sink : nullptr; }
    ~SinkGuard() { g_prof_sink = prev; }
};

#define HIPCHK(expr)                          \
    do {                                      \
        hipError_t e_ = (expr);               \
        if (e_ != hipSuccess) {               \
            if (h) h->last_hip = (int)e_;     \
            return GPT2_E_HIP;                \
        }                                     \
    } while (0)

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GPT2_E_UNSUPPORTED;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GPT2_E_UNSUPPORTED;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GPT2_E_UNSUPPORTED;
    return GPT2_OK;
}

int run_forward(gpt2_handle* h, const int32_t* tok, const int32_t* tgt, float dloss, float* loss_dev, bool train,
                hipStream_t s) {
    const gpt2_config& c = h->cfg;
    const int BT = c.B * c.T, C = c.C;
    int32_t* flag = (int32_t*)(h->S() + h->scr.flag);
    HIPCHK(launch_embedding_fwd(tok, h->W(h->i_wte()), h->W(h->i_wpe()), h->act<uint16_t>(h->acts.layer[0].x), c.B,
                                c.T, C, c.V, flag, s));
    for (int l = 0; l < c.L; ++l) {
        const LayerActs& la = h->acts.layer[l];
        const int64_t xnext = (l + 1 < c.L) ? h->acts.layer[l + 1].x : h->acts.xfinal;
        HIPCHK(launch_layernorm_fwd(h->act<uint16_t>(la.x), h->P(h->i_vec(l, 0)), h->P(h->i_vec(l, 1)),
                                    h->act<uint16_t>(la.ln1), h->act<float>(la.mean1), h->act<float>(la.rstd1), BT,
                                    C, s));
        HIPCHK(launch_gemm_nt(h->act<uint16_t>(la.ln1), C, h->W(h->i_mat(l, 0)), C, BT, 3 * C, C,
                              h->P(h->i_vec(l, 2)), nullptr, 0, h->act<uint16_t>(la.qkv), 3 * C, s));
        HIPCHK(launch_attention_fwd(h->act<uint16_t>(la.qkv), h->act<uint16_t>(la.att), h->act<float>(la.lse), c.B,
                                    c.T, c.H, C, s));
        HIPCHK(launch_gemm_nt(h->act<uint16_t>(la.att), C, h->W(h->i_mat(l, 1)), C, BT, C, C, h->P(h->i_vec(l, 3)),
                              h->act<uint16_t>(la.x), C, h->act<uint16_t>(la.xmid), C, s));
        HIPCHK(launch_layernorm_fwd(h->act<uint16_t>(la.xmid), h->P(h->i_vec(l, 4)), h->P(h->i_vec(l, 5)),
                                    h->act<uint16_t>(la.ln2), h->act<float>(la.mean2), h->act<float>(la.rstd2), BT,
                                    C, s));
        HIPCHK(launch_gemm_nt_gelu(h->act<uint16_t>(la.ln2), C, h->W(h->i_mat(l, 2)), C, BT, 4 * C, C,
                                   h->P(h->i_vec(l, 6)), h->act<uint16_t>(la.gprime), h->act<uint16_t>(la.gel), 4 * C,
                                   s));
        HIPCHK(launch_gemm_nt(h->act<uint16_t>(la.gel), 4 * C, h->W(h->i_mat(l, 3)), 4 * C, BT, C, 4 * C,
                              h->P(h->i_vec(l, 7)), h->act<uint16_t>(la.xmid), C, h->act<uint16_t>(xnext), C, s));
    }
    HIPCHK(launch_layernorm_fwd(h->act<uint16_t>(h->acts.xfinal), h->P(h->i_lnf(0)), h->P(h->i_lnf(1)),
                                h->act<uint16_t>(h->acts.lnf), h->act<float>(h->acts.meanf),
                                h->act<float>(h->acts.rstdf), BT, C, s));
    HIPCHK(launch_gemm_nt(h->act<uint16_t>(h->acts.lnf), C, h->W(h->i_wte()), C, BT, c.Vp, C, nullptr, nullptr, 0,
                          h->act<uint16_t>(h->acts.logits), c.Vp, s));
    if (tgt) {
        HIPCHK(launch_xent(h->act<uint16_t>(h->acts.logits), tgt, h->act<float>(h->acts.loss_rows), BT, c.V, c.Vp,
                           dloss, train ? 1 : 0, flag, s));
        float* ldst = loss_dev ? loss_dev : (float*)(h->S() + h->scr.loss);
        HIPCHK(launch_mean(h->act<float>(h->acts.loss_rows), tgt, BT, ldst, s));
    }
    return GPT2_OK;
}

// Weight-gradient product `which` of block l (its dY tensors: the residual-stream
// gradients at the block output and at x_mid, dpre, dqkv, all kept until the
// products of every block run together after the last block).
TnJobDesc block_dw_job(gpt2_handle* h, int l, int which, const uint16_t* d_out, const uint16_t* d_mid,
                       const uint16_t* d_pre, const uint16_t* d_qkv) {
    const gpt2_config& c = h->cfg;
    const int C = c.C;
    const LayerActs& la = h->acts.layer[l];
    switch (which) {
        case 0:  // FC-proj: x_next = x_mid + gel . W_fp^T + b_fp
            return {d_out, C, h->act<uint16_t>(la.gel), 4 * C, C, 4 * C, h->G(h->i_mat(l, 3)), h->G(h->i_vec(l, 7))};
        case 1:  // FC: pre = ln2 . W_fc^T + b_fc
            return {d_pre, 4 * C, h->act<uint16_t>(la.ln2), C, 4 * C, C, h->G(h->i_mat(l, 2)), h->G(h->i_vec(l, 6))};
        case 2:  // attention projection: x_mid = x + att . W_p^T + b_p
            return {d_mid, C, h->act<uint16_t>(la.att), C, C, C, h->G(h->i_mat(l, 1)), h->G(h->i_vec(l, 3))};
        default:  // QKV: qkv = ln1 . W_qkv^T + b_qkv
            return {d_qkv, 3 * C, h->act<uint16_t>(la.ln1), C, 3 * C, C, h->G(h->i_mat(l, 0)), h->G(h->i_vec(l, 2))};
    }
}

int run_backward(gpt2_handle* h, hipStream_t s) {
    const gpt2_config& c = h->cfg;
    const int BT = c.B * c.T, C = c.C;
    const ActsPlan& A = h->acts;
    float* splitk = (float*)(h->S() + h->scr.splitk);
    const int64_t splitk_n = h->scr.splitk_elems;
    uint16_t* d_ln = h->act<uint16_t>(A.d_ln);
    uint16_t* d_att = h->act<uint16_t>(A.d_att);
    uint16_t* dlogits = h->act<uint16_t>(A.logits);

    // lm_head (tied): d_lnf = dlogits . wte ; dwte += dlogits^T . lnf
    HIPCHK(launch_gemm_nt(dlogits, c.Vp, h->WT(h->i_wte()), c.Vp, BT, C, c.Vp, nullptr, nullptr, 0, d_ln, C, s));
    HIPCHK(launch_gemm_tn_acc(dlogits, c.Vp, h->act<uint16_t>(A.lnf), C, BT, c.Vp, C, h->G(h->i_wte()), nullptr,
                              splitk, splitk_n, s));
    // final LN: the last block's output gradient
    // LayerNorm parameter gradients: each backward leaves its column partials in
    // slot k of ln_partial (dw[k], db[k] are their targets); one fold at the end
    float* lnp = (float*)(h->S() + h->scr.ln_partial);
    const int64_t lns = h->scr.ln_slot_elems;
    std::vector<float*> ln_dw, ln_db;
    auto ln_slot = [&](int iw, int ib) {
        ln_dw.push_back(h->G(iw));
        ln_db.push_back(h->G(ib));
        return lnp + (int64_t)(ln_dw.size() - 1) * lns;
    };
    HIPCHK(launch_layernorm_bwd(h->act<uint16_t>(A.xfinal), d_ln, h->P(h->i_lnf(0)), h->act<float>(A.meanf),
                                h->act<float>(A.rstdf), h->act<uint16_t>(A.d_out[c.L - 1]),
                                h->act<uint16_t>(A.d_out[c.L - 1]), 0, nullptr, nullptr,
                                ln_slot(h->i_lnf(0), h->i_lnf(1)), BT, C, s));
    std::vector<TnJobDesc> jobs(4 * (size_t)c.L);
    for (int l = c.L - 1; l >= 0; --l) {
        const LayerActs& la = A.layer[l];
        uint16_t* d_out = h->act<uint16_t>(A.d_out[l]);                       // gradient at the block output
        uint16_t* d_mid = h->act<uint16_t>(A.d_mid[l]);                       // at x_mid
        uint16_t* d_in = h->act<uint16_t>(l > 0 ? A.d_out[l - 1] : A.d_in0);  // at the block input
        uint16_t* d_big = h->act<uint16_t>(A.d_big[l]);
        uint16_t* d_qkv = h->act<uint16_t>(A.d_qkv[l]);
        // FC-proj input gradient, taken through GELU in the epilogue: d_big = dpre = dgel * GELU'(pre)
        HIPCHK(launch_gemm_nt_dgelu(d_out, C, h->WT(h->i_mat(l, 3)), C, BT, 4 * C, C, h->act<uint16_t>(la.gprime), d_big,
                                    4 * C, s));
        // FC input gradient, then LN2: d_mid = d_out + LN2'(d_ln)
        HIPCHK(launch_gemm_nt(d_big, 4 * C, h->WT(h->i_mat(l, 2)), 4 * C, BT, C, 4 * C, nullptr, nullptr, 0, d_ln, C,
                              s));
        HIPCHK(launch_layernorm_bwd(h->act<uint16_t>(la.xmid), d_ln, h->P(h->i_vec(l, 4)), h->act<float>(la.mean2),
                                    h->act<float>(la.rstd2), d_out, d_mid, 1, nullptr, nullptr,
                                    ln_slot(h->i_vec(l, 4), h->i_vec(l, 5)), BT, C, s));
        // attention projection input gradient, attention, QKV input gradient
        HIPCHK(launch_gemm_nt(d_mid, C, h->WT(h->i_mat(l, 1)), C, BT, C, C, nullptr, nullptr, 0, d_att, C, s));
        HIPCHK(launch_attention_bwd(h->act<uint16_t>(la.qkv), h->act<uint16_t>(la.att), d_att,
                                    h->act<float>(la.lse), d_qkv, (float*)(h->S() + h->scr.dvec), c.B, c.T, c.H, C,
                                    s));
        HIPCHK(launch_gemm_nt(d_qkv, 3 * C, h->WT(h->i_mat(l, 0)), 3 * C, BT, C, 3 * C, nullptr, nullptr, 0, d_ln, C,
                              s));
        // LN1: d_in = d_mid + LN1'(d_ln)
        HIPCHK(launch_layernorm_bwd(h->act<uint16_t>(la.x), d_ln, h->P(h->i_vec(l, 0)), h->act<float>(la.mean1),
                                    h->act<float>(la.rstd1), d_mid, d_in, 1, nullptr, nullptr,
                                    ln_slot(h->i_vec(l, 0), h->i_vec(l, 1)), BT, C, s));
        for (int k = 0; k < 4; ++k) jobs[4 * (size_t)l + k] = block_dw_job(h, l, k, d_out, d_mid, d_big, d_qkv);
    }
    // all blocks' weight and bias gradients, in grouped calls of up to DW_GROUP_BLOCKS blocks
    for (int l0 = 0; l0 < c.L; l0 += DW_GROUP_BLOCKS) {
        const int nb = std::min(DW_GROUP_BLOCKS, c.L - l0);
        HIPCHK(launch_gemm_tn_group(jobs.data() + 4 * (size_t)l0, 4 * nb, BT, splitk, splitk_n, s));
    }
    for (int k0 = 0; k0 < (int)ln_dw.size(); k0 += LN_FOLD_MAX) {
        const int n = std::min(LN_FOLD_MAX, (int)ln_dw.size() - k0);
        HIPCHK(launch_layernorm_fold(lnp + (int64_t)k0 * lns, lns, n, ln_dw.data() + k0, ln_db.data() + k0, BT, C, s));
    }
    HIPCHK(launch_embedding_bwd(h->last_tok, h->act<uint16_t>(A.d_in0), h->G(h->i_wte()), h->G(h->i_wpe()), c.B, c.T, C, c.V,
                                (int32_t*)(h->S() + h->scr.emb_work), h->scr.emb_work_elems, s));
    return GPT2_OK;
}

int refresh_shadow(gpt2_handle* h, hipStream_t s) {
    // bf16 transposed copies of wte and the four matrices per block, one batched launch
    std::vector<const uint16_t*> src;
    std::vector<uint16_t*> dst;
    std::vector<int> rows, cols;
    for (const Tensor& t : h->tens) {
        if (t.toff < 0) continue;
        src.push_back(h->bufs.shadow + t.off);
        dst.push_back(h->bufs.shadow_t + t.toff);
        rows.push_back((int)t.rows);
        cols.push_back((int)t.cols);
    }
    HIPCHK(launch_transpose_bf16_batch(src.data(), dst.data(), rows.data(), cols.data(), (int)src.size(), s));
    return GPT2_OK;
}

}  // namespace

extern "C" {

int gpt2_sizes(const gpt2_config* cfg, gpt2_sizes_t* out) {
    if (!out || !config_ok(cfg)) return GPT2_E_INVALID;
    auto t = tensors_of(*cfg);
    int64_t n = 0, nd = 0, nt = 0;
    for (auto& x : t) {
        n += x.rows * x.cols;
        if (x.decayed) nd += x.rows * x.cols;
        if (x.toff >= 0) nt += x.rows * x.cols;
    }
    out->n_params = n;
    out->n_params_real = n - (int64_t)(cfg->Vp - cfg->V) * cfg->C;
    out->n_decay = nd;
    out->n_shadow_t = nt;
    out->n_tensors = (int64_t)t.size();
    out->acts_bytes = plan_acts(*cfg).total;
    out->scratch_bytes = plan_scratch(*cfg).total;
    return GPT2_OK;
}

int gpt2_tensor_info(const gpt2_config* cfg, int32_t index, gpt2_tensor_info_t* out) {
    if (!out || !config_ok(cfg)) return GPT2_E_INVALID;
    auto t = tensors_of(*cfg);
    if (index < 0 || index >= (int32_t)t.size()) return GPT2_E_INVALID;
    const Tensor& x = t[index];
    std::memset(out, 0, sizeof(*out));
    std::snprintf(out->name, sizeof(out->name), "%s", x.name.c_str());
    out->offset = x.off;
    out->rows = x.rows;
    out->cols = x.cols;
    out->decayed = x.decayed ? 1 : 0;
    out->shadow_t_offset = x.toff;
    return GPT2_OK;
}

int gpt2_init(const gpt2_config* cfg, uint64_t seed, const float* host_init, const gpt2_buffers* bufs,
              hipStream_t s, gpt2_handle** out) {
    gpt2_handle* h = nullptr;
    if (!out || !bufs || !config_ok(cfg)) return GPT2_E_INVALID;
    *out = nullptr;
    const void* ptrs[] = {bufs->params, bufs->grads, bufs->m, bufs->v, bufs->shadow, bufs->shadow_t, bufs->acts,
                          bufs->scratch};
    for (const void* p : ptrs)
        if (!p || !aligned(p)) return GPT2_E_INVALID;
    int dev = check_device();
    if (dev != GPT2_OK) return dev;
    h = new gpt2_handle();
    h->cfg = *cfg;
    h->bufs = *bufs;
    h->tens = tensors_of(*cfg);
    h->acts = plan_acts(*cfg);
    h->scr = plan_scratch(*cfg);
    gpt2_sizes_t sz;
    gpt2_sizes(cfg, &sz);
    h->n_params = sz.n_params;
    h->n_decay = sz.n_decay;
    auto fail = [&](hipError_t e) {
        delete h;
        (void)e;
        return GPT2_E_HIP;
    };
    if (host_init) {
        hipError_t e = hipMemcpyAsync(bufs->params, host_init, sz.n_params * sizeof(float), hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return fail(e);
    } else {
        const double resid_std = 0.02 / std::sqrt(2.0 * cfg->L);
        for (int i = 0; i < (int)h->tens.size(); ++i) {
            const Tensor& t = h->tens[i];
            const int64_t n = t.rows * t.cols;
            hipError_t e;
            if (t.decayed) {
                const bool resid = t.name.size() >= 13 && t.name.compare(t.name.size() - 13, 13, "c_proj.weight") == 0;
                const int64_t zero_from = (i == 0) ? (int64_t)cfg->V * cfg->C : n;
                e = launch_init_normal(bufs->params + t.off, n, seed, i, resid ? resid_std : 0.02, zero_from, s);
            } else {
                const bool gain = t.name.find("ln_") != std::string::npos && t.name.find(".weight") != std::string::npos;
                e = launch_fill_f32(bufs->params + t.off, gain ? 1.0f : 0.0f, n, s);
            }
            if (e != hipSuccess) return fail(e);
        }
    }
    hipError_t e = launch_cast_bf16(bufs->params, bufs->shadow, sz.n_decay, s);
    if (e != hipSuccess) return fail(e);
    if (refresh_shadow(h, s) != GPT2_OK) return fail(hipErrorUnknown);
    for (float* p : {bufs->grads, bufs->m, bufs->v}) {
        e = launch_fill_f32(p, 0.0f, sz.n_params, s);
        if (e != hipSuccess) return fail(e);
    }
    e = hipMemsetAsync(bufs->scratch, 0, 256, s);
    if (e != hipSuccess) return fail(e);
    h->sink.h = h;
    *out = h;
    return GPT2_OK;
}

int gpt2_forward(gpt2_handle* h, const int32_t* tok, const int32_t* tgt, float dloss_scale, float* loss_dev,
                 hipStream_t s) {
    if (!h || !tok) return GPT2_E_INVALID;
    SinkGuard guard(h);
    h->grad_ready = false;
    int r = run_forward(h, tok, tgt, dloss_scale, loss_dev, true, s);
    if (r == GPT2_OK && tgt) {
        h->grad_ready = true;
        h->last_tok = tok;
    }
    return r;
}

int gpt2_backward(gpt2_handle* h, hipStream_t s) {
    if (!h) return GPT2_E_INVALID;
    if (!h->grad_ready) return GPT2_E_STATE;
    SinkGuard guard(h);
    h->grad_ready = false;
    return run_backward(h, s);
}

int gpt2_lane_init(gpt2_handle* h, float* grads, void* acts, void* scratch, hipStream_t s, gpt2_handle** out) {
    if (!out) return GPT2_E_INVALID;
    *out = nullptr;
    if (!h || h->is_lane || !grads || !acts || !scratch || !aligned(grads) || !aligned(acts) || !aligned(scratch))
        return GPT2_E_INVALID;
    if ((int)h->lanes.size() >= GPT2_MAX_LANES) return GPT2_E_STATE;
    // the lane's buffers may not overlap the model's or another lane's (shared gradient
    // accumulators would be counted twice, shared activations or scratch would race)
    struct Span {
        const void* p;
        int64_t n;
    };
    auto spans_of = [](const gpt2_handle* x, std::vector<Span>& v) {
        const int64_t pb = x->n_params * (int64_t)sizeof(float);
        v.push_back({x->bufs.grads, pb});
        v.push_back({x->bufs.acts, x->acts.total});
        v.push_back({x->bufs.scratch, x->scr.total});
        if (!x->is_lane) {
            v.push_back({x->bufs.params, pb});
            v.push_back({x->bufs.m, pb});
            v.push_back({x->bufs.v, pb});
            v.push_back({x->bufs.shadow, x->n_decay * (int64_t)sizeof(uint16_t)});
            int64_t nt = 0;
            for (const Tensor& t : x->tens)
                if (t.toff >= 0) nt += t.rows * t.cols;
            v.push_back({x->bufs.shadow_t, nt * (int64_t)sizeof(uint16_t)});
        }
    };
    std::vector<Span> used;
    spans_of(h, used);
    for (const gpt2_handle* x : h->lanes) spans_of(x, used);
    const Span mine[3] = {{grads, h->n_params * (int64_t)sizeof(float)}, {acts, h->acts.total}, {scratch, h->scr.total}};
    auto overlap = [](const Span& a, const Span& b) {
        const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
        return a0 < b0 + (uintptr_t)b.n && b0 < a0 + (uintptr_t)a.n;
    };
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlap(mine[i], mine[j])) return GPT2_E_INVALID;
        for (const Span& u : used)
            if (overlap(mine[i], u)) return GPT2_E_INVALID;
    }
    gpt2_handle* l = new gpt2_handle();
    l->cfg = h->cfg;
    l->bufs = h->bufs;
    l->bufs.grads = grads;
    l->bufs.acts = acts;
    l->bufs.scratch = scratch;
    l->tens = h->tens;
    l->acts = h->acts;
    l->scr = h->scr;
    l->n_params = h->n_params;
    l->n_decay = h->n_decay;
    l->is_lane = true;
    l->parent = h;
    hipError_t e = launch_fill_f32(grads, 0.0f, l->n_params, s);
    if (e == hipSuccess) e = hipMemsetAsync(scratch, 0, 256, s);
    if (e != hipSuccess) {
        h->last_hip = (int)e;
        delete l;
        return GPT2_E_HIP;
    }
    l->sink.h = l;
    h->lanes.push_back(l);
    *out = l;
    return GPT2_OK;
}

int gpt2_clip_adamw(gpt2_handle* h, const gpt2_adamw_args* a, float* grad_norm_dev, hipStream_t s) {
    if (!h || !a || a->t < 1 || !(a->max_norm > 0.0f)) return GPT2_E_INVALID;
    if (h->is_lane) return GPT2_E_STATE;
    SinkGuard guard(h);
    AdamwHostArgs ha;
    ha.lr = a->lr;
    ha.beta1 = a->beta1;
    ha.beta2 = a->beta2;
    ha.eps = a->eps;
    ha.wd = a->weight_decay;
    ha.max_norm = a->max_norm;
    ha.inv_bc1 = (float)(1.0 / (1.0 - std::pow((double)a->beta1, (double)a->t)));
    ha.inv_bc2 = (float)(1.0 / (1.0 - std::pow((double)a->beta2, (double)a->t)));
    float* g[GPT2_MAX_LANES + 1];
    int ng = 0;
    g[ng++] = h->bufs.grads;
    for (gpt2_handle* l : h->lanes) g[ng++] = l->bufs.grads;
    HIPCHK(launch_clip_adamw(h->bufs.params, g, ng, h->bufs.m, h->bufs.v, h->bufs.shadow, h->n_params, h->n_decay, ha,
                             grad_norm_dev, (double*)(h->S() + h->scr.norm_partial),
                             (float*)(h->S() + h->scr.scale), s));
    return refresh_shadow(h, s);
}

int gpt2_eval_loss(gpt2_handle* h, const int32_t* tok, const int32_t* tgt, float* loss_host, hipStream_t s) {
    if (!h || !tok || !tgt || !loss_host) return GPT2_E_INVALID;
    h->grad_ready = false;
    float* dev_loss = (float*)(h->S() + h->scr.loss);
    int r;
    {
        SinkGuard guard(h);
        r = run_forward(h, tok, tgt, 0.0f, dev_loss, false, s);
    }
    if (r != GPT2_OK) return r;
    HIPCHK(hipMemcpyAsync(loss_host, dev_loss, sizeof(float), hipMemcpyDeviceToHost, s));
    return gpt2_sync_status(h, s);
}

int gpt2_sync_status(gpt2_handle* h, hipStream_t s) {
    if (!h) return GPT2_E_INVALID;
    int32_t flag = 0;
    HIPCHK(hipMemcpyAsync(&flag, h->S() + h->scr.flag, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    if (flag) {
        HIPCHK(hipMemsetAsync(h->S() + h->scr.flag, 0, sizeof(int32_t), s));
        HIPCHK(hipStreamSynchronize(s));
        return GPT2_E_DATA;
    }
    return GPT2_OK;
}

const uint16_t* gpt2_logits_ptr(const gpt2_handle* h) { return h ? h->act<uint16_t>(h->acts.logits) : nullptr; }
const float* gpt2_row_loss_ptr(const gpt2_handle* h) { return h ? h->act<float>(h->acts.loss_rows) : nullptr; }
const uint16_t* gpt2_residual_ptr(const gpt2_handle* h, int32_t l) {
    if (!h || l < 0 || l > h->cfg.L) return nullptr;
    return h->act<uint16_t>(l == h->cfg.L ? h->acts.xfinal : h->acts.layer[l].x);
}
int gpt2_last_hip_error(const gpt2_handle* h) { return h ? h->last_hip : 0; }

void gpt2_destroy(gpt2_handle* h) {
    if (!h) return;
    if (h->parent) {
        auto& v = h->parent->lanes;
        v.erase(std::remove(v.begin(), v.end(), h), v.end());
    }
    for (gpt2_handle* l : h->lanes) l->parent = nullptr;
    for (auto e : h->ev0) (void)hipEventDestroy(e);  // nothing to report from a destructor
    for (auto e : h->ev1) (void)hipEventDestroy(e);
    delete h;
}

const char* gpt2_strerror(int st) {
    switch (st) {
        case GPT2_OK: return "ok";
        case GPT2_E_INVALID: return "invalid argument or configuration";
        case GPT2_E_SHAPE: return "unsupported shape";
        case GPT2_E_STATE: return "call order violated";
        case GPT2_E_HIP: return "HIP runtime error";
        case GPT2_E_DATA: return "token or target id outside [0, V)";
        case GPT2_E_UNSUPPORTED: return "no gfx950 GPU";
    }
    return "unknown status";
}

int gpt2_prof_enable(gpt2_handle* h, int32_t kclass) {
    if (!h || kclass < -1 || kclass >= KC_COUNT) return GPT2_E_INVALID;
    if (kclass != 0 && h->ev0.empty()) {
        h->ev0.resize(PROF_MAX);
        h->ev1.resize(PROF_MAX);
        for (int i = 0; i < PROF_MAX; ++i) {
            HIPCHK(hipEventCreate(&h->ev0[i]));
            HIPCHK(hipEventCreate(&h->ev1[i]));
        }
    }
    h->prof_class = kclass;
    h->recs.clear();
    return GPT2_OK;
}

int gpt2_prof_read(gpt2_handle* h, hipStream_t s, int32_t kclass, double* total_ms, int64_t* launches,
                   double* work) {
    if (!h || !total_ms || !launches || !work) return GPT2_E_INVALID;
    HIPCHK(hipStreamSynchronize(s));
    double tot = 0.0, wk = 0.0;
    int64_t n = 0;
    for (size_t i = 0; i < h->recs.size(); ++i) {
        if (kclass != -1 && h->recs[i].cls != kclass) continue;
        float ms = 0.f;
        HIPCHK(hipEventElapsedTime(&ms, h->ev0[i], h->ev1[i]));
        tot += ms;
        wk += h->recs[i].work;
        ++n;
    }
    *total_ms = tot;
    *launches = n;
    *work = wk;
    return GPT2_OK;
}

const char* gpt2_prof_class_name(int32_t kclass) {
    static const char* names[KC_COUNT] = {
        "none", "gemm_nt", "gemm_nt_gelu", "gemm_tn_acc", "gemm_tn_splitk", "splitk_reduce", "attn_fwd",
        "attn_dvec", "attn_dkdv", "attn_dq", "xent", "layernorm_fwd", "layernorm_bwd", "fold_partials",
        "bias_gelu_bwd", "colsum", "embedding_fwd", "embedding_bwd_wte", "embedding_bwd_wpe", "sumsq",
        "norm_finalize", "adamw", "transpose_bf16", "mean", "bias_gelu_fwd", "gemm_nt_dgelu", "other"};
    return (kclass >= 0 && kclass < KC_COUNT) ? names[kclass] : nullptr;
}

// ---------------------------------------------------------------- kernel-level entry points

#define KCHK(expr)                                            \
    do {                                                      \
        hipError_t e_ = (expr);                               \
        if (e_ == hipErrorInvalidValue) return GPT2_E_SHAPE;  \
        if (e_ != hipSuccess) return GPT2_E_HIP;              \
    } while (0)

int gpt2k_scratch_bytes(int32_t kind, int64_t a, int64_t b, int64_t c, int64_t* out) {
    if (!out || a < 0 || b < 0 || c < 0) return GPT2_E_INVALID;
    switch (kind) {
        case 1: *out = layernorm_bwd_partial_elems(a, (int)b) * 4; return GPT2_OK;
        case 2: *out = colsum_partial_elems(a, (int)b) * 4; return GPT2_OK;
        case 3: *out = gemm_tn_partial_elems((int)a, (int)b, (int)c) * 4; return GPT2_OK;
        case 4: *out = adamw_partial_elems(a) * 8 + 256; return GPT2_OK;
        case 5: *out = embedding_bwd_work_elems(a, (int)b, (int)c) * 4; return GPT2_OK;
    }
    return GPT2_E_INVALID;
}

int gpt2k_xent(uint16_t* logits, const int32_t* tgt, float* loss_rows, int64_t rows, int32_t V, int32_t Vp,
               float dloss, int32_t write_grad, int32_t* flag, hipStream_t s) {
    if (!logits || !tgt || !loss_rows || rows < 0 || V < 1 || V > Vp || Vp % 128 || Vp > 65536)
        return GPT2_E_INVALID;
    KCHK(launch_xent(logits, tgt, loss_rows, rows, V, Vp, dloss, write_grad, flag, s));
    return GPT2_OK;
}

int gpt2k_layernorm_fwd(const uint16_t* x, const float* w, const float* b, uint16_t* y, float* mean, float* rstd,
                        int64_t rows, int32_t C, hipStream_t s) {
    if (!x || !w || !b || !y || !mean || !rstd || rows < 0) return GPT2_E_INVALID;
    if (!layernorm_supports(C)) return GPT2_E_SHAPE;
    KCHK(launch_layernorm_fwd(x, w, b, y, mean, rstd, rows, C, s));
    return GPT2_OK;
}

int gpt2k_layernorm_bwd(const uint16_t* x, const uint16_t* dy, const float* w, const float* mean, const float* rstd,
                        uint16_t* dres, int32_t accumulate, float* dw, float* db, void* scratch,
                        int64_t scratch_bytes, int64_t rows, int32_t C, hipStream_t s) {
    if (!x || !dy || !w || !mean || !rstd || !dres || !dw || !db || !scratch || rows < 0) return GPT2_E_INVALID;
    if (!layernorm_supports(C)) return GPT2_E_SHAPE;
    if (scratch_bytes < layernorm_bwd_partial_elems(rows, C) * 4) return GPT2_E_INVALID;
    KCHK(launch_layernorm_bwd(x, dy, w, mean, rstd, dres, dres, accumulate, dw, db, (float*)scratch, rows, C, s));
    return GPT2_OK;
}

int gpt2k_bias_gelu_fwd(const uint16_t* u, const float* b, uint16_t* pre, uint16_t* g, int64_t rows, int32_t N,
                        hipStream_t s) {
    if (!u || !b || !pre || !g || rows < 0 || N <= 0 || N % 8) return GPT2_E_INVALID;
    KCHK(launch_bias_gelu_fwd(u, b, pre, g, rows, N, s));
    return GPT2_OK;
}

int gpt2k_bias_gelu_bwd(const uint16_t* pre, const uint16_t* dg, uint16_t* dpre, float* db, void* scratch,
                        int64_t scratch_bytes, int64_t rows, int32_t N, hipStream_t s) {
    if (!pre || !dg || !dpre || !db || !scratch || rows < 0 || N <= 0 || N % 8) return GPT2_E_INVALID;
    if (scratch_bytes < colsum_partial_elems(rows, N) * 4) return GPT2_E_INVALID;
    KCHK(launch_bias_gelu_bwd(pre, dg, dpre, db, (float*)scratch, rows, N, s));
    return GPT2_OK;
}

int gpt2k_bias_grad(const uint16_t* dY, float* db, void* scratch, int64_t scratch_bytes, int64_t M, int32_t N,
                    hipStream_t s) {
    if (!dY || !db || !scratch || M < 0 || N <= 0 || N % 8) return GPT2_E_INVALID;
    if (scratch_bytes < colsum_partial_elems(M, N) * 4) return GPT2_E_INVALID;
    KCHK(launch_bias_grad(dY, N, db, (float*)scratch, M, N, s));
    return GPT2_OK;
}

int gpt2k_gemm_nt(const uint16_t* A, const uint16_t* B, const float* bias, const uint16_t* res, uint16_t* out,
                  int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (!A || !B || !out || M < 1 || N < 1 || K < 64 || K % 64 || N % 8 || M > INT32_MAX || N > INT32_MAX)
        return GPT2_E_INVALID;
    KCHK(launch_gemm_nt(A, K, B, K, (int)M, (int)N, (int)K, bias, res, N, out, N, s));
    return GPT2_OK;
}

int gpt2k_gemm_nt_gelu(const uint16_t* A, const uint16_t* B, const float* bias, uint16_t* gprime, uint16_t* g,
                       int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (!A || !B || !bias || !gprime || !g || M < 1 || N < 1 || K < 64 || K % 64 || N % 8 || M > INT32_MAX)
        return GPT2_E_INVALID;
    KCHK(launch_gemm_nt_gelu(A, K, B, K, (int)M, (int)N, (int)K, bias, gprime, g, N, s));
    return GPT2_OK;
}

int gpt2k_gemm_nt_dgelu(const uint16_t* A, const uint16_t* B, const uint16_t* gprime, uint16_t* out, int64_t M,
                        int64_t N, int64_t K, hipStream_t s) {
    if (!A || !B || !gprime || !out || M < 1 || N < 1 || K < 64 || K % 64 || N % 8 || M > INT32_MAX)
        return GPT2_E_INVALID;
    KCHK(launch_gemm_nt_dgelu(A, K, B, K, (int)M, (int)N, (int)K, gprime, out, N, s));
    return GPT2_OK;
}

int gpt2k_gemm_tn_acc(const uint16_t* dY, const uint16_t* X, float* dW, float* db, void* scratch,
                      int64_t scratch_bytes, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (!dY || !X || !dW || M < 64 || M % 64 || N < 8 || N % 8 || K < 8 || K % 8 || M > INT32_MAX)
        return GPT2_E_INVALID;
    KCHK(launch_gemm_tn_acc(dY, N, X, K, (int)M, (int)N, (int)K, dW, db, (float*)scratch,
                            scratch ? scratch_bytes / 4 : 0,
                            s));
    return GPT2_OK;
}

int gpt2k_attention_fwd(const uint16_t* qkv, uint16_t* out, float* lse, int32_t B, int32_t T, int32_t H, int32_t C,
                        hipStream_t s) {
    if (!qkv || !out || !lse || B < 1 || T < 64 || T % 64 || H < 1 || C % H) return GPT2_E_INVALID;
    if (C / H != 32 && C / H != 64) return GPT2_E_SHAPE;
    KCHK(launch_attention_fwd(qkv, out, lse, B, T, H, C, s));
    return GPT2_OK;
}

int gpt2k_attention_bwd(const uint16_t* qkv, const uint16_t* out, const uint16_t* dout, const float* lse,
                        uint16_t* dqkv, float* dvec, int32_t B, int32_t T, int32_t H, int32_t C, hipStream_t s) {
    if (!qkv || !out || !dout || !lse || !dqkv || !dvec || B < 1 || T < 64 || T % 64 || H < 1 || C % H)
        return GPT2_E_INVALID;
    if (C / H != 32 && C / H != 64) return GPT2_E_SHAPE;
    KCHK(launch_attention_bwd(qkv, out, dout, lse, dqkv, dvec, B, T, H, C, s));
    return GPT2_OK;
}

int gpt2k_clip_adamw(float* p, float* g, float* m, float* v, uint16_t* shadow, int64_t n, int64_t n_decay,
                     const gpt2_adamw_args* a, float* norm_dev, void* scratch, int64_t scratch_bytes,
                     hipStream_t s) {
    if (!p || !g || !m || !v || !a || !scratch || n < 4 || n % 4 || n_decay < 0 || n_decay > n || n_decay % 4 ||
        a->t < 1 || !(a->max_norm > 0.0f))
        return GPT2_E_INVALID;
    if (scratch_bytes < adamw_partial_elems(n) * 8 + 256) return GPT2_E_INVALID;
    AdamwHostArgs ha{a->lr, a->beta1, a->beta2, a->eps, a->weight_decay, a->max_norm,
                     (float)(1.0 / (1.0 - std::pow((double)a->beta1, (double)a->t))),
                     (float)(1.0 / (1.0 - std::pow((double)a->beta2, (double)a->t)))};
    char* sc = (char*)scratch;
    KCHK(launch_clip_adamw(p, g, m, v, shadow, n, n_decay, ha, norm_dev, (double*)(sc + 256), (float*)sc, s));
    return GPT2_OK;
}

int gpt2k_embedding_fwd(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, uint16_t* x, int32_t B,
                        int32_t T, int32_t C, int32_t V, int32_t* flag, hipStream_t s) {
    if (!tok || !wte || !wpe || !x || B < 1 || T < 1 || C < 8 || C % 8 || V < 1) return GPT2_E_INVALID;
    KCHK(launch_embedding_fwd(tok, wte, wpe, x, B, T, C, V, flag, s));
    return GPT2_OK;
}

int gpt2k_embedding_bwd(const int32_t* tok, const uint16_t* dx, float* dwte, float* dwpe, int32_t B, int32_t T,
                        int32_t C, int32_t V, void* scratch, int64_t scratch_bytes, hipStream_t s) {
    if (!tok || !dx || !dwte || !dwpe || !scratch || B < 1 || T < 1 || C < 8 || C % 8 || V < 1 ||
        (int64_t)B * T > INT32_MAX)
        return GPT2_E_INVALID;
    if (scratch_bytes < embedding_bwd_work_elems((int64_t)B * T, V, C) * 4) return GPT2_E_SHAPE;
    KCHK(launch_embedding_bwd(tok, dx, dwte, dwpe, B, T, C, V, (int32_t*)scratch, scratch_bytes / 4, s));
    return GPT2_OK;
}

}  // extern "C"
