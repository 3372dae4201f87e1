// gpt2_api.hip - the C ABI of include/gpt2.h: buffer planning, argument and
// state checks, and the kernel schedule of one GPT-2 micro-step.
//
// The schedule is train_gpt2.cu's gpt2_forward / gpt2_backward / gpt2_update
// with these MI355X-side changes:
//  - bias, GELU and residual additions are epilogues of the matrix products
//    (no attproj / fcproj / residual / gelu round trips through HBM);
//  - attention never materialises the (B, NH, T, T) matrices; it keeps one
//    fp32 log-sum-exp per query row for the backward;
//  - the residual-stream gradient is fp32 (plus a bf16 copy as the next
//    products' operand in bf16 mode) and parameter gradients are fp32;
//  - every reduction is deterministic (no atomics), so two identical calls
//    give bit-identical results;
//  - the mean loss is reduced on the device (no device-to-host copy inside
//    the step).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "gpt2.h"
#include "kernels.h"

namespace {

constexpr int kPlanCUs = 256;  // split-K planning constant (MI355X: 256 CUs)
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p) { return ((uintptr_t)p % kAlign) == 0; }

struct Plan {
    // element counts
    size_t BT, C, L, Vp, NH, T, B;
    int esz;
    // byte offsets into acts
    size_t enc, ln1, ln1m, ln1r, qkv, atty, lse, res2, ln2, ln2m, ln2r, fch, fchg, res3;
    size_t lnf, lnfm, lnfr, logits, losses, tok;
    size_t dres32, dres_lp, dbtc, dbt4c, dqkv, delta;
    size_t acts_bytes;
    // per-layer strides (bytes)
    size_t s_btc, s_bt3c, s_bt4c, s_bt, s_lse;
    // scratch
    size_t flag, work, work_bytes, lnpart, scratch_bytes;
};

void param_layout(const gpt2_config& c, size_t off[16], size_t cnt[16], size_t* total) {
    const size_t Vp = c.padded_vocab_size, C = c.channels, maxT = c.max_seq_len, L = c.num_layers;
    const size_t n[16] = {Vp * C, maxT * C, L * C, L * C, L * 3 * C * C, L * 3 * C, L * C * C, L * C,
                          L * C, L * C, L * 4 * C * C, L * 4 * C, L * C * 4 * C, L * C, C, C};
    size_t t = 0;
    for (int i = 0; i < 16; i++) {
        off[i] = t;
        cnt[i] = n[i];
        t += n[i];
    }
    *total = t;
}

int check_config(const gpt2_config* cfg, int precision, int B, int T) {
    if (!cfg) return GPT2_E_ARG;
    if (precision != GPT2_FP32 && precision != GPT2_BF16 && precision != GPT2_BF16_SR) return GPT2_E_ARG;
    if (cfg->num_layers < 1 || cfg->num_heads < 1 || cfg->channels < 1 || cfg->vocab_size < 1 ||
        cfg->max_seq_len < 1 || cfg->padded_vocab_size < cfg->vocab_size)
        return GPT2_E_ARG;
    if (B < 1 || T < 1 || T > cfg->max_seq_len) return GPT2_E_SHAPE;
    if (cfg->channels % cfg->num_heads) return GPT2_E_SHAPE;
    const int hs = cfg->channels / cfg->num_heads;
    if (hs != 16 && hs != 32 && hs != 64 && hs != 128) return GPT2_E_SHAPE;
    if (cfg->channels % 8 || cfg->channels > 2048 || cfg->padded_vocab_size % 8) return GPT2_E_SHAPE;
    if (cfg->padded_vocab_size > 53248) return GPT2_E_SHAPE;
    if ((long)B * T > (1L << 30) / 4) return GPT2_E_SHAPE;
    return GPT2_OK;
}

// split-K workspace of dW[OC,IC] += dY^T X (M=OC, N=IC, K=BT; fp32 mode,
// where the weight gradients are separate launches) and of dX[BT,IC] = dY W
// (M=BT, N=IC, K=OC)
size_t dw_workspace(size_t OC, size_t IC, size_t BT, int esz) {
    GemmDesc d = {};
    d.M = (int)OC; d.N = (int)IC; d.K = (int)BT; d.ldc = (long)IC; d.epi = GEMM_ACCUM; d.split_ok = 1;
    return gemm_workspace_bytes(d, esz, kPlanCUs);
}
size_t fwd_workspace(size_t BT, size_t OC, size_t IC, int esz, int epi) {
    GemmDesc d = {};
    d.M = (int)BT; d.N = (int)OC; d.K = (int)IC; d.ldc = (long)OC; d.ldaux = (long)OC; d.epi = epi;
    d.a_kmajor = 1; d.b_kmajor = 1;
    d.split_ok = esz == 4;
    return gemm_workspace_bytes(d, esz, kPlanCUs);
}
size_t dx_workspace(size_t BT, size_t IC, size_t OC, int esz, int epi) {
    GemmDesc d = {};
    d.M = (int)BT; d.N = (int)IC; d.K = (int)OC; d.ldc = (long)IC; d.ldaux = (long)IC; d.epi = epi; d.split_ok = 1;
    d.a_kmajor = 1; d.b_kmajor = 0;  // the layout of dx_desc: the chooser's speeds depend on it
    return gemm_workspace_bytes(d, esz, kPlanCUs);
}

Plan make_plan(const gpt2_config& c, int precision, int B, int T) {
    Plan p;
    p.esz = precision == GPT2_FP32 ? 4 : 2;
    p.B = B; p.T = T; p.BT = (size_t)B * T; p.C = c.channels; p.L = c.num_layers;
    p.Vp = c.padded_vocab_size; p.NH = c.num_heads;
    const size_t e = p.esz, BT = p.BT, C = p.C, L = p.L;
    p.s_btc = align_up(BT * C * e);
    p.s_bt3c = align_up(BT * 3 * C * e);
    p.s_bt4c = align_up(BT * 4 * C * e);
    p.s_bt = align_up(BT * 4);
    p.s_lse = align_up((size_t)B * p.NH * T * 4);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += align_up(bytes); return r; };
    p.enc = take(p.s_btc);
    p.ln1 = take(L * p.s_btc);
    p.ln1m = take(L * p.s_bt);
    p.ln1r = take(L * p.s_bt);
    p.qkv = take(L * p.s_bt3c);
    p.atty = take(L * p.s_btc);
    p.lse = take(L * p.s_lse);
    p.res2 = take(L * p.s_btc);
    p.ln2 = take(L * p.s_btc);
    p.ln2m = take(L * p.s_bt);
    p.ln2r = take(L * p.s_bt);
    p.fch = take(L * p.s_bt4c);
    p.fchg = take(L * p.s_bt4c);
    p.res3 = take(L * p.s_btc);
    p.lnf = take(p.s_btc);
    p.lnfm = take(p.s_bt);
    p.lnfr = take(p.s_bt);
    p.logits = take(BT * p.Vp * e);
    p.losses = take(BT * 4);
    p.tok = take(BT * 4);
    p.dres32 = take(BT * C * 4);
    // In bf16 mode every layer's weight gradients run in one launch at the
    // end of the backward pass, so the output gradients they read are kept
    // per layer: the residual gradient's bf16 copy entering fcproj (slot 2l)
    // and entering attproj (slot 2l + 1), fc's pre-activation gradient and
    // the qkv gradient.  In fp32 mode one buffer of each is reused.
    const bool keep = precision != GPT2_FP32;
    p.dres_lp = keep ? take(2 * L * p.s_btc) : p.dres32;
    p.dbtc = take(p.s_btc);
    p.dbt4c = take((keep ? L : 1) * p.s_bt4c);
    p.dqkv = take((keep ? L : 1) * p.s_bt3c);
    p.delta = take(p.s_lse);
    p.acts_bytes = o;
    // scratch: device flag, a workspace shared (in stream order) by the
    // split-K partials (of every product that may split) and the
    // encoder-backward sort, and the partial column
    // sums of all 2L + 1 LayerNorm backwards of a pass (summed by one launch
    // after the last of them)
    size_t w = 0;
    w = std::max(w, fwd_workspace(BT, 3 * C, C, p.esz, GEMM_BIAS));
    w = std::max(w, fwd_workspace(BT, C, C, p.esz, GEMM_BIAS_RESID));
    w = std::max(w, fwd_workspace(BT, 4 * C, C, p.esz, GEMM_BIAS_GELU));
    w = std::max(w, fwd_workspace(BT, C, 4 * C, p.esz, GEMM_BIAS_RESID));
    w = std::max(w, fwd_workspace(BT, p.Vp, C, p.esz, GEMM_STORE));
    w = std::max(w, dx_workspace(BT, C, p.Vp, p.esz, GEMM_STORE));
    w = std::max(w, dx_workspace(BT, 4 * C, C, p.esz, GEMM_GELU_BWD));
    w = std::max(w, dx_workspace(BT, C, 4 * C, p.esz, GEMM_STORE));
    w = std::max(w, dx_workspace(BT, C, C, p.esz, GEMM_STORE));
    w = std::max(w, dx_workspace(BT, C, 3 * C, p.esz, GEMM_STORE));
    w = std::max(w, encoder_bwd_workspace_bytes((int)BT, (int)C));
    if (!keep) {
        w = std::max(w, dw_workspace(p.Vp, C, BT, p.esz));
        w = std::max(w, dw_workspace(3 * C, C, BT, p.esz));
        w = std::max(w, dw_workspace(C, C, BT, p.esz));
        w = std::max(w, dw_workspace(4 * C, C, BT, p.esz));
        w = std::max(w, dw_workspace(C, 4 * C, BT, p.esz));
    }
    p.flag = 0;
    p.work = kAlign;
    p.work_bytes = align_up(w);
    p.lnpart = p.work + p.work_bytes;
    p.scratch_bytes = p.lnpart + align_up((2 * L + 1) * (size_t)layernorm_bwd_partial_rows((int)BT, (int)C, (int)e) * 2 * C * 4);
    return p;
}

}  // namespace

struct gpt2_ctx {
    gpt2_config cfg;
    int prec;              // arithmetic of the kernels: GPT2_FP32 or GPT2_BF16
    bool sr = false;       // GPT2_BF16_SR: no master weights, stochastic rounding
    uint64_t rng = 13371337;  // xorshift64* state of the rounding seeds
    int B, T;
    size_t P;
    size_t off[16], cnt[16];
    gpt2_buffers buf;
    Plan plan;
    int last_fwd_targets;  // -1: no forward yet, 0: without targets, 1: with
    float dw_alpha = 1.0f;  // the classifier weight gradient's scale in the current backward
    // timing hooks around the launches of each point (caller-owned events)
    struct Hook {
        void* const* start = nullptr;
        void* const* end = nullptr;
        int n = 0, i = 0;
    } hooks[GPT2_TP_COUNT];
    char* acts() const { return (char*)buf.acts; }
    template <typename X> X* act(size_t ofs) const { return (X*)(acts() + ofs); }
    template <typename X> X* act_l(size_t ofs, size_t stride, int l) const { return (X*)(acts() + ofs + stride * l); }
    int* flag() const { return (int*)((char*)buf.scratch + plan.flag); }
    float* work() const { return (float*)((char*)buf.scratch + plan.work); }
    float* lnpart(int slot) const {
        return (float*)((char*)buf.scratch + plan.lnpart) +
               (size_t)slot * layernorm_bwd_partial_rows((int)plan.BT, (int)plan.C, plan.esz) * 2 * plan.C;
    }
};

namespace {

int hip_rc(int e) { return e == 0 ? GPT2_OK : GPT2_E_HIP; }

// Runs launch(), bracketed by the timing hook of `point` if one is set.
template <typename F>
int timed(gpt2_ctx* c, int point, hipStream_t s, F&& launch) {
    gpt2_ctx::Hook& h = c->hooks[point];
    const int k = h.n > 0 ? h.i++ % h.n : -1;
    if (k >= 0 && hipEventRecord((hipEvent_t)h.start[k], s) != hipSuccess) return GPT2_E_HIP;
    const int e = launch();
    if (e != 0) return e;
    if (k >= 0 && hipEventRecord((hipEvent_t)h.end[k], s) != hipSuccess) return GPT2_E_HIP;
    return 0;
}

// train_gpt2.cu, random_u32: Marsaglia's xorshift on 64 bits with the
// xorshift* output multiplier, upper 32 bits of the product
uint32_t xorshift_u32(uint64_t* st) {
    uint64_t x = *st;
    x ^= x >> 12;
    x ^= x << 25;
    x ^= x >> 27;
    *st = x;
    return (uint32_t)((x * 0x2545F4914F6CDD1DULL) >> 32);
}
#define TRY(x) do { int _e = (x); if (_e != 0) return GPT2_E_HIP; } while (0)

template <typename T>
T* prm(gpt2_ctx* c, int i, size_t l = 0, size_t per = 0) { return (T*)c->buf.params + c->off[i] + l * per; }
float* grd(gpt2_ctx* c, int i, size_t l = 0, size_t per = 0) { return (float*)c->buf.grads + c->off[i] + l * per; }

// Y[M, N] = X[M, K] W[N, K]^T with the epilogue; fp32 products may split K
// (their epilogue then runs in the reduction), bf16 ones do not
GemmDesc fwd_desc(int M, int N, int K, const void* X, const void* W, void* Y, int epi, const void* bias,
                  const void* aux_in, void* aux_out, int esz) {
    GemmDesc d = {};
    d.M = M; d.N = N; d.K = K;
    d.A = X; d.lda = K; d.a_kmajor = 1;
    d.B = W; d.ldb = K; d.b_kmajor = 1;
    d.C = Y; d.ldc = N; d.epi = epi; d.alpha = 1.0f;
    d.bias = bias; d.aux_in = aux_in; d.aux_out = aux_out; d.ldaux = N;
    d.split_ok = esz == 4;
    return d;
}
// dX[BT, IC] = alpha * dY[BT, OC] W[OC, IC]
GemmDesc dx_desc(int BT, int IC, int OC, const void* dY, const void* W, void* dX, int epi, const void* aux_in,
                 float alpha) {
    GemmDesc d = {};
    d.M = BT; d.N = IC; d.K = OC;
    d.A = dY; d.lda = OC; d.a_kmajor = 1;
    d.B = W; d.ldb = IC; d.b_kmajor = 0;
    d.C = dX; d.ldc = IC; d.epi = epi; d.alpha = alpha;
    d.aux_in = aux_in; d.ldaux = IC;
    d.split_ok = 1;
    return d;
}
// dW[OC, IC] += alpha * dY[BT, OC]^T X[BT, IC]; db[OC] += alpha * column sums of dY (db may be NULL)
GemmDesc dw_desc(int BT, int IC, int OC, const void* dY, const void* X, float* dW, float alpha, float* db) {
    GemmDesc d = {};
    d.M = OC; d.N = IC; d.K = BT;
    d.A = dY; d.lda = OC; d.a_kmajor = 0;
    d.B = X; d.ldb = IC; d.b_kmajor = 0;
    d.C = dW; d.ldc = IC; d.epi = GEMM_ACCUM; d.alpha = alpha;
    d.dbias = db;
    d.split_ok = 1;
    return d;
}

int gemm(gpt2_ctx* c, const GemmDesc& d, hipStream_t s, int cus = kPlanCUs) {
    return gemm_launch(d, c->plan.esz, c->work(), c->plan.work_bytes, cus, s);
}

template <typename T>
int forward_impl(gpt2_ctx* c, const int32_t* inputs, const int32_t* targets, float* d_losses, float* d_mean,
                 hipStream_t s) {
    const Plan& p = c->plan;
    const int B = c->B, Tn = c->T, BT = (int)p.BT, C = (int)p.C, L = (int)p.L, NH = (int)p.NH;
    const int V = c->cfg.vocab_size, Vp = (int)p.Vp;
    const size_t CC = (size_t)C * C;
    T* enc = c->act<T>(p.enc);
    TRY(encoder_fwd_launch<T>(enc, c->act<int>(p.tok), inputs, prm<T>(c, 0), prm<T>(c, 1), B, Tn, C, V, c->flag(), s));
    for (int l = 0; l < L; l++) {
        const T* res = l == 0 ? enc : c->act_l<T>(p.res3, p.s_btc, l - 1);
        T* ln1 = c->act_l<T>(p.ln1, p.s_btc, l);
        T* qkv = c->act_l<T>(p.qkv, p.s_bt3c, l);
        T* atty = c->act_l<T>(p.atty, p.s_btc, l);
        T* res2 = c->act_l<T>(p.res2, p.s_btc, l);
        T* ln2 = c->act_l<T>(p.ln2, p.s_btc, l);
        T* fch = c->act_l<T>(p.fch, p.s_bt4c, l);
        T* fchg = c->act_l<T>(p.fchg, p.s_bt4c, l);
        T* res3 = c->act_l<T>(p.res3, p.s_btc, l);
        TRY(timed(c, GPT2_TP_LN_FWD, s, [&] {
            return layernorm_fwd_launch<T>(ln1, c->act_l<float>(p.ln1m, p.s_bt, l), c->act_l<float>(p.ln1r, p.s_bt, l),
                                           res, prm<T>(c, 2, l, C), prm<T>(c, 3, l, C), BT, C, s);
        }));
        TRY(timed(c, GPT2_TP_LAYER_FWD, s, [&] {
            return gemm(c, fwd_desc(BT, 3 * C, C, ln1, prm<T>(c, 4, l, 3 * CC), qkv, GEMM_BIAS, prm<T>(c, 5, l, 3 * C),
                                    nullptr, nullptr, (int)sizeof(T)), s);
        }));
        TRY(timed(c, GPT2_TP_ATTN_FWD, s, [&] {
            return attention_fwd_launch<T>(atty, c->act_l<float>(p.lse, p.s_lse, l), qkv, B, Tn, C, NH, s);
        }));
        TRY(timed(c, GPT2_TP_LAYER_FWD, s, [&] {
            return gemm(c, fwd_desc(BT, C, C, atty, prm<T>(c, 6, l, CC), res2, GEMM_BIAS_RESID, prm<T>(c, 7, l, C), res,
                                    nullptr, (int)sizeof(T)), s);
        }));
        TRY(timed(c, GPT2_TP_LN_FWD, s, [&] {
            return layernorm_fwd_launch<T>(ln2, c->act_l<float>(p.ln2m, p.s_bt, l), c->act_l<float>(p.ln2r, p.s_bt, l),
                                           res2, prm<T>(c, 8, l, C), prm<T>(c, 9, l, C), BT, C, s);
        }));
        TRY(timed(c, GPT2_TP_LAYER_FWD, s, [&] {
            return gemm(c, fwd_desc(BT, 4 * C, C, ln2, prm<T>(c, 10, l, 4 * CC), fchg, GEMM_BIAS_GELU,
                                    prm<T>(c, 11, l, 4 * C), nullptr, fch, (int)sizeof(T)), s);
        }));
        TRY(timed(c, GPT2_TP_LAYER_FWD, s, [&] {
            return gemm(c, fwd_desc(BT, C, 4 * C, fchg, prm<T>(c, 12, l, 4 * CC), res3, GEMM_BIAS_RESID,
                                    prm<T>(c, 13, l, C), res2, nullptr, (int)sizeof(T)), s);
        }));
    }
    const T* resL = c->act_l<T>(p.res3, p.s_btc, L - 1);
    T* lnf = c->act<T>(p.lnf);
    TRY(timed(c, GPT2_TP_LN_FWD, s, [&] {
        return layernorm_fwd_launch<T>(lnf, c->act<float>(p.lnfm), c->act<float>(p.lnfr), resL, prm<T>(c, 14),
                                       prm<T>(c, 15), BT, C, s);
    }));
    T* logits = c->act<T>(p.logits);
    TRY(timed(c, GPT2_TP_CLASSIFIER_FWD, s, [&] {
        return gemm(c, fwd_desc(BT, Vp, C, lnf, prm<T>(c, 0), logits, GEMM_STORE, nullptr, nullptr, nullptr,
                                (int)sizeof(T)), s);
    }));
    if (targets) {
        float* losses = c->act<float>(p.losses);
        TRY(timed(c, GPT2_TP_CE, s,
                  [&] { return classifier_ce_launch<T>(logits, losses, targets, BT, V, Vp, c->flag(), s); }));
        if (d_losses) TRY((int)hipMemcpyAsync(d_losses, losses, (size_t)BT * 4, hipMemcpyDeviceToDevice, s));
        if (d_mean) TRY(mean_launch(d_mean, losses, BT, s));
    }
    return GPT2_OK;
}

// dW += dY^T X (M = OC, N = IC, K = BT) and db += column sums of dY for
// layers l0 .. l1 - 1 in one launch (and the classifier's tied-weight
// gradient first in the tile order when cls: its 197 x 3 tiles are the
// largest product).  Every tile of that launch runs the whole contraction,
// so it takes ceil(tiles / CUs) rounds of about equal length; when leaving
// the attention projections (C x C products) out saves a round and their own
// launch on 128x256 tiles (half the work per tile, about 0.71 of a round
// each) costs less, they follow in a second launch (124M at B*T = 8192:
// 1887 tiles, 8 rounds, become 1779 + 216 half tiles).
int dw_group(gpt2_ctx* c, int l0, int l1, bool cls, hipStream_t s) {
    const Plan& p = c->plan;
    const int BT = (int)p.BT, C = (int)p.C, Vp = (int)p.Vp;
    const size_t CC = (size_t)C * C, e = 2;
    const long sbtc = (long)(p.s_btc / e), sbt4c = (long)(p.s_bt4c / e), sbt3c = (long)(p.s_bt3c / e);
    const float alpha = c->dw_alpha;
    GemmGroupItem it[5];
    int n = 0, ia = -1;
    auto item = [&](const void* A, long lda, long sA, const void* Bm, long ldb, long sB, float* Cm, long sC, float* db,
                    long sdb, int M, int N, int cnt, float a) {
        GemmGroupItem& g = it[n++];
        g.A = A; g.lda = lda; g.sA = sA; g.B = Bm; g.ldb = ldb; g.sB = sB; g.C = Cm; g.ldc = N; g.sC = sC;
        g.dbias = db; g.sBias = sdb; g.M = M; g.N = N; g.K = BT; g.count = cnt; g.alpha = a;
    };
    const int cnt = l1 - l0;
    auto act = [&](size_t ofs, size_t stride, int l) { return (const bf16_t*)(c->acts() + ofs + stride * l); };
    if (cls) item(c->act<bf16_t>(p.logits), Vp, 0, c->act<bf16_t>(p.lnf), C, 0, grd(c, 0), 0, nullptr, 0, Vp, C, 1, alpha);
    if (cnt > 0) {
        // fcproj: dY = residual gradient entering it (slots 2l), X = fc GELU output
        item(act(p.dres_lp, 2 * p.s_btc, l0), C, 2 * sbtc, act(p.fchg, p.s_bt4c, l0), 4 * C, sbt4c,
             grd(c, 12, l0, 4 * CC), (long)(4 * CC), grd(c, 13, l0, C), C, C, 4 * C, cnt, 1.0f);
        // fc: dY = pre-activation gradient, X = ln2
        item(act(p.dbt4c, p.s_bt4c, l0), 4 * C, sbt4c, act(p.ln2, p.s_btc, l0), C, sbtc, grd(c, 10, l0, 4 * CC),
             (long)(4 * CC), grd(c, 11, l0, 4 * C), 4 * C, 4 * C, C, cnt, 1.0f);
        // attproj: dY = residual gradient entering it (slots 2l + 1), X = attention output
        item(act(p.dres_lp + p.s_btc, 2 * p.s_btc, l0), C, 2 * sbtc, act(p.atty, p.s_btc, l0), C, sbtc,
             grd(c, 6, l0, CC), (long)CC, grd(c, 7, l0, C), C, C, C, cnt, 1.0f);
        ia = n - 1;
        // qkv: dY = qkv gradient, X = ln1
        item(act(p.dqkv, p.s_bt3c, l0), 3 * C, sbt3c, act(p.ln1, p.s_btc, l0), C, sbtc, grd(c, 4, l0, 3 * CC),
             (long)(3 * CC), grd(c, 5, l0, 3 * C), 3 * C, 3 * C, C, cnt, 1.0f);
    }
    if (n == 0) return 0;
    if (ia >= 0 && n > 1) {
        GemmGroupItem rest[5];
        int nr = 0;
        for (int i = 0; i < n; i++)
            if (i != ia) rest[nr++] = it[i];
        auto rounds = [](long tiles) { return (tiles + kPlanCUs - 1) / kPlanCUs; };
        const long r_all = rounds(gemm_dw_group_tiles(it, n, 0));
        const long r_rest = rounds(gemm_dw_group_tiles(rest, nr, 0));
        const long r_att = rounds(gemm_dw_group_tiles(&it[ia], 1, 1));
        if ((double)r_rest + 0.71 * (double)r_att < (double)r_all - 0.1) {
            const int e = gemm_dw_group_launch(rest, nr, s, 0);
            return e ? e : gemm_dw_group_launch(&it[ia], 1, s, 1);
        }
    }
    return gemm_dw_group_launch(it, n, s, 0);
}

template <typename T>
int backward_impl(gpt2_ctx* c, float dloss, hipStream_t s) {
    const Plan& p = c->plan;
    const int B = c->B, Tn = c->T, BT = (int)p.BT, C = (int)p.C, L = (int)p.L, NH = (int)p.NH, Vp = (int)p.Vp;
    const size_t CC = (size_t)C * C;
    // bf16: weight gradients of all layers in one launch at the end, from
    // output gradients kept per layer; fp32: each right after its input
    const bool grouped = c->prec == GPT2_BF16;
    const float alpha = dloss > 0.f ? dloss : 1.0f / (float)BT;
    c->dw_alpha = alpha;
    T* logits = c->act<T>(p.logits);  // holds softmax - onehot
    T* lnf = c->act<T>(p.lnf);
    T* dbtc = c->act<T>(p.dbtc);
    float* dres = c->act<float>(p.dres32);
    // per-layer slots (bf16) or the single buffer (fp32)
    auto dres_in = [&](int l, int which) {  // 0: entering fcproj, 1: entering attproj
        return grouped ? c->act<T>(p.dres_lp + (2 * (size_t)l + which) * p.s_btc) : (T*)dres;
    };
    auto dbt4c = [&](int l) { return c->act<T>(p.dbt4c + (grouped ? (size_t)l * p.s_bt4c : 0)); };
    auto dqkv = [&](int l) { return c->act<T>(p.dqkv + (grouped ? (size_t)l * p.s_bt3c : 0)); };
    auto lp_out = [&](int l, int which) { return grouped ? dres_in(l, which) : (T*)nullptr; };
    // slots of the LayerNorm backwards' partial column sums, in the order the
    // backward runs them: the final LayerNorm, then ln2 and ln1 of layers
    // L-1 .. 0 (parameter tensors 14, 8 and 2)
    auto ln_slot = [&](int tensor, int l) { return tensor == 14 ? 0 : 1 + 2 * (L - 1 - l) + (tensor == 2 ? 1 : 0); };
    float* work = c->work();
    auto dw_now = [&](const GemmDesc& d) {
        return grouped ? 0 : timed(c, GPT2_TP_WEIGHT_GRAD, s, [&] { return gemm(c, d, s); });
    };
    // classifier (tied weights): dlnf = alpha * dlogits wte; dwte += alpha * dlogits^T lnf
    TRY(timed(c, GPT2_TP_CLASSIFIER_DX, s, [&] {
        return gemm(c, dx_desc(BT, C, Vp, logits, prm<T>(c, 0), dbtc, GEMM_STORE, nullptr, alpha), s);
    }));
    TRY(dw_now(dw_desc(BT, C, Vp, logits, lnf, grd(c, 0), alpha, nullptr)));
    const T* resL = c->act_l<T>(p.res3, p.s_btc, L - 1);
    TRY(timed(c, GPT2_TP_LN_BWD, s, [&] {
        return layernorm_bwd_launch<T>(dres, lp_out(L - 1, 0), dbtc, resL, prm<T>(c, 14), c->act<float>(p.lnfm),
                                       c->act<float>(p.lnfr), BT, C, 0, c->lnpart(ln_slot(14, 0)), s);
    }));
    for (int l = L - 1; l >= 0; l--) {
        const T* res = l == 0 ? c->act<T>(p.enc) : c->act_l<T>(p.res3, p.s_btc, l - 1);
        const T* ln1 = c->act_l<T>(p.ln1, p.s_btc, l);
        const T* qkv = c->act_l<T>(p.qkv, p.s_bt3c, l);
        const T* atty = c->act_l<T>(p.atty, p.s_btc, l);
        const T* res2 = c->act_l<T>(p.res2, p.s_btc, l);
        const T* ln2 = c->act_l<T>(p.ln2, p.s_btc, l);
        const T* fch = c->act_l<T>(p.fch, p.s_bt4c, l);
        const T* fchg = c->act_l<T>(p.fchg, p.s_bt4c, l);
        // fcproj (+ GELU backward fused into its input-gradient product)
        TRY(dw_now(dw_desc(BT, 4 * C, C, dres_in(l, 0), fchg, grd(c, 12, l, 4 * CC), 1.0f, grd(c, 13, l, C))));
        TRY(timed(c, GPT2_TP_LAYER_DX, s, [&] {
            return gemm(c, dx_desc(BT, 4 * C, C, dres_in(l, 0), prm<T>(c, 12, l, 4 * CC), dbt4c(l), GEMM_GELU_BWD, fch,
                                   1.0f), s);
        }));
        // fc
        TRY(dw_now(dw_desc(BT, C, 4 * C, dbt4c(l), ln2, grd(c, 10, l, 4 * CC), 1.0f, grd(c, 11, l, 4 * C))));
        TRY(timed(c, GPT2_TP_LAYER_DX, s, [&] {
            return gemm(c, dx_desc(BT, C, 4 * C, dbt4c(l), prm<T>(c, 10, l, 4 * CC), dbtc, GEMM_STORE, nullptr, 1.0f), s);
        }));
        TRY(timed(c, GPT2_TP_LN_BWD, s, [&] {
            return layernorm_bwd_launch<T>(dres, lp_out(l, 1), dbtc, res2, prm<T>(c, 8, l, C),
                                           c->act_l<float>(p.ln2m, p.s_bt, l), c->act_l<float>(p.ln2r, p.s_bt, l), BT,
                                           C, 1, c->lnpart(ln_slot(8, l)), s);
        }));
        // attproj
        TRY(dw_now(dw_desc(BT, C, C, dres_in(l, 1), atty, grd(c, 6, l, CC), 1.0f, grd(c, 7, l, C))));
        TRY(timed(c, GPT2_TP_LAYER_DX, s, [&] {
            return gemm(c, dx_desc(BT, C, C, dres_in(l, 1), prm<T>(c, 6, l, CC), dbtc, GEMM_STORE, nullptr, 1.0f), s);
        }));
        // attention
        TRY(timed(c, GPT2_TP_ATTN_BWD, s, [&] {
            return attention_bwd_launch<T>(dqkv(l), c->act<float>(p.delta), dbtc, atty, qkv,
                                           c->act_l<float>(p.lse, p.s_lse, l), B, Tn, C, NH, s);
        }));
        // qkv
        TRY(dw_now(dw_desc(BT, C, 3 * C, dqkv(l), ln1, grd(c, 4, l, 3 * CC), 1.0f, grd(c, 5, l, 3 * C))));
        TRY(timed(c, GPT2_TP_LAYER_DX, s, [&] {
            return gemm(c, dx_desc(BT, C, 3 * C, dqkv(l), prm<T>(c, 4, l, 3 * CC), dbtc, GEMM_STORE, nullptr, 1.0f), s);
        }));
        TRY(timed(c, GPT2_TP_LN_BWD, s, [&] {
            return layernorm_bwd_launch<T>(dres, l > 0 ? lp_out(l - 1, 0) : (T*)nullptr, dbtc, res,
                                           prm<T>(c, 2, l, C), c->act_l<float>(p.ln1m, p.s_bt, l),
                                           c->act_l<float>(p.ln1r, p.s_bt, l), BT, C, 1, c->lnpart(ln_slot(2, l)), s);
        }));

    }
    // the LayerNorm parameters' gradients: every slot's partial sums in one
    // launch (up to kMaxLnSlots slots per launch)
    TRY(timed(c, GPT2_TP_LN_BWD, s, [&] {
        const int slots = 2 * L + 1;
        for (int s0 = 0; s0 < slots; s0 += kMaxLnSlots) {
            LnFinishArgs fa = {};
            for (int j = 0; j < slots; j++) {
                if (j < s0 || j >= s0 + kMaxLnSlots) continue;
                float*& w = fa.dw[j - s0];
                float*& b = fa.db[j - s0];
                if (j == 0) {
                    w = grd(c, 14);
                    b = grd(c, 15);
                } else {
                    const int l = L - 1 - (j - 1) / 2;
                    const bool ln1 = (j - 1) % 2 == 1;
                    w = grd(c, ln1 ? 2 : 8, l, C);
                    b = grd(c, ln1 ? 3 : 9, l, C);
                }
            }
            const int r =
                layernorm_bwd_finish_launch(fa, std::min(kMaxLnSlots, slots - s0), c->lnpart(s0), BT, C, p.esz, s);
            if (r != 0) return r;
        }
        return 0;
    }));
    // every weight gradient of the step in one launch (running the classifier's
    // or half of the layers' beside the chain on a second stream was slower)
    if (grouped) TRY(timed(c, GPT2_TP_WEIGHT_GRAD, s, [&] { return dw_group(c, 0, L, true, s); }));
    // the encoder backward adds into wte's gradient after the classifier's
    TRY(timed(c, GPT2_TP_ENCODER_BWD, s,
              [&] { return encoder_bwd_launch(grd(c, 0), grd(c, 1), dres, c->act<int>(p.tok), B, Tn, C, work, s); }));
    return GPT2_OK;
}

// Model-file header (train_gpt2.cu, gpt2_build_from_checkpoint): 256 int32.
constexpr int kCkptMagic = 20240326, kCkptHeaderInts = 256;

int read_ckpt_header(FILE* f, gpt2_config* cfg, int* prec) {
    int32_t h[kCkptHeaderInts];
    if (fread(h, sizeof(int32_t), kCkptHeaderInts, f) != (size_t)kCkptHeaderInts) return GPT2_E_FILE;
    if (h[0] != kCkptMagic || (h[1] != 3 && h[1] != 5)) return GPT2_E_FILE;
    gpt2_config c;
    c.max_seq_len = h[2];
    c.vocab_size = h[3];
    c.num_layers = h[4];
    c.num_heads = h[5];
    c.channels = h[6];
    c.padded_vocab_size = h[7];
    if (check_config(&c, GPT2_FP32, 1, 1) != GPT2_OK) return GPT2_E_FILE;
    *cfg = c;
    *prec = h[1] == 3 ? GPT2_FP32 : GPT2_BF16;
    return GPT2_OK;
}

}  // namespace

extern "C" {

int gpt2_query_sizes(const gpt2_config* cfg, int precision, int B, int T, gpt2_sizes* out) {
    int rc = check_config(cfg, precision, B, T);
    if (rc) return rc;
    if (!out) return GPT2_E_ARG;
    size_t off[16], cnt[16], P;
    param_layout(*cfg, off, cnt, &P);
    Plan p = make_plan(*cfg, precision, B, T);
    out->params = align_up(P * p.esz);
    out->master = precision == GPT2_BF16 ? align_up(P * 4) : 0;  // none for GPT2_FP32, GPT2_BF16_SR
    out->grads = out->adam_m = out->adam_v = align_up(P * 4);
    out->acts = p.acts_bytes;
    out->scratch = p.scratch_bytes;
    return GPT2_OK;
}

int gpt2_param_layout(const gpt2_config* cfg, size_t offset[16], size_t count[16], size_t* total) {
    if (!cfg || !offset || !count || !total) return GPT2_E_ARG;
    if (cfg->num_layers < 1 || cfg->channels < 1 || cfg->padded_vocab_size < 1 || cfg->max_seq_len < 1)
        return GPT2_E_ARG;
    param_layout(*cfg, offset, count, total);
    return GPT2_OK;
}

int gpt2_init(gpt2_ctx** out, const gpt2_config* cfg, int precision, int B, int T, const gpt2_buffers* bufs,
              void* hip_stream) {
    if (!out) return GPT2_E_ARG;
    *out = nullptr;
    int rc = check_config(cfg, precision, B, T);
    if (rc) return rc;
    if (!bufs || !bufs->params || !bufs->grads || !bufs->adam_m || !bufs->adam_v || !bufs->acts || !bufs->scratch)
        return GPT2_E_ARG;
    if (precision == GPT2_BF16 && !bufs->master) return GPT2_E_ARG;
    const void* ptrs[7] = {bufs->params, bufs->master, bufs->grads, bufs->adam_m, bufs->adam_v, bufs->acts, bufs->scratch};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return GPT2_E_ALIGN;
    gpt2_ctx* c = new (std::nothrow) gpt2_ctx();
    if (!c) return GPT2_E_ARG;
    c->cfg = *cfg;
    c->prec = precision == GPT2_FP32 ? GPT2_FP32 : GPT2_BF16;
    c->sr = precision == GPT2_BF16_SR;
    c->B = B;
    c->T = T;
    param_layout(*cfg, c->off, c->cnt, &c->P);
    c->buf = *bufs;
    if (precision != GPT2_BF16) c->buf.master = nullptr;
    c->plan = make_plan(*cfg, precision, B, T);
    c->last_fwd_targets = -1;
    hipStream_t s = (hipStream_t)hip_stream;
    int e = 0;
    e |= fill_f32_launch((float*)c->buf.adam_m, 0.f, c->P, s);
    e |= fill_f32_launch((float*)c->buf.adam_v, 0.f, c->P, s);
    e |= fill_i32_launch(c->flag(), 0, 64, s);
    if (precision == GPT2_BF16) e |= cast_f32_to_bf16_launch((bf16_t*)c->buf.params, (const float*)c->buf.master, c->P, s);
    if (e) {
        delete c;
        return GPT2_E_HIP;
    }
    *out = c;
    return GPT2_OK;
}

int gpt2_forward(gpt2_ctx* c, const int32_t* d_inputs, const int32_t* d_targets, float* d_losses,
                 float* d_mean_loss, void* hip_stream) {
    if (!c || !d_inputs) return GPT2_E_ARG;
    if (!aligned(d_inputs) || (d_targets && !aligned(d_targets)) || (d_losses && !aligned(d_losses)) ||
        (d_mean_loss && ((uintptr_t)d_mean_loss % 4)))
        return GPT2_E_ALIGN;
    hipStream_t s = (hipStream_t)hip_stream;
    int rc = c->prec == GPT2_BF16 ? forward_impl<bf16_t>(c, d_inputs, d_targets, d_losses, d_mean_loss, s)
                                  : forward_impl<float>(c, d_inputs, d_targets, d_losses, d_mean_loss, s);
    c->last_fwd_targets = rc == GPT2_OK ? (d_targets ? 1 : 0) : -1;
    return rc;
}

int gpt2_zero_grad(gpt2_ctx* c, void* hip_stream) {
    if (!c) return GPT2_E_ARG;
    return hip_rc(fill_f32_launch((float*)c->buf.grads, 0.f, c->P, (hipStream_t)hip_stream));
}

int gpt2_backward(gpt2_ctx* c, float dloss, void* hip_stream) {
    if (!c) return GPT2_E_ARG;
    if (c->last_fwd_targets != 1) return GPT2_E_STATE;
    if (!(dloss == dloss)) return GPT2_E_ARG;  // NaN
    hipStream_t s = (hipStream_t)hip_stream;
    int rc = c->prec == GPT2_BF16 ? backward_impl<bf16_t>(c, dloss, s) : backward_impl<float>(c, dloss, s);
    // the in-place softmax - onehot has been consumed; a new forward is needed
    c->last_fwd_targets = -1;
    return rc;
}

int gpt2_adamw_update(gpt2_ctx* c, float lr, float beta1, float beta2, float eps, float weight_decay, int t,
                      void* hip_stream) {
    if (!c || t < 1) return GPT2_E_ARG;
    if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f)) return GPT2_E_ARG;
    hipStream_t s = (hipStream_t)hip_stream;
    if (c->sr) {
        const uint32_t seed = xorshift_u32(&c->rng);
        const float c1 = 1.0f - powf(beta1, (float)t), c2 = 1.0f - powf(beta2, (float)t);
        return hip_rc(timed(c, GPT2_TP_ADAMW, s, [&] {
            return adamw_sr_launch((bf16_t*)c->buf.params, (const float*)c->buf.grads, (float*)c->buf.adam_m,
                                   (float*)c->buf.adam_v, c->P, lr, beta1, beta2, c1, c2, eps, weight_decay, seed, s);
        }));
    }
    const float c1 = (float)(1.0 - pow((double)beta1, t));
    const float c2 = (float)(1.0 - pow((double)beta2, t));
    return hip_rc(timed(c, GPT2_TP_ADAMW, s, [&] {
        if (c->prec == GPT2_BF16)
            return adamw_launch<bf16_t>((bf16_t*)c->buf.params, (float*)c->buf.master, (const float*)c->buf.grads,
                                        (float*)c->buf.adam_m, (float*)c->buf.adam_v, c->P, lr, beta1, beta2, c1, c2,
                                        eps, weight_decay, s);
        return adamw_launch<float>((float*)c->buf.params, nullptr, (const float*)c->buf.grads, (float*)c->buf.adam_m,
                                   (float*)c->buf.adam_v, c->P, lr, beta1, beta2, c1, c2, eps, weight_decay, s);
    }));
}

int gpt2_set_rng_state(gpt2_ctx* c, uint64_t state, uint64_t* old) {
    if (!c) return GPT2_E_ARG;
    if (old) *old = c->rng;
    if (state) c->rng = state;
    return GPT2_OK;
}

int gpt2_check_device_error(gpt2_ctx* c, void* hip_stream) {
    if (!c) return GPT2_E_ARG;
    hipStream_t s = (hipStream_t)hip_stream;
    if (hipStreamSynchronize(s) != hipSuccess) return GPT2_E_HIP;
    int flag = 0;
    if (hipMemcpy(&flag, c->flag(), sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return GPT2_E_HIP;
    if (flag) {
        if (fill_i32_launch(c->flag(), 0, 64, s) != 0) return GPT2_E_HIP;
        if (hipStreamSynchronize(s) != hipSuccess) return GPT2_E_HIP;
        return GPT2_E_TOKEN;
    }
    return GPT2_OK;
}

int gpt2_act_tensor(gpt2_ctx* c, int which, void** d_ptr, size_t* count) {
    if (!c || !d_ptr || !count) return GPT2_E_ARG;
    const Plan& p = c->plan;
    switch (which) {
        case GPT2_T_LOGITS: *d_ptr = c->act<char>(p.logits); *count = p.BT * p.Vp; return GPT2_OK;
        case GPT2_T_LNF: *d_ptr = c->act<char>(p.lnf); *count = p.BT * p.C; return GPT2_OK;
        case GPT2_T_RESIDUAL: *d_ptr = c->act<char>(p.res3 + p.s_btc * (p.L - 1)); *count = p.BT * p.C; return GPT2_OK;
        case GPT2_T_DRESIDUAL: *d_ptr = c->act<char>(p.dres32); *count = p.BT * p.C; return GPT2_OK;
        case GPT2_T_ENCODED: *d_ptr = c->act<char>(p.enc); *count = p.BT * p.C; return GPT2_OK;
        default: return GPT2_E_ARG;
    }
}

int gpt2_set_timing_events(gpt2_ctx* c, int point, void* const* d_start_events, void* const* d_end_events, int n) {
    if (!c || point < 0 || point >= GPT2_TP_COUNT || n < 0 || (n > 0 && (!d_start_events || !d_end_events)))
        return GPT2_E_ARG;
    gpt2_ctx::Hook& h = c->hooks[point];
    h.start = n > 0 ? d_start_events : nullptr;
    h.end = n > 0 ? d_end_events : nullptr;
    h.n = n;
    h.i = 0;
    return GPT2_OK;
}

int gpt2_set_classifier_events(gpt2_ctx* c, void* const* d_start_events, void* const* d_end_events, int n) {
    return gpt2_set_timing_events(c, GPT2_TP_CLASSIFIER_FWD, d_start_events, d_end_events, n);
}

int gpt2_free(gpt2_ctx* c) {
    delete c;
    return GPT2_OK;
}

int gpt2_sample(gpt2_ctx* c, const float* d_coins, int32_t* d_tokens, int t, void* hip_stream) {
    if (!c || !d_coins || !d_tokens) return GPT2_E_ARG;
    if (t < 1 || t >= c->T) return GPT2_E_ARG;
    if (!aligned(d_tokens) || ((uintptr_t)d_coins % 4)) return GPT2_E_ALIGN;
    if (c->last_fwd_targets != 0) return GPT2_E_STATE;
    const hipStream_t s = (hipStream_t)hip_stream;
    const Plan& p = c->plan;
    const int V = c->cfg.vocab_size, Vp = (int)p.Vp;
    const int rc = c->prec == GPT2_BF16
                       ? sample_launch<bf16_t>(d_tokens, c->act<bf16_t>(p.logits), d_coins, c->B, c->T, t, V, Vp, s)
                       : sample_launch<float>(d_tokens, c->act<float>(p.logits), d_coins, c->B, c->T, t, V, Vp, s);
    return hip_rc(rc);
}

int gpt2_generate(gpt2_ctx* c, int32_t* d_tokens, const float* d_coins, int t_begin, int t_end, void* hip_stream) {
    if (!c || !d_tokens || !d_coins) return GPT2_E_ARG;
    if (t_begin < 1 || t_end < t_begin || t_end > c->T) return GPT2_E_ARG;
    for (int t = t_begin; t < t_end; t++) {
        int rc = gpt2_forward(c, d_tokens, nullptr, nullptr, nullptr, hip_stream);
        if (rc != GPT2_OK) return rc;
        rc = gpt2_sample(c, d_coins + (size_t)(t - t_begin) * c->B, d_tokens, t, hip_stream);
        if (rc != GPT2_OK) return rc;
    }
    return GPT2_OK;
}

int gpt2_checkpoint_header(const char* path, gpt2_config* cfg, int* file_precision) {
    if (!path || !cfg || !file_precision) return GPT2_E_ARG;
    FILE* f = fopen(path, "rb");
    if (!f) return GPT2_E_FILE;
    const int rc = read_ckpt_header(f, cfg, file_precision);
    fclose(f);
    return rc;
}

int gpt2_checkpoint_read(const char* path, float* h_params, size_t count) {
    if (!path || !h_params) return GPT2_E_ARG;
    FILE* f = fopen(path, "rb");
    if (!f) return GPT2_E_FILE;
    gpt2_config c;
    int prec = 0;
    int rc = read_ckpt_header(f, &c, &prec);
    if (rc == GPT2_OK) {
        size_t off[16], cnt[16], P = 0;
        param_layout(c, off, cnt, &P);
        if (count != P) {
            rc = GPT2_E_ARG;
        } else if (prec == GPT2_FP32) {
            if (fread(h_params, sizeof(float), P, f) != P) rc = GPT2_E_FILE;
        } else {
            // bf16 values, read in chunks and widened: a bf16 value is the
            // upper 16 bits of the fp32 with the same value
            constexpr size_t CH = 1 << 16;
            uint16_t buf[CH];
            for (size_t i = 0; i < P && rc == GPT2_OK; i += CH) {
                const size_t n = std::min(CH, P - i);
                if (fread(buf, sizeof(uint16_t), n, f) != n) {
                    rc = GPT2_E_FILE;
                    break;
                }
                for (size_t j = 0; j < n; j++) {
                    const uint32_t u = (uint32_t)buf[j] << 16;
                    memcpy(&h_params[i + j], &u, 4);
                }
            }
        }
    }
    fclose(f);
    return rc;
}

const char* gpt2_strerror(int code) {
    switch (code) {
        case GPT2_OK: return "ok";
        case GPT2_E_ARG: return "invalid argument";
        case GPT2_E_SHAPE: return "unsupported shape";
        case GPT2_E_STATE: return "call order violated (backward needs a forward with targets)";
        case GPT2_E_TOKEN: return "token or target id outside [0, vocab_size)";
        case GPT2_E_ALIGN: return "pointer not 256-byte aligned";
        case GPT2_E_HIP: return "HIP runtime or kernel launch failure";
        case GPT2_E_FILE: return "model file missing, unreadable or invalid";
        default: return "unknown error";
    }
}

}  // extern "C"
