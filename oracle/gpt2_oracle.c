/*
 * gpt2_oracle.c - CPU oracle for the GPT-2 training step (TEST INFRASTRUCTURE).
 *
 * Plain, slow, single-threaded C in double precision (one exception:
 * orc_adamw_sr works in fp32, the page's precision, because an fp32 value
 * decides its stochastic rounding).  Each function writes out
 * one definition from the pages; comments name the page and the kernel or host
 * routine whose computation it follows.  Loops are in the order of the
 * definition; the only liberty taken is the loop nest of the two backward
 * matrix products, which runs the reduction index outermost so that the inner
 * loop walks contiguous memory.  That keeps, for every output element, the
 * summation in increasing order of the reduced index, exactly as the written-out
 * sum.  No blocking, no fusion across definitions, no threads.
 *
 * Pages: "train_gpt2.cu" (llm.c, mixed precision; the authority), and
 * "train_gpt2_fp32.cu" (llm.c fp32 version; its text lost every '+' sign, so it
 * is only used as a cross-check), and the POPCORNBENCH "Kimi-K2.6 l2_p99"
 * transcript for the standalone Linear -> GELU -> softmax op.
 */
#include "gpt2_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Parameter layout: train_gpt2.cu, ParameterTensors and fill_in_parameter_sizes. */
size_t orc_param_layout(const orc_config* cfg, size_t offset[16], size_t count[16]) {
    size_t Vp = (size_t)cfg->padded_vocab_size, C = (size_t)cfg->channels;
    size_t maxT = (size_t)cfg->max_seq_len, L = (size_t)cfg->num_layers;
    size_t c[16];
    c[0] = Vp * C;          /* wte */
    c[1] = maxT * C;        /* wpe */
    c[2] = L * C;           /* ln1w */
    c[3] = L * C;           /* ln1b */
    c[4] = L * 3 * C * C;   /* qkvw */
    c[5] = L * 3 * C;       /* qkvb */
    c[6] = L * C * C;       /* attprojw */
    c[7] = L * C;           /* attprojb */
    c[8] = L * C;           /* ln2w */
    c[9] = L * C;           /* ln2b */
    c[10] = L * 4 * C * C;  /* fcw */
    c[11] = L * 4 * C;      /* fcb */
    c[12] = L * C * 4 * C;  /* fcprojw */
    c[13] = L * C;          /* fcprojb */
    c[14] = C;              /* lnfw */
    c[15] = C;              /* lnfb */
    size_t total = 0;
    for (int i = 0; i < 16; i++) {
        if (offset) offset[i] = total;
        if (count) count[i] = c[i];
        total += c[i];
    }
    return total;
}

/* train_gpt2.cu, encoder_forward_kernel2: the token row plus the position row. */
void orc_encoder_forward(double* out, const int* tok, const double* wte, const double* wpe,
                         int B, int T, int C) {
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            int ix = tok[b * T + t];
            for (int c = 0; c < C; c++)
                out[((size_t)b * T + t) * C + c] = wte[(size_t)ix * C + c] + wpe[(size_t)t * C + c];
        }
}

/* train_gpt2.cu, encoder_backward_kernel: every position's gradient is added
 * into its token's row and its position's row. */
void orc_encoder_backward(double* dwte, double* dwpe, const double* dout, const int* tok,
                          int B, int T, int C) {
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            int ix = tok[b * T + t];
            const double* d = dout + ((size_t)b * T + t) * C;
            for (int c = 0; c < C; c++) {
                dwte[(size_t)ix * C + c] += d[c];
                dwpe[(size_t)t * C + c] += d[c];
            }
        }
}

/* train_gpt2.cu, layernorm_forward_kernel3: mean, then the biased variance of
 * the centred row, rstd = 1/sqrt(var + 1e-5), then (x - mean) * rstd * w + b. */
void orc_layernorm_forward(double* out, double* mean, double* rstd, const double* x,
                           const double* w, const double* b, int N, int C) {
    const double eps = 1e-5;
    for (int n = 0; n < N; n++) {
        const double* xr = x + (size_t)n * C;
        double m = 0.0;
        for (int c = 0; c < C; c++) m += xr[c];
        m /= C;
        double var = 0.0;
        for (int c = 0; c < C; c++) {
            double d = xr[c] - m;
            var += d * d;
        }
        var /= C;
        double s = 1.0 / sqrt(var + eps);
        for (int c = 0; c < C; c++)
            out[(size_t)n * C + c] = (xr[c] - m) * s * w[c] + b[c];
        if (mean) mean[n] = m;
        if (rstd) rstd[n] = s;
    }
}

/* train_gpt2.cu, layernorm_backward_kernel6 (and train_gpt2_fp32.cu,
 * layernorm_backward_kernel2): with norm = (x - mean) * rstd and
 * dnorm = w * dout, the input gradient is
 * rstd * (dnorm - mean_c(dnorm) - norm * mean_c(dnorm * norm)); the weight
 * gradient is the sum over rows of norm * dout and the bias gradient the sum of
 * dout.  All three are added into their outputs. */
void orc_layernorm_backward(double* dx, double* dw, double* db, const double* dout,
                            const double* x, const double* w, const double* mean,
                            const double* rstd, int N, int C) {
    for (int n = 0; n < N; n++) {
        const double* xr = x + (size_t)n * C;
        const double* dy = dout + (size_t)n * C;
        double m = mean[n], s = rstd[n];
        double dnorm_mean = 0.0, dnorm_norm_mean = 0.0;
        for (int c = 0; c < C; c++) {
            double norm = (xr[c] - m) * s;
            double dnorm = w[c] * dy[c];
            dnorm_mean += dnorm;
            dnorm_norm_mean += dnorm * norm;
        }
        dnorm_mean /= C;
        dnorm_norm_mean /= C;
        for (int c = 0; c < C; c++) {
            double norm = (xr[c] - m) * s;
            double dnorm = w[c] * dy[c];
            if (db) db[c] += dy[c];
            if (dw) dw[c] += norm * dy[c];
            dx[(size_t)n * C + c] += s * (dnorm - dnorm_mean - norm * dnorm_norm_mean);
        }
    }
}

/* train_gpt2.cu, matmul_forward_cublaslt: out = inp @ weight^T + bias, weight
 * stored (out_features, in_features). */
void orc_matmul_forward(double* out, const double* x, const double* w, const double* bias,
                        int N, int K, int OC) {
    for (int n = 0; n < N; n++) {
        const double* xr = x + (size_t)n * K;
        for (int o = 0; o < OC; o++) {
            const double* wr = w + (size_t)o * K;
            double acc = 0.0;
            for (int k = 0; k < K; k++) acc += xr[k] * wr[k];
            out[(size_t)n * OC + o] = acc + (bias ? bias[o] : 0.0);
        }
    }
}

/* train_gpt2.cu, matmul_backward: the input gradient dout @ weight overwrites;
 * the weight gradient dout^T @ inp and the bias gradient (column sums of dout,
 * matmul_backward_bias_kernel4) are added. */
void orc_matmul_backward(double* dx, double* dw, double* db, const double* dout,
                         const double* x, const double* w, int N, int K, int OC) {
    if (dx) {
        for (int n = 0; n < N; n++) {
            double* dxr = dx + (size_t)n * K;
            for (int k = 0; k < K; k++) dxr[k] = 0.0;
            for (int o = 0; o < OC; o++) {  /* dx[n,k] = sum over o, in increasing o */
                double g = dout[(size_t)n * OC + o];
                const double* wr = w + (size_t)o * K;
                for (int k = 0; k < K; k++) dxr[k] += g * wr[k];
            }
        }
    }
    if (dw) {
        double* acc = (double*)calloc((size_t)OC * K, sizeof(double));
        for (int n = 0; n < N; n++) {        /* dw[o,k] = sum over n, in increasing n */
            const double* xr = x + (size_t)n * K;
            for (int o = 0; o < OC; o++) {
                double g = dout[(size_t)n * OC + o];
                double* ar = acc + (size_t)o * K;
                for (int k = 0; k < K; k++) ar[k] += g * xr[k];
            }
        }
        for (size_t i = 0; i < (size_t)OC * K; i++) dw[i] += acc[i];
        free(acc);
    }
    if (db) {
        for (int o = 0; o < OC; o++) {
            double s = 0.0;
            for (int n = 0; n < N; n++) s += dout[(size_t)n * OC + o];
            db[o] += s;
        }
    }
}

/* train_gpt2.cu, attention_forward: q, k, v of head h are the channel slices
 * [h*HS, (h+1)*HS) of the three C-wide thirds of a qkv row (permute_kernel);
 * preatt = q k^T scaled by 1/sqrt(HS); softmax over the causal prefix s <= t
 * (softmax_forward_kernel5 only ever writes s <= t); y = att v, re-assembled as
 * (B, T, NH*HS) (unpermute_kernel). */
void orc_attention_forward(double* out, double* att, const double* qkv,
                           int B, int T, int C, int NH) {
    int HS = C / NH;
    double scale = 1.0 / sqrt((double)HS);
    size_t C3 = 3 * (size_t)C;
    double* srow = (double*)malloc((size_t)T * sizeof(double));
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++)
            for (int t = 0; t < T; t++) {
                const double* q = qkv + ((size_t)b * T + t) * C3 + (size_t)h * HS;
                double maxv = -INFINITY;
                for (int s = 0; s <= t; s++) {
                    const double* k = qkv + ((size_t)b * T + s) * C3 + C + (size_t)h * HS;
                    double dot = 0.0;
                    for (int d = 0; d < HS; d++) dot += q[d] * k[d];
                    srow[s] = dot * scale;
                    if (srow[s] > maxv) maxv = srow[s];
                }
                double sum = 0.0;
                for (int s = 0; s <= t; s++) sum += exp(srow[s] - maxv);
                double* arow = att + (((size_t)b * NH + h) * T + t) * T;
                for (int s = 0; s < T; s++) arow[s] = (s <= t) ? exp(srow[s] - maxv) / sum : 0.0;
                double* o = out + ((size_t)b * T + t) * C + (size_t)h * HS;
                for (int d = 0; d < HS; d++) {
                    double acc = 0.0;
                    for (int s = 0; s <= t; s++)
                        acc += arow[s] * qkv[((size_t)b * T + s) * C3 + 2 * (size_t)C + (size_t)h * HS + d];
                    o[d] = acc;
                }
            }
    free(srow);
}

/* train_gpt2.cu, attention_backward: datt = dy v^T and dv = att^T dy; then
 * softmax_autoregressive_backward_kernel: dpreatt[t,s] = scale * att[t,s] *
 * (datt[t,s] - sum_{s'<=t} att[t,s'] datt[t,s']) for s <= t; then dq = dpreatt k
 * and dk = dpreatt^T q; the three are written back in the (B, T, 3, NH, HS)
 * layout (permute_kernel_backward). */
void orc_attention_backward(double* dqkv, const double* dout, const double* qkv,
                            const double* att, int B, int T, int C, int NH) {
    int HS = C / NH;
    double scale = 1.0 / sqrt((double)HS);
    size_t C3 = 3 * (size_t)C;
    memset(dqkv, 0, (size_t)B * T * C3 * sizeof(double));
    double* datt = (double*)malloc((size_t)T * sizeof(double));
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++)
            for (int t = 0; t < T; t++) {
                const double* arow = att + (((size_t)b * NH + h) * T + t) * T;
                const double* dy = dout + ((size_t)b * T + t) * C + (size_t)h * HS;
                const double* q = qkv + ((size_t)b * T + t) * C3 + (size_t)h * HS;
                double* dq = dqkv + ((size_t)b * T + t) * C3 + (size_t)h * HS;
                for (int s = 0; s <= t; s++) {
                    const double* v = qkv + ((size_t)b * T + s) * C3 + 2 * (size_t)C + (size_t)h * HS;
                    double* dv = dqkv + ((size_t)b * T + s) * C3 + 2 * (size_t)C + (size_t)h * HS;
                    double dot = 0.0;
                    for (int d = 0; d < HS; d++) {
                        dot += dy[d] * v[d];
                        dv[d] += arow[s] * dy[d];
                    }
                    datt[s] = dot;
                }
                double local = 0.0;
                for (int s = 0; s <= t; s++) local += arow[s] * datt[s];
                for (int s = 0; s <= t; s++) {
                    double dpre = scale * arow[s] * (datt[s] - local);
                    const double* k = qkv + ((size_t)b * T + s) * C3 + C + (size_t)h * HS;
                    double* dk = dqkv + ((size_t)b * T + s) * C3 + C + (size_t)h * HS;
                    for (int d = 0; d < HS; d++) {
                        dq[d] += dpre * k[d];
                        dk[d] += dpre * q[d];
                    }
                }
            }
    free(datt);
}

/* train_gpt2.cu, gelu_forward_kernel2: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
void orc_gelu_forward(double* out, const double* x, size_t n) {
    const double s = sqrt(2.0 / M_PI);
    for (size_t i = 0; i < n; i++) {
        double xi = x[i];
        out[i] = 0.5 * xi * (1.0 + tanh(s * (xi + 0.044715 * xi * xi * xi)));
    }
}

/* train_gpt2.cu, gelu_backward_kernel: with u = sqrt(2/pi)(x + 0.044715 x^3),
 * gelu'(x) = 0.5 (1 + tanh u) + 0.5 x sech^2(u) sqrt(2/pi) (1 + 3*0.044715 x^2),
 * sech^2 = 1 / cosh^2. */
void orc_gelu_backward(double* dx, const double* x, const double* dout, size_t n) {
    const double s = sqrt(2.0 / M_PI);
    for (size_t i = 0; i < n; i++) {
        double xi = x[i];
        double u = s * (xi + 0.044715 * xi * xi * xi);
        double ch = cosh(u);
        double local = 0.5 * (1.0 + tanh(u)) + xi * 0.5 * (1.0 / (ch * ch)) * s * (1.0 + 3.0 * 0.044715 * xi * xi);
        dx[i] = local * dout[i];
    }
}

/* train_gpt2.cu, residual_forward_kernel. */
void orc_residual_forward(double* out, const double* a, const double* b, size_t n) {
    for (size_t i = 0; i < n; i++) out[i] = a[i] + b[i];
}

/* train_gpt2.cu, fused_classifier_kernel3 (forward half): softmax over the V
 * real columns (the padded ones never enter), loss = -log p[target], written as
 * logsumexp - z[target], which is the same number without the underflow of
 * log(exp(...)). */
double orc_crossentropy_forward(double* losses, double* probs, const double* logits,
                                const int* targets, int N, int V, int Vp) {
    double total = 0.0;
    for (int n = 0; n < N; n++) {
        const double* z = logits + (size_t)n * Vp;
        double maxv = -INFINITY;
        for (int i = 0; i < V; i++) if (z[i] > maxv) maxv = z[i];
        double sum = 0.0;
        for (int i = 0; i < V; i++) sum += exp(z[i] - maxv);
        double lse = maxv + log(sum);
        losses[n] = lse - z[targets[n]];
        total += losses[n];
        if (probs) {
            for (int i = 0; i < V; i++) probs[(size_t)n * Vp + i] = exp(z[i] - lse);
            for (int i = V; i < Vp; i++) probs[(size_t)n * Vp + i] = 0.0;
        }
    }
    return total / N;
}

/* train_gpt2.cu, fused_classifier_kernel3 (backward half): (p - onehot) * dloss;
 * padded columns get exactly 0. */
void orc_crossentropy_backward(double* dlogits, const double* probs, const int* targets,
                               double dloss, int N, int V, int Vp) {
    for (int n = 0; n < N; n++)
        for (int i = 0; i < Vp; i++) {
            double g = 0.0;
            if (i < V) g = (probs[(size_t)n * Vp + i] - (i == targets[n] ? 1.0 : 0.0)) * dloss;
            dlogits[(size_t)n * Vp + i] = g;
        }
}

/* train_gpt2.cu, adamw_kernel3 with gpt2_update's bias corrections 1 - beta^t:
 * m = beta1 m + (1-beta1) g; v = beta2 v + (1-beta2) g^2;
 * p -= lr (mhat / (sqrt(vhat) + eps) + wd p). */
void orc_adamw(double* params, const double* grads, double* m, double* v, size_t n,
               double lr, double beta1, double beta2, double eps, double weight_decay, int t) {
    double c1 = 1.0 - pow(beta1, t), c2 = 1.0 - pow(beta2, t);
    for (size_t i = 0; i < n; i++) {
        double g = grads[i];
        m[i] = beta1 * m[i] + (1.0 - beta1) * g;
        v[i] = beta2 * v[i] + (1.0 - beta2) * g * g;
        double mhat = m[i] / c1, vhat = v[i] / c2;
        params[i] -= lr * (mhat / (sqrt(vhat) + eps) + weight_decay * params[i]);
    }
}

/* SquirrelNoise5, Squirrel Eiserloh's published noise function (the one
 * train_gpt2.cu uses): a 32-bit position is multiplied by a constant, the seed
 * added, then the bits are mixed by right xor-shifts of 9, 11, 13, 15 and 17
 * interleaved with adding, multiplying by and adding three more constants.
 * All arithmetic modulo 2^32. */
static uint32_t orc_squirrel5(uint32_t pos, uint32_t seed) {
    uint32_t h = pos * 0xd2a80a3fu;
    h += seed;
    h ^= h >> 9;
    h += 0xa884f197u;
    h ^= h >> 11;
    h *= 0x6c736f4bu;
    h ^= h >> 13;
    h += 0xb79f3abbu;
    h ^= h >> 15;
    h *= 0x1b56c4f5u;
    h ^= h >> 17;
    return h;
}

/* train_gpt2.cu, Get2dNoiseUint: position x + 198491317 y (mod 2^32). */
uint32_t orc_noise2d(int x, int y, uint32_t seed) {
    return orc_squirrel5((uint32_t)x + 198491317u * (uint32_t)y, seed);
}

/* train_gpt2.cu, random_u32: xorshift (shifts 12, 25, 27) of the 64-bit state,
 * then the upper half of the state times 0x2545F4914F6CDD1D (xorshift*). */
uint32_t orc_xorshift_u32(uint64_t* state) {
    uint64_t s = *state;
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    *state = s;
    return (uint32_t)((s * 0x2545F4914F6CDD1DULL) >> 32);
}

/* fp32 -> bf16, round to nearest even (finite inputs). */
static uint16_t orc_bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* train_gpt2.cu, stochastic_rounding: the low 16 bits of x are set to ones
 * if they exceed r (r < 2^16), cleared otherwise; then round to nearest-even
 * bf16.  x rounds up exactly for the r below its low 16 bits. */
uint16_t orc_sr_bf16(float x, uint32_t r) {
    uint32_t bits;
    memcpy(&bits, &x, 4);
    bits = (bits & 0xffffu) > r ? (bits | 0xffffu) : (bits & 0xffff0000u);
    float y;
    memcpy(&y, &bits, 4);
    return orc_bf16_rne(y);
}

/* train_gpt2.cu, adamw_kernel3 with master_params == NULL, in the page's
 * precision (fp32, one rounding per operation; the moment updates are the
 * page's lerp, two fused multiply-adds), with gpt2_update's corrections
 * 1 - powf(beta, t) and stochastic_rounding: parameter i, launched by the page
 * as thread i % 512 of block i / 512, draws the noise Get2dNoiseUint at that
 * position with the per-call seed, and that value is the seed of a second
 * Get2dNoiseUint at the same position (the page passes the first draw as the
 * rounding's seed); the low 16 bits r of the second draw decide: the new
 * value's low 16 bits are set to ones if they exceed r, cleared otherwise,
 * and the result is rounded to nearest-even bf16.  params hold bf16 bit
 * patterns. */
void orc_adamw_sr(uint16_t* params, const float* grads, float* m, float* v, size_t n, float lr, float beta1,
                  float beta2, float eps, float weight_decay, int t, uint32_t seed) {
    const float c1 = 1.0f - powf(beta1, (float)t), c2 = 1.0f - powf(beta2, (float)t);
    for (size_t i = 0; i < n; i++) {
        const float g = grads[i];
        m[i] = fmaf(beta1, m[i], fmaf(-beta1, g, g));
        const float g2 = g * g;
        v[i] = fmaf(beta2, v[i], fmaf(-beta2, g2, g2));
        const float mhat = m[i] / c1, vhat = v[i] / c2;
        uint32_t ob = (uint32_t)params[i] << 16;
        float old;
        memcpy(&old, &ob, 4);
        const float den = sqrtf(vhat) + eps;
        const float upd = mhat / den + weight_decay * old;
        const float x = old - lr * upd;
        const int tx = (int)(i % 512), bx = (int)(i / 512);
        const uint32_t r = orc_noise2d(tx, bx, orc_noise2d(tx, bx, seed)) & 0xffffu;
        params[i] = orc_sr_bf16(x, r);
    }
}

static double* dalloc(size_t n) {
    return (double*)calloc(n ? n : 1, sizeof(double));
}

/* train_gpt2.cu, gpt2_forward then gpt2_backward: the forward is the encoder,
 * L blocks of ln1 -> qkv -> attention -> attproj -> residual -> ln2 -> fc ->
 * gelu -> fcproj -> residual, then lnf and the tied classifier over all Vp
 * columns.  The backward visits the same steps in reverse, with one residual
 * gradient buffer that the LayerNorm backwards add into. */
double orc_gpt2_step(const orc_config* cfg, const double* params, const int* inputs,
                     const int* targets, int B, int T, double dloss,
                     double* losses_out, double* logits_out, double* grads) {
    int V = cfg->vocab_size, Vp = cfg->padded_vocab_size, L = cfg->num_layers;
    int NH = cfg->num_heads, C = cfg->channels;
    if (B <= 0 || T <= 0 || T > cfg->max_seq_len || C % NH != 0 || V > Vp) return -2.0;
    for (int i = 0; i < B * T; i++) {
        if (inputs[i] < 0 || inputs[i] >= V) return -2.0;
        if (targets && (targets[i] < 0 || targets[i] >= V)) return -2.0;
    }
    size_t off[16], cnt[16];
    orc_param_layout(cfg, off, cnt);
    const double *wte = params + off[0], *wpe = params + off[1];
    const double *ln1w = params + off[2], *ln1b = params + off[3];
    const double *qkvw = params + off[4], *qkvb = params + off[5];
    const double *apw = params + off[6], *apb = params + off[7];
    const double *ln2w = params + off[8], *ln2b = params + off[9];
    const double *fcw = params + off[10], *fcb = params + off[11];
    const double *fpw = params + off[12], *fpb = params + off[13];
    const double *lnfw = params + off[14], *lnfb = params + off[15];

    size_t BT = (size_t)B * T, BTC = BT * C;
    double* encoded = dalloc(BTC);
    double* ln1 = dalloc(L * BTC);
    double* ln1m = dalloc(L * BT);
    double* ln1r = dalloc(L * BT);
    double* qkv = dalloc(L * BTC * 3);
    double* atty = dalloc(L * BTC);
    double* att = dalloc((size_t)L * B * NH * T * T);
    double* attproj = dalloc(BTC);
    double* res2 = dalloc(L * BTC);
    double* ln2 = dalloc(L * BTC);
    double* ln2m = dalloc(L * BT);
    double* ln2r = dalloc(L * BT);
    double* fch = dalloc(L * BTC * 4);
    double* fchg = dalloc(L * BTC * 4);
    double* fcproj = dalloc(BTC);
    double* res3 = dalloc(L * BTC);
    double* lnf = dalloc(BTC);
    double* lnfm = dalloc(BT);
    double* lnfr = dalloc(BT);
    double* logits = dalloc(BT * Vp);
    double* losses = dalloc(BT);

    orc_encoder_forward(encoded, inputs, wte, wpe, B, T, C);
    for (int l = 0; l < L; l++) {
        const double* res = l == 0 ? encoded : res3 + (size_t)(l - 1) * BTC;
        double* l_ln1 = ln1 + l * BTC;
        double* l_qkv = qkv + l * BTC * 3;
        double* l_atty = atty + l * BTC;
        double* l_att = att + (size_t)l * B * NH * T * T;
        double* l_res2 = res2 + l * BTC;
        double* l_ln2 = ln2 + l * BTC;
        double* l_fch = fch + l * BTC * 4;
        double* l_fchg = fchg + l * BTC * 4;
        double* l_res3 = res3 + l * BTC;
        orc_layernorm_forward(l_ln1, ln1m + l * BT, ln1r + l * BT, res, ln1w + (size_t)l * C,
                              ln1b + (size_t)l * C, (int)BT, C);
        orc_matmul_forward(l_qkv, l_ln1, qkvw + (size_t)l * 3 * C * C, qkvb + (size_t)l * 3 * C,
                           (int)BT, C, 3 * C);
        orc_attention_forward(l_atty, l_att, l_qkv, B, T, C, NH);
        orc_matmul_forward(attproj, l_atty, apw + (size_t)l * C * C, apb + (size_t)l * C, (int)BT, C, C);
        orc_residual_forward(l_res2, res, attproj, BTC);
        orc_layernorm_forward(l_ln2, ln2m + l * BT, ln2r + l * BT, l_res2, ln2w + (size_t)l * C,
                              ln2b + (size_t)l * C, (int)BT, C);
        orc_matmul_forward(l_fch, l_ln2, fcw + (size_t)l * 4 * C * C, fcb + (size_t)l * 4 * C,
                           (int)BT, C, 4 * C);
        orc_gelu_forward(l_fchg, l_fch, BTC * 4);
        orc_matmul_forward(fcproj, l_fchg, fpw + (size_t)l * 4 * C * C, fpb + (size_t)l * C,
                           (int)BT, 4 * C, C);
        orc_residual_forward(l_res3, l_res2, fcproj, BTC);
    }
    const double* res_last = res3 + (size_t)(L - 1) * BTC;
    orc_layernorm_forward(lnf, lnfm, lnfr, res_last, lnfw, lnfb, (int)BT, C);
    orc_matmul_forward(logits, lnf, wte, NULL, (int)BT, C, Vp);
    if (logits_out) memcpy(logits_out, logits, BT * Vp * sizeof(double));

    double mean_loss = -1.0;
    if (targets) {
        double* probs = dalloc(BT * Vp);
        mean_loss = orc_crossentropy_forward(losses, probs, logits, targets, (int)BT, V, Vp);
        if (losses_out) memcpy(losses_out, losses, BT * sizeof(double));
        if (grads) {
            double dl = dloss > 0.0 ? dloss : 1.0 / (double)BT;
            double *g_wte = grads + off[0], *g_wpe = grads + off[1];
            double *g_ln1w = grads + off[2], *g_ln1b = grads + off[3];
            double *g_qkvw = grads + off[4], *g_qkvb = grads + off[5];
            double *g_apw = grads + off[6], *g_apb = grads + off[7];
            double *g_ln2w = grads + off[8], *g_ln2b = grads + off[9];
            double *g_fcw = grads + off[10], *g_fcb = grads + off[11];
            double *g_fpw = grads + off[12], *g_fpb = grads + off[13];
            double *g_lnfw = grads + off[14], *g_lnfb = grads + off[15];
            double* dlogits = probs; /* overwritten in place, as the fused classifier does */
            orc_crossentropy_backward(dlogits, probs, targets, dl, (int)BT, V, Vp);
            double* dres = dalloc(BTC);      /* the residual-stream gradient */
            double* dbtc = dalloc(BTC);
            double* dbt4c = dalloc(BTC * 4);
            double* dbt3c = dalloc(BTC * 3);
            orc_matmul_backward(dbtc, g_wte, NULL, dlogits, lnf, wte, (int)BT, C, Vp);
            orc_layernorm_backward(dres, g_lnfw, g_lnfb, dbtc, res_last, lnfw, lnfm, lnfr, (int)BT, C);
            for (int l = L - 1; l >= 0; l--) {
                const double* res = l == 0 ? encoded : res3 + (size_t)(l - 1) * BTC;
                orc_matmul_backward(dbt4c, g_fpw + (size_t)l * 4 * C * C, g_fpb + (size_t)l * C, dres,
                                    fchg + l * BTC * 4, fpw + (size_t)l * 4 * C * C, (int)BT, 4 * C, C);
                orc_gelu_backward(dbt4c, fch + l * BTC * 4, dbt4c, BTC * 4);
                orc_matmul_backward(dbtc, g_fcw + (size_t)l * 4 * C * C, g_fcb + (size_t)l * 4 * C, dbt4c,
                                    ln2 + l * BTC, fcw + (size_t)l * 4 * C * C, (int)BT, C, 4 * C);
                orc_layernorm_backward(dres, g_ln2w + (size_t)l * C, g_ln2b + (size_t)l * C, dbtc,
                                       res2 + l * BTC, ln2w + (size_t)l * C, ln2m + l * BT, ln2r + l * BT,
                                       (int)BT, C);
                orc_matmul_backward(dbtc, g_apw + (size_t)l * C * C, g_apb + (size_t)l * C, dres,
                                    atty + l * BTC, apw + (size_t)l * C * C, (int)BT, C, C);
                orc_attention_backward(dbt3c, dbtc, qkv + l * BTC * 3, att + (size_t)l * B * NH * T * T,
                                       B, T, C, NH);
                orc_matmul_backward(dbtc, g_qkvw + (size_t)l * 3 * C * C, g_qkvb + (size_t)l * 3 * C, dbt3c,
                                    ln1 + l * BTC, qkvw + (size_t)l * 3 * C * C, (int)BT, C, 3 * C);
                orc_layernorm_backward(dres, g_ln1w + (size_t)l * C, g_ln1b + (size_t)l * C, dbtc, res,
                                       ln1w + (size_t)l * C, ln1m + l * BT, ln1r + l * BT, (int)BT, C);
            }
            orc_encoder_backward(g_wte, g_wpe, dres, inputs, B, T, C);
            free(dres); free(dbtc); free(dbt4c); free(dbt3c);
        }
        free(probs);
    }
    free(encoded); free(ln1); free(ln1m); free(ln1r); free(qkv); free(atty); free(att);
    free(attproj); free(res2); free(ln2); free(ln2m); free(ln2r); free(fch); free(fchg);
    free(fcproj); free(res3); free(lnf); free(lnfm); free(lnfr); free(logits); free(losses);
    return mean_loss;
}

/* POPCORNBENCH "Kimi-K2.6 l2_p99" problem statement: a Linear layer
 * (x W^T + b), then GELU (tanh form, as the configs fix it), then softmax over
 * each row. */
void orc_fused_linear_gelu_softmax(double* Y, const double* X, const double* W, const double* b,
                                   int M, int K, int N, const int* rows, int nrows) {
    int R = rows ? nrows : M;
    double* z = (double*)malloc((size_t)N * sizeof(double));
    double* g = (double*)malloc((size_t)N * sizeof(double));
    for (int r = 0; r < R; r++) {
        int m = rows ? rows[r] : r;
        orc_matmul_forward(z, X + (size_t)m * K, W, b, 1, K, N);
        orc_gelu_forward(g, z, (size_t)N);
        double maxv = -INFINITY;
        for (int j = 0; j < N; j++) if (g[j] > maxv) maxv = g[j];
        double sum = 0.0;
        for (int j = 0; j < N; j++) sum += exp(g[j] - maxv);
        for (int j = 0; j < N; j++) Y[(size_t)r * N + j] = exp(g[j] - maxv) / sum;
    }
    free(z);
    free(g);
}
