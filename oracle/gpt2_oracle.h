/*
 * gpt2_oracle.h - CPU oracle for the GPT-2 training step (TEST INFRASTRUCTURE).
 *
 * This is the checker, not the product.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant with the HIP library; neither includes the other.
 *
 * Everything here is plain, single-threaded C in double precision, written out
 * from the definitions on the train_gpt2.cu page (llm.c, mixed-precision
 * version), cross-checked against the train_gpt2_fp32.cu page where that page
 * is legible, and from the Linear -> GELU -> softmax problem statement on the
 * POPCORNBENCH "Kimi-K2.6 l2_p99" transcript page.  All tensors are row-major,
 * host memory, caller-owned.  Functions documented "+=" add into their output;
 * "=" overwrite it.
 */
#ifndef GPT2_ORACLE_H
#define GPT2_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int max_seq_len;       /* maxT */
    int vocab_size;        /* V */
    int padded_vocab_size; /* Vp >= V */
    int num_layers;        /* L */
    int num_heads;         /* NH */
    int channels;          /* C */
} orc_config;

/* The 16 parameter tensors in the pages' order (GPT2 ParameterTensors,
 * fill_in_parameter_sizes): wte, wpe, ln1w, ln1b, qkvw, qkvb, attprojw,
 * attprojb, ln2w, ln2b, fcw, fcb, fcprojw, fcprojb, lnfw, lnfb.
 * Writes element offsets and counts; returns the total parameter count. */
size_t orc_param_layout(const orc_config* cfg, size_t offset[16], size_t count[16]);

/* Token + position encoding: out[b,t,:] = wte[tok[b,t],:] + wpe[t,:]  (=). */
void orc_encoder_forward(double* out, const int* tok, const double* wte, const double* wpe,
                         int B, int T, int C);
/* dwte[tok[b,t],:] += dout[b,t,:];  dwpe[t,:] += dout[b,t,:]. */
void orc_encoder_backward(double* dwte, double* dwpe, const double* dout, const int* tok,
                          int B, int T, int C);

/* LayerNorm over the last axis of x [N,C], eps 1e-5, biased variance (=).
 * mean and rstd [N] may be NULL. */
void orc_layernorm_forward(double* out, double* mean, double* rstd, const double* x,
                           const double* w, const double* b, int N, int C);
/* LayerNorm backward: dx += ..., dw += ..., db += ... . */
void orc_layernorm_backward(double* dx, double* dw, double* db, const double* dout,
                            const double* x, const double* w, const double* mean,
                            const double* rstd, int N, int C);

/* out[n,o] = sum_k x[n,k] w[o,k] + bias[o]  (=); bias may be NULL.
 * x [N,K], w [OC,K] (out, in) row-major, out [N,OC]. */
void orc_matmul_forward(double* out, const double* x, const double* w, const double* bias,
                        int N, int K, int OC);
/* dx[n,k] = sum_o dout[n,o] w[o,k]  (=; dx may be NULL)
 * dw[o,k] += sum_n dout[n,o] x[n,k]  (dw may be NULL)
 * db[o]   += sum_n dout[n,o]         (db may be NULL). */
void orc_matmul_backward(double* dx, double* dw, double* db, const double* dout,
                         const double* x, const double* w, int N, int K, int OC);

/* Causal multi-head attention.  qkv [B,T,3C] holds q | k | v, each split into
 * NH heads of HS = C/NH channels.  out [B,T,C] (=); att [B,NH,T,T] (=) receives
 * the softmax probabilities, exactly 0 above the diagonal. */
void orc_attention_forward(double* out, double* att, const double* qkv,
                           int B, int T, int C, int NH);
/* Backward of the above given dout [B,T,C]; dqkv [B,T,3C]  (=). */
void orc_attention_backward(double* dqkv, const double* dout, const double* qkv,
                            const double* att, int B, int T, int C, int NH);

/* GELU, tanh form (=). */
void orc_gelu_forward(double* out, const double* x, size_t n);
/* dx[i] = gelu'(x[i]) * dout[i]  (=). */
void orc_gelu_backward(double* dx, const double* x, const double* dout, size_t n);

/* out = a + b  (=). */
void orc_residual_forward(double* out, const double* a, const double* b, size_t n);

/* Softmax cross-entropy over the first V of Vp columns of logits [N,Vp].
 * losses [N] (=); probs [N,Vp] (=, may be NULL; padded columns 0).
 * Returns the mean loss. */
double orc_crossentropy_forward(double* losses, double* probs, const double* logits,
                                const int* targets, int N, int V, int Vp);
/* dlogits[n,i] = (p[n,i] - [i == target]) * dloss for i < V, 0 for i >= V (=). */
void orc_crossentropy_backward(double* dlogits, const double* probs, const int* targets,
                               double dloss, int N, int V, int Vp);

/* AdamW with bias correction and decoupled weight decay; t is 1-based. */
void orc_adamw(double* params, const double* grads, double* m, double* v, size_t n,
               double lr, double beta1, double beta2, double eps, double weight_decay, int t);

/* One GPT-2 micro-step on a batch.  params: flat, in orc_param_layout order.
 * targets may be NULL (forward only, returns -1).  losses [B*T] may be NULL.
 * logits [B*T*Vp] may be NULL: if given it receives the classifier output.
 * grads: NULL for forward only, else parameter gradients are ADDED (+=) with
 * the loss scaled by dloss (dloss <= 0 means 1/(B*T)).
 * Returns the mean loss over the B*T positions, or -1 without targets,
 * or -2 on a bad argument. */
double orc_gpt2_step(const orc_config* cfg, const double* params, const int* inputs,
                     const int* targets, int B, int T, double dloss,
                     double* losses, double* logits, double* grads);

/* Standalone op: Y[m,:] = softmax_row(gelu_tanh(X[m,:] W^T + b)).
 * X [M,K], W [N,K], b [N], Y [M,N].  rows: compute only the listed rows
 * (nrows of them, Y row r of the output holds X row rows[r]); rows NULL means
 * all M rows in order. */
void orc_fused_linear_gelu_softmax(double* Y, const double* X, const double* W, const double* b,
                                   int M, int K, int N, const int* rows, int nrows);

/* train_gpt2.cu, adamw_kernel3 without master weights: the bf16 parameters
 * (bit patterns) updated in fp32 -- the page's precision, since the fp32
 * value decides the stochastic rounding -- and rounded back stochastically
 * with SquirrelNoise5 noise; see gpt2_oracle.c.  m, v are fp32, "=". */
void orc_adamw_sr(uint16_t* params, const float* grads, float* m, float* v, size_t n, float lr, float beta1,
                  float beta2, float eps, float weight_decay, int t, uint32_t seed);
/* train_gpt2.cu, random_u32 (xorshift*) and Get2dNoiseUint (SquirrelNoise5). */
uint32_t orc_xorshift_u32(uint64_t* state);
uint32_t orc_noise2d(int x, int y, uint32_t seed);
/* train_gpt2.cu, stochastic_rounding of x with threshold r < 2^16 (bf16 bits). */
uint16_t orc_sr_bf16(float x, uint32_t r);

#ifdef __cplusplus
}
#endif
#endif
