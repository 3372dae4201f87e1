/*
 * gpt2_ops.h - single operations of the GPT-2 step as standalone entry points.
 *
 * Each entry point launches exactly the kernels, in exactly the launch
 * configuration, that gpt2_forward / gpt2_backward use for that operation, on
 * caller-owned device memory (256-byte aligned, row-major), asynchronously on
 * hip_stream.  They exist so that one operation can be checked and timed on
 * its own at full size.  Return: GPT2_OK or a GPT2_E_* code (see gpt2.h).
 */
#ifndef GPT2_MI355X_OPS_H
#define GPT2_MI355X_OPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* train_gpt2.cu, matmul_forward_cublaslt: y[M,N] = x[M,K] w[N,K]^T (+ bias[N]
 * when d_bias is not NULL).  precision GPT2_FP32 (fp32 tensors) or GPT2_BF16
 * (bf16 tensors, fp32 accumulation).  K and N multiples of 8.
 * Errors: GPT2_E_ARG, GPT2_E_SHAPE, GPT2_E_ALIGN, GPT2_E_HIP. */
int gpt2_linear_forward(int precision, const void* d_x, const void* d_w, const void* d_bias, void* d_y,
                        int M, int N, int K, void* hip_stream);

/* train_gpt2.cu, matmul_backward (with matmul_backward_bias_kernel4), for
 * y = x w^T + b with x [M,K], w [N,K]:
 *   dx[M,K]  = alpha * dy[M,N] w[N,K]            (overwrite; skipped if d_dx NULL)
 *   dw[N,K] += alpha * dy[M,N]^T x[M,K]          (fp32, accumulate; skipped if d_dw NULL)
 *   db[N]   += alpha * sum over rows of dy       (fp32, accumulate; needs d_dw)
 * dy, x, w, dx in the precision's type.  K and N multiples of 8.  d_work:
 * device workspace of gpt2_linear_backward_workspace() bytes (may be NULL
 * when that is 0).  Errors: GPT2_E_ARG, GPT2_E_SHAPE, GPT2_E_ALIGN, GPT2_E_HIP. */
int gpt2_linear_backward(int precision, const void* d_dy, const void* d_x, const void* d_w, void* d_dx,
                         float* d_dw, float* d_db, int M, int N, int K, float alpha, void* d_work,
                         size_t work_bytes, void* hip_stream);
size_t gpt2_linear_backward_workspace(int precision, int M, int N, int K);

/* train_gpt2.cu, attention_forward (permute, Q K^T, softmax_forward_kernel5
 * with the causal mask, P V, unpermute): for every batch b and head h, with
 * q, k, v the channel slices h*HS .. h*HS+HS-1 (HS = C/NH) of the three
 * thirds of qkv [B,T,3C],
 *   out[b,t,h*HS + d] = sum_{s <= t} softmax_s(q_t . k_s / sqrt(HS)) v_s[d],
 * out [B,T,C].  d_lse [B,NH,T] fp32 receives log2 of each row's softmax
 * denominator, log2(sum_{s <= t} exp(q_t . k_s / sqrt(HS))), which
 * gpt2_attention_backward reads.  precision GPT2_FP32 or GPT2_BF16 (bf16
 * qkv and out, fp32 scores and accumulation).  HS in {16, 32, 64, 128}.
 * Errors: GPT2_E_ARG (bad precision, NULL pointer, non-positive sizes),
 * GPT2_E_SHAPE (C not a multiple of NH or unsupported HS), GPT2_E_ALIGN,
 * GPT2_E_HIP. */
int gpt2_attention_forward(int precision, const void* d_qkv, void* d_out, float* d_lse, int B, int T, int C, int NH,
                           void* hip_stream);

/* train_gpt2.cu, attention_backward (softmax_autoregressive_backward_kernel
 * and the four batched products): dqkv [B,T,3C] (overwritten) = the gradient
 * of sum(out * dout) with respect to qkv, from dout [B,T,C] and the
 * forward's qkv, out and lse.  d_delta: B*NH*T fp32 workspace (per-row
 * sum of dout * out; contents on return unspecified).  Types, HS and errors
 * as gpt2_attention_forward. */
int gpt2_attention_backward(int precision, const void* d_dout, const void* d_qkv, const void* d_out,
                            const float* d_lse, void* d_dqkv, float* d_delta, int B, int T, int C, int NH,
                            void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results as gpt2_attention_backward, with the delta array taken
 * from a fixed device array inside the library (one per GPU, 4 MiB, held until
 * the process ends) instead of a caller workspace.  No allocation of any kind.
 * Runs on the current device (hip_stream must belong to it); the first call on
 * a device looks the array's address up.  B*NH*T may be at most 1048576
 * (GPT2_E_SHAPE otherwise).  Every call on one GPU shares that array: calls
 * that overlap on one GPU (other streams, other threads) race and give wrong
 * gradients.  Other arguments and errors as gpt2_attention_backward. */
int gpt2_attention_backward_noalloc(int precision, const void* d_dout, const void* d_qkv, const void* d_out,
                                    const float* d_lse, void* d_dqkv, int B, int T, int C, int NH,
                                    void* hip_stream);

/* POPCORNBENCH l12_default_gpt trajectory page, the problem statement (a
 * Linear layer followed by tanh-form GELU and a softmax over dim 1), in fp32:
 *   Y[m, :] = softmax_n( GELU_tanh( sum_k X[m,k] W[n,k] + b[n] ) )
 * X [M,K], W [N,K] (out, in), b [N], Y [M,N], all fp32 row-major device
 * memory owned by the caller; products use fp32 MFMA with fp32 accumulation
 * (no reduced-precision inputs).  d_work: device workspace of at least
 * fused_linear_gelu_softmax_f32_workspace(M, N) bytes (per-row, per-64-column
 * softmax partials; contents on return are unspecified).  K and N multiples of
 * 8; M == 0 is a no-op.  Asynchronous on hip_stream.
 * Errors: GPT2_E_ARG (NULL pointer, non-positive K or N, negative M, workspace
 * too small), GPT2_E_SHAPE, GPT2_E_ALIGN, GPT2_E_HIP. */
int fused_linear_gelu_softmax_f32(const float* d_X, const float* d_W, const float* d_b, float* d_Y, int M, int K,
                                  int N, void* d_work, size_t work_bytes, void* hip_stream);
size_t fused_linear_gelu_softmax_f32_workspace(int M, int N);

#ifdef __cplusplus
}
#endif
#endif
