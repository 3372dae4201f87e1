// kernels.h - host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef uint16_t bf16_t;

// ---------------------------------------------------------------- GEMM ------
// C[m,n] (op)= alpha * sum_k A(m,k) B(k,n), every matrix row-major.
//  A(m,k) = a_kmajor ? A[m*lda + k] : A[k*lda + m]
//  B(k,n) = b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
// Epilogues (per output element v = alpha * acc):
enum GemmEpi {
    GEMM_STORE = 0,      // C = v
    GEMM_BIAS = 1,       // C = v + bias[n]
    GEMM_BIAS_GELU = 2,  // aux_out = v + bias[n]; C = gelu(aux_out)
    GEMM_BIAS_RESID = 3, // C = aux_in + v + bias[n]
    GEMM_GELU_BWD = 4,   // C = v * gelu'(aux_in)
    GEMM_ACCUM = 5,      // C (fp32) += v
    GEMM_BIAS_GELU_SMX = 6,  // C = gelu(v + bias[n]); aux_out (float2, ldaux per row) gets, per row
                             // and 64-column block j, (max, sum exp(C - max)) over that block
};
struct GemmDesc {
    int M, N, K;
    const void* A; long lda; int a_kmajor;
    const void* B; long ldb; int b_kmajor;
    void* C; long ldc;        // C element type: the activation type, or fp32 for GEMM_ACCUM
    int epi;
    float alpha;
    const void* bias;         // activation/param type, [N]
    const void* aux_in;       // activation type, ld = ldaux
    void* aux_out;            // activation type, ld = ldaux
    long ldaux;
    float* dbias;             // GEMM_ACCUM only (may be NULL): dbias[m] += alpha * sum_k A(m,k)
    int split_ok;             // GEMM_STORE / GEMM_ACCUM may split K (needs workspace)
};
// Weight-gradient products of several layers in one launch (bf16 operands,
// both contraction-strided; fp32 gradients):
//   C_l[m,n] += alpha * sum_k A_l[k*lda + m] * B_l[k*ldb + n]
//   dbias_l[m] += alpha * sum_k A_l[k*lda + m]          (when dbias != NULL)
// for product l = 0 .. count-1 of each item, with X_l = X + l * sX (elements).
// Up to 8 items; no K split and no workspace (one tile per workgroup over the
// whole contraction; tile 0: 256x256 with 128x64 outputs per wave, tile 1:
// 128x256 with 64x64 per wave).  Returns 0 or a hipError_t.
struct GemmGroupItem {
    const void* A; long lda; long sA;
    const void* B; long ldb; long sB;
    float* C; long ldc; long sC;
    float* dbias; long sBias;
    int M, N, K, count;
    float alpha;
};
int gemm_dw_group_launch(const GemmGroupItem* items, int n, hipStream_t s, int tile = 0);
// Workgroups (tiles) such a launch takes.
long gemm_dw_group_tiles(const GemmGroupItem* items, int n, int tile);
// Row softmax from the per-64-column partials of GEMM_BIAS_GELU_SMX:
// Y[m, :] = exp(Y[m, :] - M_m) / S_m, in place (fp32, N % 4 == 0).
int softmax_finish_launch(float* Y, const float2* part, int M, int N, int np, hipStream_t s);

// Workspace (fp32) needed by gemm_launch for split-K (0 if it will not split).
size_t gemm_workspace_bytes(const GemmDesc& d, int elem_bytes, int num_cus);
// Returns 0 or a hipError_t.  ws may be NULL if gemm_workspace_bytes(d) == 0.
int gemm_launch(const GemmDesc& d, int elem_bytes, float* ws, size_t ws_bytes, int num_cus, hipStream_t s);


// ---------------------------------------------------------- LayerNorm -------
template <typename T>
int layernorm_fwd_launch(T* out, float* mean, float* rstd, const T* x, const T* w, const T* b,
                         int N, int C, hipStream_t s);
// dres (fp32) = (accumulate ? dres : 0) + dx; dres_lp (may be NULL) = T(dres).
// The weight and bias column sums of each workgroup's rows go to `partial`:
// layernorm_bwd_partial_rows(N, C, sizeof(T)) rows of 2C floats (weight sums,
// then bias).
template <typename T>
int layernorm_bwd_launch(float* dres, T* dres_lp, const T* dy, const T* x, const T* w, const float* mean,
                         const float* rstd, int N, int C, int accumulate, float* partial, hipStream_t s);
int layernorm_bwd_partial_rows(int N, int C, int esz);
// For slots j = 0 .. slots-1 (LayerNorm backwards of N rows whose partial
// rows lie one after another, slot j at partial + j * rows * 2C):
// dw[j][c] += sum of the slot's weight sums, db[j][c] += of its bias sums
// (fp32), each in workgroup order.
constexpr int kMaxLnSlots = 128;
struct LnFinishArgs {
    float* dw[kMaxLnSlots];
    float* db[kMaxLnSlots];
};
int layernorm_bwd_finish_launch(const LnFinishArgs& a, int slots, const float* partial, int N, int C, int esz,
                                hipStream_t s);

// ---------------------------------------------------------- attention -------
// qkv [B,T,3C] -> out [B,T,C], lse [B,NH,T] (base-2 log-sum-exp of the scaled scores)
template <typename T>
int attention_fwd_launch(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s);
// dqkv [B,T,3C] (=) from dout [B,T,C]; delta [B,NH,T] fp32 scratch.
template <typename T>
int attention_bwd_launch(T* dqkv, float* delta, const T* dout, const T* out, const T* qkv,
                         const float* lse, int B, int T_, int C, int NH, hipStream_t s);

// ------------------------------------------------------- elementwise etc. ---
template <typename T>
int encoder_fwd_launch(T* out, int* tok_copy, const int* tok, const T* wte, const T* wpe,
                       int B, int T_, int C, int V, int* flag, hipStream_t s);
// dwte[tok] += dres rows, dwpe[t] += sum_b dres; fp32.  tok already clamped.
// work: encoder_bwd_workspace_bytes(B*T, C) bytes (256-aligned).
int encoder_bwd_launch(float* dwte, float* dwpe, const float* dres, const int* tok,
                       int B, int T_, int C, void* work, hipStream_t s);
size_t encoder_bwd_workspace_bytes(int BT, int C);
// in place: logits -> softmax - onehot (padded columns 0); losses [N] fp32
template <typename T>
int classifier_ce_launch(T* logits, float* losses, const int* targets, int N, int V, int Vp,
                         int* flag, hipStream_t s);
int mean_launch(float* out, const float* x, int n, hipStream_t s);

// tokens[b*T + t] = the token drawn from softmax(logits[b, t-1, :V]) with coins[b]
template <typename T>
int sample_launch(int32_t* tokens, const T* logits, const float* coins, int B, int T_, int t, int V, int Vp,
                  hipStream_t s);
template <typename PT>
int adamw_launch(PT* params, float* master, const float* grads, float* m, float* v, size_t n,
                 float lr, float beta1, float beta2, float c1, float c2, float eps, float wd,
                 hipStream_t s);
// bf16 parameters without master weights, stochastic rounding seeded by seed
int adamw_sr_launch(bf16_t* params, const float* grads, float* m, float* v, size_t n, float lr, float b1, float b2,
                    float c1, float c2, float eps, float wd, uint32_t seed, hipStream_t s);
int fill_f32_launch(float* p, float value, size_t n, hipStream_t s);
int fill_i32_launch(int* p, int value, size_t n, hipStream_t s);
int cast_f32_to_bf16_launch(bf16_t* dst, const float* src, size_t n, hipStream_t s);
