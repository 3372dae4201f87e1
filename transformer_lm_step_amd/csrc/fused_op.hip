// fused_op.hip - Y = softmax_row(GELU_tanh(X W^T + b)) in fp32 (gfx950).
//
// The operation of the POPCORNBENCH l12_default_gpt trajectory page (its
// problem statement: a Linear layer, then tanh-form GELU, then a softmax over
// each output row; X [M,K], W [N,K] as nn.Linear stores it, b [N]).
//
// Two launches.  The fp32-MFMA product kernel applies bias and GELU in its
// epilogue, stores G, and leaves per row and per 64-column block the pair
// (max_j G, sum_j exp(G - max)); so no pass over G is needed to find the row
// maximum.  The second kernel merges a row's pairs (m, s) into the row's
// (M, S = sum s exp(m - M)) in a fixed order and rewrites the row in place as
// exp(G - M) / S.  HBM traffic beyond the product: G written once, read and
// rewritten once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device.h"
#include "gpt2.h"
#include "gpt2_ops.h"
#include "kernels.h"

namespace {

// (m, s) pairs combine as m = max(m1, m2), s = s1 exp(m1 - m) + s2 exp(m2 - m);
// a pair with s = 0 (no columns) is the identity.
DEV float2 smx_merge(float2 a, float2 b) {
    if (a.y == 0.f) return b;
    if (b.y == 0.f) return a;
    const float m = fmaxf(a.x, b.x);
    return make_float2(m, a.y * expf(a.x - m) + b.y * expf(b.x - m));
}

// one 256-thread workgroup per row
__global__ __launch_bounds__(256) void softmax_finish_kernel(float* __restrict__ Y, const float2* __restrict__ part,
                                                             int N, int np) {
    __shared__ float2 red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const float2* pr = part + (size_t)row * np;
    float2 acc = make_float2(-INFINITY, 0.f);
    for (int i = tid; i < np; i += 256) acc = smx_merge(acc, pr[i]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        float2 other;
        other.x = __shfl_xor(acc.x, o, 64);
        other.y = __shfl_xor(acc.y, o, 64);
        acc = smx_merge(acc, other);
    }
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    acc = smx_merge(smx_merge(red[0], red[1]), smx_merge(red[2], red[3]));
    const float mx = acc.x, inv = 1.0f / acc.y;
    float* y = Y + (size_t)row * N;
    for (int c = 4 * tid; c < N; c += 4 * 256) {
        float v[4];
        load4<float>(y + c, v);
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = expf(v[r] - mx) * inv;
        store4<float>(y + c, v);
    }
}

bool al(const void* p) { return ((uintptr_t)p % 256) == 0; }

}  // namespace

int softmax_finish_launch(float* Y, const float2* part, int M, int N, int np, hipStream_t s) {
    if (M <= 0) return 0;
    hipLaunchKernelGGL(softmax_finish_kernel, dim3(M), dim3(256), 0, s, Y, part, N, np);
    return (int)hipGetLastError();
}

extern "C" size_t fused_linear_gelu_softmax_f32_workspace(int M, int N) {
    if (M <= 0 || N <= 0) return 0;
    return (size_t)M * (size_t)((N + 63) / 64) * sizeof(float2);
}

extern "C" int fused_linear_gelu_softmax_f32(const float* X, const float* W, const float* b, float* Y, int M, int K,
                                             int N, void* work, size_t work_bytes, void* hip_stream) {
    if (M < 0 || N <= 0 || K <= 0) return GPT2_E_ARG;
    if (M == 0) return GPT2_OK;
    if (!X || !W || !b || !Y || !work) return GPT2_E_ARG;
    if (K % 8 || N % 8) return GPT2_E_SHAPE;
    if (!al(X) || !al(W) || !al(b) || !al(Y) || !al(work)) return GPT2_E_ALIGN;
    if (work_bytes < fused_linear_gelu_softmax_f32_workspace(M, N)) return GPT2_E_ARG;
    const int np = (N + 63) / 64;
    hipStream_t s = (hipStream_t)hip_stream;
    GemmDesc d = {};
    d.M = M; d.N = N; d.K = K;
    d.A = X; d.lda = K; d.a_kmajor = 1;
    d.B = W; d.ldb = K; d.b_kmajor = 1;
    d.C = Y; d.ldc = N;
    d.epi = GEMM_BIAS_GELU_SMX; d.alpha = 1.0f;
    d.bias = b; d.aux_out = work; d.ldaux = np;
    if (gemm_launch(d, 4, nullptr, 0, 256, s) != 0) return GPT2_E_HIP;
    if (softmax_finish_launch(Y, (const float2*)work, M, N, np, s) != 0) return GPT2_E_HIP;
    return GPT2_OK;
}
