// ops_api.hip - standalone entry points of single operations (include/gpt2_ops.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gpt2.h"
#include "gpt2_ops.h"
#include "kernels.h"

namespace {
bool al(const void* p) { return ((uintptr_t)p % 256) == 0; }
}

extern "C" int gpt2_linear_forward(int precision, const void* x, const void* w, const void* bias, void* y, int M,
                                   int N, int K, void* hip_stream) {
    if (precision != GPT2_FP32 && precision != GPT2_BF16) return GPT2_E_ARG;
    if (!x || !w || !y || M < 0 || N < 0 || K < 0) return GPT2_E_ARG;
    if (K % 8 || N % 8) return GPT2_E_SHAPE;
    if (!al(x) || !al(w) || !al(y) || (bias && !al(bias))) return GPT2_E_ALIGN;
    GemmDesc d = {};
    d.M = M; d.N = N; d.K = K;
    d.A = x; d.lda = K; d.a_kmajor = 1;
    d.B = w; d.ldb = K; d.b_kmajor = 1;
    d.C = y; d.ldc = N; d.epi = bias ? GEMM_BIAS : GEMM_STORE; d.alpha = 1.0f;
    d.bias = bias; d.ldaux = N;
    const int e = gemm_launch(d, precision == GPT2_BF16 ? 2 : 4, nullptr, 0, 256, (hipStream_t)hip_stream);
    return e == 0 ? GPT2_OK : GPT2_E_HIP;
}
