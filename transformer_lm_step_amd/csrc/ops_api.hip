// ops_api.hip - standalone entry points of single operations (include/gpt2_ops.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

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

namespace {
GemmDesc bwd_dx_desc(const void* dy, const void* w, void* dx, int M, int N, int K, float alpha) {
    GemmDesc d = {};
    d.M = M; d.N = K; d.K = N;
    d.A = dy; d.lda = N; d.a_kmajor = 1;
    d.B = w; d.ldb = K; d.b_kmajor = 0;
    d.C = dx; d.ldc = K; d.epi = GEMM_STORE; d.alpha = alpha; d.ldaux = K;
    d.split_ok = 1;
    return d;
}
GemmDesc bwd_dw_desc(const void* dy, const void* x, float* dw, float* db, int M, int N, int K, float alpha) {
    GemmDesc d = {};
    d.M = N; d.N = K; d.K = M;
    d.A = dy; d.lda = N; d.a_kmajor = 0;
    d.B = x; d.ldb = K; d.b_kmajor = 0;
    d.C = dw; d.ldc = K; d.epi = GEMM_ACCUM; d.alpha = alpha; d.dbias = db;
    d.split_ok = 1;
    return d;
}
}  // namespace

// bf16 weight gradients run as the step runs them: the grouped weight-gradient
// launch (one product, whole contraction per tile, no workspace); fp32 ones
// through the K-split products
extern "C" size_t gpt2_linear_backward_workspace(int precision, int M, int N, int K) {
    const int esz = precision == GPT2_BF16 ? 2 : 4;
    const size_t a = gemm_workspace_bytes(bwd_dx_desc(nullptr, nullptr, nullptr, M, N, K, 1.f), esz, 256);
    const size_t b = esz == 2 ? 0 : gemm_workspace_bytes(bwd_dw_desc(nullptr, nullptr, nullptr, nullptr, M, N, K, 1.f),
                                                         esz, 256);
    return a > b ? a : b;
}

extern "C" int gpt2_linear_backward(int precision, const void* dy, const void* x, const void* w, void* dx, float* dw,
                                    float* db, int M, int N, int K, float alpha, void* work, size_t work_bytes,
                                    void* hip_stream) {
    if (precision != GPT2_FP32 && precision != GPT2_BF16) return GPT2_E_ARG;
    if (!dy || M < 0 || N < 0 || K < 0 || (dx && !w) || (dw && !x) || (db && !dw)) return GPT2_E_ARG;
    if (K % 8 || N % 8) return GPT2_E_SHAPE;
    if (!al(dy) || (x && !al(x)) || (w && !al(w)) || (dx && !al(dx)) || (dw && !al(dw)) || (db && !al(db)) ||
        (work && !al(work)))
        return GPT2_E_ALIGN;
    const int esz = precision == GPT2_BF16 ? 2 : 4;
    hipStream_t s = (hipStream_t)hip_stream;
    if (dx) {
        const GemmDesc d = bwd_dx_desc(dy, w, dx, M, N, K, alpha);
        const size_t need = gemm_workspace_bytes(d, esz, 256);
        if (need > 0 && (work == nullptr || work_bytes < need)) return GPT2_E_ARG;
        if (gemm_launch(d, esz, (float*)work, work_bytes, 256, s) != 0) return GPT2_E_HIP;
    }
    if (dw && esz == 2) {
        GemmGroupItem it = {};
        it.A = dy; it.lda = N; it.B = x; it.ldb = K; it.C = dw; it.ldc = K; it.dbias = db;
        it.M = N; it.N = K; it.K = M; it.count = 1; it.alpha = alpha;
        // 128x256 tiles (half the work each, about 0.71 of a 256x256 tile's
        // time) where they take fewer rounds of the 256 CUs' worth
        const long r0 = (gemm_dw_group_tiles(&it, 1, 0) + 255) / 256, r1 = (gemm_dw_group_tiles(&it, 1, 1) + 255) / 256;
        const int tile = 0.71 * (double)r1 < (double)r0 - 0.1 ? 1 : 0;
        if (gemm_dw_group_launch(&it, 1, s, tile) != 0) return GPT2_E_HIP;
    } else if (dw) {
        const GemmDesc d = bwd_dw_desc(dy, x, dw, db, M, N, K, alpha);
        const size_t need = gemm_workspace_bytes(d, esz, 256);
        if (need > 0 && (work == nullptr || work_bytes < need)) return GPT2_E_ARG;
        if (gemm_launch(d, esz, (float*)work, work_bytes, 256, s) != 0) return GPT2_E_HIP;
    }
    return GPT2_OK;
}

namespace {
int attn_args(int precision, int B, int T, int C, int NH) {
    if (precision != GPT2_FP32 && precision != GPT2_BF16) return GPT2_E_ARG;
    if (B <= 0 || T <= 0 || C <= 0 || NH <= 0) return GPT2_E_ARG;
    if (C % NH) return GPT2_E_SHAPE;
    const int hs = C / NH;
    if (hs != 16 && hs != 32 && hs != 64 && hs != 128) return GPT2_E_SHAPE;
    return GPT2_OK;
}
}  // namespace

extern "C" int gpt2_attention_forward(int precision, const void* qkv, void* out, float* lse, int B, int T, int C,
                                      int NH, void* hip_stream) {
    const int e = attn_args(precision, B, T, C, NH);
    if (e != GPT2_OK) return e;
    if (!qkv || !out || !lse) return GPT2_E_ARG;
    if (!al(qkv) || !al(out) || !al(lse)) return GPT2_E_ALIGN;
    const hipStream_t s = (hipStream_t)hip_stream;
    const int r = precision == GPT2_BF16
                      ? attention_fwd_launch<bf16_t>((bf16_t*)out, lse, (const bf16_t*)qkv, B, T, C, NH, s)
                      : attention_fwd_launch<float>((float*)out, lse, (const float*)qkv, B, T, C, NH, s);
    return r == 0 ? GPT2_OK : GPT2_E_HIP;
}

extern "C" int gpt2_attention_backward(int precision, const void* dout, const void* qkv, const void* out,
                                       const float* lse, void* dqkv, float* delta, int B, int T, int C, int NH,
                                       void* hip_stream) {
    const int e = attn_args(precision, B, T, C, NH);
    if (e != GPT2_OK) return e;
    if (!dout || !qkv || !out || !lse || !dqkv || !delta) return GPT2_E_ARG;
    if (!al(dout) || !al(qkv) || !al(out) || !al(lse) || !al(dqkv) || !al(delta)) return GPT2_E_ALIGN;
    const hipStream_t s = (hipStream_t)hip_stream;
    const int r = precision == GPT2_BF16
                      ? attention_bwd_launch<bf16_t>((bf16_t*)dqkv, delta, (const bf16_t*)dout, (const bf16_t*)out,
                                                     (const bf16_t*)qkv, lse, B, T, C, NH, s)
                      : attention_bwd_launch<float>((float*)dqkv, delta, (const float*)dout, (const float*)out,
                                                    (const float*)qkv, lse, B, T, C, NH, s);
    return r == 0 ? GPT2_OK : GPT2_E_HIP;
}

// ------------------------------------------------ allocation-free variant ---
// The attention backward's only scratch is the per-row delta array (B*NH*T
// fp32).  gpt2_attention_backward_noalloc keeps it in this fixed device array
// instead of a caller workspace: one copy per GPU, alive until the process
// ends, shared by every call on that GPU.
constexpr long kNoAllocDeltaMax = 1L << 20;  // fp32 elements: 4 MiB
static __device__ __align__(256) float scratch[kNoAllocDeltaMax];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices];  // device address of scratch, per device

// The device address of the current device's copy of scratch (looked up on
// the first call on that device).  In host code the array's own name is not
// a device address, so kernels get this pointer instead.
int scratch_address(float** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GPT2_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GPT2_E_HIP;
        g_scratch_dev[dev] = (float*)p;
    }
    *out = g_scratch_dev[dev];
    return GPT2_OK;
}
}  // namespace

extern "C" int gpt2_attention_backward_noalloc(int precision, const void* dout, const void* qkv, const void* out,
                                               const float* lse, void* dqkv, int B, int T, int C, int NH,
                                               void* hip_stream) {
    const int e = attn_args(precision, B, T, C, NH);
    if (e != GPT2_OK) return e;
    if ((long)B * NH * T > kNoAllocDeltaMax) return GPT2_E_SHAPE;
    if (!dout || !qkv || !out || !lse || !dqkv) return GPT2_E_ARG;
    if (!al(dout) || !al(qkv) || !al(out) || !al(lse) || !al(dqkv)) return GPT2_E_ALIGN;
    float* delta = nullptr;
    const int a = scratch_address(&delta);
    if (a != GPT2_OK) return a;
    const hipStream_t s = (hipStream_t)hip_stream;
    const int r = precision == GPT2_BF16
                      ? attention_bwd_launch<bf16_t>((bf16_t*)dqkv, delta, (const bf16_t*)dout, (const bf16_t*)out,
                                                     (const bf16_t*)qkv, lse, B, T, C, NH, s)
                      : attention_bwd_launch<float>((float*)dqkv, delta, (const float*)dout, (const float*)out,
                                                    (const float*)qkv, lse, B, T, C, NH, s);
    return r == 0 ? GPT2_OK : GPT2_E_HIP;
}
