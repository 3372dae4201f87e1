// sample.hip - drawing the next token from the logits (gfx950).
//
// train_gpt2.cu, sample_softmax and the generation loop: the token at position t
// of batch row b is drawn from softmax(logits[b, t-1, :V]) by inverse CDF with a
// caller-supplied coin in [0, 1).  Here the draw runs on the device, one
// workgroup per batch row, so a generation loop needs no host round trip per
// token.  Probabilities p_i = exp(z_i - max z) and their running sums are
// fp64 (the page accumulates the normaliser in double; subtracting the maximum
// changes nothing in exact arithmetic and keeps every exponential finite).
//
// Order of the sums (fixed, so the draw is deterministic): wave w of the 16
// owns the contiguous segment [w*seg, (w+1)*seg) of the V columns (seg a
// multiple of 64) and reads it 64 consecutive columns at a time (coalesced).
// Pass 1: the row maximum.  Pass 2: each wave's segment total (per-lane sums,
// then a fixed-order wave reduction); Z = the totals added in wave order.
// Pass 3: each wave walks its segment again from the prefix of the totals
// before it, with an in-wave inclusive scan per 64 columns; the CDF value at i
// is that prefix plus the scanned sum up to i.  The token is the smallest i
// with coin * Z < cdf_i, V - 1 if none.
#include <math.h>

#include "device.h"
#include "kernels.h"

namespace {

constexpr int SAMPLE_WAVES = 16;

DEV double shfl_up_f64(double v, int d) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = __shfl_up((uint32_t)u, d, 64), hi = __shfl_up((uint32_t)(u >> 32), d, 64);
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
DEV double shfl_xor_f64(double v, int d) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = __shfl_xor((uint32_t)u, d, 64), hi = __shfl_xor((uint32_t)(u >> 32), d, 64);
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

template <typename T>
__global__ __launch_bounds__(64 * SAMPLE_WAVES) void sample_kernel(int32_t* __restrict__ tokens,
                                                                   const T* __restrict__ logits,
                                                                   const float* __restrict__ coins, int T_, int t,
                                                                   int V, int Vp) {
    __shared__ float smax[SAMPLE_WAVES];
    __shared__ double stot[SAMPLE_WAVES];
    __shared__ int sidx;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const T* z = logits + ((size_t)b * T_ + (t - 1)) * Vp;
    const int seg = (V + 64 * SAMPLE_WAVES - 1) / (64 * SAMPLE_WAVES) * 64;
    const int s0 = wave * seg, s1 = min(s0 + seg, V);

    float m = -INFINITY;
    for (int i = tid; i < V; i += 64 * SAMPLE_WAVES) m = fmaxf(m, to_f<T>(z[i]));
    m = wave_max(m);
    if (lane == 0) smax[wave] = m;
    if (tid == 0) sidx = V;
    __syncthreads();
    m = smax[0];
#pragma unroll
    for (int w = 1; w < SAMPLE_WAVES; w++) m = fmaxf(m, smax[w]);
    const double md = (double)m;

    double s = 0.0;
    for (int i = s0 + lane; i < s1; i += 64) s += exp((double)to_f<T>(z[i]) - md);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) s += shfl_xor_f64(s, d);
    if (lane == 0) stot[wave] = s;
    __syncthreads();
    double pre = 0.0, Z = 0.0;
#pragma unroll
    for (int w = 0; w < SAMPLE_WAVES; w++) {
        if (w == wave) pre = Z;
        Z += stot[w];
    }
    const double target = (double)coins[b] * Z;
    double run = pre;
    for (int j0 = s0; j0 < s1; j0 += 64) {
        const int i = j0 + lane;
        double e = i < s1 ? exp((double)to_f<T>(z[i]) - md) : 0.0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const double o = shfl_up_f64(e, d);
            if (lane >= d) e += o;
        }
        const double cdf = run + e;
        const uint64_t hit = __ballot(i < s1 && target < cdf);
        if (hit) {
            if (lane == 0) atomicMin(&sidx, j0 + (int)__builtin_ctzll(hit));
            break;
        }
        run += __shfl(e, 63, 64);
    }
    __syncthreads();
    if (tid == 0) tokens[(size_t)b * T_ + t] = sidx < V ? sidx : V - 1;
}

}  // namespace

template <typename T>
int sample_launch(int32_t* tokens, const T* logits, const float* coins, int B, int T_, int t, int V, int Vp,
                  hipStream_t s) {
    if (B <= 0) return 0;
    hipLaunchKernelGGL((sample_kernel<T>), dim3(B), dim3(64 * SAMPLE_WAVES), 0, s, tokens, logits, coins, T_, t, V,
                       Vp);
    return (int)hipGetLastError();
}

template int sample_launch<float>(int32_t*, const float*, const float*, int, int, int, int, int, hipStream_t);
template int sample_launch<bf16_t>(int32_t*, const bf16_t*, const float*, int, int, int, int, int, hipStream_t);
