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
// Order of the sums (fixed, so the draw is deterministic): thread k owns the
// contiguous chunk [k*ch, (k+1)*ch) of the V columns and sums its p_i in index
// order; the chunk totals are prefix-summed in thread order; the CDF value at i
// is the chunk's prefix plus the in-chunk running sum up to i.  The token is the
// smallest i with coin * Z < cdf_i (Z = sum of all chunk totals), V - 1 if none.
#include <math.h>

#include "device.h"
#include "kernels.h"

namespace {

constexpr int SAMPLE_THREADS = 512;

template <typename T>
__global__ __launch_bounds__(SAMPLE_THREADS) void sample_kernel(int32_t* __restrict__ tokens,
                                                                const T* __restrict__ logits,
                                                                const float* __restrict__ coins, int T_, int t,
                                                                int V, int Vp) {
    __shared__ float smax[SAMPLE_THREADS / 64];
    __shared__ double spre[SAMPLE_THREADS];
    __shared__ double stot;
    __shared__ int sidx;
    const int b = blockIdx.x, tid = threadIdx.x;
    const T* z = logits + ((size_t)b * T_ + (t - 1)) * Vp;
    const int ch = (V + SAMPLE_THREADS - 1) / SAMPLE_THREADS;
    const int i0 = min(tid * ch, V), i1 = min(i0 + ch, V);

    float m = -INFINITY;
    for (int i = i0; i < i1; i++) m = fmaxf(m, to_f<T>(z[i]));
    m = wave_max(m);
    if ((tid & 63) == 0) smax[tid >> 6] = m;
    if (tid == 0) sidx = V;
    __syncthreads();
    m = smax[0];
#pragma unroll
    for (int w = 1; w < SAMPLE_THREADS / 64; w++) m = fmaxf(m, smax[w]);
    const double md = (double)m;

    double s = 0.0;
    for (int i = i0; i < i1; i++) s += exp((double)to_f<T>(z[i]) - md);
    spre[tid] = s;
    __syncthreads();
    if (tid == 0) {  // exclusive prefix of the chunk totals, in thread order
        double acc = 0.0;
        for (int k = 0; k < SAMPLE_THREADS; k++) {
            const double v = spre[k];
            spre[k] = acc;
            acc += v;
        }
        stot = acc;
    }
    __syncthreads();
    const double target = (double)coins[b] * stot;
    double cdf = spre[tid];
    for (int i = i0; i < i1; i++) {
        cdf += exp((double)to_f<T>(z[i]) - md);
        if (target < cdf) {
            atomicMin(&sidx, i);
            break;
        }
    }
    __syncthreads();
    if (tid == 0) tokens[(size_t)b * T_ + t] = sidx < V ? sidx : V - 1;
}

}  // namespace

template <typename T>
int sample_launch(int32_t* tokens, const T* logits, const float* coins, int B, int T_, int t, int V, int Vp,
                  hipStream_t s) {
    if (B <= 0) return 0;
    hipLaunchKernelGGL((sample_kernel<T>), dim3(B), dim3(SAMPLE_THREADS), 0, s, tokens, logits, coins, T_, t, V, Vp);
    return (int)hipGetLastError();
}

template int sample_launch<float>(int32_t*, const float*, const float*, int, int, int, int, int, hipStream_t);
template int sample_launch<bf16_t>(int32_t*, const bf16_t*, const float*, int, int, int, int, int, hipStream_t);
