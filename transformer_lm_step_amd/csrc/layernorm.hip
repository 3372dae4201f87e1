// layernorm.hip - LayerNorm forward and backward (gfx950).
//
// train_gpt2.cu, layernorm_forward_kernel3 and layernorm_backward_kernel6:
//   forward  mean = sum(x)/C, var = sum((x-mean)^2)/C (biased, two passes),
//            rstd = 1/sqrt(var + 1e-5), y = (x - mean) * rstd * w + b
//   backward norm = (x-mean)*rstd, dnorm = w*dy,
//            dx = rstd * (dnorm - mean(dnorm) - norm * mean(dnorm*norm)),
//            dw += sum_rows norm*dy, db += sum_rows dy.
// The input gradient is added into the fp32 residual-gradient buffer (the
// residual stream's backward); the first LayerNorm of the backward pass
// (the final one of the forward) stores instead, so the buffer needs no
// separate zeroing.
//
// One wave64 per row; the row lives in registers as 16-byte vectors (lane l
// owns vectors l, l+64, ...), so x is read once.  Statistics are fp32 in both
// precisions.  The parameter gradients are reduced deterministically: each
// workgroup sums its rows in registers, combines its 4 waves through LDS in
// wave order, writes one partial row, and a second kernel sums the partials
// in workgroup order.
#include "device.h"
#include "kernels.h"

namespace {

// Backward workgroups take 2 rows per wave: 8 waves (16 rows) when a row
// fits in at most 2 vectors per lane, else 4 waves (8 rows, and the workspace
// is sized for this smaller count).  Fewer, larger workgroups leave fewer
// per-workgroup partial sums for the finishing reduction to read.
constexpr int ROWS_PER_BLOCK_BWD = 8;
#ifndef LN_BWD_WAVES
#define LN_BWD_WAVES 8
#endif
template <int NV> constexpr int ln_bwd_waves() { return NV <= 2 ? LN_BWD_WAVES : 4; }

// NV: 16-byte vectors per lane, ceil(C / (64 * VEC)), fixed at launch so the
// row buffers take only the registers C needs.
template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_fwd_kernel(T* __restrict__ out, float* __restrict__ mean,
                                                     float* __restrict__ rstd, const T* __restrict__ x,
                                                     const T* __restrict__ w, const T* __restrict__ b,
                                                     int N, int C) {
    constexpr int VEC = VecT<T>::N;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= N) return;
    const int nvec = C / VEC;
    const T* xr = x + (size_t)row * C;
    float xv[NV][VEC];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int v = lane + 64 * i;
        if (v < nvec) {
            unpack16<T>(ld16(xr + v * VEC), xv[i]);
#pragma unroll
            for (int e = 0; e < VEC; e++) s += xv[i][e];
        }
    }
    const float m = wave_sum(s) / (float)C;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int v = lane + 64 * i;
        if (v < nvec) {
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                const float d = xv[i][e] - m;
                q += d * d;
            }
        }
    }
    const float rs = 1.0f / sqrtf(wave_sum(q) / (float)C + 1e-5f);
    T* o = out + (size_t)row * C;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int v = lane + 64 * i;
        if (v < nvec) {
            float wv[VEC], bv[VEC], y[VEC];
            unpack16<T>(ld16(w + v * VEC), wv);
            unpack16<T>(ld16(b + v * VEC), bv);
#pragma unroll
            for (int e = 0; e < VEC; e++) y[e] = (xv[i][e] - m) * rs * wv[e] + bv[e];
            st16(o + v * VEC, pack16<T>(y));
        }
    }
    if (lane == 0) {
        mean[row] = m;
        rstd[row] = rs;
    }
}

template <typename T, int NV>
__global__ __launch_bounds__(64 * ln_bwd_waves<NV>()) void ln_bwd_kernel(float* __restrict__ dres, T* __restrict__ dres_lp,
                                                     float* __restrict__ partial, const T* __restrict__ dy,
                                                     const T* __restrict__ x, const T* __restrict__ w,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     int N, int C, int accumulate) {
    constexpr int VEC = VecT<T>::N;
    __shared__ float red[2 * 2048];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nvec = C / VEC;
    float dw_acc[NV][VEC], db_acc[NV][VEC], wv[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int v = lane + 64 * i;
#pragma unroll
        for (int e = 0; e < VEC; e++) { dw_acc[i][e] = 0.f; db_acc[i][e] = 0.f; wv[i][e] = 0.f; }
        if (v < nvec) unpack16<T>(ld16(w + v * VEC), wv[i]);
    }
    constexpr int NWV = ln_bwd_waves<NV>();
    const int r0 = blockIdx.x * 2 * NWV;
    const int r1 = min(r0 + 2 * NWV, N);
    for (int row = r0 + wave; row < r1; row += NWV) {
        const float m = mean[row], rs = rstd[row];
        const T* xr = x + (size_t)row * C;
        const T* gr = dy + (size_t)row * C;
        float nv[NV][VEC], gv[NV][VEC];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int v = lane + 64 * i;
            if (v < nvec) {
                float xv[VEC];
                unpack16<T>(ld16(xr + v * VEC), xv);
                unpack16<T>(ld16(gr + v * VEC), gv[i]);
#pragma unroll
                for (int e = 0; e < VEC; e++) {
                    nv[i][e] = (xv[e] - m) * rs;
                    const float dn = wv[i][e] * gv[i][e];
                    s1 += dn;
                    s2 += dn * nv[i][e];
                }
            }
        }
        const float mdn = wave_sum(s1) / (float)C;
        const float mdnn = wave_sum(s2) / (float)C;
        float* dr = dres + (size_t)row * C;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int v = lane + 64 * i;
            if (v < nvec) {
                float o[VEC];
                if (accumulate) {
                    load4<float>(dr + v * VEC, o);
                    if constexpr (VEC == 8) load4<float>(dr + v * VEC + 4, o + 4);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; e++) o[e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < VEC; e++) {
                    const float dn = wv[i][e] * gv[i][e];
                    o[e] += rs * (dn - mdn - nv[i][e] * mdnn);
                    dw_acc[i][e] += nv[i][e] * gv[i][e];
                    db_acc[i][e] += gv[i][e];
                }
                store4<float>(dr + v * VEC, o);
                if constexpr (VEC == 8) store4<float>(dr + v * VEC + 4, o + 4);
                if (dres_lp != nullptr) st16(dres_lp + (size_t)row * C + v * VEC, pack16<T>(o));
            }
        }
    }
    // combine the waves in order 0, 1, 2, ...
    for (int wv_turn = 0; wv_turn < NWV; wv_turn++) {
        if (wave == wv_turn) {
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int v = lane + 64 * i;
                if (v < nvec) {
#pragma unroll
                    for (int e = 0; e < VEC; e++) {
                        const int c = v * VEC + e;
                        if (wv_turn == 0) {
                            red[c] = dw_acc[i][e];
                            red[2048 + c] = db_acc[i][e];
                        } else {
                            red[c] += dw_acc[i][e];
                            red[2048 + c] += db_acc[i][e];
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
    float* p = partial + (size_t)blockIdx.x * 2 * C;
    for (int c = threadIdx.x; c < C; c += 64 * NWV) {
        p[c] = red[c];
        p[C + c] = red[2048 + c];
    }
}

// dw[c] += sum_blocks partial[blk][c]; db[c] += sum_blocks partial[blk][C + c].
// 16 columns per workgroup (so 2C/16 workgroups share the reads) and 64
// phases of blocks per column (block k goes to phase k % 64); each thread
// issues all of its reads before adding (one round trip instead of a chain),
// and the phases are combined in order 0..63 through LDS.
constexpr int FIN_PH = 64, FIN_COLS = 16, FIN_MAXR = 16;  // up to FIN_PH * FIN_MAXR partial rows at once
__global__ __launch_bounds__(FIN_COLS * FIN_PH) void ln_bwd_finish_kernel(float* __restrict__ dw,
                                                                         float* __restrict__ db,
                                                                         const float* __restrict__ partial, int C,
                                                                         int blocks) {
    __shared__ float red[FIN_PH][FIN_COLS];
    const int col = threadIdx.x % FIN_COLS, ph = threadIdx.x / FIN_COLS;
    const int j = blockIdx.x * FIN_COLS + col;
    float s = 0.f;
    if (j < 2 * C) {
        for (int k0 = ph; k0 < blocks; k0 += FIN_PH * FIN_MAXR) {
            float v[FIN_MAXR];
#pragma unroll
            for (int i = 0; i < FIN_MAXR; i++) {
                const int k = k0 + i * FIN_PH;
                v[i] = k < blocks ? partial[(size_t)k * 2 * C + j] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < FIN_MAXR; i++) s += v[i];
        }
    }
    red[ph][col] = s;
    __syncthreads();
    if (ph == 0 && j < 2 * C) {
        float t = red[0][col];
        for (int q = 1; q < FIN_PH; q++) t += red[q][col];
        if (j < C) dw[j] += t;
        else db[j - C] += t;
    }
}

}  // namespace

template <typename T, int NV>
void ln_fwd_nv(T* out, float* mean, float* rstd, const T* x, const T* w, const T* b, int N, int C, hipStream_t s) {
    hipLaunchKernelGGL((ln_fwd_kernel<T, NV>), dim3((N + 3) / 4), dim3(256), 0, s, out, mean, rstd, x, w, b, N, C);
}

template <typename T>
int layernorm_fwd_launch(T* out, float* mean, float* rstd, const T* x, const T* w, const T* b,
                         int N, int C, hipStream_t s) {
    if (N <= 0) return 0;
    const int nv = (C / VecT<T>::N + 63) / 64;
    switch (nv) {
        case 1: ln_fwd_nv<T, 1>(out, mean, rstd, x, w, b, N, C, s); break;
        case 2: ln_fwd_nv<T, 2>(out, mean, rstd, x, w, b, N, C, s); break;
        case 3: ln_fwd_nv<T, 3>(out, mean, rstd, x, w, b, N, C, s); break;
        case 4: ln_fwd_nv<T, 4>(out, mean, rstd, x, w, b, N, C, s); break;
        default:
            if constexpr (sizeof(T) == 4) {
                if (nv <= 8) { ln_fwd_nv<T, 8>(out, mean, rstd, x, w, b, N, C, s); break; }
            }
            return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

size_t layernorm_bwd_workspace_bytes(int N, int C) {
    return (size_t)((N + ROWS_PER_BLOCK_BWD - 1) / ROWS_PER_BLOCK_BWD) * 2 * C * sizeof(float);
}

template <typename T, int NV>
int ln_bwd_nv(float* dres, T* dres_lp, const T* dy, const T* x, const T* w, const float* mean, const float* rstd,
              int N, int C, int accumulate, float* partial, hipStream_t s) {
    constexpr int NWV = ln_bwd_waves<NV>();
    const int blocks = (N + 2 * NWV - 1) / (2 * NWV);
    hipLaunchKernelGGL((ln_bwd_kernel<T, NV>), dim3(blocks), dim3(64 * NWV), 0, s, dres, dres_lp, partial, dy, x, w,
                       mean, rstd, N, C, accumulate);
    return blocks;
}

template <typename T>
int layernorm_bwd_launch(float* dres, T* dres_lp, float* dw, float* db, const T* dy, const T* x,
                         const T* w, const float* mean, const float* rstd, int N, int C,
                         int accumulate, float* partial, hipStream_t s) {
    if (N <= 0) return 0;
    const int nv = (C / VecT<T>::N + 63) / 64;
    int blocks = 0;
    switch (nv) {
        case 1: blocks = ln_bwd_nv<T, 1>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
        case 2: blocks = ln_bwd_nv<T, 2>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
        case 3: blocks = ln_bwd_nv<T, 3>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
        case 4: blocks = ln_bwd_nv<T, 4>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
        default:
            if constexpr (sizeof(T) == 4) {
                if (nv <= 8) {
                    blocks = ln_bwd_nv<T, 8>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s);
                    break;
                }
            }
            return (int)hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(ln_bwd_finish_kernel, dim3((2 * C + FIN_COLS - 1) / FIN_COLS), dim3(FIN_COLS * FIN_PH), 0, s,
                       dw, db, partial, C, blocks);
    return (int)hipGetLastError();
}

template int layernorm_fwd_launch<float>(float*, float*, float*, const float*, const float*, const float*, int, int, hipStream_t);
template int layernorm_fwd_launch<bf16_t>(bf16_t*, float*, float*, const bf16_t*, const bf16_t*, const bf16_t*, int, int, hipStream_t);
template int layernorm_bwd_launch<float>(float*, float*, float*, float*, const float*, const float*, const float*,
                                         const float*, const float*, int, int, int, float*, hipStream_t);
template int layernorm_bwd_launch<bf16_t>(float*, bf16_t*, float*, float*, const bf16_t*, const bf16_t*, const bf16_t*,
                                          const float*, const float*, int, int, int, float*, hipStream_t);
