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
// A row is spread over LPR lanes of a wave (32 for rows of up to 96 16-byte
// vectors, so a 768-wide bf16 row is exactly 3 vectors per lane; 64 for
// wider ones) and lives in registers, so x is read once.  Statistics are
// fp32 in both precisions.  The parameter gradients are reduced
// deterministically: each workgroup sums its rows in registers, combines
// the two row groups of a wave and then its 4 waves through LDS in a fixed
// order, writes one partial row, and a second kernel sums the partials in
// workgroup order.
#include "device.h"
#include "kernels.h"

namespace {

// sum over the LPR lanes of this row (the same bits in all of them)
template <int LPR>
DEV float row_sum(float v) {
    return lane_reduce<LPR>(v, AddOp());
}

// Forward: LPR lanes per row (half a wave while a row is at most 3 vectors
// per lane, else a whole wave), so a wave holds 64 / LPR rows per step; the
// reads of all STEPS steps of a wave are issued before any row is reduced.
// NV: 16-byte vectors per lane, ceil(C / VEC / LPR); two passes over the
// registers give the exact two-pass variance.
constexpr int LNF_WAVES = 4, LNF_ROWS = 16;  // rows per workgroup

template <typename T, int NV, int LPR>
__global__ __launch_bounds__(64 * LNF_WAVES) void ln_fwd_kernel(T* __restrict__ out, float* __restrict__ mean,
                                                              float* __restrict__ rstd, const T* __restrict__ x,
                                                              const T* __restrict__ w, const T* __restrict__ b,
                                                              int N, int C) {
    constexpr int VEC = VecT<T>::N;
    constexpr int RPS = 64 / LPR, STEPS = LNF_ROWS / LNF_WAVES / RPS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hl = lane % LPR, grp = lane / LPR;
    const int nvec = C / VEC;
    auto row_of = [&](int p) { return blockIdx.x * LNF_ROWS + RPS * (wave + LNF_WAVES * p) + grp; };
    // the lane's weight and bias vectors, requested with the rows (not after
    // the row sums, which would add a dependent round trip per step)
    uint4 wraw[NV], braw[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int v = hl + LPR * i;
        wraw[i] = ld16(w + (size_t)(v < nvec ? v : 0) * VEC);
        braw[i] = ld16(b + (size_t)(v < nvec ? v : 0) * VEC);
    }
    uint4 raw[STEPS][NV];
#pragma unroll
    for (int p = 0; p < STEPS; p++) {
        const int row = row_of(p);
        const size_t base = (size_t)(row < N ? row : 0) * C;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int v = hl + LPR * i;
            raw[p][i] = ld16(x + base + (size_t)(v < nvec ? v : 0) * VEC);
        }
    }
#pragma unroll
    for (int p = 0; p < STEPS; p++) {
        const int row = row_of(p);
        float xv[NV][VEC];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const bool in = hl + LPR * i < nvec;
            unpack16<T>(raw[p][i], xv[i]);
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                if (!in) xv[i][e] = 0.f;
                s += xv[i][e];
            }
        }
        const float m = row_sum<LPR>(s) / (float)C;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const bool in = hl + LPR * i < nvec;
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                const float d = in ? xv[i][e] - m : 0.f;
                q += d * d;
            }
        }
        const float rs = 1.0f / sqrtf(row_sum<LPR>(q) / (float)C + 1e-5f);
        if (row < N) {
            T* o = out + (size_t)row * C;
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int v = hl + LPR * i;
                if (v < nvec) {
                    float wv[VEC], bv[VEC], y[VEC];
                    unpack16<T>(wraw[i], wv);
                    unpack16<T>(braw[i], bv);
#pragma unroll
                    for (int e = 0; e < VEC; e++) y[e] = (xv[i][e] - m) * rs * wv[e] + bv[e];
                    st16(o + v * VEC, pack16<T>(y));
                }
            }
            if (hl == 0) {
                mean[row] = m;
                rstd[row] = rs;
            }
        }
    }
}

// Backward: LPR lanes per row -- half a wave for rows of up to 96 vectors
// (a 768-wide bf16 row is exactly 3 vectors per lane), a whole wave for
// wider ones.  A wave takes 4 rows, in steps of 64 / LPR rows at a
// time; all reads of a step (x, dy and, when accumulating, the fp32
// residual gradient) are issued together, one step ahead of the one being
// computed.  NV: vectors per lane, ceil(C / VEC / LPR).
// Workgroup shape: half-wave rows in 4 waves x 16 rows (5% faster in the
// 124M step than 8 x 32), whole-wave rows in 8 waves x 32 rows (5% faster in
// the 1558M step than 4 x 16); 4 rows per wave either way.
template <int LPR>
struct LnbShape {
    static constexpr int WAVES = LPR == 32 ? 4 : 8, ROWS = LPR == 32 ? 16 : 32;
};

template <typename T, int NV>
struct LnRow {
    static constexpr int VEC = VecT<T>::N;
    uint4 x[NV], g[NV];
    float4 r[NV][VEC / 4];
    float m, rs;  // the row's mean and 1/std (0 past the last row)
};

template <typename T, int NV, int LPR, bool WITH_R>
DEV void ln_row_load(LnRow<T, NV>& d, const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ dres,
                     const float* __restrict__ mean, const float* __restrict__ rstd, int row, int N, int C, int hl,
                     bool acc) {
    constexpr int VEC = VecT<T>::N;
    const int nvec = C / VEC;
    const bool ok = row < N;
    const size_t base = (size_t)(ok ? row : 0) * C;
    d.m = mean[ok ? row : 0];
    d.rs = rstd[ok ? row : 0];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int v = hl + LPR * i;
        const bool in = ok && v < nvec;
        const size_t o = base + (size_t)(in ? v : 0) * VEC;
        d.x[i] = ld16(x + o);
        d.g[i] = ld16(dy + o);
        if constexpr (WITH_R) {
#pragma unroll
            for (int q = 0; q < VEC / 4; q++)
                d.r[i][q] = acc ? *reinterpret_cast<const float4*>(dres + o + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

template <typename T, int NV, int LPR>
__global__ __launch_bounds__(64 * LnbShape<LPR>::WAVES) void ln_bwd_kernel(float* __restrict__ dres, T* __restrict__ dres_lp,
                                                     float* __restrict__ partial, const T* __restrict__ dy,
                                                     const T* __restrict__ x, const T* __restrict__ w,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     int N, int C, int accumulate) {
    constexpr int VEC = VecT<T>::N;
    __shared__ float red[2 * 2048];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int LNB_WAVES = LnbShape<LPR>::WAVES, LNB_ROWS = LnbShape<LPR>::ROWS;
    constexpr int RPS = 64 / LPR, STEPS = LNB_ROWS / LNB_WAVES / RPS;  // rows per step, steps per wave
    const int hl = lane % LPR, half = lane / LPR;
    const int nvec = C / VEC;
    const bool acc = accumulate != 0;
    float dw_acc[NV][VEC], db_acc[NV][VEC], wv[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int v = hl + LPR * i;
#pragma unroll
        for (int e = 0; e < VEC; e++) { dw_acc[i][e] = 0.f; db_acc[i][e] = 0.f; wv[i][e] = 0.f; }
        if (v < nvec) unpack16<T>(ld16(w + v * VEC), wv[i]);
    }
    // row of step p of this wave and lane group
    const int r0 = blockIdx.x * LNB_ROWS;
    auto row_of = [&](int p) { return r0 + RPS * (wave + LNB_WAVES * p) + half; };
    // Wide rows (a whole wave per row) have no room for a second set of row
    // registers: each step loads its own, and the residual gradient is read
    // after the row sums.
    constexpr bool PREF = LPR == 32;
    LnRow<T, NV> cur, nxt;
    ln_row_load<T, NV, LPR, PREF>(cur, x, dy, dres, mean, rstd, row_of(0), N, C, hl, acc);
#pragma unroll(PREF ? STEPS : 1)
    for (int p = 0; p < STEPS; p++) {
        if (PREF && p + 1 < STEPS) ln_row_load<T, NV, LPR, PREF>(nxt, x, dy, dres, mean, rstd, row_of(p + 1), N, C, hl, acc);
        if (!PREF && p > 0) ln_row_load<T, NV, LPR, PREF>(cur, x, dy, dres, mean, rstd, row_of(p), N, C, hl, acc);
        const int row = row_of(p);
        const bool ok = row < N;
        const float m = cur.m, rs = cur.rs;
        float nv[NV][VEC], gv[NV][VEC];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const bool in = ok && hl + LPR * i < nvec;
            float xv[VEC];
            unpack16<T>(cur.x[i], xv);
            unpack16<T>(cur.g[i], gv[i]);
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                if (!in) gv[i][e] = 0.f;
                nv[i][e] = in ? (xv[e] - m) * rs : 0.f;
                const float dn = wv[i][e] * gv[i][e];
                s1 += dn;
                s2 += dn * nv[i][e];
            }
        }
        const float mdn = row_sum<LPR>(s1) / (float)C;
        const float mdnn = row_sum<LPR>(s2) / (float)C;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int v = hl + LPR * i;
            float o[VEC];
            if constexpr (PREF) {
#pragma unroll
                for (int q = 0; q < VEC / 4; q++) {
                    o[4 * q] = cur.r[i][q].x; o[4 * q + 1] = cur.r[i][q].y;
                    o[4 * q + 2] = cur.r[i][q].z; o[4 * q + 3] = cur.r[i][q].w;
                }
            } else {
                const size_t ro = (size_t)(ok ? row : 0) * C + (size_t)(v < nvec ? v : 0) * VEC;
#pragma unroll
                for (int e = 0; e < VEC; e++) o[e] = 0.f;
                if (acc) {
                    load4<float>(dres + ro, o);
                    if constexpr (VEC == 8) load4<float>(dres + ro + 4, o + 4);
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                const float dn = wv[i][e] * gv[i][e];
                o[e] += rs * (dn - mdn - nv[i][e] * mdnn);
                dw_acc[i][e] += nv[i][e] * gv[i][e];
                db_acc[i][e] += gv[i][e];
            }
            if (ok && v < nvec) {
                float* dr = dres + (size_t)row * C + v * VEC;
                store4<float>(dr, o);
                if constexpr (VEC == 8) store4<float>(dr + 4, o + 4);
                if (dres_lp != nullptr) st16(dres_lp + (size_t)row * C + v * VEC, pack16<T>(o));
            }
        }
        if (PREF && p + 1 < STEPS) cur = nxt;
    }
    // the two halves of the wave (same columns, different rows; half 0's sum
    // first in both), then the waves in order 0, 1, 2, ... through LDS
    if constexpr (LPR == 32) {
#pragma unroll
        for (int i = 0; i < NV; i++)
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                dw_acc[i][e] = xor32_combine(dw_acc[i][e], AddOp());
                db_acc[i][e] = xor32_combine(db_acc[i][e], AddOp());
            }
    }
    for (int turn = 0; turn < LNB_WAVES; turn++) {
        if (wave == turn && half == 0) {
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int v = hl + LPR * i;
                if (v < nvec) {
#pragma unroll
                    for (int e = 0; e < VEC; e++) {
                        const int c = v * VEC + e;
                        if (turn == 0) {
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
    float* pp = partial + (size_t)blockIdx.x * 2 * C;
    for (int c = threadIdx.x; c < C; c += 64 * LNB_WAVES) {
        pp[c] = red[c];
        pp[C + c] = red[2048 + c];
    }
}

// For every LayerNorm backward (slot) of a pass: dw[c] += sum_blocks
// partial[blk][c], db[c] += sum_blocks partial[blk][C + c], over that slot's
// partial rows.  One launch for all slots (blockIdx.y); 32 columns per
// workgroup, so each workgroup reads whole 128-byte lines (with 16, two
// workgroups on different XCDs fetched every line), and 32 phases of blocks
// per column (block k goes to phase k % 32); each thread issues all of its
// reads before adding (one round trip instead of a chain), and the phases
// are combined in order 0..31 through LDS.  MAXR (partial rows per thread
// and pass) is the smallest of 4, 8, 16 that covers the rows in one pass
// where it can, so few of the unconditional reads are repeats.
constexpr int FIN_PH = 32, FIN_COLS = 32;
template <int FIN_MAXR>
__global__ __launch_bounds__(FIN_COLS * FIN_PH) void ln_bwd_finish_kernel(const LnFinishArgs a,
                                                                         const float* __restrict__ partial, int C,
                                                                         int blocks) {
    __shared__ float red[FIN_PH][FIN_COLS];
    const int slot = blockIdx.y;
    const float* part = partial + (size_t)slot * blocks * 2 * C;
    const int col = threadIdx.x % FIN_COLS, ph = threadIdx.x / FIN_COLS;
    const int j = blockIdx.x * FIN_COLS + col;
    float s = 0.f;
    if (j < 2 * C) {
        for (int k0 = ph; k0 < blocks; k0 += FIN_PH * FIN_MAXR) {
            float v[FIN_MAXR];
#pragma unroll
            for (int i = 0; i < FIN_MAXR; i++) {
                // unconditional load (a row past the end re-reads row k0), so
                // the loads overlap
                const int k = k0 + i * FIN_PH;
                v[i] = part[(size_t)(k < blocks ? k : k0) * 2 * C + j];
            }
#pragma unroll
            for (int i = 0; i < FIN_MAXR; i++)
                if (k0 + i * FIN_PH < blocks) s += v[i];
        }
    }
    red[ph][col] = s;
    __syncthreads();
    if (ph == 0 && j < 2 * C) {
        float t = red[0][col];
        for (int q = 1; q < FIN_PH; q++) t += red[q][col];
        if (j < C) a.dw[slot][j] += t;
        else a.db[slot][j - C] += t;
    }
}

}  // namespace

template <typename T, int NV, int LPR = 32>
void ln_fwd_nv(T* out, float* mean, float* rstd, const T* x, const T* w, const T* b, int N, int C, hipStream_t s) {
    hipLaunchKernelGGL((ln_fwd_kernel<T, NV, LPR>), dim3((N + LNF_ROWS - 1) / LNF_ROWS), dim3(64 * LNF_WAVES), 0, s, out,
                       mean, rstd, x, w, b, N, C);
}

template <typename T>
int layernorm_fwd_launch(T* out, float* mean, float* rstd, const T* x, const T* w, const T* b,
                         int N, int C, hipStream_t s) {
    if (N <= 0) return 0;
    const int nvec = C / VecT<T>::N;
    const int nv32 = (nvec + 31) / 32, nv64 = (nvec + 63) / 64;
    if (nv32 <= 3) {
        switch (nv32) {
            case 1: ln_fwd_nv<T, 1>(out, mean, rstd, x, w, b, N, C, s); break;
            case 2: ln_fwd_nv<T, 2>(out, mean, rstd, x, w, b, N, C, s); break;
            default: ln_fwd_nv<T, 3>(out, mean, rstd, x, w, b, N, C, s); break;
        }
    } else {
        switch (nv64) {
            case 2: ln_fwd_nv<T, 2, 64>(out, mean, rstd, x, w, b, N, C, s); break;
            case 3: ln_fwd_nv<T, 3, 64>(out, mean, rstd, x, w, b, N, C, s); break;
            case 4: ln_fwd_nv<T, 4, 64>(out, mean, rstd, x, w, b, N, C, s); break;
            default:
                if constexpr (sizeof(T) == 4) {
                    if (nv64 <= 8) { ln_fwd_nv<T, 8, 64>(out, mean, rstd, x, w, b, N, C, s); break; }
                }
                return (int)hipErrorInvalidValue;
        }
    }
    return (int)hipGetLastError();
}

// rows per workgroup of the backward of N rows of C elements of esz bytes
// (the LPR choice of layernorm_bwd_launch)
int lnb_rows(int C, int esz) {
    const int nvec = C / (16 / esz);
    return (nvec + 31) / 32 <= 3 ? LnbShape<32>::ROWS : LnbShape<64>::ROWS;
}
int layernorm_bwd_partial_rows(int N, int C, int esz) { return (N + lnb_rows(C, esz) - 1) / lnb_rows(C, esz); }

template <typename T, int NV, int LPR = 32>
void ln_bwd_nv(float* dres, T* dres_lp, const T* dy, const T* x, const T* w, const float* mean, const float* rstd,
               int N, int C, int accumulate, float* partial, hipStream_t s) {
    hipLaunchKernelGGL((ln_bwd_kernel<T, NV, LPR>), dim3((N + LnbShape<LPR>::ROWS - 1) / LnbShape<LPR>::ROWS),
                       dim3(64 * LnbShape<LPR>::WAVES), 0, s, dres,
                       dres_lp, partial, dy, x, w, mean, rstd, N, C, accumulate);
}

template <typename T>
int layernorm_bwd_launch(float* dres, T* dres_lp, const T* dy, const T* x, const T* w, const float* mean,
                         const float* rstd, int N, int C, int accumulate, float* partial, hipStream_t s) {
    if (N <= 0) return 0;
    // half a wave per row while that takes at most 3 vectors per lane, else a wave
    const int nvec = C / VecT<T>::N;
    const int nv32 = (nvec + 31) / 32, nv64 = (nvec + 63) / 64;
    if (nv32 <= 3) {
        switch (nv32) {
            case 1: ln_bwd_nv<T, 1>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
            case 2: ln_bwd_nv<T, 2>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
            default: ln_bwd_nv<T, 3>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
        }
    } else {
        switch (nv64) {
            case 2: ln_bwd_nv<T, 2, 64>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
            case 3: ln_bwd_nv<T, 3, 64>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
            case 4: ln_bwd_nv<T, 4, 64>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s); break;
            default:
                if constexpr (sizeof(T) == 4) {
                    if (nv64 <= 8) {
                        ln_bwd_nv<T, 8, 64>(dres, dres_lp, dy, x, w, mean, rstd, N, C, accumulate, partial, s);
                        break;
                    }
                }
                return (int)hipErrorInvalidValue;
        }
    }
    return (int)hipGetLastError();
}

int layernorm_bwd_finish_launch(const LnFinishArgs& a, int slots, const float* partial, int N, int C, int esz,
                                hipStream_t s) {
    if (N <= 0 || slots <= 0) return 0;
    if (slots > kMaxLnSlots) return (int)hipErrorInvalidValue;
    const int blocks = layernorm_bwd_partial_rows(N, C, esz);
    const dim3 grid((2 * C + FIN_COLS - 1) / FIN_COLS, slots);
    if (blocks <= FIN_PH * 4) hipLaunchKernelGGL(ln_bwd_finish_kernel<4>, grid, dim3(FIN_COLS * FIN_PH), 0, s, a, partial, C, blocks);
    else if (blocks <= FIN_PH * 8) hipLaunchKernelGGL(ln_bwd_finish_kernel<8>, grid, dim3(FIN_COLS * FIN_PH), 0, s, a, partial, C, blocks);
    else hipLaunchKernelGGL(ln_bwd_finish_kernel<16>, grid, dim3(FIN_COLS * FIN_PH), 0, s, a, partial, C, blocks);
    return (int)hipGetLastError();
}

template int layernorm_fwd_launch<float>(float*, float*, float*, const float*, const float*, const float*, int, int, hipStream_t);
template int layernorm_fwd_launch<bf16_t>(bf16_t*, float*, float*, const bf16_t*, const bf16_t*, const bf16_t*, int, int, hipStream_t);
template int layernorm_bwd_launch<float>(float*, float*, const float*, const float*, const float*, const float*,
                                         const float*, int, int, int, float*, hipStream_t);
template int layernorm_bwd_launch<bf16_t>(float*, bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*, const float*,
                                          const float*, int, int, int, float*, hipStream_t);
