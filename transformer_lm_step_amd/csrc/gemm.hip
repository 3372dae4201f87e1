// gemm.hip - MFMA matrix products with fused epilogues (gfx950).
//
// Every Linear layer of the step runs through this kernel (train_gpt2.cu,
// matmul_forward_cublaslt and matmul_backward; the classifier of gpt2_forward
// and gpt2_backward):
//   forward  Y[BT,OC]  = X[BT,IC] W[OC,IC]^T (+ bias, + GELU or + residual)
//   backward dX[BT,IC] = dY[BT,OC] W[OC,IC]          (overwrite; GELU' fused)
//            dW[OC,IC] += dY[BT,OC]^T X[BT,IC]       (accumulate, fp32)
// i.e. C[m,n] = sum_k A(m,k) B(k,n) with A and B either contraction-major
// (k contiguous) or contraction-strided.
//
// Design (one workgroup = 256 threads = 4 wave64s):
//  - 128x128 output tile per workgroup, 2x2 waves of 64x64, each wave a 4x4
//    grid of 16x16 MFMA tiles (64 fp32 accumulators per lane).
//  - Per stage the workgroup stages a 128 x BK slab of A and of B in LDS, both
//    stored "row x contraction" with k contiguous (BK = 64 bf16 / 32 fp32,
//    i.e. 128 bytes per row, rows padded by 16 bytes so that the 16-byte
//    fragment reads of 8 consecutive lanes hit distinct banks).
//  - Global loads are 16-byte vectors.  A k-contiguous operand is copied as
//    is; a k-strided operand is read as 4 k-rows x one 16-byte vector and
//    transposed in registers into 4-element k-runs before the LDS store, so
//    the fragment reads are the same 16-byte loads for both layouts.
//  - Two LDS stages: the next slab is fetched into registers while the current
//    one feeds the MFMAs, then stored into the other stage; one barrier per
//    stage.
//  - The MFMA A operand is the B slab and the B operand the A slab, so each
//    lane ends with 4 consecutive output columns of one row: the epilogue
//    reads bias / residual / GELU input and writes the output as 4-wide
//    vectors.
//  - Tile order: blocks are handed to the 8 XCDs round-robin; block ids are
//    remapped so that each XCD walks a contiguous run of tiles, and tiles run
//    in groups of 8 row-tiles so neighbours share operand slabs in that XCD's
//    L2.
//  - Weight-gradient products (K = B*T, few output tiles) split K across
//    workgroups; each split writes fp32 partials to workspace and a second
//    kernel adds them into dW in split order, so results are deterministic.
#include "device.h"
#include "kernels.h"

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int NTHREADS = 256;

template <typename T>
struct Cfg {
    static constexpr int BK = 128 / (int)sizeof(T);  // contraction depth per stage
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDSK = BK + PAD;            // LDS row pitch (elements)
    static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte vector
    static constexpr int KSTEPS = BK / 32;           // MFMA steps per stage
};

enum { EPI_SPLIT = 100 };

struct Args {
    const void* A; long lda;
    const void* B; long ldb;
    void* C; long ldc;
    const void* bias;
    const void* aux_in; void* aux_out; long ldaux;
    float* ws;
    int M, N, K;
    int kps;  // k-tiles per split
    float alpha;
};

// Load this thread's share of a 128-row x BK slab of X(r, k) into registers.
template <typename T, bool KMAJ>
DEV void slab_load(uint4 (&r)[4], const T* __restrict__ p, long ld, int r0, int R, int k0, int K, int tid) {
    using C = Cfg<T>;
    const uint4 z = make_uint4(0, 0, 0, 0);
    if constexpr (KMAJ) {
        // 8 vectors per row; thread covers rows tid/8 + 32i, vector tid%8
        const int kk = k0 + (tid & 7) * C::VEC;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int gr = r0 + (tid >> 3) + 32 * i;
            r[i] = (gr < R && kk < K) ? ld16(p + (long)gr * ld + kk) : z;
        }
    } else {
        // 4 consecutive k-rows x one vector of VEC r-values
        constexpr int KQ = C::BK / 4;
        const int kq = tid % KQ, rg = tid / KQ;
        const int gr = r0 + rg * C::VEC;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int kk = k0 + 4 * kq + i;
            r[i] = (kk < K && gr < R) ? ld16(p + (long)kk * ld + gr) : z;
        }
    }
}

template <typename T, bool KMAJ>
DEV void slab_store(const uint4 (&r)[4], T* __restrict__ s, int tid) {
    using C = Cfg<T>;
    if constexpr (KMAJ) {
        const int col = (tid & 7) * C::VEC;
#pragma unroll
        for (int i = 0; i < 4; i++) st16(s + ((tid >> 3) + 32 * i) * C::LDSK + col, r[i]);
    } else {
        constexpr int KQ = C::BK / 4;
        const int kq = tid % KQ, rg = tid / KQ;
        store_t4<T>(s + rg * C::VEC * C::LDSK + 4 * kq, C::LDSK, r);
    }
}

template <typename T, bool AK, bool BKM, int EPI, typename OutT>
__global__ __launch_bounds__(NTHREADS, 2) void gemm_kernel(const Args g) {
    using C = Cfg<T>;
    __shared__ __attribute__((aligned(16))) T sA[2][BM * C::LDSK];
    __shared__ __attribute__((aligned(16))) T sB[2][BN * C::LDSK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l16 = lane & 15, g4 = lane >> 4;

    // ---- tile order: XCD-contiguous runs, then groups of 8 row-tiles
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int nb = gridDim.x;
    int b = blockIdx.x;
    const int full = (nb / 8) * 8;
    if (b < full) b = (b % 8) * (nb / 8) + (b / 8);
    const int GM = 8;
    const int in_group = GM * tiles_n;
    const int group = b / in_group;
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int tm = first_m + ((b % in_group) % gsz);
    const int tn = (b % in_group) / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    const int ktiles = (g.K + C::BK - 1) / C::BK;
    const int kt0 = blockIdx.y * g.kps;
    const int kt1 = min(kt0 + g.kps, ktiles);

    const T* __restrict__ A = (const T*)g.A;
    const T* __restrict__ B = (const T*)g.B;

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[4], rb[4];
    if (kt0 < kt1) {
        slab_load<T, AK>(ra, A, g.lda, m0, g.M, kt0 * C::BK, g.K, tid);
        slab_load<T, BKM>(rb, B, g.ldb, n0, g.N, kt0 * C::BK, g.K, tid);
        slab_store<T, AK>(ra, sA[0], tid);
        slab_store<T, BKM>(rb, sB[0], tid);
    }
    __syncthreads();

    for (int kt = kt0; kt < kt1; kt++) {
        const int cur = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        if (more) {
            slab_load<T, AK>(ra, A, g.lda, m0, g.M, (kt + 1) * C::BK, g.K, tid);
            slab_load<T, BKM>(rb, B, g.ldb, n0, g.N, (kt + 1) * C::BK, g.K, tid);
        }
        const T* a_s = sA[cur];
        const T* b_s = sB[cur];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ks++) {
            Frag<T> fa[4], fb[4];
            const int kofs = ks * 32 + 8 * g4;
#pragma unroll
            for (int t = 0; t < 4; t++) frag_ld(fb[t], b_s + (wn * 64 + 16 * t + l16) * C::LDSK + kofs);
#pragma unroll
            for (int t = 0; t < 4; t++) frag_ld(fa[t], a_s + (wm * 64 + 16 * t + l16) * C::LDSK + kofs);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) mma(acc[i][j], fb[j], fa[i]);
        }
        if (more) {
            slab_store<T, AK>(ra, sA[cur ^ 1], tid);
            slab_store<T, BKM>(rb, sB[cur ^ 1], tid);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds C[m][n .. n+3]
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = m0 + wm * 64 + 16 * i + l16;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = n0 + wn * 64 + 16 * j + 4 * g4;
            if (n >= g.N) continue;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; r++) v[r] = g.alpha * acc[i][j][r];
            if constexpr (EPI == EPI_SPLIT) {
                float* w = g.ws + (size_t)blockIdx.y * g.M * g.N + (size_t)m * g.N + n;
                store4<float>(w, v);
            } else if constexpr (EPI == GEMM_ACCUM) {
                float* c = (float*)g.C + (size_t)m * g.ldc + n;
                float o[4];
                load4<float>(c, o);
#pragma unroll
                for (int r = 0; r < 4; r++) o[r] += v[r];
                store4<float>(c, o);
            } else {
                if constexpr (EPI == GEMM_BIAS || EPI == GEMM_BIAS_GELU || EPI == GEMM_BIAS_RESID) {
                    float bb[4];
                    load4<T>((const T*)g.bias + n, bb);
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] += bb[r];
                }
                if constexpr (EPI == GEMM_BIAS_GELU) {
                    T* pre = (T*)g.aux_out + (size_t)m * g.ldaux + n;
                    store4<T>(pre, v);
                    float pr[4];
                    load4<T>(pre, pr);  // GELU of the stored (rounded) pre-activation
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] = gelu_f(pr[r]);
                }
                if constexpr (EPI == GEMM_BIAS_RESID) {
                    float res[4];
                    load4<T>((const T*)g.aux_in + (size_t)m * g.ldaux + n, res);
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] += res[r];
                }
                if constexpr (EPI == GEMM_GELU_BWD) {
                    float pr[4];
                    load4<T>((const T*)g.aux_in + (size_t)m * g.ldaux + n, pr);
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] *= gelu_grad_f(pr[r]);
                }
                store4<OutT>((OutT*)g.C + (size_t)m * g.ldc + n, v);
            }
        }
    }
}

// C[i] += sum_z ws[z*MN + i], z in increasing order (n4 float4 groups)
__global__ void splitk_reduce_kernel(float* __restrict__ C, const float* __restrict__ ws, size_t MN, int splits) {
    size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= MN) return;
    float4 s = *reinterpret_cast<const float4*>(ws + i);
    for (int z = 1; z < splits; z++) {
        float4 w = *reinterpret_cast<const float4*>(ws + (size_t)z * MN + i);
        s.x += w.x; s.y += w.y; s.z += w.z; s.w += w.w;
    }
    float4 c = *reinterpret_cast<float4*>(C + i);
    c.x += s.x; c.y += s.y; c.z += s.z; c.w += s.w;
    *reinterpret_cast<float4*>(C + i) = c;
}

template <typename T>
__global__ void bias_partial_kernel(float* __restrict__ partial, const T* __restrict__ dY, int M, int N, long ldy) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const int r0 = blockIdx.y * 256, r1 = min(r0 + 256, M);
    float s = 0.f;
    for (int m = r0; m < r1; m++) s += to_f<T>(dY[(long)m * ldy + n]);
    partial[(size_t)blockIdx.y * N + n] = s;
}

__global__ void bias_finish_kernel(float* __restrict__ db, const float* __restrict__ partial, int N, int chunks) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float s = 0.f;
    for (int c = 0; c < chunks; c++) s += partial[(size_t)c * N + n];
    db[n] += s;
}

int split_count(const GemmDesc& d, int elem_bytes, int num_cus) {
    if (d.epi != GEMM_ACCUM) return 1;
    const int bk = 128 / elem_bytes;
    const long tiles = (long)((d.M + BM - 1) / BM) * ((d.N + BN - 1) / BN);
    const int ktiles = (d.K + bk - 1) / bk;
    const long want = 2L * num_cus;
    if (tiles >= want) return 1;
    int s = (int)((want + tiles - 1) / tiles);
    s = min(s, max(1, ktiles / 4));
    s = min(s, 32);
    if (s <= 1) return 1;
    const int kps = (ktiles + s - 1) / s;
    return (ktiles + kps - 1) / kps;
}

template <typename T, bool AK, bool BKM, int EPI, typename OutT>
void launch_t(const Args& a, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_kernel<T, AK, BKM, EPI, OutT>), grid, dim3(NTHREADS), 0, s, a);
}

template <typename T, int EPI, typename OutT>
void launch_layout(const GemmDesc& d, const Args& a, dim3 grid, hipStream_t s) {
    if (d.a_kmajor && d.b_kmajor) launch_t<T, true, true, EPI, OutT>(a, grid, s);
    else if (d.a_kmajor && !d.b_kmajor) launch_t<T, true, false, EPI, OutT>(a, grid, s);
    else if (!d.a_kmajor && !d.b_kmajor) launch_t<T, false, false, EPI, OutT>(a, grid, s);
    else launch_t<T, false, true, EPI, OutT>(a, grid, s);
}

template <typename T>
int gemm_launch_t(const GemmDesc& d, float* ws, size_t ws_bytes, int num_cus, hipStream_t s) {
    constexpr int BK = Cfg<T>::BK;
    const int tiles = ((d.M + BM - 1) / BM) * ((d.N + BN - 1) / BN);
    const int ktiles = (d.K + BK - 1) / BK;
    const int splits = split_count(d, (int)sizeof(T), num_cus);
    Args a;
    a.A = d.A; a.lda = d.lda; a.B = d.B; a.ldb = d.ldb; a.C = d.C; a.ldc = d.ldc;
    a.bias = d.bias; a.aux_in = d.aux_in; a.aux_out = d.aux_out; a.ldaux = d.ldaux;
    a.ws = ws; a.M = d.M; a.N = d.N; a.K = d.K; a.alpha = d.alpha;
    if (tiles == 0) return 0;
    if (splits > 1) {
        const size_t need = (size_t)splits * d.M * d.N * sizeof(float);
        if (ws == nullptr || ws_bytes < need || d.ldc != d.N) return (int)hipErrorInvalidValue;
        a.kps = (ktiles + splits - 1) / splits;
        launch_layout<T, EPI_SPLIT, float>(d, a, dim3(tiles, splits), s);
        const size_t MN = (size_t)d.M * d.N;
        const unsigned blocks = (unsigned)((MN / 4 + 255) / 256);
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, (float*)d.C, ws, MN, splits);
        return (int)hipGetLastError();
    }
    a.kps = ktiles;
    const dim3 grid(tiles, 1);
    switch (d.epi) {
        case GEMM_STORE: launch_layout<T, GEMM_STORE, T>(d, a, grid, s); break;
        case GEMM_BIAS: launch_layout<T, GEMM_BIAS, T>(d, a, grid, s); break;
        case GEMM_BIAS_GELU: launch_layout<T, GEMM_BIAS_GELU, T>(d, a, grid, s); break;
        case GEMM_BIAS_RESID: launch_layout<T, GEMM_BIAS_RESID, T>(d, a, grid, s); break;
        case GEMM_GELU_BWD: launch_layout<T, GEMM_GELU_BWD, T>(d, a, grid, s); break;
        case GEMM_ACCUM: launch_layout<T, GEMM_ACCUM, float>(d, a, grid, s); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(const GemmDesc& d, int elem_bytes, int num_cus) {
    const int s = split_count(d, elem_bytes, num_cus);
    return s > 1 ? (size_t)s * d.M * d.N * sizeof(float) : 0;
}

int gemm_launch(const GemmDesc& d, int elem_bytes, float* ws, size_t ws_bytes, int num_cus, hipStream_t s) {
    if (elem_bytes == 2) return gemm_launch_t<bf16_t>(d, ws, ws_bytes, num_cus, s);
    if (elem_bytes == 4) return gemm_launch_t<float>(d, ws, ws_bytes, num_cus, s);
    return (int)hipErrorInvalidValue;
}

size_t bias_grad_workspace_bytes(int M, int N) {
    return (size_t)((M + 255) / 256) * N * sizeof(float);
}

template <typename T>
int bias_grad_launch(float* db, const T* dY, int M, int N, long ldy, float* partial, hipStream_t s) {
    const int chunks = (M + 255) / 256;
    if (chunks == 0 || N == 0) return 0;
    hipLaunchKernelGGL(bias_partial_kernel<T>, dim3((N + 255) / 256, chunks), dim3(256), 0, s, partial, dY, M, N, ldy);
    hipLaunchKernelGGL(bias_finish_kernel, dim3((N + 255) / 256), dim3(256), 0, s, db, partial, N, chunks);
    return (int)hipGetLastError();
}
template int bias_grad_launch<float>(float*, const float*, int, int, long, float*, hipStream_t);
template int bias_grad_launch<bf16_t>(float*, const bf16_t*, int, int, long, float*, hipStream_t);
