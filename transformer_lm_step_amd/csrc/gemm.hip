// gemm.hip - MFMA matrix products with fused epilogues (gfx950).
//
// Every Linear layer of the step runs through this kernel (train_gpt2.cu,
// matmul_forward_cublaslt and matmul_backward with matmul_backward_bias_kernel4;
// the tied classifier of gpt2_forward and gpt2_backward):
//   forward  Y[BT,OC]  = X[BT,IC] W[OC,IC]^T (+ bias, + GELU or + residual)
//   backward dX[BT,IC] = dY[BT,OC] W[OC,IC]          (overwrite; GELU' fused)
//            dW[OC,IC] += dY[BT,OC]^T X[BT,IC]       (accumulate, fp32;
//                                                     bias gradient fused)
// i.e. C[m,n] = sum_k A(m,k) B(k,n) with A and B either contraction-major
// (k contiguous) or contraction-strided.
//
// Design (one workgroup = 256 threads = 4 wave64s in a 2x2 grid):
//  - BM x BN output tile per workgroup (256x256, 256x128, 128x256, 256x96 or
//    128x128, chosen per shape), each wave a (BM/2)x(BN/2) grid of 16x16
//    MFMA tiles.  The big tiles keep up to 256 fp32 accumulators per lane
//    and run one workgroup per CU; 128x128 runs two.
//  - Per stage the workgroup stages a BM x BK slab of A and a BN x BK slab of
//    B in LDS, both stored "row x contraction" with k contiguous (BK = 64 bf16
//    / 32 fp32, i.e. 128 bytes per row, rows padded by 16 bytes so that the
//    16-byte fragment reads of 8 consecutive lanes hit distinct banks).
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
//  - Products with few output tiles and a long K (weight gradients, K = B*T;
//    the classifier's input gradient, K = Vp) split K across workgroups; each
//    split writes fp32 partials to workspace and a second kernel combines them
//    in split order, so results are deterministic.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace {

constexpr int NTHREADS = 256;

template <typename T, int BM_, int BN_, int WTM_ = 64, int WTN_ = 64, int SK_ = 1>
struct Tile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int SK = SK_;  // waves sharing one output tile, each a slice of every stage's depth
    static constexpr int BK = 128 / (int)sizeof(T);  // contraction depth per stage
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDSK = BK + PAD;            // LDS row pitch (elements)
    static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte vector
    static constexpr int KSTEPS = BK / 32;           // MFMA steps per stage
    static constexpr int WTM = WTM_, WTN = WTN_;     // output tile of one wave
    static constexpr int WM = BM / WTM, WN = BN / WTN;
    static constexpr int NT = 64 * WM * WN * SK;     // threads per workgroup
    static constexpr int TM = WTM / 16, TN = WTN / 16;  // 16x16 MFMA tiles per wave
    static constexpr int OCC = NT == 256 && WTM == 64 && WTN == 64 ? 2 : 1;  // workgroups per CU
    // slab prefetch distance and fragment buffers, within the register budget
    // of NT/256 * OCC waves per SIMD
    static constexpr int DEPTH = WTM * WTN == 64 * 64 ? (NT <= 512 ? 2 : 1)
                                 : WTM * WTN == 128 * 64 ? (NT <= 256 ? 2 : 1) : 1;
    static constexpr int FBUF = DEPTH;
};

// Wave tile selector used by the kernels' template argument WT: 64 -> 64x64,
// 96 -> 64x96, 128 -> 128x64, 144 -> 64x144 outputs per wave (128x128 waves
// need 256 accumulators per lane, which the compiler only fits by spilling);
// 97 -> 64x96 with the depth sliced: two waves per output tile, each taking
// one 32-deep half of every stage, their sums added at the end.
template <typename T, int BM, int BN, int WT>
using TileOf = Tile<T, BM, BN, (WT == 128 || WT == 256 ? 128 : 64),
                    (WT == 256 ? 128 : WT == 96 || WT == 97 ? 96 : WT == 144 ? 144 : 64), (WT == 97 ? 2 : 1)>;

// Per-thread register count for staging an R x BK slab (both layouts).
template <int R, int NT> struct StageRegs {
    static constexpr int KM = (R * 8 + NT - 1) / NT;            // k-major: R*8 vectors
    static constexpr int KS_BLOCKS = (2 * R + NT - 1) / NT;     // k-strided: 2R blocks of 4
    static constexpr int N = (KM > 4 * KS_BLOCKS) ? KM : 4 * KS_BLOCKS;
};

enum { EPI_SPLIT = 100 };
constexpr int kMaxGroup = 8;  // problem classes of one grouped launch

struct Args {
    const void* A; long lda;
    const void* B; long ldb;
    void* C; long ldc;
    const void* bias;
    const void* aux_in; void* aux_out; long ldaux;
    float* ws;
    float* dbias;   // GEMM_ACCUM only: dbias[m] += alpha * sum_k A(m,k) (or split partials in wsb)
    float* wsb;
    int M, N, K;
    int kps;  // k-tiles per split
    float alpha;
};

// Staging of an R-row x BK slab of X(r, k) with buffer loads.  Each operand
// tile gets a buffer resource whose base is the slab's first element and
// whose byte range ends at the end of the operand's valid data, so rows past
// the matrix (and, for a k-strided operand, contraction rows past K) read as
// zeros in hardware.  Per-lane byte offsets are loop invariant; moving to the
// next slab only changes the (scalar) resource.  The one case the range cannot
// cover -- contraction indices past K inside a row of a k-contiguous operand,
// when K is not a multiple of BK -- is sent to an out-of-range offset.
template <typename T, int R, bool KMAJ, int NT>
struct SlabAddr {
    uint32_t off[StageRegs<R, NT>::N];   // per-lane byte offsets within a slab
    int krel[KMAJ ? StageRegs<R, NT>::N : 1];
    DEV void init(long ld, int tid) {
        constexpr int VEC = 16 / (int)sizeof(T), BK = 128 / (int)sizeof(T);
        if constexpr (KMAJ) {
#pragma unroll
            for (int i = 0; i < StageRegs<R, NT>::KM; i++) {
                const int idx = tid + NT * i;
                krel[i] = (idx & 7) * VEC;
                off[i] = (uint32_t)(((long)(idx >> 3) * ld + krel[i]) * (long)sizeof(T));
            }
        } else {
            constexpr int KQ = BK / 4;
#pragma unroll
            for (int bl = 0; bl < StageRegs<R, NT>::KS_BLOCKS; bl++) {
                const int idx = tid + NT * bl;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    off[4 * bl + i] = (uint32_t)(((long)(4 * (idx % KQ) + i) * ld + (idx / KQ) * VEC) * (long)sizeof(T));
            }
        }
    }
};

// p: operand base; (r0, k0): slab origin; Rmax rows, K contraction length.
template <typename T, int R, bool KMAJ, int NT>
DEV void slab_load(uint4* r, const SlabAddr<T, R, KMAJ, NT>& ad, const T* __restrict__ p, long ld, int r0, int Rmax,
                   int k0, int K) {
    if constexpr (KMAJ) {
        const T* base = p + (long)r0 * ld + k0;
        const long end = (long)Rmax * ld;  // elements
        const uint32_t bytes = rsrc_range((end - ((long)r0 * ld + k0)) * (long)sizeof(T));
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
        const int klim = K - k0;
#pragma unroll
        for (int i = 0; i < StageRegs<R, NT>::KM; i++) r[i] = buf_ld16(rs, ad.krel[i] < klim ? ad.off[i] : kBufOOB);
    } else {
        const T* base = p + (long)k0 * ld + r0;
        const long end = (long)K * ld;
        const uint32_t bytes = rsrc_range((end - ((long)k0 * ld + r0)) * (long)sizeof(T));
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
        for (int i = 0; i < 4 * StageRegs<R, NT>::KS_BLOCKS; i++) r[i] = buf_ld16(rs, ad.off[i]);
    }
}

template <typename T, int R, bool KMAJ, int NT>
DEV void slab_store(const uint4* r, T* __restrict__ s, int tid) {
    constexpr int VEC = 16 / (int)sizeof(T), BK = 128 / (int)sizeof(T), LDSK = BK + 16 / (int)sizeof(T);
    if constexpr (KMAJ) {
#pragma unroll
        for (int i = 0; i < StageRegs<R, NT>::KM; i++) {
            const int idx = tid + NT * i;
            if ((R * 8) % NT == 0 || idx < R * 8) st16(s + (idx >> 3) * LDSK + (idx & 7) * VEC, r[i]);
        }
    } else {
        constexpr int KQ = BK / 4;
#pragma unroll
        for (int bl = 0; bl < StageRegs<R, NT>::KS_BLOCKS; bl++) {
            const int idx = tid + NT * bl;
            if ((2 * R) % NT == 0 || idx < 2 * R) {
                const int kq = idx % KQ, rg = idx / KQ;
                const uint4 t[4] = {r[4 * bl], r[4 * bl + 1], r[4 * bl + 2], r[4 * bl + 3]};
                store_t4<T>(s + rg * VEC * LDSK + 4 * kq, LDSK, t);
            }
        }
    }
}

// Epilogue of one workgroup tile: lane holds C[m][n .. n+3] for its
// TM x TN 16x16 MFMA tiles.
// XS (bf16 outputs staged through LDS): the bias is already in the
// accumulators, and every store is a buffer store whose out-of-range lanes
// are sent past the resource range, so each wave issues exactly
// TM * SPI (twice that with the GELU pre-activation) store instructions.
template <typename T, typename TL, int EPI, typename OutT, bool STG = false, bool XS = false>
DEV void gemm_epilogue(const Args& g, const f32x4_t (&acc)[TL::TM][TL::TN], int m0, int n0, int wm, int wn, int l16,
                       int g4, bf16_t* stage = nullptr) {
    constexpr int TM = TL::TM, TN = TL::TN;
    if constexpr (EPI == GEMM_BIAS_GELU_SMX) {
        // G = gelu(v + bias) stored, plus (max, sum exp(G - max)) of each row
        // over this wave's 64 columns; a row's 64 values sit in the 4 lanes
        // l16 + 16 g (4 tiles x 4 values each), combined with two shuffles.
        static_assert(TL::WTN == 64, "partials are per 64 columns");
        const int nw = n0 + wn * 64;
        float2* part = (float2*)g.aux_out;
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const int m = m0 + wm * TL::WTM + 16 * i + l16;
            float v[TN][4];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int n = nw + 16 * j + 4 * g4;
                const bool ok = n < g.N;
                float bb[4] = {0.f, 0.f, 0.f, 0.f};
                if (ok) load4<T>((const T*)g.bias + n, bb);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    v[j][r] = gelu_f<T>(g.alpha * acc[i][j][r] + bb[r]);
                    if (ok) mx = fmaxf(mx, v[j][r]);
                }
                if (ok && m < g.M) store4<OutT>((OutT*)g.C + (size_t)m * g.ldc + n, v[j]);
            }
            mx = xor32_combine(xor16_combine(mx, MaxOp()), MaxOp());
            float sm = 0.f;
#pragma unroll
            for (int j = 0; j < TN; j++)
                if (nw + 16 * j + 4 * g4 < g.N)
#pragma unroll
                    for (int r = 0; r < 4; r++) sm += expf(v[j][r] - mx);
            sm = xor32_combine(xor16_combine(sm, AddOp()), AddOp());
            if (g4 == 0 && m < g.M && nw < g.N) part[(size_t)m * g.ldaux + nw / 64] = make_float2(mx, sm);
        }
        return;
    }
    // The epilogue's global reads (bias, residual, stored pre-activation,
    // accumulator) are issued ahead of the stores they feed: the compiler cannot
    // tell that the output aliases none of them and would otherwise order each
    // read after the previous tile's store, one memory round trip per 16x16
    // tile.
    constexpr bool HAS_BIAS = !XS && (EPI == GEMM_BIAS || EPI == GEMM_BIAS_GELU || EPI == GEMM_BIAS_RESID);
    constexpr bool HAS_AUX = EPI == GEMM_BIAS_RESID || EPI == GEMM_GELU_BWD || EPI == GEMM_ACCUM;
    using AuxT = std::conditional_t<EPI == GEMM_ACCUM, float, T>;
    using Raw = std::conditional_t<sizeof(AuxT) == 2, uint2, float4>;
    const int nb = n0 + wn * TL::WTN + 4 * g4;
    const int mb = m0 + wm * TL::WTM + l16;
    // (reads are unconditional, from a clamped in-range address, and unused
    // lanes' values are discarded: a read under a branch would be waited for
    // before the branch closes)
    float bb[TN][4];
    if constexpr (HAS_BIAS) {
        using RawB = std::conditional_t<sizeof(T) == 2, uint2, float4>;
        RawB rb[TN];
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int n = nb + 16 * j;
            rb[j] = *reinterpret_cast<const RawB*>((const T*)g.bias + (n < g.N ? n : 0));
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            if constexpr (sizeof(T) == 2) {
                const uint2 u = (const uint2&)rb[j];
                bb[j][0] = __uint_as_float(u.x << 16); bb[j][1] = __uint_as_float(u.x & 0xffff0000u);
                bb[j][2] = __uint_as_float(u.y << 16); bb[j][3] = __uint_as_float(u.y & 0xffff0000u);
            } else {
                const float4 u = (const float4&)rb[j];
                bb[j][0] = u.x; bb[j][1] = u.y; bb[j][2] = u.z; bb[j][3] = u.w;
            }
        }
    }
    // auxiliary reads in groups of G tile rows (at most 32 registers per
    // group); group gi + 1 is requested before group gi is stored.  With 16
    // waves per workgroup (128 registers per lane) one tile row at a time.
    constexpr bool TIGHT = TL::NT >= 1024 || TL::SK > 1;
    constexpr int RPR = (int)sizeof(Raw) / 4;
    constexpr int G = !HAS_AUX ? TM : TIGHT ? 1 : (TM * TN * RPR <= 32 ? TM : std::max(1, 32 / (TN * RPR)));
    constexpr int NBUF = HAS_AUX && !TIGHT ? 2 : 1;
    static_assert(TM % G == 0, "tile rows split evenly into groups");
    Raw aux[NBUF][HAS_AUX ? G : 1][HAS_AUX ? TN : 1];
    auto load_group = [&](int gi, Raw (&dst)[HAS_AUX ? G : 1][HAS_AUX ? TN : 1]) {
        if constexpr (HAS_AUX) {
            const AuxT* src = EPI == GEMM_ACCUM ? (const AuxT*)g.C : (const AuxT*)g.aux_in;
            const size_t ld = EPI == GEMM_ACCUM ? (size_t)g.ldc : (size_t)g.ldaux;
#pragma unroll
            for (int ii = 0; ii < G; ii++)
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int m = mb + 16 * (gi * G + ii), n = nb + 16 * j;
                    const bool ok = m < g.M && n < g.N;
                    dst[ii][j] = *reinterpret_cast<const Raw*>(src + (ok ? (size_t)m * ld + n : 0));
                }
        }
    };
    // bf16 outputs with a staging area (16 rows of this wave's columns in
    // LDS): a 16-row slice of the wave's tile is written to LDS as computed
    // (lane: one row, 4 columns per 16-column tile) and read back as 16-byte
    // pieces of whole rows, so each store instruction writes full 128-byte
    // lines instead of 32 bytes in each of 16 rows.
    constexpr int SRP = TL::WTN + 8;            // staging row pitch (elements)
    constexpr int SPR = TL::WTN / 8;            // 16-byte pieces per row
    constexpr int SPI = (16 * SPR + 63) / 64;   // store instructions per slice
    constexpr bool STAGED = STG && sizeof(OutT) == 2 && EPI != EPI_SPLIT && EPI != GEMM_ACCUM &&
                            EPI != GEMM_BIAS_GELU_SMX;
    auto put = [&](int j, const float* v) {  // this lane's 4 values of tile j into the slice
        st8(stage + l16 * SRP + 16 * j + 4 * g4, make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
    };
    auto flush = [&](void* dst, long ld, int mrow0, int ncol0) {  // slice rows -> memory
        if constexpr (XS) {
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc((bf16_t*)dst + (size_t)mrow0 * ld, rsrc_range(((long)g.M - mrow0) * ld * 2));
#pragma unroll
            for (int k = 0; k < SPI; k++) {
                const int slot = (l16 + 16 * g4) + 64 * k;
                const bool in = slot < 16 * SPR;
                const int sl = in ? slot : 0;
                const int row = sl / SPR, col = 8 * (sl % SPR);
                const uint4 d = ld16(stage + row * SRP + col);
                const bool ok = in && ncol0 + col < g.N;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i_t, d), rs,
                                                       ok ? (int)((row * ld + ncol0 + col) * 2) : (int)kBufOOB, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < SPI; k++) {
            const int slot = (l16 + 16 * g4) + 64 * k;
            const int row = slot / SPR, col = 8 * (slot % SPR);
            if (slot < 16 * SPR) {
                const uint4 d = ld16(stage + row * SRP + col);
                const int m = mrow0 + row, n = ncol0 + col;
                if (m < g.M && n < g.N) st16((bf16_t*)dst + (size_t)m * ld + n, d);
            }
        }
    };
    // fp32 outputs (split partials, accumulated weight gradients) the same
    // way, 8 rows at a time (a staged row is 4x wider than a bf16 one)
    constexpr bool STAGED32 = STG && sizeof(OutT) == 4 && (EPI == EPI_SPLIT || EPI == GEMM_ACCUM);
    constexpr int SRP32 = TL::WTN + 4, SPR32 = TL::WTN / 4, SPI32 = (8 * SPR32 + 63) / 64;
    float* const stage32 = (float*)stage;
    auto flush32 = [&](float* dst, long ld, int mrow0, int ncol0) {
#pragma unroll
        for (int k = 0; k < SPI32; k++) {
            const int slot = (l16 + 16 * g4) + 64 * k;
            const int row = slot / SPR32, col = 4 * (slot % SPR32);
            if (slot < 8 * SPR32) {
                const uint4 d = ld16(stage32 + row * SRP32 + col);
                const int m = mrow0 + row, n = ncol0 + col;
                if (m < g.M && n < g.N) st16(dst + (size_t)m * ld + n, d);
            }
        }
    };
    if constexpr (!TIGHT) load_group(0, aux[0]);
#pragma unroll
    for (int i = 0; i < TM; i++) {
        if constexpr (HAS_AUX) {
            if (TIGHT) load_group(i, aux[0]);
            else if (i % G == 0 && i + G < TM) load_group(i / G + 1, aux[(i / G + 1) % NBUF]);
        }
        const int m = mb + 16 * i;
        if constexpr (STAGED32) {
            float vo[TN][4];
#pragma unroll
            for (int j = 0; j < TN; j++) {
#pragma unroll
                for (int r = 0; r < 4; r++) vo[j][r] = g.alpha * acc[i][j][r];
                if constexpr (EPI == GEMM_ACCUM) {
                    const float4 u = (const float4&)aux[(i / G) % NBUF][i % G][j];
                    vo[j][0] += u.x; vo[j][1] += u.y; vo[j][2] += u.z; vo[j][3] += u.w;
                }
            }
            float* const dst = EPI == EPI_SPLIT ? g.ws + (size_t)blockIdx.y * g.M * g.N : (float*)g.C;
            const long ld = EPI == EPI_SPLIT ? (long)g.N : g.ldc;
            const int mrow0 = m0 + wm * TL::WTM + 16 * i, ncol0 = n0 + wn * TL::WTN;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                if ((l16 >> 3) == h) {
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        *reinterpret_cast<float4*>(stage32 + (l16 - 8 * h) * SRP32 + 16 * j + 4 * g4) =
                            make_float4(vo[j][0], vo[j][1], vo[j][2], vo[j][3]);
                }
                flush32(dst, ld, mrow0 + 8 * h, ncol0);
            }
            continue;
        }
        if constexpr (STAGED) {
            // every lane takes part in the slice exchange, in range or not
            float vo[TN][4], vp[TN][4];
#pragma unroll
            for (int j = 0; j < TN; j++) {
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; r++) v[r] = g.alpha * acc[i][j][r];
                float a[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (HAS_AUX) {
                    const uint2 u = (const uint2&)aux[(i / G) % NBUF][i % G][j];
                    a[0] = __uint_as_float(u.x << 16); a[1] = __uint_as_float(u.x & 0xffff0000u);
                    a[2] = __uint_as_float(u.y << 16); a[3] = __uint_as_float(u.y & 0xffff0000u);
                }
                if constexpr (HAS_BIAS) {
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] += bb[j][r];
                }
                if constexpr (EPI == GEMM_BIAS_GELU) {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        vp[j][r] = v[r];
                        v[r] = gelu_f<T>(to_f<T>(from_f<T>(v[r])));
                    }
                }
                if constexpr (EPI == GEMM_BIAS_RESID) {
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] += a[r];
                }
                if constexpr (EPI == GEMM_GELU_BWD) {
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] *= gelu_grad_f<T>(a[r]);
                }
#pragma unroll
                for (int r = 0; r < 4; r++) vo[j][r] = v[r];
            }
            const int mrow0 = m0 + wm * TL::WTM + 16 * i, ncol0 = n0 + wn * TL::WTN;
            if constexpr (EPI == GEMM_BIAS_GELU) {
#pragma unroll
                for (int j = 0; j < TN; j++) put(j, vp[j]);
                flush(g.aux_out, g.ldaux, mrow0, ncol0);
            }
#pragma unroll
            for (int j = 0; j < TN; j++) put(j, vo[j]);
            flush(g.C, g.ldc, mrow0, ncol0);
            continue;
        }
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int n = nb + 16 * j;
            if (n >= g.N) continue;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; r++) v[r] = g.alpha * acc[i][j][r];
            float a[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (HAS_AUX) {
                const Raw& ru = aux[(i / G) % NBUF][i % G][j];
                if constexpr (sizeof(AuxT) == 2) {
                    const uint2 u = (const uint2&)ru;
                    a[0] = __uint_as_float(u.x << 16); a[1] = __uint_as_float(u.x & 0xffff0000u);
                    a[2] = __uint_as_float(u.y << 16); a[3] = __uint_as_float(u.y & 0xffff0000u);
                } else {
                    const float4 u = (const float4&)ru;
                    a[0] = u.x; a[1] = u.y; a[2] = u.z; a[3] = u.w;
                }
            }
            if constexpr (EPI == EPI_SPLIT) {
                float* w = g.ws + (size_t)blockIdx.y * g.M * g.N + (size_t)m * g.N + n;
                store4<float>(w, v);
            } else if constexpr (EPI == GEMM_ACCUM) {
#pragma unroll
                for (int r = 0; r < 4; r++) v[r] += a[r];
                store4<float>((float*)g.C + (size_t)m * g.ldc + n, v);
            } else {
                if constexpr (HAS_BIAS) {
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] += bb[j][r];
                }
                if constexpr (EPI == GEMM_BIAS_GELU) {
                    store4<T>((T*)g.aux_out + (size_t)m * g.ldaux + n, v);
                    // GELU of the stored (rounded) pre-activation
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] = gelu_f<T>(to_f<T>(from_f<T>(v[r])));
                }
                if constexpr (EPI == GEMM_BIAS_RESID) {
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] += a[r];
                }
                if constexpr (EPI == GEMM_GELU_BWD) {
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] *= gelu_grad_f<T>(a[r]);
                }
                store4<OutT>((OutT*)g.C + (size_t)m * g.ldc + n, v);
            }
        }
    }
}

template <typename T, int BM, int BN, int WT, bool AK, bool BKM, int EPI, typename OutT, bool BIAS>
__global__ __launch_bounds__((TileOf<T, BM, BN, WT>::NT), (TileOf<T, BM, BN, WT>::OCC)) void gemm_kernel(const Args g) {
    using TL = TileOf<T, BM, BN, WT>;
    constexpr int LDSK = TL::LDSK, BK = TL::BK, TM = TL::TM, TN = TL::TN, NT = TL::NT;
    __shared__ __attribute__((aligned(16))) T sA[2][BM * LDSK];
    __shared__ __attribute__((aligned(16))) T sB[2][BN * LDSK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % TL::WM, wn = wave / TL::WM;
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

    const int ktiles = (g.K + BK - 1) / BK;
    const int kt0 = blockIdx.y * g.kps;
    const int kt1 = min(kt0 + g.kps, ktiles);

    const T* __restrict__ A = (const T*)g.A;
    const T* __restrict__ B = (const T*)g.B;

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fused bias gradient (weight-gradient products): the A slab holds dY^T, so
    // its row sums over k are the column sums of dY.  Only the first column
    // tile of each row tile does it.
    const bool do_bias = BIAS && tn == 0;
    constexpr int TPR = NT / BM;        // threads per slab row (2 or 4)
    constexpr int EPT = BK / TPR;       // elements each sums per stage
    float bsum = 0.f;

    // Operand slabs are prefetched into registers DEPTH stages ahead of their
    // use: with DEPTH = 2 (two workgroups per CU) the slab for stage kt+2 is
    // requested at the start of stage kt and written to LDS at the end of
    // stage kt+1, so a global load has two stages of MFMA work to arrive; the
    // big tiles (one workgroup per CU, accumulators filling the register file)
    // prefetch one stage ahead.
    constexpr int DEPTH = TL::DEPTH;
    constexpr int NRA = StageRegs<BM, NT>::N, NRB = StageRegs<BN, NT>::N;
    uint4 ra0[NRA], rb0[NRB], ra1[DEPTH == 2 ? NRA : 1], rb1[DEPTH == 2 ? NRB : 1];
    SlabAddr<T, BM, AK, NT> adA;
    SlabAddr<T, BN, BKM, NT> adB;
    adA.init(g.lda, tid);
    adB.init(g.ldb, tid);
    if (kt0 < kt1) {
        slab_load<T, BM, AK, NT>(ra0, adA, A, g.lda, m0, g.M, kt0 * BK, g.K);
        slab_load<T, BN, BKM, NT>(rb0, adB, B, g.ldb, n0, g.N, kt0 * BK, g.K);
        slab_store<T, BM, AK, NT>(ra0, sA[0], tid);
        slab_store<T, BN, BKM, NT>(rb0, sB[0], tid);
        if constexpr (DEPTH == 2) {
            const int k1 = min(kt0 + 1, kt1 - 1);
            slab_load<T, BM, AK, NT>(ra1, adA, A, g.lda, m0, g.M, k1 * BK, g.K);
            slab_load<T, BN, BKM, NT>(rb1, adB, B, g.ldb, n0, g.N, k1 * BK, g.K);
        }
    }
    __syncthreads();

    // One stage: the loop body has no branches, fragments of step ks+1 are
    // read while step ks runs, and the instruction groups are interleaved
    // explicitly: global loads first, then MFMAs alternating with the next
    // step's LDS reads, then MFMAs alternating with the LDS writes of the
    // prefetched slab.
    constexpr int NF = TM + TN;                                // fragment reads per step
    constexpr int NMMA = TM * TN * (sizeof(T) == 2 ? 1 : 8);  // MFMAs per step
    auto stage = [&](int kt, uint4* lda_, uint4* ldb_, const uint4* sta_, const uint4* stb_) {
        const int cur = (kt - kt0) & 1;
        const int nk = min(kt + DEPTH, kt1 - 1);
        slab_load<T, BM, AK, NT>(lda_, adA, A, g.lda, m0, g.M, nk * BK, g.K);
        slab_load<T, BN, BKM, NT>(ldb_, adB, B, g.ldb, n0, g.N, nk * BK, g.K);
        const T* a_s = sA[cur];
        const T* b_s = sB[cur];
        Frag<T> fa[TL::FBUF][TM], fb[TL::FBUF][TN];
#pragma unroll
        for (int t = 0; t < TN; t++) frag_ld(fb[0][t], b_s + (wn * TL::WTN + 16 * t + l16) * LDSK + 8 * g4);
#pragma unroll
        for (int t = 0; t < TM; t++) frag_ld(fa[0][t], a_s + (wm * TL::WTM + 16 * t + l16) * LDSK + 8 * g4);
#pragma unroll
        for (int ks = 0; ks < TL::KSTEPS; ks++) {
            const int c = TL::FBUF == 2 ? (ks & 1) : 0;
            if (TL::FBUF == 2 && ks + 1 < TL::KSTEPS) {
                const int kofs = (ks + 1) * 32 + 8 * g4;
#pragma unroll
                for (int t = 0; t < TN; t++) frag_ld(fb[c ^ 1][t], b_s + (wn * TL::WTN + 16 * t + l16) * LDSK + kofs);
#pragma unroll
                for (int t = 0; t < TM; t++) frag_ld(fa[c ^ 1][t], a_s + (wm * TL::WTM + 16 * t + l16) * LDSK + kofs);
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) mma(acc[i][j], fb[c][j], fa[c][i]);
            if (TL::FBUF == 1 && ks + 1 < TL::KSTEPS) {
                const int kofs = (ks + 1) * 32 + 8 * g4;
#pragma unroll
                for (int t = 0; t < TN; t++) frag_ld(fb[0][t], b_s + (wn * TL::WTN + 16 * t + l16) * LDSK + kofs);
#pragma unroll
                for (int t = 0; t < TM; t++) frag_ld(fa[0][t], a_s + (wm * TL::WTM + 16 * t + l16) * LDSK + kofs);
            }
        }
        if constexpr (BIAS) {
            // (every workgroup sums, only the first column tile keeps the result:
            // a uniform branch here would split the scheduling region)
            const T* rowp = a_s + (tid / TPR) * LDSK + (tid % TPR) * EPT;
#pragma unroll
            for (int q = 0; q < EPT / TL::VEC; q++) {
                float f[TL::VEC];
                unpack16<T>(ld16(rowp + q * TL::VEC), f);
#pragma unroll
                for (int e = 0; e < TL::VEC; e++) bsum += f[e];
            }
        }
        slab_store<T, BM, AK, NT>(sta_, sA[cur ^ 1], tid);
        slab_store<T, BN, BKM, NT>(stb_, sB[cur ^ 1], tid);
        __builtin_amdgcn_sched_group_barrier(0x020, NRA + NRB, 0);  // global loads
        __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);         // step-0 fragments
#pragma unroll
        for (int ks = 0; ks < TL::KSTEPS; ks++) {
            if (ks + 1 < TL::KSTEPS) {
#pragma unroll
                for (int q = 0; q < NF; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, NMMA / NF > 0 ? NMMA / NF : 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, NMMA / 16 > 0 ? NMMA / 16 : 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
                }
            }
        }
        __syncthreads();
    };
    if constexpr (DEPTH == 2) {
        for (int kt = kt0; kt < kt1; kt += 2) {
            stage(kt, ra0, rb0, ra1, rb1);
            if (kt + 1 < kt1) stage(kt + 1, ra1, rb1, ra0, rb0);
        }
    } else {
        for (int kt = kt0; kt < kt1; kt++) stage(kt, ra0, rb0, ra0, rb0);
    }

    if (do_bias) {
        if constexpr (TPR >= 2) bsum += dpp_mov<kDppQuadXor1>(bsum);
        if constexpr (TPR >= 4) bsum += dpp_mov<kDppQuadXor2>(bsum);
        const int m = m0 + tid / TPR;
        if ((tid % TPR) == 0 && m < g.M) {
            if constexpr (EPI == EPI_SPLIT) g.wsb[(size_t)blockIdx.y * g.M + m] = g.alpha * bsum;
            else g.dbias[m] += g.alpha * bsum;
        }
    }

    gemm_epilogue<T, TL, EPI, OutT>(g, acc, m0, n0, wm, wn, l16, g4);
}

// ------------------------------------------------------------ direct to LDS --
// bf16 products whose operand slabs go from global memory straight into LDS
// (buffer loads with the LDS-destination bit): no staging registers, no LDS
// store instructions, and no wait on a load until the barrier before the
// stage that consumes it.  Each wave's 16-byte lane loads fill 1 KB of LDS
// contiguously (lane i -> base + 16 i), so the LDS layout is chosen by which
// global element each lane fetches:
//  - a k-contiguous slab (R rows x 64 contraction elements) keeps rows of 128
//    bytes with the 16-byte chunk c of row r stored at chunk c ^ (r & 7), so
//    the fragment reads of 8 consecutive rows hit 8 different bank groups;
//  - a k-strided slab (rows of the operand contiguous in memory) is stored as
//    64 contraction rows of R elements, its 32-byte unit u of contraction row
//    k at unit u ^ f(k), and fragments are read with the LDS transpose load
//    (ds_read_b64_tr_b16: within 16 lanes, lane l gets element l%16 of four
//    consecutive rows), two per fragment, which gives lane (row, group g) the
//    contraction indices 8g..8g+7 -- the same slots as the k-contiguous read,
//    so both layouts feed the same MFMA code.
// Two stages in separate LDS arrays: loads for stage kt+1 are issued right
// after the barrier that opens stage kt and waited for at the next one.
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;


// Stage depth BK (contraction elements per stage) and stage count NS per tile:
// 64-deep stages; two for the square tiles (a 256x256 stage is 64 KB), three
// for the rectangular ones whose three stages fit in LDS beside the epilogue's
// bias row (a 128x192 stage is 40 KB), which run their short-K products 10-20%
// faster than with two; two for 256x192 (56 KB a stage).
template <int BM, int BN>
struct DtlCfg {
    static constexpr int BK = 64;
    static constexpr int NS = BM != BN && 3 * (BM + BN) * BK * 2 <= 150 * 1024 ? 3 : 2;
    static_assert(NS >= 2 && NS <= 4, "the stage loop unrolls 2 to 4 stage buffers");
    static_assert(BK == 32 || BK == 64, "stages are one or two 32-deep MFMA steps");
};

// chunk swizzle of a k-contiguous slab row (16-byte chunks; 8 per 64-deep
// row, 4 per 32-deep row): 8 consecutive rows land in 8 different bank groups
template <int BK>
DEV int dtl_swz(int r) {
    return BK == 64 ? (r & 7) : ((r >> 1) & 3);
}
// Unit swizzle of a k-strided slab: contraction row k holds its R / 16 units
// of 16 rows permuted by the key dtl_fk(k) -- an XOR for power-of-two unit
// counts, a rotation otherwise.  The 16 contraction rows one transposing read
// takes (k = 8 g + q, q < 4, g < 4) get keys 0..15 (mod the unit count), so
// with a unit count that is a multiple of four, and so a row pitch that is a
// multiple of 128 bytes, their units fall evenly on the four 32-byte bank
// groups.
template <int R>
DEV int dtl_fk(int k) {
    constexpr int U = R / 16;
    const int f = (k & 3) | (((k >> 3) & 3) << 2);
    return (U & (U - 1)) == 0 ? (f & (U - 1)) : f % U;
}
template <int R>
DEV int dtl_lds_unit(int g, int k) {  // LDS unit holding unit g of row k
    constexpr int U = R / 16;
    if constexpr ((U & (U - 1)) == 0) {
        return g ^ dtl_fk<R>(k);
    } else {
        const int u = g - dtl_fk<R>(k);
        return u < 0 ? u + U : u;
    }
}
template <int R>
DEV int dtl_glob_unit(int u, int k) {  // unit of row k held in LDS unit u
    constexpr int U = R / 16;
    if constexpr ((U & (U - 1)) == 0) {
        return u ^ dtl_fk<R>(k);
    } else {
        const int g = u + dtl_fk<R>(k);
        return g >= U ? g - U : g;
    }
}

template <int R_, bool KMAJ_, int NW_, int BK_>
struct DtlSlab {
    static constexpr int R = R_, NW = NW_, BK = BK_;
    static constexpr bool KMAJ = KMAJ_;
    static constexpr int NQ = R * BK / 512 / NW;  // 1 KB load instructions per wave per stage
    static_assert(NQ >= 1 && (R * BK / 512) % NW == 0, "slab must split evenly over the waves");
    uint32_t off[NQ];  // per-lane byte offset from the slab origin in global memory
    int kc[KMAJ ? NQ : 1];
    DEV void init(long ld, int lane, int wave) {
#pragma unroll
        for (int q = 0; q < NQ; q++) {
            const int j = wave + NW * q;  // which 1 KB of the slab
            if constexpr (KMAJ) {
                constexpr int CPR = BK / 8;      // 16-byte chunks per row
                constexpr int RPK = 64 / CPR;    // rows per 1 KB
                const int r = RPK * j + lane / CPR;
                const int c = (lane % CPR) ^ dtl_swz<BK>(r);
                kc[q] = 8 * c;
                off[q] = (uint32_t)(((long)r * ld + 8 * c) * 2);
            } else {
                const int e = 512 * j + 8 * lane;  // element of the slab, in LDS order
                const int k = e / R, c = e % R;
                const int r = 16 * dtl_glob_unit<R>(c >> 4, k) + (c & 8);
                off[q] = (uint32_t)(((long)k * ld + r) * 2);
            }
        }
    }
};

// Issue this wave's loads of the slab at (rows r0.., contraction k0..) into dst
// (per-lane offsets and, k-contiguous, contraction indices from DtlSlab).
template <int R, bool KMAJ, int NW, int BK>
DEV void dtl_issue(const uint32_t* off, const int* kc, bf16_t* dst, const bf16_t* __restrict__ p, long ld, int r0,
                   int Rmax, int k0, int K, int wave) {
    constexpr int NQ = R * BK / 512 / NW;
    if constexpr (KMAJ) {
        const long org = (long)r0 * ld + k0;
        const uint32_t bytes = rsrc_range(((long)Rmax * ld - org) * 2);
        const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(p + org, bytes);
        const int klim = K - k0;
        // every load of the wave starts at the same chunk of its row (the chunk
        // swizzle repeats every 8 rows and each load is 512 / BK rows further
        // on), so one offset and one contraction index serve all NQ loads
        const uint32_t qstride = (uint32_t)((512 / BK) * NW * ld * 2);
        const bool kin = kc[0] < klim;
#pragma unroll
        for (int q = 0; q < NQ; q++) lds_dma16(rs, kin ? off[0] + q * qstride : kBufOOB, dst + (wave + NW * q) * 512);
    } else {
        const long org = (long)k0 * ld + r0;
        const uint32_t bytes = rsrc_range(((long)K * ld - org) * 2);
        const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(p + org, bytes);
#pragma unroll
        for (int q = 0; q < NQ; q++) lds_dma16(rs, off[q], dst + (wave + NW * q) * 512);
    }
}

// Per-lane element offsets of the fragment reads of one operand: KT tiles of 16
// rows starting at wave row wb, for each 32-deep MFMA step of a stage.
template <int R, bool KMAJ, int KT, int BK, int NKS = BK / 32>
struct DtlFrag {
    static constexpr int KS = NKS;
    int ofs[KT][KS];  // [tile][step] (k-strided: the first of the two transpose reads)
    DEV void init(int wb, int l16, int g4, int ks0 = 0) {
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int rb = wb + 16 * t;
#pragma unroll
            for (int kk = 0; kk < KS; kk++) {
                const int ks = ks0 + kk;
                if constexpr (KMAJ) {
                    ofs[t][kk] = (rb + l16) * BK + (((4 * ks + g4) ^ dtl_swz<BK>(rb + l16)) << 3);
                } else {
                    // (rows k and k + 4, the two transposing reads, share their unit key)
                    const int k = 32 * ks + 8 * g4 + (l16 >> 2);
                    ofs[t][kk] = k * R + (dtl_lds_unit<R>(rb >> 4, k) << 4) + 4 * (l16 & 3);
                }
            }
        }
    }
};

template <int R, bool KMAJ>
DEV void dtl_frag_ld(Frag<bf16_t>& f, const bf16_t* s, int ofs) {
    if constexpr (KMAJ) {
        frag_ld(f, s + ofs);
    } else {
        const v4s_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(s + ofs));
        const v4s_t b =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(s + ofs + 4 * R));
        typedef short v8s_t __attribute__((ext_vector_type(8)));
        const v8s_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        f.v = __builtin_bit_cast(bf16x8_t, ab);
    }
}

// Whether a tile shape and epilogue run the persistent tile loop (launches
// then have at most one workgroup per resident slot).  Only epilogues that
// read no activations do: a read issued behind the next tile's loads waits
// for them (vector memory operations complete in order), and the next tile's
// first stage waits for the stores before it, so an epilogue that reads
// (residual, stored pre-activation, accumulator) measured slower persistent;
// the fused bias sum and split partials stay one tile per workgroup too.
// Whether a tile keeps two stages of fragments in registers (the stage loop
// that reads stage kt + 1's fragments before stage kt's MFMAs): only where
// both sets and the accumulators fit the registers each wave has at the
// tile's occupancy (512 per SIMD lane shared by the waves on that SIMD).
// Two waves per SIMD leave 256 registers per lane; there the epilogues of
// the forward layouts (bias, GELU, residual reads) and the fused bias sum
// still spill, so only the input-gradient layout's stores take it.
template <int BM, int BN, int WT, bool AK, bool BKM, int EPI>
constexpr bool dtl_rp() {
    using TL = TileOf<bf16_t, BM, BN, WT>;
    constexpr int per_simd = (TL::NT / 64) * TL::OCC / 4;
    constexpr int regs = 512 / (per_simd < 1 ? 1 : per_simd);
    constexpr int KS = DtlCfg<BM, BN>::BK / 32 / TL::SK;
    constexpr bool fits = 2 * (TL::TM + TL::TN) * KS * 4 + TL::TM * TL::TN * 4 + 48 <= regs;
    return per_simd <= 1 ? fits : fits && AK && !BKM && (EPI == GEMM_STORE || EPI == GEMM_GELU_BWD);
}

template <int BM, int BN, int WT, int EPI, bool BIAS>
constexpr bool dtl_persistent() {
    constexpr int NT = TileOf<bf16_t, BM, BN, WT>::NT;
    if (BIAS || TileOf<bf16_t, BM, BN, WT>::SK > 1) return false;
    return EPI == GEMM_STORE || EPI == GEMM_BIAS || (EPI == GEMM_BIAS_GELU && NT <= 512);
}

// One launch for a list of weight-gradient products: problem class c holds
// count[c] products of one shape at fixed strides (the layers of the model),
// and global tile u belongs to class c when begin[c] <= u < begin[c + 1].
// Every product accumulates into its own fp32 gradient, so one tile per
// workgroup and no K split: the whole contraction (B*T) runs in one tile.
struct GroupArgs {
    const void* A[kMaxGroup];
    const void* B[kMaxGroup];
    float* C[kMaxGroup];
    float* dbias[kMaxGroup];
    long lda[kMaxGroup], ldb[kMaxGroup], ldc[kMaxGroup];
    long sA[kMaxGroup], sB[kMaxGroup], sC[kMaxGroup], sBias[kMaxGroup];  // per-product strides (elements)
    int M[kMaxGroup], N[kMaxGroup], K[kMaxGroup], tiles_m[kMaxGroup], tiles_n[kMaxGroup];
    float alpha[kMaxGroup];
    int begin[kMaxGroup + 1];
    int np, total;
};

// a[c] for a wave-uniform c (a chain of scalar selects, no indexed load)
template <typename X, int N>
DEV X pick(const X (&a)[N], int c) {
    X r = a[0];
#pragma unroll
    for (int i = 1; i < N; i++) r = c == i ? a[i] : r;
    return r;
}

template <bool GRP>
using KernArgs = std::conditional_t<GRP, GroupArgs, Args>;

template <int BM, int BN, int WT, bool AK, bool BKM, int EPI, typename OutT, bool BIAS, bool GRP = false>
__global__ __launch_bounds__((TileOf<bf16_t, BM, BN, WT>::NT), (TileOf<bf16_t, BM, BN, WT>::OCC)) void
gemm_dtl_kernel(const KernArgs<GRP> ka) {
    using T = bf16_t;
    static_assert(!GRP || (EPI == GEMM_ACCUM && !AK && !BKM), "grouped launches are weight-gradient products");
    using TL = TileOf<T, BM, BN, WT>;
    constexpr int TM = TL::TM, TN = TL::TN, NT = TL::NT, NW = NT / 64;
    constexpr int BK = DtlCfg<BM, BN>::BK, NS = DtlCfg<BM, BN>::NS, SK = TL::SK, KS = BK / 32 / SK;
    static_assert(SK == 1 || (SK == 2 && BK / 32 == 2 && !BIAS && !GRP), "two depth slices of a 64-deep stage");
    static_assert(!BIAS || !AK, "the fused bias sum reads a k-strided A slab");
    // one LDS array per stage and operand, so the compiler can tell which
    // buffer an LDS-destination load writes and which one a fragment read uses
    __shared__ __attribute__((aligned(1024))) T sA0[BM * BK];
    __shared__ __attribute__((aligned(1024))) T sA1[BM * BK];
    __shared__ __attribute__((aligned(1024))) T sA2[NS > 2 ? BM * BK : 8];
    __shared__ __attribute__((aligned(1024))) T sA3[NS > 3 ? BM * BK : 8];
    __shared__ __attribute__((aligned(1024))) T sB0[BN * BK];
    __shared__ __attribute__((aligned(1024))) T sB1[BN * BK];
    __shared__ __attribute__((aligned(1024))) T sB2[NS > 2 ? BN * BK : 8];
    __shared__ __attribute__((aligned(1024))) T sB3[NS > 3 ? BN * BK : 8];
    __shared__ float sbias[BIAS ? (NT / (BM / 4)) * BM : 1];

    const int tid = threadIdx.x;
    // (the wave index is the same in all lanes; readfirstlane lets the
    // compiler see that, so branches on it are scalar)
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // SK = 2: waves w and w + WM * WN hold the same outputs over the two
    // 32-deep halves of every stage
    const int kslice = wave / (TL::WM * TL::WN), wsub = wave % (TL::WM * TL::WN);
    const int wm = wsub % TL::WM, wn = wsub / TL::WM;
    const int l16 = lane & 15, g4 = lane >> 4;

    // Tiles are numbered u = 0 .. ntiles-1 and mapped so that the tiles of
    // one XCD (u % 8, as workgroups are handed out round-robin) form a
    // contiguous run, walked in groups of 8 row-tiles.  Persistent launches
    // have fewer workgroups than tiles: workgroup w takes tiles w, w + G,
    // w + 2G, ... (G = gridDim.x, a multiple of 8, so every tile stays on the
    // XCD the numbering intends), and the first stages of its next tile are
    // requested before the epilogue of the current one.
    constexpr bool PERSIST = !GRP && dtl_persistent<BM, BN, WT, EPI, BIAS>();
    constexpr bool RP = dtl_rp<BM, BN, WT, AK, BKM, EPI>();
    // bf16 outputs are staged through the LDS buffers of stage NS - 1, which
    // no load targets until the next tile's first stage: the larger of its two
    // slabs, or (64x144 waves) the first half of the waves in the A slab and
    // the second half in the B slab
    constexpr bool STAGE_ONE = NW * 16 * (TL::WTN + 8) <= (BM > BN ? BM : BN) * BK;
    constexpr bool STAGE_TWO = !STAGE_ONE && (NW / 2) * 16 * (TL::WTN + 8) <= (BM < BN ? BM : BN) * BK;
    constexpr bool CAN_STAGE = STAGE_ONE || STAGE_TWO;
    // Persistent bf16-output tiles (XS): the bias is the accumulators' initial
    // value, and the epilogue's stores stay in flight while the next tile
    // starts -- each wave issues exactly XS_STORES of them, so the waits of
    // the next tile's first stages allow that many younger operations.
    constexpr bool XS = PERSIST && CAN_STAGE && std::is_same<OutT, bf16_t>::value &&
                        (EPI == GEMM_STORE || EPI == GEMM_BIAS || EPI == GEMM_BIAS_GELU);
    constexpr int XS_SPI = (16 * (TL::WTN / 8) + 63) / 64;
    constexpr int XS_STORES = XS ? TM * XS_SPI * (EPI == GEMM_BIAS_GELU ? 2 : 1) : 0;
    constexpr bool ACC_BIAS = XS && (EPI == GEMM_BIAS || EPI == GEMM_BIAS_GELU);
    static_assert(BN <= 512, "one 1 KB load holds a tile's bias columns");
    __shared__ __attribute__((aligned(1024))) T sBiasRow[ACC_BIAS ? 512 : 8];  // the tile's bias columns
    Args g;
    int u = blockIdx.x;
    int tm, tn;
    if constexpr (GRP) {
        // global tile u (XCD-contiguous runs as below) -> class c, product l,
        // tile (tm, tn) of that product.  Neighbouring tiles (same XCD, run
        // at the same time) share the panel of the larger operand: column
        // tiles fastest when A (M x K) is the larger, row tiles fastest
        // otherwise, so that panel is fetched from HBM once per product
        const int nt = ka.total, full = (nt / 8) * 8;
        if (u < full) u = (u % 8) * (nt / 8) + (u / 8);
        int c = 0;
#pragma unroll
        for (int i = 1; i < kMaxGroup; i++) c = (i < ka.np && u >= ka.begin[i]) ? i : c;
        const int tmc = pick(ka.tiles_m, c), per = tmc * pick(ka.tiles_n, c);
        const int v = u - pick(ka.begin, c), l = v / per, w = v % per;
        if (pick(ka.M, c) >= pick(ka.N, c)) {
            const int tnc = per / tmc;
            tn = w % tnc;
            tm = w / tnc;
        } else {
            tm = w % tmc;
            tn = w / tmc;
        }
        g.A = (const T*)pick(ka.A, c) + l * pick(ka.sA, c);
        g.B = (const T*)pick(ka.B, c) + l * pick(ka.sB, c);
        g.C = pick(ka.C, c) + l * pick(ka.sC, c);
        float* const db = pick(ka.dbias, c);
        g.dbias = db ? db + l * pick(ka.sBias, c) : nullptr;
        g.lda = pick(ka.lda, c); g.ldb = pick(ka.ldb, c); g.ldc = pick(ka.ldc, c);
        g.M = pick(ka.M, c); g.N = pick(ka.N, c); g.K = pick(ka.K, c);
        g.alpha = pick(ka.alpha, c);
        g.kps = (g.K + 63) / 64;
        g.bias = nullptr; g.aux_in = nullptr; g.aux_out = nullptr; g.ldaux = 0; g.ws = nullptr; g.wsb = nullptr;
    } else {
        g = ka;
    }
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    auto tile_of = [&](int u, int& tm_, int& tn_) {
        const int full = (ntiles / 8) * 8;
        if (u < full) u = (u % 8) * (ntiles / 8) + (u / 8);
        const int GM = 8;
        const int in_group = GM * tiles_n;
        const int first_m = (u / in_group) * GM;
        const int gsz = min(tiles_m - first_m, GM);
        tm_ = first_m + ((u % in_group) % gsz);
        tn_ = (u % in_group) / gsz;
    };
    if constexpr (!GRP) tile_of(u, tm, tn);
    int m0 = tm * BM, n0 = tn * BN;

    // g.kps counts 64-deep k-tiles (the unit of the K split); stages are BK deep
    constexpr int SPT = 64 / BK;  // stages per 64-deep k-tile
    const int ktiles = (g.K + 63) / 64;
    const int kt0 = blockIdx.y * g.kps * SPT;
    const int kt1 = min(blockIdx.y * g.kps + g.kps, ktiles) * SPT;
    const T* __restrict__ A = (const T*)g.A;
    const T* __restrict__ B = (const T*)g.B;

    f32x4_t acc[TM][TN];

    // Waves that issue the LDS-destination loads: in the 8-wave tiles only
    // waves 0-3, one per SIMD, each issuing twice the share.  A
    // 1 KB load holds the CU's vector-memory path for many cycles and a wave
    // issues in order, so a loading wave stalls at the start of each stage;
    // its SIMD partner (wave w + 4) runs its MFMAs meanwhile instead of
    // stalling too (2-8% on the 8-wave tiles).
    constexpr int NL = NW == 8 ? 4 : NW;
    const bool loads = NL == NW || wave < NL;
    const int lw = NL == NW ? wave : wave % NL;
    DtlSlab<BM, AK, NL, BK> dA;
    DtlSlab<BN, BKM, NL, BK> dB;
    dA.init(g.lda, lane, lw);
    dB.init(g.ldb, lane, lw);
    DtlFrag<BM, AK, TM, BK, KS> fA;
    DtlFrag<BN, BKM, TN, BK, KS> fB;
    fA.init(wm * TL::WTM, l16, g4, kslice * KS);
    fB.init(wn * TL::WTN, l16, g4, kslice * KS);
    constexpr int NQS = DtlSlab<BM, AK, NL, BK>::NQ + DtlSlab<BN, BKM, NL, BK>::NQ;
    static_assert((NS - 1) * NQS <= 63, "vmcnt range");

    // fused bias gradient: column sums over k of the k-strided A slab
    constexpr int MQ = BM / 4, KG = NT / MQ, KPG = BK / KG;
    static_assert(!BIAS || KPG >= 1, "bias partial layout");
    const int bq = tid % MQ, bkg = tid / MQ;
    float bs[4] = {0.f, 0.f, 0.f, 0.f};
    const bool do_bias = BIAS && tn == 0 && g.dbias != nullptr;

    auto issue_at = [&](int kt, T* a_dst, T* b_dst, int mm0, int nn0) {
        if (loads) {
            dtl_issue<BM, AK, NL, BK>(dA.off, dA.kc, a_dst, A, g.lda, mm0, g.M, kt * BK, g.K, wave);
            dtl_issue<BN, BKM, NL, BK>(dB.off, dB.kc, b_dst, B, g.ldb, nn0, g.N, kt * BK, g.K, wave);
        }
    };
    auto issue = [&](int kt, T* a_dst, T* b_dst) { issue_at(kt, a_dst, b_dst, m0, n0); };
    // one stage's fragments of this wave (both operands, every 32-deep step)
    struct FragSet {
        Frag<T> fa[KS][TM], fb[KS][TN];
    };
    auto bias_sum = [&](const T* a_s) {
        if constexpr (BIAS) {
#pragma unroll
            for (int i = 0; i < KPG; i++) {
                const int k = bkg * KPG + i;
                const int m = 4 * bq;
                const uint2 v = *reinterpret_cast<const uint2*>(
                    a_s + k * BM + (dtl_lds_unit<BM>(m >> 4, k) << 4) + (m & 15));
                bs[0] += __uint_as_float(v.x << 16);
                bs[1] += __uint_as_float(v.x & 0xffff0000u);
                bs[2] += __uint_as_float(v.y << 16);
                bs[3] += __uint_as_float(v.y & 0xffff0000u);
            }
        }
    };
    auto read_frags = [&](const T* a_s, const T* b_s, FragSet& f) {
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
#pragma unroll
            for (int t = 0; t < TN; t++) dtl_frag_ld<BN, BKM>(f.fb[ks][t], b_s, fB.ofs[t][ks]);
#pragma unroll
            for (int t = 0; t < TM; t++) dtl_frag_ld<BM, AK>(f.fa[ks][t], a_s, fA.ofs[t][ks]);
        }
        bias_sum(a_s);
    };
    auto mfmas = [&](const FragSet& f) {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) mma(acc[i][j], f.fb[ks][j], f.fa[ks][i]);
    };
    auto compute = [&](const T* a_s, const T* b_s) {
        FragSet f;
        read_frags(a_s, b_s, f);
        mfmas(f);
    };
    // stage kt lives in buffer kt % NS.  Opening stage kt: wait for its loads
    // (allowing the NS-2 later stages already issued to stay in flight; near
    // the end, where fewer were issued, wait for all), barrier, then issue the
    // loads of stage kt + NS - 1 into the buffer stage kt - 1 just released.
    // The barrier is a bare s_barrier: __syncthreads()'s workgroup fence would
    // also wait for the later stages' loads still in flight.  Each wave's vmcnt
    // wait covers its own loads into stage kt, and the fragments of stage kt-1
    // (the buffer about to be refilled) are consumed by MFMAs before it; the
    // memory clobber keeps the compiler from moving LDS accesses across it.
    // pend: the previous tile's epilogue stores (XS) were issued after the
    // loads of this tile's first NS - 1 stages, so those stages' waits allow
    // them to stay outstanding (vector memory operations complete in order)
    bool pend = false;
    // (LGK: 0xffff leaves the LDS counter alone, 0xc0ff also waits for this
    // wave's LDS reads)
    auto wait_stage = [&](int kt, auto lgk) {
        constexpr int LGK = decltype(lgk)::value;
        constexpr int base = (NS - 2) * NQS;
        constexpr int with = base + XS_STORES > 63 ? 63 : base + XS_STORES;
        if (kt + NS - 2 >= kt1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & LGK);
        else if (XS_STORES > 0 && pend && kt - kt0 <= NS - 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(with) & LGK);
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(base) & LGK);
    };
    auto open = [&](int kt) {
        wait_stage(kt, std::integral_constant<int, 0xffff>());
        asm volatile("s_barrier" ::: "memory");
    };
    // RP: wait until stage kt has landed (the stages issued after it may stay
    // in flight), with this wave's fragment reads of the stage before
    // complete, then barrier
    auto open_rp = [&](int kt) {
        wait_stage(kt, std::integral_constant<int, 0xc0ff>());
        asm volatile("s_barrier" ::: "memory");
    };
    auto bufA = [&](int b) { return b == 0 ? sA0 : b == 1 ? sA1 : b == 2 ? sA2 : sA3; };
    auto bufB = [&](int b) { return b == 0 ? sB0 : b == 1 ? sB1 : b == 2 ? sB2 : sB3; };
#define GEMM_DTL_STAGE(I)                                                                          \
    {                                                                                              \
        const int kt = kb + (I);                                                                   \
        if (kt < kt1) {                                                                            \
            open(kt);                                                                              \
            if (kt + NS - 1 < kt1) issue(kt + NS - 1, sA##I##p, sB##I##p);                         \
            compute(sA##I, sB##I);                                                                 \
        }                                                                                          \
    }
    // buffers for "the stage NS - 1 ahead" of stage i: (i + NS - 1) % NS
    T* const sA0p = NS == 2 ? sA1 : NS == 3 ? sA2 : sA3;
    T* const sB0p = NS == 2 ? sB1 : NS == 3 ? sB2 : sB3;
    T* const sA1p = NS == 2 ? sA0 : NS == 3 ? sA0 : sA0;
    T* const sB1p = NS == 2 ? sB0 : NS == 3 ? sB0 : sB0;
    T* const sA2p = NS == 3 ? sA1 : sA1;
    T* const sB2p = NS == 3 ? sB1 : sB1;
    T* const sA3p = sA2;
    T* const sB3p = sB2;
    // the first NS - 1 stages of the tile at (mm0, nn0)
    auto prologue = [&](int mm0, int nn0) {
#pragma unroll
        for (int i = 0; i < NS - 1; i++) {
            const int kt = kt0 + i;
            if (kt < kt1) {
                T* ad = i == 0 ? sA0 : i == 1 ? sA1 : sA2;
                T* bd = i == 0 ? sB0 : i == 1 ? sB1 : sB2;
                issue_at(kt, ad, bd, mm0, nn0);
            }
        }
    };
    // ACC_BIAS: the tile's bias columns go to LDS with the first stage's
    // loads (one 1 KB load, ahead of them, so the wait for that stage covers
    // it) and are added to the accumulators after the last stage, so the
    // epilogue reads nothing from global memory
    auto bias_issue = [&](int nn0) {
        if constexpr (ACC_BIAS) {
            if (wave == 0) {
                const __amdgpu_buffer_rsrc_t rs =
                    uniform_rsrc((const T*)g.bias + nn0, rsrc_range(((long)g.N - nn0) * 2));
                lds_dma16(rs, (uint32_t)lane * 16, sBiasRow);
            }
        }
    };
    auto add_bias = [&]() {
        if constexpr (ACC_BIAS) {
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const uint2 u2 = ld8(sBiasRow + wn * TL::WTN + 4 * g4 + 16 * j);
                const f32x4_t b0 = {__uint_as_float(u2.x << 16), __uint_as_float(u2.x & 0xffff0000u),
                                    __uint_as_float(u2.y << 16), __uint_as_float(u2.y & 0xffff0000u)};
#pragma unroll
                for (int i = 0; i < TM; i++) acc[i][j] += b0;
            }
        }
    };
    bias_issue(n0);
    prologue(m0, n0);
    while (true) {
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (ACC_BIAS && kt0 >= kt1) {  // no stage waited for the bias load (empty contraction)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            asm volatile("s_barrier" ::: "memory");
        }
        if constexpr (RP) {
            // Fragments one stage ahead in registers: the reads of stage kt + 1
            // are issued before the MFMAs of stage kt, so their LDS latency is
            // covered by that stage's matrix work.  Stage kt's buffer is free
            // once every wave holds its fragments (lgkmcnt(0) before the
            // barrier), so the loads of stage kt + NS go into it right away.
            FragSet f0, f1;
            open_rp(kt0);
            if (kt0 + NS - 1 < kt1) issue(kt0 + NS - 1, bufA(NS - 1), bufB(NS - 1));
            if (kt0 < kt1) read_frags(sA0, sB0, f0);
            constexpr int U = NS == 3 ? 6 : NS;  // stages per unrolled pass (even, a multiple of NS)
            for (int kb = kt0; kb < kt1; kb += U) {
#pragma unroll
                for (int i = 0; i < U; i++) {
                    const int kt = kb + i;
                    if (kt < kt1) {
                        FragSet& fc = (i & 1) ? f1 : f0;
                        FragSet& fn = (i & 1) ? f0 : f1;
                        if (kt + 1 < kt1) {
                            open_rp(kt + 1);
                            if (kt + NS < kt1) issue(kt + NS, bufA(i % NS), bufB(i % NS));
                            read_frags(bufA((i + 1) % NS), bufB((i + 1) % NS), fn);
                        }
                        mfmas(fc);
                    }
                }
            }
        } else {
            for (int kb = kt0; kb < kt1; kb += NS) {
                GEMM_DTL_STAGE(0)
                GEMM_DTL_STAGE(1)
                if constexpr (NS > 2) GEMM_DTL_STAGE(2)
                if constexpr (NS > 3) GEMM_DTL_STAGE(3)
            }
        }
        if constexpr (SK == 2) {
            // the two slices swap their partial sums one accumulator row at a
            // time (each slice's row in a slab of its own) and both add: fp32
            // addition commutes, so both hold the same sum; slice 1 then ends
            float* const mine = reinterpret_cast<float*>(kslice == 0 ? sB0 : sB1);
            const float* const other = reinterpret_cast<const float*>(kslice == 0 ? sB1 : sB0);
            static_assert((NT / 2) * TN * 16 <= BN * BK * 2, "a slice's accumulator row fits one B slab");
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the last fragment reads are done
            asm volatile("s_barrier" ::: "memory");
#pragma unroll
            for (int i = 0; i < TM; i++) {
#pragma unroll
                for (int j = 0; j < TN; j++)
                    *reinterpret_cast<f32x4_t*>(mine + ((wsub * TN + j) * 64 + lane) * 4) = acc[i][j];
                __builtin_amdgcn_s_waitcnt(0xc07f);
                asm volatile("s_barrier" ::: "memory");
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = acc[i][j] + *reinterpret_cast<const f32x4_t*>(other + ((wsub * TN + j) * 64 + lane) * 4);
                __builtin_amdgcn_s_waitcnt(0xc07f);
                asm volatile("s_barrier" ::: "memory");
            }
            if (kslice != 0) return;
        }
        // the bias (its load landed before the first stage's), added after the
        // sum as the epilogue would: the same rounding
        add_bias();
        // next tile: once every wave is done with the stage buffers (the last
        // stages were waited for with vmcnt(0), so no load into them is in
        // flight), request its first stages, then store this one.  The next
        // tile's first stage waits for everything older than its later stages,
        // these stores included.
        const int un = u + (int)gridDim.x;
        const bool more = PERSIST && un < ntiles;
        int tm1 = 0, tn1 = 0;
        if (more) {
            tile_of(un, tm1, tn1);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's fragment reads are done
            asm volatile("s_barrier" ::: "memory");
            bias_issue(tn1 * BN);
            prologue(tm1 * BM, tn1 * BN);
        }
        if constexpr (BIAS) {
            float* red = sbias;  // KG x BM floats
#pragma unroll
            for (int e = 0; e < 4; e++) red[bkg * BM + 4 * bq + e] = bs[e];
            __syncthreads();
            if (do_bias && tid < BM) {
                float t = 0.f;
                for (int q = 0; q < KG; q++) t += red[q * BM + tid];
                const int m = m0 + tid;
                if (m < g.M) {
                    if constexpr (EPI == EPI_SPLIT) g.wsb[(size_t)blockIdx.y * g.M + m] = g.alpha * t;
                    else g.dbias[m] += g.alpha * t;
                }
            }
        }
        // the staging buffer: every wave must be done reading it first
        T* const lastA = NS == 2 ? sA1 : NS == 3 ? sA2 : sA3;
        T* const lastB = NS == 2 ? sB1 : NS == 3 ? sB2 : sB3;
        T* const stage = STAGE_TWO ? (wave < NW / 2 ? lastA : lastB) + (wave % (NW / 2)) * 16 * (TL::WTN + 8)
                                   : (BN >= BM ? lastB : lastA) + wave * 16 * (TL::WTN + 8);
        if (CAN_STAGE && !more && SK == 1) {
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            asm volatile("s_barrier" ::: "memory");
        }
        gemm_epilogue<T, TL, EPI, OutT, CAN_STAGE, XS>(g, acc, m0, n0, wm, wn, l16, g4, stage);
        if (!more) break;
        pend = true;
        u = un;
        m0 = tm1 * BM;
        n0 = tn1 * BN;
    }
#undef GEMM_DTL_STAGE
}

// v = sum_z ws[z*MN + i], z in increasing order (float4 groups of a row-major
// M x N output, N % 4 == 0), then the product's epilogue on v, in the order the
// tile epilogue applies it (alpha is already in the partials):
//   GEMM_ACCUM  C (fp32) += v          GEMM_STORE  C = v
//   GEMM_BIAS   C = v + bias[n]        GEMM_BIAS_RESID  C = v + bias[n] + aux_in
//   GEMM_BIAS_GELU  aux_out = v + bias[n]; C = gelu(aux_out as stored)
//   GEMM_GELU_BWD   C = v * gelu'(aux_in)
// aux_in / aux_out have the output's row pitch N.  Blocks past the first
// cblocks (when db is given) do the bias-gradient partials:
// db[m] += sum_z wsb[z*M + m], z in increasing order.
template <typename OutT, int EPI>
__global__ void splitk_reduce_kernel(OutT* __restrict__ C, const float* __restrict__ ws, size_t MN, int splits,
                                     int cblocks, float* __restrict__ db, const float* __restrict__ wsb, int M, int N,
                                     const OutT* __restrict__ bias, const OutT* __restrict__ aux_in,
                                     OutT* __restrict__ aux_out) {
    if ((int)blockIdx.x >= cblocks) {
        const int m = ((int)blockIdx.x - cblocks) * blockDim.x + threadIdx.x;
        if (m >= M) return;
        float t = 0.f;
        for (int z = 0; z < splits; z++) t += wsb[(size_t)z * M + m];
        db[m] += t;
        return;
    }
    size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= MN) return;
    float s[4];
    load4<float>(ws + i, s);
    for (int z = 1; z < splits; z++) {
        float w[4];
        load4<float>(ws + (size_t)z * MN + i, w);
#pragma unroll
        for (int r = 0; r < 4; r++) s[r] += w[r];
    }
    if constexpr (EPI == GEMM_ACCUM) {
        float c[4];
        load4<float>((const float*)C + i, c);
#pragma unroll
        for (int r = 0; r < 4; r++) s[r] += c[r];
    }
    const int n = (int)(i % (size_t)N);
    if constexpr (EPI == GEMM_BIAS || EPI == GEMM_BIAS_GELU || EPI == GEMM_BIAS_RESID) {
        float bb[4];
        load4<OutT>(bias + n, bb);
#pragma unroll
        for (int r = 0; r < 4; r++) s[r] += bb[r];
    }
    if constexpr (EPI == GEMM_BIAS_GELU) {
        store4<OutT>(aux_out + i, s);
#pragma unroll
        for (int r = 0; r < 4; r++) s[r] = gelu_f<OutT>(to_f<OutT>(from_f<OutT>(s[r])));
    }
    if constexpr (EPI == GEMM_BIAS_RESID || EPI == GEMM_GELU_BWD) {
        float a[4];
        load4<OutT>(aux_in + i, a);
#pragma unroll
        for (int r = 0; r < 4; r++) s[r] = EPI == GEMM_BIAS_RESID ? s[r] + a[r] : s[r] * gelu_grad_f<OutT>(a[r]);
    }
    store4<OutT>(C + i, s);
}

// ---------------------------------------------------------------- dispatch --
struct Choice {
    int bm, bn, wt, splits, occ, num_cus;
};

// Tile configurations per element type, with their measured relative per-CU
// throughput per operand layout (MI355X, bf16, direct-to-LDS kernel, time per
// round of resident workgroups on the 8192 x 50304 x 768 classifier products,
// so wave quantisation is left to the cost model; 1.00 = the best tile of that
// layout; the 128x128 input-gradient figure is from the 8192 x 768 x 3072
// products, where the classifier's is confounded by its K split; the smaller
// weight-gradient tiles are set from the whole training step, where the
// 128-row-wave tile with its K split is ~20% faster on those products than
// 128x256 or 128x128 with theirs; so are the forward figure of 256x128 and the
// input-gradient figure of 128x256: inside the step the layer products read
// operands that are no longer in cache, and these tiles, one workgroup per CU
// with two stages in flight, run them 5-15% faster than 128x128).  Forward:
// 256x256 3.3 TFLOP/s per CU; weight gradient: 256x256
// with 128-row waves 3.9 TFLOP/s per CU.  The 128-row-wave tile's
// input-gradient figure is set from the step as well: on the classifier's
// input gradient (K = Vp, split) it beats the 16-wave 256x256 tile, whose
// epilogue cannot stage its stores through LDS.  The 256x192 tile (8 waves of
// 64x96, two stages) is set from the qkv and fc forward products (8192 x 2304
// and 8192 x 3072, K = 768, with their bias and GELU epilogues), where it runs
// 11-14% faster than 128x192 and 256x128 (1.5 and 2 rounds of tiles against 3);
// on the classifier (N = 50304, the weights streaming from HBM rather than
// staying in L2) it is 5% slower than 256x256, so it is offered only up to
// N = 8192 (max_n).  On the input-gradient layout (B k-strided, a rotation
// swizzle for its 12-unit slab) it takes the fcproj input gradient with the
// GELU backward (8192 x 3072, K = 768) in 2 rounds instead of 3 of 128x256,
// 6.5% faster; on the classifier input gradient (2 K splits of 25k instead of
// 8 of 256x256) it was 1.6% slower in the step, so it takes no K split
// (max_split).  The 256x288 tile (8 waves of 64x144, two stages; the
// most MFMA work per fragment read of the tiles here) covers the 124M qkv
// forward product (8192 x 2304) in exactly one round of 256 tiles, 19%
// faster than 1.5 rounds of 256x192, and the 1558M fc forward (8192 x 6400,
// 2.9 rounds) 10-15% faster than 256x192.  Where it leaves CUs idle (the
// 1558M attproj, 192 tiles) it was 4% slower than 224 tiles of 256x256, so
// it is offered only when its tiles fill every CU at least once (fill).
// The depth-sliced 128x192 tile (8 waves: two per 64x96 output tile, one per
// 32-deep half of each stage, partial sums swapped through LDS at the end)
// keeps the 256 tiles of the N = 768 products with two waves per SIMD
// instead of one: fc and qkv input gradients 11-17% faster than 128x256,
// fcproj forward 9-12% faster than the 4-wave 128x192.  With K = 768 the
// final exchange is not paid back (attproj forward 4% slower), so it is
// offered from K = 1536 (min_k), and without K splits.
struct TileCfg {
    int bm, bn, wt, occ;
    double speed[3];  // forward, input gradient, weight gradient
    int max_n;        // largest N the tile is offered for (0: any)
    bool fill;        // offered only with at least one tile per CU
    int max_split;    // most K splits the tile is offered with (0: any)
    int min_k;        // shortest contraction the tile is offered for (0: any)
};
const TileCfg kCfgBf16[] = {{256, 256, 64, 1, {0.99, 1.00, 0.75}, 0},
                            {256, 128, 64, 1, {0.92, 0.76, 0.66}, 0},
                            {128, 256, 64, 1, {0.71, 0.92, 0.70}, 0},
                            {128, 128, 64, 2, {0.81, 0.82, 0.70}, 0},
                            {256, 256, 128, 1, {1.00, 1.01, 1.00}, 0},
                            // forward products only (128x192: equal to
                            // 128x256 on the input gradients; 256x288: a
                            // k-strided slab needs a multiple of 64 rows)
                            {128, 192, 96, 1, {0.92, 0.0, 0.0}, 0},
                            {256, 192, 96, 1, {1.42, 0.98, 0.0}, 8192, false, 1},
                            {256, 288, 144, 1, {1.32, 0.0, 0.0}, 8192, true},
                            {128, 192, 97, 1, {1.045, 0.80, 0.0}, 8192, false, 1, 1536},
};
constexpr int kNumCfgBf16 = sizeof(kCfgBf16) / sizeof(kCfgBf16[0]);
const TileCfg kCfgF32[] = {{128, 128, 64, 2, {1.0, 1.0, 1.0}, 0}};

// Pick the tile and the K split minimising a simple cost: waves of
// workgroups over the CUs times the work per workgroup, plus the split
// partials' extra HBM traffic.  Split-K where the caller allows it
// (split_ok) for plain-store and accumulate epilogues, and in fp32 for the
// bias / GELU / residual / GELU-backward epilogues too (every epilogue moves
// into the reduction).
Choice choose(const GemmDesc& d, int elem_bytes, int num_cus) {
    const bool bf16 = elem_bytes == 2;
    const TileCfg* cfgs = bf16 ? kCfgBf16 : kCfgF32;
    const int ncfg = bf16 ? kNumCfgBf16 : 1;
    const int bk = 128 / elem_bytes;
    const int ktiles = (d.K + bk - 1) / bk;
    // fp32 products also split with a bias, GELU, residual or GELU-backward
    // epilogue (it moves into the reduction): their tiles are 4x as costly
    // per element, so a small row count leaves most CUs idle otherwise
    const bool epi_ok = d.epi == GEMM_ACCUM || d.epi == GEMM_STORE ||
                        (!bf16 && (d.epi == GEMM_BIAS || d.epi == GEMM_BIAS_GELU || d.epi == GEMM_BIAS_RESID ||
                                   d.epi == GEMM_GELU_BWD) &&
                         d.ldaux == d.N);
    const bool can_split = d.split_ok && epi_ok && (d.N % 4 == 0) && d.ldc == d.N;
    const int lay = d.a_kmajor && d.b_kmajor ? 0 : (d.a_kmajor ? 1 : 2);
    const double flop_rate = 2.5e15 / 256.0;  // per CU, dense bf16
    const double hbm = 5.0e12;                // bytes/s usable
    Choice best = {cfgs[0].bm, cfgs[0].bn, cfgs[0].wt, 1, cfgs[0].occ, num_cus};
    double best_cost = 1e300;
    for (int c = 0; c < ncfg; c++) {
        const TileCfg& t = cfgs[c];
        if (t.max_n > 0 && d.N > t.max_n) continue;
        if (t.min_k > 0 && d.K < t.min_k) continue;
        const long tiles = (long)((d.M + t.bm - 1) / t.bm) * ((d.N + t.bn - 1) / t.bn);
        if (t.fill && tiles < num_cus) continue;
        int max_split = can_split ? std::min(32, std::max(1, ktiles / 4)) : 1;
        if (t.max_split > 0) max_split = std::min(max_split, t.max_split);
        for (int s = 1; s <= max_split; s++) {
            const int kps = (ktiles + s - 1) / s;
            const int sp = (ktiles + kps - 1) / kps;
            if (sp != s) continue;
            const long units = tiles * sp;
            const long slots = (long)num_cus * t.occ;
            // waves of workgroups; with two per CU the last partial wave
            // overlaps the previous one, so it is counted in half steps
            double rounds = t.occ == 1 ? (double)((units + slots - 1) / slots)
                                       : std::max(1.0, std::ceil(2.0 * units / slots) / 2.0);
            const double speed = t.speed[lay];
            double cost = rounds * (2.0 * t.bm * t.bn * (double)kps * bk) / (flop_rate * speed / t.occ);
            if (sp > 1) cost += (double)(sp + 1) * d.M * d.N * 4.0 / hbm;
            if (cost < best_cost * 0.999) {
                best_cost = cost;
                best = {t.bm, t.bn, t.wt, sp, t.occ, num_cus};
            }
        }
    }
    return best;
}

template <typename T, int BM, int BN, int WT, bool AK, bool BKM, int EPI, typename OutT, bool BIAS = false>
void launch_t(const Args& a, dim3 grid, int slots, hipStream_t s) {
    using TL = TileOf<T, BM, BN, WT>;
    if constexpr (sizeof(T) == 2) {
        if (dtl_persistent<BM, BN, WT, EPI, BIAS>() && grid.y == 1) grid.x = std::min((int)grid.x, slots);
        hipLaunchKernelGGL((gemm_dtl_kernel<BM, BN, WT, AK, BKM, EPI, OutT, BIAS>), grid, dim3(TL::NT), 0, s, a);
    } else
        hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WT, AK, BKM, EPI, OutT, BIAS>), grid, dim3(TL::NT), 0, s, a);
}

// Instantiated (layout, epilogue) pairs: forward products (A and B
// k-contiguous), input-gradient products (A k-contiguous, B k-strided) and
// weight-gradient products (both k-strided).
template <typename T, int BM, int BN, int WT>
int launch_epi(const GemmDesc& d, const Args& a, dim3 grid, int slots, int epi, hipStream_t s) {
    const int lay = (d.a_kmajor ? 2 : 0) | (d.b_kmajor ? 1 : 0);
    // k-strided slabs (input- and weight-gradient layouts) need a multiple of
    // four 16-row units (the swizzle's bank spread)
    constexpr bool KSTRIDED = BM % 64 == 0 && BN % 64 == 0;
    if (lay != 3 && !KSTRIDED) return (int)hipErrorInvalidValue;
    if (lay == 3) {
        switch (epi) {
            case GEMM_STORE: launch_t<T, BM, BN, WT, true, true, GEMM_STORE, T>(a, grid, slots, s); return 0;
            case GEMM_BIAS: launch_t<T, BM, BN, WT, true, true, GEMM_BIAS, T>(a, grid, slots, s); return 0;
            case GEMM_BIAS_GELU: launch_t<T, BM, BN, WT, true, true, GEMM_BIAS_GELU, T>(a, grid, slots, s); return 0;
            case GEMM_BIAS_RESID: launch_t<T, BM, BN, WT, true, true, GEMM_BIAS_RESID, T>(a, grid, slots, s); return 0;
            case GEMM_BIAS_GELU_SMX:
                if constexpr (sizeof(T) == 4) {
                    launch_t<T, BM, BN, WT, true, true, GEMM_BIAS_GELU_SMX, T>(a, grid, slots, s);
                    return 0;
                }
                break;
            case EPI_SPLIT:  // fp32 forward products split over K (bf16 ones never do)
                if constexpr (sizeof(T) == 4) {
                    launch_t<T, BM, BN, WT, true, true, EPI_SPLIT, float>(a, grid, slots, s);
                    return 0;
                }
                break;
        }
    } else if constexpr (!KSTRIDED) {
        return (int)hipErrorInvalidValue;
    } else if (lay == 2) {
        switch (epi) {
            case GEMM_STORE: launch_t<T, BM, BN, WT, true, false, GEMM_STORE, T>(a, grid, slots, s); return 0;
            case GEMM_GELU_BWD: launch_t<T, BM, BN, WT, true, false, GEMM_GELU_BWD, T>(a, grid, slots, s); return 0;
            case EPI_SPLIT: launch_t<T, BM, BN, WT, true, false, EPI_SPLIT, float>(a, grid, slots, s); return 0;
        }
    } else if constexpr (TileOf<T, BM, BN, WT>::SK > 1) {
        return (int)hipErrorInvalidValue;  // depth-sliced tiles: forward and input-gradient layouts
    } else if (lay == 0) {
        const bool bias = a.dbias != nullptr;
        switch (epi) {
            case GEMM_ACCUM:
                if (bias) launch_t<T, BM, BN, WT, false, false, GEMM_ACCUM, float, true>(a, grid, slots, s);
                else launch_t<T, BM, BN, WT, false, false, GEMM_ACCUM, float, false>(a, grid, slots, s);
                return 0;
            case EPI_SPLIT:
                if (bias) launch_t<T, BM, BN, WT, false, false, EPI_SPLIT, float, true>(a, grid, slots, s);
                else launch_t<T, BM, BN, WT, false, false, EPI_SPLIT, float, false>(a, grid, slots, s);
                return 0;
        }
    }
    return (int)hipErrorInvalidValue;
}

template <typename T>
int launch_tile(const GemmDesc& d, const Args& a, const Choice& ch, dim3 grid, int epi, hipStream_t s) {
    // resident workgroup slots, a multiple of 8 (one XCD cycle)
    const int slots = std::max(8, (ch.num_cus * ch.occ) / 8 * 8);
    if constexpr (sizeof(T) == 2) {
        if (ch.wt == 128) {
            if (ch.bm == 256 && ch.bn == 256) return launch_epi<T, 256, 256, 128>(d, a, grid, slots, epi, s);
            return (int)hipErrorInvalidValue;
        }
        if (ch.wt == 96 && ch.bm == 128 && ch.bn == 192) return launch_epi<T, 128, 192, 96>(d, a, grid, slots, epi, s);
        if (ch.wt == 96 && ch.bm == 256 && ch.bn == 192) return launch_epi<T, 256, 192, 96>(d, a, grid, slots, epi, s);
        if (ch.wt == 144 && ch.bm == 256 && ch.bn == 288) return launch_epi<T, 256, 288, 144>(d, a, grid, slots, epi, s);
        if (ch.wt == 97 && ch.bm == 128 && ch.bn == 192) return launch_epi<T, 128, 192, 97>(d, a, grid, slots, epi, s);
        if (ch.bm == 256 && ch.bn == 256) return launch_epi<T, 256, 256, 64>(d, a, grid, slots, epi, s);
        if (ch.bm == 256 && ch.bn == 128) return launch_epi<T, 256, 128, 64>(d, a, grid, slots, epi, s);
        if (ch.bm == 128 && ch.bn == 256) return launch_epi<T, 128, 256, 64>(d, a, grid, slots, epi, s);
    }
    if (ch.bm == 128 && ch.bn == 128) return launch_epi<T, 128, 128, 64>(d, a, grid, slots, epi, s);
    return (int)hipErrorInvalidValue;
}

template <typename T>
int gemm_launch_t(const GemmDesc& d, float* ws, size_t ws_bytes, int num_cus, hipStream_t s) {
    constexpr int BK = 128 / (int)sizeof(T);
    const Choice ch = choose(d, (int)sizeof(T), num_cus);
    const int tiles = ((d.M + ch.bm - 1) / ch.bm) * ((d.N + ch.bn - 1) / ch.bn);
    const int ktiles = (d.K + BK - 1) / BK;
    Args a;
    a.A = d.A; a.lda = d.lda; a.B = d.B; a.ldb = d.ldb; a.C = d.C; a.ldc = d.ldc;
    a.bias = d.bias; a.aux_in = d.aux_in; a.aux_out = d.aux_out; a.ldaux = d.ldaux;
    a.ws = ws; a.M = d.M; a.N = d.N; a.K = d.K; a.alpha = d.alpha;
    a.dbias = d.epi == GEMM_ACCUM ? d.dbias : nullptr;
    a.wsb = nullptr;
    if (tiles == 0) return 0;
    // the bias is added to the unscaled sum (bf16 tiles start their
    // accumulators at it), so products with a bias take alpha = 1
    if ((d.epi == GEMM_BIAS || d.epi == GEMM_BIAS_GELU || d.epi == GEMM_BIAS_RESID || d.epi == GEMM_BIAS_GELU_SMX) &&
        d.alpha != 1.0f)
        return (int)hipErrorInvalidValue;
    if (ch.splits > 1) {
        const size_t MN = (size_t)d.M * d.N;
        const size_t need = (size_t)ch.splits * (MN + d.M) * sizeof(float);
        if (ws == nullptr || ws_bytes < need || d.ldc != d.N) return (int)hipErrorInvalidValue;
        a.kps = (ktiles + ch.splits - 1) / ch.splits;
        if (a.dbias) a.wsb = ws + (size_t)ch.splits * MN;
        int e = launch_tile<T>(d, a, ch, dim3(tiles, ch.splits), EPI_SPLIT, s);
        if (e) return e;
        const int cblocks = (int)((MN / 4 + 255) / 256);
        const int bblocks = a.dbias ? (d.M + 255) / 256 : 0;
        const T* bias = (const T*)d.bias;
        const T* aux_in = (const T*)d.aux_in;
        T* aux_out = (T*)d.aux_out;
        switch (d.epi) {
            case GEMM_ACCUM:
                hipLaunchKernelGGL((splitk_reduce_kernel<float, GEMM_ACCUM>), dim3(cblocks + bblocks), dim3(256), 0, s,
                                   (float*)d.C, ws, MN, ch.splits, cblocks, d.dbias, a.wsb, d.M, d.N, nullptr, nullptr,
                                   nullptr);
                break;
#define GEMM_SPLIT_REDUCE(E)                                                                                      \
    case E:                                                                                                       \
        hipLaunchKernelGGL((splitk_reduce_kernel<T, E>), dim3(cblocks), dim3(256), 0, s, (T*)d.C, ws, MN, ch.splits, \
                           cblocks, (float*)nullptr, (const float*)nullptr, d.M, d.N, bias, aux_in, aux_out);       \
        break;
            GEMM_SPLIT_REDUCE(GEMM_STORE)
            GEMM_SPLIT_REDUCE(GEMM_BIAS)
            GEMM_SPLIT_REDUCE(GEMM_BIAS_GELU)
            GEMM_SPLIT_REDUCE(GEMM_BIAS_RESID)
            GEMM_SPLIT_REDUCE(GEMM_GELU_BWD)
#undef GEMM_SPLIT_REDUCE
            default:
                return (int)hipErrorInvalidValue;
        }
        return (int)hipGetLastError();
    }
    a.kps = ktiles;
    int e = launch_tile<T>(d, a, ch, dim3(tiles, 1), d.epi, s);
    if (e) return e;
    return (int)hipGetLastError();
}

}  // namespace

namespace {
template <int BM, int BN, int WT>
int dw_group_t(const GemmGroupItem* items, int n, hipStream_t s) {
    if (n < 1 || n > kMaxGroup || !items) return (int)hipErrorInvalidValue;
    GroupArgs ga = {};
    long total = 0;
    for (int i = 0; i < n; i++) {
        const GemmGroupItem& it = items[i];
        if (it.M < 0 || it.N < 0 || it.K < 0 || it.count < 0) return (int)hipErrorInvalidValue;
        ga.A[i] = it.A; ga.B[i] = it.B; ga.C[i] = it.C; ga.dbias[i] = it.dbias;
        ga.lda[i] = it.lda; ga.ldb[i] = it.ldb; ga.ldc[i] = it.ldc;
        ga.sA[i] = it.sA; ga.sB[i] = it.sB; ga.sC[i] = it.sC; ga.sBias[i] = it.sBias;
        ga.M[i] = it.M; ga.N[i] = it.N; ga.K[i] = it.K; ga.alpha[i] = it.alpha;
        ga.tiles_m[i] = (it.M + BM - 1) / BM;
        ga.tiles_n[i] = (it.N + BN - 1) / BN;
        ga.begin[i] = (int)total;
        total += (long)ga.tiles_m[i] * ga.tiles_n[i] * it.count;
        if (total > (1L << 30)) return (int)hipErrorInvalidValue;
    }
    for (int i = n; i <= kMaxGroup; i++) ga.begin[i] = (int)total;
    for (int i = n; i < kMaxGroup; i++) ga.tiles_m[i] = ga.tiles_n[i] = 1;
    ga.np = n;
    ga.total = (int)total;
    if (total == 0) return 0;
    using TL = TileOf<bf16_t, BM, BN, WT>;
    hipLaunchKernelGGL((gemm_dtl_kernel<BM, BN, WT, false, false, GEMM_ACCUM, float, true, true>), dim3((unsigned)total),
                       dim3(TL::NT), 0, s, ga);
    return (int)hipGetLastError();
}
}  // namespace

int gemm_dw_group_launch(const GemmGroupItem* items, int n, hipStream_t s, int tile) {
    if (tile == 0) return dw_group_t<256, 256, 128>(items, n, s);
    if (tile == 1) return dw_group_t<128, 256, 64>(items, n, s);
    return (int)hipErrorInvalidValue;
}

long gemm_dw_group_tiles(const GemmGroupItem* items, int n, int tile) {
    const int bm = tile == 0 ? 256 : 128, bn = 256;
    long t = 0;
    for (int i = 0; i < n; i++)
        t += (long)((items[i].M + bm - 1) / bm) * ((items[i].N + bn - 1) / bn) * items[i].count;
    return t;
}

size_t gemm_workspace_bytes(const GemmDesc& d, int elem_bytes, int num_cus) {
    const Choice ch = choose(d, elem_bytes, num_cus);
    return ch.splits > 1 ? (size_t)ch.splits * ((size_t)d.M * d.N + d.M) * sizeof(float) : 0;
}

int gemm_launch(const GemmDesc& d, int elem_bytes, float* ws, size_t ws_bytes, int num_cus, hipStream_t s) {
    if (elem_bytes == 2) return gemm_launch_t<bf16_t>(d, ws, ws_bytes, num_cus, s);
    if (elem_bytes == 4) return gemm_launch_t<float>(d, ws, ws_bytes, num_cus, s);
    return (int)hipErrorInvalidValue;
}
