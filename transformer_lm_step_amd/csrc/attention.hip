// attention.hip - causal multi-head attention, forward and backward (gfx950).
//
// What is computed is train_gpt2.cu's attention_forward / attention_backward
// (permute_kernel, the two batched products, softmax_forward_kernel5,
// softmax_autoregressive_backward_kernel, unpermute_kernel): per (b, h),
//   S = Q K^T / sqrt(HS), P = softmax over the causal prefix s <= t, O = P V,
//   dP = dO V^T, dV = P^T dO, dS = P * (dP - rowsum(P * dP)) / sqrt(HS),
//   dQ = dS K, dK = dS^T Q.
// Q, K, V are read in place from the qkv activation (B, T, 3, NH, HS) and O is
// written as (B, T, NH, HS), so the page's permute / unpermute copies vanish.
//
// The T x T matrices are never stored.  The forward keeps, per query row, the
// running maximum and sum of an online softmax (base 2: scores are scaled by
// log2(e)/sqrt(HS)) and stores lse2 = max + log2(sum); the backward rebuilds
// P = exp2(S * log2(e)/sqrt(HS) - lse2) tile by tile.  rowsum(P * dP) equals
// rowsum(dO * O) (delta): computed up front by its own pass, or (bf16, head
// size 64) by the dQ kernel, which then runs first.  The backward runs as two kernels
// so that every output element is produced by exactly one workgroup with a
// fixed summation order (no atomics): one per 64-key block accumulating dK and
// dV over the query blocks at or after it, one per 64-query block accumulating
// dQ over the key blocks at or before it.
//
// Tiling: a workgroup is 4 wave64s and owns a 64-row block (queries in the
// forward and dQ kernels, keys in the dK/dV kernel); each wave owns 16 of those
// rows, held as MFMA fragments in registers for the whole kernel.  The other
// side (64 keys or 64 queries per step) is staged in LDS, as row x d (for the
// S / dP products) and as d x row (for the P V, dS K, P^T dO, dS^T Q
// products).  Score tiles are computed transposed where needed so that the
// lane owning a row's statistics also owns that row in the next product, and
// a 16x16 score tile pair is fed straight back as the next MFMA's operand
// (slot j of lane group g <-> row 32c + 16*(j/4) + 4g + j%4, the same map on
// both operands).  Workgroups are issued longest-first along the causal
// triangle, with every row block of a (batch, head) pair on the same XCD
// (attn_block).
#include <math.h>

#include <type_traits>

#include "device.h"
#include "kernels.h"


namespace {

constexpr float LOG2E = 1.4426950408889634f;
// stage buffers of the streamed key/value (or query/output-gradient) blocks
constexpr int ATTN_FWD_NS = 2, ATTN_BWD_NS = 2;
// waves (16 query rows each) per forward workgroup: 128 rows per workgroup
// halve the K/V traffic of 64 (28.7 against 29.5 us per 124M layer)
constexpr int ATTN_FWD_WAVES = 8;
typedef short v4s_t __attribute__((ext_vector_type(4)));

// Row block `blk` (0 = the one with the most work) and (batch, head) of this
// workgroup; the grid is one-dimensional, nb row blocks x B*NH pairs.  The
// workgroup id runs over the pairs fastest, so all longest blocks are issued
// first (the causal triangle's work per block ranges from 1 to nb tiles).
// Consecutive ids go to the eight XCDs in turn, so when B*NH is a multiple of 8
// every block of a pair runs on one XCD and the pair's K/V (forward, dQ) or
// Q/dO (dK/dV) is fetched into that XCD's L2 once.  Issuing the blocks
// row-fastest instead spreads a pair over all XCDs and gives XCD x only the
// blocks x and x + 8 - up to 2.4 times another XCD's work.
DEV void attn_block(int nb, int NH, int& blk, int& h, int& b) {
    const int nhb = gridDim.x / nb;
    blk = blockIdx.x / nhb;
    const int hb = blockIdx.x - blk * nhb;
    h = hb % NH;
    b = hb / NH;
}

// The forward holds three workgroups per CU (66 registers, 32 KB of LDS), so
// at the GPT-2 124M shape its launch is a single round, and the dispatcher
// hands out workgroup ids in passes of one per CU: a CU's resident blocks
// come from the same position of consecutive passes.  Issued longest-first,
// a CU would take the longest block of every pass (up to 1.3 times the mean
// work); reversing every second one of the resident passes, in groups of 8 ids so
// that every id keeps its XCD, pairs a long block with short ones (within 4%
// of the mean).  Later passes (larger launches) start as slots free up and
// keep the longest-first order.  P: CUs per pass (a multiple of 8).  The
// backward kernels use the same order with their own resident counts: dQ
// holds five 4-wave workgroups per CU (94 registers, 32 KB of LDS), dK/dV
// four (121 registers, 33 KB); there the reversal took the pair from 82 to
// 80 µs at the GPT-2 124M layer shape (1.5 rounds of 1536 workgroups, the
// later ones filling slots as they free up).
constexpr int kAttnCUs = 256, kAttnFwdResident = 3, kAttnDqResident = 5, kAttnDkdvResident = 4;
DEV void attn_block_snake(int nb, int NH, int P, int resident, int& blk, int& h, int& b) {
    int o = blockIdx.x;
    const int pass = o / P, j = o - pass * P;
    if ((pass & 1) && pass < resident && (pass + 1) * P <= (int)gridDim.x)
        o = pass * P + (P - 8 - (j & ~7)) + (j & 7);
    const int nhb = gridDim.x / nb;
    blk = o / nhb;
    const int hb = o - blk * nhb;
    h = hb % NH;
    b = hb / NH;
}

// Maximum over the four 16-lane groups of a wave that hold one query's scores
// (lanes l, l ^ 16, l ^ 32, l ^ 48): two lane swaps, no LDS round trip.
DEV float max_over_groups(float x) { return xor32_combine(xor16_combine(x, MaxOp()), MaxOp()); }

template <typename T, int HS>
struct ACfg {
    static constexpr int KD = HS < 32 ? 32 : HS;         // d extent padded to one MFMA step
    static constexpr int DSTEPS = KD / 32;               // MFMA steps over d
    static constexpr int DT = HS / 16;                   // 16-wide d tiles of an output
    static constexpr int RP = KD + 16 / (int)sizeof(T);  // pitch of row x d tiles
    static constexpr int TP = 64 + 16 / (int)sizeof(T);  // pitch of d x row tiles
    static constexpr int VEC = VecT<T>::N;
    // bf16: operands needed as d x row (V^T, K^T, Q^T, dO^T) are read from the
    // row x d tiles with the LDS transpose load instead of being staged twice
    static constexpr bool TR = sizeof(T) == 2;
    static constexpr int VP = HS + 16;  // pitch of the forward's V tile: HS values + 16 ones
};

// A 16-row x 32-contraction MFMA fragment of X^T from a row-major LDS tile
// X[row][d] (8-byte aligned rows): slots 0..3 are rows k0..k0+3 and slots 4..7
// rows k1..k1+3 of column d0 + l16.  ds_read_b64_tr_b16: within each group of
// 16 lanes, lane l receives element l of the four 4-element pieces read by
// lanes 4j..4j+3 (j = 0..3), so lane s reads row k + s/4, columns 4(s%4)...
DEV void frag_tr(Frag<bf16_t>& f, const bf16_t* tile, int pitch, int k0, int k1, int d0, int l16) {
    typedef short v8s_t __attribute__((ext_vector_type(8)));
    const int col = d0 + 4 * (l16 & 3);
    const v4s_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s_t*)(tile + (k0 + (l16 >> 2)) * pitch + col));
    const v4s_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s_t*)(tile + (k1 + (l16 >> 2)) * pitch + col));
    const v8s_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    f.v = __builtin_bit_cast(bf16x8_t, ab);
}

// This lane's row (global index `row`) of a head slice as DSTEPS fragments over d.
template <typename T, int HS>
DEV void row_frags(Frag<T>* f, const T* src, long rs, int row, int T_, int g4) {
#pragma unroll
    for (int ks = 0; ks < ACfg<T, HS>::DSTEPS; ks++) {
        const int d0 = 32 * ks + 8 * g4;
        if (row < T_ && d0 < HS) frag_gld(f[ks], src + (long)row * rs + d0);
        else frag_zero(f[ks]);
    }
}

// Register-staged copies of the same two layouts, split into a load (issued
// one block ahead, so its latency hides behind the current block's MFMAs) and
// an LDS store.  FULL: rows row0..row0+63 are all < T (no row check).
// COLS columns (zero past HS) of 64 rows into an LDS tile of pitch PITCH.
// Per-thread element offsets within a block are computed once (init); a load
// only adds the block's row origin, a wave-uniform value.
template <typename T, int HS, int COLS = ACfg<T, HS>::KD, int PITCH = ACfg<T, HS>::RP>
struct RowsStage {
    using A = ACfg<T, HS>;
    static constexpr int VPR = COLS / A::VEC;
    static constexpr int ITEMS = 64 * VPR;
    static constexpr int N = (ITEMS + 255) / 256;
    uint4 r[N];
    uint32_t off[N];  // row * rs + d0 (elements)
    int row[N];       // row within the block; >= 64 (or past HS) marks an idle slot
    DEV void init(long rs, int tid) {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = tid + 256 * i;
            const int rr = idx / VPR, d0 = (idx % VPR) * A::VEC;
            const bool live = (ITEMS % 256 == 0 || idx < ITEMS) && d0 < HS;
            row[i] = live ? rr : 1 << 20;
            off[i] = live ? (uint32_t)(rr * rs + d0) : 0u;
        }
    }
    template <bool FULL>
    DEV void load(const T* src, long rs, int row0, int T_) {
        const T* base = src + (long)row0 * rs;
        const int lim = T_ - row0;
#pragma unroll
        for (int i = 0; i < N; i++) {
            const bool ok = FULL ? row[i] < 64 : row[i] < lim;
            r[i] = ok ? ld16(base + off[i]) : make_uint4(0, 0, 0, 0);
        }
    }
    DEV void store(T* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = tid + 256 * i;
            if (ITEMS % 256 == 0 || idx < ITEMS) st16(dst + (idx / VPR) * PITCH + (idx % VPR) * A::VEC, r[i]);
        }
    }
};
template <typename T, int HS>
struct RowsTStage {
    using A = ACfg<T, HS>;
    static constexpr int DG = HS / A::VEC;
    static constexpr int ITEMS = 16 * DG;  // (4-row group, 16-byte column) pairs
    static constexpr int N = (ITEMS + 255) / 256;
    uint4 r[N][4];
    template <bool FULL>
    DEV void load(const T* src, long rs, int row0, int T_, int tid) {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = tid + 256 * i;
            const int kq = idx % 16, dg = idx / 16;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int gr = row0 + 4 * kq + j;
                r[i][j] = (idx < ITEMS && (FULL || gr < T_)) ? ld16(src + (long)gr * rs + dg * A::VEC)
                                                             : make_uint4(0, 0, 0, 0);
            }
        }
    }
    DEV void store(T* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = tid + 256 * i;
            if (ITEMS % 256 == 0 || idx < ITEMS) store_t4<T>(dst + (idx / 16) * A::VEC * A::TP + 4 * (idx % 16), A::TP, r[i]);
        }
    }
};

// ------------------------------------------------------------------ forward -
// Per 64-key block and wave (16 query rows): S^T = K Q^T (HS/32 MFMA steps per
// 16-key tile), online softmax in fp32 on the lane-owned scores, O^T += V^T P^T.
// The scores' scale is folded into the exponent (one FMA per score), exp2 is
// the hardware instruction (results below 2^-126 flush to zero, far below
// anything that reaches bf16 or the loss), the causal mask is only evaluated
// on the diagonal block, and the row sums come out of the P V product itself:
// V^T is extended by 16 rows of ones, so that extra output tile holds
// sum_key P for every query.  O is rescaled only when some row's maximum grew.
template <typename T, int HS>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(T* __restrict__ out, float* __restrict__ lse,
                                                       const T* __restrict__ qkv, int T_, int C, int NH,
                                                       float sl2) {
    using A = ACfg<T, HS>;
    constexpr int DT1 = A::DT + 1;  // output tiles incl. the row-sum tile
    __shared__ __attribute__((aligned(16))) T sK[64 * A::RP];
    // V as d x key (transposed staging) or, bf16, as key x d with 16 columns of ones
    __shared__ __attribute__((aligned(16))) T sVt[A::TR ? 64 * A::VP : (HS + 16) * A::TP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nb = (T_ + 63) / 64;
    int blk, h, b;
    attn_block(nb, NH, blk, h, b);
    const int qb = nb - 1 - blk;
    const long rs = 3L * C;
    const T* Qh = qkv + (long)b * T_ * rs + h * HS;
    const T* Kh = Qh + C;
    const T* Vh = Qh + 2 * C;
    const int q = qb * 64 + wave * 16 + l16;

    // the ones rows of the extended V^T (written once)
    for (int i = tid; i < 16 * 64; i += 256) {
        if constexpr (A::TR) sVt[(i / 16) * A::VP + HS + (i % 16)] = from_f<T>(1.0f);
        else sVt[(HS + i / 64) * A::TP + (i % 64)] = from_f<T>(1.0f);
    }

    Frag<T> fq[A::DSTEPS];
    row_frags<T, HS>(fq, Qh, rs, q, T_, g4);

    float m_run = -INFINITY;  // running max of the raw scores of this lane's query
    f32x4_t o[DT1];
#pragma unroll
    for (int dt = 0; dt < DT1; dt++) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    RowsStage<T, HS> pk;
    std::conditional_t<A::TR, RowsStage<T, HS, HS, A::VP>, RowsTStage<T, HS>> pv;
    pk.init(rs, tid);
    if constexpr (A::TR) pv.init(rs, tid);
    auto prefetch = [&](int kb) {
        if (kb < qb) {
            pk.template load<true>(Kh, rs, kb * 64, T_);
            if constexpr (A::TR) pv.template load<true>(Vh, rs, kb * 64, T_);
            else pv.template load<true>(Vh, rs, kb * 64, T_, tid);
        } else {
            pk.template load<false>(Kh, rs, kb * 64, T_);
            if constexpr (A::TR) pv.template load<false>(Vh, rs, kb * 64, T_);
            else pv.template load<false>(Vh, rs, kb * 64, T_, tid);
        }
    };
    prefetch(0);
    auto block = [&](int kb, auto diag) {
        __syncthreads();
        pk.store(sK, tid);
        pv.store(sVt, tid);
        __syncthreads();
        if (kb < qb) prefetch(kb + 1);
        // S^T tiles: lane holds S^T[key = 16kt + 4g4 + r][query = l16]
        f32x4_t s[4];
#pragma unroll
        for (int kt = 0; kt < 4; kt++) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < A::DSTEPS; ks++) {
                Frag<T> fk;
                frag_ld(fk, sK + (16 * kt + l16) * A::RP + 32 * ks + 8 * g4);
                mma(s[kt], fk, fq[ks]);
            }
        }
        if constexpr (decltype(diag)::value) {
#pragma unroll
            for (int kt = 0; kt < 4; kt++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    if (kb * 64 + 16 * kt + 4 * g4 + r > q) s[kt][r] = -INFINITY;
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
            mloc = fmaxf(mloc, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
        mloc = max_over_groups(mloc);
        const float m_new = fmaxf(m_run, mloc);
        if (__any(m_new > m_run)) {
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
#pragma unroll
            for (int dt = 0; dt < DT1; dt++) o[dt] *= alpha;
        }
        m_run = m_new;
        const float mc = -m_new * sl2;
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
#pragma unroll
            for (int r = 0; r < 4; r++) s[kt][r] = __builtin_amdgcn_exp2f(fmaf(s[kt][r], sl2, mc));
        // O^T[d][q] += V^T[d][key] P^T[key][q], 32 keys per step; d-tile DT is the row sum
#pragma unroll
        for (int c = 0; c < 2; c++) {
            float pv[8] = {s[2 * c][0], s[2 * c][1], s[2 * c][2], s[2 * c][3],
                           s[2 * c + 1][0], s[2 * c + 1][1], s[2 * c + 1][2], s[2 * c + 1][3]};
            Frag<T> fp;
            frag_from(fp, pv);
#pragma unroll
            for (int dt = 0; dt < DT1; dt++) {
                Frag<T> fv;
                if constexpr (A::TR) {
                    frag_tr(fv, sVt, A::VP, 32 * c + 4 * g4, 32 * c + 16 + 4 * g4, 16 * dt, l16);
                } else {
                    const T* vr = sVt + (16 * dt + l16) * A::TP + 32 * c + 4 * g4;
                    frag_ld2(fv, vr, vr + 16);
                }
                mma(o[dt], fv, fp);
            }
        }
    };
    for (int kb = 0; kb < qb; kb++) block(kb, std::false_type{});
    block(qb, std::true_type{});

    if (q < T_) {
        const float l_run = o[A::DT][0];
        const float inv = 1.0f / l_run;
        T* orow = out + ((long)b * T_ + q) * C + h * HS;
#pragma unroll
        for (int dt = 0; dt < A::DT; dt++) {
            float v[4] = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
            store4<T>(orow + 16 * dt + 4 * g4, v);
        }
        if (g4 == 0) lse[((long)b * NH + h) * T_ + q] = m_run * sl2 + log2f(l_run);
    }
}

// ------------------------------------------------- forward, bf16, HS = 64 --
// The same computation as attn_fwd_kernel, with the K and V blocks copied from
// global memory straight into LDS (buffer loads with the LDS-destination bit)
// NS - 1 blocks ahead into NS stage buffers: no registers hold staged data, no
// LDS store instructions are issued, and a wave waits for a block's loads only
// when that block is about to be used.  One barrier per block makes the
// block's loads (issued by all the waves) visible and frees the stage buffer
// the next loads overwrite.  Each wave's 16-byte lane loads fill 1 KB (8 rows
// of 128 bytes) contiguously, so the layout is set by which element a lane
// fetches:
//   K block: 16-byte chunk c of key row r at chunk c ^ (r & 7), so the S^T
//            fragment reads of 8 consecutive rows hit 8 different bank groups;
//   V block: 32-byte unit u (16 d values) of key row r at unit u ^ ((r >> 1) & 3),
//            so each transposing read of V^T (rows 4g..4g+3 for lane group g)
//            covers every bank once per 32 lanes.
// Rows past T_ read as zeros (buffer range).  Each lane sums the fp32
// weights of its 16 keys per block, and the four lane groups of a query are
// added once at the end.
//
// A workgroup of NWV waves owns QR = 16 NWV query rows (one 16-row group per
// wave) and streams the 64-key blocks 0 .. (its last row) / 64.  Every K/V
// block a workgroup loads feeds all its rows: with 128 rows per workgroup the
// K/V traffic from L2 is half that of 64, and the step's kernels all run at
// about the same L2 request rate, so that traffic sets the time.  A wave skips
// the blocks past its own rows (it still takes part in the loads and
// barriers) and masks only the blocks that reach past its first row.
template <int NS, int NWV>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void attn_fwd_dtl_kernel(bf16_t* __restrict__ out,
                                                                      float* __restrict__ lse,
                                                                      const bf16_t* __restrict__ qkv, int T_, int C,
                                                                      int NH, float sl2) {
    constexpr int HS = 64, BLK = 64 * HS, QR = 16 * NWV, NLD = 8 / NWV;  // NLD: 1 KB loads per wave per operand
    static_assert(NWV == 4 || NWV == 8, "64 or 128 query rows per workgroup");
    __shared__ __attribute__((aligned(1024))) bf16_t sKV[NS][2][BLK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nb = (T_ + QR - 1) / QR;
    int blk, h, b;
    attn_block_snake(nb, NH, kAttnCUs, kAttnFwdResident, blk, h, b);
    const int qb = nb - 1 - blk;
    const long rs = 3L * C;
    const bf16_t* Qh = qkv + (long)b * T_ * rs + h * HS;
    const bf16_t* Kh = Qh + C;
    const bf16_t* Vh = Qh + 2 * C;
    const int qw = qb * QR + wave * 16;  // this wave's first row
    const int q = qw + l16;
    // the last key block any row of the workgroup sees
    const int kb_last = min((qb * QR + QR - 1) / 64, (T_ - 1) / 64);

    Frag<bf16_t> fq[2];
    row_frags<bf16_t, HS>(fq, Qh, rs, q, T_, g4);

    // byte offsets (from the block's first row) of this lane's K and V loads:
    // load i of wave w fills rows 8 (w + NWV i) .. + 7 of the block
    uint32_t koff[NLD], voff[NLD];
#pragma unroll
    for (int i = 0; i < NLD; i++) {
        const int r = 8 * (wave + NWV * i) + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        const int u = ((lane & 7) >> 1) ^ ((r >> 1) & 3);
        koff[i] = (uint32_t)(((long)r * rs + 8 * c) * 2);
        voff[i] = (uint32_t)(((long)r * rs + 16 * u + 8 * (lane & 1)) * 2);
    }
    auto issue = [&](int kb) {
        const long org = (long)kb * 64 * rs;
        const int rows = min(64, T_ - kb * 64);
        const uint32_t bytes = (uint32_t)(((long)(rows - 1) * rs + HS) * 2);
        const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(Kh + org, bytes);
        const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(Vh + org, bytes);
        bf16_t* st = sKV[kb % NS][0];
#pragma unroll
        for (int i = 0; i < NLD; i++) lds_dma16(rk, koff[i], st + (wave + NWV * i) * 512);
#pragma unroll
        for (int i = 0; i < NLD; i++) lds_dma16(rv, voff[i], st + BLK + (wave + NWV * i) * 512);
    };
    // fragment read offsets (elements): S^T operand K rows 16 kt + l16, chunk
    // 4 ks + g4; V^T operand rows 32 c + 4 g4 + l16 / 4 (+ 16), d tile dt
    int kofs[2], vofs[4];
#pragma unroll
    for (int ks = 0; ks < 2; ks++) kofs[ks] = l16 * 64 + (((4 * ks + g4) ^ (l16 & 7)) << 3);
    const int vf = (2 * g4 + (l16 >> 3)) & 3;
#pragma unroll
    for (int dt = 0; dt < 4; dt++) vofs[dt] = (4 * g4 + (l16 >> 2)) * 64 + ((dt ^ vf) << 4) + 4 * (l16 & 3);

    float m_run = -INFINITY, l_part = 0.f;
    f32x4_t o[4];
#pragma unroll
    for (int dt = 0; dt < 4; dt++) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < NS - 1; p++)
        if (p <= kb_last) issue(p);
    auto block = [&](int kb, auto diag) {
        // this wave's loads of block kb are done once at most those of the
        // blocks issued after it (up to NS - 2) are outstanding
        if (NS > 2 && kb + NS - 2 <= kb_last) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NLD));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("s_barrier" ::: "memory");
        if (kb + NS - 1 <= kb_last) issue(kb + NS - 1);
        const bf16_t* sK = sKV[kb % NS][0];
        const bf16_t* sV = sK + BLK;
        f32x4_t s[4];
#pragma unroll
        for (int kt = 0; kt < 4; kt++) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                Frag<bf16_t> fk;
                frag_ld(fk, sK + kt * 1024 + kofs[ks]);
                mma(s[kt], fk, fq[ks]);
            }
        }
        if constexpr (decltype(diag)::value) {
#pragma unroll
            for (int kt = 0; kt < 4; kt++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    if (kb * 64 + 16 * kt + 4 * g4 + r > q) s[kt][r] = -INFINITY;
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
            mloc = fmaxf(mloc, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
        mloc = max_over_groups(mloc);
        // A row's running maximum moves only when its block maximum lies more
        // than 8 (in exp2 units) above it; until then the weights
        // exp2((s - m_run) sl2) stay below 2^8 and the accumulators need no
        // rescaling.  The row sums and the log-sum-exp use the same m_run, so
        // the result is the same softmax.  The decision is per row (rows that
        // do not move scale by exp2(0) = 1 exactly), so no row's result
        // depends on another row's scores.
        const bool up = (mloc - m_run) * sl2 > 8.0f;
        if (__any(up)) {
            const float m_new = up ? fmaxf(m_run, mloc) : m_run;
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
#pragma unroll
            for (int dt = 0; dt < 4; dt++) o[dt] *= alpha;
            l_part *= alpha;
            m_run = m_new;
        }
        const float mc = -m_run * sl2;
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
#pragma unroll
            for (int r = 0; r < 4; r++) s[kt][r] = __builtin_amdgcn_exp2f(fmaf(s[kt][r], sl2, mc));
        l_part += ((s[0][0] + s[0][1]) + (s[0][2] + s[0][3])) + ((s[1][0] + s[1][1]) + (s[1][2] + s[1][3])) +
                  (((s[2][0] + s[2][1]) + (s[2][2] + s[2][3])) + ((s[3][0] + s[3][1]) + (s[3][2] + s[3][3])));
#pragma unroll
        for (int c = 0; c < 2; c++) {
            float pv[8] = {s[2 * c][0], s[2 * c][1], s[2 * c][2], s[2 * c][3],
                           s[2 * c + 1][0], s[2 * c + 1][1], s[2 * c + 1][2], s[2 * c + 1][3]};
            Frag<bf16_t> fp;
            frag_from(fp, pv);
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                const bf16_t* v0 = sV + c * 2048 + vofs[dt];
                const v4s_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)v0);
                const v4s_t bb =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(v0 + 1024));
                Frag<bf16_t> fv;
                fv.v = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, bb, 0, 1, 2, 3, 4, 5, 6, 7));
                mma(o[dt], fv, fp);
            }
        }
    };
    // a block past this wave's rows: the wave still waits for its own loads,
    // passes the barrier and issues its share of the next block
    auto skip_block = [&](int kb) {
        if (NS > 2 && kb + NS - 2 <= kb_last) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 2 * NLD));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("s_barrier" ::: "memory");
        if (kb + NS - 1 <= kb_last) issue(kb + NS - 1);
    };
    // (a wave's 16 rows lie in one 64-key block, kd: blocks before it are
    // whole, kd is masked, later ones are the other waves')
    const int kd = qw / 64;
    for (int kb = 0; kb < kd; kb++) block(kb, std::false_type{});
    block(kd, std::true_type{});
    for (int kb = kd + 1; kb <= kb_last; kb++) skip_block(kb);

    const float l_run = xor32_combine(xor16_combine(l_part, AddOp()), AddOp());
    if (q < T_) {
        const float inv = 1.0f / l_run;
        bf16_t* orow = out + ((long)b * T_ + q) * C + h * HS;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
            float v[4] = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
            store4<bf16_t>(orow + 16 * dt + 4 * g4, v);
        }
        if (g4 == 0) lse[((long)b * NH + h) * T_ + q] = m_run * sl2 + log2f(l_run);
    }
}

// ---------------------------------------------------------------- backward --
// delta[b,h,t] = sum_d dO[b,t,h,d] * O[b,t,h,d]
template <typename T, int HS>
__global__ void attn_delta_kernel(float* __restrict__ delta, const T* __restrict__ dout, const T* __restrict__ out,
                                  int B, int T_, int C, int NH) {
    constexpr int VEC = VecT<T>::N;
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;  // over B*T*NH, head fastest
    if (i >= (long)B * T_ * NH) return;
    const int h = (int)(i % NH);
    const long bt = i / NH;
    const T* a = dout + bt * C + h * HS;
    const T* o = out + bt * C + h * HS;
    float s = 0.f;
#pragma unroll 2
    for (int d = 0; d < HS; d += VEC) {
        float x[VEC], y[VEC];
        unpack16<T>(ld16(a + d), x);
        unpack16<T>(ld16(o + d), y);
#pragma unroll
        for (int e = 0; e < VEC; e++) s += x[e] * y[e];
    }
    const long b = bt / T_, t = bt % T_;
    delta[(b * NH + h) * T_ + t] = s;
}

// dK/dV: one workgroup per 64-key block, looping over the query blocks at or
// after it.  Query rows past T carry lse = +inf, so their P is exactly zero and
// only the diagonal block needs the causal test; the 1/sqrt(HS) factor of dS is
// applied once to dK at the end.
template <typename T, int HS>
__global__ __launch_bounds__(256, (sizeof(T) == 4 && HS == 128) ? 1 : 2) void attn_bwd_dkdv_kernel(T* __restrict__ dqkv, const T* __restrict__ dout,
                                                               const T* __restrict__ qkv, const float* __restrict__ lse,
                                                               const float* __restrict__ delta, int T_, int C, int NH,
                                                               float sl2, float scale) {
    using A = ACfg<T, HS>;
    __shared__ __attribute__((aligned(16))) T sQ[64 * A::RP];
    __shared__ __attribute__((aligned(16))) T sdO[64 * A::RP];
    __shared__ __attribute__((aligned(16))) T sQt[A::TR ? 8 : HS * A::TP];
    __shared__ __attribute__((aligned(16))) T sdOt[A::TR ? 8 : HS * A::TP];
    __shared__ __attribute__((aligned(16))) float sL[64];
    __shared__ __attribute__((aligned(16))) float sD[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nqb = (T_ + 63) / 64;
    int kb, h, b;
    attn_block(nqb, NH, kb, h, b);
    const long rs = 3L * C;
    const T* Qh = qkv + (long)b * T_ * rs + h * HS;
    const T* Kh = Qh + C;
    const T* Vh = Qh + 2 * C;
    const T* dOh = dout + (long)b * T_ * C + h * HS;
    const float* lse_h = lse + ((long)b * NH + h) * T_;
    const float* del_h = delta + ((long)b * NH + h) * T_;
    const int key = kb * 64 + wave * 16 + l16;

    Frag<T> fk[A::DSTEPS], fv[A::DSTEPS];
    row_frags<T, HS>(fk, Kh, rs, key, T_, g4);
    row_frags<T, HS>(fv, Vh, rs, key, T_, g4);
    f32x4_t dk[A::DT], dv[A::DT];
#pragma unroll
    for (int dt = 0; dt < A::DT; dt++) {
        dk[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dv[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    RowsStage<T, HS> pq, pdo;
    pq.init(rs, tid);
    pdo.init(C, tid);
    RowsTStage<T, HS> pqt, pdot;
    float pl = INFINITY, pd = 0.f;
    auto prefetch = [&](int qb) {
        if ((qb + 1) * 64 <= T_) {
            pq.template load<true>(Qh, rs, qb * 64, T_);
            pdo.template load<true>(dOh, C, qb * 64, T_);
            if constexpr (!A::TR) {
                pqt.template load<true>(Qh, rs, qb * 64, T_, tid);
                pdot.template load<true>(dOh, C, qb * 64, T_, tid);
            }
        } else {
            pq.template load<false>(Qh, rs, qb * 64, T_);
            pdo.template load<false>(dOh, C, qb * 64, T_);
            if constexpr (!A::TR) {
                pqt.template load<false>(Qh, rs, qb * 64, T_, tid);
                pdot.template load<false>(dOh, C, qb * 64, T_, tid);
            }
        }
        const int qq = qb * 64 + (tid & 63);
        pl = qq < T_ ? lse_h[qq] : INFINITY;
        pd = qq < T_ ? del_h[qq] : 0.f;
    };
    prefetch(kb);
    auto block = [&](int qb, auto diag) {
        __syncthreads();
        pq.store(sQ, tid);
        pdo.store(sdO, tid);
        if constexpr (!A::TR) {
            pqt.store(sQt, tid);
            pdot.store(sdOt, tid);
        }
        if (tid < 64) {
            sL[tid] = pl;
            sD[tid] = pd;
        }
        __syncthreads();
        if (qb + 1 < nqb) prefetch(qb + 1);
        // S[q][key] and dP[q][key]: lane holds q = 16qt + 4g4 + r, key = l16 (+ block offsets)
        f32x4_t p[4], ds[4];
#pragma unroll
        for (int qt = 0; qt < 4; qt++) {
            p[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            ds[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < A::DSTEPS; ks++) {
                Frag<T> fa;
                frag_ld(fa, sQ + (16 * qt + l16) * A::RP + 32 * ks + 8 * g4);
                mma(p[qt], fa, fk[ks]);
                frag_ld(fa, sdO + (16 * qt + l16) * A::RP + 32 * ks + 8 * g4);
                mma(ds[qt], fa, fv[ks]);
            }
        }
#pragma unroll
        for (int qt = 0; qt < 4; qt++) {
            const float4 L4 = *reinterpret_cast<const float4*>(sL + 16 * qt + 4 * g4);
            const float4 D4 = *reinterpret_cast<const float4*>(sD + 16 * qt + 4 * g4);
            const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
            const float Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float pr = __builtin_amdgcn_exp2f(fmaf(p[qt][r], sl2, -Lr[r]));
                if constexpr (decltype(diag)::value)
                    if (key > qb * 64 + 16 * qt + 4 * g4 + r) pr = 0.f;
                p[qt][r] = pr;
                ds[qt][r] = pr * (ds[qt][r] - Dr[r]);
            }
        }
        // dV^T[d][key] += dO^T[d][q] P[q][key];  dK^T[d][key] += Q^T[d][q] dS[q][key]
#pragma unroll
        for (int c = 0; c < 2; c++) {
            float pv[8] = {p[2 * c][0], p[2 * c][1], p[2 * c][2], p[2 * c][3],
                           p[2 * c + 1][0], p[2 * c + 1][1], p[2 * c + 1][2], p[2 * c + 1][3]};
            float sv[8] = {ds[2 * c][0], ds[2 * c][1], ds[2 * c][2], ds[2 * c][3],
                           ds[2 * c + 1][0], ds[2 * c + 1][1], ds[2 * c + 1][2], ds[2 * c + 1][3]};
            Frag<T> fp, fs;
            frag_from(fp, pv);
            frag_from(fs, sv);
#pragma unroll
            for (int dt = 0; dt < A::DT; dt++) {
                Frag<T> fa;
                if constexpr (A::TR) {
                    frag_tr(fa, sdO, A::RP, 32 * c + 4 * g4, 32 * c + 16 + 4 * g4, 16 * dt, l16);
                    mma(dv[dt], fa, fp);
                    frag_tr(fa, sQ, A::RP, 32 * c + 4 * g4, 32 * c + 16 + 4 * g4, 16 * dt, l16);
                    mma(dk[dt], fa, fs);
                } else {
                    const int ofs = (16 * dt + l16) * A::TP + 32 * c + 4 * g4;
                    frag_ld2(fa, sdOt + ofs, sdOt + ofs + 16);
                    mma(dv[dt], fa, fp);
                    frag_ld2(fa, sQt + ofs, sQt + ofs + 16);
                    mma(dk[dt], fa, fs);
                }
            }
        }
    };
    block(kb, std::true_type{});
    for (int qb = kb + 1; qb < nqb; qb++) block(qb, std::false_type{});
    if (key < T_) {
        T* row = dqkv + ((long)b * T_ + key) * rs + h * HS;
#pragma unroll
        for (int dt = 0; dt < A::DT; dt++) {
            float kv[4] = {dk[dt][0] * scale, dk[dt][1] * scale, dk[dt][2] * scale, dk[dt][3] * scale};
            float vv[4] = {dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]};
            store4<T>(row + C + 16 * dt + 4 * g4, kv);
            store4<T>(row + 2 * C + 16 * dt + 4 * g4, vv);
        }
    }
}

// dQ: one workgroup per 64-query block, looping over the key blocks at or
// before it (all full but the diagonal one); 1/sqrt(HS) applied at the end.
template <typename T, int HS>
__global__ __launch_bounds__(256, (sizeof(T) == 4 && HS == 128) ? 1 : 2) void attn_bwd_dq_kernel(T* __restrict__ dqkv, const T* __restrict__ dout,
                                                             const T* __restrict__ qkv, const float* __restrict__ lse,
                                                             const float* __restrict__ delta, int T_, int C, int NH,
                                                             float sl2, float scale) {
    using A = ACfg<T, HS>;
    __shared__ __attribute__((aligned(16))) T sK[64 * A::RP];
    __shared__ __attribute__((aligned(16))) T sV[64 * A::RP];
    __shared__ __attribute__((aligned(16))) T sKt[A::TR ? 8 : HS * A::TP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nb = (T_ + 63) / 64;
    int blk, h, b;
    attn_block(nb, NH, blk, h, b);
    const int qb = nb - 1 - blk;
    const long rs = 3L * C;
    const T* Qh = qkv + (long)b * T_ * rs + h * HS;
    const T* Kh = Qh + C;
    const T* Vh = Qh + 2 * C;
    const T* dOh = dout + (long)b * T_ * C + h * HS;
    const int q = qb * 64 + wave * 16 + l16;
    const float Lq = q < T_ ? lse[((long)b * NH + h) * T_ + q] : INFINITY;
    const float Dq = q < T_ ? delta[((long)b * NH + h) * T_ + q] : 0.f;

    Frag<T> fq[A::DSTEPS], fo[A::DSTEPS];
    row_frags<T, HS>(fq, Qh, rs, q, T_, g4);
    row_frags<T, HS>(fo, dOh, C, q, T_, g4);
    f32x4_t dq[A::DT];
#pragma unroll
    for (int dt = 0; dt < A::DT; dt++) dq[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    RowsStage<T, HS> pk, pv;
    RowsTStage<T, HS> pkt;
    pk.init(rs, tid);
    pv.init(rs, tid);
    auto prefetch = [&](int kb) {
        if (kb < qb) {
            pk.template load<true>(Kh, rs, kb * 64, T_);
            pv.template load<true>(Vh, rs, kb * 64, T_);
            if constexpr (!A::TR) pkt.template load<true>(Kh, rs, kb * 64, T_, tid);
        } else {
            pk.template load<false>(Kh, rs, kb * 64, T_);
            pv.template load<false>(Vh, rs, kb * 64, T_);
            if constexpr (!A::TR) pkt.template load<false>(Kh, rs, kb * 64, T_, tid);
        }
    };
    prefetch(0);
    auto block = [&](int kb, auto diag) {
        __syncthreads();
        pk.store(sK, tid);
        pv.store(sV, tid);
        if constexpr (!A::TR) pkt.store(sKt, tid);
        __syncthreads();
        if (kb < qb) prefetch(kb + 1);
        // S^T[key][q], dP^T[key][q]: lane holds key = 16kt + 4g4 + r, q = l16
        f32x4_t s[4], dp[4];
#pragma unroll
        for (int kt = 0; kt < 4; kt++) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < A::DSTEPS; ks++) {
                Frag<T> fa;
                frag_ld(fa, sK + (16 * kt + l16) * A::RP + 32 * ks + 8 * g4);
                mma(s[kt], fa, fq[ks]);
                frag_ld(fa, sV + (16 * kt + l16) * A::RP + 32 * ks + 8 * g4);
                mma(dp[kt], fa, fo[ks]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float pr = __builtin_amdgcn_exp2f(fmaf(s[kt][r], sl2, -Lq));
                if constexpr (decltype(diag)::value)
                    if (kb * 64 + 16 * kt + 4 * g4 + r > q) pr = 0.f;
                s[kt][r] = pr * (dp[kt][r] - Dq);  // dS^T / scale
            }
        // dQ^T[d][q] += K^T[d][key] dS^T[key][q]
#pragma unroll
        for (int c = 0; c < 2; c++) {
            float sv[8] = {s[2 * c][0], s[2 * c][1], s[2 * c][2], s[2 * c][3],
                           s[2 * c + 1][0], s[2 * c + 1][1], s[2 * c + 1][2], s[2 * c + 1][3]};
            Frag<T> fs;
            frag_from(fs, sv);
#pragma unroll
            for (int dt = 0; dt < A::DT; dt++) {
                Frag<T> fa;
                if constexpr (A::TR) {
                    frag_tr(fa, sK, A::RP, 32 * c + 4 * g4, 32 * c + 16 + 4 * g4, 16 * dt, l16);
                } else {
                    const T* kr = sKt + (16 * dt + l16) * A::TP + 32 * c + 4 * g4;
                    frag_ld2(fa, kr, kr + 16);
                }
                mma(dq[dt], fa, fs);
            }
        }
    };
    for (int kb = 0; kb < qb; kb++) block(kb, std::false_type{});
    block(qb, std::true_type{});
    if (q < T_) {
        T* row = dqkv + ((long)b * T_ + q) * rs + h * HS;
#pragma unroll
        for (int dt = 0; dt < A::DT; dt++) {
            float v[4] = {dq[dt][0] * scale, dq[dt][1] * scale, dq[dt][2] * scale, dq[dt][3] * scale};
            store4<T>(row + 16 * dt + 4 * g4, v);
        }
    }
}

// ------------------------------------------------ backward, bf16, HS = 64 --
// The dK/dV and dQ kernels with their streamed blocks (Q and dO, or K and V)
// copied straight into LDS like the forward's K and V.  Every streamed tile
// is read both as rows (16-byte fragment reads) and transposed (the LDS
// transpose read), so all use one layout: 64 rows of 128 bytes, 16-byte chunk
// c of row r at chunk c ^ (r & 7).  Both reads then cover every bank once per
// 32 lanes: a row read spreads 8 consecutive rows over 8 chunk positions, and
// a transpose read (rows 4g..4g+3 for lane group g, a 32-byte d tile = two
// chunks) lands its 8 rows on 8 different (row parity, chunk) pairs.

// This wave's two 1 KB loads of a 64 x 64 bf16 tile in that layout.
struct Tile64 {
    uint32_t off[2];  // byte offsets from the tile's first row, row stride ld elements
    DEV void init(long ld, int lane, int wave) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int r = 8 * (wave + 4 * i) + (lane >> 3);
            const int c = (lane & 7) ^ (r & 7);
            off[i] = (uint32_t)(((long)r * ld + 8 * c) * 2);
        }
    }
    // rows row0 .. min(row0 + 64, T_) - 1 of src (row stride ld); rows past T_ read as zeros
    DEV void issue(const bf16_t* src, long ld, int row0, int T_, bf16_t* dst, int wave) const {
        const int rows = min(64, T_ - row0);
        const uint32_t bytes = (uint32_t)(((long)(rows - 1) * ld + 64) * 2);
        const __amdgpu_buffer_rsrc_t r = uniform_rsrc(src + (long)row0 * ld, bytes);
#pragma unroll
        for (int i = 0; i < 2; i++) lds_dma16(r, off[i], dst + (wave + 4 * i) * 512);
    }
};

// Fragment read offsets (elements) within such a tile.  Row reads: rows
// 16 t + l16 (t added as t * 1024), chunk 4 ks + g4.  Transpose reads of d tile
// dt: rows 32 c + 4 g4 + l16 / 4 and 16 rows further (c added as c * 2048),
// columns 16 dt + 4 (l16 % 4).
struct Tile64Ofs {
    int row[2], tr[4];
    DEV void init(int l16, int g4) {
#pragma unroll
        for (int ks = 0; ks < 2; ks++) row[ks] = l16 * 64 + (((4 * ks + g4) ^ (l16 & 7)) << 3);
        const int r = 4 * g4 + (l16 >> 2);
#pragma unroll
        for (int dt = 0; dt < 4; dt++) tr[dt] = r * 64 + (((2 * dt + ((l16 >> 1) & 1)) ^ (r & 7)) << 3) + 4 * (l16 & 1);
    }
};

DEV void tr_frag(Frag<bf16_t>& f, const bf16_t* p) {
    const v4s_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)p);
    const v4s_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(p + 1024));
    f.v = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// dK/dV for one 64-key block over the query blocks at or after it; lse and
// delta of the next query block are read into registers one block ahead and
// put in LDS (two slots) before the barrier that opens the block.
template <int NS>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_dtl_kernel(bf16_t* __restrict__ dqkv,
                                                                const bf16_t* __restrict__ dout,
                                                                const bf16_t* __restrict__ qkv,
                                                                const float* __restrict__ lse,
                                                                const float* __restrict__ delta, int T_, int C,
                                                                int NH, float sl2, float scale) {
    constexpr int HS = 64, BLK = 64 * HS;
    __shared__ __attribute__((aligned(1024))) bf16_t sQO[NS][2][BLK];
    __shared__ __attribute__((aligned(16))) float sLD[NS][2][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nqb = (T_ + 63) / 64;
    int kb, h, b;
    attn_block_snake(nqb, NH, kAttnCUs, kAttnDkdvResident, kb, h, b);
    const long rs = 3L * C;
    const bf16_t* Qh = qkv + (long)b * T_ * rs + h * HS;
    const bf16_t* Kh = Qh + C;
    const bf16_t* Vh = Qh + 2 * C;
    const bf16_t* dOh = dout + (long)b * T_ * C + h * HS;
    const float* lse_h = lse + ((long)b * NH + h) * T_;
    const float* del_h = delta + ((long)b * NH + h) * T_;
    const int key = kb * 64 + wave * 16 + l16;

    Frag<bf16_t> fk[2], fv[2];
    row_frags<bf16_t, HS>(fk, Kh, rs, key, T_, g4);
    row_frags<bf16_t, HS>(fv, Vh, rs, key, T_, g4);
    f32x4_t dk[4], dv[4];
#pragma unroll
    for (int dt = 0; dt < 4; dt++) {
        dk[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dv[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    Tile64 tq, to;
    tq.init(rs, lane, wave);
    to.init(C, lane, wave);
    Tile64Ofs ofs;
    ofs.init(l16, g4);
    auto issue = [&](int qb) {
        bf16_t* st = sQO[qb % NS][0];
        tq.issue(Qh, rs, qb * 64, T_, st, wave);
        to.issue(dOh, C, qb * 64, T_, st + BLK, wave);
    };
    // query rows past T_: lse = +inf makes their P exactly zero
    float pl = INFINITY, pd = 0.f;
    auto load_ld = [&](int qb) {
        const int qq = qb * 64 + lane;
        pl = qq < T_ ? lse_h[qq] : INFINITY;
        pd = qq < T_ ? del_h[qq] : 0.f;
    };
    if (wave == 0) load_ld(kb);
#pragma unroll
    for (int p = 0; p < NS - 1; p++)
        if (kb + p < nqb) issue(kb + p);
    auto block = [&](int qb, auto diag) {
        float* sL = sLD[qb % NS][0];
        float* sD = sLD[qb % NS][1];
        if (wave == 0) {
            sL[lane] = pl;
            sD[lane] = pd;
        }
        if (NS > 2 && qb + NS - 2 < nqb) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 4));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the lse / delta writes are done
        asm volatile("s_barrier" ::: "memory");
        if (qb + NS - 1 < nqb) issue(qb + NS - 1);
        if (wave == 0 && qb + 1 < nqb) load_ld(qb + 1);
        const bf16_t* sQ = sQO[qb % NS][0];
        const bf16_t* sdO = sQ + BLK;
        // S[q][key] and dP[q][key] - delta[q] (the dP accumulators start at
        // -delta): lane holds q = 16qt + 4g4 + r, key = l16 (+ block offsets)
        f32x4_t p[4], ds[4];
#pragma unroll
        for (int qt = 0; qt < 4; qt++) {
            p[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const float4 D4 = *reinterpret_cast<const float4*>(sD + 16 * qt + 4 * g4);
            ds[qt] = f32x4_t{-D4.x, -D4.y, -D4.z, -D4.w};
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                Frag<bf16_t> fa;
                frag_ld(fa, sQ + qt * 1024 + ofs.row[ks]);
                mma(p[qt], fa, fk[ks]);
                frag_ld(fa, sdO + qt * 1024 + ofs.row[ks]);
                mma(ds[qt], fa, fv[ks]);
            }
        }
#pragma unroll
        for (int qt = 0; qt < 4; qt++) {
            const float4 L4 = *reinterpret_cast<const float4*>(sL + 16 * qt + 4 * g4);
            const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float pr = __builtin_amdgcn_exp2f(fmaf(p[qt][r], sl2, -Lr[r]));
                if constexpr (decltype(diag)::value)
                    if (key > qb * 64 + 16 * qt + 4 * g4 + r) pr = 0.f;
                p[qt][r] = pr;
                ds[qt][r] = pr * ds[qt][r];
            }
        }
        // dV^T[d][key] += dO^T[d][q] P[q][key];  dK^T[d][key] += Q^T[d][q] dS[q][key]
#pragma unroll
        for (int c = 0; c < 2; c++) {
            float pv[8] = {p[2 * c][0], p[2 * c][1], p[2 * c][2], p[2 * c][3],
                           p[2 * c + 1][0], p[2 * c + 1][1], p[2 * c + 1][2], p[2 * c + 1][3]};
            float sv[8] = {ds[2 * c][0], ds[2 * c][1], ds[2 * c][2], ds[2 * c][3],
                           ds[2 * c + 1][0], ds[2 * c + 1][1], ds[2 * c + 1][2], ds[2 * c + 1][3]};
            Frag<bf16_t> fp, fs;
            frag_from(fp, pv);
            frag_from(fs, sv);
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                Frag<bf16_t> fa;
                tr_frag(fa, sdO + c * 2048 + ofs.tr[dt]);
                mma(dv[dt], fa, fp);
                tr_frag(fa, sQ + c * 2048 + ofs.tr[dt]);
                mma(dk[dt], fa, fs);
            }
        }
    };
    block(kb, std::true_type{});
    for (int qb = kb + 1; qb < nqb; qb++) block(qb, std::false_type{});
    if (key < T_) {
        bf16_t* row = dqkv + ((long)b * T_ + key) * rs + h * HS;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
            float kv[4] = {dk[dt][0] * scale, dk[dt][1] * scale, dk[dt][2] * scale, dk[dt][3] * scale};
            float vv[4] = {dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]};
            store4<bf16_t>(row + C + 16 * dt + 4 * g4, kv);
            store4<bf16_t>(row + 2 * C + 16 * dt + 4 * g4, vv);
        }
    }
}

// dQ for one 64-query block over the key blocks at or before it.  It also
// computes the block's delta = rowsum(dO * O) itself (each query row belongs
// to exactly one workgroup here) and stores it for the dK/dV kernel, which
// runs after it: no separate delta pass.
template <int NS>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_dtl_kernel(bf16_t* __restrict__ dqkv,
                                                              const bf16_t* __restrict__ dout,
                                                              const bf16_t* __restrict__ out,
                                                              const bf16_t* __restrict__ qkv,
                                                              const float* __restrict__ lse,
                                                              float* __restrict__ delta, int T_, int C,
                                                              int NH, float sl2, float scale) {
    constexpr int HS = 64, BLK = 64 * HS;
    __shared__ __attribute__((aligned(1024))) bf16_t sKV[NS][2][BLK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nb = (T_ + 63) / 64;
    int blk, h, b;
    attn_block_snake(nb, NH, kAttnCUs, kAttnDqResident, blk, h, b);
    const int qb = nb - 1 - blk;
    const long rs = 3L * C;
    const bf16_t* Qh = qkv + (long)b * T_ * rs + h * HS;
    const bf16_t* Kh = Qh + C;
    const bf16_t* Vh = Qh + 2 * C;
    const bf16_t* dOh = dout + (long)b * T_ * C + h * HS;
    const int q = qb * 64 + wave * 16 + l16;
    const float Lq = q < T_ ? lse[((long)b * NH + h) * T_ + q] : INFINITY;

    Frag<bf16_t> fq[2], fo[2], fy[2];
    row_frags<bf16_t, HS>(fq, Qh, rs, q, T_, g4);
    row_frags<bf16_t, HS>(fo, dOh, C, q, T_, g4);
    row_frags<bf16_t, HS>(fy, out + (long)b * T_ * C + h * HS, C, q, T_, g4);
    // delta of this lane's query: its 16 of the 64 d values (d = 32 ks + 8 g4
    // + j), then the four lane groups holding the query added in a fixed order
    float Dq = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int j = 0; j < 8; j++) Dq += (float)fo[ks].v[j] * (float)fy[ks].v[j];
    Dq = xor32_combine(xor16_combine(Dq, AddOp()), AddOp());
    if (q < T_ && g4 == 0) delta[((long)b * NH + h) * T_ + q] = Dq;
    f32x4_t dq[4];
#pragma unroll
    for (int dt = 0; dt < 4; dt++) dq[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    Tile64 tkv;
    tkv.init(rs, lane, wave);
    Tile64Ofs ofs;
    ofs.init(l16, g4);
    auto issue = [&](int kb) {
        bf16_t* st = sKV[kb % NS][0];
        tkv.issue(Kh, rs, kb * 64, T_, st, wave);
        tkv.issue(Vh, rs, kb * 64, T_, st + BLK, wave);
    };
#pragma unroll
    for (int p = 0; p < NS - 1; p++)
        if (p <= qb) issue(p);
    auto block = [&](int kb, auto diag) {
        if (NS > 2 && kb + NS - 2 <= qb) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * 4));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("s_barrier" ::: "memory");
        if (kb + NS - 1 <= qb) issue(kb + NS - 1);
        const bf16_t* sK = sKV[kb % NS][0];
        const bf16_t* sV = sK + BLK;
        // S^T[key][q], dP^T[key][q] - delta[q] (the dP accumulators start at
        // -delta): lane holds key = 16kt + 4g4 + r, q = l16
        f32x4_t s[4], dp[4];
#pragma unroll
        for (int kt = 0; kt < 4; kt++) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[kt] = f32x4_t{-Dq, -Dq, -Dq, -Dq};
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                Frag<bf16_t> fa;
                frag_ld(fa, sK + kt * 1024 + ofs.row[ks]);
                mma(s[kt], fa, fq[ks]);
                frag_ld(fa, sV + kt * 1024 + ofs.row[ks]);
                mma(dp[kt], fa, fo[ks]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float pr = __builtin_amdgcn_exp2f(fmaf(s[kt][r], sl2, -Lq));
                if constexpr (decltype(diag)::value)
                    if (kb * 64 + 16 * kt + 4 * g4 + r > q) pr = 0.f;
                s[kt][r] = pr * dp[kt][r];  // dS^T / scale
            }
        // dQ^T[d][q] += K^T[d][key] dS^T[key][q]
#pragma unroll
        for (int c = 0; c < 2; c++) {
            float sv[8] = {s[2 * c][0], s[2 * c][1], s[2 * c][2], s[2 * c][3],
                           s[2 * c + 1][0], s[2 * c + 1][1], s[2 * c + 1][2], s[2 * c + 1][3]};
            Frag<bf16_t> fs;
            frag_from(fs, sv);
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                Frag<bf16_t> fa;
                tr_frag(fa, sK + c * 2048 + ofs.tr[dt]);
                mma(dq[dt], fa, fs);
            }
        }
    };
    for (int kb = 0; kb < qb; kb++) block(kb, std::false_type{});
    block(qb, std::true_type{});
    if (q < T_) {
        bf16_t* row = dqkv + ((long)b * T_ + q) * rs + h * HS;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
            float v[4] = {dq[dt][0] * scale, dq[dt][1] * scale, dq[dt][2] * scale, dq[dt][3] * scale};
            store4<bf16_t>(row + 16 * dt + 4 * g4, v);
        }
    }
}

template <typename T, int HS>
int fwd_hs(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s) {
    const int nb = (T_ + 63) / 64;
    const float sl2 = LOG2E / sqrtf((float)HS);
    if constexpr (std::is_same_v<T, bf16_t> && HS == 64) {
        // direct-to-LDS loads address a batch's rows with 32-bit byte offsets
        if ((long)T_ * 3 * C * 2 < (1L << 31)) {
            constexpr int NWV = ATTN_FWD_WAVES;
            const int nq = (T_ + 16 * NWV - 1) / (16 * NWV);
            hipLaunchKernelGGL((attn_fwd_dtl_kernel<ATTN_FWD_NS, NWV>), dim3(nq * NH * B), dim3(64 * NWV), 0, s, out,
                               lse, qkv, T_, C, NH, sl2);
            return (int)hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attn_fwd_kernel<T, HS>), dim3(nb * NH * B), dim3(256), 0, s, out, lse, qkv, T_, C, NH, sl2);
    return (int)hipGetLastError();
}

template <typename T, int HS>
int bwd_hs(T* dqkv, float* delta, const T* dout, const T* out, const T* qkv, const float* lse,
           int B, int T_, int C, int NH, hipStream_t s) {
    const int nb = (T_ + 63) / 64;
    const float scale = 1.0f / sqrtf((float)HS);
    const float sl2 = LOG2E * scale;
    const long rows = (long)B * T_ * NH;
    if constexpr (std::is_same_v<T, bf16_t> && HS == 64) {
        if ((long)T_ * 3 * C * 2 < (1L << 31)) {
            // dQ first: it writes delta, which dK/dV reads
            hipLaunchKernelGGL((attn_bwd_dq_dtl_kernel<ATTN_BWD_NS>), dim3(nb * NH * B), dim3(256), 0, s, dqkv, dout,
                               out, qkv, lse, delta, T_, C, NH, sl2, scale);
            hipLaunchKernelGGL((attn_bwd_dkdv_dtl_kernel<ATTN_BWD_NS>), dim3(nb * NH * B), dim3(256), 0, s, dqkv,
                               dout, qkv, lse, delta, T_, C, NH, sl2, scale);
            return (int)hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attn_delta_kernel<T, HS>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                       delta, dout, out, B, T_, C, NH);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HS>), dim3(nb * NH * B), dim3(256), 0, s, dqkv, dout, qkv, lse,
                       delta, T_, C, NH, sl2, scale);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HS>), dim3(nb * NH * B), dim3(256), 0, s, dqkv, dout, qkv, lse,
                       delta, T_, C, NH, sl2, scale);
    return (int)hipGetLastError();
}

}  // namespace

template <typename T>
int attention_fwd_launch(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s) {
    if (B <= 0 || T_ <= 0) return 0;
    switch (C / NH) {
        case 16: return fwd_hs<T, 16>(out, lse, qkv, B, T_, C, NH, s);
        case 32: return fwd_hs<T, 32>(out, lse, qkv, B, T_, C, NH, s);
        case 64: return fwd_hs<T, 64>(out, lse, qkv, B, T_, C, NH, s);
        case 128: return fwd_hs<T, 128>(out, lse, qkv, B, T_, C, NH, s);
        default: return (int)hipErrorInvalidValue;
    }
}

template <typename T>
int attention_bwd_launch(T* dqkv, float* delta, const T* dout, const T* out, const T* qkv,
                         const float* lse, int B, int T_, int C, int NH, hipStream_t s) {
    if (B <= 0 || T_ <= 0) return 0;
    switch (C / NH) {
        case 16: return bwd_hs<T, 16>(dqkv, delta, dout, out, qkv, lse, B, T_, C, NH, s);
        case 32: return bwd_hs<T, 32>(dqkv, delta, dout, out, qkv, lse, B, T_, C, NH, s);
        case 64: return bwd_hs<T, 64>(dqkv, delta, dout, out, qkv, lse, B, T_, C, NH, s);
        case 128: return bwd_hs<T, 128>(dqkv, delta, dout, out, qkv, lse, B, T_, C, NH, s);
        default: return (int)hipErrorInvalidValue;
    }
}

template int attention_fwd_launch<float>(float*, float*, const float*, int, int, int, int, hipStream_t);
template int attention_fwd_launch<bf16_t>(bf16_t*, float*, const bf16_t*, int, int, int, int, hipStream_t);
template int attention_bwd_launch<float>(float*, float*, const float*, const float*, const float*, const float*,
                                         int, int, int, int, hipStream_t);
template int attention_bwd_launch<bf16_t>(bf16_t*, float*, const bf16_t*, const bf16_t*, const bf16_t*, const float*,
                                          int, int, int, int, hipStream_t);
