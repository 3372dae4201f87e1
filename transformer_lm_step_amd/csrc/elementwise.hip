// elementwise.hip - token/position encoder, fused softmax cross-entropy,
// AdamW and small utilities (gfx950).
#include <math.h>

#include <algorithm>

#include "device.h"
#include "kernels.h"

namespace {

// ------------------------------------------------------------ encoder fwd ---
// train_gpt2.cu, encoder_forward_kernel2: out[b,t,:] = wte[tok[b,t],:] + wpe[t,:].
// One thread per 16-byte vector.  Token ids outside [0, V) raise *flag and are
// replaced by 0 so that no read leaves the table; the (clamped) ids are copied
// for the backward pass.
template <typename T>
__global__ void encoder_fwd_kernel(T* __restrict__ out, int* __restrict__ tok_copy, const int* __restrict__ tok,
                                   const T* __restrict__ wte, const T* __restrict__ wpe, int BT, int T_, int C,
                                   int V, int* __restrict__ flag) {
    constexpr int VEC = VecT<T>::N;
    const int vpr = C / VEC;
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)BT * vpr) return;
    const int bt = (int)(i / vpr), c0 = (int)(i % vpr) * VEC;
    int ix = tok[bt];
    if (ix < 0 || ix >= V) {
        if (c0 == 0) flag[0] = 1;
        ix = 0;
    }
    if (c0 == 0) tok_copy[bt] = ix;
    const int t = bt % T_;
    float a[VEC], p[VEC];
    unpack16<T>(ld16(wte + (long)ix * C + c0), a);
    unpack16<T>(ld16(wpe + (long)t * C + c0), p);
#pragma unroll
    for (int e = 0; e < VEC; e++) a[e] += p[e];
    st16(out + (long)bt * C + c0, pack16<T>(a));
}

// ------------------------------------------------------------ encoder bwd ---
// train_gpt2.cu, encoder_backward_kernel, without atomics: dwte[v] += the
// residual-gradient rows of every position holding token v, summed in a
// fixed order.  Positions are taken in blocks of up to 16384, one block
// after the other (so every row of dwte receives its blocks' sums in block
// order); within a block, all deterministic:
//  1. the keys (id << shift | position) are sorted by rank (enc_rank_kernel):
//     equal ids end up adjacent, in increasing position order;
//  2. one workgroup per chunk of 16 sorted entries sums each run of equal ids
//     in order.  A run that neither continues from the previous chunk nor into
//     the next one is complete and is added into dwte by that workgroup;
//     otherwise the piece goes to workspace (a run continuing from the
//     previous chunk is a "head" piece, one that starts here and continues is
//     a "tail" piece);
//  3. for every tail piece, one workgroup adds the head pieces of the
//     following chunks that continue the run, in chunk order, and adds the
//     total into dwte.
// Rows are split over the threads by float4 column, and each thread requests
// every row it needs (up to 16) before adding any: a chunk costs one round
// trip to memory, not one per entry.  The loads are unconditional (a skipped
// entry reads a row that another load of the same thread reads anyway), since
// a load under a branch is waited for before the branch closes.
constexpr int ENC_CHUNK = 16;
constexpr int ENC_SORT_MAX = 16384;

// Keys (id << shift | position) are distinct, so a key's place in sorted
// order is the number of keys below it.  Each workgroup stages all keys in LDS
// and ranks 64 of them: lane l of wave w counts the keys below key
// 64 * blockIdx.x + l among the w-th sixteenth of the keys (every lane of a
// wave reads the same LDS words), and the 16 partial counts are added.
constexpr int ENC_RANK_WAVES = 16;
__global__ __launch_bounds__(64 * ENC_RANK_WAVES) void enc_rank_kernel(unsigned* __restrict__ sorted,
                                                                       const int* __restrict__ tok, int BT, int shift) {
    constexpr int NT = 64 * ENC_RANK_WAVES, NWV = ENC_RANK_WAVES;
    __shared__ __attribute__((aligned(16))) unsigned keys[ENC_SORT_MAX];
    __shared__ int part[NWV][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n4 = (BT + 3) & ~3;
    // staged 16 ids per thread at a time: all loads issued before the stores
    for (int j0 = 0; j0 < n4; j0 += NT * 16) {
        unsigned k[16];
#pragma unroll
        for (int u = 0; u < 16; u++) {
            const int j = j0 + NT * u + threadIdx.x;
            // the load is used unconditionally (masked, not selected), so
            // the 16 loads overlap instead of each waiting under a branch
            const unsigned t = (unsigned)tok[min(j, BT - 1)];
            k[u] = (t << shift) | (unsigned)j | (j < BT ? 0u : 0xffffffffu);
        }
#pragma unroll
        for (int u = 0; u < 16; u++) {
            const int j = j0 + NT * u + threadIdx.x;
            if (j < n4) keys[j] = k[u];
        }
    }
    __syncthreads();
    const int i = blockIdx.x * 64 + lane;
    const unsigned ki = i < BT ? keys[i] : 0u;
    const int W = n4 / 4;  // 16-byte words of keys, split into NWV parts
    const int j0 = 4 * (wave * W / NWV), j1 = 4 * ((wave + 1) * W / NWV);
    int cnt = 0;
#pragma unroll 8
    for (int j = j0; j < j1; j += 4) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(&keys[j]);
        cnt += (k4.x < ki) + (k4.y < ki) + (k4.z < ki) + (k4.w < ki);
    }
    part[wave][lane] = cnt;
    __syncthreads();
    if (wave == 0 && i < BT) {
        int r = 0;
#pragma unroll
        for (int w = 0; w < NWV; w++) r += part[w][lane];
        sorted[r] = ki;
    }
}

// One workgroup per chunk c of sorted entries e0 .. e0 + n - 1.
__global__ __launch_bounds__(256) void enc_chunk_kernel(float* __restrict__ dwte, float* __restrict__ headws,
                                                        float* __restrict__ tailws, int* __restrict__ meta,
                                                        const float* __restrict__ dres,
                                                        const unsigned* __restrict__ sorted, int BT, int C,
                                                        int shift) {
    const int c = blockIdx.x;
    const int e0 = c * ENC_CHUNK, n = min(ENC_CHUNK, BT - e0);
    const unsigned pmask = (1u << shift) - 1u;
    const int prev = e0 > 0 ? (int)(sorted[e0 - 1] >> shift) : -1;
    const int next = e0 + n < BT ? (int)(sorted[e0 + n] >> shift) : -1;
    unsigned key[ENC_CHUNK];
    int tk[ENC_CHUNK];
#pragma unroll
    for (int i = 0; i < ENC_CHUNK; i++) {
        key[i] = i < n ? sorted[e0 + i] : 0u;
        tk[i] = i < n ? (int)(key[i] >> shift) : -2;
    }
    // entry i closes a run when the next entry holds another id; the run's
    // piece is a head (continues from the previous chunk), a tail (continues
    // into the next chunk) or complete
    const int nvec = C / 4;
    for (int vv = threadIdx.x; vv < nvec; vv += blockDim.x) {
        float x[ENC_CHUNK][4], w[ENC_CHUNK][4];
        int run_start = 0;
#pragma unroll
        for (int i = 0; i < ENC_CHUNK; i++) {
            // entries past n re-read entry n - 1's rows; w[i] is the id's
            // current gradient row, used where entry i closes a complete run
            const int ii = min(i, n - 1);
            load4<float>(dres + (long)(key[ii] & pmask) * C + vv * 4, x[i]);
            load4<float>(dwte + (long)tk[ii] * C + vv * 4, w[i]);
        }
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < ENC_CHUNK; i++) {
            if (i < n) {
#pragma unroll
                for (int q = 0; q < 4; q++) acc[q] += x[i][q];
                const bool last = i == n - 1;
                const bool end = last || tk[i + (i + 1 < ENC_CHUNK ? 1 : 0)] != tk[i];
                if (end) {
                    const bool head = run_start == 0 && prev == tk[i];
                    const bool tail = last && next == tk[i];
                    float o[4];
                    float* dst;
                    if (!head && !tail) {
#pragma unroll
                        for (int q = 0; q < 4; q++) o[q] = w[i][q] + acc[q];
                        dst = dwte + (long)tk[i] * C;
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; q++) o[q] = 0.f + acc[q];
                        dst = (head ? headws : tailws) + (long)c * C;
                    }
                    store4<float>(dst + vv * 4, o);
#pragma unroll
                    for (int q = 0; q < 4; q++) acc[q] = 0.f;
                    run_start = i + 1;
                }
            }
        }
    }
    if (threadIdx.x == 0) {
        // the chunk's head piece (and whether it also runs into the next
        // chunk), and the id of its tail piece
        int head_tok = -1, head_cont = 0, tail_tok = -1;
        if (prev == tk[0]) {
            head_tok = tk[0];
            head_cont = (tk[n - 1] == tk[0] && next == tk[0]) ? 1 : 0;
        }
        if (next == tk[n - 1] && !(head_cont && tk[n - 1] == head_tok)) tail_tok = tk[n - 1];
        meta[3 * c + 0] = head_tok;
        meta[3 * c + 1] = head_cont;
        meta[3 * c + 2] = tail_tok;
    }
}

// One workgroup per chunk c with a tail piece of id v: the run continues as
// the head pieces of chunks c+1 .. cl, where cl holds v's last entry (found by
// a binary search over the sorted keys); those pieces are added in chunk
// order, each thread requesting 16 of them before adding.
__global__ __launch_bounds__(256) void enc_fix_kernel(float* __restrict__ dwte, const float* __restrict__ headws,
                                                      const float* __restrict__ tailws, const int* __restrict__ meta,
                                                      const unsigned* __restrict__ sorted, int BT, int shift, int C) {
    constexpr int NB = 16;
    const int c = blockIdx.x;
    const int v = meta[3 * c + 2];
    if (v < 0) return;
    // first index with a key above every key of v
    const unsigned lim = ((unsigned)(v + 1)) << shift;
    int lo = (c + 1) * ENC_CHUNK, hi = BT;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sorted[mid] < lim) lo = mid + 1;
        else hi = mid;
    }
    const int cl = (lo - 1) / ENC_CHUNK;
    const int nvec = C / 4;
    for (int vv = threadIdx.x; vv < nvec; vv += blockDim.x) {
        float acc[4], o[4];
        load4<float>(tailws + (long)c * C + vv * 4, acc);
        load4<float>(dwte + (long)v * C + vv * 4, o);
        for (int c2 = c + 1; c2 <= cl; c2 += NB) {
            float h[NB][4];
#pragma unroll
            for (int u = 0; u < NB; u++)  // past cl: re-read piece cl (unused)
                load4<float>(headws + (long)min(c2 + u, cl) * C + vv * 4, h[u]);
#pragma unroll
            for (int u = 0; u < NB; u++)
                if (c2 + u <= cl)
#pragma unroll
                    for (int q = 0; q < 4; q++) acc[q] += h[u][q];
        }
#pragma unroll
        for (int q = 0; q < 4; q++) o[q] += acc[q];
        store4<float>(dwte + (long)v * C + vv * 4, o);
    }
}

// dwpe[t, :] += sum over b of dres[b*T + t, :]  (b in increasing order)
__global__ void encoder_bwd_wpe_kernel(float* __restrict__ dwpe, const float* __restrict__ dres, int B, int T_, int C) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index over T*C
    if (i >= (long)T_ * C / 4) return;
    const long t = i / (C / 4), c = (i % (C / 4)) * 4;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < B; b++) {
        float x[4];
        load4<float>(dres + ((long)b * T_ + t) * C + c, x);
#pragma unroll
        for (int e = 0; e < 4; e++) s[e] += x[e];
    }
    float o[4];
    load4<float>(dwpe + t * C + c, o);
#pragma unroll
    for (int e = 0; e < 4; e++) o[e] += s[e];
    store4<float>(dwpe + t * C + c, o);
}

// The logits row is read once and its gradient written once: non-temporal
// accesses (400 -> 363 us per 8192 x 50304 bf16 launch inside the step).
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
DEV uint4 ld16_stream(const void* p) {
    const u32x4_nt t = __builtin_nontemporal_load((const u32x4_nt*)p);
    return make_uint4(t.x, t.y, t.z, t.w);
}
DEV void st16_stream(void* p, const uint4& v) {
    const u32x4_nt t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, (u32x4_nt*)p);
}

// ---------------------------------------------------- softmax + cross-ent. --
// train_gpt2.cu, fused_classifier_kernel3 and prepare_softmax_blockwide:
// one workgroup per row.  The row (Vp logits) is read once into registers;
// block-wide max and sum of exp over the first V columns give
// lse = max + log(sum); loss = lse - z[target]; the row is overwritten in
// place with softmax - onehot for columns < V and with 0 for the padded
// columns.  The loss-gradient scale is applied later, by the classifier's
// backward products.  Columns >= V are set to -inf in registers right after
// the load, so every pass treats all elements alike (exp2(-inf) = 0 both in
// the sum and in the written gradient).  Each element's exponential is taken
// once, exp2(z log2(e) - max log2(e)) (one FMA and the hardware exp2), summed,
// and kept in the row's registers (in the row's precision) for the write,
// which scales it by 1/sum.
template <typename T, int NT, int NV>
__global__ __launch_bounds__(NT, NT == 512 ? 4 : 2) void classifier_ce_kernel(T* __restrict__ logits, float* __restrict__ losses,
                                                           const int* __restrict__ targets, int V, int Vp,
                                                           int* __restrict__ flag) {
    constexpr int VEC = VecT<T>::N;
    constexpr int NW = NT / 64;
    constexpr float L2E = 1.4426950408889634f;
    __shared__ float red[NW];
    __shared__ float zt_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long row = blockIdx.x;
    T* z = logits + row * Vp;
    int tgt = targets[row];
    if (tgt < 0 || tgt >= V) {
        if (tid == 0) flag[0] = 1;
        tgt = 0;
    }
    if (tid == 0) zt_s = to_f<T>(z[tgt]);
    const int nvec = Vp / VEC;
    uint4 reg[NV];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int v = tid + NT * k;
        if (v < nvec) {
            reg[k] = ld16_stream(z + (long)v * VEC);
            float f[VEC];
            unpack16<T>(reg[k], f);
            if ((v + 1) * VEC > V) {
#pragma unroll
                for (int e = 0; e < VEC; e++)
                    if (v * VEC + e >= V) f[e] = -INFINITY;
                reg[k] = pack16<T>(f);
            }
#pragma unroll
            for (int e = 0; e < VEC; e++) mx = fmaxf(mx, f[e]);
        }
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < NW; w++) mx = fmaxf(mx, red[w]);
    const float mc = -mx * L2E;
    float sm = 0.f;
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int v = tid + NT * k;
        if (v < nvec) {
            float f[VEC];
            unpack16<T>(reg[k], f);
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                f[e] = __builtin_amdgcn_exp2f(fmaf(f[e], L2E, mc));
                sm += f[e];
            }
            reg[k] = pack16<T>(f);  // the row now holds exp(z - max)
        }
    }
    sm = wave_sum(sm);
    __syncthreads();  // everyone has read red[] (max)
    if (lane == 0) red[wave] = sm;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) tot += red[w];
    const float lse = mx + __logf(tot);
    if (tid == 0) losses[row] = lse - zt_s;
    const float inv = 1.0f / tot;
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int v = tid + NT * k;
        if (v < nvec) {
            float f[VEC];
            unpack16<T>(reg[k], f);
#pragma unroll
            for (int e = 0; e < VEC; e++) f[e] *= inv;
            st16_stream(z + (long)v * VEC, pack16<T>(f));
        }
    }
    // the target column: softmax - 1, from the same exponential (recomputed
    // from the target logit exactly as the sum pass took it), stored by the
    // thread that stored its vector, after it
    if (tid == (tgt / VEC) % NT) {
        const float et = to_f<T>(from_f<T>(__builtin_amdgcn_exp2f(fmaf(zt_s, L2E, mc))));
        __builtin_nontemporal_store(from_f<T>(et * inv - 1.0f), z + tgt);
    }
}

// out[0] = mean of x[0..n): fixed-order reduction in one workgroup
__global__ __launch_bounds__(1024) void mean_kernel(float* __restrict__ out, const float* __restrict__ x, int n) {
    __shared__ float red[16];
    float s = 0.f;
    for (int i = threadIdx.x; i < n; i += 1024) s += x[i];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int w = 0; w < 16; w++) t += red[w];
        out[0] = t / (float)n;
    }
}

// ------------------------------------------------------------------ AdamW ---
// train_gpt2.cu, adamw_kernel3 (master-weight path) and gpt2_update's bias
// corrections c1 = 1 - beta1^t, c2 = 1 - beta2^t.  Four parameters per thread.
template <typename PT>
DEV void adamw_one(float g, float& m, float& v, float& p, float lr, float b1, float b2, float c1, float c2,
                   float eps, float wd) {
    m = fmaf(b1, m, fmaf(-b1, g, g));          // b1*m + (1-b1)*g
    v = fmaf(b2, v, fmaf(-b2, g * g, g * g));  // b2*v + (1-b2)*g^2
    const float mh = m / c1, vh = v / c2;
    p = p - lr * (mh / (sqrtf(vh) + eps) + wd * p);
}

// Each optimizer element is read and written once per step: non-temporal
// accesses keep these streams from displacing other data in the caches
// (AdamW over the 124M parameters: 680 -> 629 us, and 601 us with one
// workgroup per 1024 parameters instead of a grid-stride loop).
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
DEV void load4_stream(const float* p, float* x) {
    const f32x4_nt t = __builtin_nontemporal_load((const f32x4_nt*)p);
    x[0] = t.x;
    x[1] = t.y;
    x[2] = t.z;
    x[3] = t.w;
}
DEV void store4_stream(float* p, const float* x) {
    const f32x4_nt t = {x[0], x[1], x[2], x[3]};
    __builtin_nontemporal_store(t, (f32x4_nt*)p);
}

template <typename PT>
__global__ void adamw_kernel(PT* __restrict__ params, float* __restrict__ master, const float* __restrict__ grads,
                             float* __restrict__ mom, float* __restrict__ var, size_t n, float lr, float b1, float b2,
                             float c1, float c2, float eps, float wd) {
    const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
        if (i + 4 <= n) {
            float g[4], m[4], v[4], p[4];
            load4_stream(grads + i, g);
            load4_stream(mom + i, m);
            load4_stream(var + i, v);
            if constexpr (sizeof(PT) == 2) load4_stream(master + i, p);
            else load4<float>((const float*)params + i, p);
#pragma unroll
            for (int e = 0; e < 4; e++) adamw_one<PT>(g[e], m[e], v[e], p[e], lr, b1, b2, c1, c2, eps, wd);
            store4_stream(mom + i, m);
            store4_stream(var + i, v);
            if constexpr (sizeof(PT) == 2) {
                store4_stream(master + i, p);
                store4<bf16_t>((bf16_t*)params + i, p);
            } else {
                store4<float>((float*)params + i, p);
            }
        } else {
            for (size_t k = i; k < n; k++) {
                float g = grads[k], m = mom[k], v = var[k];
                float p = (sizeof(PT) == 2) ? master[k] : (float)((const float*)params)[k];
                adamw_one<PT>(g, m, v, p, lr, b1, b2, c1, c2, eps, wd);
                mom[k] = m;
                var[k] = v;
                if constexpr (sizeof(PT) == 2) {
                    master[k] = p;
                    ((bf16_t*)params)[k] = f2bf(p);
                } else {
                    ((float*)params)[k] = p;
                }
            }
        }
    }
}

// train_gpt2.cu, adamw_kernel3 without master weights: the bf16 parameter is
// updated in fp32 and rounded back to bf16 stochastically.
//
// SquirrelNoise5 (Squirrel Eiserloh's published noise function, version 5):
// position times a constant, plus the seed, then alternating xor-shifts and
// constant additions / multiplications.
DEV uint32_t squirrel5(uint32_t pos, uint32_t seed) {
    uint32_t x = pos * 0xd2a80a3fu + seed;
    x ^= x >> 9;
    x += 0xa884f197u;
    x ^= x >> 11;
    x *= 0x6c736f4bu;
    x ^= x >> 13;
    x += 0xb79f3abbu;
    x ^= x >> 15;
    x *= 0x1b56c4f5u;
    x ^= x >> 17;
    return x;
}

// One parameter, in the page's order of fp32 operations, none contracted
// beyond the explicit fused multiply-adds of the moment updates.
DEV bf16_t adamw_sr_one(uint32_t i, uint16_t p16, float g, float& m, float& v, float lr, float b1, float b2,
                        float c1, float c2, float eps, float wd, uint32_t seed) {
#pragma clang fp contract(off)
    m = fmaf(b1, m, fmaf(-b1, g, g));
    const float g2 = g * g;
    v = fmaf(b2, v, fmaf(-b2, g2, g2));
    const float mh = m / c1, vh = v / c2;
    const float old = bf2f(p16);
    const float den = sqrtf(vh) + eps;
    const float step = mh / den + wd * old;
    const float x = old - lr * step;
    // noise of the page's 512-thread launch position (i mod 512, i div 512)
    const uint32_t pos = (i & 511u) + 198491317u * (i >> 9);
    const uint32_t r = squirrel5(pos, squirrel5(pos, seed)) & 0xffffu;
    uint32_t bits = __float_as_uint(x);
    bits = (bits & 0xffffu) > r ? (bits | 0xffffu) : (bits & 0xffff0000u);
    return f2bf(__uint_as_float(bits));
}

__global__ void adamw_sr_kernel(bf16_t* __restrict__ params, const float* __restrict__ grads,
                                float* __restrict__ mom, float* __restrict__ var, size_t n, float lr, float b1,
                                float b2, float c1, float c2, float eps, float wd, uint32_t seed) {
    const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
        if (i + 4 <= n) {
            float g[4], m[4], v[4];
            load4_stream(grads + i, g);
            load4_stream(mom + i, m);
            load4_stream(var + i, v);
            const uint2 pv = ld8(params + i);
            const uint16_t pin[4] = {(uint16_t)(pv.x & 0xffffu), (uint16_t)(pv.x >> 16), (uint16_t)(pv.y & 0xffffu),
                                     (uint16_t)(pv.y >> 16)};
            uint16_t pout[4];
#pragma unroll
            for (int e = 0; e < 4; e++)
                pout[e] = adamw_sr_one((uint32_t)(i + e), pin[e], g[e], m[e], v[e], lr, b1, b2, c1, c2, eps, wd, seed);
            store4_stream(mom + i, m);
            store4_stream(var + i, v);
            st8(params + i, make_uint2(pout[0] | ((uint32_t)pout[1] << 16), pout[2] | ((uint32_t)pout[3] << 16)));
        } else {
            for (size_t k = i; k < n; k++) {
                float m = mom[k], v = var[k];
                params[k] = adamw_sr_one((uint32_t)k, params[k], grads[k], m, v, lr, b1, b2, c1, c2, eps, wd, seed);
                mom[k] = m;
                var[k] = v;
            }
        }
    }
}

__global__ void fill_f32_kernel(float* __restrict__ p, float value, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
        if (i + 4 <= n) *reinterpret_cast<float4*>(p + i) = make_float4(value, value, value, value);
        else for (size_t k = i; k < n; k++) p[k] = value;
    }
}

__global__ void fill_i32_kernel(int* __restrict__ p, int value, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

__global__ void cast_bf16_kernel(bf16_t* __restrict__ dst, const float* __restrict__ src, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
        if (i + 4 <= n) {
            float f[4];
            load4<float>(src + i, f);
            store4<bf16_t>(dst + i, f);
        } else {
            for (size_t k = i; k < n; k++) dst[k] = f2bf(src[k]);
        }
    }
}

unsigned grid_for(size_t n4) {  // grid-stride launches: at most 8 blocks of 256 per CU slot
    size_t b = (n4 + 255) / 256;
    if (b > 65536) b = 65536;
    return (unsigned)(b ? b : 1);
}

}  // namespace

template <typename T>
int encoder_fwd_launch(T* out, int* tok_copy, const int* tok, const T* wte, const T* wpe, int B, int T_, int C,
                       int V, int* flag, hipStream_t s) {
    const long n = (long)B * T_ * (C / VecT<T>::N);
    if (n == 0) return 0;
    hipLaunchKernelGGL(encoder_fwd_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, out, tok_copy, tok,
                       wte, wpe, B * T_, T_, C, V, flag);
    return (int)hipGetLastError();
}

size_t encoder_bwd_workspace_bytes(int BT, int C) {
    const int nb = BT < ENC_SORT_MAX ? BT : ENC_SORT_MAX;  // positions per block
    const size_t nch = (nb + ENC_CHUNK - 1) / ENC_CHUNK;
    return ((size_t)nb * 4 + 255) / 256 * 256 + (nch * 12 + 255) / 256 * 256 + 2 * nch * C * 4;
}

int encoder_bwd_launch(float* dwte, float* dwpe, const float* dres, const int* tok, int B, int T_, int C,
                       void* work, hipStream_t s) {
    const long BT = (long)B * T_;
    if (BT == 0) return 0;
    if (work == nullptr) return (int)hipErrorInvalidValue;
    for (long p0 = 0; p0 < BT; p0 += ENC_SORT_MAX) {
        const int nb = (int)std::min<long>(ENC_SORT_MAX, BT - p0);
        int shift = 0;
        while ((1 << shift) < nb) shift++;
        const int nch = (nb + ENC_CHUNK - 1) / ENC_CHUNK;
        char* w = (char*)work;
        unsigned* sorted = (unsigned*)w;
        w += ((size_t)nb * 4 + 255) / 256 * 256;
        int* meta = (int*)w;
        w += ((size_t)nch * 12 + 255) / 256 * 256;
        float* headws = (float*)w;
        float* tailws = headws + (size_t)nch * C;
        const float* dr = dres + p0 * C;
        const int* tk = tok + p0;
        hipLaunchKernelGGL(enc_rank_kernel, dim3((nb + 63) / 64), dim3(64 * ENC_RANK_WAVES), 0, s, sorted, tk, nb,
                           shift);
        const int thr = std::min(256, (C / 4 + 63) / 64 * 64);
        hipLaunchKernelGGL(enc_chunk_kernel, dim3(nch), dim3(thr), 0, s, dwte, headws, tailws, meta, dr, sorted, nb, C,
                           shift);
        hipLaunchKernelGGL(enc_fix_kernel, dim3(nch), dim3(thr), 0, s, dwte, headws, tailws, meta, sorted, nb, shift,
                           C);
    }
    const long n4 = (long)T_ * C / 4;
    hipLaunchKernelGGL(encoder_bwd_wpe_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dwpe, dres, B, T_, C);
    return (int)hipGetLastError();
}

template <typename T>
int classifier_ce_launch(T* logits, float* losses, const int* targets, int N, int V, int Vp, int* flag, hipStream_t s) {
    if (N == 0) return 0;
    if constexpr (sizeof(T) == 2) {
        hipLaunchKernelGGL((classifier_ce_kernel<T, 512, 13>), dim3(N), dim3(512), 0, s, logits, losses, targets, V, Vp, flag);
    } else {
        hipLaunchKernelGGL((classifier_ce_kernel<T, 1024, 13>), dim3(N), dim3(1024), 0, s, logits, losses, targets, V, Vp, flag);
    }
    return (int)hipGetLastError();
}

int mean_launch(float* out, const float* x, int n, hipStream_t s) {
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, out, x, n);
    return (int)hipGetLastError();
}

template <typename PT>
int adamw_launch(PT* params, float* master, const float* grads, float* m, float* v, size_t n, float lr, float b1,
                 float b2, float c1, float c2, float eps, float wd, hipStream_t s) {
    if (n == 0) return 0;
    const size_t blocks = ((n + 3) / 4 + 255) / 256;  // one pass: 4 parameters per thread
    if (blocks > 0x7fffffffu) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(adamw_kernel<PT>, dim3((unsigned)blocks), dim3(256), 0, s, params, master, grads, m, v, n,
                       lr, b1, b2, c1, c2, eps, wd);
    return (int)hipGetLastError();
}

int adamw_sr_launch(bf16_t* params, const float* grads, float* m, float* v, size_t n, float lr, float b1, float b2,
                    float c1, float c2, float eps, float wd, uint32_t seed, hipStream_t s) {
    if (n == 0) return 0;
    const size_t blocks = ((n + 3) / 4 + 255) / 256;  // one pass: 4 parameters per thread
    if (blocks > 0x7fffffffu) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(adamw_sr_kernel, dim3((unsigned)blocks), dim3(256), 0, s, params, grads, m, v, n, lr, b1, b2,
                       c1, c2, eps, wd, seed);
    return (int)hipGetLastError();
}

int fill_f32_launch(float* p, float value, size_t n, hipStream_t s) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for((n + 3) / 4)), dim3(256), 0, s, p, value, n);
    return (int)hipGetLastError();
}

int fill_i32_launch(int* p, int value, size_t n, hipStream_t s) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, value, n);
    return (int)hipGetLastError();
}

int cast_f32_to_bf16_launch(bf16_t* dst, const float* src, size_t n, hipStream_t s) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for((n + 3) / 4)), dim3(256), 0, s, dst, src, n);
    return (int)hipGetLastError();
}

template int encoder_fwd_launch<float>(float*, int*, const int*, const float*, const float*, int, int, int, int, int*, hipStream_t);
template int encoder_fwd_launch<bf16_t>(bf16_t*, int*, const int*, const bf16_t*, const bf16_t*, int, int, int, int, int*, hipStream_t);
template int classifier_ce_launch<float>(float*, float*, const int*, int, int, int, int*, hipStream_t);
template int classifier_ce_launch<bf16_t>(bf16_t*, float*, const int*, int, int, int, int*, hipStream_t);
template int adamw_launch<float>(float*, float*, const float*, float*, float*, size_t, float, float, float, float, float, float, float, hipStream_t);
template int adamw_launch<bf16_t>(bf16_t*, float*, const float*, float*, float*, size_t, float, float, float, float, float, float, float, hipStream_t);
