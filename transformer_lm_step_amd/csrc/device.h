// device.h - device-side building blocks shared by the gfx950 kernels.
//
// Element types: activations and parameters are either fp32 (`float`) or bf16
// stored as `uint16_t` (`bf16_t`).  All arithmetic is fp32.  Global memory is
// moved in 16-byte vectors (`uint4`): 4 fp32 or 8 bf16 elements.
//
// Matrix-core fragments: every product runs on 16x16 output tiles of the
// gfx950 MFMA unit with a 32-deep contraction per step.  A fragment is what
// one lane feeds into one such step: 8 contraction-consecutive elements of one
// row (A operand) or one column (B operand).  Lane l covers row/column l%16
// and contraction slots 8*(l/16) .. 8*(l/16)+7; the 16x16 fp32 result tile
// leaves lane l holding rows 4*(l/16)+r (r = 0..3) of column l%16.
//  - bf16: one v_mfma_f32_16x16x32_bf16 per step.
//  - fp32: eight v_mfma_f32_16x16x4f32 per step, the j-th consuming slot j of
//    every lane, so the 32 slots are contracted exactly once, in fp32.
// Because only the pairing of A and B slots matters, a fragment may map its
// 8 slots to any 8 distinct contraction indices as long as both operands use
// the same map (the attention kernels use this to feed a result tile straight
// back in as an operand).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

#define DEV __device__ __forceinline__

// ---------------------------------------------------------------- scalars ---

DEV float bf2f(uint32_t u16) { return __uint_as_float(u16 << 16); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
DEV uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f = {lo, hi};
    bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}
DEV bf16_t f2bf(float f) { return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xffffu); }

template <typename T> DEV float to_f(T v);
template <> DEV float to_f<float>(float v) { return v; }
template <> DEV float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> DEV T from_f(float v);
template <> DEV float from_f<float>(float v) { return v; }
template <> DEV bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// ---------------------------------------------------------------- vectors ---

template <typename T> struct VecT;
template <> struct VecT<float> { static constexpr int N = 4; };
template <> struct VecT<bf16_t> { static constexpr int N = 8; };

// unpack a 16-byte vector to VecT<T>::N floats
template <typename T> DEV void unpack16(const uint4& v, float* f);
template <> DEV void unpack16<float>(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
template <> DEV void unpack16<bf16_t>(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
template <typename T> DEV uint4 pack16(const float* f);
template <> DEV uint4 pack16<float>(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}
template <> DEV uint4 pack16<bf16_t>(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

DEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Raw buffer access (gfx9 buffer resource: base, byte range, dword data
// format).  A load whose byte offset falls outside [0, bytes) returns zeros.
typedef int v4i_t __attribute__((ext_vector_type(4)));
DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
DEV uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
constexpr uint32_t kBufOOB = 0x80000000u;  // an offset past any range used here
// Byte range of a buffer resource from the valid bytes past its base: clamped
// to [0, 2^31 - 1], so that it fits the 32-bit field and kBufOOB stays past
// it.  Operands larger than 2 GiB keep their full extent reachable, since
// every per-lane offset inside one staged slab is far below 2 GiB.
DEV uint32_t rsrc_range(long bytes) {
    return (uint32_t)(bytes < 0 ? 0L : bytes > 0x7fffffffL ? 0x7fffffffL : bytes);
}

// s_waitcnt immediate that waits until at most n vector memory operations of
// this wave are outstanding (LDS and export counters left at their maxima)
DEV constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// One 16-byte-per-lane buffer load into LDS at lds (wave-uniform; lane i
// lands at lds + 16 i).  Written as inline assembly so that the compiler does
// not track it: its own wait insertion cannot tell the stage buffers apart and
// would wait for every load in flight before each fragment read.  A kernel
// that uses it waits for these loads itself (vmcnt before the barrier of the
// stage that consumes them, and for all of them before its loop ends), and
// issues no other vector memory access while they are in flight: the
// compiler's own vmcnt waits do not count them and would also wait for them.
DEV void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, const void* lds) {
    const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
                 "s"(__builtin_amdgcn_readfirstlane(a))
                 : "memory", "m0");
}

// The buffer resource of an LDS-destination load must sit in scalar registers;
// built from readfirstlane'd fields it does even where the compiler holds the
// tile coordinates in vector registers (all lanes hold the same values).
DEV __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
    const uint64_t u = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}

// v if ok, else zeros (component-wise select, no branch and no memory)
DEV uint4 keep16(bool ok, const uint4& v) {
    const uint32_t m = ok ? 0xffffffffu : 0u;
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}
DEV void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
DEV uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
DEV void st8(void* p, const uint2& v) { *reinterpret_cast<uint2*>(p) = v; }

// store 4 consecutive values (8 bytes for bf16, 16 bytes for fp32)
template <typename T> DEV void store4(T* p, const float* f);
template <> DEV void store4<float>(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}
template <> DEV void store4<bf16_t>(bf16_t* p, const float* f) {
    st8(p, make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])));
}
template <typename T> DEV void load4(const T* p, float* f);
template <> DEV void load4<float>(const float* p, float* f) {
    float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
template <> DEV void load4<bf16_t>(const bf16_t* p, float* f) {
    uint2 v = ld8(p);
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
}

// ------------------------------------------------------------- reductions ---
// Cross-lane sums and maxima without a round trip through the LDS crossbar
// (where a shuffle goes): DPP row permutations -- mirror within 16 lanes,
// mirror within 8, then the two exchanges inside each group of 4 -- combine
// the lanes of a 16-lane row, and the gfx950 lane-swap instructions pair lane
// l with l ^ 16 and with l ^ 32.  In every step a lane and its partner combine
// the same two values (the swaps always put the lower lane's value first), so
// all lanes of a group end with the same bits.  Every lane of the wave must be
// active.

struct AddOp {
    DEV float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
    DEV float operator()(float a, float b) const { return fmaxf(a, b); }
};

template <int CTRL>
DEV float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141, kDppQuadXor1 = 0xb1, kDppQuadXor2 = 0x4e;

// op(v(l), v(l ^ 16)) and op(v(l), v(l ^ 32)), the lower lane's value first
template <typename Op>
DEV float xor16_combine(float v, Op op) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
DEV float xor32_combine(float v, Op op) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// op over each aligned group of LANES (16, 32 or 64) lanes
template <int LANES, typename Op>
DEV float lane_reduce(float v, Op op) {
    static_assert(LANES == 16 || LANES == 32 || LANES == 64, "groups of 16, 32 or 64 lanes");
    v = op(v, dpp_mov<kDppRowMirror>(v));
    v = op(v, dpp_mov<kDppRowHalfMirror>(v));
    v = op(v, dpp_mov<kDppQuadXor1>(v));
    v = op(v, dpp_mov<kDppQuadXor2>(v));
    if constexpr (LANES >= 32) v = xor16_combine(v, op);
    if constexpr (LANES == 64) v = xor32_combine(v, op);
    return v;
}

DEV float wave_sum(float v) { return lane_reduce<64>(v, AddOp()); }
DEV float wave_max(float v) { return lane_reduce<64>(v, MaxOp()); }

// -------------------------------------------------------------- fragments ---

template <typename T> struct Frag;
template <> struct Frag<bf16_t> { bf16x8_t v; };
template <> struct Frag<float> { float v[8]; };

DEV void mma(f32x4_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
DEV void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int j = 0; j < 8; j++) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// 8 consecutive elements from LDS (16-byte aligned)
DEV void frag_ld(Frag<bf16_t>& f, const bf16_t* p) {
    f.v = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}
DEV void frag_ld(Frag<float>& f, const float* p) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// slots 0..3 from p0, slots 4..7 from p1 (each 4 consecutive elements)
DEV void frag_ld2(Frag<bf16_t>& f, const bf16_t* p0, const bf16_t* p1) {
    uint2 a = *reinterpret_cast<const uint2*>(p0);
    uint2 b = *reinterpret_cast<const uint2*>(p1);
    f.v = __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}
DEV void frag_ld2(Frag<float>& f, const float* p0, const float* p1) {
    float4 a = *reinterpret_cast<const float4*>(p0);
    float4 b = *reinterpret_cast<const float4*>(p1);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// from 8 fp32 values held in registers
DEV void frag_from(Frag<bf16_t>& f, const float* x) {
    f.v = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                  pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
}
DEV void frag_from(Frag<float>& f, const float* x) {
#pragma unroll
    for (int j = 0; j < 8; j++) f.v[j] = x[j];
}
DEV void frag_zero(Frag<bf16_t>& f) { f.v = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0)); }
DEV void frag_zero(Frag<float>& f) {
#pragma unroll
    for (int j = 0; j < 8; j++) f.v[j] = 0.0f;
}
// 8 consecutive elements straight from global memory (16 B per bf16 fragment)
DEV void frag_gld(Frag<bf16_t>& f, const bf16_t* p) { frag_ld(f, p); }
DEV void frag_gld(Frag<float>& f, const float* p) { frag_ld(f, p); }

// ---------------------------------------------------------------- GELU ------
// train_gpt2.cu, gelu_forward_kernel2 / gelu_backward_kernel (tanh form).
#define GELU_K0 0.7978845608028654f  // sqrt(2/pi)
#define GELU_K1 0.044715f

// tanh for the GELU epilogues.  fp32 products use the library tanhf (1 ulp);
// bf16 products use tanh(u) = 1 - 2 / (exp(2u) + 1) with the hardware exp2
// and reciprocal, whose absolute error (a few ulp of 1) is far below bf16's
// resolution, and which saturates to +-1 for large |u|.
template <typename T>
DEV float tanh_f(float u) {
    if constexpr (sizeof(T) == 2) {
        const float e = __builtin_amdgcn_exp2f(u * 2.8853900817779268f);  // exp(2u)
        return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
    } else {
        return tanhf(u);
    }
}
template <typename T>
DEV float gelu_f(float x) {
    float u = GELU_K0 * (x + GELU_K1 * x * x * x);
    return 0.5f * x * (1.0f + tanh_f<T>(u));
}
template <typename T>
DEV float gelu_grad_f(float x) {
    float u = GELU_K0 * (x + GELU_K1 * x * x * x);
    float th = tanh_f<T>(u);
    float sech2 = 1.0f - th * th;  // 1/cosh^2(u)
    return 0.5f * (1.0f + th) + 0.5f * x * sech2 * GELU_K0 * (1.0f + 3.0f * GELU_K1 * x * x);
}

// ------------------------------------------------------------- transpose ----
// r[i] holds one 16-byte vector of row i (4 rows).  Writes, for every element
// e of the vector, the 4 values (r[0][e], r[1][e], r[2][e], r[3][e]) to
// dst + e*pitch (8 bytes for bf16, 16 bytes for fp32).
DEV uint32_t vec_h16(const uint4& v, int e) {
    uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
DEV uint32_t vec_w32(const uint4& v, int e) {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}
template <typename T>
DEV void store_t4(T* dst, int pitch, const uint4 (&r)[4]) {
#pragma unroll
    for (int e = 0; e < VecT<T>::N; e++) {
        if constexpr (sizeof(T) == 2) {
            st8(dst + e * pitch, make_uint2(vec_h16(r[0], e) | (vec_h16(r[1], e) << 16),
                                            vec_h16(r[2], e) | (vec_h16(r[3], e) << 16)));
        } else {
            st16(dst + e * pitch, make_uint4(vec_w32(r[0], e), vec_w32(r[1], e), vec_w32(r[2], e), vec_w32(r[3], e)));
        }
    }
}
