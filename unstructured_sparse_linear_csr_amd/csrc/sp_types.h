// Element types of the dense operands and sparse values, and the vectors the
// kernels gather them in.  fp32 is the card's precision; fp16 and bf16 are
// the mixed-precision inputs (16-bit storage, fp32 arithmetic and
// accumulation): every element is widened to fp32 exactly when used, and a
// product of two 16-bit elements is exact in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spk {

// bfloat16 carried as its raw bits: the upper half of an fp32.
struct bf16 {
    unsigned short bits;
};

enum class Dtype { f32 = 0, f16 = 1, bf16 = 2 };

template <typename E> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ float f32(float v) { return v; }
};
template <> struct Elem<_Float16> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float f32(_Float16 v) { return (float)v; }
    // the two elements of a dword, element 0 in the low half
    static __device__ __forceinline__ float lo(unsigned u)
    {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
    }
    static __device__ __forceinline__ float hi(unsigned u)
    {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16));
    }
};
template <> struct Elem<bf16> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float f32(bf16 v)
    {
        return __uint_as_float((unsigned)v.bits << 16);
    }
    static __device__ __forceinline__ float lo(unsigned u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float hi(unsigned u)
    {
        return __uint_as_float(u & 0xffff0000u);
    }
};

// A vector of kVec consecutive elements of type E as one load: 16 bytes
// (4 fp32 or 8 16-bit elements) or a single element.  T is the raw register
// form; to_f32 widens it, fma multiplies it by a scalar into kVec fp32
// accumulators (element order 0, 1, ...), fma2 adds the products of two
// scalars with two vectors (a0 * b0, then a1 * b1), dot adds the dot product
// of two vectors to an fp32 sum, store writes kVec fp32 results.
template <typename E, int kVec> struct GVec;

template <> struct GVec<float, 4> {
    using T = float4;
    static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    static __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
        return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]),
                           __uint_as_float(v[2]), __uint_as_float(v[3]));
    }
    static __device__ __forceinline__ T load(const float *p)
    {
        return *reinterpret_cast<const float4 *>(p);
    }
    static __device__ __forceinline__ void to_f32(const T &b, float *f)
    {
        f[0] = b.x;
        f[1] = b.y;
        f[2] = b.z;
        f[3] = b.w;
    }
    static __device__ __forceinline__ void fma(float a, const T &b, float *acc)
    {
        acc[0] = fmaf(a, b.x, acc[0]);
        acc[1] = fmaf(a, b.y, acc[1]);
        acc[2] = fmaf(a, b.z, acc[2]);
        acc[3] = fmaf(a, b.w, acc[3]);
    }
    static __device__ __forceinline__ void fma2(float a0, float a1, const T &b0, const T &b1,
                                                float *acc)
    {
        fma(a0, b0, acc);
        fma(a1, b1, acc);
    }
    // element order 0 ... 3, one FMA each
    static __device__ __forceinline__ float dot(const T &x, const T &y, float acc)
    {
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        return fmaf(x.w, y.w, acc);
    }
    static __device__ __forceinline__ void store(float *dst, const float *acc)
    {
        *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
};

template <> struct GVec<float, 1> {
    using T = float;
    static __device__ __forceinline__ T zero() { return 0.f; }
    static __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ T load(const float *p) { return *p; }
    static __device__ __forceinline__ void to_f32(const T &b, float *f) { f[0] = b; }
    static __device__ __forceinline__ void fma(float a, const T &b, float *acc)
    {
        acc[0] = fmaf(a, b, acc[0]);
    }
    static __device__ __forceinline__ void fma2(float a0, float a1, const T &b0, const T &b1,
                                                float *acc)
    {
        fma(a0, b0, acc);
        fma(a1, b1, acc);
    }
    static __device__ __forceinline__ float dot(const T &x, const T &y, float acc)
    {
        return fmaf(x, y, acc);
    }
    static __device__ __forceinline__ void store(float *dst, const float *acc) { *dst = acc[0]; }
};

// Eight 16-bit elements in one 16-byte load.
template <typename E> struct GVec16x8 {
    using T = uint4;
    static __device__ __forceinline__ T zero() { return make_uint4(0u, 0u, 0u, 0u); }
    static __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
        return make_uint4(v[0], v[1], v[2], v[3]);
    }
    static __device__ __forceinline__ T load(const E *p)
    {
        return *reinterpret_cast<const uint4 *>(p);
    }
    static __device__ __forceinline__ void to_f32(const T &b, float *f)
    {
        const unsigned w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = Elem<E>::lo(w[i]);
            f[2 * i + 1] = Elem<E>::hi(w[i]);
        }
    }
    static __device__ __forceinline__ void fma(float a, const T &b, float *acc)
    {
        float f[8];
        to_f32(b, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(a, f[i], acc[i]);
    }
    // fp16: a0 * b0, then a1 * b1, one FMA per element (v_fma_mix_f32).  bf16
    // (a0 and a1 are widened bf16 values): for each column, the two products
    // a0 * b0[j] + a1 * b1[j], both exact in fp32, are added to the sum by one
    // v_dot2c_f32_bf16 (the two entries' elements paired by a byte permute)
    // instead of a shift or mask plus an FMA per element.
    static __device__ __forceinline__ void fma2(float a0, float a1, const T &b0, const T &b1,
                                                float *acc)
    {
        if constexpr (__is_same(E, bf16)) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            // v_perm_b32 selectors over the byte string (second operand:
            // bytes 0-3, first operand: bytes 4-7): the low halves of both
            // words, or their high halves, as one (low, high) pair
            constexpr unsigned kLoHalves = 0x05040100u, kHiHalves = 0x07060302u;
            const bf16x2 a = __builtin_bit_cast(
                bf16x2, __builtin_amdgcn_perm(__float_as_uint(a1), __float_as_uint(a0), kHiHalves));
            const unsigned w0[4] = {b0.x, b0.y, b0.z, b0.w};
            const unsigned w1[4] = {b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned lo = __builtin_amdgcn_perm(w1[i], w0[i], kLoHalves);
                const unsigned hi = __builtin_amdgcn_perm(w1[i], w0[i], kHiHalves);
                acc[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(
                    a, __builtin_bit_cast(bf16x2, lo), acc[2 * i], false);
                acc[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                    a, __builtin_bit_cast(bf16x2, hi), acc[2 * i + 1], false);
            }
        } else {
            fma(a0, b0, acc);
            fma(a1, b1, acc);
        }
    }
    // gfx950's v_dot2c_f32_bf16 / v_dot2c_f32_f16 add the two exact products
    // of elements (0, 1), then (2, 3), ... to the sum: one instruction per pair
    // (bf16: instead of a shift or mask plus an FMA per element; fp16: instead
    // of one v_fma_mix_f32 per element).  fp16 subnormal operands enter the
    // products unflushed (tested).
    static __device__ __forceinline__ float dot(const T &x, const T &y, float acc)
    {
        const unsigned xw[4] = {x.x, x.y, x.z, x.w};
        const unsigned yw[4] = {y.x, y.y, y.z, y.w};
        if constexpr (__is_same(E, bf16)) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xw[i]),
                                                      __builtin_bit_cast(bf16x2, yw[i]), acc,
                                                      false);
        } else {
            typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, xw[i]),
                                             __builtin_bit_cast(f16x2, yw[i]), acc, false);
        }
        return acc;
    }
    static __device__ __forceinline__ void store(float *dst, const float *acc)
    {
        reinterpret_cast<float4 *>(dst)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        reinterpret_cast<float4 *>(dst)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
};
template <> struct GVec<_Float16, 8> : GVec16x8<_Float16> {};
template <> struct GVec<bf16, 8> : GVec16x8<bf16> {};

// One 16-bit element.
template <typename E> struct GVec16x1 {
    using T = unsigned short;
    static __device__ __forceinline__ T zero() { return 0; }
    static __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ T load(const E *p)
    {
        return *reinterpret_cast<const unsigned short *>(p);
    }
    static __device__ __forceinline__ void to_f32(const T &b, float *f)
    {
        f[0] = Elem<E>::lo((unsigned)b);
    }
    static __device__ __forceinline__ void fma(float a, const T &b, float *acc)
    {
        acc[0] = fmaf(a, Elem<E>::lo((unsigned)b), acc[0]);
    }
    static __device__ __forceinline__ void fma2(float a0, float a1, const T &b0, const T &b1,
                                                float *acc)
    {
        fma(a0, b0, acc);
        fma(a1, b1, acc);
    }
    static __device__ __forceinline__ float dot(const T &x, const T &y, float acc)
    {
        return fmaf(Elem<E>::lo((unsigned)x), Elem<E>::lo((unsigned)y), acc);
    }
    static __device__ __forceinline__ void store(float *dst, const float *acc) { *dst = acc[0]; }
};
template <> struct GVec<_Float16, 1> : GVec16x1<_Float16> {};
template <> struct GVec<bf16, 1> : GVec16x1<bf16> {};

// Four consecutive sparse values (a CSR segment) widened to fp32: one
// 16-byte load for fp32, 8 bytes for 16-bit types (4-element aligned).
template <typename E> __device__ __forceinline__ void load4_f32(const E *p, float *f);
template <> __device__ __forceinline__ void load4_f32<float>(const float *p, float *f)
{
    const float4 v = *reinterpret_cast<const float4 *>(p);
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
}
template <typename E> __device__ __forceinline__ void load4_f32(const E *p, float *f)
{
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    f[0] = Elem<E>::lo(v.x);
    f[1] = Elem<E>::hi(v.x);
    f[2] = Elem<E>::lo(v.y);
    f[3] = Elem<E>::hi(v.y);
}

// Loads kN consecutive elements of type E (kN * bytes <= 16) and widens them.
// (through a buffer resource; out-of-range offsets read as zeros)
template <typename E, int kN>
__device__ __forceinline__ void load_widen(__amdgpu_buffer_rsrc_t r, unsigned off, float *f)
{
    constexpr int kBytes = kN * (int)Elem<E>::kBytes;
    unsigned w[4];
    if constexpr (kBytes == 16) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
        w[0] = x[0], w[1] = x[1], w[2] = x[2], w[3] = x[3];
    } else if constexpr (kBytes == 8) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
        w[0] = x[0], w[1] = x[1];
    } else {
        static_assert(kBytes == 4, "4, 8 or 16 bytes");
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    if constexpr (__is_same(E, float)) {
#pragma unroll
        for (int i = 0; i < kN; ++i) f[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < kN / 2; ++i) {
            f[2 * i] = Elem<E>::lo(w[i]);
            f[2 * i + 1] = Elem<E>::hi(w[i]);
        }
    }
}

}  // namespace spk
