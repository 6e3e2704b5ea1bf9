// kda_device.h -- small device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_t;  // bfloat16 storage: the upper half of a float32

constexpr float kLog2e = 1.4426950408889634f;

// ---- bfloat16 conversion (round to nearest, ties to even) ----------------
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// by the hardware conversion (a NaN stays a quiet NaN); two values at a time
// pack into one 32-bit word with a single instruction
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, b2_t{(__bf16)a, (__bf16)b});
}

// ---- typed scalar load/store for the two storage types -------------------
template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void st(T* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// Two consecutive elements as floats (4-byte aligned for bf16, 8 for float).
template <typename T> __device__ __forceinline__ f32x2 ld2(const T* p);
template <> __device__ __forceinline__ f32x2 ld2<float>(const float* p)
{
    return *reinterpret_cast<const f32x2*>(p);
}
template <> __device__ __forceinline__ f32x2 ld2<bf16_t>(const bf16_t* p)
{
    uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    f32x2 r;
    r.x = __uint_as_float(u << 16);
    r.y = __uint_as_float(u & 0xffff0000u);
    return r;
}

// Four consecutive elements as floats (8-byte aligned for bf16, 16 for float).
template <typename T> __device__ __forceinline__ f32x4 ld4(const T* p);
template <> __device__ __forceinline__ f32x4 ld4<float>(const float* p)
{
    return *reinterpret_cast<const f32x4*>(p);
}
template <> __device__ __forceinline__ f32x4 ld4<bf16_t>(const bf16_t* p)
{
    uint2 u = *reinterpret_cast<const uint2*>(p);
    f32x4 r;
    r.x = __uint_as_float(u.x << 16);
    r.y = __uint_as_float(u.x & 0xffff0000u);
    r.z = __uint_as_float(u.y << 16);
    r.w = __uint_as_float(u.y & 0xffff0000u);
    return r;
}

template <typename T> __device__ __forceinline__ void st4(T* p, f32x4 v);
template <> __device__ __forceinline__ void st4<float>(float* p, f32x4 v)
{
    *reinterpret_cast<f32x4*>(p) = v;
}
template <> __device__ __forceinline__ void st4<bf16_t>(bf16_t* p, f32x4 v)
{
    uint2 u;
    u.x = pack_bf16x2(v.x, v.y);
    u.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<uint2*>(p) = u;
}

// ---- math --------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// ---------------------------------------------------------------- buffers
// Raw buffer over [base, base + bytes): loads beyond return 0, stores beyond
// are dropped (the descriptor's range check).
// Every descriptor built here is wave-uniform; readfirstlane states that to
// the compiler, which otherwise may build it in vector registers and wrap
// each load in a loop over the distinct values.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    const uint32_t nr = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)nr), 0x00020000);
}
// Workgroup barrier for LDS hand-offs only: waits for this wavefront's LDS
// accesses (lgkmcnt(0)), not for its outstanding global loads and stores as
// __syncthreads() does; the memory clobber keeps the compiler from moving
// memory accesses across it. Global data a wavefront loaded into LDS must be
// waited for (vmcnt) by that wavefront before the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// The activations use the hardware exp2, log2 and reciprocal (about one ulp
// each): the memory-bound kernels that apply them per element would otherwise
// be bound by full-precision division and log1p sequences.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// softplus(x) = max(x, 0) + ln(1 + e^-|x|) on the hardware base-2 exponential
// and logarithm: e^-|x| lies in (0, 1], so the logarithm sees [1, 2] and
// needs no denormal handling, and an exponential below the float32 normal
// range flushes to 0, which the formula absorbs; ln(1 + e) by e - e^2/2 where
// 1 + e would drop e's low bits (relative error < e^2/3). About half the
// instructions of the library forms, which handle denormal arguments: this
// kernel was bound by them.
constexpr float kLn2 = 0.69314718055994531f;
__device__ __forceinline__ float softplus_hw(float x)
{
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    const float l = e < 0x1p-10f ? e * (1.0f - 0.5f * e) : kLn2 * __builtin_amdgcn_logf(1.0f + e);
    return fmaxf(x, 0.0f) + l;
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}); log1p(e) by its
// series e - e^2/2 where 1 + e would drop e's low bits (relative error < e^2/3)
__device__ __forceinline__ float softplusf_(float x)
{
    const float e = __expf(-fabsf(x));
    const float l = e < 0x1p-10f ? e * (1.0f - 0.5f * e) : __logf(1.0f + e);
    return fmaxf(x, 0.0f) + l;
}

// Sum over the 64 lanes of a wavefront (every lane gets the total).
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Sum over aligned groups of G lanes (G a power of two <= 64; every lane of a
// group gets its group's total).
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// ---- 16-byte vectors of a storage type ------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;  // elements per 16 bytes
    __device__ static void unpack(const u32x4_t& u, float* f)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    // round to nearest even by the hardware conversion (two values per instruction)
    __device__ static u32x4_t pack(const float* f)
    {
        u32x4_t u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
            const b2 h = {(__bf16)f[2 * i], (__bf16)f[2 * i + 1]};
            u[i] = __builtin_bit_cast(uint32_t, h);
        }
        return u;
    }
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ static void unpack(const u32x4_t& u, float* f)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
    }
    __device__ static u32x4_t pack(const float* f)
    {
        return u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
};
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4_t& u) { *reinterpret_cast<u32x4_t*>(p) = u; }

// Maximum over aligned groups of G lanes (G a power of two <= 64; every lane
// of a group gets its group's maximum).
template <int G>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// Maximum over the 64 lanes of a wavefront (every lane gets it).
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

}  // namespace kda
