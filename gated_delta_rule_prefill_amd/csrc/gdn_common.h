// Device helpers shared by the gfx950 kernels: element types, 16x16 MFMA fragment traits,
// wave64 reductions. CDNA4 only (wave64, MFMA); nothing here is portable on purpose.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 with round-to-nearest-even (the compiler lowers the conversion to the
// gfx950 hardware convert, which rounds to nearest even).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------------------
// 16 x 16 MFMA tile conventions (one wave computes one 16x16 fp32 tile D += A * B):
//   A fragment (rows of A, K contiguous):  lane l holds A[l & 15][kb*KB + (l >> 4)*KPL + i]
//   B fragment (columns of B):             lane l holds B[kb*KB + (l >> 4)*KPL + i][l & 15]
//   accumulator:                           acc[i] = D[(l >> 4)*4 + i][l & 15],  i < 4
// Both operands use the same k <-> (lane group, element) assignment, so the contraction
// is the full sum over k whatever order the hardware pairs them in.
// bf16: v_mfma_f32_16x16x32_bf16 (KB = 32, 8 consecutive k per lane, one 16-byte load).
// fp32: v_mfma_f32_16x16x4_f32   (KB = 4, 1 k per lane).
// ---------------------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int KB = 32;
    static constexpr int KPL = 8;
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag load(const bf16* p) {
        return *reinterpret_cast<const bf16x8*>(p);
    }
    __device__ __forceinline__ static frag zero() {
        frag z;
#pragma unroll
        for (int i = 0; i < 8; i++) z[i] = (bf16)0.0f;
        return z;
    }
};

template <> struct Mma<float> {
    static constexpr int KB = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag load(const float* p) { return *p; }
    __device__ __forceinline__ static frag zero() { return 0.0f; }
};

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

// Workgroup barrier for hand-offs through LDS only: waits for this wave's LDS (and scalar)
// memory operations, then s_barrier. Unlike __syncthreads(), whose workgroup release fence
// also drains every outstanding global load and store, in-flight global traffic (a prefetch
// of the next chunk's operands, output stores) keeps flowing across it. The memory clobber
// stops the compiler from moving LDS accesses across the barrier. Only for barriers that
// order LDS accesses.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (WAVE - 1)); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x / WAVE); }
// Compiler-only memory fence: memory operations are not moved across it (no wait is
// emitted). Placed after a prefetch so the loads are issued there and not sunk below the
// arithmetic that follows.
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// SiLU in fp32 after the short convolution: x * 1 / (1 + 2^(-x log2 e)) on the hardware
// exp2 and reciprocal (about 1 ulp each; an overflowing exponential gives 1/inf = 0, so the
// result tends to -0 for very negative x and to x for large x). Every convolution kernel
// calls this, so the standalone convolution and the ones fused into the prefill and the
// decode step agree bit for bit.
__device__ __forceinline__ float silu_f32(float x) {
    const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
    return x * __builtin_amdgcn_rcpf(1.f + e);
}

// Rotation inside each 16-lane row of the wave (DPP row_ror:D): lane l receives the value
// of lane (l & ~15) | ((l - D) & 15).
// Every lane has a source in a rotation, so no fallback value is needed.
template <int D>
__device__ __forceinline__ float row_ror(float v) {
    static_assert(D >= 1 && D <= 15, "row_ror distance");
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + D, 0xF, 0xF, true));
}
template <int D>
__device__ __forceinline__ bf16x8 row_ror(bf16x8 v) {
    static_assert(D >= 1 && D <= 15, "row_ror distance");
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    i32x4 t = __builtin_bit_cast(i32x4, v);
#pragma unroll
    for (int i = 0; i < 4; i++) t[i] = __builtin_amdgcn_mov_dpp(t[i], 0x120 + D, 0xF, 0xF, true);
    return __builtin_bit_cast(bf16x8, t);
}

// Sum across lanes that share (lane % width) ... reduction over the `width`-lane groups
// formed by xor distances 1..width/2.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, WAVE);
    return x;
}

// Pack/unpack 4 or 8 consecutive elements of T to/from fp32.
template <typename T, int N> struct Vec;
template <> struct Vec<float, 4> {
    typedef f32x4 type;
};
template <> struct Vec<bf16, 4> {
    typedef bf16x4 type;
};

template <typename T>
__device__ __forceinline__ void load4(const T* p, float out[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float out[4]) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}
template <>
__device__ __forceinline__ void load4<bf16>(const bf16* p, float out[4]) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    out[0] = (float)v[0]; out[1] = (float)v[1]; out[2] = (float)v[2]; out[3] = (float)v[3];
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float in[4]);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float in[4]) {
    f32x4 v = {in[0], in[1], in[2], in[3]};
    *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const float in[4]) {
    bf16x4 v;
    v[0] = (bf16)in[0]; v[1] = (bf16)in[1]; v[2] = (bf16)in[2]; v[3] = (bf16)in[3];
    *reinterpret_cast<bf16x4*>(p) = v;
}

// store4 with the non-temporal hint, for outputs nothing reads back soon: their lines do
// not linger dirty in the caches, where the next kernel would pay for their write-back
template <typename T>
__device__ __forceinline__ void store4_nt(T* p, const float in[4]);
template <>
__device__ __forceinline__ void store4_nt<float>(float* p, const float in[4]) {
    f32x4 v = {in[0], in[1], in[2], in[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
template <>
__device__ __forceinline__ void store4_nt<bf16>(bf16* p, const float in[4]) {
    bf16x4 v;
    v[0] = (bf16)in[0]; v[1] = (bf16)in[1]; v[2] = (bf16)in[2]; v[3] = (bf16)in[3];
    uint64_t bits;
    __builtin_memcpy(&bits, &v, 8);
    __builtin_nontemporal_store(bits, reinterpret_cast<uint64_t*>(p));
}

// 8 consecutive elements <-> fp32 (one 16-byte access for bf16, two for fp32)
template <typename T>
__device__ __forceinline__ void load8(const T* p, float out[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float out[8]) {
    load4<float>(p, out);
    load4<float>(p + 4, out + 4);
}
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float out[8]) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = (float)v[i];
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float in[8]);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float in[8]) {
    store4<float>(p, in);
    store4<float>(p + 4, in + 4);
}
template <>
__device__ __forceinline__ void store8<bf16>(bf16* p, const float in[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = (bf16)in[i];
    *reinterpret_cast<bf16x8*>(p) = v;
}

}  // namespace gdn
