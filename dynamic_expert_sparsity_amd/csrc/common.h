// Internal helpers shared by the HIP kernels of libbeam_moe (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef uint16_t bf16_t;  // bfloat16 storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct elem;
template <> struct elem<float> {
    __device__ static __forceinline__ float load(const float *p) { return *p; }
    __device__ static __forceinline__ void store(float *p, float v) { *p = v; }
};
template <> struct elem<bf16_t> {
    __device__ static __forceinline__ float load(const bf16_t *p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ void store(bf16_t *p, float v) { *p = f32_to_bf16(v); }
};

// SiLU(a) = a * sigmoid(a) = a / (1 + e^-a).  `precise` keeps libm's expf
// (float32 path); otherwise the hardware exp2 with a log2(e) prescale.
template <bool precise>
__device__ __forceinline__ float silu(float a) {
    float e = precise ? expf(-a) : __expf(-a);
    return a / (1.0f + e);
}

// SiLU with the hardware exp2 and reciprocal (about 1 ulp each), for
// results rounded to bfloat16.
__device__ __forceinline__ float silu_fast(float a) {
    return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Sum over the 64 lanes of a wave, in a fixed order (deterministic): within
// each row of 16 lanes by DPP moves (swap neighbours, swap pairs, mirror
// within 8, mirror within 16; both partners of a step add the same pair),
// then the four row sums in row order.  Every lane gets the result.
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}

// Dot product of 8 bf16 pairs (16-byte chunks) added to acc, float32.  Each
// 32-bit element is copied to a scalar before the bit cast: a bit cast taken
// directly of a vector element compiled to the first element every time.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_bf16(const u32x4 &a, const u32x4 &b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ai = a[i], bi = b[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ai),
                                              __builtin_bit_cast(bf16x2_t, bi), acc, false);
    }
    return acc;
}

// One MFMA: D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16).
// Lane l supplies A[l % 16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l % 16] and
// holds D[4*(l/16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16-byte scalar load of a workgroup-uniform address (one s_load_dwordx4,
// completed inside the asm block).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 sload16(const void *p) {
    i32x4 v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
// 16-byte load that is not expected to be reused (weights streamed once).
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

}  // namespace beam
