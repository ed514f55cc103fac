// Device helpers shared by the libmoedec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moedec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int wave_id_uniform() {
    // Wave index inside the block, forced into an SGPR so that everything
    // derived from it is wave-uniform (scalar loads of activations).
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Streaming 16-byte load of weights that are read once per call.
__device__ __forceinline__ u32x4 load_stream16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off, 64);
        uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off, 64);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// E8M0 scale byte -> float32 2^(b-127); valid for codes 1..254.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __uint_as_float(b << 23); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Two E2M1 codes (byte `sel` of `w`, low nibble first) times `scale` as a
// bf16 pair; exact for the scales in the domain (E2M1 x 2^k fits bf16).
#define MOEDEC_FP4X2_BF16(w, scale, sel) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((w), (scale), (sel))
// Same as two float32 values.
#define MOEDEC_FP4X2_F32(w, scale, sel) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((w), (scale), (sel))
// Two E4M3 codes (16-bit half `hi` of `w`, low byte first) as a bf16 pair.
#define MOEDEC_FP8X2_BF16(w, hi) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), 1.0f, (hi))

// acc + a.x*b.x + a.y*b.y with bf16 inputs, float32 accumulate.
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

}  // namespace moedec
