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

// Cross-lane exchange without LDS.  DPP row_ror:n rotates within each 16-lane
// row; gfx950's permlane16/32 swaps exchange rows 0<->1, 2<->3 and the two
// 32-lane halves.  Reductions below leave the result in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// {value of lane l, value of lane l ^ 16} in some order (same pair in both lanes)
__device__ __forceinline__ u32x2 swap16(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return u32x2{r[0], r[1]};
}
__device__ __forceinline__ u32x2 swap32(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return u32x2{r[0], r[1]};
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += __uint_as_float(dpp_u32<kRowRor1>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kRowRor2>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kRowRor4>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kRowRor8>(__float_as_uint(v)));
    u32x2 p = swap16(__float_as_uint(v));
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    p = swap32(__float_as_uint(v));
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum of the four lanes l, l^16, l^32, l^48 (one per 16-lane row), in every lane.
__device__ __forceinline__ float row_sum_f32(float v) {
    u32x2 p = swap16(__float_as_uint(v));
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    p = swap32(__float_as_uint(v));
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Kept for the LM-head kernels: plain wave sum in every lane.
__device__ __forceinline__ float wave_sum(float v) { return wave_sum_f32(v); }

// Wave sums of N values at once (N a power of two, <= 64).  Each cross-lane
// step pairs two values and keeps one of them per half of the exchanging
// lanes, so the set halves while the partial sums double: N values cost
// N - 1 pair steps plus (6 - log2 N) single steps instead of 6 N.  On return
// lane l holds the sum of v[l >> (6 - log2 N)] over all 64 lanes.
constexpr int kRowMirror = 0x140, kRowHalfMirror = 0x141, kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;

template <int D>
__device__ __forceinline__ float pair_sum(float a, float b) {
    // lanes with bit D clear return a + a(partner), lanes with it set b + b(partner)
    if constexpr (D == 32 || D == 16) {
        const auto r = (D == 32)
            ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
            : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        constexpr int kCtrl = D == 8 ? kRowMirror : D == 4 ? kRowHalfMirror : D == 2 ? kQuadSwap2 : kQuadSwap1;
        const float sa = a + __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(a)));
        const float sb = b + __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(b)));
        return (lane_id() & D) ? sb : sa;
    }
}

template <int D>
__device__ __forceinline__ float partner_sum(float a) {
    if constexpr (D == 32 || D == 16) {
        const u32x2 p = (D == 32) ? swap32(__float_as_uint(a)) : swap16(__float_as_uint(a));
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    } else {
        constexpr int kCtrl = D == 8 ? kRowMirror : D == 4 ? kRowHalfMirror : D == 2 ? kQuadSwap2 : kQuadSwap1;
        return a + __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(a)));
    }
}

template <int N, int D = 32>
__device__ __forceinline__ float multi_sum(float (&v)[N]) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
    if constexpr (N == 1) {
        float r = v[0];
        if constexpr (D >= 32) r = partner_sum<32>(r);
        if constexpr (D >= 16) r = partner_sum<16>(r);
        if constexpr (D >= 8) r = partner_sum<8>(r);
        if constexpr (D >= 4) r = partner_sum<4>(r);
        if constexpr (D >= 2) r = partner_sum<2>(r);
        if constexpr (D >= 1) r = partner_sum<1>(r);
        return r;
    } else {
        float h[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) h[i] = pair_sum<D>(v[i], v[i + N / 2]);
        return multi_sum<N / 2, D / 2>(h);
    }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t o;
    o = dpp_u32<kRowRor1>(v); v = o > v ? o : v;
    o = dpp_u32<kRowRor2>(v); v = o > v ? o : v;
    o = dpp_u32<kRowRor4>(v); v = o > v ? o : v;
    o = dpp_u32<kRowRor8>(v); v = o > v ? o : v;
    u32x2 p = swap16(v); v = p[0] > p[1] ? p[0] : p[1];
    p = swap32(v);
    return p[0] > p[1] ? p[0] : p[1];
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    uint32_t o;
    o = dpp_u32<kRowRor1>(v); v = o < v ? o : v;
    o = dpp_u32<kRowRor2>(v); v = o < v ? o : v;
    o = dpp_u32<kRowRor4>(v); v = o < v ? o : v;
    o = dpp_u32<kRowRor8>(v); v = o < v ? o : v;
    u32x2 p = swap16(v); v = p[0] < p[1] ? p[0] : p[1];
    p = swap32(v);
    return p[0] < p[1] ? p[0] : p[1];
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = dpp_u32<CTRL>((uint32_t)v), hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<kRowRor1>(v));
    v = max_u64(v, dpp_u64<kRowRor2>(v));
    v = max_u64(v, dpp_u64<kRowRor4>(v));
    v = max_u64(v, dpp_u64<kRowRor8>(v));
    {
        const u32x2 lo = swap16((uint32_t)v), hi = swap16((uint32_t)(v >> 32));
        v = max_u64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
    }
    {
        const u32x2 lo = swap32((uint32_t)v), hi = swap32((uint32_t)(v >> 32));
        v = max_u64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
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
// Two E4M3 codes (bytes 0-1, or 2-3 when hi) to exact float32 values.
#define MOEDEC_FP8X2_F32(w, hi) __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((w), 1.0f, (hi))

// acc + a.x*b.x + a.y*b.y with bf16 inputs, float32 accumulate.
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

// E4M3 magnitude code (0x00..0x7E) of a non-negative float32 q: nearest
// value, ties to the even code, saturating at 448.  At and above 2^-6 the code
// keeps 3 of the 23 mantissa bits (round to nearest even on the 20 dropped
// bits) and rebiases the exponent from 127 to 7; below 2^-6 it is q / 2^-9
// rounded to the nearest even integer, read from the low bits of q + 2^14
// (whose float32 spacing is 2^-9).  Values above 448 and NaN give codes above
// 0x7E and are clamped to it; CLAMP = false leaves that out for quotients
// known to stay below 464, the midpoint above 448.
template <bool CLAMP = true>
__device__ __forceinline__ uint32_t e4m3_mag_code(float q) {
    const uint32_t b = __float_as_uint(q);
    const uint32_t nrm = (b + (0x7FFFFu - (120u << 23)) + ((b >> 20) & 1u)) >> 20;
    const uint32_t sub = __float_as_uint(q + 16384.0f) - 0x46800000u;
    const uint32_t c = b >= 0x3C800000u ? nrm : sub;
    if constexpr (CLAMP) return c < 0x7Eu ? c : 0x7Eu;
    return c;
}

// MXFP8 (E4M3 elements sharing one power-of-two scale per 32 values).  A
// block whose largest magnitude has float32 bits amax_bits (sign clear) has
// scale X = 2^(floor(log2 amax) - 8), clamped at 2^-127 (also for an all-zero
// block): E8M0 byte mx8_scale_byte, exact reciprocal mx8_inv (byte <= 246).
__device__ __forceinline__ uint32_t mx8_scale_byte(uint32_t amax_bits) {
    return (uint32_t)max((int)((amax_bits >> 23) & 0xFFu) - 8, 0);
}
__device__ __forceinline__ float mx8_inv(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }
__device__ __forceinline__ void mx8_scale(uint32_t amax_bits, float& X, float& inv) {
    const uint32_t b = mx8_scale_byte(amax_bits);
    X = b ? __uint_as_float(b << 23) : 0x1p-127f;
    inv = mx8_inv(b);
}

// E4M3 code of v / X (an exact product), nearest-even, saturating, sign kept.
__device__ __forceinline__ uint32_t mx8_code(float v, float inv) {
    const float q = v * inv;
    return e4m3_mag_code<true>(fabsf(q)) | ((__float_as_uint(q) >> 24) & 0x80u);
}

// v rounded to its MXFP8 value e4m3(v / X) * X: the quotient (exact) keeps 3
// mantissa bits at and above 2^-6 and becomes a multiple of 2^-9 below,
// nearest-even either way, and saturates at 448; the sign is kept.
__device__ __forceinline__ float mx8_round(float v, float X, float inv) {
    const float q = fabsf(v * inv);
    const uint32_t b = __float_as_uint(q);
    float r = b >= 0x3C800000u ? __uint_as_float((b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u)
                               : (q + 16384.0f) - 16384.0f;
    r = fminf(r, 448.0f);
    return copysignf(r * X, v);
}

// RMSNorm factors inv[m] = 1 / sqrt(mean(r_m^2) + eps) of M_T tokens of H
// float32 values, by a block of 256 threads that holds the residual as
// 16-byte pieces: piece p = threadIdx.x + 256 i (held in xv[i], p <
// n_pieces) is elements 4p'..4p'+3 of token p / per_tok, p' = p mod per_tok.
// Order: per-thread sums of ((a^2 + b^2) + (c^2 + d^2)) per piece, a wave
// sum, then the four waves' sums added pairwise.  Every kernel that forms
// x = bf16(r * inv) from r takes its factors from here, so all of them form
// the same x bit for bit.  Contains a block barrier.
template <int M_T, int P>
__device__ __forceinline__ void rmsnorm_factors(const u32x4 (&xv)[P], int n_pieces, int per_tok, int H,
                                                float eps, float (&inv)[M_T]) {
    __shared__ float s_ss[4][M_T];
    const int tid = threadIdx.x;
    float ss[M_T];
#pragma unroll
    for (int m = 0; m < M_T; ++m) ss[m] = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int p = tid + 256 * i;
        if (p < n_pieces) {
            const int pm = p / per_tok;
            const float v0 = __uint_as_float(xv[i][0]), v1 = __uint_as_float(xv[i][1]);
            const float v2 = __uint_as_float(xv[i][2]), v3 = __uint_as_float(xv[i][3]);
            const float sq = (v0 * v0 + v1 * v1) + (v2 * v2 + v3 * v3);
#pragma unroll
            for (int m = 0; m < M_T; ++m) ss[m] += (m == pm) ? sq : 0.f;
        }
    }
    const int w = tid / kWave;
#pragma unroll
    for (int m = 0; m < M_T; ++m) {
        const float t = wave_sum_f32(ss[m]);
        if ((tid & (kWave - 1)) == 0) s_ss[w][m] = t;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M_T; ++m)
        inv[m] = 1.0f / sqrtf(((s_ss[0][m] + s_ss[1][m]) + (s_ss[2][m] + s_ss[3][m])) / (float)H + eps);
}

}  // namespace moedec
