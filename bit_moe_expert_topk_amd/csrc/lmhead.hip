// LM head: one-time FP8 (E4M3) quantisation with a float32 scale per row, and
// the per-token vocabulary GEMV on the FP8 codes, plus the bf16 comparator.
//
// The pages: the 157,184 x 2,560 vocabulary projection is read in full for
// every generated token; the checkpoint keeps it in bf16, and applying a
// dynamic FP8 configuration only when the head is built halves that read
// (news article yoususu.cn/post/959, "where the speed comes from"; knowledge
// card at ai.cheesepanini.fun, method point #2).
//
// GEMV layout: rows stay row-major.  One wave works on R rows at a time; for
// every row each lane loads the same 16-byte column chunks (chunk lane + 64t),
// so its slice of x is loaded into registers once and reused for every row
// the wave visits.  Rows are summed across the wave at the end.
#include "device_common.h"
#include "launch.h"

namespace moedec {

namespace {

// E4M3 code of a float32, nearest-even, saturating to +-448, sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E00000u) return sign | 0x7Eu;                // |v| >= 448
    if (a >= 0x3C800000u) {                                    // |v| >= 2^-6: normal
        const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);   // keep 3 mantissa bits
        return sign | ((rounded - (120u << 23)) >> 20);        // rebias 127 -> 7
    }
    // subnormal: multiple of 2^-9, 0..8 (8 is the least normal, code 0x08)
    const float scaled = __uint_as_float(a) * 512.0f;
    return sign | (uint32_t)__builtin_rintf(scaled);
}

constexpr int kRows = 4;   // rows per wave step

constexpr int pow2_ceil(int n) { return n <= 1 ? 1 : 2 * pow2_ceil((n + 1) / 2); }
constexpr int log2_exact(int n) { return n <= 1 ? 0 : 1 + log2_exact(n / 2); }

// Writes the R x M_T row sums of a wave step: acc[r][m] summed over the wave
// (multi_sum: lane l ends with value l >> kShift) and scaled by scale(r).
template <int R, int M_T, typename Scale>
__device__ __forceinline__ void store_row_sums(const float (&acc)[R][M_T], int v, int v1, int V,
                                               float* __restrict__ logits, Scale scale) {
    constexpr int kN = pow2_ceil(R * M_T);
    constexpr int kShift = 6 - log2_exact(kN);
    float vals[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i) vals[i] = (i < R * M_T) ? acc[i / M_T][i % M_T] : 0.f;
    const float tot = multi_sum<kN>(vals);
    const int lane = lane_id();
    const int idx = lane >> kShift;
    if ((lane & ((1 << kShift) - 1)) == 0 && idx < R * M_T) {
        const int r = idx / M_T, m = idx - (idx / M_T) * M_T;
        if (v + r < v1) logits[(size_t)m * V + v + r] = tot * scale(v + r);
    }
}

template <int T>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ w, int V,
                                                        int H, uint8_t* __restrict__ codes,
                                                        float* __restrict__ rs) {
    const int lane = lane_id();
    const int n_ch = H / 8;                                   // 8 bf16 per chunk
    const int waves = gridDim.x * (blockDim.x >> 6);
    for (int v = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); v < V; v += waves) {
        const uint8_t* row = reinterpret_cast<const uint8_t*>(w) + (size_t)v * H * 2;
        // unconditional loads (clamped chunk index): all in flight at once
        u32x4 c[T];
#pragma unroll
        for (int t = 0; t < T; ++t) c[t] = load_stream16(row + (size_t)min(lane + 64 * t, n_ch - 1) * 16);
        uint32_t amax = 0;
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = c[t][i] & 0x7FFFu, hi = (c[t][i] >> 16) & 0x7FFFu;
                amax = lo > amax ? lo : amax;
                amax = hi > amax ? hi : amax;
            }
        }
        amax = wave_max_u32(amax);
        const float a = bf16_to_f32(amax);
        const float s = (a == 0.f) ? 1.0f : a / 448.0f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int ch = lane + 64 * t;
            if (ch < n_ch) {
                u32x2 out;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    uint32_t word = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const uint32_t d = c[t][2 * i + (b >> 1)];
                        const uint32_t bits = (b & 1) ? (d >> 16) : (d & 0xFFFFu);
                        word |= f32_to_e4m3_sat(bf16_to_f32(bits) / s) << (8 * b);
                    }
                    out[i] = word;
                }
                *reinterpret_cast<u32x2*>(codes + (size_t)v * H + (size_t)ch * 8) = out;
            }
        }
        if (lane == 0) rs[v] = s;
    }
}

// FP8 GEMV.  T = 16-byte chunks per lane per row (ceil(H / 16 / 64)), R rows
// per wave step.  Each lane keeps its slice of x (every token) in registers
// and reuses it for every row the wave visits; the R x M_T row sums of a
// step are reduced together (store_row_sums).
template <int M_T, int T, int R>
__global__ __launch_bounds__(256) void gemv_fp8_kernel(const uint8_t* __restrict__ codes,
                                                       const float* __restrict__ rs, int V, int H,
                                                       const uint32_t* __restrict__ x,
                                                       float* __restrict__ logits,
                                                       int rows_per_wave) {
    const int lane = lane_id();
    const int n_ch = H / 16;
    const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    // x slice of this lane: chunk lane+64t covers 16 bf16 = 8 pairs per token
    uint32_t xr[M_T][T][8];
#pragma unroll
    for (int m = 0; m < M_T; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int ch = lane + 64 * t;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t xv = x[(size_t)m * (H / 2) + min(ch, n_ch - 1) * 8 + j];
                xr[m][t][j] = (ch < n_ch) ? xv : 0u;     // chunks past H multiply by zero
            }
        }
    const int v0 = gw * rows_per_wave;
    const int v1 = min(V, v0 + rows_per_wave);
    for (int v = v0; v < v1; v += R) {
        // unconditional loads (clamped row and chunk): rows past v1 are computed
        // but never stored, chunks past H meet zero activations
        u32x4 c[R][T];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
                c[r][t] = load_stream16(codes + (size_t)min(v + r, v1 - 1) * H +
                                        (size_t)min(lane + 64 * t, n_ch - 1) * 16);
        float acc[R][M_T];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M_T; ++m) acc[r][m] = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bf16x2 wp = (j & 1) ? MOEDEC_FP8X2_BF16(c[r][t][j >> 1], true)
                                              : MOEDEC_FP8X2_BF16(c[r][t][j >> 1], false);
#pragma unroll
                    for (int m = 0; m < M_T; ++m)
                        acc[r][m] = dot2_bf16(wp, as_bf16x2(xr[m][t][j]), acc[r][m]);
                }
        store_row_sums<R, M_T>(acc, v, v1, V, logits, [&](int row) { return rs[row]; });
    }
}

template <int M_T, int T>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(const uint16_t* __restrict__ wt, int V,
                                                        int H, const uint32_t* __restrict__ x,
                                                        float* __restrict__ logits,
                                                        int rows_per_wave) {
    const int lane = lane_id();
    const int n_ch = H / 8;
    const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    uint32_t xr[M_T][T][4];
#pragma unroll
    for (int m = 0; m < M_T; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int ch = lane + 64 * t;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t xv = x[(size_t)m * (H / 2) + min(ch, n_ch - 1) * 4 + j];
                xr[m][t][j] = (ch < n_ch) ? xv : 0u;
            }
        }
    const uint8_t* base = reinterpret_cast<const uint8_t*>(wt);
    const int v0 = gw * rows_per_wave;
    const int v1 = min(V, v0 + rows_per_wave);
    for (int v = v0; v < v1; v += kRows) {
        u32x4 c[kRows][T];
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
                c[r][t] = load_stream16(base + ((size_t)min(v + r, v1 - 1) * H +
                                                (size_t)min(lane + 64 * t, n_ch - 1) * 8) * 2);
        float acc[kRows][M_T];
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int m = 0; m < M_T; ++m) acc[r][m] = 0.f;
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int m = 0; m < M_T; ++m)
                        acc[r][m] = dot2_bf16(as_bf16x2(c[r][t][j]), as_bf16x2(xr[m][t][j]), acc[r][m]);
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int m = 0; m < M_T; ++m) {
                const float tot = wave_sum(acc[r][m]);
                if (lane == 0 && v + r < v1) logits[(size_t)m * V + v + r] = tot;
            }
    }
}

constexpr int kRowsPerWave = 16;   // bf16 GEMV

// 8 rows per wave step and 32 rows per wave: 59.5 us (M = 1) and 73 us (M = 4)
// on the 157,184 x 2,560 head, against 66 and 124 us for 4 rows, 16 rows per
// wave and one reduction per row.
constexpr int kFp8Rows = 8;
constexpr int kFp8RowsPerWave = 32;

template <int M_T, int T>
hipError_t gemv_fp8_t(const uint8_t* codes, const float* rs, int V, int H, const uint32_t* x,
                      float* logits, hipStream_t s) {
    const int waves = (V + kFp8RowsPerWave - 1) / kFp8RowsPerWave;
    const dim3 grid((waves + 3) / 4), blk(256);
    hipLaunchKernelGGL((gemv_fp8_kernel<M_T, T, kFp8Rows>), grid, blk, 0, s, codes, rs, V, H, x, logits,
                       kFp8RowsPerWave);
    return hipGetLastError();
}

template <int M_T>
hipError_t gemv_fp8_m(const uint8_t* codes, const float* rs, int V, int H, const uint32_t* x,
                      float* logits, hipStream_t s) {
    switch ((H / 16 + 63) / 64) {
        case 1: return gemv_fp8_t<M_T, 1>(codes, rs, V, H, x, logits, s);
        case 2: return gemv_fp8_t<M_T, 2>(codes, rs, V, H, x, logits, s);
        case 3: return gemv_fp8_t<M_T, 3>(codes, rs, V, H, x, logits, s);
        default: return gemv_fp8_t<M_T, 4>(codes, rs, V, H, x, logits, s);
    }
}

template <int M_T>
hipError_t gemv_bf16_m(const uint16_t* w, int V, int H, const uint32_t* x, float* logits,
                       hipStream_t s) {
    const int T = (H / 8 + 63) / 64;
    const int waves = (V + kRowsPerWave - 1) / kRowsPerWave;
    const dim3 grid((waves + 3) / 4), blk(256);
    switch (T) {
        case 1: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 1>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
        case 2: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 2>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
        case 3: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 3>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
        case 4: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 4>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
        case 5: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 5>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
        case 6: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 6>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
        case 7: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 7>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
        default: hipLaunchKernelGGL((gemv_bf16_kernel<M_T, 8>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead_quant(const uint16_t* w, int V, int H, uint8_t* codes, float* rs,
                               hipStream_t s) {
    const int T = (H / 8 + 63) / 64;      // H <= 8192 -> T <= 16
    const int waves = V < 8192 ? V : 8192;
    const dim3 grid((waves + 3) / 4), blk(256);
    switch ((T + 3) / 4) {
        case 1: hipLaunchKernelGGL(quant_fp8_kernel<4>, grid, blk, 0, s, w, V, H, codes, rs); break;
        case 2: hipLaunchKernelGGL(quant_fp8_kernel<8>, grid, blk, 0, s, w, V, H, codes, rs); break;
        case 3: hipLaunchKernelGGL(quant_fp8_kernel<12>, grid, blk, 0, s, w, V, H, codes, rs); break;
        default: hipLaunchKernelGGL(quant_fp8_kernel<16>, grid, blk, 0, s, w, V, H, codes, rs); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_fp8(const uint8_t* codes, const float* rs, int V, int H,
                           const uint16_t* x, int M, float* logits, hipStream_t s) {
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    switch (M) {
        case 1: return gemv_fp8_m<1>(codes, rs, V, H, x32, logits, s);
        case 2: return gemv_fp8_m<2>(codes, rs, V, H, x32, logits, s);
        case 3: return gemv_fp8_m<3>(codes, rs, V, H, x32, logits, s);
        default: return gemv_fp8_m<4>(codes, rs, V, H, x32, logits, s);
    }
}

hipError_t launch_gemv_bf16(const uint16_t* w, int V, int H, const uint16_t* x, int M,
                            float* logits, hipStream_t s) {
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    switch (M) {
        case 1: return gemv_bf16_m<1>(w, V, H, x32, logits, s);
        case 2: return gemv_bf16_m<2>(w, V, H, x32, logits, s);
        case 3: return gemv_bf16_m<3>(w, V, H, x32, logits, s);
        default: return gemv_bf16_m<4>(w, V, H, x32, logits, s);
    }
}

}  // namespace moedec
