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
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "launch.h"
#include "route_device.h"

namespace moedec {

namespace {

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

// Quotient |w| / s of a bf16 magnitude (its 15 low bits, placed in the top of
// a float) by the row scale.  FAST replaces the division by the product with
// the rounded reciprocal y = 1/s and one correction with the exact remainder
// (Markstein's method: q0 = w*y, r = w - q0*s by fused multiply-add, q = q0 +
// r*y).  For every bf16 w and every s >= 2^-90 of a bf16 absmax this equals
// the IEEE quotient wherever the quotient is at least 2^-14; below that both
// round to E4M3 code 0.  Rows with a smaller scale divide.
template <bool FAST>
__device__ __forceinline__ float row_quotient(uint32_t mag_bits, float s, float y) {
    const float w = __uint_as_float(mag_bits);
    if constexpr (FAST) {
        const float q0 = w * y;
        const float r = __builtin_fmaf(-q0, s, w);
        return __builtin_fmaf(r, y, q0);
    } else {
        return w / s;
    }
}

// Four E4M3 codes of the four bf16 values in (d0, d1), low half first; the
// sign bit of each code is the bf16 sign bit (the scale is positive).  With a
// normal scale s = fl32(a / 448) >= a / 448 * (1 - 2^-24) and |w| <= a, every
// quotient is at most one float32 step above 448, which rounds to 448: FAST
// needs no clamp.  Subnormal scales lose precision, so the dividing path clamps.
template <bool FAST>
__device__ __forceinline__ uint32_t quant4(uint32_t d0, uint32_t d1, float s, float y) {
    const uint32_t c0 = e4m3_mag_code<!FAST>(row_quotient<FAST>((d0 & 0x7FFFu) << 16, s, y));
    const uint32_t c1 = e4m3_mag_code<!FAST>(row_quotient<FAST>(d0 & 0x7FFF0000u, s, y));
    const uint32_t c2 = e4m3_mag_code<!FAST>(row_quotient<FAST>((d1 & 0x7FFFu) << 16, s, y));
    const uint32_t c3 = e4m3_mag_code<!FAST>(row_quotient<FAST>(d1 & 0x7FFF0000u, s, y));
    const uint32_t sign = ((d0 >> 8) & 0x80u) | ((d0 >> 16) & 0x8000u) | ((d1 << 8) & 0x800000u) |
                          (d1 & 0x80000000u);
    return (c0 | (c1 << 8) | (c2 << 16) | (c3 << 24)) | sign;
}

constexpr int kRows = 4;   // rows per wave step

constexpr int pow2_ceil(int n) { return n <= 1 ? 1 : 2 * pow2_ceil((n + 1) / 2); }
constexpr int log2_exact(int n) { return n <= 1 ? 0 : 1 + log2_exact(n / 2); }

// Argmax key of logit `val` at row `row`: larger logit first, then the lower
// row (float_order puts -0.0 and +0.0 together, so the row decides there too).
__device__ __forceinline__ uint64_t argmax_key(float val, int row) {
    return ((uint64_t)float_order(val) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, off);
        const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    return k;
}

// Writes the R x M_T row sums of a wave step: acc[r][m] summed over the wave
// (multi_sum: lane l ends with value l >> kShift) and scaled by scale(r).
// Logits are stored when `logits` is non-null; `best` keeps this lane's
// running argmax key (its token is (lane >> kShift) % M_T in every step).
template <int R, int M_T, bool KEYS, typename Scale>
__device__ __forceinline__ void store_row_sums(const float (&acc)[R][M_T], int v, int v1, int V,
                                               float* __restrict__ logits, Scale scale, uint64_t& best) {
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
        if (v + r < v1) {
            const float val = tot * scale(v + r);
            if (!KEYS || logits) logits[(size_t)m * V + v + r] = val;
            if constexpr (KEYS) {
                const uint64_t key = argmax_key(val, v + r);
                best = key > best ? key : best;
            }
        }
    }
}

// Quantisation.  T = 16-byte chunks (8 bf16) per lane per row, exactly
// ceil(H / 8 / 64); each wave quantises one row per step, all of its loads in
// flight at once, and many waves per SIMD keep the rows overlapping.
template <int T>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ w, int V,
                                                        int H, uint8_t* __restrict__ codes,
                                                        float* __restrict__ rs) {
    const int lane = lane_id();
    const int n_ch = H / 8;
    const int waves = gridDim.x * (blockDim.x >> 6);
    for (int v = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); v < V; v += waves) {
        // unconditional loads (clamped chunk index): all in flight at once
        const uint8_t* row = reinterpret_cast<const uint8_t*>(w) + (size_t)v * H * 2;
        u32x4 c[T];
#pragma unroll
        for (int t = 0; t < T; ++t) c[t] = load_stream16(row + (size_t)min(lane + 64 * t, n_ch - 1) * 16);
        uint32_t am = 0;
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) am = max(am, max(c[t][i] & 0x7FFFu, (c[t][i] >> 16) & 0x7FFFu));
        }
        const float a = bf16_to_f32(wave_max_u32(am));
        const float s = (a == 0.f) ? 1.0f : a / 448.0f;
        const float y = 1.0f / s;
        const bool fast = s >= 0x1p-90f && s <= 0x1.fffffep127f;   // wave-uniform
        uint8_t* out_row = codes + (size_t)v * H;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int ch = lane + 64 * t;
            if (64 * (t + 1) <= n_ch || ch < n_ch) {
                const u32x4 d = c[t];
                u32x2 o;
                if (fast) {
                    o[0] = quant4<true>(d[0], d[1], s, y);
                    o[1] = quant4<true>(d[2], d[3], s, y);
                } else {
                    o[0] = quant4<false>(d[0], d[1], s, y);
                    o[1] = quant4<false>(d[2], d[3], s, y);
                }
                *reinterpret_cast<u32x2*>(out_row + (size_t)ch * 8) = o;
            }
        }
        if (lane == 0) rs[v] = s;
    }
}

// FP8 GEMV.  T = 16-byte chunks per lane per row (ceil(H / 16 / 64)), R rows
// per wave step.  Each lane keeps its slice of x (every token) in registers
// and reuses it for every row the wave visits; the R x M_T row sums of a
// step are reduced together (store_row_sums).
// KEYS (the greedy epilogue): this wave's argmax key per token at
// keys[wave * M_T + m] (0 when the wave has no rows); logits may be null.
template <int M_T, int T, int R, bool KEYS>
__global__ __launch_bounds__(256) void gemv_fp8_kernel(const uint8_t* __restrict__ codes,
                                                       const float* __restrict__ rs, int V, int H,
                                                       const uint32_t* __restrict__ x,
                                                       float* __restrict__ logits,
                                                       int rows_per_wave, uint64_t* __restrict__ keys) {
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
    uint64_t best = 0;
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
        store_row_sums<R, M_T, KEYS>(acc, v, v1, V, logits, [&](int row) { return rs[row]; }, best);
    }
    if constexpr (KEYS) {
        constexpr int kShift = 6 - log2_exact(pow2_ceil(R * M_T));
        const int lane_m = (lane >> kShift) % M_T;
#pragma unroll
        for (int m = 0; m < M_T; ++m) {
            const uint64_t k = wave_max_u64(lane_m == m ? best : 0ull);
            if (lane == 0) keys[(size_t)gw * M_T + m] = k;
        }
    }
}

// Greedy token per row of x: the maximum over the waves' keys, one block of
// 1,024 threads whose loads go out in batches of kArgBatch (a 157,184-row
// head has 4,912 waves: one batch).
constexpr int kArgThreads = 1024;
constexpr int kArgBatch = 8;

template <int M_T>
__global__ __launch_bounds__(kArgThreads) void argmax_reduce_kernel(const uint64_t* __restrict__ keys,
                                                                    int n_waves, int32_t* __restrict__ ids) {
    __shared__ uint64_t s_best[kArgThreads / 64][M_T];
    const int w = threadIdx.x >> 6, lane = lane_id();
    uint64_t b[M_T];
#pragma unroll
    for (int m = 0; m < M_T; ++m) b[m] = 0;
    for (int i0 = threadIdx.x; i0 < n_waves; i0 += kArgThreads * kArgBatch) {
        uint64_t k[kArgBatch][M_T];
#pragma unroll
        for (int j = 0; j < kArgBatch; ++j) {
            const int i = i0 + kArgThreads * j;
#pragma unroll
            for (int m = 0; m < M_T; ++m) k[j][m] = (i < n_waves) ? keys[(size_t)i * M_T + m] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < kArgBatch; ++j)
#pragma unroll
            for (int m = 0; m < M_T; ++m) b[m] = k[j][m] > b[m] ? k[j][m] : b[m];
    }
#pragma unroll
    for (int m = 0; m < M_T; ++m) {
        const uint64_t t = wave_max_u64(b[m]);
        if (lane == 0) s_best[w][m] = t;
    }
    __syncthreads();
    if (threadIdx.x < M_T) {
        uint64_t t = 0;
        for (int i = 0; i < kArgThreads / 64; ++i) t = s_best[i][threadIdx.x] > t ? s_best[i][threadIdx.x] : t;
        ids[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)t);
    }
}

template <int M_T, int T, int R>
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
    for (int v = v0; v < v1; v += R) {
        u32x4 c[R][T];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
                c[r][t] = load_stream16(base + ((size_t)min(v + r, v1 - 1) * H +
                                                (size_t)min(lane + 64 * t, n_ch - 1) * 8) * 2);
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
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int m = 0; m < M_T; ++m)
                        acc[r][m] = dot2_bf16(as_bf16x2(c[r][t][j]), as_bf16x2(xr[m][t][j]), acc[r][m]);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M_T; ++m) {
                const float tot = wave_sum(acc[r][m]);
                if (lane == 0 && v + r < v1) logits[(size_t)m * V + v + r] = tot;
            }
    }
}

// bf16 GEMV: 16 rows per wave, 4 per step, for a vocabulary-sized matrix; a
// short one (a router's 512 rows) takes one row per wave so that its few
// megabytes spread over as many waves as it has rows (latency-bound).
constexpr int kRowsPerWave = 16;
constexpr int kShortRows = 16384;

template <int M_T, int T>
void launch_bf16_t(const uint16_t* w, int V, int H, const uint32_t* x, float* logits, hipStream_t s) {
    if (V <= kShortRows) {
        const dim3 grid((V + 3) / 4), blk(256);
        hipLaunchKernelGGL((gemv_bf16_kernel<M_T, T, 1>), grid, blk, 0, s, w, V, H, x, logits, 1);
    } else {
        const int waves = (V + kRowsPerWave - 1) / kRowsPerWave;
        const dim3 grid((waves + 3) / 4), blk(256);
        hipLaunchKernelGGL((gemv_bf16_kernel<M_T, T, kRows>), grid, blk, 0, s, w, V, H, x, logits, kRowsPerWave);
    }
}

// 8 rows per wave step and 32 rows per wave: 59.5 us (M = 1) and 73 us (M = 4)
// on the 157,184 x 2,560 head, against 66 and 124 us for 4 rows, 16 rows per
// wave and one reduction per row.
constexpr int kFp8Rows = 8;
constexpr int kFp8RowsPerWave = 32;

int fp8_waves(int V) {                              // waves launched (4 per block)
    const int waves = (V + kFp8RowsPerWave - 1) / kFp8RowsPerWave;
    return 4 * ((waves + 3) / 4);
}

template <int M_T, int T>
hipError_t gemv_fp8_t(const uint8_t* codes, const float* rs, int V, int H, const uint32_t* x,
                      float* logits, uint64_t* keys, int32_t* ids, hipStream_t s) {
    const int n_waves = fp8_waves(V);
    const dim3 grid(n_waves / 4), blk(256);
    if (!keys) {
        hipLaunchKernelGGL((gemv_fp8_kernel<M_T, T, kFp8Rows, false>), grid, blk, 0, s, codes, rs, V, H, x,
                           logits, kFp8RowsPerWave, nullptr);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemv_fp8_kernel<M_T, T, kFp8Rows, true>), grid, blk, 0, s, codes, rs, V, H, x, logits,
                       kFp8RowsPerWave, keys);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((argmax_reduce_kernel<M_T>), dim3(1), dim3(kArgThreads), 0, s, keys, n_waves, ids);
    return hipGetLastError();
}

template <int M_T>
hipError_t gemv_fp8_m(const uint8_t* codes, const float* rs, int V, int H, const uint32_t* x,
                      float* logits, uint64_t* keys, int32_t* ids, hipStream_t s) {
    switch ((H / 16 + 63) / 64) {
        case 1: return gemv_fp8_t<M_T, 1>(codes, rs, V, H, x, logits, keys, ids, s);
        case 2: return gemv_fp8_t<M_T, 2>(codes, rs, V, H, x, logits, keys, ids, s);
        case 3: return gemv_fp8_t<M_T, 3>(codes, rs, V, H, x, logits, keys, ids, s);
        default: return gemv_fp8_t<M_T, 4>(codes, rs, V, H, x, logits, keys, ids, s);
    }
}

template <int M_T>
hipError_t gemv_bf16_m(const uint16_t* w, int V, int H, const uint32_t* x, float* logits,
                       hipStream_t s) {
    switch ((H / 8 + 63) / 64) {
        case 1: launch_bf16_t<M_T, 1>(w, V, H, x, logits, s); break;
        case 2: launch_bf16_t<M_T, 2>(w, V, H, x, logits, s); break;
        case 3: launch_bf16_t<M_T, 3>(w, V, H, x, logits, s); break;
        case 4: launch_bf16_t<M_T, 4>(w, V, H, x, logits, s); break;
        case 5: launch_bf16_t<M_T, 5>(w, V, H, x, logits, s); break;
        case 6: launch_bf16_t<M_T, 6>(w, V, H, x, logits, s); break;
        case 7: launch_bf16_t<M_T, 7>(w, V, H, x, logits, s); break;
        default: launch_bf16_t<M_T, 8>(w, V, H, x, logits, s); break;
    }
    return hipGetLastError();
}

// Rows are handed out grid-stride, so the grid is sized to what is resident
// at once (occupancy of the instantiation times the CU count), not beyond.
template <int T>
hipError_t quant_t(const uint16_t* w, int V, int H, uint8_t* codes, float* rs, hipStream_t s) {
    static std::atomic<int> resident{0};            // blocks resident on the whole device
    int blocks = resident.load(std::memory_order_relaxed);
    if (blocks == 0) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(&quant_fp8_kernel<T>), 256, 0);
        if (e != hipSuccess) return e;
        blocks = std::max(1, cus * per_cu);
        resident.store(blocks, std::memory_order_relaxed);
    }
    const int need = (V + 3) / 4;                   // one row per wave step, 4 waves per block
    const dim3 grid(need < blocks ? need : blocks), blk(256);
    hipLaunchKernelGGL((quant_fp8_kernel<T>), grid, blk, 0, s, w, V, H, codes, rs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead_quant(const uint16_t* w, int V, int H, uint8_t* codes, float* rs,
                               hipStream_t s) {
    switch ((H / 8 + 63) / 64) {          // 16 <= H <= 8192, H % 16 == 0 -> T in 1..16
        case 1: return quant_t<1>(w, V, H, codes, rs, s);
        case 2: return quant_t<2>(w, V, H, codes, rs, s);
        case 3: return quant_t<3>(w, V, H, codes, rs, s);
        case 4: return quant_t<4>(w, V, H, codes, rs, s);
        case 5: return quant_t<5>(w, V, H, codes, rs, s);
        case 6: return quant_t<6>(w, V, H, codes, rs, s);
        case 7: return quant_t<7>(w, V, H, codes, rs, s);
        case 8: return quant_t<8>(w, V, H, codes, rs, s);
        case 9: case 10: return quant_t<10>(w, V, H, codes, rs, s);
        case 11: case 12: return quant_t<12>(w, V, H, codes, rs, s);
        default: return quant_t<16>(w, V, H, codes, rs, s);
    }
}

hipError_t launch_gemv_fp8(const uint8_t* codes, const float* rs, int V, int H,
                           const uint16_t* x, int M, float* logits, hipStream_t s,
                           uint64_t* keys, int32_t* ids) {
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    switch (M) {
        case 1: return gemv_fp8_m<1>(codes, rs, V, H, x32, logits, keys, ids, s);
        case 2: return gemv_fp8_m<2>(codes, rs, V, H, x32, logits, keys, ids, s);
        case 3: return gemv_fp8_m<3>(codes, rs, V, H, x32, logits, keys, ids, s);
        default: return gemv_fp8_m<4>(codes, rs, V, H, x32, logits, keys, ids, s);
    }
}

size_t lmhead_argmax_keys_bytes(int V, int M) { return (size_t)fp8_waves(V) * M * sizeof(uint64_t); }

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
