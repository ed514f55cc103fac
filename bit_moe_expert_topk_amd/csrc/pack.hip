// One-time repacking of canonical MXFP4 expert matrices into the layout the
// FFN kernel streams.  For one expert:
//
//   gate/up, unit rg = rows 16rg..16rg+15 of both W_gate and W_up, chunk pair c:
//     codes  [I/16][KBH4][2][64][16]  half 0 = gate, half 1 = up; lane l holds
//            the 16 code bytes of row 16rg + (l & 15), MX block 4c + (l >> 4)
//     scales [I/16][KBH4][64] u16     low byte gate, high byte up, same lane map
//   down, unit g = output rows 16g..16g+15, chunk c:
//     codes  [H/16][KBI4][64][16]     lane l: row 16g + (l & 15), MX block 4c + (l >> 4)
//     scales [H/16][KBI4][64] u8
//
// KBH4 = ceil(H/32 / 4), KBI4 = ceil(I/32 / 4).  MX blocks beyond the matrix
// (when the block count is not a multiple of four) hold zero codes and scale
// 127 (= 1.0), so they contribute exactly zero.  The packing is a pure byte
// permutation of the canonical codes [N][K/2] (low nibble = even k) and scales
// [N][K/32] plus that padding.
#include "device_common.h"
#include "launch.h"

namespace moedec {

namespace {

constexpr uint8_t kPadScale = 127;

__device__ __forceinline__ void unit_coords(size_t u, int n_chunks, int& lane, int& c, size_t& grp) {
    lane = (int)(u & 63);
    const size_t rest = u >> 6;
    c = (int)(rest % n_chunks);
    grp = rest / n_chunks;
}

// One thread per 16-byte code unit of the gate/up stream.
__global__ __launch_bounds__(256) void pack_gateup_codes_kernel(
    const uint8_t* __restrict__ gc, const uint8_t* __restrict__ uc, int n_exp, int H, int I,
    uint8_t* __restrict__ out) {
    const int kb = H / 32, kb4 = (kb + 3) / 4, units_per_e = I / 16;
    const size_t total = (size_t)n_exp * units_per_e * kb4 * 2 * 64;
    for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < total;
         u += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u & 63);
        size_t rest = u >> 6;
        const int half = (int)(rest & 1);
        rest >>= 1;
        const int c = (int)(rest % kb4);
        rest /= kb4;
        const int rg = (int)(rest % units_per_e);
        const size_t e = rest / units_per_e;
        const int row = 16 * rg + (lane & 15);
        const int q = 4 * c + (lane >> 4);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (q < kb) {
            const uint8_t* src = (half ? uc : gc) + (e * I + row) * (size_t)(H / 2) + 16 * q;
            v = *reinterpret_cast<const u32x4*>(src);
        }
        *reinterpret_cast<u32x4*>(out + u * 16) = v;
    }
}

__global__ __launch_bounds__(256) void pack_gateup_scales_kernel(
    const uint8_t* __restrict__ gs, const uint8_t* __restrict__ us, int n_exp, int H, int I,
    uint16_t* __restrict__ out) {
    const int kb = H / 32, kb4 = (kb + 3) / 4, units_per_e = I / 16;
    const size_t total = (size_t)n_exp * units_per_e * kb4 * 64;
    for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < total;
         u += (size_t)gridDim.x * blockDim.x) {
        int lane, c;
        size_t grp;
        unit_coords(u, kb4, lane, c, grp);
        const int rg = (int)(grp % units_per_e);
        const size_t e = grp / units_per_e;
        const int row = 16 * rg + (lane & 15);
        const int q = 4 * c + (lane >> 4);
        uint16_t v = (uint16_t)(kPadScale | (kPadScale << 8));
        if (q < kb) {
            const size_t i = (e * I + row) * (size_t)kb + q;
            v = (uint16_t)(gs[i] | (us[i] << 8));
        }
        out[u] = v;
    }
}

__global__ __launch_bounds__(256) void pack_down_codes_kernel(const uint8_t* __restrict__ dc,
                                                              int n_exp, int H, int I,
                                                              uint8_t* __restrict__ out) {
    const int kb = I / 32, kb4 = (kb + 3) / 4, units_per_e = H / 16;
    const size_t total = (size_t)n_exp * units_per_e * kb4 * 64;
    for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < total;
         u += (size_t)gridDim.x * blockDim.x) {
        int lane, c;
        size_t grp;
        unit_coords(u, kb4, lane, c, grp);
        const int g = (int)(grp % units_per_e);
        const size_t e = grp / units_per_e;
        const int row = 16 * g + (lane & 15);
        const int q = 4 * c + (lane >> 4);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (q < kb) v = *reinterpret_cast<const u32x4*>(dc + (e * H + row) * (size_t)(I / 2) + 16 * q);
        *reinterpret_cast<u32x4*>(out + u * 16) = v;
    }
}

__global__ __launch_bounds__(256) void pack_down_scales_kernel(const uint8_t* __restrict__ ds,
                                                               int n_exp, int H, int I,
                                                               uint8_t* __restrict__ out) {
    const int kb = I / 32, kb4 = (kb + 3) / 4, units_per_e = H / 16;
    const size_t total = (size_t)n_exp * units_per_e * kb4 * 64;
    for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < total;
         u += (size_t)gridDim.x * blockDim.x) {
        int lane, c;
        size_t grp;
        unit_coords(u, kb4, lane, c, grp);
        const int g = (int)(grp % units_per_e);
        const size_t e = grp / units_per_e;
        const int row = 16 * g + (lane & 15);
        const int q = 4 * c + (lane >> 4);
        out[u] = (q < kb) ? ds[(e * H + row) * (size_t)kb + q] : kPadScale;
    }
}

// ---------------------------------------------------------------------------
// FP8 shared expert: bf16 W_gate, W_up [I][H] and W_down [H][I] quantised per
// output row to E4M3 with a float32 scale (s = absmax / 448, 1 for an all-zero
// row; code = E4M3 nearest-even, saturating, of fl32(w / s)) and laid out in
// 16-byte lanes that hold 16 codes each:
//   gate/up  codes [I/16][KH8][2][64][16]  unit rg, chunk c, half (0 gate,
//            1 up), lane l: row 16rg + (l & 15), k = 64c + 16(l >> 4) + b
//   down     codes [H/16][KI8][64][16]     row block rb, chunk c, lane l:
//            row 16rb + (l & 15), k = 64c + 16(l >> 4) + b
//   scales   gate [I], up [I] (one array of 2I), down [H], float32
// KH8 = 2 ceil(H/32 / 4), KI8 = 2 ceil(I/32 / 4) (twice the MXFP4 chunk counts:
// a chunk holds 64 values per row instead of 128); codes past H or I are 0.

// One wave per row of the three matrices (gate rows, up rows, down rows):
// the row's float32 scale.
__global__ __launch_bounds__(256) void shared_fp8_scales_kernel(const uint16_t* __restrict__ g,
                                                                const uint16_t* __restrict__ u,
                                                                const uint16_t* __restrict__ d, int H, int I,
                                                                float* __restrict__ gu_s,
                                                                float* __restrict__ dn_s) {
    const int lane = lane_id();
    const int n_rows = 2 * I + H;
    const int waves = gridDim.x * (blockDim.x >> 6);
    for (int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < n_rows; r += waves) {
        const uint16_t* row = r < I ? g + (size_t)r * H : r < 2 * I ? u + (size_t)(r - I) * H
                                                                    : d + (size_t)(r - 2 * I) * I;
        const int K = r < 2 * I ? H : I;
        uint32_t am = 0;
        for (int k = lane; k < K; k += kWave) am = max(am, row[k] & 0x7FFFu);
        const float a = bf16_to_f32(wave_max_u32(am));
        const float sc = (a == 0.f) ? 1.0f : a / 448.0f;
        if (lane == 0) {
            if (r < 2 * I) gu_s[r] = sc;
            else dn_s[r - 2 * I] = sc;
        }
    }
}

// The 16 codes of one output lane: w[k0 .. k0 + 15] of a row divided by its
// scale (IEEE division) and encoded; k past K gives code 0.
__device__ __forceinline__ u32x4 e4m3_lane(const uint16_t* __restrict__ row, int k0, int K, float sc) {
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        const int k = k0 + b;
        uint32_t code = 0;
        if (k < K) {
            const uint32_t wb = row[k];
            const float q = bf16_to_f32(wb & 0x7FFFu) / sc;
            code = e4m3_mag_code<true>(q) | ((wb >> 8) & 0x80u);
        }
        out[b >> 2] |= code << (8 * (b & 3));
    }
    return out;
}

// One thread per 16-byte output lane of the gate/up layout, then of the down layout.
__global__ __launch_bounds__(256) void shared_fp8_codes_kernel(const uint16_t* __restrict__ g,
                                                               const uint16_t* __restrict__ u,
                                                               const uint16_t* __restrict__ d, int H, int I,
                                                               const float* __restrict__ gu_s,
                                                               const float* __restrict__ dn_s,
                                                               uint8_t* __restrict__ gu_c,
                                                               uint8_t* __restrict__ dn_c) {
    const int kh8 = 2 * ((H / 32 + 3) / 4), ki8 = 2 * ((I / 32 + 3) / 4);
    const size_t n_gu = (size_t)(I / 16) * kh8 * 2 * 64, n_dn = (size_t)(H / 16) * ki8 * 64;
    for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < n_gu + n_dn;
         t += (size_t)gridDim.x * blockDim.x) {
        if (t < n_gu) {
            const int lane = (int)(t & 63);
            size_t rest = t >> 6;
            const int half = (int)(rest & 1);
            rest >>= 1;
            const int c = (int)(rest % kh8);
            const int rg = (int)(rest / kh8);
            const int r = 16 * rg + (lane & 15);
            const uint16_t* row = (half ? u : g) + (size_t)r * H;
            const float sc = gu_s[half * I + r];
            *reinterpret_cast<u32x4*>(gu_c + t * 16) = e4m3_lane(row, 64 * c + 16 * (lane >> 4), H, sc);
        } else {
            const size_t v = t - n_gu;
            const int lane = (int)(v & 63);
            const size_t rest = v >> 6;
            const int c = (int)(rest % ki8);
            const int rb = (int)(rest / ki8);
            const int r = 16 * rb + (lane & 15);
            *reinterpret_cast<u32x4*>(dn_c + v * 16) =
                e4m3_lane(d + (size_t)r * I, 64 * c + 16 * (lane >> 4), I, dn_s[r]);
        }
    }
}

unsigned grid_for(size_t items) {
    size_t b = (items + 255) / 256;
    if (b > 65536) b = 65536;
    return (unsigned)(b == 0 ? 1 : b);
}

}  // namespace

void packed_sizes(int H, int I, moedec_mxfp4_sizes* out) {
    const size_t kbh4 = (size_t)(H / 32 + 3) / 4, kbi4 = (size_t)(I / 32 + 3) / 4;
    out->gu_codes = (size_t)(I / 16) * kbh4 * 2048;
    out->gu_scales = (size_t)(I / 16) * kbh4 * 128;
    out->dn_codes = (size_t)(H / 16) * kbi4 * 1024;
    out->dn_scales = (size_t)(H / 16) * kbi4 * 64;
}

hipError_t launch_pack_gateup(const uint8_t* gc, const uint8_t* gs, const uint8_t* uc,
                              const uint8_t* us, int n_exp, int H, int I, uint8_t* oc,
                              uint8_t* os, hipStream_t s) {
    moedec_mxfp4_sizes sz;
    packed_sizes(H, I, &sz);
    const size_t units = (size_t)n_exp * sz.gu_codes / 16;
    hipLaunchKernelGGL(pack_gateup_codes_kernel, dim3(grid_for(units)), dim3(256), 0, s, gc, uc,
                       n_exp, H, I, oc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t words = (size_t)n_exp * sz.gu_scales / 2;
    hipLaunchKernelGGL(pack_gateup_scales_kernel, dim3(grid_for(words)), dim3(256), 0, s, gs, us,
                       n_exp, H, I, reinterpret_cast<uint16_t*>(os));
    return hipGetLastError();
}

void shared_fp8_sizes(int H, int I, moedec_mxfp4_sizes* out) {
    const size_t kh8 = 2 * (size_t)((H / 32 + 3) / 4), ki8 = 2 * (size_t)((I / 32 + 3) / 4);
    out->gu_codes = (size_t)(I / 16) * kh8 * 2 * 1024;
    out->gu_scales = (size_t)2 * I * sizeof(float);
    out->dn_codes = (size_t)(H / 16) * ki8 * 1024;
    out->dn_scales = (size_t)H * sizeof(float);
}

hipError_t launch_pack_shared_fp8(const uint16_t* g, const uint16_t* u, const uint16_t* d, int H, int I,
                                  uint8_t* gu_c, float* gu_s, uint8_t* dn_c, float* dn_s, hipStream_t s) {
    hipLaunchKernelGGL(shared_fp8_scales_kernel, dim3(grid_for((size_t)(2 * I + H) * 64)), dim3(256), 0, s,
                       g, u, d, H, I, gu_s, dn_s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    moedec_mxfp4_sizes sz;
    shared_fp8_sizes(H, I, &sz);
    const size_t lanes = (sz.gu_codes + sz.dn_codes) / 16;
    hipLaunchKernelGGL(shared_fp8_codes_kernel, dim3(grid_for(lanes)), dim3(256), 0, s, g, u, d, H, I, gu_s,
                       dn_s, gu_c, dn_c);
    return hipGetLastError();
}

hipError_t launch_pack_down(const uint8_t* dc, const uint8_t* ds, int n_exp, int H, int I,
                            uint8_t* oc, uint8_t* os, hipStream_t s) {
    moedec_mxfp4_sizes sz;
    packed_sizes(H, I, &sz);
    const size_t units = (size_t)n_exp * sz.dn_codes / 16;
    hipLaunchKernelGGL(pack_down_codes_kernel, dim3(grid_for(units)), dim3(256), 0, s, dc, n_exp,
                       H, I, oc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t bytes = (size_t)n_exp * sz.dn_scales;
    hipLaunchKernelGGL(pack_down_scales_kernel, dim3(grid_for(bytes)), dim3(256), 0, s, ds, n_exp,
                       H, I, os);
    return hipGetLastError();
}

}  // namespace moedec
