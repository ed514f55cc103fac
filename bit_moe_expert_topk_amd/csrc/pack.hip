// One-time repacking of canonical MXFP4 expert matrices into the layout the
// FFN kernels stream: for every step of the K loop, one 64-lane wave reads
// one contiguous 1 KiB chunk whose lane l holds the 16 code bytes (32 E2M1
// values, one MX block) of the row that lane owns.  Scales follow the same
// lane ownership, four blocks per 32-bit word.  Pure byte permutation; scale
// padding bytes are zero.
#include "device_common.h"
#include "launch.h"

namespace moedec {

// Gate/up: 64-lane chunk (e, r, q): lanes 0..31 = gate rows 32r..32r+31,
// lanes 32..63 = up rows, block q.  One thread per 16-byte unit.
__global__ __launch_bounds__(256) void pack_gateup_codes_kernel(
    const uint8_t* __restrict__ gc, const uint8_t* __restrict__ uc, int n_exp, int H, int I,
    uint8_t* __restrict__ out) {
    const int KB = H / 32;
    const size_t units = (size_t)n_exp * (I / 32) * KB * 64;
    for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < units;
         u += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u & 63);
        size_t rest = u >> 6;
        const int q = (int)(rest % KB);
        rest /= KB;
        const int r = (int)(rest % (I / 32));
        const size_t e = rest / (I / 32);
        const int row = 32 * r + (lane & 31);
        const uint8_t* src = (lane < 32 ? gc : uc) + (e * I + row) * (size_t)(H / 2) + 16 * q;
        *reinterpret_cast<u32x4*>(out + u * 16) = *reinterpret_cast<const u32x4*>(src);
    }
}

// Scale words: word (e, g, p, lane) byte b = scale of block 4p+b of the
// lane's row.  `two` selects the gate/up pairing (rows from two matrices,
// 32 per group) versus down (64 rows of one matrix per group).
__global__ __launch_bounds__(256) void pack_scales_kernel(
    const uint8_t* __restrict__ sa, const uint8_t* __restrict__ sb, int n_exp, int n_rows,
    int KB, bool two, uint8_t* __restrict__ out) {
    const int KB4 = (KB + 3) / 4;
    const int rows_per_group = two ? 32 : 64;
    const int groups = n_rows / rows_per_group;
    const size_t words = (size_t)n_exp * groups * KB4 * 64;
    for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < words;
         u += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u & 63);
        size_t rest = u >> 6;
        const int p = (int)(rest % KB4);
        rest /= KB4;
        const int g = (int)(rest % groups);
        const size_t e = rest / groups;
        const uint8_t* src;
        int row;
        if (two) {
            row = 32 * g + (lane & 31);
            src = lane < 32 ? sa : sb;
        } else {
            row = 64 * g + lane;
            src = sa;
        }
        const uint8_t* rp = src + (e * n_rows + row) * (size_t)KB;
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int q = 4 * p + b;
            if (q < KB) word |= (uint32_t)rp[q] << (8 * b);
        }
        *reinterpret_cast<uint32_t*>(out + u * 4) = word;
    }
}

// Down: chunk (e, g, q): lane l = row 64g+l, block q.
__global__ __launch_bounds__(256) void pack_down_codes_kernel(const uint8_t* __restrict__ dc,
                                                              int n_exp, int H, int I,
                                                              uint8_t* __restrict__ out) {
    const int KB = I / 32;
    const size_t units = (size_t)n_exp * (H / 64) * KB * 64;
    for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < units;
         u += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u & 63);
        size_t rest = u >> 6;
        const int q = (int)(rest % KB);
        rest /= KB;
        const int g = (int)(rest % (H / 64));
        const size_t e = rest / (H / 64);
        const uint8_t* src = dc + (e * H + 64 * g + lane) * (size_t)(I / 2) + 16 * q;
        *reinterpret_cast<u32x4*>(out + u * 16) = *reinterpret_cast<const u32x4*>(src);
    }
}

static unsigned grid_for(size_t items) {
    size_t b = (items + 255) / 256;
    if (b > 65536) b = 65536;
    return (unsigned)(b == 0 ? 1 : b);
}

hipError_t launch_pack_gateup(const uint8_t* gc, const uint8_t* gs, const uint8_t* uc,
                              const uint8_t* us, int n_exp, int H, int I, uint8_t* oc,
                              uint8_t* os, hipStream_t s) {
    const size_t units = (size_t)n_exp * (I / 32) * (H / 32) * 64;
    hipLaunchKernelGGL(pack_gateup_codes_kernel, dim3(grid_for(units)), dim3(256), 0, s, gc, uc,
                       n_exp, H, I, oc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int KB = H / 32;
    const size_t words = (size_t)n_exp * (I / 32) * ((KB + 3) / 4) * 64;
    hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(words)), dim3(256), 0, s, gs, us, n_exp,
                       I, KB, true, os);
    return hipGetLastError();
}

hipError_t launch_pack_down(const uint8_t* dc, const uint8_t* ds, int n_exp, int H, int I,
                            uint8_t* oc, uint8_t* os, hipStream_t s) {
    const size_t units = (size_t)n_exp * (H / 64) * (I / 32) * 64;
    hipLaunchKernelGGL(pack_down_codes_kernel, dim3(grid_for(units)), dim3(256), 0, s, dc, n_exp,
                       H, I, oc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int KB = I / 32;
    const size_t words = (size_t)n_exp * (H / 64) * ((KB + 3) / 4) * 64;
    hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(words)), dim3(256), 0, s, ds, ds, n_exp,
                       H, KB, false, os);
    return hipGetLastError();
}

}  // namespace moedec
