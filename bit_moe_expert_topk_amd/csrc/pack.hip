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
