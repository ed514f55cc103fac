// Routed + shared SwiGLU expert FFN on packed MXFP4 weights, M = 1..4 tokens.
//
// The pages' premise: at batch 1 decode is bound by reading weights, the MoE
// experts being the largest share, and their MXFP4 kernel is what lifted
// throughput first (knowledge card at ai.cheesepanini.fun, background and
// method point #1; news article yoususu.cn/post/959, "where the speed comes
// from").  A verify window of 4 tokens touches up to 32 experts (card, method
// point #3): the dispatch table lists each active expert once with its token
// mask, so each expert's bytes are streamed once for all tokens using it.
//
// Kernel 1 (gate/up): one block per (slot, group of 32 intermediate rows).
//   Lane l of every wave owns one row -- gate row 32r+l for l < 32, up row
//   32r+l-32 for l >= 32 -- and walks its MX blocks; the 4 waves split the
//   blocks.  Weights arrive as one coalesced 1 KiB chunk per wave step; two
//   E2M1 codes become a scaled bf16 pair in one gfx950 conversion, and
//   v_dot2 accumulates pair products with the activation pair, which is the
//   same for all lanes and so comes from scalar registers.  Products are
//   exact (E2M1 x 2^k x bf16 fits in float32), accumulation is float32.  The
//   gate and up sums meet across lanes l and l+32; h = silu(g) * u stays float32.
// Kernel 2 (down + combine): one block per (slot, group of 64 output rows);
//   lane owns an output row, waves split the blocks of I, h comes from scalar
//   loads.  Each block writes its weighted partial row-group; the last block
//   to finish a row-group (atomic ticket) sums the slots' partials in slot
//   order -- deterministic -- writes y in float32 and rounds it once to bf16.
#include "device_common.h"
#include "launch.h"

namespace moedec {

namespace {

struct GateUpArgs {
    const uint8_t* codes;
    const uint8_t* scales;
    const uint8_t* sh_codes;
    const uint8_t* sh_scales;
    size_t codes_stride, scales_stride;   // bytes per routed expert
    int E, H, I, KB, KB4, M;
    const uint32_t* x;                    // [M][H/2] bf16 pairs
    const moedec_dispatch* disp;
    float* h;                             // [max_slots][M][I]
};

struct DownArgs {
    const uint8_t* codes;
    const uint8_t* scales;
    const uint8_t* sh_codes;
    const uint8_t* sh_scales;
    size_t codes_stride, scales_stride;
    int E, H, I, KB, KB4, M, max_slots;
    const float* h;                       // [max_slots][M][I]
    const moedec_dispatch* disp;
    float* part;                          // [H/64][max_slots][M][64]
    uint32_t* tickets;                    // [H/64]
    uint16_t* y_bf16;                     // [M][H]
    float* y_f32;                         // [M][H] or null
};

constexpr int kWavesPerBlock = 4;
constexpr int kGroupsInFlight = 5;  // scale words (4 MX blocks each) preloaded per wave

template <int M_T>
__global__ __launch_bounds__(256) void gateup_kernel(GateUpArgs a) {
    const int slot = blockIdx.y;
    const moedec_dispatch* __restrict__ disp = a.disp;
    if (slot >= disp->n_slots) return;
    const int e = disp->expert[slot];
    if (e < 0 || e > a.E) return;          // not a table from moe_route_topk
    const uint32_t mask = disp->token_mask[slot];
    const int r = blockIdx.x;
    const uint8_t* cb = (e == a.E ? a.sh_codes : a.codes + (size_t)e * a.codes_stride) +
                        (size_t)r * a.KB * 1024;
    const uint8_t* sb = (e == a.E ? a.sh_scales : a.scales + (size_t)e * a.scales_stride) +
                        (size_t)r * a.KB4 * 256;
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const uint32_t* __restrict__ x = a.x;
    const int xrow = a.H / 2;

    float acc[M_T];
#pragma unroll
    for (int m = 0; m < M_T; ++m) acc[m] = 0.f;

    for (int p0 = w; p0 < a.KB4; p0 += kWavesPerBlock * kGroupsInFlight) {
        u32x4 c[kGroupsInFlight][4];
        uint32_t sc[kGroupsInFlight];
#pragma unroll
        for (int gi = 0; gi < kGroupsInFlight; ++gi) {
            const int p = p0 + kWavesPerBlock * gi;
            if (p < a.KB4) {
                sc[gi] = *reinterpret_cast<const uint32_t*>(sb + (size_t)p * 256 + lane * 4);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int q = 4 * p + b;
                    if (q < a.KB) c[gi][b] = load_stream16(cb + (size_t)q * 1024 + lane * 16);
                }
            }
        }
#pragma unroll
        for (int gi = 0; gi < kGroupsInFlight; ++gi) {
            const int p = p0 + kWavesPerBlock * gi;
            if (p >= a.KB4) break;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int q = 4 * p + b;
                if (q >= a.KB) break;
                const float s = e8m0_to_f32((sc[gi] >> (8 * b)) & 0xFFu);
                bf16x2 wp[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t word = c[gi][b][j >> 2];
                    switch (j & 3) {
                        case 0: wp[j] = MOEDEC_FP4X2_BF16(word, s, 0); break;
                        case 1: wp[j] = MOEDEC_FP4X2_BF16(word, s, 1); break;
                        case 2: wp[j] = MOEDEC_FP4X2_BF16(word, s, 2); break;
                        default: wp[j] = MOEDEC_FP4X2_BF16(word, s, 3); break;
                    }
                }
#pragma unroll
                for (int m = 0; m < M_T; ++m) {
                    if (!((mask >> m) & 1u)) continue;
                    const uint32_t* xq = x + (size_t)m * xrow + q * 16;
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[m] = dot2_bf16(wp[j], as_bf16x2(xq[j]), acc[m]);
                }
            }
        }
    }

    __shared__ float red[kWavesPerBlock][M_T][64];
#pragma unroll
    for (int m = 0; m < M_T; ++m) red[w][m][lane] = acc[m];
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int m = 0; m < M_T; ++m) {
            float t = red[0][m][lane];
#pragma unroll
            for (int v = 1; v < kWavesPerBlock; ++v) t += red[v][m][lane];
            const float other = __shfl_xor(t, 32, 64);   // up for gate lanes
            if (lane < 32 && ((mask >> m) & 1u)) {
                const float g = t, u = other;
                const float hv = g / (1.f + expf(-g)) * u;
                a.h[((size_t)slot * a.M + m) * a.I + 32 * r + lane] = hv;
            }
        }
    }
}

template <int M_T>
__global__ __launch_bounds__(256) void down_kernel(DownArgs a) {
    const int slot = blockIdx.y;
    const moedec_dispatch* __restrict__ disp = a.disp;
    // every slot below n_slots must arrive at the ticket exactly once
    const int n_slots = min(disp->n_slots, a.max_slots);
    if (slot >= n_slots) return;
    const int e_raw = disp->expert[slot];
    const bool valid = e_raw >= 0 && e_raw <= a.E;
    const int e = valid ? e_raw : a.E;
    const uint32_t mask = valid ? disp->token_mask[slot] : 0u;   // no work, still arrives
    const int g = blockIdx.x;
    const uint8_t* cb = (e == a.E ? a.sh_codes : a.codes + (size_t)e * a.codes_stride) +
                        (size_t)g * a.KB * 1024;
    const uint8_t* sb = (e == a.E ? a.sh_scales : a.scales + (size_t)e * a.scales_stride) +
                        (size_t)g * a.KB4 * 256;
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const float* __restrict__ h = a.h + (size_t)slot * a.M * a.I;

    float acc[M_T];
#pragma unroll
    for (int m = 0; m < M_T; ++m) acc[m] = 0.f;

    for (int p0 = w; p0 < a.KB4; p0 += kWavesPerBlock * kGroupsInFlight) {
        u32x4 c[kGroupsInFlight][4];
        uint32_t sc[kGroupsInFlight];
#pragma unroll
        for (int gi = 0; gi < kGroupsInFlight; ++gi) {
            const int p = p0 + kWavesPerBlock * gi;
            if (p < a.KB4) {
                sc[gi] = *reinterpret_cast<const uint32_t*>(sb + (size_t)p * 256 + lane * 4);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int q = 4 * p + b;
                    if (q < a.KB) c[gi][b] = load_stream16(cb + (size_t)q * 1024 + lane * 16);
                }
            }
        }
#pragma unroll
        for (int gi = 0; gi < kGroupsInFlight; ++gi) {
            const int p = p0 + kWavesPerBlock * gi;
            if (p >= a.KB4) break;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int q = 4 * p + b;
                if (q >= a.KB) break;
                const float s = e8m0_to_f32((sc[gi] >> (8 * b)) & 0xFFu);
                f32x2 wv[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t word = c[gi][b][j >> 2];
                    switch (j & 3) {
                        case 0: wv[j] = MOEDEC_FP4X2_F32(word, s, 0); break;
                        case 1: wv[j] = MOEDEC_FP4X2_F32(word, s, 1); break;
                        case 2: wv[j] = MOEDEC_FP4X2_F32(word, s, 2); break;
                        default: wv[j] = MOEDEC_FP4X2_F32(word, s, 3); break;
                    }
                }
#pragma unroll
                for (int m = 0; m < M_T; ++m) {
                    if (!((mask >> m) & 1u)) continue;
                    const float* hq = h + (size_t)m * a.I + q * 32;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        acc[m] = fmaf(wv[j].x, hq[2 * j], acc[m]);
                        acc[m] = fmaf(wv[j].y, hq[2 * j + 1], acc[m]);
                    }
                }
            }
        }
    }

    __shared__ float red[kWavesPerBlock][M_T][64];
    __shared__ int s_last;
#pragma unroll
    for (int m = 0; m < M_T; ++m) red[w][m][lane] = acc[m];
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int m = 0; m < M_T; ++m) {
            float t = red[0][m][lane];
#pragma unroll
            for (int v = 1; v < kWavesPerBlock; ++v) t += red[v][m][lane];
            const float wt = ((mask >> m) & 1u) ? disp->weight[slot][m] : 0.f;
            a.part[(((size_t)g * a.max_slots + slot) * a.M + m) * 64 + lane] = t * wt;
        }
        __threadfence();
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t ticket = atomicAdd(&a.tickets[g], 1u);
        s_last = (ticket == (uint32_t)(n_slots - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (w == 0) {
        for (int m = 0; m < a.M; ++m) {
            float y = 0.f;
            for (int s2 = 0; s2 < n_slots; ++s2)
                y += __builtin_nontemporal_load(
                    &a.part[(((size_t)g * a.max_slots + s2) * a.M + m) * 64 + lane]);
            const size_t o = (size_t)m * a.H + 64 * g + lane;
            if (a.y_f32) a.y_f32[o] = y;
            a.y_bf16[o] = f32_to_bf16_rne(y);
        }
        if (lane == 0) atomicExch(&a.tickets[g], 0u);
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

FfnLayout ffn_layout(int M, int k_max, int H, int I) {
    FfnLayout L;
    L.max_slots = M * k_max + 1;
    L.h_off = 0;
    L.part_off = align256((size_t)L.max_slots * M * I * sizeof(float));
    L.ticket_off = L.part_off + align256((size_t)(H / 64) * L.max_slots * M * 64 * sizeof(float));
    L.total = L.ticket_off + align256((size_t)(H / 64) * sizeof(uint32_t));
    return L;
}

hipError_t launch_expert_ffn(const moedec_moe_weights& w, const uint16_t* x, int M,
                             const moedec_dispatch* disp, int k_max, uint16_t* y_bf16,
                             float* y_f32, void* ws, hipStream_t s) {
    const FfnLayout L = ffn_layout(M, k_max, w.H, w.I);
    uint8_t* base = static_cast<uint8_t*>(ws);
    float* h = reinterpret_cast<float*>(base + L.h_off);
    const int KBH = w.H / 32, KBI = w.I / 32;

    GateUpArgs ga;
    ga.codes = w.gu_codes;
    ga.scales = w.gu_scales;
    ga.sh_codes = w.sh_gu_codes;
    ga.sh_scales = w.sh_gu_scales;
    ga.codes_stride = (size_t)w.I * w.H;
    ga.KB = KBH;
    ga.KB4 = (KBH + 3) / 4;
    ga.scales_stride = (size_t)(w.I / 32) * ga.KB4 * 256;
    ga.E = w.E;
    ga.H = w.H;
    ga.I = w.I;
    ga.M = M;
    ga.x = reinterpret_cast<const uint32_t*>(x);
    ga.disp = disp;
    ga.h = h;
    const dim3 g1(w.I / 32, L.max_slots), blk(256);
    switch (M) {
        case 1: hipLaunchKernelGGL(gateup_kernel<1>, g1, blk, 0, s, ga); break;
        case 2: hipLaunchKernelGGL(gateup_kernel<2>, g1, blk, 0, s, ga); break;
        case 3: hipLaunchKernelGGL(gateup_kernel<3>, g1, blk, 0, s, ga); break;
        default: hipLaunchKernelGGL(gateup_kernel<4>, g1, blk, 0, s, ga); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    DownArgs da;
    da.codes = w.dn_codes;
    da.scales = w.dn_scales;
    da.sh_codes = w.sh_dn_codes;
    da.sh_scales = w.sh_dn_scales;
    da.codes_stride = (size_t)w.H * w.I / 2;
    da.KB = KBI;
    da.KB4 = (KBI + 3) / 4;
    da.scales_stride = (size_t)(w.H / 64) * da.KB4 * 256;
    da.E = w.E;
    da.H = w.H;
    da.I = w.I;
    da.M = M;
    da.max_slots = L.max_slots;
    da.h = h;
    da.disp = disp;
    da.part = reinterpret_cast<float*>(base + L.part_off);
    da.tickets = reinterpret_cast<uint32_t*>(base + L.ticket_off);
    da.y_bf16 = y_bf16;
    da.y_f32 = y_f32;
    const dim3 g2(w.H / 64, L.max_slots);
    switch (M) {
        case 1: hipLaunchKernelGGL(down_kernel<1>, g2, blk, 0, s, da); break;
        case 2: hipLaunchKernelGGL(down_kernel<2>, g2, blk, 0, s, da); break;
        case 3: hipLaunchKernelGGL(down_kernel<3>, g2, blk, 0, s, da); break;
        default: hipLaunchKernelGGL(down_kernel<4>, g2, blk, 0, s, da); break;
    }
    return hipGetLastError();
}

}  // namespace moedec
