// MoE layer for many tokens at once (a prefill chunk, a long verify window):
// the same routed + shared SwiGLU layer as the decode kernel, computed as a
// grouped GEMM on bf16 matrix cores.
//
// Decoding a token streams weights; filling a long prompt is bound by matrix
// arithmetic instead (news article yoususu.cn/post/959, "two easily missed
// details": prefill is pure matrix compute, decode is bandwidth).  With T
// tokens each of the E routed experts multiplies the T*k/E tokens that chose
// it, read once for all of them (knowledge card at ai.cheesepanini.fun,
// method point 3); the shared expert multiplies all T.
//
// Steps (one stream, in order):
//   route    one wave per token: top-k of its logits (route_device.h), the
//            routing weights, and per-expert token counts
//   plan     one block: exclusive scan of the counts into pair offsets, and
//            the tile list (group, first row) in units of 32*NS tokens
//   scatter  each (token, choice) pair gets a row in its expert's group; the
//            shared group holds token t at row T*k + t
//   gate/up  per (tile, 128 intermediate rows): g = W_gate x, u = W_up x on
//            MFMA 32x32x16 bf16 with float32 accumulation, h = silu(g) * u,
//            stored as h = hi + lo (two bf16, 16 significant bits)
//   down     per (tile, 128 output rows): y_pair = W_down hi + W_down lo
//   combine  y[t] = sum_j w[t][j] * y_pair[row(t, j)] + y_pair[T*k + t] in
//            float32 in that order, then rounded once to bf16
//
// Weights stay in the decode kernel's packed layout (pack.hip): lane l of a
// 16-row unit holds the 32 codes of MX block (l >> 4) of row (l & 15).  The
// MFMA contracts over k in any order as long as both operands use the same
// one, so a lane feeds the matrix core the 8 codes of its own block per step
// and the activations are read from LDS at the matching k.  MFMA operand
// lanes: A lane l = row l % 32 (here a weight row), B lane l = column l % 32
// (a token), each supplying 8 consecutive k of its half (l / 32); D register
// r of lane l = row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
//
// Block -> work mapping is XCD-aware: block b runs on XCD b % 8, and each XCD
// takes a contiguous range of (tile, row block) items, so the row blocks of
// one token tile (which share its activations) and the tiles of one expert
// (which share its weights) meet in the same L2.
#include "device_common.h"
#include "launch.h"
#include "route_device.h"

namespace moedec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 128;   // 4 waves x 32 weight rows
constexpr int kSub = 32;             // tokens per MFMA column block
constexpr int kSlab = 64;            // k per pipeline step: two MX blocks
constexpr int kLdsRow = kSlab + 8;   // bf16 per LDS row, 16 B of padding
constexpr int kXcds = 8;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Eight E2M1 codes (one dword, low nibble first) times a power-of-two scale
// as eight bf16 values (exact in the scale domain).
__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t w, float scale) {
    const bf16x2 a = MOEDEC_FP4X2_BF16(w, scale, 0), b = MOEDEC_FP4X2_BF16(w, scale, 1);
    const bf16x2 c = MOEDEC_FP4X2_BF16(w, scale, 2), d = MOEDEC_FP4X2_BF16(w, scale, 3);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// The work item of this block, or false when it has none.  Items are (tile,
// row block) pairs, n_items = tiles * n_rb; XCD x takes items
// [x * per, (x + 1) * per).
struct Item {
    int group, start, rows, rb;
};

__device__ __forceinline__ bool block_item(const int32_t* n_tiles_p, const int2* tiles,
                                           const int32_t* counts, int n_rb, int tile_tokens, Item& it) {
    const int n_items = __builtin_amdgcn_readfirstlane(*n_tiles_p) * n_rb;
    const int per = (n_items + kXcds - 1) / kXcds;
    const int idx = blockIdx.x / kXcds;
    if (idx >= per) return false;
    const int item = (blockIdx.x % kXcds) * per + idx;
    if (item >= n_items) return false;
    const int tile = item / n_rb;
    const int2 t = tiles[tile];
    it.group = t.x;
    it.start = t.y;
    it.rows = min(tile_tokens, counts[t.x] - t.y);
    it.rb = item - tile * n_rb;
    return true;
}

// ----------------------------------------------------------------------------
// Routing, counting, plan and scatter.

__global__ __launch_bounds__(kThreads) void zero_counts_kernel(int32_t* counts, int32_t* cursor, int n) {
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) {
        counts[i] = 0;
        cursor[i] = 0;
    }
}

template <int KPL>
__global__ __launch_bounds__(kThreads) void route_count_kernel(const float* __restrict__ logits, int T, int E,
                                                               int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts,
                                                               int32_t* __restrict__ counts) {
    __shared__ uint64_t s_buf[kThreads / kWave][kTopkBufWords];
    const int wv = threadIdx.x >> 6, lane = lane_id();
    const int t = blockIdx.x * (kThreads / kWave) + wv;
    if (t >= T) return;
    float w;
    const uint64_t key = wave_topk<KPL>(logits + (size_t)t * E, E, k, w, s_buf[wv]);
    if (lane < k) {
        const int id = key_to_index(key);
        ids[(size_t)t * k + lane] = id;
        wts[(size_t)t * k + lane] = w;
        atomicAdd(&counts[id], 1);
    }
}

// One block.  counts[0..E) from the route kernel; the shared group E gets T.
// off[g] = first pair row of group g (off[E + 1] = total); tiles list every
// (group, first row) in steps of tile_tokens; *n_tiles their number.
constexpr int kPlanPerThread = (MOEDEC_MAX_E + 1 + kThreads - 1) / kThreads;

__global__ __launch_bounds__(kThreads) void plan_kernel(int32_t* __restrict__ counts, int E, int T,
                                                        int tile_tokens, int32_t* __restrict__ off,
                                                        int2* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                        int32_t* __restrict__ counts_out) {
    __shared__ int s_pairs[kThreads], s_tiles[kThreads];
    const int tid = threadIdx.x, G = E + 1;
    if (tid == 0) counts[E] = T;
    __syncthreads();
    int c[kPlanPerThread];
    int my_pairs = 0, my_tiles = 0;
#pragma unroll
    for (int i = 0; i < kPlanPerThread; ++i) {
        const int g = tid * kPlanPerThread + i;
        c[i] = g < G ? counts[g] : 0;
        my_pairs += c[i];
        my_tiles += (c[i] + tile_tokens - 1) / tile_tokens;
    }
    s_pairs[tid] = my_pairs;
    s_tiles[tid] = my_tiles;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {    // inclusive scan (Hillis-Steele)
        const int a = tid >= d ? s_pairs[tid - d] : 0, b = tid >= d ? s_tiles[tid - d] : 0;
        __syncthreads();
        s_pairs[tid] += a;
        s_tiles[tid] += b;
        __syncthreads();
    }
    int p = s_pairs[tid] - my_pairs, q = s_tiles[tid] - my_tiles;
#pragma unroll
    for (int i = 0; i < kPlanPerThread; ++i) {
        const int g = tid * kPlanPerThread + i;
        if (g < G) {
            off[g] = p;
            if (counts_out) counts_out[g] = c[i];
            for (int s = 0; s < c[i]; s += tile_tokens) tiles[q++] = int2{g, s};
            p += c[i];
        }
    }
    if (tid == kThreads - 1) {
        off[G] = s_pairs[tid];
        *n_tiles = s_tiles[tid];
    }
}

// One thread per routed pair, then one per token for the shared group.  The
// row a pair gets inside its group depends on atomic arrival order; no value
// depends on it (each row of the products is computed on its own).
__global__ __launch_bounds__(kThreads) void scatter_kernel(const int32_t* __restrict__ ids, int T, int k,
                                                           const int32_t* __restrict__ off,
                                                           int32_t* __restrict__ cursor,
                                                           int32_t* __restrict__ tok_of,
                                                           int32_t* __restrict__ pos, int E) {
    const size_t n_routed = (size_t)T * k;
    for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < n_routed + T;
         i += (size_t)gridDim.x * kThreads) {
        if (i < n_routed) {
            const int e = ids[i];
            const int row = off[e] + atomicAdd(&cursor[e], 1);
            tok_of[row] = (int)(i / k);
            pos[i] = row;
        } else {
            const int t = (int)(i - n_routed);
            tok_of[off[E] + t] = t;
        }
    }
}

// ----------------------------------------------------------------------------
// gate/up: block = (tile of up to 32*NS tokens of one group, 128 intermediate
// rows); wave w owns rows 32w..32w+31 of that block for both W_gate and W_up.

template <int NS>
struct GateUpLds {
    uint16_t x[2][NS * kSub][kLdsRow];
};

template <int NS>
__global__ __launch_bounds__(kThreads, 2) void gateup_kernel(
    const uint8_t* __restrict__ gu_codes, const uint16_t* __restrict__ gu_scales, size_t e_codes,
    size_t e_scales, const uint8_t* __restrict__ sh_codes, const uint16_t* __restrict__ sh_scales,
    const uint16_t* __restrict__ x, int H, int I, int E, const int32_t* __restrict__ n_tiles,
    const int2* __restrict__ tiles, const int32_t* __restrict__ counts, const int32_t* __restrict__ off,
    const int32_t* __restrict__ tok_of, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
    constexpr int TT = NS * kSub;
    constexpr int kUnits = TT * (kSlab / 8) / kThreads;   // 16-byte x units per thread per slab
    __shared__ __align__(16) GateUpLds<NS> L;

    Item it;
    if (!block_item(n_tiles, tiles, counts, (I + kRowsPerBlock - 1) / kRowsPerBlock, TT, it)) return;

    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id_uniform();
    const int kb4 = (H / 32 + 3) / 4, n_slabs = 2 * kb4;
    const int n_sub = (it.rows + kSub - 1) / kSub;
    const int pair0 = off[it.group] + it.start;

    // activations: unit u = tid + 256 v covers row u >> 3, 8 bf16 at (u & 7) * 8
    const uint16_t* xrow[kUnits];
#pragma unroll
    for (int v = 0; v < kUnits; ++v) {
        const int u = tid + kThreads * v, row = u >> 3;
        xrow[v] = row < it.rows ? x + (size_t)tok_of[pair0 + row] * H + (u & 7) * 8 : nullptr;
    }
    auto load_x = [&](int slab, u32x4 (&r)[kUnits]) {
#pragma unroll
        for (int v = 0; v < kUnits; ++v) {
            const int k0 = slab * kSlab + ((tid + kThreads * v) & 7) * 8;
            r[v] = (xrow[v] && k0 < H) ? *reinterpret_cast<const u32x4*>(xrow[v] + slab * kSlab)
                                       : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_x = [&](int buf, const u32x4 (&r)[kUnits]) {
#pragma unroll
        for (int v = 0; v < kUnits; ++v) {
            const int u = tid + kThreads * v;
            *reinterpret_cast<u32x4*>(&L.x[buf][u >> 3][(u & 7) * 8]) = r[v];
        }
    };

    // weights of this wave: rows n0 .. n0 + 31
    const int n0 = it.rb * kRowsPerBlock + 32 * wv;
    const bool has_rows = n0 < I;
    const uint8_t* cbase = it.group < E ? gu_codes + (size_t)it.group * e_codes : sh_codes;
    const uint16_t* sbase = it.group < E ? gu_scales + (size_t)it.group * e_scales / 2 : sh_scales;
    const int r = lane & 31, half = lane >> 5;
    const size_t unit = (size_t)(n0 / 16 + (r >> 4));
    const int li0 = (r & 15) + 16 * half;     // lane inside the unit for MX block q = half (+ 32 per p)
    auto load_w = [&](int slab, u32x4& g, u32x4& u, uint32_t& sc) {
        if (!has_rows) return;
        const int c = slab >> 1, li = li0 + 32 * (slab & 1);
        const uint8_t* p = cbase + ((unit * kb4 + c) * 2) * 1024 + li * 16;
        g = load_stream16(p);
        u = load_stream16(p + 1024);
        sc = sbase[(unit * kb4 + c) * 64 + li];
    };

    f32x16 acc_g[NS], acc_u[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        acc_g[s] = f32x16{};
        acc_u[s] = f32x16{};
    }

    u32x4 xr[kUnits];
    u32x4 wg = {0u, 0u, 0u, 0u}, wu = {0u, 0u, 0u, 0u};
    uint32_t ws = 0x7F7Fu;
    load_x(0, xr);
    load_w(0, wg, wu, ws);
    store_x(0, xr);
    __syncthreads();

    for (int slab = 0; slab < n_slabs; ++slab) {
        const int buf = slab & 1;
        u32x4 ng = {0u, 0u, 0u, 0u}, nu = {0u, 0u, 0u, 0u};
        uint32_t ns = 0x7F7Fu;
        if (slab + 1 < n_slabs) {
            load_x(slab + 1, xr);
            load_w(slab + 1, ng, nu, ns);
        }
        if (has_rows) {
            const float sg = e8m0_to_f32(ws & 0xFF), su = e8m0_to_f32((ws >> 8) & 0xFF);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 ag = fp4x8_bf16(wg[st], sg), au = fp4x8_bf16(wu[st], su);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (s < n_sub) {
                        const bf16x8 b = lds_bf16x8(&L.x[buf][s * kSub + r][32 * half + 8 * st]);
                        acc_g[s] = mfma_bf16(ag, b, acc_g[s]);
                        acc_u[s] = mfma_bf16(au, b, acc_u[s]);
                    }
                }
            }
        }
        if (slab + 1 < n_slabs) store_x(buf ^ 1, xr);
        __syncthreads();
        wg = ng;
        wu = nu;
        ws = ns;
    }

    if (!has_rows) return;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int row = s * kSub + r;
        if (s >= n_sub || row >= it.rows) continue;
        const size_t pr = (size_t)(pair0 + row) * I;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            uint32_t hi2[2], lo2[2];
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                uint16_t hb[2], lb[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const float g = acc_g[s][4 * r4 + e + d], u = acc_u[s][4 * r4 + e + d];
                    const float h = g / (1.f + expf(-g)) * u;
                    hb[d] = f32_to_bf16_rne(h);
                    lb[d] = f32_to_bf16_rne(h - bf16_to_f32(hb[d]));
                }
                hi2[e / 2] = hb[0] | ((uint32_t)hb[1] << 16);
                lo2[e / 2] = lb[0] | ((uint32_t)lb[1] << 16);
            }
            const int n = n0 + 8 * r4 + 4 * half;
            *reinterpret_cast<u32x2*>(h_hi + pr + n) = u32x2{hi2[0], hi2[1]};
            *reinterpret_cast<u32x2*>(h_lo + pr + n) = u32x2{lo2[0], lo2[1]};
        }
    }
}

// ----------------------------------------------------------------------------
// down: block = (tile, 128 output rows); wave w owns output rows 32w..32w+31.
// Both halves of h go through the same weights into one accumulator.

template <int NS>
struct DownLds {
    uint16_t h[2][2][NS * kSub][kLdsRow];   // [buffer][hi, lo][token][k]
};

template <int NS>
__global__ __launch_bounds__(kThreads, 2) void down_kernel(
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales, size_t e_codes,
    size_t e_scales, const uint8_t* __restrict__ sh_codes, const uint8_t* __restrict__ sh_scales,
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int H, int I, int E,
    const int32_t* __restrict__ n_tiles, const int2* __restrict__ tiles, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ off, float* __restrict__ y_pair) {
    constexpr int TT = NS * kSub;
    constexpr int kUnits = TT * (kSlab / 8) / kThreads;
    __shared__ __align__(16) DownLds<NS> L;

    Item it;
    if (!block_item(n_tiles, tiles, counts, (H + kRowsPerBlock - 1) / kRowsPerBlock, TT, it)) return;

    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id_uniform();
    const int kb4 = (I / 32 + 3) / 4, n_slabs = 2 * kb4;
    const int n_sub = (it.rows + kSub - 1) / kSub;
    const int pair0 = off[it.group] + it.start;

    auto load_h = [&](int slab, u32x4 (&rh)[kUnits], u32x4 (&rl)[kUnits]) {
#pragma unroll
        for (int v = 0; v < kUnits; ++v) {
            const int u = tid + kThreads * v, row = u >> 3;
            const int k0 = slab * kSlab + (u & 7) * 8;
            if (row < it.rows && k0 < I) {
                const size_t o = (size_t)(pair0 + row) * I + k0;
                rh[v] = *reinterpret_cast<const u32x4*>(h_hi + o);
                rl[v] = *reinterpret_cast<const u32x4*>(h_lo + o);
            } else {
                rh[v] = u32x4{0u, 0u, 0u, 0u};
                rl[v] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_h = [&](int buf, const u32x4 (&rh)[kUnits], const u32x4 (&rl)[kUnits]) {
#pragma unroll
        for (int v = 0; v < kUnits; ++v) {
            const int u = tid + kThreads * v;
            *reinterpret_cast<u32x4*>(&L.h[buf][0][u >> 3][(u & 7) * 8]) = rh[v];
            *reinterpret_cast<u32x4*>(&L.h[buf][1][u >> 3][(u & 7) * 8]) = rl[v];
        }
    };

    const int n0 = it.rb * kRowsPerBlock + 32 * wv;
    const bool has_rows = n0 < H;
    const uint8_t* cbase = it.group < E ? dn_codes + (size_t)it.group * e_codes : sh_codes;
    const uint8_t* sbase = it.group < E ? dn_scales + (size_t)it.group * e_scales : sh_scales;
    const int r = lane & 31, half = lane >> 5;
    const size_t unit = (size_t)(n0 / 16 + (r >> 4));
    const int li0 = (r & 15) + 16 * half;
    auto load_w = [&](int slab, u32x4& w, uint32_t& sc) {
        if (!has_rows) return;
        const int c = slab >> 1, li = li0 + 32 * (slab & 1);
        w = load_stream16(cbase + (unit * kb4 + c) * 1024 + li * 16);
        sc = sbase[(unit * kb4 + c) * 64 + li];
    };

    f32x16 acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = f32x16{};

    u32x4 hr[kUnits], lr[kUnits];
    u32x4 w = {0u, 0u, 0u, 0u};
    uint32_t ws = 0x7Fu;
    load_h(0, hr, lr);
    load_w(0, w, ws);
    store_h(0, hr, lr);
    __syncthreads();

    for (int slab = 0; slab < n_slabs; ++slab) {
        const int buf = slab & 1;
        u32x4 nw = {0u, 0u, 0u, 0u};
        uint32_t ns = 0x7Fu;
        if (slab + 1 < n_slabs) {
            load_h(slab + 1, hr, lr);
            load_w(slab + 1, nw, ns);
        }
        if (has_rows) {
            const float sc = e8m0_to_f32(ws & 0xFF);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 a = fp4x8_bf16(w[st], sc);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (s < n_sub) {
                        const bf16x8 bh = lds_bf16x8(&L.h[buf][0][s * kSub + r][32 * half + 8 * st]);
                        const bf16x8 bl = lds_bf16x8(&L.h[buf][1][s * kSub + r][32 * half + 8 * st]);
                        acc[s] = mfma_bf16(a, bh, acc[s]);
                        acc[s] = mfma_bf16(a, bl, acc[s]);
                    }
                }
            }
        }
        if (slab + 1 < n_slabs) store_h(buf ^ 1, hr, lr);
        __syncthreads();
        w = nw;
        ws = ns;
    }

    if (!has_rows) return;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int row = s * kSub + r;
        if (s >= n_sub || row >= it.rows) continue;
        float* dst = y_pair + (size_t)(pair0 + row) * H + n0 + 4 * half;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<float4*>(dst + 8 * r4) =
                float4{acc[s][4 * r4], acc[s][4 * r4 + 1], acc[s][4 * r4 + 2], acc[s][4 * r4 + 3]};
    }
}

// ----------------------------------------------------------------------------
// combine: one thread per 4 consecutive outputs of one token.

__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y_pair,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ wts, int T, int k, int H,
                                                           int shared_row0, uint16_t* __restrict__ y_bf16,
                                                           float* __restrict__ y_f32) {
    const int q = H / 4;
    for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < (size_t)T * q;
         i += (size_t)gridDim.x * kThreads) {
        const int t = (int)(i / q), n = (int)(i - (size_t)t * q) * 4;
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const float wj = wts[(size_t)t * k + j];
            const float4 v = *reinterpret_cast<const float4*>(y_pair + (size_t)pos[(size_t)t * k + j] * H + n);
            acc.x = fmaf(wj, v.x, acc.x);
            acc.y = fmaf(wj, v.y, acc.y);
            acc.z = fmaf(wj, v.z, acc.z);
            acc.w = fmaf(wj, v.w, acc.w);
        }
        const float4 v = *reinterpret_cast<const float4*>(y_pair + (size_t)(shared_row0 + t) * H + n);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
        const size_t o = (size_t)t * H + n;
        if (y_f32) *reinterpret_cast<float4*>(y_f32 + o) = acc;
        const uint32_t b0 = f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
        const uint32_t b1 = f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
        *reinterpret_cast<u32x2*>(y_bf16 + o) = u32x2{b0, b1};
    }
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int grid_cap(size_t work, int cap) {
    const size_t g = (work + kThreads - 1) / kThreads;
    return (int)(g < (size_t)cap ? (g ? g : 1) : cap);
}

template <int NS>
hipError_t launch_gemms(const moedec_moe_weights& w, const uint16_t* x, const PrefillLayout& lay,
                        uint8_t* base, hipStream_t s) {
    moedec_mxfp4_sizes sz;
    packed_sizes(w.H, w.I, &sz);
    const int32_t* n_tiles = reinterpret_cast<const int32_t*>(base + lay.n_tiles_off);
    const int2* tiles = reinterpret_cast<const int2*>(base + lay.tiles_off);
    const int32_t* counts = reinterpret_cast<const int32_t*>(base + lay.counts_off);
    const int32_t* off = reinterpret_cast<const int32_t*>(base + lay.off_off);
    const int32_t* tok_of = reinterpret_cast<const int32_t*>(base + lay.tok_of_off);
    uint16_t* h_hi = reinterpret_cast<uint16_t*>(base + lay.h_hi_off);
    uint16_t* h_lo = reinterpret_cast<uint16_t*>(base + lay.h_lo_off);
    float* y_pair = reinterpret_cast<float*>(base + lay.y_pair_off);

    const size_t gu_items = (size_t)lay.max_tiles * ((w.I + kRowsPerBlock - 1) / kRowsPerBlock);
    hipLaunchKernelGGL(gateup_kernel<NS>, dim3((unsigned)(kXcds * ((gu_items + kXcds - 1) / kXcds))),
                       dim3(kThreads), 0, s, static_cast<const uint8_t*>(w.gu_codes),
                       reinterpret_cast<const uint16_t*>(w.gu_scales), sz.gu_codes, sz.gu_scales,
                       static_cast<const uint8_t*>(w.sh_gu_codes), reinterpret_cast<const uint16_t*>(w.sh_gu_scales),
                       x, w.H, w.I, w.E, n_tiles, tiles, counts, off, tok_of, h_hi, h_lo);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t dn_items = (size_t)lay.max_tiles * ((w.H + kRowsPerBlock - 1) / kRowsPerBlock);
    hipLaunchKernelGGL(down_kernel<NS>, dim3((unsigned)(kXcds * ((dn_items + kXcds - 1) / kXcds))),
                       dim3(kThreads), 0, s, static_cast<const uint8_t*>(w.dn_codes),
                       static_cast<const uint8_t*>(w.dn_scales), sz.dn_codes, sz.dn_scales,
                       static_cast<const uint8_t*>(w.sh_dn_codes), static_cast<const uint8_t*>(w.sh_dn_scales),
                       h_hi, h_lo, w.H, w.I, w.E, n_tiles, tiles, counts, off, y_pair);
    return hipGetLastError();
}

}  // namespace

int prefill_sub_tiles(int T, int E, int k) {
    const long avg = (long)T * k / E;   // tokens per routed expert on average
    return avg >= 64 ? 4 : (avg >= 24 ? 2 : 1);
}

PrefillLayout prefill_layout(int T, int E, int k, int H, int I) {
    PrefillLayout l{};
    l.ns = prefill_sub_tiles(T, E, k);
    const int tile_tokens = l.ns * kSub;
    const size_t P = (size_t)T * k + T, G = (size_t)E + 1;
    l.max_tiles = (int)(P / tile_tokens + G);
    size_t o = 0;
    l.counts_off = o;   o = align256(o + (G + 1) * 4);
    l.cursor_off = o;   o = align256(o + (G + 1) * 4);
    l.off_off = o;      o = align256(o + (G + 1) * 4);
    l.n_tiles_off = o;  o = align256(o + 4);
    l.tiles_off = o;    o = align256(o + (size_t)l.max_tiles * 8);
    l.ids_off = o;      o = align256(o + (size_t)T * k * 4);
    l.w_off = o;        o = align256(o + (size_t)T * k * 4);
    l.pos_off = o;      o = align256(o + (size_t)T * k * 4);
    l.tok_of_off = o;   o = align256(o + P * 4);
    l.h_hi_off = o;     o = align256(o + P * I * 2);
    l.h_lo_off = o;     o = align256(o + P * I * 2);
    l.y_pair_off = o;   o = align256(o + P * H * 4);
    l.total = o;
    return l;
}

hipError_t launch_prefill(const moedec_moe_weights& w, const uint16_t* x, const float* logits, int T, int k,
                          int32_t* ids_out, float* w_out, int32_t* counts_out, uint16_t* y_bf16, float* y_f32,
                          void* ws, hipStream_t s) {
    const PrefillLayout lay = prefill_layout(T, w.E, k, w.H, w.I);
    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(base + lay.counts_off);
    int32_t* cursor = reinterpret_cast<int32_t*>(base + lay.cursor_off);
    int32_t* off = reinterpret_cast<int32_t*>(base + lay.off_off);
    int32_t* ids = ids_out ? ids_out : reinterpret_cast<int32_t*>(base + lay.ids_off);
    float* wts = w_out ? w_out : reinterpret_cast<float*>(base + lay.w_off);
    const int G = w.E + 1;

    hipLaunchKernelGGL(zero_counts_kernel, dim3(grid_cap(G + 1, 8)), dim3(kThreads), 0, s, counts, cursor, G + 1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 rgrid((T + kThreads / kWave - 1) / (kThreads / kWave));
    if (w.E <= 512)
        hipLaunchKernelGGL(route_count_kernel<8>, rgrid, dim3(kThreads), 0, s, logits, T, w.E, k, ids, wts, counts);
    else
        hipLaunchKernelGGL(route_count_kernel<16>, rgrid, dim3(kThreads), 0, s, logits, T, w.E, k, ids, wts, counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, s, counts, w.E, T, lay.ns * kSub, off,
                       reinterpret_cast<int2*>(base + lay.tiles_off),
                       reinterpret_cast<int32_t*>(base + lay.n_tiles_off), counts_out);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    int32_t* pos = reinterpret_cast<int32_t*>(base + lay.pos_off);
    hipLaunchKernelGGL(scatter_kernel, dim3(grid_cap((size_t)T * (k + 1), 4096)), dim3(kThreads), 0, s, ids, T, k,
                       off, cursor, reinterpret_cast<int32_t*>(base + lay.tok_of_off), pos, w.E);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    switch (lay.ns) {
        case 4: err = launch_gemms<4>(w, x, lay, base, s); break;
        case 2: err = launch_gemms<2>(w, x, lay, base, s); break;
        default: err = launch_gemms<1>(w, x, lay, base, s); break;
    }
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(combine_kernel, dim3(grid_cap((size_t)T * (w.H / 4), 8192)), dim3(kThreads), 0, s,
                       reinterpret_cast<const float*>(base + lay.y_pair_off), pos, wts, T, k, w.H, T * k, y_bf16,
                       y_f32);
    return hipGetLastError();
}

}  // namespace moedec
