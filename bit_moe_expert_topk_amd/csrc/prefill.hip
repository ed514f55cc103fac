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
//   route    one wave per token: top-k of its logits (route_device.h) and
//            the routing weights
//   count    the routed pairs in chunks: per-chunk expert counts in LDS
//   plan     one block: a column scan of the chunk counts into per-expert
//            totals and each chunk's first row inside every expert's group,
//            then an exclusive scan of the totals into pair offsets, and the
//            tile list (group, first row) in units of 32*NS tokens
//   scatter  each (token, choice) pair gets a row in its expert's group; the
//            shared group holds token t at row T*k + t
//   gate/up  per (tile, 128 intermediate rows): g = W_gate x, u = W_up x on
//            MFMA 32x32x16 bf16 with float32 accumulation, h = silu(g) * u,
//            stored as h = hi + lo (two bf16, 16 significant bits)
//   down     per (up to 64 tokens of a tile, 256 output rows): y_pair =
//            W_down hi + W_down lo
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
// The W4A8 variant (moe_layer_mxfp4_prefill_a8) runs the same steps with
// MXFP8 activations: x quantised once (in the routing launch), gate/up and
// down on the block-scaled fp4 x fp8 matrix instruction, h quantised in the
// gate/up epilogue; see the W4A8 section below.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kSub = 32;             // tokens per MFMA column block
constexpr int kSlab = 64;            // k per pipeline step: two MX blocks
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

// One wave per token (block `blk` takes tokens 4 blk .. 4 blk + 3).
template <int KPL>
__device__ __forceinline__ void route_body(const float* __restrict__ logits, int T, int E, int k,
                                           int32_t* __restrict__ ids, float* __restrict__ wts, int blk) {
    __shared__ uint64_t s_buf[kThreads / kWave][kTopkBufWords];
    const int wv = threadIdx.x >> 6, lane = lane_id();
    const int t = blk * (kThreads / kWave) + wv;
    if (t >= T) return;
    float w;
    const uint64_t key = wave_topk<KPL>(logits + (size_t)t * E, E, k, w, s_buf[wv]);
    if (lane < k) {
        ids[(size_t)t * k + lane] = key_to_index(key);
        wts[(size_t)t * k + lane] = w;
    }
}

template <int KPL>
__global__ __launch_bounds__(kThreads) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ wts) {
    route_body<KPL>(logits, T, E, k, ids, wts, blockIdx.x);
}

// Counting without device-scope atomics.  Those serialise per address: with
// E counters each one takes T*k/E atomics in a row, which made this step
// grow linearly with T (about 140 us for the routing of 32,768 tokens over
// 512 experts).  Instead the T*k routed pairs (token-major) are cut into
// n_chunks chunks of `chunk` pairs; block c counts its chunk's experts with
// LDS atomics and writes the row hist[c][0..E); a column scan gives every
// expert's total (counts) and each chunk's first row inside every group
// (base[c][e]); the scatter block of chunk c ranks its pairs in LDS again.
constexpr int kCountThreads = 1024;
constexpr int kMaxChunks = 64;
constexpr int kChunkMin = 2048;

__global__ __launch_bounds__(kCountThreads) void count_kernel(const int32_t* __restrict__ ids, int n_routed,
                                                              int chunk, int E, int32_t* __restrict__ hist) {
    __shared__ int s_cnt[MOEDEC_MAX_E];
    for (int e = threadIdx.x; e < E; e += kCountThreads) s_cnt[e] = 0;
    __syncthreads();
    const int first = blockIdx.x * chunk, last = min(n_routed, first + chunk);
    for (int i = first + threadIdx.x; i < last; i += kCountThreads) atomicAdd(&s_cnt[ids[i]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kCountThreads) hist[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// One block, thread e for routed expert e.  The column scan of the per-chunk
// counts (all of a column's loads in flight at once) gives each chunk's first
// row inside group e (base[c][e]) and the group's total; an exclusive scan
// over experts of the totals and of their tile counts (inside each wave by
// lane shifts, then over the wave totals) gives off[e], the group's first pair
// row, and its place in the tile list (group, first row) in steps of
// tile_tokens.  The shared group E holds T rows after every routed pair and
// its tiles come last; *n_tiles is the list's length.
static_assert(MOEDEC_MAX_E <= kCountThreads, "one plan thread per routed expert");

__global__ __launch_bounds__(kCountThreads) void plan_kernel(const int32_t* __restrict__ hist, int n_chunks, int E,
                                                             int T, int tile_tokens, int32_t* __restrict__ base,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ off, int2* __restrict__ tiles,
                                                             int32_t* __restrict__ n_tiles,
                                                             int32_t* __restrict__ counts_out) {
    constexpr int kWaves = kCountThreads / kWave;
    __shared__ int s_pairs[kWaves], s_tiles[kWaves];
    const int e = threadIdx.x, lane = lane_id(), wv = e / kWave;
    int cnt = 0;
    if (e < E) {
        int v[kMaxChunks];
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) v[c] = c < n_chunks ? hist[(size_t)c * E + e] : 0;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            if (c < n_chunks) base[(size_t)c * E + e] = cnt;
            cnt += v[c];
        }
    }
    const int nt = (cnt + tile_tokens - 1) / tile_tokens;
    int ip = cnt, it = nt;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int a = __shfl_up(ip, d), b = __shfl_up(it, d);
        if (lane >= d) {
            ip += a;
            it += b;
        }
    }
    if (lane == kWave - 1) {
        s_pairs[wv] = ip;
        s_tiles[wv] = it;
    }
    __syncthreads();
    int below_p = 0, below_t = 0, all_p = 0, all_t = 0;
    for (int i = 0; i < kWaves; ++i) {
        if (i < wv) {
            below_p += s_pairs[i];
            below_t += s_tiles[i];
        }
        all_p += s_pairs[i];
        all_t += s_tiles[i];
    }
    if (e < E) {
        counts[e] = cnt;
        off[e] = below_p + ip - cnt;
        if (counts_out) counts_out[e] = cnt;
        int q = below_t + it - nt;
        for (int r = 0; r < cnt; r += tile_tokens) tiles[q++] = int2{e, r};
    }
    const int shared_tiles = (T + tile_tokens - 1) / tile_tokens;
    for (int i = e; i < shared_tiles; i += kCountThreads) tiles[all_t + i] = int2{E, i * tile_tokens};
    if (e == 0) {
        counts[E] = T;
        off[E] = all_p;
        off[E + 1] = all_p + T;
        if (counts_out) counts_out[E] = T;
        *n_tiles = all_t + shared_tiles;
    }
}

// Block c places the pairs of chunk c: row = off[e] + base[c][e] + its rank
// among the chunk's pairs of expert e (LDS atomic, in arrival order; no value
// depends on the order of rows inside a group, each row of the products is
// computed on its own).  The blocks also write the shared group's rows.
__global__ __launch_bounds__(kCountThreads) void scatter_kernel(const int32_t* __restrict__ ids, int T, int k,
                                                                int chunk, const int32_t* __restrict__ off,
                                                                const int32_t* __restrict__ base,
                                                                int32_t* __restrict__ tok_of,
                                                                int32_t* __restrict__ pos, int E) {
    __shared__ int s_cnt[MOEDEC_MAX_E];
    for (int e = threadIdx.x; e < E; e += kCountThreads) s_cnt[e] = 0;
    __syncthreads();
    const int n_routed = T * k;
    const int first = blockIdx.x * chunk, last = min(n_routed, first + chunk);
    const int32_t* b = base + (size_t)blockIdx.x * E;
    for (int i = first + threadIdx.x; i < last; i += kCountThreads) {
        const int e = ids[i];
        const int row = off[e] + b[e] + atomicAdd(&s_cnt[e], 1);
        tok_of[row] = i / k;
        pos[i] = row;
    }
    const int shared0 = off[E];
    for (int t = blockIdx.x * kCountThreads + threadIdx.x; t < T; t += gridDim.x * kCountThreads)
        tok_of[shared0 + t] = t;
}

// ----------------------------------------------------------------------------
// Pipeline shared by both products.  Everything a step multiplies flows
// through a ring of LDS slots filled by direct global->LDS loads, each
// slot holding one 64-k slab: the B operand (activations, or the two halves of
// h) and each wave's own A-operand codes and scales.  A wave's load
// instruction writes 64 lanes x 16 B (or 4 B) contiguously, lane l at 16 l
// (4 l).  B rows are 128 B; inside a row the eight 16-byte units sit at slot
// u ^ ((row >> 1) & 7), so the 16 lanes that read one unit of 16 consecutive
// rows hit 16 distinct bank groups.
//
// With S slots, step j (j = 1 - S .. n_slabs - 1; the first S - 1 only
// fill): for j >= 0 wait until this thread's loads of slab j are done (loads
// retire in order, and only those of slabs j + 1 .. j + S - 2 were issued
// after them) and barrier (every thread's part of slab j is in LDS, every
// wave is done with slab j - 1); then load slab j + S - 1 into the slot slab
// j - 1 used and multiply slab j.  Loads past the last slab repeat the last
// one into that free slot, keeping every count fixed.  The step takes the slot it writes and the slot it reads as restrict
// pointers: that tells the compiler the ring write does not feed this step's
// LDS reads, so it adds no wait of its own between them.  No register is
// loaded from global memory inside the loop, so every vmcnt wait there is
// the one written here.

constexpr int kGuWaveBytes = 2048 + 256;    // gate codes, up codes, scale dwords
constexpr int kDnWaveBytes = 2048 + 512;    // codes of two row tiles, their scale dwords

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt at their no-wait values).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void lds_load16(const void* src, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ void lds_load4(const void* src, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}

__device__ __forceinline__ int lds_slot(int row, int unit) { return row * 128 + ((unit ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ bf16x8 lds_b(const uint8_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

template <int S>
__device__ __forceinline__ int next_slot(int s) { return s + 1 == S ? 0 : s + 1; }

// ----------------------------------------------------------------------------
// gate/up: block = (tile of up to 32*NS tokens of one group, 32*W intermediate
// rows); wave w owns rows 32w..32w+31 of that block for both W_gate and W_up.
// Each of the block's ceil(I / 32W) row blocks reads the tile's activations
// again (from L2), so wider blocks cut that traffic.

template <int NS, int W>
struct GuCtx {
    static constexpr int kX = NS * kSub * 128 / (8 * 128 * W);   // ring-fill instructions per wave
    const uint16_t* xsrc[kX];   // token row of this lane's ring unit, instruction v
    int xk[kX];                 // its k offset inside a slab
    const uint8_t* codes;       // this lane's 16 code bytes of MX block q = half of chunk 0
    const uint8_t* scales;      // the scale dword holding this lane's 16-bit gate/up scale pair, chunk 0
    int n_slabs, H, wv, lane;
    int sc_shift;               // 0 or 16: this lane's half of the scale dword
    bool has_rows;
    int boff[4];                // LDS offsets of this lane's B operand, steps 0..3
};

template <int NS, int W, int S, int NSUB>
__device__ __forceinline__ void gu_step(uint8_t* __restrict__ wr, const uint8_t* __restrict__ rd,
                                        const GuCtx<NS, W>& c, int j, f32x16 (&acc_g)[NS], f32x16 (&acc_u)[NS]) {
    constexpr int kX = NS * kSub * 128;
    {
        const int sl = min(j + S - 1, c.n_slabs - 1);
#pragma unroll
        for (int v = 0; v < GuCtx<NS, W>::kX; ++v) {
            const int k = sl * kSlab + c.xk[v];
            lds_load16(c.xsrc[v] + (k < c.H ? k : 0), wr + (W * v + c.wv) * 1024);
        }
        if (c.has_rows) {
            uint8_t* wb = wr + kX + c.wv * kGuWaveBytes;
            const uint8_t* p = c.codes + (size_t)(sl >> 1) * 2048 + (sl & 1) * 512;
            lds_load16(p, wb);
            lds_load16(p + 1024, wb + 1024);
            lds_load4(c.scales + (size_t)(sl >> 1) * 128 + (sl & 1) * 64, wb + 2048);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (c.has_rows && j >= 0) {
        // every LDS read of the slab first (weights, then B in the order the
        // products use them), so the matrix core never waits on one
        const uint8_t* wb = rd + kX + c.wv * kGuWaveBytes;
        const u32x4 cg = *reinterpret_cast<const u32x4*>(wb + c.lane * 16);
        const u32x4 cu = *reinterpret_cast<const u32x4*>(wb + 1024 + c.lane * 16);
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(wb + 2048 + c.lane * 4) >> c.sc_shift;
        bf16x8 b[4][NSUB];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int s = 0; s < NSUB; ++s) b[st][s] = lds_b(rd + s * kSub * 128 + c.boff[st]);
        const float sg = e8m0_to_f32(sc & 0xFF), su = e8m0_to_f32((sc >> 8) & 0xFF);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf16x8 ag = fp4x8_bf16(cg[st], sg), au = fp4x8_bf16(cu[st], su);
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                acc_g[s] = mfma_bf16(ag, b[st][s], acc_g[s]);
                acc_u[s] = mfma_bf16(au, b[st][s], acc_u[s]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int NS, int W>
constexpr int gu_slot_bytes() { return NS * kSub * 128 + W * kGuWaveBytes; }

template <int NS, int W, int S, int NSUB>
__device__ __forceinline__ void gu_main(uint8_t (&ring)[S][(gu_slot_bytes<NS, W>())], const GuCtx<NS, W>& c,
                                        f32x16 (&acc_g)[NS], f32x16 (&acc_u)[NS]) {
    constexpr int kG = GuCtx<NS, W>::kX;   // loads per fill without weights
    int ws = 0, rs = 1;                    // slot written, slot read (nothing read before j = 0)
    for (int j = 1 - S; j < c.n_slabs; ++j) {
        if (j >= 0) {
            if (c.has_rows) wait_vm<(S - 2) * (kG + 3)>(); else wait_vm<(S - 2) * kG>();
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        gu_step<NS, W, S, NSUB>(&ring[ws][0], &ring[rs][0], c, j, acc_g, acc_u);
        ws = next_slot<S>(ws);
        rs = next_slot<S>(rs);
    }
    wait_vm<0>();    // no ring write may land after the block's LDS is released
}

template <int NS, int W, int S>
__global__ __launch_bounds__(64 * W) void gateup_kernel(
    const uint8_t* __restrict__ gu_codes, const uint8_t* __restrict__ gu_scales, size_t e_codes,
    size_t e_scales, const uint8_t* __restrict__ sh_codes, const uint8_t* __restrict__ sh_scales,
    const uint16_t* __restrict__ x, int H, int I, int E, const int32_t* __restrict__ n_tiles,
    const int2* __restrict__ tiles, const int32_t* __restrict__ counts, const int32_t* __restrict__ off,
    const int32_t* __restrict__ tok_of, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
    constexpr int TT = NS * kSub;
    static_assert(GuCtx<NS, W>::kX >= 1, "every wave fills part of each slab");
    __shared__ __align__(1024) uint8_t ring[S][(gu_slot_bytes<NS, W>())];

    Item it;
    if (!block_item(n_tiles, tiles, counts, (I + 32 * W - 1) / (32 * W), TT, it)) return;

    const int lane = lane_id(), wv = wave_id_uniform();
    const int n_sub = (it.rows + kSub - 1) / kSub;
    const int pair0 = off[it.group] + it.start;
    const int r = lane & 31, half = lane >> 5;
    const int kb4 = (H / 32 + 3) / 4;

    GuCtx<NS, W> c;
    c.n_slabs = 2 * kb4;
    c.H = H;
    c.wv = wv;
    c.lane = lane;
#pragma unroll
    for (int v = 0; v < GuCtx<NS, W>::kX; ++v) {
        const int row = 8 * (W * v + wv) + (lane >> 3);
        c.xsrc[v] = x + (size_t)tok_of[pair0 + min(row, it.rows - 1)] * H;
        c.xk[v] = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
    }
    const int n0 = it.rb * 32 * W + 32 * wv;
    c.has_rows = n0 < I;
    {
        const uint8_t* cb = it.group < E ? gu_codes + (size_t)it.group * e_codes : sh_codes;
        const uint8_t* sb = it.group < E ? gu_scales + (size_t)it.group * e_scales : sh_scales;
        const size_t unit = (size_t)(n0 / 16 + (r >> 4));
        const int li0 = (r & 15) + 16 * half;
        c.codes = cb + unit * kb4 * 2048 + li0 * 16;
        c.scales = sb + unit * kb4 * 128 + ((2 * li0) & ~3);   // 16-bit scale pairs, dword holding li0
        c.sc_shift = 16 * (li0 & 1);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) c.boff[st] = lds_slot(r, 4 * half + st);

    f32x16 acc_g[NS], acc_u[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        acc_g[s] = f32x16{};
        acc_u[s] = f32x16{};
    }
    if (NS == 4 && n_sub == 4) gu_main<NS, W, S, (NS >= 4 ? 4 : 1)>(ring, c, acc_g, acc_u);
    else if (NS >= 3 && n_sub == 3) gu_main<NS, W, S, (NS >= 3 ? 3 : 1)>(ring, c, acc_g, acc_u);
    else if (NS >= 2 && n_sub == 2) gu_main<NS, W, S, (NS >= 2 ? 2 : 1)>(ring, c, acc_g, acc_u);
    else gu_main<NS, W, S, 1>(ring, c, acc_g, acc_u);

    if (!c.has_rows) return;
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
// down: block = (32*ND tokens of a gate/up tile, 64*W output rows); wave w
// owns output rows 64w..64w+63 as two 32-row MFMA tiles.  A gate/up tile of TT
// tokens splits into TT / (32 ND) parts.  Both halves of h go through the same
// weights into one accumulator.

template <int ND, int W>
struct DnCtx {
    static constexpr int kX = ND * kSub * 128 / (8 * 128 * W);   // ring-fill instructions per wave and plane
    size_t hrow[kX];
    int hk[kX];
    const uint16_t* h_hi;
    const uint16_t* h_lo;
    const uint8_t* codes0;    // row tile 0; tile 1 is two units (2 * kb4 chunks) further
    const uint8_t* scales0;   // the scale dword holding this lane's byte, chunk 0
    size_t t1_codes, t1_scales;
    int n_slabs, I, wv, lane;
    int sc_shift;
    bool has_rows;
    int boff[4];
};

template <int ND, int W>
constexpr int dn_slot_bytes() { return 2 * ND * kSub * 128 + W * kDnWaveBytes; }

template <int ND, int W, int S, int NSUB>
__device__ __forceinline__ void dn_step(uint8_t* __restrict__ wr, const uint8_t* __restrict__ rd,
                                        const DnCtx<ND, W>& c, int j, f32x16 (&acc)[2][ND]) {
    constexpr int kPlane = ND * kSub * 128;
    {
        const int sl = min(j + S - 1, c.n_slabs - 1);
#pragma unroll
        for (int v = 0; v < DnCtx<ND, W>::kX; ++v) {
            const int k = sl * kSlab + c.hk[v];
            const size_t o = c.hrow[v] + (k < c.I ? k : 0);
            lds_load16(c.h_hi + o, wr + (W * v + c.wv) * 1024);
            lds_load16(c.h_lo + o, wr + kPlane + (W * v + c.wv) * 1024);
        }
        if (c.has_rows) {
            uint8_t* wb = wr + 2 * kPlane + c.wv * kDnWaveBytes;
            const uint8_t* p = c.codes0 + (size_t)(sl >> 1) * 1024 + (sl & 1) * 512;
            const uint8_t* s = c.scales0 + (size_t)(sl >> 1) * 64 + (sl & 1) * 32;
            lds_load16(p, wb);
            lds_load16(p + c.t1_codes, wb + 1024);
            lds_load4(s, wb + 2048);
            lds_load4(s + c.t1_scales, wb + 2304);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (c.has_rows && j >= 0) {
        const uint8_t* wb = rd + 2 * kPlane + c.wv * kDnWaveBytes;
        const u32x4 c0 = *reinterpret_cast<const u32x4*>(wb + c.lane * 16);
        const u32x4 c1 = *reinterpret_cast<const u32x4*>(wb + 1024 + c.lane * 16);
        const uint32_t w0 = *reinterpret_cast<const uint32_t*>(wb + 2048 + c.lane * 4);
        const uint32_t w1 = *reinterpret_cast<const uint32_t*>(wb + 2304 + c.lane * 4);
        bf16x8 bh[4][NSUB], bl[4][NSUB];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                const uint8_t* p = rd + s * kSub * 128 + c.boff[st];
                bh[st][s] = lds_b(p);
                bl[st][s] = lds_b(p + kPlane);
            }
        const float s0 = e8m0_to_f32((w0 >> c.sc_shift) & 0xFF), s1 = e8m0_to_f32((w1 >> c.sc_shift) & 0xFF);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf16x8 a0 = fp4x8_bf16(c0[st], s0), a1 = fp4x8_bf16(c1[st], s1);
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                acc[0][s] = mfma_bf16(a0, bh[st][s], acc[0][s]);
                acc[1][s] = mfma_bf16(a1, bh[st][s], acc[1][s]);
                acc[0][s] = mfma_bf16(a0, bl[st][s], acc[0][s]);
                acc[1][s] = mfma_bf16(a1, bl[st][s], acc[1][s]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int ND, int W, int S, int NSUB>
__device__ __forceinline__ void dn_main(uint8_t (&ring)[S][(dn_slot_bytes<ND, W>())], const DnCtx<ND, W>& c,
                                        f32x16 (&acc)[2][ND]) {
    constexpr int kG = 2 * DnCtx<ND, W>::kX;
    int ws = 0, rs = 1;
    for (int j = 1 - S; j < c.n_slabs; ++j) {
        if (j >= 0) {
            if (c.has_rows) wait_vm<(S - 2) * (kG + 4)>(); else wait_vm<(S - 2) * kG>();
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        dn_step<ND, W, S, NSUB>(&ring[ws][0], &ring[rs][0], c, j, acc);
        ws = next_slot<S>(ws);
        rs = next_slot<S>(rs);
    }
    wait_vm<0>();
}

template <int ND, int W, int S>
__global__ __launch_bounds__(64 * W) void down_kernel(
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales, size_t e_codes,
    size_t e_scales, const uint8_t* __restrict__ sh_codes, const uint8_t* __restrict__ sh_scales,
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int H, int I, int E, int tile_tokens,
    const int32_t* __restrict__ n_tiles, const int2* __restrict__ tiles, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ off, float* __restrict__ y_pair) {
    constexpr int TD = ND * kSub;
    static_assert(DnCtx<ND, W>::kX >= 1, "every wave fills part of each slab");
    __shared__ __align__(1024) uint8_t ring[S][(dn_slot_bytes<ND, W>())];

    const int parts = tile_tokens / TD, n_rb = (H + 64 * W - 1) / (64 * W);
    Item it;
    if (!block_item(n_tiles, tiles, counts, parts * n_rb, tile_tokens, it)) return;
    const int part = it.rb / n_rb;
    it.rb -= part * n_rb;
    it.rows = min(it.rows - part * TD, TD);
    if (it.rows <= 0) return;
    it.start += part * TD;

    const int lane = lane_id(), wv = wave_id_uniform();
    const int n_sub = (it.rows + kSub - 1) / kSub;
    const int pair0 = off[it.group] + it.start;
    const int r = lane & 31, half = lane >> 5;
    const int kb4 = (I / 32 + 3) / 4;

    DnCtx<ND, W> c;
    c.n_slabs = 2 * kb4;
    c.I = I;
    c.wv = wv;
    c.lane = lane;
    c.h_hi = h_hi;
    c.h_lo = h_lo;
#pragma unroll
    for (int v = 0; v < DnCtx<ND, W>::kX; ++v) {
        const int row = 8 * (W * v + wv) + (lane >> 3);
        c.hrow[v] = (size_t)(pair0 + min(row, it.rows - 1)) * I;
        c.hk[v] = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
    }
    const int n0 = it.rb * 64 * W + 64 * wv;
    c.has_rows = n0 < H;
    {
        const uint8_t* cb = it.group < E ? dn_codes + (size_t)it.group * e_codes : sh_codes;
        const uint8_t* sb = it.group < E ? dn_scales + (size_t)it.group * e_scales : sh_scales;
        const size_t unit = (size_t)(n0 / 16 + (r >> 4));
        const int li0 = (r & 15) + 16 * half;
        c.codes0 = cb + unit * kb4 * 1024 + li0 * 16;
        c.scales0 = sb + unit * kb4 * 64 + (li0 & ~3);
        c.sc_shift = 8 * (li0 & 3);
        c.t1_codes = (size_t)2 * kb4 * 1024;
        c.t1_scales = (size_t)2 * kb4 * 64;
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) c.boff[st] = lds_slot(r, 4 * half + st);

    f32x16 acc[2][ND];
#pragma unroll
    for (int s = 0; s < ND; ++s) {
        acc[0][s] = f32x16{};
        acc[1][s] = f32x16{};
    }
    if (ND == 2 && n_sub == 2) dn_main<ND, W, S, (ND >= 2 ? 2 : 1)>(ring, c, acc);
    else dn_main<ND, W, S, 1>(ring, c, acc);

    if (!c.has_rows) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int s = 0; s < ND; ++s) {
            const int row = s * kSub + r;
            if (s >= n_sub || row >= it.rows) continue;
            float* dst = y_pair + (size_t)(pair0 + row) * H + n0 + 32 * t + 4 * half;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<float4*>(dst + 8 * r4) =
                    float4{acc[t][s][4 * r4], acc[t][s][4 * r4 + 1], acc[t][s][4 * r4 + 2], acc[t][s][4 * r4 + 3]};
        }
    }
}

// ----------------------------------------------------------------------------
// W4A8: MXFP8 activations (E4M3 elements, one E8M0 scale per 32 values along
// the reduction axis) into v_mfma_scale_f32_32x32x64_f8f6f4, A = the MXFP4
// weights as stored (E2M1 codes and their E8M0 bytes, no conversion), B = the
// activations.  Operand lanes (checked with an in-bounds probe): A lane l =
// row l % 32 with the 32 codes of MX block l / 32 of the 64-k step (the packed
// layout's 16-byte lane chunk) and that block's scale; B lane l = column
// l % 32 with k 16 (l/32) .. +15 and 32 + 16 (l/32) .. +15, and the scale of
// block l / 32.  D as for the bf16 MFMA.
//
// x is quantised by quant_x8_body ([T][H] codes, [T][SB] scale bytes, SB = 4 *
// ceil(H/128), padding blocks 127); h by the gate/up epilogue ([P][I] codes,
// [P][SBI] scale bytes): the 32 rows of a wave's MFMA tile are one MX block of
// h for each token, split over lanes l and l ^ 32.  Per slab the ring carries
// the activation codes (64 B per token row, in 1 KB pieces of 16 rows spread
// over the waves), the rows' scale dwords of the slab's 128-k chunk, and each
// wave's weights (A8Ring below).

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The MXFP8 scale rule and encoder (mx8_scale_byte, mx8_inv, mx8_code) are in
// device_common.h, shared with the decode layer.

__device__ __forceinline__ f32x16 mfma_a4b8(const u32x4& a, const i32x8& b, uint32_t sa, uint32_t sb, f32x16 c) {
    const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, b, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

// One thread per 32-value block of one token; blocks blk = 0 .. nblk - 1 of
// the launch stride over them.
__device__ __forceinline__ void quant_x8_body(const uint16_t* __restrict__ x, int T, int H, int sb,
                                              uint8_t* __restrict__ x8, uint8_t* __restrict__ xs, int blk,
                                              int nblk) {
    const int nb = H / 32;
    for (size_t i = blk * (size_t)kThreads + threadIdx.x; i < (size_t)T * sb; i += (size_t)nblk * kThreads) {
        const int t = (int)(i / sb), b = (int)(i - (size_t)t * sb);
        if (b >= nb) {
            xs[i] = 127;
            continue;
        }
        const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)t * H + b * 32);
        u32x4 d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = src[q];
        uint32_t am = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) am = max(am, max(d[q][e] & 0x7FFFu, (d[q][e] >> 16) & 0x7FFFu));
        const uint32_t sbyte = mx8_scale_byte(am << 16);
        const float inv = mx8_inv(sbyte);
        u32x4 o[2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const uint32_t w0 = d[q][e], w1 = d[q][e + 1];
                const uint32_t c = mx8_code(bf16_to_f32(w0 & 0xFFFFu), inv) |
                                   (mx8_code(bf16_to_f32(w0 >> 16), inv) << 8) |
                                   (mx8_code(bf16_to_f32(w1 & 0xFFFFu), inv) << 16) |
                                   (mx8_code(bf16_to_f32(w1 >> 16), inv) << 24);
                o[q >> 1][(q & 1) * 2 + (e >> 1)] = c;
            }
        u32x4* dst = reinterpret_cast<u32x4*>(x8 + (size_t)t * H + b * 32);
        dst[0] = o[0];
        dst[1] = o[1];
        xs[i] = (uint8_t)sbyte;
    }
}

// The W4A8 call's first launch: blocks [0, route_blocks) route (route_body),
// the others quantise x (quant_x8_body).  The two read different inputs, so
// the routing's latency-bound waves and the quantisation's streaming share
// one grid instead of following each other.
template <int KPL>
__global__ __launch_bounds__(kThreads) void route_quant_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                               int32_t* __restrict__ ids, float* __restrict__ wts,
                                                               int route_blocks, const uint16_t* __restrict__ x,
                                                               int H, int sb, uint8_t* __restrict__ x8,
                                                               uint8_t* __restrict__ xs) {
    if ((int)blockIdx.x < route_blocks)
        route_body<KPL>(logits, T, E, k, ids, wts, blockIdx.x);
    else
        quant_x8_body(x, T, H, sb, x8, xs, blockIdx.x - route_blocks, gridDim.x - route_blocks);
}

// Activation rows in a ring slot: 64 B per row, 16-byte unit u at u ^ ((row >> 2) & 3).
__device__ __forceinline__ int a8_slot(int row, int unit) { return row * 64 + ((unit ^ ((row >> 2) & 3)) << 4); }

// The B operand of row `row`: units h and 2 + h.
__device__ __forceinline__ i32x8 a8_b(const uint8_t* base, int row, int half) {
    const u32x4 p = *reinterpret_cast<const u32x4*>(base + a8_slot(row, half));
    const u32x4 q = *reinterpret_cast<const u32x4*>(base + a8_slot(row, 2 + half));
    return i32x8{(int)p[0], (int)p[1], (int)p[2], (int)p[3], (int)q[0], (int)q[1], (int)q[2], (int)q[3]};
}

// Ring slot of the W4A8 products: the activation codes (64 B per token row:
// 16-byte unit u at u ^ ((row >> 2) & 3)), the rows' scale dwords of the
// slab's 128-k chunk (row r at 4 r; kScW waves load them, 64 rows each),
// then each wave's weights.  A wave's fill is 1 code load, 1 scale load if
// it is one of the first kScW waves, and its weight loads.
template <int TR>
struct A8Ring {
    static constexpr int kCodes = TR * 64;
    static constexpr int kScales = TR * 4 < 256 ? 256 : TR * 4;
    static constexpr int kScW = kScales / 256;
};

// s_waitcnt for `per` loads per fill and S - 2 fills in flight (per <= 8).
template <int S>
__device__ __forceinline__ void wait_fills(int per) {
    switch (per) {
        case 1: wait_vm<(S - 2) * 1>(); break;
        case 2: wait_vm<(S - 2) * 2>(); break;
        case 3: wait_vm<(S - 2) * 3>(); break;
        case 4: wait_vm<(S - 2) * 4>(); break;
        case 5: wait_vm<(S - 2) * 5>(); break;
        case 6: wait_vm<(S - 2) * 6>(); break;
        case 7: wait_vm<(S - 2) * 7>(); break;
        default: wait_vm<(S - 2) * 8>(); break;
    }
}

// gate/up, W4A8: block = (32*NS tokens, 32*W intermediate rows), W waves;
// an activation slab is 2*NS pieces of 1 KB (16 token rows each), wave wv
// filling pieces wv, wv + W, ...
template <int NS, int W, int NSUB, int S>
__device__ __forceinline__ void ga8_step(uint8_t* __restrict__ wr, const uint8_t* __restrict__ rd,
                                         const uint8_t* const (&xsrc)[2 * NS / W], const int (&xk)[2 * NS / W],
                                         const uint8_t* ssrc, const uint8_t* codes,
                                         const uint8_t* scales, int sc_shift, int n_slabs, int H, int wv, int lane,
                                         bool has_rows, int j, f32x16 (&acc_g)[NS], f32x16 (&acc_u)[NS]) {
    using R = A8Ring<NS * kSub>;
    constexpr int kW = R::kCodes + R::kScales;
    {
        const int sl = min(j + S - 1, n_slabs - 1);
#pragma unroll
        for (int v = 0; v < 2 * NS / W; ++v) {
            const int k = sl * kSlab + xk[v];
            lds_load16(xsrc[v] + (k < H ? k : 0), wr + (W * v + wv) * 1024);
        }
        if (wv < R::kScW) lds_load4(ssrc + 4 * (sl >> 1), wr + R::kCodes + wv * 256);
        if (has_rows) {
            uint8_t* wb = wr + kW + wv * kGuWaveBytes;
            const uint8_t* p = codes + (size_t)(sl >> 1) * 2048 + (sl & 1) * 512;
            lds_load16(p, wb);
            lds_load16(p + 1024, wb + 1024);
            lds_load4(scales + (size_t)(sl >> 1) * 128 + (sl & 1) * 64, wb + 2048);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (has_rows && j >= 0) {
        const int r = lane & 31, half = lane >> 5;
        const uint8_t* wb = rd + kW + wv * kGuWaveBytes;
        const u32x4 cg = *reinterpret_cast<const u32x4*>(wb + lane * 16);
        const u32x4 cu = *reinterpret_cast<const u32x4*>(wb + 1024 + lane * 16);
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(wb + 2048 + lane * 4) >> sc_shift;
        const int sbyte = 2 * (j & 1) + half;
        i32x8 b[NSUB];
        uint32_t bs[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            b[s] = a8_b(rd, s * kSub + r, half);
            bs[s] = rd[R::kCodes + 4 * (s * kSub + r) + sbyte];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            acc_g[s] = mfma_a4b8(cg, b[s], sc & 0xFF, bs[s], acc_g[s]);
            acc_u[s] = mfma_a4b8(cu, b[s], (sc >> 8) & 0xFF, bs[s], acc_u[s]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int NS, int W>
constexpr int ga8_slot_bytes() {
    return A8Ring<NS * kSub>::kCodes + A8Ring<NS * kSub>::kScales + W * kGuWaveBytes;
}

template <int NS, int W, int NSUB, int S>
__device__ __forceinline__ void ga8_main(uint8_t (&ring)[S][(ga8_slot_bytes<NS, W>())],
                                         const uint8_t* const (&xsrc)[2 * NS / W], const int (&xk)[2 * NS / W],
                                         const uint8_t* ssrc, const uint8_t* codes, const uint8_t* scales,
                                         int sc_shift, int n_slabs, int H, int wv, int lane, bool has_rows,
                                         f32x16 (&acc_g)[NS], f32x16 (&acc_u)[NS]) {
    const int per = 2 * NS / W + (wv < A8Ring<NS * kSub>::kScW) + (has_rows ? 3 : 0);
    int ws = 0, rs = 1;
    for (int j = 1 - S; j < n_slabs; ++j) {
        if (j >= 0) {
            wait_fills<S>(per);
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        ga8_step<NS, W, NSUB, S>(&ring[ws][0], &ring[rs][0], xsrc, xk, ssrc, codes, scales, sc_shift, n_slabs, H, wv,
                              lane, has_rows, j, acc_g, acc_u);
        ws = next_slot<S>(ws);
        rs = next_slot<S>(rs);
    }
    wait_vm<0>();
}

template <int NS, int W, int S>
__global__ __launch_bounds__(64 * W) void gateup_a8_kernel(
    const uint8_t* __restrict__ gu_codes, const uint8_t* __restrict__ gu_scales, size_t e_codes,
    size_t e_scales, const uint8_t* __restrict__ sh_codes, const uint8_t* __restrict__ sh_scales,
    const uint8_t* __restrict__ x8, const uint8_t* __restrict__ xs, int H, int I, int E, int sb,
    const int32_t* __restrict__ n_tiles, const int2* __restrict__ tiles, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ off, const int32_t* __restrict__ tok_of, uint8_t* __restrict__ h8,
    uint8_t* __restrict__ hs, int sbi) {
    constexpr int TT = NS * kSub, kRows = 32 * W, XL = 2 * NS / W;
    static_assert(XL >= 1 && XL * W == 2 * NS, "every wave fills whole 1 KB pieces of each slab");
    __shared__ __align__(1024) uint8_t ring[S][(ga8_slot_bytes<NS, W>())];

    Item it;
    if (!block_item(n_tiles, tiles, counts, (I + kRows - 1) / kRows, TT, it)) return;
    const int lane = lane_id(), wv = wave_id_uniform();
    const int n_sub = (it.rows + kSub - 1) / kSub;
    const int pair0 = off[it.group] + it.start;
    const int r = lane & 31, half = lane >> 5;
    const int kb4 = (H / 32 + 3) / 4, n_slabs = 2 * kb4;

    // code fill: piece q = W v + wv covers rows 16 q .. 16 q + 15, lane l row 16 q + l / 4
    const uint8_t* xsrc[XL];
    int xk[XL];
#pragma unroll
    for (int v = 0; v < XL; ++v) {
        const int frow = 16 * (W * v + wv) + (lane >> 2);
        xsrc[v] = x8 + (size_t)tok_of[pair0 + min(frow, it.rows - 1)] * H;
        xk[v] = ((lane & 3) ^ ((frow >> 2) & 3)) * 16;
    }
    // scale fill (first waves): lane l row 64 wv + l
    const uint8_t* ssrc = xs + (size_t)tok_of[pair0 + min(64 * wv + lane, it.rows - 1)] * sb;

    const int n0 = it.rb * kRows + 32 * wv;
    const bool has_rows = n0 < I;
    const uint8_t* cb = it.group < E ? gu_codes + (size_t)it.group * e_codes : sh_codes;
    const uint8_t* sbp = it.group < E ? gu_scales + (size_t)it.group * e_scales : sh_scales;
    const size_t unit = (size_t)((has_rows ? n0 : 0) / 16 + (r >> 4));
    const int li0 = (r & 15) + 16 * half;
    const uint8_t* codes = cb + unit * kb4 * 2048 + li0 * 16;
    const uint8_t* scales = sbp + unit * kb4 * 128 + ((2 * li0) & ~3);
    const int sc_shift = 16 * (li0 & 1);

    f32x16 acc_g[NS], acc_u[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        acc_g[s] = f32x16{};
        acc_u[s] = f32x16{};
    }
    if (NS == 4 && n_sub == 4)
        ga8_main<NS, W, (NS >= 4 ? 4 : 1), S>(ring, xsrc, xk, ssrc, codes, scales, sc_shift, n_slabs, H, wv, lane,
                                           has_rows, acc_g, acc_u);
    else if (NS >= 3 && n_sub == 3)
        ga8_main<NS, W, (NS >= 3 ? 3 : 1), S>(ring, xsrc, xk, ssrc, codes, scales, sc_shift, n_slabs, H, wv, lane,
                                           has_rows, acc_g, acc_u);
    else if (NS >= 2 && n_sub == 2)
        ga8_main<NS, W, (NS >= 2 ? 2 : 1), S>(ring, xsrc, xk, ssrc, codes, scales, sc_shift, n_slabs, H, wv, lane,
                                           has_rows, acc_g, acc_u);
    else
        ga8_main<NS, W, 1, S>(ring, xsrc, xk, ssrc, codes, scales, sc_shift, n_slabs, H, wv, lane, has_rows, acc_g,
                           acc_u);

    if (!has_rows) return;
    // h = silu(g) * u, then its MXFP8: rows n0 .. n0 + 31 of one token are one
    // block, held by lanes r and r + 32
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s >= n_sub) continue;                               // block-uniform
        float hv[16];
        uint32_t am = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float g = acc_g[s][e], u = acc_u[s][e];
            hv[e] = g / (1.f + expf(-g)) * u;
            am = max(am, __float_as_uint(hv[e]) & 0x7FFFFFFFu);
        }
        const u32x2 pr = swap32(am);
        const uint32_t sbyte = mx8_scale_byte(max(pr[0], pr[1]));
        const float inv = mx8_inv(sbyte);
        const int row = s * kSub + r;
        if (row >= it.rows) continue;
        const size_t pp = (size_t)(pair0 + row);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const uint32_t c = mx8_code(hv[4 * r4], inv) | (mx8_code(hv[4 * r4 + 1], inv) << 8) |
                               (mx8_code(hv[4 * r4 + 2], inv) << 16) | (mx8_code(hv[4 * r4 + 3], inv) << 24);
            *reinterpret_cast<uint32_t*>(h8 + pp * I + n0 + 8 * r4 + 4 * half) = c;
        }
        if (half == 0) hs[pp * sbi + n0 / 32] = (uint8_t)sbyte;
    }
}

// down, W4A8: block = (32*ND tokens of a gate/up tile, 64*W output rows), W =
// 2*ND waves; wave w owns rows 64 w .. 64 w + 63 as two 32-row tiles.  Scale
// bytes of h past I/32 are never written and are read as 127 (1.0) instead:
// their codes meet zero weights.
template <int ND, int W, int NSUB, int S>
__device__ __forceinline__ void da8_step(uint8_t* __restrict__ wr, const uint8_t* __restrict__ rd,
                                         const uint8_t* const (&hsrc)[2 * ND / W], const int (&hk)[2 * ND / W],
                                         const uint8_t* ssrc, const uint8_t* codes0,
                                         const uint8_t* scales0, size_t t1c, size_t t1s, int sc_shift, int n_slabs,
                                         int I, int wv, int lane, bool has_rows, int j, f32x16 (&acc)[2][ND]) {
    using R = A8Ring<ND * kSub>;
    constexpr int kW = R::kCodes + R::kScales;
    {
        const int sl = min(j + S - 1, n_slabs - 1);
#pragma unroll
        for (int v = 0; v < 2 * ND / W; ++v) {
            const int k = sl * kSlab + hk[v];
            lds_load16(hsrc[v] + (k < I ? k : 0), wr + (W * v + wv) * 1024);
        }
        if (wv < R::kScW) lds_load4(ssrc + 4 * (sl >> 1), wr + R::kCodes + wv * 256);
        if (has_rows) {
            uint8_t* wb = wr + kW + wv * kDnWaveBytes;
            const uint8_t* p = codes0 + (size_t)(sl >> 1) * 1024 + (sl & 1) * 512;
            const uint8_t* sp = scales0 + (size_t)(sl >> 1) * 64 + (sl & 1) * 32;
            lds_load16(p, wb);
            lds_load16(p + t1c, wb + 1024);
            lds_load4(sp, wb + 2048);
            lds_load4(sp + t1s, wb + 2304);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (has_rows && j >= 0) {
        const int r = lane & 31, half = lane >> 5;
        const uint8_t* wb = rd + kW + wv * kDnWaveBytes;
        const u32x4 c0 = *reinterpret_cast<const u32x4*>(wb + lane * 16);
        const u32x4 c1 = *reinterpret_cast<const u32x4*>(wb + 1024 + lane * 16);
        const uint32_t s0 = (*reinterpret_cast<const uint32_t*>(wb + 2048 + lane * 4) >> sc_shift) & 0xFF;
        const uint32_t s1 = (*reinterpret_cast<const uint32_t*>(wb + 2304 + lane * 4) >> sc_shift) & 0xFF;
        const int sbyte = 2 * (j & 1) + half;
        const bool real = 2 * j + half < I / 32;
        i32x8 b[NSUB];
        uint32_t bs[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            b[s] = a8_b(rd, s * kSub + r, half);
            bs[s] = real ? (uint32_t)rd[R::kCodes + 4 * (s * kSub + r) + sbyte] : 127u;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            acc[0][s] = mfma_a4b8(c0, b[s], s0, bs[s], acc[0][s]);
            acc[1][s] = mfma_a4b8(c1, b[s], s1, bs[s], acc[1][s]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int ND, int W>
constexpr int da8_slot_bytes() {
    return A8Ring<ND * kSub>::kCodes + A8Ring<ND * kSub>::kScales + W * kDnWaveBytes;
}

template <int ND, int W, int NSUB, int S>
__device__ __forceinline__ void da8_main(uint8_t (&ring)[S][(da8_slot_bytes<ND, W>())],
                                         const uint8_t* const (&hsrc)[2 * ND / W], const int (&hk)[2 * ND / W],
                                         const uint8_t* ssrc, const uint8_t* codes0, const uint8_t* scales0,
                                         size_t t1c, size_t t1s, int sc_shift, int n_slabs, int I, int wv, int lane,
                                         bool has_rows, f32x16 (&acc)[2][ND]) {
    const int per = 2 * ND / W + (wv < A8Ring<ND * kSub>::kScW) + (has_rows ? 4 : 0);
    int ws = 0, rs = 1;
    for (int j = 1 - S; j < n_slabs; ++j) {
        if (j >= 0) {
            wait_fills<S>(per);
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        da8_step<ND, W, NSUB, S>(&ring[ws][0], &ring[rs][0], hsrc, hk, ssrc, codes0, scales0, t1c, t1s, sc_shift,
                              n_slabs, I, wv, lane, has_rows, j, acc);
        ws = next_slot<S>(ws);
        rs = next_slot<S>(rs);
    }
    wait_vm<0>();
}

template <int ND, int W, int S>
__global__ __launch_bounds__(64 * W) void down_a8_kernel(
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales, size_t e_codes,
    size_t e_scales, const uint8_t* __restrict__ sh_codes, const uint8_t* __restrict__ sh_scales,
    const uint8_t* __restrict__ h8, const uint8_t* __restrict__ hs, int H, int I, int E, int sbi,
    int tile_tokens, const int32_t* __restrict__ n_tiles, const int2* __restrict__ tiles,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ off, float* __restrict__ y_pair) {
    constexpr int TD = ND * kSub, kRows = 64 * W, XL = 2 * ND / W;
    static_assert(XL >= 1 && XL * W == 2 * ND, "every wave fills whole 1 KB pieces of each slab");
    __shared__ __align__(1024) uint8_t ring[S][(da8_slot_bytes<ND, W>())];

    const int parts = tile_tokens / TD, n_rb = (H + kRows - 1) / kRows;
    Item it;
    if (!block_item(n_tiles, tiles, counts, parts * n_rb, tile_tokens, it)) return;
    const int part = it.rb / n_rb;
    it.rb -= part * n_rb;
    it.rows = min(it.rows - part * TD, TD);
    if (it.rows <= 0) return;
    it.start += part * TD;

    const int lane = lane_id(), wv = wave_id_uniform();
    const int n_sub = (it.rows + kSub - 1) / kSub;
    const int pair0 = off[it.group] + it.start;
    const int r = lane & 31, half = lane >> 5;
    const int kb4 = (I / 32 + 3) / 4, n_slabs = 2 * kb4;

    const uint8_t* hsrc[XL];
    int hk[XL];
#pragma unroll
    for (int v = 0; v < XL; ++v) {
        const int frow = 16 * (W * v + wv) + (lane >> 2);
        hsrc[v] = h8 + (size_t)(pair0 + min(frow, it.rows - 1)) * I;
        hk[v] = ((lane & 3) ^ ((frow >> 2) & 3)) * 16;
    }
    const uint8_t* ssrc = hs + (size_t)(pair0 + min(64 * wv + lane, it.rows - 1)) * sbi;

    const int n0 = it.rb * kRows + 64 * wv;
    const bool has_rows = n0 < H;
    const uint8_t* cb = it.group < E ? dn_codes + (size_t)it.group * e_codes : sh_codes;
    const uint8_t* sbp = it.group < E ? dn_scales + (size_t)it.group * e_scales : sh_scales;
    const size_t unit = (size_t)((has_rows ? n0 : 0) / 16 + (r >> 4));
    const int li0 = (r & 15) + 16 * half;
    const uint8_t* codes0 = cb + unit * kb4 * 1024 + li0 * 16;
    const uint8_t* scales0 = sbp + unit * kb4 * 64 + (li0 & ~3);
    const size_t t1c = (size_t)2 * kb4 * 1024, t1s = (size_t)2 * kb4 * 64;
    const int sc_shift = 8 * (li0 & 3);

    f32x16 acc[2][ND];
#pragma unroll
    for (int s = 0; s < ND; ++s) {
        acc[0][s] = f32x16{};
        acc[1][s] = f32x16{};
    }
    if (ND == 4 && n_sub == 4)
        da8_main<ND, W, (ND >= 4 ? 4 : 1), S>(ring, hsrc, hk, ssrc, codes0, scales0, t1c, t1s, sc_shift, n_slabs, I, wv,
                                           lane, has_rows, acc);
    else if (ND >= 3 && n_sub == 3)
        da8_main<ND, W, (ND >= 3 ? 3 : 1), S>(ring, hsrc, hk, ssrc, codes0, scales0, t1c, t1s, sc_shift, n_slabs, I, wv,
                                           lane, has_rows, acc);
    else if (ND >= 2 && n_sub == 2)
        da8_main<ND, W, (ND >= 2 ? 2 : 1), S>(ring, hsrc, hk, ssrc, codes0, scales0, t1c, t1s, sc_shift, n_slabs, I, wv,
                                           lane, has_rows, acc);
    else
        da8_main<ND, W, 1, S>(ring, hsrc, hk, ssrc, codes0, scales0, t1c, t1s, sc_shift, n_slabs, I, wv, lane,
                           has_rows, acc);

    if (!has_rows) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int s = 0; s < ND; ++s) {
            const int row = s * kSub + r;
            if (s >= n_sub || row >= it.rows) continue;
            float* dst = y_pair + (size_t)(pair0 + row) * H + n0 + 32 * t + 4 * half;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<float4*>(dst + 8 * r4) =
                    float4{acc[t][s][4 * r4], acc[t][s][4 * r4 + 1], acc[t][s][4 * r4 + 2], acc[t][s][4 * r4 + 3]};
        }
    }
}

// ----------------------------------------------------------------------------
// combine: one wave per 256 consecutive outputs of one token (4 per lane), so
// the token's pair rows and weights are wave-uniform and every lane's k + 1
// row reads are in flight together.  y[t] = sum_j w[t][j] * y_pair[pos(t, j)]
// (fmaf, j ascending) + y_pair[shared row], then one RNE to bf16.

template <int KMAX>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y_pair,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ wts, int T, int k, int H,
                                                           int shared_row0, uint16_t* __restrict__ y_bf16,
                                                           float* __restrict__ y_f32) {
    const int per_tok = (H + 255) / 256;
    const int piece = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6));
    if (piece >= T * per_tok) return;
    const int t = piece / per_tok;
    const int n = (piece - t * per_tok) * 256 + lane_id() * 4;
    if (n >= H) return;
    f32x4 v[KMAX], vs;
    float w[KMAX];
    // choices past k repeat the last one (loads without branches, all in
    // flight at once); they are not added
    int pj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const size_t jj = (size_t)t * k + min(j, k - 1);
        pj[j] = pos[jj];
        w[j] = wts[jj];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y_pair + (size_t)pj[j] * H + n));
    vs = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y_pair + (size_t)(shared_row0 + t) * H + n));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
            acc[0] = fmaf(w[j], v[j][0], acc[0]);
            acc[1] = fmaf(w[j], v[j][1], acc[1]);
            acc[2] = fmaf(w[j], v[j][2], acc[2]);
            acc[3] = fmaf(w[j], v[j][3], acc[3]);
        }
    }
    acc[0] += vs[0];
    acc[1] += vs[1];
    acc[2] += vs[2];
    acc[3] += vs[3];
    const size_t o = (size_t)t * H + n;
    if (y_f32) *reinterpret_cast<f32x4*>(y_f32 + o) = acc;
    const uint32_t b0 = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    const uint32_t b1 = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<u32x2*>(y_bf16 + o) = u32x2{b0, b1};
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

    // Wider blocks for the larger tiles: 8 waves (one block per CU, a 4-slot
    // ring) where every wave still fills part of each slab.
    constexpr int WG = NS >= 2 ? 8 : 4, SG = NS >= 2 ? 4 : 3;
    const size_t gu_items = (size_t)lay.max_tiles * ((w.I + 32 * WG - 1) / (32 * WG));
    hipLaunchKernelGGL((gateup_kernel<NS, WG, SG>), dim3((unsigned)(kXcds * ((gu_items + kXcds - 1) / kXcds))),
                       dim3(64 * WG), 0, s, static_cast<const uint8_t*>(w.gu_codes),
                       static_cast<const uint8_t*>(w.gu_scales), sz.gu_codes, sz.gu_scales,
                       static_cast<const uint8_t*>(w.sh_gu_codes), static_cast<const uint8_t*>(w.sh_gu_scales),
                       x, w.H, w.I, w.E, n_tiles, tiles, counts, off, tok_of, h_hi, h_lo);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    constexpr int ND = NS >= 2 ? 2 : 1;
    constexpr int WD = ND >= 2 ? 8 : 4, SD = ND >= 2 ? 4 : 3;
    const size_t dn_items = (size_t)lay.max_tiles * (NS / ND) * ((w.H + 64 * WD - 1) / (64 * WD));
    hipLaunchKernelGGL((down_kernel<ND, WD, SD>), dim3((unsigned)(kXcds * ((dn_items + kXcds - 1) / kXcds))),
                       dim3(64 * WD), 0, s, static_cast<const uint8_t*>(w.dn_codes),
                       static_cast<const uint8_t*>(w.dn_scales), sz.dn_codes, sz.dn_scales,
                       static_cast<const uint8_t*>(w.sh_dn_codes), static_cast<const uint8_t*>(w.sh_dn_scales),
                       h_hi, h_lo, w.H, w.I, w.E, NS * kSub, n_tiles, tiles, counts, off, y_pair);
    return hipGetLastError();
}

template <int NS>
hipError_t launch_gemms_a8(const moedec_moe_weights& w, const PrefillLayout& lay, uint8_t* base, hipStream_t s) {
    moedec_mxfp4_sizes sz;
    packed_sizes(w.H, w.I, &sz);
    const int32_t* n_tiles = reinterpret_cast<const int32_t*>(base + lay.n_tiles_off);
    const int2* tiles = reinterpret_cast<const int2*>(base + lay.tiles_off);
    const int32_t* counts = reinterpret_cast<const int32_t*>(base + lay.counts_off);
    const int32_t* off = reinterpret_cast<const int32_t*>(base + lay.off_off);
    const int32_t* tok_of = reinterpret_cast<const int32_t*>(base + lay.tok_of_off);
    uint8_t* h8 = base + lay.h8_off;
    uint8_t* hs = base + lay.hs_off;

    // One wave per 1 KB piece of the activation slab: 8-wave blocks for 128-token
    // tiles (one block per CU).  Two 4-wave blocks per CU instead, whose waves
    // would run out of step, measured 20 % slower: the tile's x is read by twice
    // as many row blocks.
    constexpr int WG = 2 * NS, SG = NS >= 2 ? 4 : 3;
    const size_t gu_items = (size_t)lay.max_tiles * ((w.I + 32 * WG - 1) / (32 * WG));
    hipLaunchKernelGGL((gateup_a8_kernel<NS, WG, SG>), dim3((unsigned)(kXcds * ((gu_items + kXcds - 1) / kXcds))),
                       dim3(64 * WG), 0, s, static_cast<const uint8_t*>(w.gu_codes),
                       static_cast<const uint8_t*>(w.gu_scales), sz.gu_codes, sz.gu_scales,
                       static_cast<const uint8_t*>(w.sh_gu_codes), static_cast<const uint8_t*>(w.sh_gu_scales),
                       base + lay.x8_off, base + lay.xs_off, w.H, w.I, w.E, lay.sb, n_tiles, tiles, counts, off,
                       tok_of, h8, hs, lay.sbi);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    constexpr int ND = NS;
    constexpr int WD = 2 * ND, SD = ND >= 2 ? 4 : 3;
    const size_t dn_items = (size_t)lay.max_tiles * (NS / ND) * ((w.H + 64 * WD - 1) / (64 * WD));
    hipLaunchKernelGGL((down_a8_kernel<ND, WD, SD>), dim3((unsigned)(kXcds * ((dn_items + kXcds - 1) / kXcds))),
                       dim3(64 * WD), 0, s, static_cast<const uint8_t*>(w.dn_codes),
                       static_cast<const uint8_t*>(w.dn_scales), sz.dn_codes, sz.dn_scales,
                       static_cast<const uint8_t*>(w.sh_dn_codes), static_cast<const uint8_t*>(w.sh_dn_scales), h8,
                       hs, w.H, w.I, w.E, lay.sbi, NS * kSub, n_tiles, tiles, counts, off,
                       reinterpret_cast<float*>(base + lay.y_pair_off));
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
    l.hist_off = o;     o = align256(o + (size_t)kMaxChunks * E * 4);
    l.base_off = o;     o = align256(o + (size_t)kMaxChunks * E * 4);
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
    // MXFP8 path: x's codes and scales, and h's in the space of h_hi / h_lo
    l.sb = 4 * ((H / 32 + 3) / 4);
    l.sbi = 4 * ((I / 32 + 3) / 4);
    l.x8_off = o;       o = align256(o + (size_t)T * H);
    l.xs_off = o;       o = align256(o + (size_t)T * l.sb);
    l.h8_off = l.h_hi_off;
    l.hs_off = align256(l.h8_off + P * I);
    l.total = o;
    return l;
}

hipError_t launch_prefill(const moedec_moe_weights& w, const uint16_t* x, const float* logits, int T, int k,
                          int32_t* ids_out, float* w_out, int32_t* counts_out, uint16_t* y_bf16, float* y_f32,
                          void* ws, hipStream_t s, bool a8) {
    const PrefillLayout lay = prefill_layout(T, w.E, k, w.H, w.I);
    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(base + lay.counts_off);
    int32_t* hist = reinterpret_cast<int32_t*>(base + lay.hist_off);
    int32_t* chunk_base = reinterpret_cast<int32_t*>(base + lay.base_off);
    int32_t* off = reinterpret_cast<int32_t*>(base + lay.off_off);
    int32_t* ids = ids_out ? ids_out : reinterpret_cast<int32_t*>(base + lay.ids_off);
    float* wts = w_out ? w_out : reinterpret_cast<float*>(base + lay.w_off);

    const int n_routed = T * k;
    const int chunk = std::max(kChunkMin, (n_routed + kMaxChunks - 1) / kMaxChunks);
    const int n_chunks = (n_routed + chunk - 1) / chunk;
    const int route_blocks = (T + kThreads / kWave - 1) / (kThreads / kWave);
    if (a8) {
        const int qblocks = grid_cap((size_t)T * lay.sb, 8192);
        auto rq = w.E <= 512 ? route_quant_kernel<8> : route_quant_kernel<16>;
        hipLaunchKernelGGL(rq, dim3(route_blocks + qblocks), dim3(kThreads), 0, s, logits, T, w.E, k, ids, wts,
                           route_blocks, x, w.H, lay.sb, base + lay.x8_off, base + lay.xs_off);
    } else {
        auto r = w.E <= 512 ? route_kernel<8> : route_kernel<16>;
        hipLaunchKernelGGL(r, dim3(route_blocks), dim3(kThreads), 0, s, logits, T, w.E, k, ids, wts);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(count_kernel, dim3(n_chunks), dim3(kCountThreads), 0, s, ids, n_routed, chunk, w.E, hist);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kCountThreads), 0, s, hist, n_chunks, w.E, T, lay.ns * kSub,
                       chunk_base, counts, off, reinterpret_cast<int2*>(base + lay.tiles_off),
                       reinterpret_cast<int32_t*>(base + lay.n_tiles_off), counts_out);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    int32_t* pos = reinterpret_cast<int32_t*>(base + lay.pos_off);
    hipLaunchKernelGGL(scatter_kernel, dim3(n_chunks), dim3(kCountThreads), 0, s, ids, T, k, chunk, off, chunk_base,
                       reinterpret_cast<int32_t*>(base + lay.tok_of_off), pos, w.E);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    if (a8) {
        switch (lay.ns) {
            case 4: err = launch_gemms_a8<4>(w, lay, base, s); break;
            case 2: err = launch_gemms_a8<2>(w, lay, base, s); break;
            default: err = launch_gemms_a8<1>(w, lay, base, s); break;
        }
    } else {
        switch (lay.ns) {
            case 4: err = launch_gemms<4>(w, x, lay, base, s); break;
            case 2: err = launch_gemms<2>(w, x, lay, base, s); break;
            default: err = launch_gemms<1>(w, x, lay, base, s); break;
        }
    }
    if (err != hipSuccess) return err;
    const size_t pieces = (size_t)T * ((w.H + 255) / 256);
    const dim3 cgrid((unsigned)((pieces + kThreads / kWave - 1) / (kThreads / kWave)));
    auto combine = k <= 8 ? combine_kernel<8> : (k <= 16 ? combine_kernel<16> : combine_kernel<MOEDEC_MAX_K>);
    hipLaunchKernelGGL(combine, cgrid, dim3(kThreads), 0, s,
                       reinterpret_cast<const float*>(base + lay.y_pair_off), pos, wts, T, k, w.H, T * k, y_bf16,
                       y_f32);
    return hipGetLastError();
}

}  // namespace moedec
