// Routed + shared SwiGLU expert FFN on packed MXFP4 weights, M = 1..4 tokens,
// in one kernel launch -- optionally with the top-k routing fused in front.
//
// The pages' premise: at batch 1 decode is bound by reading weights, the MoE
// experts being the largest share, and their MXFP4 kernel is what lifted
// throughput first (knowledge card at ai.cheesepanini.fun, background and
// method point #1; news article yoususu.cn/post/959, "where the speed comes
// from").  A verify window of 4 tokens touches up to 32 experts (card, method
// point #3): each active expert's bytes are streamed once for all the tokens
// that use it.
//
// Grid.  A persistent grid of three blocks per CU, small enough that every
// block is resident at once (checked against the occupancy before each
// launch), walks the work units round-robin
// (unit = blockIdx.x + i * gridDim.x).  Unit order is: gate/up units, then the
// down units of slot groups 1.., then those of group 0.  Every block therefore
// finishes all its gate/up units before it can wait for anything, and all its
// other down units before it waits as a combiner, so no wait can close a cycle.
// When four blocks per CU give every unit a block of its own (ONE: one token),
// the grid is one block per unit, all resident, and no block waits on itself;
// the shared expert's gate/up blocks then skip routing and load their weights
// first thing.
//
// Prologue (every block).  The block builds an LDS table of the layer's slots:
// slot 0 is the shared expert (weight 1, every token), slots 1.. the distinct
// routed experts in ascending id, each with its token mask and per-token
// weights -- read from a moe_route_topk dispatch table, or computed right here
// from the router logits (one wave per token).  (slot, token) pairs are
// counted in slot order and cut into groups of at most pair_cap pairs so that
// a group's h fits in LDS.
//
// Units.
//   * gate/up (slot s, rg): h = silu(W_gate x) * (W_up x) for the 16
//     intermediate rows 16rg..16rg+15 of the slot's expert, full K = H, every
//     token the slot serves; each h value is published as one 64-bit word
//     (launch generation, value).
//   * down (group, g): for output rows 16 SUB g .. 16 SUB (g + 1) - 1 (SUB = 2,
//     or 1 for one token in the persistent grid), the sum over the group's slots of
//     W_down[e] (w * h).  It issues its weight loads, then loads the
//     group's tagged h words -- re-reading those whose tag is stale -- stages
//     w * h in LDS and finishes.  With one group it writes y; otherwise groups
//     >= 1 publish tagged partial rows and the group-0 unit adds them in group
//     order and writes y (deterministic).
// Synchronisation uses no atomic read-modify-writes, no flags and no cache
// flushes.  Data crossing CUs (h, partial rows) is written as 64-bit words
// holding the value and the launch generation, with device-coherent stores
// (single-copy atomic, through to the level all CUs share), and read with
// device-coherent loads: a reader knows a word is from this launch when its
// tag matches.  The generation is a launch count kept in kMaxGrid workspace
// words that every launch advances together (block b writes words b, b +
// grid, ...), so each block reads it from its own word and all blocks of a
// launch agree, whatever grids earlier launches used; nothing needs resetting
// between calls.
//
// Lanes.  A 64-lane wave reads one 1 KiB chunk per load step: lane l holds the
// 16 code bytes (32 E2M1 values, one MX block) of row 16u + (l & 15) and MX
// block 4c + (l >> 4), so the four 16-lane rows of the wave cover four
// consecutive MX blocks of the same 16 rows.  Gate/up chunks come in pairs
// (gate rows, then the same up rows) sharing the activations.  Two codes
// become a scaled bf16 (gate/up) or float32 (down) pair in one gfx950
// conversion; bf16 x E2M1 x 2^k products are exact in float32 and every sum
// is float32.  Activations are read from LDS, each 16-lane row broadcasting
// its own MX block; LDS rows are padded so the four rows hit different banks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "launch.h"
#include "route_device.h"

namespace moedec {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnitRows = 16;
constexpr int kXBlock = 80;          // LDS bytes per 32-value block of x (64 + 16 pad)
constexpr int kHBlock = 144;         // LDS bytes per 32-value block of h (128 + 16 pad)
// A down unit covers SUB consecutive 16-row blocks: lane l takes the rows
// 16 (SUB g + j) + (l & 15), j < SUB, of the same MX block, so every h value it
// reads feeds SUB rows and SUB times fewer units stage h.  Several tokens:
// 32 rows (their h staging traffic is what bounds the down phase); one token:
// 16 rows (its down units are bound by each wave's serial arithmetic, which
// fewer, larger units would lengthen: 16.8 against 14.9 us).
template <int M_T, bool ONE>
constexpr int dn_sub() { return (M_T == 1 && !ONE) ? 1 : 2; }
// Down chunks (per 16-row block) per load batch; two batches (A, B) are in
// flight before h is staged.  With one unit per block (ONE) a single batch of
// 5 covers a one-token unit of three 768-wide pairs (4.5 chunks per wave) and
// frees the registers of the second set.
template <int M_T, bool ONE>
constexpr int dn_batch() { return ONE ? 5 : (dn_sub<M_T, ONE>() == 2 ? 2 : 7); }
// 16-byte loads of tagged h in flight per thread while staging.  A slot
// group holds at most as many pairs as one batch stages (see ffn_layout), so
// a down unit sees h after a single round trip once it is there.
template <int M_T, bool ONE>
constexpr int stage_batch() { return ONE ? 5 : 8; }
constexpr int kMaxGroups = MOEDEC_MAX_M * MOEDEC_MAX_K + MOEDEC_MAX_M;
constexpr int kMaxPairs = kMaxGroups + MOEDEC_MAX_M;
constexpr int kMaxGrid = 4096;
// Co-resident blocks per CU.  The general form keeps a block's next gate/up
// unit and a second down batch in flight (168 VGPRs per lane: three blocks).
// When the grid has a block for every unit (ONE, one token), neither is
// needed and at most 128 VGPRs give four blocks per CU: a one-token 2560 x 768
// layer's 672 units then all start at once, so every down unit issues its
// weight loads right after routing.  The generation words let the grid differ
// between launches.
template <bool ONE>
constexpr int blocks_per_cu() { return ONE ? 4 : 3; }
constexpr uint32_t kSpinLimit = 1u << 20;   // bounded waits; reached only if co-residency fails
static_assert(kMaxGrid * sizeof(uint32_t) == kWsStatusOffset, "the error word follows the launch counters");

struct FfnArgs {
    const uint8_t* gu_codes;
    const uint8_t* gu_scales;
    const uint8_t* dn_codes;
    const uint8_t* dn_scales;
    const uint8_t* sh_gu_codes;
    const uint8_t* sh_gu_scales;
    const uint8_t* sh_dn_codes;
    const uint8_t* sh_dn_scales;
    size_t gu_codes_stride, gu_scales_stride, dn_codes_stride, dn_scales_stride;
    int E, H, I, k;
    int kbh, kbh4, kbi, kbi4;        // MX blocks along H / I and groups of four
    int gu_units;                    // I / 16
    int dn_units;                    // H / (16 * dn_sub)
    int max_slots, max_groups, pair_cap;
    int n_gu, n_units;
    int writer;                      // the block that writes routing outputs and x_out (runs a gate/up unit)
    int pair_bytes, red_off;         // LDS layout
    int a8;                          // nonzero: MXFP8 activations (x into gate/up, h into down)
    const uint16_t* x;               // [M][H] bf16 (null when r_in is given)
    const float* r_in;               // [M][H] residual: x = bf16(RMSNorm(r_in)), or null
    float* r_out;                    // [M][H] r_in + y, or null
    uint16_t* x_out;                 // [M][H] the normalised x (the writer block writes it), or null
    float eps;                       // RMSNorm epsilon
    const moedec_dispatch* disp;     // slots from moe_route_topk, or
    const float* logits;             // [M][E]: route here
    int32_t* ids_out;                // routing outputs of the fused path (the writer block), nullable
    float* w_out;
    moedec_dispatch* disp_out;
    uint32_t* gens;                  // [kMaxGrid] per-block launch counters
    uint32_t* err;                   // set when a wait gave up
    uint64_t* h;                     // [max_slots][M][I] tagged words (generation << 32 | float)
    uint64_t* part;                  // [max_groups][M][H] tagged partial rows
    int h_bytes;                     // size of h (device-coherent buffer loads)
    uint16_t* y_bf16;                // [M][H] or null
    float* y_f32;                    // [M][H] or null
    // The shared expert in FP8 (instantiations with SH8): sh_gu_codes and
    // sh_dn_codes then hold the FP8 layout of pack.hip and these its row scales.
    const float* sh8_gu_scale;       // gate [I], then up [I]
    const float* sh8_dn_scale;       // [H]
};

struct SlotTable {
    int n_slots, n_groups;
    int32_t expert[MOEDEC_MAX_SLOTS];            // E = shared expert, -1 = unusable entry
    uint32_t mask[MOEDEC_MAX_SLOTS];
    float weight[MOEDEC_MAX_SLOTS][MOEDEC_MAX_M];
    int start[MOEDEC_MAX_SLOTS + 1];             // first (slot, token) pair of each slot
    int gfirst[kMaxGroups + 1];                  // first slot of each group
    int pair[kMaxPairs];                         // current down unit: pair -> slot << 8 | token
};

struct RouteScratch {                            // lives in the dynamic LDS during the prologue
    int32_t id[MOEDEC_MAX_M][MOEDEC_MAX_K];
    float w[MOEDEC_MAX_M][MOEDEC_MAX_K];
    uint32_t bits[MOEDEC_MAX_E / 32];
    int pre[MOEDEC_MAX_E / 32 + 1];
    int32_t expert[MOEDEC_MAX_SLOTS];
    uint32_t mask[MOEDEC_MAX_SLOTS];
    float weight[MOEDEC_MAX_SLOTS][MOEDEC_MAX_M];
};

// Device-coherent ("sc1") stores and loads: they bypass the per-XCD L2 so that
// data written by one CU is seen by every other without flushing caches.
__device__ __forceinline__ void store_tagged(uint64_t* p, uint32_t gen, float v) {
    __hip_atomic_store(p, ((uint64_t)gen << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_tagged(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kBufferRsrcWord3 = 0x00020000;    // raw 32-bit buffer, gfx9 family
constexpr int kLoadCoherent = 16;               // cache-policy bit sc1


__device__ __forceinline__ bf16x2 fp4x2_bf16(uint32_t word, float s, int sel) {
    switch (sel) {
        case 0: return MOEDEC_FP4X2_BF16(word, s, 0);
        case 1: return MOEDEC_FP4X2_BF16(word, s, 1);
        case 2: return MOEDEC_FP4X2_BF16(word, s, 2);
        default: return MOEDEC_FP4X2_BF16(word, s, 3);
    }
}

__device__ __forceinline__ f32x2 fp4x2_f32(uint32_t word, float s, int sel) {
    switch (sel) {
        case 0: return MOEDEC_FP4X2_F32(word, s, 0);
        case 1: return MOEDEC_FP4X2_F32(word, s, 1);
        case 2: return MOEDEC_FP4X2_F32(word, s, 2);
        default: return MOEDEC_FP4X2_F32(word, s, 3);
    }
}

// ---------------------------------------------------------------------------
// prologue: the slot table

// Table from a dispatch table (moe_route_topk's, or the caller's): slot 0 is
// the shared expert (listed last in the table), then the valid routed entries
// in table order.  Entries with an expert id outside [0, E) or an empty token
// mask are dropped, so every slot serves at least one token.  Wave 0.
template <int M_T>
__device__ void table_from_dispatch(const FfnArgs& a, SlotTable& T) {
    if (wave_id_uniform() != 0) return;
    const int lane = lane_id();
    const moedec_dispatch* __restrict__ d = a.disp;
    const uint32_t full = (1u << M_T) - 1u;
    const int n_tab = max(1, min(d->n_slots, a.max_slots));
    if (lane == 0) {
        T.expert[0] = a.E;
        T.mask[0] = full;
#pragma unroll
        for (int m = 0; m < M_T; ++m) T.weight[0][m] = d->weight[n_tab - 1][m];
    }
    int n = 1;
    for (int s0 = 1; s0 < n_tab; s0 += kWave) {
        const int s = s0 + lane;
        const int tab = min(s, n_tab - 1) - 1;            // clamped: always in bounds
        const int e = d->expert[tab];
        const uint32_t msk = d->token_mask[tab] & full;
        const bool valid = s < n_tab && e >= 0 && e < a.E && msk != 0u;
        const uint64_t bal = __ballot(valid);
        const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (valid) {
            T.expert[pos] = e;
            T.mask[pos] = msk;
#pragma unroll
            for (int m = 0; m < M_T; ++m) T.weight[pos][m] = d->weight[tab][m];
        }
        n += __popcll(bal);
    }
    if (lane == 0) T.n_slots = n;
}

// One token (M = 1): wave 0 builds the whole table from its top-k -- slot
// 1 + rank(id) for each chosen expert, one (slot, token) pair per slot, and
// the group bounds -- and the writer block writes the routing outputs from registers.
__device__ void table_from_logits_one(const FfnArgs& a, SlotTable& T, uint64_t* buf, const float (&lv)[16]) {
    if (wave_id_uniform() != 0) return;
    const int lane = lane_id();
    const int k = a.k;
    float wv;
    const uint64_t key = (a.E <= 512) ? wave_topk_of<8>(*reinterpret_cast<const float(*)[8]>(lv), a.E, k, wv, buf)
                                      : wave_topk_of<16>(lv, a.E, k, wv, buf);
    const int id = key_to_index(key);
    const int rank = wave_rank_ids(lane < k ? id : 0x7FFFFFFF, k);
    const int n = k + 1;
    if (lane < k) {
        T.expert[1 + rank] = id;
        T.mask[1 + rank] = 1u;
        T.weight[1 + rank][0] = wv;
        T.start[1 + rank] = 1 + rank;
    }
    const int ng = min((n - 1) / a.pair_cap + 1, a.max_groups);
    if (lane == 0) {
        T.expert[0] = a.E;
        T.mask[0] = 1u;
        T.weight[0][0] = 1.f;
        T.start[0] = 0;
        T.start[n] = n;
        T.n_slots = n;
        T.n_groups = ng;
    }
    for (int g = lane; g <= ng; g += kWave) T.gfirst[g] = min(g * a.pair_cap, n);
    if ((int)blockIdx.x == a.writer) {          // the routing outputs, as moe_route_topk writes them
        if (lane < k) {
            if (a.ids_out) a.ids_out[lane] = id;
            if (a.w_out) a.w_out[lane] = wv;
        }
        if (a.disp_out) {
            moedec_dispatch* __restrict__ o = a.disp_out;
            if (lane < k) {
                o->expert[rank] = id;
                o->token_mask[rank] = 1u;
                o->weight[rank][0] = wv;
#pragma unroll
                for (int m = 1; m < MOEDEC_MAX_M; ++m) o->weight[rank][m] = 0.f;
            }
            for (int i = k + lane; i < MOEDEC_MAX_SLOTS; i += kWave) {
                const bool shared = i == k;
                o->expert[i] = shared ? a.E : 0;
                o->token_mask[i] = shared ? 1u : 0u;
#pragma unroll
                for (int m = 0; m < MOEDEC_MAX_M; ++m) o->weight[i][m] = (shared && m == 0) ? 1.f : 0.f;
            }
            if (lane == 0) {
                o->n_slots = n;
                o->M = 1;
            }
        }
    }
}

// Several tokens: one wave per token selects its experts, the block groups
// the choices by expert (the pair counts and groups follow in table_groups).
template <int M_T>
__device__ void table_from_logits(const FfnArgs& a, SlotTable& T, uint64_t* buf, const float (&lv)[16]) {
    __shared__ RouteScratch R;
    const int w = wave_id_uniform(), lane = lane_id(), tid = threadIdx.x;
    const uint32_t full = (1u << M_T) - 1u;
    if (w < M_T) {
        float wv;
        uint64_t* wbuf = buf + kTopkBufWords * w;
        const uint64_t key = (a.E <= 512)
            ? wave_topk_of<8>(*reinterpret_cast<const float(*)[8]>(lv), a.E, a.k, wv, wbuf)
            : wave_topk_of<16>(lv, a.E, a.k, wv, wbuf);
        if (lane < a.k) {
            R.id[w][lane] = key_to_index(key);
            R.w[w][lane] = wv;
        }
    }
    __syncthreads();
    const int n_routed = block_group_by_expert(R.id, R.w, M_T, a.k, R.bits, R.pre, R.expert, R.mask, R.weight);
    for (int s = tid; s <= n_routed; s += kThreads) {
        if (s == 0) {
            T.expert[0] = a.E;
            T.mask[0] = full;
#pragma unroll
            for (int m = 0; m < M_T; ++m) T.weight[0][m] = 1.f;
        } else {
            T.expert[s] = R.expert[s - 1];
            T.mask[s] = R.mask[s - 1];
#pragma unroll
            for (int m = 0; m < M_T; ++m) T.weight[s][m] = R.weight[s - 1][m];
        }
    }
    if (tid == 0) T.n_slots = n_routed + 1;
    if ((int)blockIdx.x == a.writer) {          // the routing outputs, as moe_route_topk writes them
        for (int t = tid; t < M_T * a.k; t += kThreads) {
            const int m = t / a.k, r = t - m * a.k;
            if (a.ids_out) a.ids_out[t] = R.id[m][r];
            if (a.w_out) a.w_out[t] = R.w[m][r];
        }
        if (a.disp_out) {
            moedec_dispatch* __restrict__ o = a.disp_out;
            for (int i = tid; i < MOEDEC_MAX_SLOTS; i += kThreads) {
                const bool routed = i < n_routed, shared = i == n_routed;
                o->expert[i] = routed ? R.expert[i] : (shared ? a.E : 0);
                o->token_mask[i] = routed ? R.mask[i] : (shared ? full : 0u);
#pragma unroll
                for (int m = 0; m < MOEDEC_MAX_M; ++m)
                    o->weight[i][m] = (routed && m < M_T) ? R.weight[i][m] : ((shared && m < M_T) ? 1.f : 0.f);
            }
            if (tid == 0) {
                o->n_slots = n_routed + 1;
                o->M = M_T;
            }
        }
    }
}

// Pair counts and slot groups (wave 0).
__device__ void table_groups(const FfnArgs& a, SlotTable& T) {
    if (wave_id_uniform() != 0) return;
    const int lane = lane_id();
    const int n = T.n_slots;
    int carry = 0, last_start = 0;
    for (int base = 0; base < n; base += kWave) {
        const int s = base + lane;
        static_assert(MOEDEC_MAX_M < 8, "pair counts take three bits");
        const int cnt = (s < n) ? __popc(T.mask[s]) : 0;          // 0..MOEDEC_MAX_M
        // exclusive prefix of the counts, bit by bit: one ballot per bit
        int excl = 0, total = 0;
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            const uint64_t bal = __ballot((cnt >> b) & 1);
            excl += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)) << b;
            total += __popcll(bal) << b;
        }
        const int start = carry + excl;
        if (s < n) T.start[s] = start;
        const uint64_t nz = __ballot(cnt > 0);                      // the last slot with a pair
        if (nz) last_start = __builtin_amdgcn_readlane(start, 63 - __clzll((long long)nz));
        carry += total;
    }
    // more groups than launched only with a table not made for this k_max: the rest is dropped
    const int ng = min(last_start / a.pair_cap + 1, a.max_groups);
    if (lane == 0) {
        T.start[n] = carry;
        T.n_groups = ng;
        T.gfirst[0] = 0;
        T.gfirst[ng] = n;
    }
    __builtin_amdgcn_wave_barrier();
    for (int base = 0; base < n; base += kWave) {
        const int s = base + lane;
        if (s > 0 && s < n) {
            const int gs = min(T.start[s] / a.pair_cap, ng);
            const int gp = min(T.start[s - 1] / a.pair_cap, ng);
            for (int g = gp + 1; g <= gs; ++g) T.gfirst[g] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// gate/up unit

// The weights of one gate/up unit in flight: NB chunk pairs per wave.
template <int NB>
struct GuLoads {
    u32x4 cg[NB], cu[NB];
    uint32_t sc[NB];
};

// Issue a gate/up unit's weight loads (nothing when the slot is unused).
template <int M_T, int NB>
__device__ __forceinline__ void gateup_issue_e(const FfnArgs& a, int e, int rg, GuLoads<NB>& L) {
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const uint8_t* cb = (e == a.E) ? a.sh_gu_codes : a.gu_codes + (size_t)e * a.gu_codes_stride;
    const uint8_t* sb = (e == a.E) ? a.sh_gu_scales : a.gu_scales + (size_t)e * a.gu_scales_stride;
    // this wave's chunk pairs (each = 1 KiB gate + 1 KiB up, four MX blocks)
    const int cpw = (a.kbh4 + kWaves - 1) / kWaves;
    const int c_begin = w * cpw;
    const int c_end = min(a.kbh4, c_begin + cpw);
    const uint8_t* ub = cb + (size_t)rg * a.kbh4 * 2048 + lane * 16;
    const uint8_t* usb = sb + (size_t)rg * a.kbh4 * 128 + lane * 2;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = max(0, min(c_begin + i, c_end - 1));   // clamped; extra loads unused
        L.cg[i] = load_stream16(ub + (size_t)c * 2048);
        L.cu[i] = load_stream16(ub + (size_t)c * 2048 + 1024);
        L.sc[i] = *reinterpret_cast<const uint16_t*>(usb + (size_t)c * 128);
    }
}

// FP8 shared expert (SH8): a wave's chunks (64 values per row each, 16 codes
// per lane) go in rounds of NB; this issues round `round` of unit rg.
template <int NB>
__device__ __forceinline__ void gateup_fp8_issue(const FfnArgs& a, int rg, int round, GuLoads<NB>& L) {
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const int kh8 = 2 * a.kbh4;
    const int cpw = (kh8 + kWaves - 1) / kWaves;
    const int c_begin = w * cpw;
    const int c_end = min(kh8, c_begin + cpw);
    const uint8_t* ub = a.sh_gu_codes + (size_t)rg * kh8 * 2048 + lane * 16;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = max(0, min(c_begin + round * NB + i, c_end - 1));   // clamped; extra loads unused
        L.cg[i] = load_stream16(ub + (size_t)c * 2048);
        L.cu[i] = load_stream16(ub + (size_t)c * 2048 + 1024);
    }
}

template <int M_T, int NB, bool SH8 = false>
__device__ __forceinline__ void gateup_issue(const FfnArgs& a, const SlotTable& T, int u, GuLoads<NB>& L) {
    const int s = u / a.gu_units;
    const int rg = u - s * a.gu_units;
    if (s >= T.n_slots) return;
    const int e = T.expert[s];
    if (e < 0) return;
    if (SH8 && e == a.E) {
        gateup_fp8_issue<NB>(a, rg, 0, L);
        return;
    }
    gateup_issue_e<M_T, NB>(a, e, rg, L);
}

// The end of a gate/up unit: sum the four 16-lane rows (cross-lane), then the
// four waves (LDS); with SCALED, times the row scales sg, su (wave 0's lanes);
// h = silu(g) * u, published as tagged words.
template <int M_T, bool SCALED>
__device__ __forceinline__ void gateup_finish(const FfnArgs& a, uint8_t* lds, int s, int rg, uint32_t mask,
                                              const float (&accg)[M_T], const float (&accu)[M_T], uint32_t gen,
                                              float sg, float su) {
    const int w = wave_id_uniform();
    const int lane = lane_id();
    float* red = reinterpret_cast<float*>(lds + a.red_off);    // [waves][M_T][2][16]
#pragma unroll
    for (int m = 0; m < M_T; ++m) {
        const float g = row_sum_f32(accg[m]);
        const float uu = row_sum_f32(accu[m]);
        if (lane < kUnitRows) {
            red[((w * M_T + m) * 2 + 0) * kUnitRows + lane] = g;
            red[((w * M_T + m) * 2 + 1) * kUnitRows + lane] = uu;
        }
    }
    __syncthreads();
    if (w == 0) {
        if (lane < kUnitRows) {
#pragma unroll
            for (int m = 0; m < M_T; ++m) {
                if (!((mask >> m) & 1u)) continue;
                float g = 0.f, uu = 0.f;
#pragma unroll
                for (int v = 0; v < kWaves; ++v) {
                    g += red[((v * M_T + m) * 2 + 0) * kUnitRows + lane];
                    uu += red[((v * M_T + m) * 2 + 1) * kUnitRows + lane];
                }
                if constexpr (SCALED) {
                    g *= sg;
                    uu *= su;
                }
                const float hv = g / (1.f + expf(-g)) * uu;
                store_tagged(&a.h[((size_t)s * M_T + m) * a.I + kUnitRows * rg + lane], gen, hv);
            }
        }
    }
}

// Finish a gate/up unit whose loads gateup_issue put in L: the dot products
// with x (LDS), the reduction over lanes and waves, h = silu(g) * u and its
// publication.
template <int M_T, int NB>
__device__ void gateup_compute(const FfnArgs& a, const SlotTable& T, uint8_t* lds, int u, uint32_t gen,
                               const GuLoads<NB>& L) {
    const int s = u / a.gu_units;
    const int rg = u - s * a.gu_units;
    if (s >= T.n_slots) return;
    const int e = T.expert[s];
    if (e < 0) return;
    const uint32_t mask = T.mask[s];
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const int cpw = (a.kbh4 + kWaves - 1) / kWaves;
    const int c_begin = w * cpw;
    const int c_end = min(a.kbh4, c_begin + cpw);
    const int n_c = c_end - c_begin;

    const int xtok = a.kbh4 * 4 * kXBlock;      // x was staged in LDS by the prologue
    const int quarter = lane >> 4;
    float accg[M_T], accu[M_T];
#pragma unroll
    for (int m = 0; m < M_T; ++m) accg[m] = accu[m] = 0.f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (i < n_c) {
            const int c = c_begin + i;
            const float sg = e8m0_to_f32(L.sc[i] & 0xFFu);
            const float su = e8m0_to_f32(L.sc[i] >> 8);
            bf16x2 wg[16], wu[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                wg[j] = fp4x2_bf16(L.cg[i][j >> 2], sg, j & 3);
                wu[j] = fp4x2_bf16(L.cu[i][j >> 2], su, j & 3);
            }
            const uint8_t* xq = lds + (4 * c + quarter) * kXBlock;
#pragma unroll
            for (int m = 0; m < M_T; ++m) {
                if (M_T > 1 && !((mask >> m) & 1u)) continue;   // the slot does not serve token m
                const u32x4* xp = reinterpret_cast<const u32x4*>(xq + m * xtok);
                u32x4 xr[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) xr[v] = xp[v];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const bf16x2 xx = as_bf16x2(xr[j >> 2][j & 3]);
                    accg[m] = dot2_bf16(wg[j], xx, accg[m]);
                    accu[m] = dot2_bf16(wu[j], xx, accu[m]);
                }
            }
        }
        if (M_T > 2) __builtin_amdgcn_sched_barrier(0);
    }

    gateup_finish<M_T, false>(a, lds, s, rg, mask, accg, accu, gen, 1.f, 1.f);
}

// The shared expert's gate/up unit rg in FP8 (SH8): round 0 of its loads is in
// L (gateup_fp8_issue), later rounds are issued here; codes become exact bf16
// pairs that meet x (LDS) in float32 dot products, and the row scales multiply
// the finished sums.
template <int M_T, int NB>
__device__ void gateup_fp8_unit(const FfnArgs& a, const SlotTable& T, uint8_t* lds, int rg, uint32_t gen,
                                GuLoads<NB> L) {
    const uint32_t mask = T.mask[0];
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const int kh8 = 2 * a.kbh4;
    const int cpw = (kh8 + kWaves - 1) / kWaves;
    const int c_begin = w * cpw;
    const int n_c = min(kh8, c_begin + cpw) - c_begin;
    float sg = 1.f, su = 1.f;                           // row scales, needed by wave 0's lanes < 16
    if (w == 0 && lane < kUnitRows) {
        sg = a.sh8_gu_scale[kUnitRows * rg + lane];
        su = a.sh8_gu_scale[a.I + kUnitRows * rg + lane];
    }
    const int xtok = a.kbh4 * 4 * kXBlock;
    const int quarter = lane >> 4;
    float accg[M_T], accu[M_T];
#pragma unroll
    for (int m = 0; m < M_T; ++m) accg[m] = accu[m] = 0.f;
    for (int round = 0; round * NB < n_c; ++round) {
        if (round > 0) gateup_fp8_issue<NB>(a, rg, round, L);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (round * NB + i < n_c) {
                const int c = c_begin + round * NB + i;
                bf16x2 wg[8], wu[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    wg[j] = (j & 1) ? MOEDEC_FP8X2_BF16(L.cg[i][j >> 1], true) : MOEDEC_FP8X2_BF16(L.cg[i][j >> 1], false);
                    wu[j] = (j & 1) ? MOEDEC_FP8X2_BF16(L.cu[i][j >> 1], true) : MOEDEC_FP8X2_BF16(L.cu[i][j >> 1], false);
                }
                // the lane's 16 values of x: block 2c + quarter / 2, half quarter % 2
                const uint8_t* xq = lds + (2 * c + (quarter >> 1)) * kXBlock + (quarter & 1) * 32;
#pragma unroll
                for (int m = 0; m < M_T; ++m) {
                    if (M_T > 1 && !((mask >> m) & 1u)) continue;
                    const u32x4* xp = reinterpret_cast<const u32x4*>(xq + m * xtok);
                    const u32x4 xr[2] = {xp[0], xp[1]};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const bf16x2 xx = as_bf16x2(xr[j >> 2][j & 3]);
                        accg[m] = dot2_bf16(wg[j], xx, accg[m]);
                        accu[m] = dot2_bf16(wu[j], xx, accu[m]);
                    }
                }
            }
            if (M_T > 2) __builtin_amdgcn_sched_barrier(0);
        }
    }
    gateup_finish<M_T, true>(a, lds, 0, rg, mask, accg, accu, gen, sg, su);
}

// ---------------------------------------------------------------------------
// down unit

template <int M_T, bool ONE, bool SH8 = false, bool A8 = false>
__device__ void down_unit(const FfnArgs& a, SlotTable& T, uint8_t* lds, int d, uint32_t gen) {
    const int n_nc = (a.max_groups - 1) * a.dn_units;    // units of groups 1.. come first
    int grp, g;
    if (d < n_nc) {
        grp = 1 + d / a.dn_units;
        g = d - (grp - 1) * a.dn_units;
    } else {
        grp = 0;
        g = d - n_nc;
    }
    const int n_groups = T.n_groups;
    if (grp >= n_groups) return;
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const int tid = threadIdx.x;
    const int sb = T.gfirst[grp], se = T.gfirst[grp + 1];
    const int pbase = T.start[sb];
    const int n_pairs = T.start[se] - pbase;

    // this wave's items: (slot, chunk), chunk fastest, over the group's slots.
    // With SH8 the shared expert (slot 0, first in group 0) is FP8: its chunks
    // hold 64 values per row, so it has twice the chunks (kbi8) of a slot.
    const bool sh8g = SH8 && grp == 0;
    const int kbi8 = 2 * a.kbi4;
    const int n_items = (se - sb) * a.kbi4 + (sh8g ? a.kbi4 : 0);
    auto item_pos = [&](int i, int& ls, int& ch) {
        if (sh8g && i >= kbi8) {
            ls = 1 + (i - kbi8) / a.kbi4;
            ch = (i - kbi8) - (ls - 1) * a.kbi4;
        } else if (sh8g) {
            ls = 0;
            ch = i;
        } else {
            ls = i / a.kbi4;
            ch = i - ls * a.kbi4;
        }
    };
    auto item_len = [&](int ls) { return (sh8g && ls == 0) ? kbi8 : a.kbi4; };
    const int i_begin = (w * n_items) / kWaves;
    const int i_end = ((w + 1) * n_items) / kWaves;
    constexpr int SUB = dn_sub<M_T, ONE>();
    constexpr int kDnBatch = dn_batch<M_T, ONE>();
    const size_t rg_codes = (size_t)(SUB * g) * a.kbi4 * 1024;
    const size_t rg_scales = (size_t)(SUB * g) * a.kbi4 * 64;
    const int sub_codes = a.kbi4 * 1024, sub_scales = a.kbi4 * 64;   // next 16-row block
    // Weights go in batches of kDnBatch chunks into two register sets (A, B):
    // batches 0 and 1 before h is staged, each next batch while the previous
    // computes.
    // (ONE: one register set; later batches load after the previous computes)
    constexpr int kSetB = ONE ? 1 : kDnBatch;
    u32x4 cwA[kDnBatch][SUB], cwB[kSetB][SUB];
    uint32_t scA[kDnBatch][SUB], scB[kSetB][SUB];
    // items past i_end load the last item again (unused); the walk over
    // (slot, chunk) is branch-free so that no per-item state is carried
    auto load_batch = [&](int i0, u32x4 (&cw)[kDnBatch][SUB], uint32_t (&scw)[kDnBatch][SUB]) {
        int ls, ch;
        item_pos(i0, ls, ch);
#pragma unroll
        for (int k = 0; k < kDnBatch; ++k) {
            const int e = max(T.expert[sb + ls], 0);
            const bool shared = e == a.E;
            if (SH8 && shared) {
                // FP8 layout: row block rb, chunk ch at (rb * kbi8 + ch) KiB
                const uint8_t* cp = a.sh_dn_codes + ((size_t)(SUB * g) * kbi8 + ch) * 1024 + lane * 16;
#pragma unroll
                for (int j = 0; j < SUB; ++j) {
                    cw[k][j] = load_stream16(cp + (size_t)j * kbi8 * 1024);
                    scw[k][j] = 0u;
                }
            } else {
                const size_t ce = shared ? 0 : (size_t)e * a.dn_codes_stride;
                const size_t se = shared ? 0 : (size_t)e * a.dn_scales_stride;
                const uint8_t* cp = (shared ? a.sh_dn_codes : a.dn_codes) + ce + rg_codes + ch * 1024 + lane * 16;
                const uint8_t* sp = (shared ? a.sh_dn_scales : a.dn_scales) + se + rg_scales + ch * 64 + lane;
#pragma unroll
                for (int j = 0; j < SUB; ++j) {
                    cw[k][j] = load_stream16(cp + j * sub_codes);
                    scw[k][j] = sp[j * sub_scales];
                }
            }
            const bool adv = i0 + k + 1 < i_end;
            const bool wrap = ch + 1 == item_len(ls);
            ls += (adv && wrap) ? 1 : 0;
            ch = adv ? (wrap ? 0 : ch + 1) : ch;
        }
    };
    // The group-0 unit finishes the rows: with a residual stream it adds r_in,
    // loaded now (ahead of the weights) rather than after the combine.
    constexpr int kRowsU = SUB * kUnitRows;                     // output rows of this unit
    float rin[M_T];
    // SH8: the FP8 shared expert's row scales of this unit's rows (group 0),
    // loaded now by the first SUB * 16 threads and kept in the reduction
    // area of LDS (unused until the end of the unit) once h is staged
    float sd_own = 0.f;
    if (sh8g && tid < SUB * kUnitRows) sd_own = a.sh8_dn_scale[kUnitRows * SUB * g + tid];
    if (grp == 0 && a.r_out != nullptr && w == 0) {
        const int row = kRowsU * g + (lane & (kRowsU - 1));
#pragma unroll
        for (int m = 0; m < M_T; ++m) rin[m] = a.r_in[(size_t)m * a.H + row];
    }
    if (i_begin < i_end) load_batch(i_begin, cwA, scA);
    if constexpr (!ONE) {
        if (i_begin + kDnBatch < i_end) load_batch(i_begin + kDnBatch, cwB, scB);
    }

    if (w == 0) {
        // the group's (slot, token) pairs
        for (int s = sb + lane; s < se; s += kWave) {
            const uint32_t msk = T.mask[s];
            int p = T.start[s] - pbase;
#pragma unroll
            for (int m = 0; m < M_T; ++m)
                if ((msk >> m) & 1u) T.pair[p++] = (s << 8) | m;
        }
    }
    __syncthreads();

    // Stage w * h: pair p, MX block q at p * pair_bytes + q * 144; padding is
    // zero.  Each 16-byte load brings two tagged h words.  The loads go out
    // right behind the weight loads; after a pause, only the loads whose tags
    // are not this launch's are issued again, until every tag of the batch
    // is, so detection and transfer take one round trip once h is there.
    {
        const __amdgpu_buffer_rsrc_t hrs =
            __builtin_amdgcn_make_buffer_rsrc(a.h, 0, a.h_bytes, kBufferRsrcWord3);
        const int per_pair = a.kbi4 * 4 * 16;              // 16-byte loads per pair, padding included
        const int total = n_pairs * per_pair;
        constexpr int kStage = stage_batch<M_T, ONE>();
        static_assert(kStage <= 32, "one done bit per load");
        const uint32_t all = (1u << kStage) - 1u;
        for (int i0 = 0; i0 < total; i0 += kThreads * kStage) {
            // Load q of this thread covers pair pf[q] >> 16, h words k, k + 1
            // with k = pf[q] & 0xFFFF.  Bit q of `done`: staged, or nothing to
            // stage (past the pairs; MX padding past I, written as zeros here).
            int pf[kStage];
            uint32_t done = 0;
#pragma unroll
            for (int q = 0; q < kStage; ++q) {
                const int idx = i0 + tid + kThreads * q;
                const int ic = min(idx, total - 1);
                const int p = ic / per_pair;
                const int k = (ic - p * per_pair) * 2;
                pf[q] = (p << 16) | k;
                if (idx >= total) {
                    done |= 1u << q;
                } else if (k >= a.I) {
                    *reinterpret_cast<float2*>(lds + p * a.pair_bytes + (k >> 5) * kHBlock + (k & 31) * 4) =
                        make_float2(0.f, 0.f);
                    done |= 1u << q;
                }
            }
            uint32_t spins = 0;
            for (;;) {
                // every attempt consumes its own loads: nothing is carried over
                u32x4 raw[kStage];
#pragma unroll
                for (int q = 0; q < kStage; ++q) {
                    if (!((done >> q) & 1u)) {
                        const int src = T.pair[pf[q] >> 16];
                        const int off = (((src >> 8) * M_T + (src & 0xFF)) * a.I + (pf[q] & 0xFFFF)) *
                                        (int)sizeof(uint64_t);
                        raw[q] = __builtin_amdgcn_raw_buffer_load_b128(hrs, off, 0, kLoadCoherent);
                    }
                }
#pragma unroll
                for (int q = 0; q < kStage; ++q) {
                    if (!((done >> q) & 1u) && raw[q][1] == gen && raw[q][3] == gen) {
                        const int p = pf[q] >> 16, k = pf[q] & 0xFFFF;
                        const int src = T.pair[p];
                        const float wt = A8 ? 1.f : T.weight[src >> 8][src & 0xFF];   // A8: weighted below
                        *reinterpret_cast<float2*>(lds + p * a.pair_bytes + (k >> 5) * kHBlock + (k & 31) * 4) =
                            make_float2(__uint_as_float(raw[q][0]) * wt, __uint_as_float(raw[q][2]) * wt);
                        done |= 1u << q;
                    }
                }
                if (__syncthreads_and(done == all)) break;
                if (++spins > kSpinLimit) {                 // never expected: flag and go on
                    if (tid == 0) atomicOr(a.err, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(4);                 // not there yet: pause before re-reading
            }
        }
    }
    if constexpr (A8) {
        // MXFP8 of each pair's h (blocks of 32 along I, 8 lanes per block,
        // four values each; padding blocks are zero), then the routing weight
        const int per_pair_blk = a.kbi4 * 4, n_blk = n_pairs * per_pair_blk;
        for (int b0 = 0; b0 < n_blk; b0 += kThreads / 8) {
            const int b = b0 + (tid >> 3);
            const bool valid = b < n_blk;
            const int p = valid ? b / per_pair_blk : 0;
            float4* hp =
                reinterpret_cast<float4*>(lds + p * a.pair_bytes + (valid ? b - p * per_pair_blk : 0) * kHBlock) +
                (tid & 7);
            const float4 v = valid ? *hp : make_float4(0.f, 0.f, 0.f, 0.f);
            uint32_t am = max(max(__float_as_uint(v.x) & 0x7FFFFFFFu, __float_as_uint(v.y) & 0x7FFFFFFFu),
                              max(__float_as_uint(v.z) & 0x7FFFFFFFu, __float_as_uint(v.w) & 0x7FFFFFFFu));
            am = max(am, dpp_u32<kQuadSwap1>(am));
            am = max(am, dpp_u32<kQuadSwap2>(am));
            am = max(am, dpp_u32<kRowHalfMirror>(am));
            float X, inv;
            mx8_scale(am, X, inv);
            if (valid) {
                const int src = T.pair[p];
                const float wt = T.weight[src >> 8][src & 0xFF];
                *hp = make_float4(mx8_round(v.x, X, inv) * wt, mx8_round(v.y, X, inv) * wt,
                                  mx8_round(v.z, X, inv) * wt, mx8_round(v.w, X, inv) * wt);
            }
        }
    }
    float* sd_lds = reinterpret_cast<float*>(lds + a.red_off);   // [SUB][16] (SH8, group 0)
    if (sh8g && tid < SUB * kUnitRows) sd_lds[tid] = sd_own;
    __syncthreads();

    const int quarter = lane >> 4;
    constexpr int kCh = SUB == 2 ? 2 : 4;                     // FMA chains per (row, token)
    float acc[kCh][SUB][M_T];
#pragma unroll
    for (int c = 0; c < kCh; ++c)
#pragma unroll
        for (int j = 0; j < SUB; ++j)
#pragma unroll
            for (int m = 0; m < M_T; ++m) acc[c][j][m] = 0.f;
    auto compute_batch = [&](int i0, const u32x4 (&cw)[kDnBatch][SUB], const uint32_t (&scw)[kDnBatch][SUB]) {
        int ls, ch;
        item_pos(i0, ls, ch);
#pragma unroll
        for (int k = 0; k < kDnBatch; ++k) {
            if (SH8 && sh8g && ls == 0 && i0 + k < i_end) {
                // FP8 item: the lane's 16 values of h (block 2ch + quarter / 2,
                // half quarter % 2) against 16 codes per row block, each code's
                // exact value times its row's scale
                const uint8_t* hq = lds + (2 * ch + (quarter >> 1)) * kHBlock + (quarter & 1) * 64;
                const uint32_t msk = (M_T == 1) ? 1u : T.mask[sb];
                int p = 0;
#pragma unroll
                for (int m = 0; m < M_T; ++m) {
                    if (M_T > 1 && !((msk >> m) & 1u)) continue;
                    const float4* hp = reinterpret_cast<const float4*>(hq + p * a.pair_bytes);
                    ++p;
                    float4 hv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) hv[v] = hp[v];
#pragma unroll
                    for (int j = 0; j < SUB; ++j) {
                        const float sj = sd_lds[j * kUnitRows + (lane & 15)];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const f32x2 w0 = MOEDEC_FP8X2_F32(cw[k][j][v], false);
                            const f32x2 w1 = MOEDEC_FP8X2_F32(cw[k][j][v], true);
                            acc[0][j][m] = fmaf(w0.x * sj, hv[v].x, acc[0][j][m]);
                            acc[1 % kCh][j][m] = fmaf(w0.y * sj, hv[v].y, acc[1 % kCh][j][m]);
                            acc[2 % kCh][j][m] = fmaf(w1.x * sj, hv[v].z, acc[2 % kCh][j][m]);
                            acc[3 % kCh][j][m] = fmaf(w1.y * sj, hv[v].w, acc[3 % kCh][j][m]);
                        }
                    }
                }
            } else if (i0 + k < i_end) {
                const int s = sb + ls;
                // one token: every slot serves it, so slot sb + j holds pair j
                // (no table lookups on the way to the LDS reads)
                const uint32_t msk = (M_T == 1) ? 1u : T.mask[s];
                const int p0 = (M_T == 1) ? ls : T.start[s] - pbase;
                float sc[SUB];
#pragma unroll
                for (int j = 0; j < SUB; ++j) sc[j] = e8m0_to_f32(scw[k][j]);
                const uint8_t* hq = lds + (4 * ch + quarter) * kHBlock;
                int p = p0;
#pragma unroll
                for (int m = 0; m < M_T; ++m) {
                    // with one token every slot of a group serves it; otherwise skip the
                    // tokens the slot does not serve (its weight is zero anyway)
                    if (M_T > 1 && !((msk >> m) & 1u)) continue;
                    // the LDS reads of this (slot, token) go out back to back, in
                    // halves when the unit has two row blocks (register pressure)
                    const float4* hp = reinterpret_cast<const float4*>(hq + p * a.pair_bytes);
                    constexpr int kHv = SUB == 2 ? 4 : 8;
                    ++p;
#pragma unroll
                    for (int v0 = 0; v0 < 8; v0 += kHv) {
                    float4 hv[kHv];
#pragma unroll
                    for (int v = 0; v < kHv; ++v) hv[v] = hp[v0 + v];
#pragma unroll
                    for (int j = 0; j < SUB; ++j) {
#pragma unroll
                        for (int vv = 0; vv < kHv; ++vv) {
                            const int v = v0 + vv;
                            // four weights: bytes 2v and 2v+1 of the lane's 16 code bytes
                            const f32x2 w0 = fp4x2_f32(cw[k][j][v >> 1], sc[j], (2 * v) & 3);
                            const f32x2 w1 = fp4x2_f32(cw[k][j][v >> 1], sc[j], (2 * v + 1) & 3);
                            acc[0][j][m] = fmaf(w0.x, hv[vv].x, acc[0][j][m]);
                            acc[1 % kCh][j][m] = fmaf(w0.y, hv[vv].y, acc[1 % kCh][j][m]);
                            acc[2 % kCh][j][m] = fmaf(w1.x, hv[vv].z, acc[2 % kCh][j][m]);
                            acc[3 % kCh][j][m] = fmaf(w1.y, hv[vv].w, acc[3 % kCh][j][m]);
                        }
                    }
                    }
                }
            }
            if (++ch == item_len(ls)) {
                ch = 0;
                ++ls;
            }
            if (M_T > 1) __builtin_amdgcn_sched_barrier(0);   // bound register pressure: one item at a time
        }
    };
    if constexpr (ONE) {
        for (int i0 = i_begin; i0 < i_end; i0 += kDnBatch) {
            if (i0 != i_begin) load_batch(i0, cwA, scA);
            compute_batch(i0, cwA, scA);
        }
    } else {
        for (int i0 = i_begin; i0 < i_end; i0 += 2 * kDnBatch) {
            compute_batch(i0, cwA, scA);
            if (i0 + 2 * kDnBatch < i_end) load_batch(i0 + 2 * kDnBatch, cwA, scA);
            if (i0 + kDnBatch < i_end) compute_batch(i0 + kDnBatch, cwB, scB);
            if (i0 + 3 * kDnBatch < i_end) load_batch(i0 + 3 * kDnBatch, cwB, scB);
        }
    }

    if (sh8g) __syncthreads();                                  // every wave is done with sd_lds
    float* red = reinterpret_cast<float*>(lds + a.red_off);    // [waves][M_T][SUB][16]
#pragma unroll
    for (int m = 0; m < M_T; ++m)
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
            float t = acc[0][j][m] + acc[1][j][m];
            if constexpr (kCh == 4) t += acc[2 % kCh][j][m] + acc[3 % kCh][j][m];
            const float r = row_sum_f32(t);
            if (lane < kUnitRows) red[((w * M_T + m) * SUB + j) * kUnitRows + lane] = r;
        }
    __syncthreads();
    if (w != 0) return;
    constexpr int kRows = SUB * kUnitRows;                      // output rows of this unit
    const int lr = lane & (kRows - 1);                          // lanes >= kRows mirror lanes < kRows
    const int row = kRows * g + lr;
    float y[M_T];
#pragma unroll
    for (int m = 0; m < M_T; ++m) {
        y[m] = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) y[m] += red[((v * M_T + m) * SUB + (lr >> 4)) * kUnitRows + (lr & 15)];
    }
    if (n_groups > 1) {
        if (grp != 0) {
            if (lane < kRows) {
#pragma unroll
                for (int m = 0; m < M_T; ++m) store_tagged(&a.part[((size_t)grp * M_T + m) * a.H + row], gen, y[m]);
            }
            return;
        }
        // group 0 adds the other groups' partial rows, in group order, once
        // their tags say they are from this launch
        const int prow = row;                                   // in bounds for every lane
        for (int gg = 1; gg < n_groups; ++gg) {
            uint64_t pv[M_T];
            uint32_t spins = 0;
            for (;;) {
                bool ok = true;
#pragma unroll
                for (int m = 0; m < M_T; ++m) {
                    pv[m] = load_tagged(&a.part[((size_t)gg * M_T + m) * a.H + prow]);
                    ok &= (uint32_t)(pv[m] >> 32) == gen;
                }
                if (__all(ok)) break;
                if (++spins > kSpinLimit) {
                    if (lane == 0) atomicOr(a.err, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
#pragma unroll
            for (int m = 0; m < M_T; ++m) y[m] += __uint_as_float((uint32_t)pv[m]);
        }
    }
    if (lane < kRows) {
#pragma unroll
        for (int m = 0; m < M_T; ++m) {
            const size_t o = (size_t)m * a.H + row;
            if (a.y_f32) a.y_f32[o] = y[m];
            if (a.y_bf16) a.y_bf16[o] = f32_to_bf16_rne(y[m]);
            if (a.r_out) a.r_out[o] = rin[m] + y[m];
        }
    }
}

// ---------------------------------------------------------------------------
// prologue pieces

// 16-byte pieces of the layer input per thread: M_T * H bf16 values, or the
// float32 residual stream (twice the bytes) when x is formed by RMSNorm.
template <int M_T, bool NORM>
constexpr int x_pieces() { return (NORM ? 4 : 2) * M_T; }

// x (or r) loads: unconditional, clamped index; H <= 4096 fits the pieces.
template <int M_T, bool NORM>
__device__ __forceinline__ void x_issue(const FfnArgs& a, u32x4 (&xv)[x_pieces<M_T, NORM>()]) {
    const int per_tok = NORM ? a.H / 4 : a.H / 8;
    const int n_pieces = M_T * per_tok;
    const u32x4* src = NORM ? reinterpret_cast<const u32x4*>(a.r_in) : reinterpret_cast<const u32x4*>(a.x);
#pragma unroll
    for (int i = 0; i < x_pieces<M_T, NORM>(); ++i) xv[i] = src[min((int)threadIdx.x + kThreads * i, n_pieces - 1)];
}

// x into the LDS x area (token m, MX block q at m * xtok + q * 80), zero past
// H.  With NORM, x = bf16(RMSNorm(r)) with unit gain: r / sqrt(mean(r^2) + eps)
// in float32, rounded to bf16 (nearest even); the writer block also exports x.
// Contains a block barrier (NORM); the caller's barrier publishes the stores.
template <int M_T, bool NORM>
__device__ void x_stage(const FfnArgs& a, const u32x4 (&xv)[x_pieces<M_T, NORM>()], uint8_t* lds) {
    constexpr int kPieces = x_pieces<M_T, NORM>();
    const int tid = threadIdx.x;
    const int per_tok = NORM ? a.H / 4 : a.H / 8;
    const int n_pieces = M_T * per_tok;
    const int xtok = a.kbh4 * 4 * kXBlock;
    if constexpr (NORM) {
        // piece p holds elements 4r..4r+3
        static_assert(kThreads == 256 && kWaves == 4, "rmsnorm_factors takes a block of 256 threads");
        float inv[M_T];
        rmsnorm_factors<M_T>(xv, n_pieces, per_tok, a.H, a.eps, inv);
        const bool export_x = (int)blockIdx.x == a.writer && a.x_out != nullptr;
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int p = tid + kThreads * i;
            if (p < n_pieces) {
                const int pm = p / per_tok;
                const int e0 = 4 * (p - pm * per_tok);
                float sc = inv[0];
#pragma unroll
                for (int m = 1; m < M_T; ++m) sc = (m == pm) ? inv[m] : sc;
                const uint32_t b0 = f32_to_bf16_rne(__uint_as_float(xv[i][0]) * sc);
                const uint32_t b1 = f32_to_bf16_rne(__uint_as_float(xv[i][1]) * sc);
                const uint32_t b2 = f32_to_bf16_rne(__uint_as_float(xv[i][2]) * sc);
                const uint32_t b3 = f32_to_bf16_rne(__uint_as_float(xv[i][3]) * sc);
                const uint2 packed = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                *reinterpret_cast<uint2*>(lds + pm * xtok + (e0 >> 5) * kXBlock + (e0 & 31) * 2) = packed;
                if (export_x) *reinterpret_cast<uint2*>(a.x_out + (size_t)pm * a.H + e0) = packed;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int p = tid + kThreads * i;
            if (p < n_pieces) {
                const int m = p / per_tok;
                const int r = p - m * per_tok;
                *reinterpret_cast<u32x4*>(lds + m * xtok + (r >> 2) * kXBlock + (r & 3) * 16) = xv[i];
            }
        }
    }
    const int pad_pieces = (a.kbh4 * 4 - a.kbh) * 4;      // MX blocks past H are zero
    for (int p = tid; p < M_T * pad_pieces; p += kThreads) {
        const int m = p / pad_pieces;
        const int r = p - m * pad_pieces;
        *reinterpret_cast<u32x4*>(lds + m * xtok + (a.kbh + (r >> 2)) * kXBlock + (r & 3) * 16) =
            u32x4{0u, 0u, 0u, 0u};
    }
}

// MXFP8 of the staged x in place (W4A8): each 32-value block of each token
// (64 bytes in the x area) by 4 lanes, 8 values each; the block's largest
// magnitude by two lane swaps, then every value rounded to its MXFP8 value
// (exact in bf16).  Runs while the first unit's weight loads are in flight;
// the caller's barrier publishes the stores.
template <int M_T>
__device__ void x_quant_lds(const FfnArgs& a, uint8_t* lds) {
    const int tid = threadIdx.x;
    const int xtok = a.kbh4 * 4 * kXBlock, n_blk = M_T * a.kbh;
    for (int b0 = 0; b0 < n_blk; b0 += kThreads / 4) {
        const int b = b0 + (tid >> 2);
        const bool valid = b < n_blk;
        const int m = valid ? b / a.kbh : 0;
        u32x4* p = reinterpret_cast<u32x4*>(lds + m * xtok + (valid ? b - m * a.kbh : 0) * kXBlock + (tid & 3) * 16);
        u32x4 v = valid ? *p : u32x4{0u, 0u, 0u, 0u};
        uint32_t am = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) am = max(am, max(v[e] & 0x7FFFu, (v[e] >> 16) & 0x7FFFu));
        am = max(am, dpp_u32<kQuadSwap1>(am));
        am = max(am, dpp_u32<kQuadSwap2>(am));
        float X, inv;
        mx8_scale(am << 16, X, inv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = mx8_round(bf16_to_f32(v[e] & 0xFFFFu), X, inv);
            const float hi = mx8_round(bf16_to_f32(v[e] >> 16), X, inv);
            v[e] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
        }
        if (valid) *p = v;
    }
}

// The launch count on the workspace: every one of the kMaxGrid words advances
// once per launch (block b takes b, b + grid, ...), so all blocks agree
// whatever the grid of earlier launches.  One thread per block.
__device__ __forceinline__ uint32_t gens_advance(const FfnArgs& a) {
    const uint32_t g = a.gens[blockIdx.x] + 1u;
    for (int j = blockIdx.x; j < kMaxGrid; j += gridDim.x) a.gens[j] = g;
    return g;
}

// A gate/up unit whose round-0 loads are in L: the FP8 shared expert's units
// (slot 0 with SH8) or an MXFP4 unit.
template <int M_T, int NB, bool SH8>
__device__ __forceinline__ void gateup_run(const FfnArgs& a, const SlotTable& T, uint8_t* lds, int u, uint32_t gen,
                                           const GuLoads<NB>& L) {
    if (SH8 && u < a.gu_units)
        gateup_fp8_unit<M_T, NB>(a, T, lds, u, gen, L);
    else
        gateup_compute<M_T, NB>(a, T, lds, u, gen, L);
}

template <int M_T, int NB, bool ROUTE, bool NORM, bool ONE, bool SH8, bool A8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(blocks_per_cu<ONE>())))
void moe_ffn_kernel(FfnArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ SlotTable T;
    __shared__ uint32_t s_gen;
    const int tid = threadIdx.x;
    const int unit0 = (int)blockIdx.x;                     // first unit (ONE: the only one)
    const bool has_gu = unit0 < a.n_gu;                    // the block runs a gate/up unit
    constexpr int kPieces = x_pieces<M_T, NORM>();

    if constexpr (ONE) {
        // The shared expert (slot 0) does not depend on routing: with a block
        // per unit, its gate/up blocks issue their weight loads first thing and
        // never route (the writer block is another), so these bytes stream
        // while the other blocks select their experts.
        if (unit0 < a.gu_units) {
            GuLoads<NB> cur;
            if constexpr (SH8)
                gateup_fp8_issue<NB>(a, unit0, 0, cur);
            else
                gateup_issue_e<M_T, NB>(a, a.E, unit0, cur);
            u32x4 xv[kPieces];
            x_issue<M_T, NORM>(a, xv);
            if (tid == kThreads - kWave) s_gen = gens_advance(a);
            if (tid == 0) {
                T.n_slots = 1;
                T.expert[0] = a.E;
                T.mask[0] = (1u << M_T) - 1u;
            }
            x_stage<M_T, NORM>(a, xv, lds);
            __syncthreads();
            if constexpr (A8) {
                x_quant_lds<M_T>(a, lds);
                __syncthreads();
            }
            gateup_run<M_T, NB, SH8>(a, T, lds, unit0, s_gen, cur);
            return;
        }
    }

    // The routing waves' logits go out first (loads return in order and the
    // top-k needs them before anything else; lane l holds entries l + 64 t).
    float lv[16];
    if (ROUTE && wave_id_uniform() < M_T) {
        const float* row = a.logits + (size_t)wave_id_uniform() * a.E;
        if (a.E <= 512)
            topk_load<8>(row, a.E, *reinterpret_cast<float(*)[8]>(lv));
        else
            topk_load<16>(row, a.E, lv);
    }
    // x does not depend on routing: its loads go out next, and are staged in
    // LDS once the slot table is built.  With a residual input the loads bring
    // r and x = bf16(RMSNorm(r)) is formed after routing.
    u32x4 xv[kPieces];
    if (has_gu) x_issue<M_T, NORM>(a, xv);
    if (tid == kThreads - kWave) s_gen = gens_advance(a);   // wave 3: keeps wave 0 free to route
    constexpr bool kDirectGroups = ROUTE && M_T == 1;     // the table arrives with its groups
    // routing borrows the reduction area (kTopkBufWords words per routing
    // wave), which the units use only after the prologue
    uint64_t* route_buf = reinterpret_cast<uint64_t*>(lds + a.red_off);
    if (kDirectGroups)
        table_from_logits_one(a, T, route_buf, lv);
    else if (ROUTE)
        table_from_logits<M_T>(a, T, route_buf, lv);
    else
        table_from_dispatch<M_T>(a, T);
    if (has_gu) x_stage<M_T, NORM>(a, xv, lds);
    __syncthreads();
    // The slot groups (pair starts, group bounds) matter only to down units.
    // A persistent block with gate/up units builds them while its first
    // unit's weight loads are in flight (that unit's barriers publish them):
    // on a busy CU wave 0 needs up to ~2.6 us for it, which must not hold up
    // the loads.  Other blocks build them here.
    const bool groups_late = !kDirectGroups && !ONE && has_gu;
    if (!kDirectGroups && !groups_late) {
        table_groups(a, T);
        __syncthreads();
    }
    const uint32_t gen = s_gen;
    // Gate/up units come first: a block's next one has its weight loads in
    // flight while the current one computes.  Then its down units.
    int u = unit0;
    if (ONE) {
        for (; u < a.n_gu; u += gridDim.x) {
            GuLoads<NB> cur;
            gateup_issue<M_T, NB, SH8>(a, T, u, cur);
            if constexpr (A8) {
                if (u == unit0) {
                    x_quant_lds<M_T>(a, lds);
                    __syncthreads();
                }
            }
            gateup_run<M_T, NB, SH8>(a, T, lds, u, gen, cur);
            __syncthreads();
        }
    } else if (u < a.n_gu) {
        // (Issuing the first down unit's weights during the last gate/up unit
        // instead was slower at 4 tokens, 34.3 against 32.4 us: they compete
        // with the gate/up stream that every down unit waits for.)
        GuLoads<NB> cur, nxt;
        gateup_issue<M_T, NB, SH8>(a, T, u, cur);
        if constexpr (A8) {
            x_quant_lds<M_T>(a, lds);
            __syncthreads();
        }
        bool groups_pending = groups_late;
        for (; u < a.n_gu; u += gridDim.x) {
            const int un = u + gridDim.x;
            if (un < a.n_gu) gateup_issue<M_T, NB, SH8>(a, T, un, nxt);
            if (groups_pending) {                          // wave 0; published by the unit's barrier
                table_groups(a, T);
                groups_pending = false;
            }
            gateup_run<M_T, NB, SH8>(a, T, lds, u, gen, cur);
            cur = nxt;
            __syncthreads();
        }
    }
    for (; u < a.n_units; u += gridDim.x) {
        down_unit<M_T, ONE, SH8, A8>(a, T, lds, u - a.n_gu, gen);
        __syncthreads();
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

constexpr size_t kLdsTarget = 40 * 1024;
constexpr int kOneTokenPairs = 3;
constexpr int kMultiTokenPairs = 4;

// CU count of the current device (cached); the grid is blocks_per_cu * CUs.
struct DeviceInfo {
    int cus = 0;
    std::mutex mu;
};
DeviceInfo g_dev[64];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    DeviceInfo& d = g_dev[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    if (d.cus == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        d.cus = cus;
    }
    return d.cus;
}

template <int M_T, int NB, bool ROUTE, bool NORM, bool ONE, bool SH8, bool A8>
hipError_t launch_variant(const FfnArgs& a, int cus, size_t lds, hipStream_t s) {
    constexpr int kBlocksPerCU = blocks_per_cu<ONE>();
    // ONE: a block per unit (the host picks ONE only when they all fit)
    const int grid = ONE ? std::min(a.n_units, kMaxGrid) : std::min(kMaxGrid, kBlocksPerCU * cus);
    // every block must be resident at once: check the occupancy of this variant
    static std::atomic<int> occ_ok[256];                      // per LDS size class of 256 B
    const size_t cls = std::min<size_t>((lds + 255) / 256, 255);
    int v = occ_ok[cls].load(std::memory_order_relaxed);
    if (v == 0) {
        int blocks = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void*>(&moe_ffn_kernel<M_T, NB, ROUTE, NORM, ONE, SH8, A8>), kThreads, lds);
        if (e != hipSuccess) return e;
        v = (blocks >= kBlocksPerCU) ? 1 : 2;
        occ_ok[cls].store(v, std::memory_order_relaxed);
    }
    if (v != 1) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((moe_ffn_kernel<M_T, NB, ROUTE, NORM, ONE, SH8, A8>), dim3(grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

template <int M_T, bool ROUTE, bool NORM, bool ONE, bool SH8, bool A8>
hipError_t launch_nb(const FfnArgs& a, int nb, int cus, size_t lds, hipStream_t s) {
    switch (nb) {
        case 1: return launch_variant<M_T, 1, ROUTE, NORM, ONE, SH8, A8>(a, cus, lds, s);
        case 2: return launch_variant<M_T, 2, ROUTE, NORM, ONE, SH8, A8>(a, cus, lds, s);
        case 4: return launch_variant<M_T, 4, ROUTE, NORM, ONE, SH8, A8>(a, cus, lds, s);
        case 5: return launch_variant<M_T, 5, ROUTE, NORM, ONE, SH8, A8>(a, cus, lds, s);
        default: return launch_variant<M_T, 8, ROUTE, NORM, ONE, SH8, A8>(a, cus, lds, s);
    }
}

// One token: a block per unit when the units fit four blocks per CU (and the
// variant's occupancy allows it), else the general three-block grid.
template <int M_T, bool ROUTE, bool NORM, bool SH8, bool A8 = false>
hipError_t launch_one(const FfnArgs& a, int nb, int cus, size_t lds, hipStream_t s) {
    if constexpr (M_T == 1) {
        FfnArgs b = a;                                  // the down units of the ONE form
        b.dn_units = a.H / (kUnitRows * dn_sub<1, true>());
        b.n_units = b.n_gu + b.max_groups * b.dn_units;
        b.writer = b.gu_units;                          // slot 1's first gate/up block routes; slot 0's do not
        if (b.n_units <= std::min(kMaxGrid, blocks_per_cu<true>() * cus)) {
            const hipError_t e = launch_nb<M_T, ROUTE, NORM, true, SH8, A8>(b, nb, cus, lds, s);
            if (e != hipErrorInvalidConfiguration) return e;
        }
    }
    return launch_nb<M_T, ROUTE, NORM, false, SH8, A8>(a, nb, cus, lds, s);
}

// routing from logits with or without the residual stream, or from a table
// (the table form takes an MXFP4 shared expert only)
template <int M_T, bool SH8>
hipError_t launch_m(const FfnArgs& a, int nb, int cus, size_t lds, hipStream_t s) {
    if (a.r_in) return launch_one<M_T, true, true, SH8>(a, nb, cus, lds, s);
    if (a.a8) {                                      // W4A8: routed from logits, MXFP4 shared expert
        if constexpr (SH8) return hipErrorInvalidValue;
        else return launch_one<M_T, true, false, false, true>(a, nb, cus, lds, s);
    }
    if (a.logits) return launch_one<M_T, true, false, SH8>(a, nb, cus, lds, s);
    if constexpr (SH8)
        return hipErrorInvalidValue;
    else
        return launch_one<M_T, false, false, false>(a, nb, cus, lds, s);
}

}  // namespace

FfnLayout ffn_layout(int M, int k_max, int H, int I) {
    FfnLayout L;
    const int kbh4 = (H / 32 + 3) / 4, kbi4 = (I / 32 + 3) / 4;
    L.max_slots = M * k_max + 1;
    L.pair_bytes = kbi4 * 4 * kHBlock;
    // the reduction area, also lent to the routing waves (kTopkBufWords each)
    const size_t red_bytes = std::max((size_t)kWaves * M * 2 * kUnitRows * sizeof(float),
                                      (size_t)M * kTopkBufWords * sizeof(uint64_t));
    const size_t x_bytes = (size_t)M * kbh4 * 4 * kXBlock;
    // a group (at most pair_cap + M - 1 pairs: it ends on a slot boundary)
    // must fit the LDS target.  Smaller groups shorten each down unit and cost
    // partial-row exchanges; on a 2560 x 768 layer the best balance was groups
    // of 3 pairs at M = 1 (14.8 us against 15.3 for 4 and 15.9 for 5), made
    // equal in size and within one staging batch so h arrives in one round
    // trip, and of kMultiTokenPairs at M = 4, staged in several batches
    // (42 us against 46 us for the LDS limit of 8 and 58 us for groups of 2).
    const int fit_lds = (int)((kLdsTarget - red_bytes) / L.pair_bytes) - (M - 1);
    const int max_pairs = M * k_max + M;
    int cap;
    if (M == 1) {
        const int loads_per_pair = kbi4 * 4 * 16;                   // 16-byte loads (two h words each)
        const int fit_stage = stage_batch<1, false>() * kThreads / loads_per_pair;
        cap = std::max(1, std::min(std::min(fit_lds, fit_stage), std::min(kOneTokenPairs, max_pairs)));
        const int n_groups = (max_pairs + cap - 1) / cap;
        cap = (max_pairs + n_groups - 1) / n_groups;                // equal groups
    } else {
        cap = std::max(1, std::min(fit_lds, std::min(kMultiTokenPairs, max_pairs)));
    }
    L.pair_cap = cap;
    L.max_groups = (max_pairs + L.pair_cap - 1) / L.pair_cap;
    const size_t h_bytes = (size_t)(L.pair_cap + M - 1) * L.pair_bytes;
    const size_t region = std::max(x_bytes, h_bytes);
    L.red_off = (int)((region + 15) & ~(size_t)15);
    L.lds_bytes = L.red_off + red_bytes;
    // the fixed-size part first, so a workspace serves any M / k_max it is big enough for
    L.ctl_off = 0;                                                      // gens + error word
    L.yt_off = 0;
    L.h_off = align256((size_t)(kMaxGrid + 64) * sizeof(uint32_t));
    L.part_off = L.h_off + align256((size_t)L.max_slots * M * I * sizeof(uint64_t));
    L.total = L.part_off + (L.max_groups > 1 ? align256((size_t)L.max_groups * M * H * sizeof(uint64_t)) : 0);
    L.grid = 0;
    return L;
}

hipError_t launch_moe(const moedec_moe_weights& w, const uint16_t* x, int M, int k_max,
                      const moedec_dispatch* disp, const float* logits, int32_t* ids_out,
                      float* w_out, moedec_dispatch* disp_out, uint16_t* y_bf16, float* y_f32,
                      void* ws, hipStream_t s, const ResidualArgs* res, bool a8) {
    const FfnLayout L = ffn_layout(M, k_max, w.H, w.I);
    const int cus = device_cus();
    if (cus <= 0) return hipErrorInvalidDevice;
    uint8_t* base = static_cast<uint8_t*>(ws);
    moedec_mxfp4_sizes sz;
    packed_sizes(w.H, w.I, &sz);

    FfnArgs a;
    a.gu_codes = w.gu_codes;
    a.gu_scales = w.gu_scales;
    a.dn_codes = w.dn_codes;
    a.dn_scales = w.dn_scales;
    a.sh_gu_codes = w.sh_gu_codes;
    a.sh_gu_scales = w.sh_gu_scales;
    a.sh_dn_codes = w.sh_dn_codes;
    a.sh_dn_scales = w.sh_dn_scales;
    a.gu_codes_stride = sz.gu_codes;
    a.gu_scales_stride = sz.gu_scales;
    a.dn_codes_stride = sz.dn_codes;
    a.dn_scales_stride = sz.dn_scales;
    a.E = w.E;
    a.H = w.H;
    a.I = w.I;
    a.k = k_max;
    a.kbh = w.H / 32;
    a.kbh4 = (a.kbh + 3) / 4;
    a.kbi = w.I / 32;
    a.kbi4 = (a.kbi + 3) / 4;
    a.gu_units = w.I / kUnitRows;
    a.dn_units = w.H / (kUnitRows * (M == 1 ? dn_sub<1, false>() : dn_sub<2, false>()));
    a.max_slots = L.max_slots;
    a.max_groups = L.max_groups;
    a.pair_cap = L.pair_cap;
    a.n_gu = L.max_slots * a.gu_units;
    a.n_units = a.n_gu + L.max_groups * a.dn_units;
    a.pair_bytes = L.pair_bytes;
    a.red_off = L.red_off;
    a.a8 = a8 ? 1 : 0;
    a.writer = 0;
    a.x = x;
    a.disp = disp;
    a.logits = logits;
    a.ids_out = ids_out;
    a.w_out = w_out;
    a.disp_out = disp_out;
    uint32_t* ctl = reinterpret_cast<uint32_t*>(base + L.ctl_off);
    a.gens = ctl;
    a.err = ctl + kMaxGrid;
    a.h = reinterpret_cast<uint64_t*>(base + L.h_off);
    a.part = reinterpret_cast<uint64_t*>(base + L.part_off);
    a.h_bytes = (int)((size_t)L.max_slots * M * w.I * sizeof(uint64_t));
    a.y_bf16 = y_bf16;
    a.y_f32 = y_f32;
    a.r_in = res ? res->r_in : nullptr;
    a.r_out = res ? res->r_out : nullptr;
    a.x_out = res ? res->x_out : nullptr;
    a.eps = res ? res->eps : 0.f;

    const int cpw = (a.kbh4 + kWaves - 1) / kWaves;   // chunk pairs per wave, <= 8 for H <= 4096
    const int nb = cpw <= 1 ? 1 : cpw <= 2 ? 2 : cpw <= 4 ? 4 : cpw <= 5 ? 5 : 8;
    if (a.r_in && !a.logits) return hipErrorInvalidValue;     // the residual form routes from logits
    const bool sh8 = w.magic == MOEDEC_MOE_MAGIC_SHARED_FP8;
    a.sh8_gu_scale = sh8 ? reinterpret_cast<const float*>(w.sh_gu_scales) : nullptr;
    a.sh8_dn_scale = sh8 ? reinterpret_cast<const float*>(w.sh_dn_scales) : nullptr;
    if (sh8) {
        switch (M) {
            case 1: return launch_m<1, true>(a, nb, cus, L.lds_bytes, s);
            case 2: return launch_m<2, true>(a, nb, cus, L.lds_bytes, s);
            case 3: return launch_m<3, true>(a, nb, cus, L.lds_bytes, s);
            default: return launch_m<4, true>(a, nb, cus, L.lds_bytes, s);
        }
    }
    switch (M) {
        case 1: return launch_m<1, false>(a, nb, cus, L.lds_bytes, s);
        case 2: return launch_m<2, false>(a, nb, cus, L.lds_bytes, s);
        case 3: return launch_m<3, false>(a, nb, cus, L.lds_bytes, s);
        default: return launch_m<4, false>(a, nb, cus, L.lds_bytes, s);
    }
}

hipError_t launch_expert_ffn(const moedec_moe_weights& w, const uint16_t* x, int M,
                             const moedec_dispatch* disp, int k_max, uint16_t* y_bf16,
                             float* y_f32, void* ws, hipStream_t s) {
    return launch_moe(w, x, M, k_max, disp, nullptr, nullptr, nullptr, nullptr, y_bf16, y_f32, ws, s);
}

}  // namespace moedec
