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

// Argmax key of logit `val` at row `row` (row < 2^20): larger logit first,
// then the lower row (float_order puts -0.0 and +0.0 together, so the row
// decides there too).  Bits 20..31 stay clear for the launch tag that the
// epilogue ORs in when it publishes a key (equal within one launch, so it
// never changes an order).
constexpr int kEpilogueRowsPerWave = 32;       // rows per wave of the GEMV with an epilogue
constexpr int kBlockRows = 4 * kEpilogueRowsPerWave;
constexpr uint32_t kRowBits = 20;
constexpr uint32_t kRowMask = (1u << kRowBits) - 1;
__device__ __forceinline__ uint64_t argmax_key(float val, int row) {
    return ((uint64_t)float_order(val) << 32) | (uint64_t)(kRowMask - (uint32_t)row);
}
__device__ __forceinline__ int32_t key_row(uint64_t key) {
    return (int32_t)(kRowMask - ((uint32_t)key & kRowMask));
}

// Maximum over groups of `WIDTH` consecutive lanes (the whole wave by default).
template <int WIDTH = kWave>
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
    for (int off = WIDTH / 2; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, off);
        const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    return k;
}

// Writes the R x M_T row sums of a wave step: acc[r][m] summed over the wave
// (multi_sum: lane l ends with value l >> kShift) and scaled by scale(r).
// Without KEYS they go to logits; with KEYS to the block's LDS rows
// (rows_lds[m][lrow + r], lrow = the step's first row within the block), so
// that no global store is in flight while the wave streams.
template <int R, int M_T, bool KEYS, typename Scale>
__device__ __forceinline__ void store_row_sums(const float (&acc)[R][M_T], int v, int v1, int V,
                                               float* __restrict__ logits, Scale scale,
                                               float* __restrict__ rows_lds, int lrow) {
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
            if constexpr (KEYS)
                rows_lds[m * kBlockRows + lrow + r] = val;
            else
                logits[(size_t)m * V + v + r] = val;
        }
    }
}

// ---------------------------------------------------------------------------
// The GEMV's tail: the greedy token or a sampled one, computed by the last
// blocks of the launch, so no second launch is needed.
//
// Cross-block protocol, without read-modify-writes, fences or cache flushes
// (as in the MoE FFN kernel): every word a block publishes for another -- its
// best key per token, and when sampling each wave's best key and every row's
// key -- is one 64-bit agent-scope atomic store whose bits 20..31 carry a tag
// of the launch.  The tag comes from a generation word per block (kMaxBlocks
// of them at the start of the workspace): each block reads its own word when
// it starts and, once done, writes the next generation to it and to every
// word it stands for in smaller grids (b, b + grid, ...), so all words stay
// equal and every block of a launch sees the same generation.  The word holds
// two 16-bit counts: launches (tags of the block keys, written by every call)
// and sampling launches (tags of the wave and row keys, written only then),
// so consecutive writes of any key always differ in tag.  The blocks launched
// last -- one per token -- poll the published words until each carries this
// launch's tag (launches on one stream are ordered, so a load returns this
// launch's store or an older one) and compute the token.  A tag is a count's
// low 11 bits with bit 11 set, so a zero-filled workspace never looks current
// and every published key is nonzero.
//
// Sampling narrows in three steps, each loaded at once into registers: the
// top_k blocks by block maximum, the top_k waves among their waves, the top_k
// rows among those waves' rows.  A block or wave outside the top_k by maximum
// has top_k others with a larger maximum, each holding a larger logit than
// any of its rows, so every step keeps all of the top_k logits.

constexpr int kTailThreads = 256;
constexpr int kMaxBlocks = 2048;                // V <= 2^18 at 128 rows per block
constexpr int kMaxWaves = 4 * kMaxBlocks;
constexpr int kSampleMaxK = 32;
constexpr int kBlockKeysPerThread = kMaxBlocks / kTailThreads;

struct TailArgs {
    uint32_t* gen;              // [kMaxBlocks] generation words; zero-filled once
    uint64_t* block_keys;       // [M_T][kMaxBlocks] tagged block maxima
    uint64_t* wave_keys;        // [M_T][kMaxWaves] tagged wave maxima (sampling)
    uint64_t* row_keys;         // [M_T][V] tagged row keys (sampling); null: greedy
    int32_t* ids;               // [M] chosen tokens; -1 when a poll gave up
    const float* u;             // [M] uniforms in [0, 1) (sampling)
    float temperature, top_p;
    int top_k;                  // 2..32 (sampling)
    int n_row_waves;            // waves that hold rows: ceil(V / rows_per_wave)
};
constexpr int kRowKeysPerThread = kSampleMaxK * kEpilogueRowsPerWave / kTailThreads;
constexpr int kSpinLimit = 1 << 16;             // polls of one word (milliseconds) before giving up
constexpr uint64_t kTagMask = 0xFFFull << kRowBits;

__device__ __forceinline__ uint64_t tag_bits(uint32_t count) {
    return (uint64_t)((count & 0x7FFu) | 0x800u) << kRowBits;
}

__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls the word at p until it carries `tag`; sets `stale` (and returns the
// last value read) when that takes more than kSpinLimit polls.
__device__ __forceinline__ uint64_t poll_current(const uint64_t* p, uint64_t tag, bool& stale) {
    uint64_t v = load_agent(p);
    for (int i = 0; (v & kTagMask) != tag && i < kSpinLimit; ++i) {
        __builtin_amdgcn_s_sleep(2);
        v = load_agent(p);
    }
    stale |= (v & kTagMask) != tag;
    return v;
}

// key[j] = run[j] for j < n_valid, else 0: the loads of a run are issued
// together (all J are in bounds); the words without this launch's tag are
// loaded again, together, until they have it (or sets `stale` after
// kSpinLimit rounds).
template <int J>
__device__ __forceinline__ void load_run(uint64_t (&key)[J], const uint64_t* run, int n_valid, uint64_t tag,
                                         bool& stale) {
    static_assert(J <= 32, "pending mask");
#pragma unroll
    for (int j = 0; j < J; ++j) key[j] = load_agent(run + j);
    uint32_t pending = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        if (j >= n_valid) key[j] = 0;
        else if ((key[j] & kTagMask) != tag) pending |= 1u << j;
    }
    for (int i = 0; pending != 0 && i < kSpinLimit; ++i) {
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (pending & (1u << j)) key[j] = load_agent(run + j);
#pragma unroll
        for (int j = 0; j < J; ++j)
            if ((pending & (1u << j)) && (key[j] & kTagMask) == tag) pending &= ~(1u << j);
    }
    stale |= pending != 0;
}

// key[j] = the word at addr(j) when valid(j), else 0 (scattered words).
template <int J, class Addr, class Valid>
__device__ __forceinline__ void load_keys(uint64_t (&key)[J], Addr addr, Valid valid, uint64_t tag, bool& stale) {
#pragma unroll
    for (int j = 0; j < J; ++j) key[j] = load_agent(addr(j));
#pragma unroll
    for (int j = 0; j < J; ++j) {
        if (!valid(j))
            key[j] = 0;
        else if ((key[j] & kTagMask) != tag)
            key[j] = poll_current(addr(j), tag, stale);
    }
}

// The k largest of the block's nonzero keys (distinct), by an 8-bit radix
// select over LDS histograms (two, used in turn), most significant digit
// first, that stops once the bin holding the k-th largest key holds exactly
// the keys still wanted.  Afterwards the k largest are the nonzero keys with
// (key >> S.shift) >= S.prefix -- all of them when there are at most k.
struct SelectScratch {
    uint32_t hist[2][256];
    uint64_t prefix;
    int rank;
    int shift;                                   // kOpen until settled
    int count;
};
constexpr int kOpen = 64;
static_assert(kTailThreads == 256, "one histogram bin per thread");

template <int J>
__device__ __forceinline__ void block_top_k(const uint64_t (&key)[J], int k, SelectScratch& S) {
    const int tid = threadIdx.x, lane = lane_id();
    if (tid == 0) {
        S.prefix = 0;
        S.rank = k;
        S.shift = kOpen;
    }
    S.hist[0][tid] = 0u;
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
        if (S.shift != kOpen) break;             // uniform: read after a barrier by every thread
        const int shift = 56 - 8 * pass, buf = pass & 1;
        const uint64_t pre = S.prefix;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint64_t kv = key[j];
            if (kv != 0 && (pass == 0 || (kv >> (shift + 8)) == pre))
                atomicAdd(&S.hist[buf][(uint32_t)(kv >> shift) & 255u], 1u);
        }
        S.hist[buf ^ 1][tid] = 0u;               // the next pass's histogram, read last a pass ago
        __syncthreads();
        if (tid < kWave) {
            // lane l holds bins 255 - 4l - j, j < 4 (largest digits first)
            uint32_t c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = S.hist[buf][255 - 4 * lane - j];
            const uint32_t mine = c[0] + c[1] + c[2] + c[3];
            uint32_t incl = mine;                // inclusive scan over the lanes
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            const uint32_t total = __shfl(incl, kWave - 1);
            uint32_t before = incl - mine;
            const uint32_t rank = (uint32_t)S.rank;
            if (pass == 0 && total <= rank) {
                if (lane == 0) {                 // at most k keys: all of them
                    S.prefix = 0;
                    S.shift = 63;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (before < rank && before + c[j] >= rank) {
                        S.prefix = (pre << 8) | (uint64_t)(255 - 4 * lane - j);
                        S.rank = (int)(rank - before);
                        if (before + c[j] == rank) S.shift = shift;
                    }
                    before += c[j];
                }
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ bool selected(const SelectScratch& S, uint64_t kv) {
    return kv != 0 && (kv >> S.shift) >= S.prefix;
}

// The token of a wave's row of sorted candidates (lane r < k holds the key of
// the r-th largest logit): softmax of logit / T over the k, the shortest
// prefix whose cumulative share reaches top_p, and the first entry of that
// prefix whose cumulative share of it exceeds u.
__device__ __forceinline__ int32_t sample_from_sorted(uint64_t key, int k, float temperature, float top_p, float u) {
    const int lane = lane_id();
    const bool on = lane < k;
    const float z = order_to_float((uint32_t)(key >> 32));
    const float z0 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(z)));
    const float e = on ? expf((z - z0) / temperature) : 0.f;
    float cum = e;                                          // inclusive scan over the lanes
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float o = __shfl_up(cum, off);
        if (lane >= off) cum += o;
    }
    const float total = __shfl(cum, k - 1);
    const int n_keep = min(k, __popcll(__ballot(on && cum < top_p * total)) + 1);
    const float kept = __shfl(cum, n_keep - 1);
    const int j = min(n_keep - 1, __popcll(__ballot(lane < n_keep && cum <= u * kept)));
    return __shfl(key_row(key), j);
}

constexpr int kCandMax = kSampleMaxK * kBlockKeysPerThread;  // candidates from top_k threads' runs
static_assert(kCandMax >= kTailThreads, "one candidate per thread fits");

struct TailScratch {
    SelectScratch S;
    uint64_t cand[kCandMax];                     // candidate keys
    uint64_t sel[kSampleMaxK];                   // the top_k keys, largest first
    uint32_t wave[kSampleMaxK];                  // selected waves
    uint64_t best[kTailThreads / kWave];
};

// Appends this thread's keys that pass `take` to L.cand (one LDS atomic per
// wave); the count ends in S.count, which must be zero before.
template <int J, class Take>
__device__ __forceinline__ void compact(const uint64_t (&key)[J], Take take, TailScratch& L) {
    const int lane = lane_id();
    int mine = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) mine += take(key[j]) ? 1 : 0;
    int incl = mine;                             // inclusive scan over the lanes
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    int base = 0;
    if (lane == kWave - 1 && incl > 0) base = atomicAdd(&L.S.count, incl);
    int at = __shfl(base, kWave - 1) + incl - mine;
#pragma unroll
    for (int j = 0; j < J; ++j)
        if (take(key[j])) {
            if (at < kCandMax) L.cand[at] = key[j];
            ++at;
        }
}

// The min(k, c) largest of the c candidates -- the nonzero keys that pass
// `take` (distinct) -- into L.sel, largest first; returns min(k, c).  Up to
// kCandMax candidates are ranked by counting (each against all, 8 LDS reads
// in flight); more fall back to a radix select over all nonzero keys first.
template <int J, class Take>
__device__ __forceinline__ int top_k_among(const uint64_t (&key)[J], int k, Take take, TailScratch& L) {
    const int tid = threadIdx.x;
    SelectScratch& S = L.S;
    if (tid == 0) S.count = 0;
    __syncthreads();
    compact(key, take, L);
    __syncthreads();
    int c = S.count;
    if (c > kCandMax) {
        block_top_k(key, k, S);                  // every thread read S.count before its barriers
        if (tid == 0) S.count = 0;
        __syncthreads();
        compact(key, [&](uint64_t kv) { return selected(S, kv); }, L);
        __syncthreads();
        c = min(S.count, k);
    }
    if (tid < c) {
        const uint64_t my = L.cand[tid];
        int r = 0;
        for (int i0 = 0; i0 < c; i0 += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint64_t o = L.cand[min(i0 + u, c - 1)];
                r += (i0 + u < c && o > my) ? 1 : 0;
            }
        }
        if (r < k) L.sel[r] = my;
    }
    __syncthreads();
    return min(c, k);
}

// Greedy token m: the largest block maximum.
__device__ __forceinline__ void greedy_token(const TailArgs& ta, int m, uint64_t tag, TailScratch& L) {
    const int tid = threadIdx.x, n_blocks = gridDim.x;
    bool stale = false;
    uint64_t bk[kBlockKeysPerThread];
    load_run(bk, ta.block_keys + (size_t)m * kMaxBlocks + tid * kBlockKeysPerThread,
             n_blocks - tid * kBlockKeysPerThread, tag, stale);
    uint64_t b = 0;
#pragma unroll
    for (int j = 0; j < kBlockKeysPerThread; ++j) b = bk[j] > b ? bk[j] : b;
    b = wave_max_u64(b);
    if (lane_id() == 0) L.best[tid >> 6] = b;
    const int bad = __syncthreads_or(stale);
    if (tid == 0) {
        uint64_t t = 0;
        for (int i = 0; i < kTailThreads / kWave; ++i) t = L.best[i] > t ? L.best[i] : t;
        ta.ids[m] = bad ? -1 : key_row(t);
    }
}

// Sampled token m (top_k >= 2).  atag: tag of the block keys; stag: of the
// wave and row keys.  Each step after the first takes as candidates the keys
// at or above the previous step's k-th largest (when it found k): the k-th
// largest row is at least the k-th largest wave maximum, which is at least
// the k-th largest block maximum, as each of those waves or blocks holds a
// row that large.
__device__ __forceinline__ void sample_token(const TailArgs& ta, int m, uint64_t atag, uint64_t stag, int V,
                                             int rows_per_wave, TailScratch& L) {
    const int tid = threadIdx.x, n_blocks = gridDim.x, k = ta.top_k;
    bool stale = false;
    // A1. the top_k blocks by maximum: the threads holding the top_k per-thread
    // maxima hold them, and only keys in those maxima's radix bins qualify
    int nb;
    {
        uint64_t bk[kBlockKeysPerThread];
        load_run(bk, ta.block_keys + (size_t)m * kMaxBlocks + tid * kBlockKeysPerThread,
                 n_blocks - tid * kBlockKeysPerThread, atag, stale);
        uint64_t tm[1] = {0};
#pragma unroll
        for (int j = 0; j < kBlockKeysPerThread; ++j) tm[0] = bk[j] > tm[0] ? bk[j] : tm[0];
        block_top_k(tm, k, L.S);
        nb = top_k_among(bk, k, [&](uint64_t kv) { return selected(L.S, kv); }, L);
    }
    uint64_t tau = nb == k ? L.sel[k - 1] : 1ull;
    if (tid < nb) L.wave[tid] = (uint32_t)key_row(L.sel[tid]) / (uint32_t)(4 * rows_per_wave);
    __syncthreads();
    // A2. the top_k waves among those blocks' waves (thread t < 4 nb: one wave)
    int nw;
    {
        const int wv = tid < 4 * nb ? (int)L.wave[tid >> 2] * 4 + (tid & 3) : 0;
        const bool ok = tid < 4 * nb && wv < ta.n_row_waves;
        uint64_t wk[1];
        load_keys(
            wk, [&](int) { return &ta.wave_keys[(size_t)m * kMaxWaves + (ok ? wv : 0)]; }, [&](int) { return ok; },
            stag, stale);
        nw = top_k_among(wk, k, [&](uint64_t kv) { return kv >= tau; }, L);   // its first barrier: L.wave read
    }
    tau = nw == k ? L.sel[k - 1] : 1ull;
    if (tid < nw) L.wave[tid] = (uint32_t)key_row(L.sel[tid]) / (uint32_t)rows_per_wave;
    __syncthreads();
    // B. the top_k rows among those waves' rows (row slot tid + 256 j), largest first
    uint64_t rk[kRowKeysPerThread];
    auto row_of = [&](int j) {
        const int r = tid + kTailThreads * j, slot = r / rows_per_wave;
        return slot < nw ? (int)L.wave[slot] * rows_per_wave + (r - slot * rows_per_wave) : V;
    };
    const uint64_t* keys = ta.row_keys + (size_t)m * V;
    load_keys(
        rk, [&](int j) { return &keys[min(row_of(j), V - 1)]; }, [&](int j) { return row_of(j) < V; }, stag,
        stale);
    top_k_among(rk, k, [&](uint64_t kv) { return kv >= tau; }, L);
    const int bad = __syncthreads_or(stale);
    // C. the draw, by wave 0
    if (tid < kWave) {
        const uint64_t sorted = tid < k ? L.sel[tid] : 0ull;
        const int32_t tok = sample_from_sorted(sorted, k, ta.temperature, ta.top_p, ta.u[m]);
        if (tid == 0) ta.ids[m] = bad ? -1 : tok;
    }
}

// Runs in every block once its waves are done (wave_best[w][m]: wave w's best
// key of token m, in LDS; gen: the block's generation word as read at its
// start).  Block gridDim.x - 1 - p, p < M_T, then computes tokens p, p +
// gridDim.x, ...; the other blocks return.
template <int M_T>
__device__ __forceinline__ void gemv_tail(const TailArgs& ta, const uint64_t (&wave_best)[4][MOEDEC_MAX_M], uint32_t gen,
                          int V, int rows_per_wave) {
    __shared__ TailScratch L;
    const int tid = threadIdx.x;
    const uint64_t atag = tag_bits(gen), stag = tag_bits(gen >> 16);
    __syncthreads();                                   // wave_best complete; every wave read gen
    if (tid < M_T) {
        uint64_t b = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) b = wave_best[i][tid] > b ? wave_best[i][tid] : b;
        __hip_atomic_store(&ta.block_keys[(size_t)tid * kMaxBlocks + blockIdx.x], b | atag, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t next = ((((gen >> 16) + (ta.row_keys ? 1u : 0u)) & 0xFFFFu) << 16) | ((gen + 1u) & 0xFFFFu);
    for (int i = blockIdx.x + gridDim.x * tid; i < kMaxBlocks; i += gridDim.x * kTailThreads)
        __hip_atomic_store(&ta.gen[i], next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int p = (int)gridDim.x - 1 - (int)blockIdx.x;
    if (p >= M_T) return;
    for (int m = p; m < M_T; m += gridDim.x) {
        if (!ta.row_keys)
            greedy_token(ta, m, atag, L);
        else
            sample_token(ta, m, atag, stag, V, rows_per_wave, L);
        __syncthreads();                               // L reused by the next token
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

// Waves per SIMD the FP8 GEMV asks the register allocator for: with an
// epilogue at up to 3 chunks per lane the kernel fits the 168 registers of
// three waves (without the hint the M = 4 variant takes one more and drops
// to two); M = 3, and the dynamic-activation variants (their quantised x
// takes more registers), would spill there and keep the default.
template <int M_T, int T, bool KEYS, bool ACT8>
constexpr int kFp8WavesPerSimd = (KEYS && T <= 3 && M_T != 3 && !ACT8) ? 3 : 1;

// FP8 GEMV.  T = 16-byte chunks per lane per row (ceil(H / 16 / 64)), R rows
// per wave step.  Each lane keeps its slice of x (every token) in registers
// and reuses it for every row the wave visits; the R x M_T row sums of a
// step are reduced together (store_row_sums).
// KEYS (the greedy or sampling epilogue; 32 rows per wave): the row sums go
// to LDS, the block then writes the logits (if any), derives the keys of its
// rows and wave groups (publishing them when sampling) and runs gemv_tail.
// ACT8 (dynamic FP8 activations): each block quantises every token row with
// the weights' rule (t = absmax / 448 over the whole row, a wave maximum;
// codes = E4M3 nearest-even of x / t), one wave per token, into LDS; the
// waves keep the E4M3 values as exact bf16 pairs in place of x and multiply
// each finished sum by t.  Every block forms the same codes, so no block
// depends on another.
template <int M_T, int T, int R, bool KEYS, bool ACT8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kFp8WavesPerSimd<M_T, T, KEYS, ACT8>)))
void gemv_fp8_kernel(const uint8_t* __restrict__ codes,
                                                       const float* __restrict__ rs, int V, int H,
                                                       const uint32_t* __restrict__ x,
                                                       float* __restrict__ logits,
                                                       int rows_per_wave, TailArgs ta) {
    const int lane = lane_id();
    uint32_t gen = 0;
    if constexpr (KEYS) gen = __hip_atomic_load(&ta.gen[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t stag = tag_bits(gen >> 16);          // tag of the wave and row keys
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
    float tok_scale[M_T];
    if constexpr (ACT8) {
        // wave m quantises token m (its slice of every token is already in
        // registers) into LDS; after one barrier every wave reads all tokens'
        // codes back as exact bf16 pairs
        __shared__ uint32_t s_xq[M_T][64 * T * 8];
        __shared__ float s_ts[M_T];
        const int wv = threadIdx.x >> 6;
#pragma unroll
        for (int m = 0; m < M_T; ++m) {
            if ((m & 3) != wv) continue;                        // wave-uniform
            uint32_t am = 0;
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j) am = max(am, max(xr[m][t][j] & 0x7FFFu, (xr[m][t][j] >> 16) & 0x7FFFu));
            const float a = bf16_to_f32(wave_max_u32(am));
            const float ts = (a == 0.f) ? 1.0f : a / 448.0f;
            const float ty = 1.0f / ts;
            const bool fast = ts >= 0x1p-90f && ts <= 0x1.fffffep127f;   // wave-uniform, as in quant_fp8_kernel
            if (lane == 0) s_ts[m] = ts;
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const uint32_t q = fast ? quant4<true>(xr[m][t][j], xr[m][t][j + 1], ts, ty)
                                            : quant4<false>(xr[m][t][j], xr[m][t][j + 1], ts, ty);
                    s_xq[m][(lane + 64 * t) * 8 + j] = __builtin_bit_cast(uint32_t, MOEDEC_FP8X2_BF16(q, false));
                    s_xq[m][(lane + 64 * t) * 8 + j + 1] = __builtin_bit_cast(uint32_t, MOEDEC_FP8X2_BF16(q, true));
                }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < M_T; ++m) {
            tok_scale[m] = s_ts[m];
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j) xr[m][t][j] = s_xq[m][(lane + 64 * t) * 8 + j];
        }
    }
    const int v0 = gw * rows_per_wave;
    const int v1 = min(V, v0 + rows_per_wave);
    __shared__ float s_rows[KEYS ? M_T : 1][kBlockRows];
    const int wrow = (threadIdx.x >> 6) * rows_per_wave;   // the wave's first row within the block
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
        if constexpr (ACT8) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M_T; ++m) acc[r][m] *= tok_scale[m];
        }
        store_row_sums<R, M_T, KEYS>(acc, v, v1, V, logits, [&](int row) { return rs[row]; }, &s_rows[0][0],
                                     wrow + (v - v0));
    }
    if constexpr (KEYS) {
        // The block's rows from LDS: logits and (sampling) row keys in
        // coalesced stores, the maximum of every 32-row wave group (published
        // when sampling), then the tail.  Entry e = m * kBlockRows + i: lanes
        // 0..31 and 32..63 of a wave hold one wave group each.
        __shared__ uint64_t s_wbest[4][MOEDEC_MAX_M];
        const int tid = threadIdx.x;
        __syncthreads();                                   // every wave's row sums are in s_rows
        const int base = blockIdx.x * kBlockRows;
#pragma unroll
        for (int e0 = 0; e0 < M_T * kBlockRows; e0 += 256) {
            const int e = e0 + tid;
            if (e < M_T * kBlockRows) {                    // wave-uniform: kBlockRows is a multiple of 64
                const int m = e / kBlockRows, i = e % kBlockRows, row = base + i;
                const bool ok = row < V;
                const float val = s_rows[m][i];
                const uint64_t key = ok ? argmax_key(val, row) : 0ull;
                if (ok && logits) logits[(size_t)m * V + row] = val;
                if (ok && ta.row_keys)
                    __hip_atomic_store(&ta.row_keys[(size_t)m * V + row], key | stag, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t wk = wave_max_u64<32>(key);
                if ((lane & 31) == 0) {
                    const int g = i / kEpilogueRowsPerWave, wv = blockIdx.x * 4 + g;
                    s_wbest[g][m] = wk;
                    if (ta.row_keys && wv < ta.n_row_waves)
                        __hip_atomic_store(&ta.wave_keys[(size_t)m * kMaxWaves + wv], wk | stag, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        gemv_tail<M_T>(ta, s_wbest, gen, V, rows_per_wave);
    }
}

// The rows of the bf16 GEMV for this wave: rows_per_wave rows from row
// wave * rows_per_wave, R per step, against the lane's x chunks xr.
template <int M_T, int T, int R>
__device__ __forceinline__ void gemv_bf16_rows(const uint16_t* __restrict__ wt, int V, int H,
                                               const uint32_t (&xr)[M_T][T][4], float* __restrict__ logits,
                                               int rows_per_wave) {
    const int lane = lane_id();
    const int n_ch = H / 8;
    const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
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

template <int M_T, int T, int R>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(const uint16_t* __restrict__ wt, int V,
                                                        int H, const uint32_t* __restrict__ x,
                                                        float* __restrict__ logits,
                                                        int rows_per_wave) {
    const int lane = lane_id();
    const int n_ch = H / 8;
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
    gemv_bf16_rows<M_T, T, R>(wt, V, H, xr, logits, rows_per_wave);
}

// Router logits from the residual stream: x = bf16(RMSNorm(r)) with unit gain,
// formed in every block from the float32 r [M_T][H] with the factors of
// rmsnorm_factors (the fused layer's order, so this x is the layer's x bit for
// bit), then the rows of gemv_bf16_rows.  H % 8 == 0, H <= 4096.
template <int M_T, int T, int R>
__global__ __launch_bounds__(256) void norm_gemv_bf16_kernel(const uint16_t* __restrict__ wt, int V,
                                                             int H, const float* __restrict__ r,
                                                             float eps, float* __restrict__ logits,
                                                             int rows_per_wave) {
    const int lane = lane_id();
    const int n_ch = H / 8;
    constexpr int kPieces = 4 * M_T;                   // 16-byte pieces per thread: H / 4 <= 4 * 256
    const int per_tok = H / 4, n_pieces = M_T * per_tok;
    const u32x4* r4 = reinterpret_cast<const u32x4*>(r);
    u32x4 rv[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) rv[i] = r4[min((int)threadIdx.x + 256 * i, n_pieces - 1)];
    float inv[M_T];
    rmsnorm_factors<M_T>(rv, n_pieces, per_tok, H, eps, inv);
    // this lane's chunks of x: chunk ch = 8 elements, from r's pieces 2ch and 2ch + 1
    uint32_t xr[M_T][T][4];
#pragma unroll
    for (int m = 0; m < M_T; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int ch = lane + 64 * t;
            const int cc = min(ch, n_ch - 1);
            const u32x4 lo = r4[m * per_tok + 2 * cc], hi = r4[m * per_tok + 2 * cc + 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t a = j < 2 ? lo[2 * j] : hi[2 * j - 4];
                const uint32_t b = j < 2 ? lo[2 * j + 1] : hi[2 * j - 3];
                const uint32_t pair = (uint32_t)f32_to_bf16_rne(__uint_as_float(a) * inv[m]) |
                                      ((uint32_t)f32_to_bf16_rne(__uint_as_float(b) * inv[m]) << 16);
                xr[m][t][j] = (ch < n_ch) ? pair : 0u;
            }
        }
    gemv_bf16_rows<M_T, T, R>(wt, V, H, xr, logits, rows_per_wave);
}

// bf16 GEMV: 16 rows per wave, 4 per step, for a vocabulary-sized matrix; a
// short one (a router's 512 rows) takes one row per wave so that its few
// megabytes spread over as many waves as it has rows (latency-bound).
constexpr int kRowsPerWave = 16;
constexpr int kShortRows = 16384;

template <int M_T, int T>
void launch_norm_bf16_t(const uint16_t* w, int V, int H, const float* r, float eps, float* logits, hipStream_t s) {
    const dim3 grid((V + 3) / 4), blk(256);                // one row per wave, as for a short matrix
    hipLaunchKernelGGL((norm_gemv_bf16_kernel<M_T, T, 1>), grid, blk, 0, s, w, V, H, r, eps, logits, 1);
}

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
static_assert(kFp8RowsPerWave == kEpilogueRowsPerWave, "the epilogue's LDS rows assume 32 rows per wave");

int fp8_waves(int V) {                              // waves launched (4 per block)
    const int waves = (V + kFp8RowsPerWave - 1) / kFp8RowsPerWave;
    return 4 * ((waves + 3) / 4);
}

// Workspace of the epilogue: the generation words [kMaxBlocks], the block
// keys [M][kMaxBlocks], the wave keys [M][kMaxWaves], then the row keys
// [M][V].
constexpr size_t kGenBytes = kMaxBlocks * sizeof(uint32_t);

template <int M_T, int T, bool ACT8>
hipError_t gemv_fp8_t(const uint8_t* codes, const float* rs, int V, int H, const uint32_t* x,
                      float* logits, const Fp8Epilogue* ep, hipStream_t s) {
    const int n_waves = fp8_waves(V);
    const dim3 grid(n_waves / 4), blk(256);
    if (!ep) {
        hipLaunchKernelGGL((gemv_fp8_kernel<M_T, T, kFp8Rows, false, ACT8>), grid, blk, 0, s, codes, rs, V, H, x,
                           logits, kFp8RowsPerWave, TailArgs{});
        return hipGetLastError();
    }
    uint8_t* ws = static_cast<uint8_t*>(ep->workspace);
    const bool sample = ep->u != nullptr && ep->top_k > 1;     // top_k = 1 is the greedy token
    TailArgs ta;
    const size_t block_bytes = (size_t)kMaxBlocks * M_T * 8, wave_bytes = (size_t)kMaxWaves * M_T * 8;
    ta.gen = reinterpret_cast<uint32_t*>(ws);
    ta.block_keys = reinterpret_cast<uint64_t*>(ws + kGenBytes);
    ta.wave_keys = reinterpret_cast<uint64_t*>(ws + kGenBytes + block_bytes);
    ta.row_keys = sample ? reinterpret_cast<uint64_t*>(ws + kGenBytes + block_bytes + wave_bytes) : nullptr;
    ta.ids = ep->ids;
    ta.u = ep->u;
    ta.temperature = ep->temperature;
    ta.top_p = ep->top_p;
    ta.top_k = ep->top_k;
    ta.n_row_waves = (V + kFp8RowsPerWave - 1) / kFp8RowsPerWave;
    hipLaunchKernelGGL((gemv_fp8_kernel<M_T, T, kFp8Rows, true, ACT8>), grid, blk, 0, s, codes, rs, V, H, x,
                       logits, kFp8RowsPerWave, ta);
    return hipGetLastError();
}

template <int M_T, bool ACT8>
hipError_t gemv_fp8_m(const uint8_t* codes, const float* rs, int V, int H, const uint32_t* x,
                      float* logits, const Fp8Epilogue* ep, hipStream_t s) {
    switch ((H / 16 + 63) / 64) {
        case 1: return gemv_fp8_t<M_T, 1, ACT8>(codes, rs, V, H, x, logits, ep, s);
        case 2: return gemv_fp8_t<M_T, 2, ACT8>(codes, rs, V, H, x, logits, ep, s);
        case 3: return gemv_fp8_t<M_T, 3, ACT8>(codes, rs, V, H, x, logits, ep, s);
        default: return gemv_fp8_t<M_T, 4, ACT8>(codes, rs, V, H, x, logits, ep, s);
    }
}

template <bool ACT8>
hipError_t gemv_fp8_any(const uint8_t* codes, const float* rs, int V, int H, const uint32_t* x, int M,
                        float* logits, const Fp8Epilogue* ep, hipStream_t s) {
    switch (M) {
        case 1: return gemv_fp8_m<1, ACT8>(codes, rs, V, H, x, logits, ep, s);
        case 2: return gemv_fp8_m<2, ACT8>(codes, rs, V, H, x, logits, ep, s);
        case 3: return gemv_fp8_m<3, ACT8>(codes, rs, V, H, x, logits, ep, s);
        default: return gemv_fp8_m<4, ACT8>(codes, rs, V, H, x, logits, ep, s);
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

template <int M_T>
hipError_t norm_gemv_bf16_m(const uint16_t* w, int V, int H, const float* r, float eps, float* logits,
                            hipStream_t s) {
    switch ((H / 8 + 63) / 64) {
        case 1: launch_norm_bf16_t<M_T, 1>(w, V, H, r, eps, logits, s); break;
        case 2: launch_norm_bf16_t<M_T, 2>(w, V, H, r, eps, logits, s); break;
        case 3: launch_norm_bf16_t<M_T, 3>(w, V, H, r, eps, logits, s); break;
        case 4: launch_norm_bf16_t<M_T, 4>(w, V, H, r, eps, logits, s); break;
        case 5: launch_norm_bf16_t<M_T, 5>(w, V, H, r, eps, logits, s); break;
        case 6: launch_norm_bf16_t<M_T, 6>(w, V, H, r, eps, logits, s); break;
        case 7: launch_norm_bf16_t<M_T, 7>(w, V, H, r, eps, logits, s); break;
        default: launch_norm_bf16_t<M_T, 8>(w, V, H, r, eps, logits, s); break;
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
                           const Fp8Epilogue* ep, bool act8) {
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    return act8 ? gemv_fp8_any<true>(codes, rs, V, H, x32, M, logits, ep, s)
                : gemv_fp8_any<false>(codes, rs, V, H, x32, M, logits, ep, s);
}

size_t lmhead_epilogue_bytes(int V, int M) {
    return kGenBytes + ((size_t)kMaxBlocks + kMaxWaves + (size_t)V) * M * sizeof(uint64_t);
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

hipError_t launch_norm_router_bf16(const uint16_t* w, int E, int H, const float* r, float eps, int M,
                                   float* logits, hipStream_t s) {
    switch (M) {
        case 1: return norm_gemv_bf16_m<1>(w, E, H, r, eps, logits, s);
        case 2: return norm_gemv_bf16_m<2>(w, E, H, r, eps, logits, s);
        case 3: return norm_gemv_bf16_m<3>(w, E, H, r, eps, logits, s);
        default: return norm_gemv_bf16_m<4>(w, E, H, r, eps, logits, s);
    }
}

}  // namespace moedec
