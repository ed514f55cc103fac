// Device-side routing shared by the route kernel and the fused MoE-layer kernel:
// exact top-k of one token's logits by one wave, softmax weights over the k
// chosen, and the expert-grouped slot list of up to four tokens.
//
// Each token goes to k of E routed experts (8 of 512 in the model the pages
// measure: knowledge card at ai.cheesepanini.fun, background; news article
// yoususu.cn/post/959, "where the speed comes from"); a 4-token verify window
// touches up to 32 experts (card, method point #3).
//
// Selection is exact: logits are compared through an order-preserving integer
// image of the float (+0.0 and -0.0 made equal), and among equal logits the
// smaller expert index wins.  A choice is returned as a 64-bit key (image <<
// 32 | ~index), so "larger key" means "larger logit, then smaller index".
#pragma once

#include "device_common.h"
#include "moedec.h"

namespace moedec {

__device__ __forceinline__ int key_to_index(uint64_t key) { return (int)(~(uint32_t)key); }

// LDS words (64-bit) wave_topk needs per wave: 64 survivors + one scratch word.
constexpr int kTopkBufWords = 72;

// Order-preserving integer image of a float32: 2^31 + |f| for f >= 0 and
// 2^31 - |f| for f < 0, with |f| the magnitude bits.  a > b as floats <=>
// ord(a) > ord(b); +0.0 and -0.0 map to the same image and every float maps
// above 0 (the value given to masked entries).  Branch-free (no compare).
__device__ __forceinline__ uint32_t float_order(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t mag = u & 0x7FFFFFFFu;
    const uint32_t neg = (uint32_t)((int32_t)u >> 31);         // all ones for a negative sign
    return 0x80000000u + ((mag ^ neg) - neg);
}

__device__ __forceinline__ float order_to_float(uint32_t ord) {
    const uint32_t d = ord - 0x80000000u;                       // signed magnitude, two's complement
    const uint32_t neg = (uint32_t)((int32_t)d >> 31);
    return __uint_as_float(((d ^ neg) - neg) | (neg & 0x80000000u));
}

// Top-k of token `row` (E logits) by the calling wave.  Lane r < k returns the
// r-th choice in selection order as a key (ord(logit) << 32 | ~index) and its
// weight exp(l_r - l_0) / sum_j exp(l_j - l_0) (the softmax over all E
// renormalised over the k chosen equals the softmax over the k chosen
// logits).  Lanes >= k return key 0, weight 0.  KPL = keys per lane,
// E <= 64 * KPL, 1 <= k <= min(E, 32).  `buf` is kTopkBufWords words of LDS
// owned by the calling wave (its contents are overwritten).
//
// Method (exact).  Any threshold T that at least k of the values reach admits
// every one of the top k.  T is found from the 64 per-lane maxima by a radix
// search over the top 16 bits of their integer image: the largest 16-bit
// prefix that at least k lane maxima reach (each such lane holds a value >= T).
// The values >= T ("survivors", typically a dozen) are compacted into LDS and
// each is ranked against all of them by (logit desc, index asc); rank r < k is
// the r-th choice.  If ties leave more than 64 survivors, the
// choices are taken one at a time instead: the largest remaining value (32-bit
// wave maximum), then the smallest index holding it (32-bit wave minimum).
// The logits of one token as the top-k reads them: lane l holds entries
// l + 64 t.  The loads are unconditional (clamped index) so that they are all
// in flight at once; lanes past E are masked by wave_topk_of.
template <int KPL>
__device__ __forceinline__ void topk_load(const float* __restrict__ row, int E, float (&v)[KPL]) {
    const int lane = lane_id();
#pragma unroll
    for (int t = 0; t < KPL; ++t) v[t] = row[min(lane + kWave * t, E - 1)];
}

template <int KPL>
__device__ __forceinline__ uint64_t wave_topk_of(const float (&v)[KPL], int E, int k, float& weight,
                                                 uint64_t* buf);

template <int KPL>
__device__ __forceinline__ uint64_t wave_topk(const float* __restrict__ row, int E, int k, float& weight,
                                              uint64_t* buf) {
    float v[KPL];
    topk_load<KPL>(row, E, v);
    return wave_topk_of<KPL>(v, E, k, weight, buf);
}

// wave_topk on logits already loaded by topk_load.
template <int KPL>
__device__ __forceinline__ uint64_t wave_topk_of(const float (&v)[KPL], int E, int k, float& weight,
                                                 uint64_t* buf) {
    // buf holds the survivors, then the k choices; one wave's LDS operations
    // complete in issue order, so the reads of one phase are done before the
    // writes of the next land
    const int lane = lane_id();
    uint32_t o[KPL];
#pragma unroll
    for (int t = 0; t < KPL; ++t) o[t] = (lane + kWave * t < E) ? float_order(v[t]) : 0u;

    uint32_t lmax = o[0];
#pragma unroll
    for (int t = 1; t < KPL; ++t) lmax = lmax > o[t] ? lmax : o[t];
    uint32_t T = 0u;
#pragma unroll
    for (int b = 31; b >= 16; --b) {
        const uint32_t c = T | (1u << b);
        if (__popcll(__ballot(lmax >= c)) >= k) T = c;
    }

    // compact the survivors (value >= T) into LDS, lane by lane: per-lane
    // counts, lane offsets by a ballot prefix sum (one ballot per count bit),
    // then every lane writes all its values -- survivors to their place,
    // the rest (and survivors past 64) to the scratch word buf[64]
    static_assert(KPL < 32, "per-lane survivor counts take five bits");
    int cnt = 0;
#pragma unroll
    for (int t = 0; t < KPL; ++t) cnt += (o[t] >= T) ? 1 : 0;
    int pos = 0, base = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        const uint64_t bal = __ballot((cnt >> b) & 1);
        pos += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)) << b;
        base += __popcll(bal) << b;
    }
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
        const bool keep = o[t] >= T;
        buf[(keep && pos < kWave) ? pos : kWave] = ((uint64_t)o[t] << 32) | (uint64_t)(~(uint32_t)(lane + kWave * t));
        pos += keep ? 1 : 0;
    }
    __builtin_amdgcn_wave_barrier();

    uint64_t mine = 0ull;
    if (base <= 16) {
        // the common case: survivor i = lane & 15 is compared with survivors
        // 4q..4q+3, q = lane >> 4 (one batch of LDS reads), and the four
        // partial counts of survivor i (lanes i, i + 16, i + 32, i + 48) are
        // summed by two lane swaps
        const int i = lane & 15, q4 = 4 * (lane >> 4);
        const uint64_t my = buf[min(i, base - 1)];
        uint64_t other[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) other[j] = buf[min(q4 + j, base - 1)];
        int r = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) r += (q4 + j < base && other[j] > my) ? 1 : 0;
        u32x2 p = swap16((uint32_t)r);
        r = (int)(p[0] + p[1]);
        p = swap32((uint32_t)r);
        r = (int)(p[0] + p[1]);
        __builtin_amdgcn_wave_barrier();
        if (lane < 16 && i < base && r < k) buf[r] = my;
        __builtin_amdgcn_wave_barrier();
        mine = (lane < k) ? buf[min(lane, k - 1)] : 0ull;
    } else if (base <= kWave) {
        // rank each survivor against all of them (broadcast one per step); rank
        // r < k is choice r
        const uint64_t my = buf[min(lane, base - 1)];
        const uint32_t my_hi = (uint32_t)(my >> 32), my_lo = (uint32_t)my;
        int r = 0;
        for (int j = 0; j < base; ++j) {
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)my_hi, j);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)my_lo, j);
            r += (hi > my_hi || (hi == my_hi && lo > my_lo)) ? 1 : 0;
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < base && r < k) buf[r] = my;
        __builtin_amdgcn_wave_barrier();
        mine = (lane < k) ? buf[min(lane, k - 1)] : 0ull;
    } else {
        uint32_t mine_o = 0u, mine_i = 0xFFFFFFFFu;
        for (int r = 0; r < k; ++r) {
            uint32_t lm[KPL];
#pragma unroll
            for (int t = 0; t < KPL; ++t) lm[t] = o[t];
#pragma unroll
            for (int w = 1; w < KPL; w <<= 1)
#pragma unroll
                for (int t = 0; t + w < KPL; t += 2 * w) lm[t] = lm[t] > lm[t + w] ? lm[t] : lm[t + w];
            const uint32_t g = wave_max_u32(lm[0]);
            uint32_t c = 0xFFFFFFFFu;                       // this lane's smallest index holding g
#pragma unroll
            for (int t = KPL - 1; t >= 0; --t) c = (o[t] == g) ? (uint32_t)(lane + kWave * t) : c;
            const uint32_t gi = wave_min_u32(c);
#pragma unroll
            for (int t = 0; t < KPL; ++t) o[t] = ((uint32_t)(lane + kWave * t) == gi) ? 0u : o[t];
            if (lane == r) {
                mine_o = g;
                mine_i = gi;
            }
        }
        mine = (lane < k) ? (((uint64_t)mine_o << 32) | (uint64_t)(~mine_i)) : 0ull;
    }
    const uint32_t first_o = (uint32_t)(__builtin_amdgcn_readfirstlane((int)(uint32_t)(mine >> 32)));
    const float top = order_to_float(first_o);
    const float ex = (lane < k) ? expf(order_to_float((uint32_t)(mine >> 32)) - top) : 0.f;
    const float sum = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(wave_sum_f32(ex))));
    weight = (lane < k) ? ex / sum : 0.f;
    return mine;
}

// One token: the k chosen experts sorted by ascending id.  Lane r < k holds
// (id_r, w_r) in selection order; returns the rank of id_r among the k ids
// (its slot among the routed experts).  Ids are distinct.
__device__ __forceinline__ int wave_rank_ids(int id, int k) {
    int rank = 0;
    for (int j = 0; j < k; ++j) {
        const int other = __builtin_amdgcn_readlane(id, j);
        rank += (other < id) ? 1 : 0;
    }
    return rank;
}

// Group M tokens' selections by expert.  Inputs (LDS): r_id[m][r], r_w[m][r]
// for m < M, r < k.  Outputs (LDS): n_routed distinct experts in ascending id
// order with, for each, its token mask and per-token weight (0 where the
// token does not use it).  `bits` (MOEDEC_MAX_E / 32 words) and `pre`
// (MOEDEC_MAX_E / 32 + 1 ints) are scratch.  Called by the whole block;
// returns n_routed to every thread.  Entries [n_routed, MOEDEC_MAX_SLOTS) of
// the outputs are zero.
__device__ __forceinline__ int block_group_by_expert(
    const int32_t (*r_id)[MOEDEC_MAX_K], const float (*r_w)[MOEDEC_MAX_K], int M, int k,
    uint32_t* bits, int* pre, int32_t* out_expert, uint32_t* out_mask,
    float (*out_weight)[MOEDEC_MAX_M]) {
    const int tid = threadIdx.x;
    const int n = blockDim.x;
    for (int i = tid; i < MOEDEC_MAX_SLOTS; i += n) {
        out_expert[i] = 0;
        out_mask[i] = 0u;
#pragma unroll
        for (int j = 0; j < MOEDEC_MAX_M; ++j) out_weight[i][j] = 0.f;
    }
    for (int i = tid; i < MOEDEC_MAX_E / 32; i += n) bits[i] = 0u;
    __syncthreads();
    const int n_entries = M * k;
    for (int t = tid; t < n_entries; t += n) {
        const int id = r_id[t / k][t % k];
        atomicOr(&bits[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    if (tid < kWave) {
        // exclusive prefix of popcounts (0..32) over the 32 bitmap words, bit
        // by bit: one ballot per bit of the count
        const int c = (tid < MOEDEC_MAX_E / 32) ? __popc(bits[tid]) : 0;
        int excl = 0, total = 0;
#pragma unroll
        for (int b = 0; b < 6; ++b) {
            const uint64_t bal = __ballot((c >> b) & 1);
            excl += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)) << b;
            total += __popcll(bal) << b;
        }
        if (tid < MOEDEC_MAX_E / 32) pre[tid] = excl;
        if (tid == 0) pre[MOEDEC_MAX_E / 32] = total;
    }
    __syncthreads();
    for (int t = tid; t < n_entries; t += n) {
        const int tm = t / k, r = t % k;
        const int id = r_id[tm][r];
        const int word = id >> 5;
        const int slot = pre[word] + __popc(bits[word] & ((1u << (id & 31)) - 1u));
        out_expert[slot] = id;
        atomicOr(&out_mask[slot], 1u << tm);
        out_weight[slot][tm] = r_w[tm][r];
    }
    __syncthreads();
    return pre[MOEDEC_MAX_E / 32];
}

}  // namespace moedec
