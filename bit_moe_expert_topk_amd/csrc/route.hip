// Top-k expert routing and the expert-grouped dispatch table.
//
// Each token goes to k of E routed experts plus the shared expert (8 of 512
// plus 1 in the model the pages measure: news article yoususu.cn/post/959,
// "where the speed comes from"; knowledge card at ai.cheesepanini.fun,
// background).  Verifying a 4-token window can touch up to 32 experts and
// that activation is what a verify costs (card, method point #3), so the
// table lists every active expert once together with the tokens it serves.
//
// Selection is exact: logits become 64-bit keys (order-preserving integer
// image of the float in the high word, inverted expert index in the low
// word), so "larger key" means "larger logit, then smaller index", and +0.0
// / -0.0 are made equal before keying.  One wave per token keeps E/64 keys
// per lane in registers and extracts the k largest by k wave-wide maxima.
#include "device_common.h"
#include "launch.h"

namespace moedec {

__device__ __forceinline__ uint64_t route_key(float f, int idx) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;                        // -0.0 -> +0.0
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(~(uint32_t)idx);
}

__device__ __forceinline__ float key_to_logit(uint64_t key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(u);
}

__device__ __forceinline__ int key_to_index(uint64_t key) { return (int)(~(uint32_t)key); }

template <int KEYS_PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int M,
                                                         int E, int k, int32_t* __restrict__ ids_out,
                                                         float* __restrict__ w_out,
                                                         moedec_dispatch* __restrict__ disp) {
    __shared__ int32_t s_id[MOEDEC_MAX_M][MOEDEC_MAX_K];
    __shared__ float s_w[MOEDEC_MAX_M][MOEDEC_MAX_K];
    __shared__ uint32_t s_bits[MOEDEC_MAX_E / 32];
    __shared__ int32_t s_pre[MOEDEC_MAX_E / 32 + 1];
    __shared__ int32_t s_exp[MOEDEC_MAX_SLOTS];
    __shared__ uint32_t s_mask[MOEDEC_MAX_SLOTS];
    __shared__ float s_wt[MOEDEC_MAX_SLOTS][MOEDEC_MAX_M];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int m = tid >> 6;  // one wave per token

    for (int i = tid; i < MOEDEC_MAX_SLOTS; i += blockDim.x) {
        s_exp[i] = 0;
        s_mask[i] = 0u;
#pragma unroll
        for (int j = 0; j < MOEDEC_MAX_M; ++j) s_wt[i][j] = 0.f;
    }
    if (tid < MOEDEC_MAX_E / 32) s_bits[tid] = 0u;

    if (m < M) {
        uint64_t key[KEYS_PER_LANE];
#pragma unroll
        for (int t = 0; t < KEYS_PER_LANE; ++t) {
            const int idx = lane + kWave * t;
            key[t] = (idx < E) ? route_key(logits[(size_t)m * E + idx], idx) : 0ull;
        }
        uint64_t mine = 0ull, first = 0ull;
        for (int r = 0; r < k; ++r) {
            uint64_t best = 0ull;
#pragma unroll
            for (int t = 0; t < KEYS_PER_LANE; ++t) best = key[t] > best ? key[t] : best;
            const uint64_t g = wave_max_u64(best);
#pragma unroll
            for (int t = 0; t < KEYS_PER_LANE; ++t)
                if (key[t] == g) key[t] = 0ull;
            if (lane == r) mine = g;
            if (r == 0) first = g;
        }
        // Softmax over the k chosen logits == full softmax renormalised over them.
        const float top = key_to_logit(first);
        const float ex = (lane < k) ? expf(key_to_logit(mine) - top) : 0.f;
        const float sum = wave_sum(ex);
        if (lane < k) {
            const float wv = ex / sum;
            const int id = key_to_index(mine);
            if (ids_out) ids_out[m * k + lane] = id;
            if (w_out) w_out[m * k + lane] = wv;
            s_id[m][lane] = id;
            s_w[m][lane] = wv;
        }
    }
    __syncthreads();
    if (disp == nullptr) return;

    const int n_entries = M * k;
    for (int t = tid; t < n_entries; t += blockDim.x) {
        const int id = s_id[t / k][t % k];
        atomicOr(&s_bits[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < MOEDEC_MAX_E / 32; ++i) {
            s_pre[i] = acc;
            acc += __popc(s_bits[i]);
        }
        s_pre[MOEDEC_MAX_E / 32] = acc;
    }
    __syncthreads();
    for (int t = tid; t < n_entries; t += blockDim.x) {
        const int tm = t / k, r = t % k;
        const int id = s_id[tm][r];
        const int word = id >> 5;
        const int slot = s_pre[word] + __popc(s_bits[word] & ((1u << (id & 31)) - 1u));
        s_exp[slot] = id;
        atomicOr(&s_mask[slot], 1u << tm);
        s_wt[slot][tm] = s_w[tm][r];
    }
    __syncthreads();
    const int n_routed = s_pre[MOEDEC_MAX_E / 32];
    if (tid == 0) {
        s_exp[n_routed] = E;                         // the shared expert serves every token
        s_mask[n_routed] = (1u << M) - 1u;
        for (int j = 0; j < M; ++j) s_wt[n_routed][j] = 1.f;
        disp->n_slots = n_routed + 1;
        disp->M = M;
    }
    __syncthreads();
    for (int i = tid; i < MOEDEC_MAX_SLOTS; i += blockDim.x) {
        disp->expert[i] = s_exp[i];
        disp->token_mask[i] = s_mask[i];
#pragma unroll
        for (int j = 0; j < MOEDEC_MAX_M; ++j) disp->weight[i][j] = s_wt[i][j];
    }
}

hipError_t launch_route_topk(const float* logits, int M, int E, int k, int32_t* ids, float* w,
                             moedec_dispatch* disp, hipStream_t s) {
    const dim3 grid(1), block(256);
    if (E <= 512)
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, M, E, k, ids, w, disp);
    else
        hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, M, E, k, ids, w, disp);
    return hipGetLastError();
}

}  // namespace moedec
