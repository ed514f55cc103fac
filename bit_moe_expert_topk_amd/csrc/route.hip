// Top-k expert routing and the expert-grouped dispatch table (one block).
//
// Each token goes to k of E routed experts plus the shared expert (8 of 512
// plus 1 in the model the pages measure: news article yoususu.cn/post/959,
// "where the speed comes from"; knowledge card at ai.cheesepanini.fun,
// background).  Verifying a 4-token window can touch up to 32 experts and
// that activation is what a verify costs (card, method point #3), so the
// table lists every active expert once together with the tokens it serves.
//
// One wave per token selects its k experts (route_device.h); the block then
// groups the M tokens' choices by expert in ascending id and appends the
// shared expert, which serves every token with weight 1.
#include "device_common.h"
#include "launch.h"
#include "route_device.h"

namespace moedec {

namespace {

template <int KPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int M,
                                                         int E, int k, int32_t* __restrict__ ids_out,
                                                         float* __restrict__ w_out,
                                                         moedec_dispatch* __restrict__ disp) {
    __shared__ int32_t s_id[MOEDEC_MAX_M][MOEDEC_MAX_K];
    __shared__ float s_w[MOEDEC_MAX_M][MOEDEC_MAX_K];
    __shared__ uint32_t s_bits[MOEDEC_MAX_E / 32];
    __shared__ int s_pre[MOEDEC_MAX_E / 32 + 1];
    __shared__ int32_t s_exp[MOEDEC_MAX_SLOTS];
    __shared__ uint32_t s_mask[MOEDEC_MAX_SLOTS];
    __shared__ float s_wt[MOEDEC_MAX_SLOTS][MOEDEC_MAX_M];
    __shared__ uint64_t s_buf[MOEDEC_MAX_M][kTopkBufWords];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int m = tid >> 6;  // one wave per token

    if (m < M) {
        float wv;
        const uint64_t key = wave_topk<KPL>(logits + (size_t)m * E, E, k, wv, s_buf[m]);
        if (lane < k) {
            const int id = key_to_index(key);
            if (ids_out) ids_out[m * k + lane] = id;
            if (w_out) w_out[m * k + lane] = wv;
            s_id[m][lane] = id;
            s_w[m][lane] = wv;
        }
    }
    __syncthreads();
    if (disp == nullptr) return;

    const int n_routed = block_group_by_expert(s_id, s_w, M, k, s_bits, s_pre, s_exp, s_mask, s_wt);
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

}  // namespace

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
