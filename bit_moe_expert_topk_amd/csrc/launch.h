// Internal launch functions (C++), called by the C ABI layer after argument
// checks.  Each returns the hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moedec.h"

namespace moedec {

hipError_t launch_route_topk(const float* logits, int M, int E, int k, int32_t* ids, float* w,
                             moedec_dispatch* disp, hipStream_t s);

hipError_t launch_pack_gateup(const uint8_t* gc, const uint8_t* gs, const uint8_t* uc,
                              const uint8_t* us, int n_exp, int H, int I, uint8_t* oc,
                              uint8_t* os, hipStream_t s);
hipError_t launch_pack_down(const uint8_t* dc, const uint8_t* ds, int n_exp, int H, int I,
                            uint8_t* oc, uint8_t* os, hipStream_t s);

// Per-expert packed MXFP4 sizes (bytes) for hidden H and intermediate I.
void packed_sizes(int H, int I, moedec_mxfp4_sizes* out);
// The FP8 shared expert's packed sizes and its one-time quantise-and-pack.
void shared_fp8_sizes(int H, int I, moedec_mxfp4_sizes* out);
hipError_t launch_pack_shared_fp8(const uint16_t* g, const uint16_t* u, const uint16_t* d, int H, int I,
                                  uint8_t* gu_c, float* gu_s, uint8_t* dn_c, float* dn_s, hipStream_t s);

// Workspace and launch layout of the fused FFN kernel.
struct FfnLayout {
    int max_slots;      // M * k_max + 1 (routed slots + the shared expert)
    int pair_cap;       // (slot, token) pairs per down slot group
    int max_groups;     // slot groups at most
    int pair_bytes;     // LDS bytes of one pair's h
    int red_off;        // LDS offset of the reduction scratch
    size_t lds_bytes;   // dynamic LDS per block
    size_t ctl_off, yt_off, h_off, part_off, total;   // workspace layout
    int grid;           // blocks per launch
};
FfnLayout ffn_layout(int M, int k_max, int H, int I);

// Byte offset of the wait-timeout word in an FFN workspace: it follows the
// 4,096 per-block launch counters.  A kernel whose bounded cross-block wait
// gave up sets it (and its results are invalid); moe_ffn_workspace_status
// reads and clears it.
constexpr size_t kWsStatusOffset = 4096 * sizeof(uint32_t);

// The file-scope scratch array behind moe_layer_mxfp4_noalloc (noalloc.hip):
// its size, and this device's address of it (looked up with
// hipGetSymbolAddress on the first call on a device, zero-filled then on `s`
// unless `s` is capturing a graph).
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
hipError_t noalloc_scratch(hipStream_t s, void** ptr);

// Residual stream of a decode stack: x = bf16(RMSNorm(r_in)) replaces the x
// input, and r_out = r_in + y is written next to y.
struct ResidualArgs {
    const float* r_in;
    float* r_out;
    uint16_t* x_out;    // the normalised x, or null
    float eps;
};

// Fused layer: routing from logits (when non-null) or the dispatch table, then the FFN.
hipError_t launch_moe(const moedec_moe_weights& w, const uint16_t* x, int M, int k_max,
                      const moedec_dispatch* disp, const float* logits, int32_t* ids_out,
                      float* w_out, moedec_dispatch* disp_out, uint16_t* y_bf16, float* y_f32,
                      void* ws, hipStream_t s, const ResidualArgs* res = nullptr, bool a8 = false);

hipError_t launch_expert_ffn(const moedec_moe_weights& w, const uint16_t* x, int M,
                             const moedec_dispatch* disp, int k_max, uint16_t* y_bf16,
                             float* y_f32, void* ws, hipStream_t s);

hipError_t launch_lmhead_quant(const uint16_t* w, int V, int H, uint8_t* codes, float* rs,
                               hipStream_t s);
// The FP8 GEMV's epilogue, run by the block launched last: the greedy token
// (u null or top_k = 1) or a sampled one (temperature, top_p, top_k <= 32,
// u[M] in [0, 1)).  V <= 2^18.  workspace: lmhead_epilogue_bytes(V, M) bytes,
// zero-filled before the first call, left ready for the next.
struct Fp8Epilogue {
    void* workspace;
    int32_t* ids;
    const float* u;
    float temperature, top_p;
    int top_k;
};
// act8: quantise each token's activations to E4M3 on the fly (per-token
// float32 scale, the weights' rule) and multiply FP8 by FP8.
hipError_t launch_gemv_fp8(const uint8_t* codes, const float* rs, int V, int H,
                           const uint16_t* x, int M, float* logits, hipStream_t s,
                           const Fp8Epilogue* ep = nullptr, bool act8 = false);
size_t lmhead_epilogue_bytes(int V, int M);
hipError_t launch_gemv_bf16(const uint16_t* w, int V, int H, const uint16_t* x, int M,
                            float* logits, hipStream_t s);
// Router logits [M][E] = bf16(RMSNorm(r)) W^T, the norm as the fused layer forms it.
// r [M][H] float32 16-byte aligned, H % 8 == 0, H <= 4096.
hipError_t launch_norm_router_bf16(const uint16_t* w, int E, int H, const float* r, float eps, int M,
                                   float* logits, hipStream_t s);

// Many-token layer (prefill.hip): workspace layout and the launch sequence.
struct PrefillLayout {
    int ns;             // 32-token column blocks per tile
    int max_tiles;      // tiles at most: (T*k + T) / (32*ns) + E + 1
    size_t counts_off, hist_off, base_off, off_off, n_tiles_off, tiles_off, ids_off, w_off, pos_off, tok_of_off,
        h_hi_off, h_lo_off, y_pair_off, total;
    // MXFP8-activation variant: scale bytes per token row of x (sb) and of h
    // (sbi), x's codes and scales, h's codes and scales (inside h_hi / h_lo)
    int sb, sbi;
    size_t x8_off, xs_off, h8_off, hs_off;
};
int prefill_sub_tiles(int T, int E, int k);
PrefillLayout prefill_layout(int T, int E, int k, int H, int I);
hipError_t launch_prefill(const moedec_moe_weights& w, const uint16_t* x, const float* logits, int T, int k,
                          int32_t* ids_out, float* w_out, int32_t* counts_out, uint16_t* y_bf16, float* y_f32,
                          void* ws, hipStream_t s, bool a8);

}  // namespace moedec
