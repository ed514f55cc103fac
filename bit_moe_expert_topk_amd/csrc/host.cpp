// C ABI of libmoedec: argument checks, the gfx950 device check, launches.
// Nothing here allocates device memory or synchronises a stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <vector>

#include "launch.h"
#include "moedec.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device verdict: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(MOEDEC_ERR_DEVICE, "no current HIP device");
    int v = g_device_ok[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(MOEDEC_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
        v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_ok[dev].store(v, std::memory_order_relaxed);
    }
    if (v != 1) return fail(MOEDEC_ERR_DEVICE, "device %d is not gfx950", dev);
    return MOEDEC_OK;
}

int launched(hipError_t err, const char* what) {
    if (err != hipSuccess)
        return fail(MOEDEC_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(err));
    g_last_error[0] = '\0';
    return MOEDEC_OK;
}

int check_mxfp4_shape(int H, int I) {
    if (H < 64 || H > 4096 || H % 64 != 0)
        return fail(MOEDEC_ERR_SHAPE, "H=%d: need 64 <= H <= 4096 and H %% 64 == 0", H);
    if (I < 32 || I > 2048 || I % 32 != 0)
        return fail(MOEDEC_ERR_SHAPE, "I=%d: need 32 <= I <= 2048 and I %% 32 == 0", I);
    return MOEDEC_OK;
}

}  // namespace

extern "C" {

int moedec_abi_version(void) { return MOEDEC_ABI_VERSION; }

const char* moedec_status_string(int status) {
    switch (status) {
        case MOEDEC_OK: return "ok";
        case MOEDEC_ERR_NULL: return "null pointer";
        case MOEDEC_ERR_ALIGN: return "misaligned pointer";
        case MOEDEC_ERR_SHAPE: return "unsupported shape";
        case MOEDEC_ERR_FORMAT: return "descriptor format mismatch";
        case MOEDEC_ERR_WORKSPACE: return "workspace too small";
        case MOEDEC_ERR_LAUNCH: return "kernel launch failed";
        case MOEDEC_ERR_DEVICE: return "device is not gfx950";
        case MOEDEC_ERR_SELFTEST: return "self-test mismatch";
        case MOEDEC_ERR_ARG: return "argument out of range";
        case MOEDEC_ERR_TIMEOUT: return "a cross-block wait gave up (results invalid)";
        default: return "unknown status";
    }
}

const char* moedec_last_error(void) { return g_last_error; }

int moe_route_topk(const float* logits, int M, int E, int k, int32_t* topk_ids, float* topk_w,
                   moedec_dispatch* dispatch, moedec_stream_t stream) {
    if (!logits) return fail(MOEDEC_ERR_NULL, "logits is NULL");
    if (!topk_ids && !topk_w && !dispatch)
        return fail(MOEDEC_ERR_NULL, "no output given (topk_ids, topk_w and dispatch all NULL)");
    if (M < 1 || M > MOEDEC_MAX_M) return fail(MOEDEC_ERR_SHAPE, "M=%d not in 1..%d", M, MOEDEC_MAX_M);
    if (E < 1 || E > MOEDEC_MAX_E) return fail(MOEDEC_ERR_SHAPE, "E=%d not in 1..%d", E, MOEDEC_MAX_E);
    if (k < 1 || k > E || k > MOEDEC_MAX_K)
        return fail(MOEDEC_ERR_SHAPE, "k=%d not in 1..min(E, %d)", k, MOEDEC_MAX_K);
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
        return fail(MOEDEC_ERR_ALIGN, "logits/topk_ids/topk_w must be 4-byte aligned");
    if (!aligned(dispatch, 16)) return fail(MOEDEC_ERR_ALIGN, "dispatch must be 16-byte aligned");
    if (int st = check_device()) return st;
    return launched(moedec::launch_route_topk(logits, M, E, k, topk_ids, topk_w, dispatch,
                                              static_cast<hipStream_t>(stream)),
                    "moe_route_topk");
}

int moedec_mxfp4_packed_sizes(int H, int I, moedec_mxfp4_sizes* out) {
    if (!out) return fail(MOEDEC_ERR_NULL, "out is NULL");
    if (int st = check_mxfp4_shape(H, I)) return st;
    moedec::packed_sizes(H, I, out);
    g_last_error[0] = '\0';
    return MOEDEC_OK;
}

int moe_pack_gateup_mxfp4(const uint8_t* gate_codes, const uint8_t* gate_scales,
                          const uint8_t* up_codes, const uint8_t* up_scales, int n_experts, int H,
                          int I, uint8_t* gu_codes, uint8_t* gu_scales, moedec_stream_t stream) {
    if (!gate_codes || !gate_scales || !up_codes || !up_scales || !gu_codes || !gu_scales)
        return fail(MOEDEC_ERR_NULL, "a pack pointer is NULL");
    if (n_experts < 1 || n_experts > MOEDEC_MAX_E + 1)
        return fail(MOEDEC_ERR_SHAPE, "n_experts=%d not in 1..%d", n_experts, MOEDEC_MAX_E + 1);
    if (int st = check_mxfp4_shape(H, I)) return st;
    if (!aligned(gate_codes, 16) || !aligned(up_codes, 16) || !aligned(gu_codes, 16))
        return fail(MOEDEC_ERR_ALIGN, "code arrays must be 16-byte aligned");
    if (!aligned(gu_scales, 2)) return fail(MOEDEC_ERR_ALIGN, "packed scales must be 2-byte aligned");
    if (int st = check_device()) return st;
    return launched(moedec::launch_pack_gateup(gate_codes, gate_scales, up_codes, up_scales,
                                               n_experts, H, I, gu_codes, gu_scales,
                                               static_cast<hipStream_t>(stream)),
                    "moe_pack_gateup_mxfp4");
}

int moe_pack_down_mxfp4(const uint8_t* down_codes, const uint8_t* down_scales, int n_experts,
                        int H, int I, uint8_t* dn_codes, uint8_t* dn_scales,
                        moedec_stream_t stream) {
    if (!down_codes || !down_scales || !dn_codes || !dn_scales)
        return fail(MOEDEC_ERR_NULL, "a pack pointer is NULL");
    if (n_experts < 1 || n_experts > MOEDEC_MAX_E + 1)
        return fail(MOEDEC_ERR_SHAPE, "n_experts=%d not in 1..%d", n_experts, MOEDEC_MAX_E + 1);
    if (int st = check_mxfp4_shape(H, I)) return st;
    if (!aligned(down_codes, 16) || !aligned(dn_codes, 16))
        return fail(MOEDEC_ERR_ALIGN, "code arrays must be 16-byte aligned");
    if (int st = check_device()) return st;
    return launched(moedec::launch_pack_down(down_codes, down_scales, n_experts, H, I, dn_codes,
                                             dn_scales, static_cast<hipStream_t>(stream)),
                    "moe_pack_down_mxfp4");
}

int moedec_shared_fp8_packed_sizes(int H, int I, moedec_mxfp4_sizes* out) {
    if (!out) return fail(MOEDEC_ERR_NULL, "out is NULL");
    if (int st = check_mxfp4_shape(H, I)) return st;
    moedec::shared_fp8_sizes(H, I, out);
    g_last_error[0] = '\0';
    return MOEDEC_OK;
}

int moe_pack_shared_fp8(const uint16_t* gate_bf16, const uint16_t* up_bf16, const uint16_t* down_bf16, int H,
                        int I, uint8_t* gu_codes, float* gu_scales, uint8_t* dn_codes, float* dn_scales,
                        moedec_stream_t stream) {
    if (!gate_bf16 || !up_bf16 || !down_bf16 || !gu_codes || !gu_scales || !dn_codes || !dn_scales)
        return fail(MOEDEC_ERR_NULL, "a pack pointer is NULL");
    if (int st = check_mxfp4_shape(H, I)) return st;
    if (!aligned(gate_bf16, 2) || !aligned(up_bf16, 2) || !aligned(down_bf16, 2) || !aligned(gu_codes, 16) ||
        !aligned(dn_codes, 16) || !aligned(gu_scales, 4) || !aligned(dn_scales, 4))
        return fail(MOEDEC_ERR_ALIGN, "code arrays 16-byte, scales 4-byte, bf16 inputs 2-byte alignment needed");
    if (int st = check_device()) return st;
    return launched(moedec::launch_pack_shared_fp8(gate_bf16, up_bf16, down_bf16, H, I, gu_codes, gu_scales,
                                                   dn_codes, dn_scales, static_cast<hipStream_t>(stream)),
                    "moe_pack_shared_fp8");
}

size_t moe_ffn_workspace_bytes(int M, int k_max, int H, int I) {
    if (M < 1 || M > MOEDEC_MAX_M || k_max < 1 || k_max > MOEDEC_MAX_K || H < 64 || H > 4096 ||
        H % 64 || I < 32 || I > 2048 || I % 32)
        return 0;
    return moedec::ffn_layout(M, k_max, H, I).total;
}

int moe_ffn_workspace_layout(int M, int k_max, int H, int I, moedec_ffn_layout* out) {
    if (!out) return fail(MOEDEC_ERR_NULL, "out is NULL");
    if (!moe_ffn_workspace_bytes(M, k_max, H, I))
        return fail(MOEDEC_ERR_SHAPE, "M=%d k_max=%d H=%d I=%d out of range", M, k_max, H, I);
    const moedec::FfnLayout L = moedec::ffn_layout(M, k_max, H, I);
    out->total_bytes = L.total;
    out->h_words = L.h_off;
    out->max_slots = L.max_slots;
    out->M = M;
    return MOEDEC_OK;
}

// Checks of a MoE call's weights, activations and sizes (not its workspace).
static int check_moe_core(const moedec_moe_weights* w, const uint16_t* x_bf16, int M, int k,
                          uint16_t* y_bf16, float* y_f32, bool residual) {
    if (!w) return fail(MOEDEC_ERR_NULL, "weights descriptor is NULL");
    if (w->magic != MOEDEC_MOE_MAGIC && w->magic != MOEDEC_MOE_MAGIC_SHARED_FP8)
        return fail(MOEDEC_ERR_FORMAT, "weights descriptor magic 0x%08x is neither 0x%08x nor 0x%08x", w->magic,
                    MOEDEC_MOE_MAGIC, MOEDEC_MOE_MAGIC_SHARED_FP8);
    if (!w->gu_codes || !w->gu_scales || !w->dn_codes || !w->dn_scales || !w->sh_gu_codes ||
        !w->sh_gu_scales || !w->sh_dn_codes || !w->sh_dn_scales)
        return fail(MOEDEC_ERR_NULL, "a weight pointer is NULL");
    if (!residual && (!x_bf16 || !y_bf16)) return fail(MOEDEC_ERR_NULL, "x or y_bf16 is NULL");
    if (M < 1 || M > MOEDEC_MAX_M) return fail(MOEDEC_ERR_SHAPE, "M=%d not in 1..%d", M, MOEDEC_MAX_M);
    if (w->E < 1 || w->E > MOEDEC_MAX_E) return fail(MOEDEC_ERR_SHAPE, "E=%d not in 1..%d", w->E, MOEDEC_MAX_E);
    if (k < 1 || k > MOEDEC_MAX_K || k > w->E)
        return fail(MOEDEC_ERR_SHAPE, "k=%d not in 1..min(E, %d)", k, MOEDEC_MAX_K);
    if (int st = check_mxfp4_shape(w->H, w->I)) return st;
    if (!aligned(w->gu_codes, 16) || !aligned(w->dn_codes, 16) || !aligned(w->sh_gu_codes, 16) ||
        !aligned(w->sh_dn_codes, 16))
        return fail(MOEDEC_ERR_ALIGN, "packed code arrays must be 16-byte aligned");
    if (!aligned(w->gu_scales, 2) || !aligned(w->sh_gu_scales, 2))
        return fail(MOEDEC_ERR_ALIGN, "packed gate/up scale arrays must be 2-byte aligned");
    if (w->magic == MOEDEC_MOE_MAGIC_SHARED_FP8 && (!aligned(w->sh_gu_scales, 4) || !aligned(w->sh_dn_scales, 4)))
        return fail(MOEDEC_ERR_ALIGN, "the FP8 shared expert's float32 scale arrays must be 4-byte aligned");
    if (!aligned(x_bf16, 16) || !aligned(y_bf16, 4) || !aligned(y_f32, 4))
        return fail(MOEDEC_ERR_ALIGN, "x must be 16-byte aligned, y_bf16 and y_f32 4-byte");
    return MOEDEC_OK;
}

static int check_moe_args(const moedec_moe_weights* w, const uint16_t* x_bf16, int M, int k,
                          uint16_t* y_bf16, float* y_f32, void* workspace, size_t workspace_bytes,
                          bool residual = false) {
    if (int st = check_moe_core(w, x_bf16, M, k, y_bf16, y_f32, residual)) return st;
    if (!workspace) return fail(MOEDEC_ERR_NULL, "workspace is NULL");
    if (!aligned(workspace, 16)) return fail(MOEDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t need = moedec::ffn_layout(M, k, w->H, w->I).total;
    if (workspace_bytes < need)
        return fail(MOEDEC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    return MOEDEC_OK;
}

int moe_expert_ffn_mxfp4(const moedec_moe_weights* w, const uint16_t* x_bf16, int M,
                         const moedec_dispatch* dispatch, int k_max, uint16_t* y_bf16, float* y_f32,
                         void* workspace, size_t workspace_bytes, moedec_stream_t stream) {
    if (int st = check_moe_args(w, x_bf16, M, k_max, y_bf16, y_f32, workspace, workspace_bytes)) return st;
    if (w->magic == MOEDEC_MOE_MAGIC_SHARED_FP8)
        return fail(MOEDEC_ERR_FORMAT, "the dispatch-table FFN takes an MXFP4 shared expert; "
                                       "use moe_layer_mxfp4 for an FP8 one");
    if (!dispatch) return fail(MOEDEC_ERR_NULL, "dispatch is NULL");
    if (!aligned(dispatch, 16)) return fail(MOEDEC_ERR_ALIGN, "dispatch must be 16-byte aligned");
    if (int st = check_device()) return st;
    return launched(moedec::launch_expert_ffn(*w, x_bf16, M, dispatch, k_max, y_bf16, y_f32,
                                              workspace, static_cast<hipStream_t>(stream)),
                    "moe_expert_ffn_mxfp4");
}

static int fused_layer(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int M, int k,
                       int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch, uint16_t* y_bf16,
                       float* y_f32, void* workspace, size_t workspace_bytes, moedec_stream_t stream, bool a8,
                       const char* name) {
    if (int st = check_moe_args(w, x_bf16, M, k, y_bf16, y_f32, workspace, workspace_bytes)) return st;
    if (a8 && w->magic == MOEDEC_MOE_MAGIC_SHARED_FP8)
        return fail(MOEDEC_ERR_FORMAT, "the W4A8 layer takes an MXFP4 shared expert");
    if (!logits) return fail(MOEDEC_ERR_NULL, "logits is NULL");
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
        return fail(MOEDEC_ERR_ALIGN, "logits/topk_ids/topk_w must be 4-byte aligned");
    if (!aligned(dispatch, 16)) return fail(MOEDEC_ERR_ALIGN, "dispatch must be 16-byte aligned");
    if (int st = check_device()) return st;
    return launched(moedec::launch_moe(*w, x_bf16, M, k, nullptr, logits, topk_ids, topk_w, dispatch,
                                       y_bf16, y_f32, workspace, static_cast<hipStream_t>(stream), nullptr, a8),
                    name);
}

int moe_layer_mxfp4(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int M,
                    int k, int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch,
                    uint16_t* y_bf16, float* y_f32, void* workspace, size_t workspace_bytes,
                    moedec_stream_t stream) {
    return fused_layer(w, x_bf16, logits, M, k, topk_ids, topk_w, dispatch, y_bf16, y_f32, workspace,
                       workspace_bytes, stream, false, "moe_layer_mxfp4");
}

int moe_layer_mxfp4_a8(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int M,
                       int k, int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch,
                       uint16_t* y_bf16, float* y_f32, void* workspace, size_t workspace_bytes,
                       moedec_stream_t stream) {
    return fused_layer(w, x_bf16, logits, M, k, topk_ids, topk_w, dispatch, y_bf16, y_f32, workspace,
                       workspace_bytes, stream, true, "moe_layer_mxfp4_a8");
}

int moe_ffn_workspace_status(void* workspace, size_t workspace_bytes, uint32_t* flags_out,
                             moedec_stream_t stream) {
    if (flags_out) *flags_out = 0;
    if (workspace && workspace_bytes < moedec::kWsStatusOffset + sizeof(uint32_t))
        return fail(MOEDEC_ERR_WORKSPACE, "workspace %zu bytes holds no status word (need > %zu)",
                    workspace_bytes, moedec::kWsStatusOffset);
    if (workspace && !aligned(workspace, 16)) return fail(MOEDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (int st = check_device()) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    size_t bytes = workspace_bytes;
    if (!ws) {
        void* p = nullptr;
        if (hipError_t e = moedec::noalloc_scratch(s, &p))
            return fail(MOEDEC_ERR_LAUNCH, "no-alloc scratch: %s", hipGetErrorString(e));
        ws = static_cast<uint8_t*>(p);
        bytes = moedec::kNoAllocScratchBytes;
    }
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, ws + moedec::kWsStatusOffset, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return fail(MOEDEC_ERR_LAUNCH, "reading the workspace status word failed");
    if (flags_out) *flags_out = word;
    if (word != 0) {
        // the calls since the last check are invalid and may have left tagged
        // words behind: clear the whole workspace so it can be used again
        if (hipMemsetAsync(ws, 0, bytes, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
            return fail(MOEDEC_ERR_LAUNCH, "clearing the workspace failed");
        return fail(MOEDEC_ERR_TIMEOUT,
                    "a cross-block wait gave up in a call on this workspace (status 0x%x): results since the "
                    "last check are invalid; the workspace was cleared", word);
    }
    g_last_error[0] = '\0';
    return MOEDEC_OK;
}

int moe_layer_mxfp4_noalloc(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int M,
                            int k, int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch,
                            uint16_t* y_bf16, float* y_f32, moedec_stream_t stream) {
    // argument checks as moe_layer_mxfp4, the workspace being the fixed scratch
    if (int st = check_moe_core(w, x_bf16, M, k, y_bf16, y_f32, false)) return st;
    const size_t need = moedec::ffn_layout(M, k, w->H, w->I).total;
    if (need > moedec::kNoAllocScratchBytes)
        return fail(MOEDEC_ERR_WORKSPACE, "M=%d k=%d H=%d I=%d needs %zu bytes of scratch > the %zu-byte "
                    "no-alloc limit", M, k, w->H, w->I, need, moedec::kNoAllocScratchBytes);
    if (!logits) return fail(MOEDEC_ERR_NULL, "logits is NULL");
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
        return fail(MOEDEC_ERR_ALIGN, "logits/topk_ids/topk_w must be 4-byte aligned");
    if (!aligned(dispatch, 16)) return fail(MOEDEC_ERR_ALIGN, "dispatch must be 16-byte aligned");
    if (int st = check_device()) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (hipError_t e = moedec::noalloc_scratch(s, &ws))
        return fail(MOEDEC_ERR_LAUNCH, "no-alloc scratch: %s", hipGetErrorString(e));
    return launched(moedec::launch_moe(*w, x_bf16, M, k, nullptr, logits, topk_ids, topk_w, dispatch,
                                       y_bf16, y_f32, ws, s),
                    "moe_layer_mxfp4_noalloc");
}

// Checks of the layer steps that start from the residual stream.
static int check_residual_layer(const moedec_moe_weights* w, const float* r_in, const float* logits, int M,
                                int k, float eps, float* r_out, uint16_t* x_bf16, float* y_f32,
                                void* workspace, size_t workspace_bytes) {
    if (int st = check_moe_args(w, x_bf16, M, k, nullptr, y_f32, workspace, workspace_bytes, true))
        return st;
    if (!r_in || !r_out || !logits) return fail(MOEDEC_ERR_NULL, "r_in, r_out or logits is NULL");
    if (!(eps >= 0.f) || eps > 1.f) return fail(MOEDEC_ERR_SHAPE, "eps=%g not in [0, 1]", (double)eps);
    if (!aligned(r_in, 16) || !aligned(r_out, 16) || !aligned(logits, 4))
        return fail(MOEDEC_ERR_ALIGN, "r_in and r_out must be 16-byte aligned, logits 4-byte");
    const size_t bytes = (size_t)M * w->H * sizeof(float);
    const auto lo_in = reinterpret_cast<uintptr_t>(r_in), lo_out = reinterpret_cast<uintptr_t>(r_out);
    if (lo_in < lo_out + bytes && lo_out < lo_in + bytes)
        return fail(MOEDEC_ERR_SHAPE, "r_out overlaps r_in (use two buffers)");
    return MOEDEC_OK;
}

int moe_layer_rmsnorm_mxfp4(const moedec_moe_weights* w, const float* r_in, const float* logits, int M,
                            int k, float eps, float* r_out, uint16_t* x_bf16, float* y_f32,
                            void* workspace, size_t workspace_bytes, moedec_stream_t stream) {
    if (int st = check_residual_layer(w, r_in, logits, M, k, eps, r_out, x_bf16, y_f32, workspace,
                                      workspace_bytes))
        return st;
    if (int st = check_device()) return st;
    moedec::ResidualArgs res{r_in, r_out, x_bf16, eps};
    return launched(moedec::launch_moe(*w, nullptr, M, k, nullptr, logits, nullptr, nullptr, nullptr,
                                       nullptr, y_f32, workspace, static_cast<hipStream_t>(stream), &res),
                    "moe_layer_rmsnorm_mxfp4");
}

int moe_layer_rmsnorm_router_mxfp4(const moedec_moe_weights* w, const uint16_t* w_router, const float* r_in,
                                   int M, int k, float eps, float* logits, float* r_out, uint16_t* x_bf16,
                                   float* y_f32, void* workspace, size_t workspace_bytes,
                                   moedec_stream_t stream) {
    if (int st = check_residual_layer(w, r_in, logits, M, k, eps, r_out, x_bf16, y_f32, workspace,
                                      workspace_bytes))
        return st;
    if (!w_router) return fail(MOEDEC_ERR_NULL, "w_router is NULL");
    if (!aligned(w_router, 16)) return fail(MOEDEC_ERR_ALIGN, "w_router must be 16-byte aligned");
    if (w->H % 8 || w->H > 4096) return fail(MOEDEC_ERR_SHAPE, "H=%d: the router needs H %% 8 == 0, H <= 4096", w->H);
    if (int st = check_device()) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (int st = launched(moedec::launch_norm_router_bf16(w_router, w->E, w->H, r_in, eps, M, logits, s),
                          "moe_layer_rmsnorm_router_mxfp4 (router)"))
        return st;
    moedec::ResidualArgs res{r_in, r_out, x_bf16, eps};
    return launched(moedec::launch_moe(*w, nullptr, M, k, nullptr, logits, nullptr, nullptr, nullptr,
                                       nullptr, y_f32, workspace, s, &res),
                    "moe_layer_rmsnorm_router_mxfp4");
}

size_t moe_prefill_workspace_bytes(int T, int E, int k, int H, int I) {
    if (T < 1 || T > MOEDEC_MAX_PREFILL_T || E < 1 || E > MOEDEC_MAX_E || k < 1 || k > MOEDEC_MAX_K || k > E)
        return 0;
    if (H < 64 || H > 4096 || H % 64 || I < 32 || I > 2048 || I % 32) return 0;
    return moedec::prefill_layout(T, E, k, H, I).total;
}

int moe_prefill_workspace_layout(int T, int E, int k, int H, int I, moedec_prefill_layout* out) {
    if (!out) return fail(MOEDEC_ERR_NULL, "out is NULL");
    if (!moe_prefill_workspace_bytes(T, E, k, H, I))
        return fail(MOEDEC_ERR_SHAPE, "T=%d E=%d k=%d H=%d I=%d out of range", T, E, k, H, I);
    const moedec::PrefillLayout l = moedec::prefill_layout(T, E, k, H, I);
    out->total_bytes = l.total;
    out->pos = l.pos_off;
    out->y_pair = l.y_pair_off;
    out->x_codes = l.x8_off;
    out->x_scales = l.xs_off;
    out->h_codes = l.h8_off;
    out->h_scales = l.hs_off;
    out->x_scale_stride = l.sb;
    out->h_scale_stride = l.sbi;
    return MOEDEC_OK;
}

static int prefill_call(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int T, int k,
                        int32_t* topk_ids, float* topk_w, int32_t* group_counts, uint16_t* y_bf16, float* y_f32,
                        void* workspace, size_t workspace_bytes, moedec_stream_t stream, bool a8,
                        const char* name) {
    if (!w) return fail(MOEDEC_ERR_NULL, "weights descriptor is NULL");
    if (w->magic == MOEDEC_MOE_MAGIC_SHARED_FP8)
        return fail(MOEDEC_ERR_FORMAT, "the many-token layer takes an MXFP4 shared expert");
    if (int st = check_moe_core(w, x_bf16, 1, k, y_bf16, y_f32, false)) return st;
    if (!aligned(w->gu_scales, 4) || !aligned(w->dn_scales, 4) || !aligned(w->sh_gu_scales, 4) ||
        !aligned(w->sh_dn_scales, 4))
        return fail(MOEDEC_ERR_ALIGN, "the many-token layer needs 4-byte aligned scale arrays");
    if (!logits) return fail(MOEDEC_ERR_NULL, "logits is NULL");
    if (T < 1 || T > MOEDEC_MAX_PREFILL_T)
        return fail(MOEDEC_ERR_SHAPE, "T=%d not in 1..%d", T, MOEDEC_MAX_PREFILL_T);
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(group_counts, 4))
        return fail(MOEDEC_ERR_ALIGN, "logits/topk_ids/topk_w/group_counts must be 4-byte aligned");
    if (!aligned(y_bf16, 8) || !aligned(y_f32, 16))
        return fail(MOEDEC_ERR_ALIGN, "y_bf16 must be 8-byte aligned, y_f32 16-byte");
    if (!workspace) return fail(MOEDEC_ERR_NULL, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(MOEDEC_ERR_ALIGN, "workspace must be 256-byte aligned");
    const size_t need = moedec::prefill_layout(T, w->E, k, w->H, w->I).total;
    if (workspace_bytes < need)
        return fail(MOEDEC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if (int st = check_device()) return st;
    return launched(moedec::launch_prefill(*w, x_bf16, logits, T, k, topk_ids, topk_w, group_counts, y_bf16,
                                           y_f32, workspace, static_cast<hipStream_t>(stream), a8),
                    name);
}

int moe_layer_mxfp4_prefill(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int T,
                            int k, int32_t* topk_ids, float* topk_w, int32_t* group_counts, uint16_t* y_bf16,
                            float* y_f32, void* workspace, size_t workspace_bytes, moedec_stream_t stream) {
    return prefill_call(w, x_bf16, logits, T, k, topk_ids, topk_w, group_counts, y_bf16, y_f32, workspace,
                        workspace_bytes, stream, false, "moe_layer_mxfp4_prefill");
}

int moe_layer_mxfp4_prefill_a8(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int T,
                               int k, int32_t* topk_ids, float* topk_w, int32_t* group_counts, uint16_t* y_bf16,
                               float* y_f32, void* workspace, size_t workspace_bytes, moedec_stream_t stream) {
    return prefill_call(w, x_bf16, logits, T, k, topk_ids, topk_w, group_counts, y_bf16, y_f32, workspace,
                        workspace_bytes, stream, true, "moe_layer_mxfp4_prefill_a8");
}

int lmhead_quant_fp8(const uint16_t* w_bf16, int V, int H, uint8_t* codes, float* row_scale,
                     moedec_lmhead_fp8* out_desc, moedec_stream_t stream) {
    if (!w_bf16 || !codes || !row_scale) return fail(MOEDEC_ERR_NULL, "w, codes or row_scale is NULL");
    if (V < 1) return fail(MOEDEC_ERR_SHAPE, "V=%d < 1", V);
    if (H < 16 || H > 8192 || H % 16)
        return fail(MOEDEC_ERR_SHAPE, "H=%d: need 16 <= H <= 8192 and H %% 16 == 0", H);
    if (!aligned(w_bf16, 16) || !aligned(codes, 16) || !aligned(row_scale, 4))
        return fail(MOEDEC_ERR_ALIGN, "w and codes must be 16-byte aligned, row_scale 4-byte");
    if (int st = check_device()) return st;
    const int st = launched(moedec::launch_lmhead_quant(w_bf16, V, H, codes, row_scale,
                                                        static_cast<hipStream_t>(stream)),
                            "lmhead_quant_fp8");
    if (st == MOEDEC_OK && out_desc) {
        out_desc->magic = MOEDEC_LMHEAD_MAGIC;
        out_desc->format = MOEDEC_FMT_E4M3FN_ROWSCALE_F32;
        out_desc->V = V;
        out_desc->H = H;
        out_desc->codes = codes;
        out_desc->row_scale = row_scale;
    }
    return st;
}

int lmhead_gemv_fp8(const moedec_lmhead_fp8* head, const uint16_t* x_bf16, int M, float* logits,
                    moedec_stream_t stream) {
    if (!head) return fail(MOEDEC_ERR_NULL, "head descriptor is NULL");
    if (head->magic != MOEDEC_LMHEAD_MAGIC)
        return fail(MOEDEC_ERR_FORMAT, "head magic 0x%08x is not an FP8 LM-head descriptor",
                    head->magic);
    if (head->format != MOEDEC_FMT_E4M3FN_ROWSCALE_F32 && head->format != MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT)
        return fail(MOEDEC_ERR_FORMAT, "head format %u is not E4M3 with per-row float32 scales",
                    head->format);
    if (!head->codes || !head->row_scale || !x_bf16 || !logits)
        return fail(MOEDEC_ERR_NULL, "codes, row_scale, x or logits is NULL");
    if (M < 1 || M > MOEDEC_MAX_M) return fail(MOEDEC_ERR_SHAPE, "M=%d not in 1..%d", M, MOEDEC_MAX_M);
    if (head->V < 1) return fail(MOEDEC_ERR_SHAPE, "V=%d < 1", head->V);
    if (head->H < 16 || head->H > 4096 || head->H % 16)
        return fail(MOEDEC_ERR_SHAPE, "H=%d: need 16 <= H <= 4096 and H %% 16 == 0", head->H);
    if (!aligned(head->codes, 16) || !aligned(head->row_scale, 4) || !aligned(x_bf16, 4) ||
        !aligned(logits, 4))
        return fail(MOEDEC_ERR_ALIGN, "codes 16-byte, row_scale/x/logits 4-byte alignment needed");
    if (int st = check_device()) return st;
    return launched(moedec::launch_gemv_fp8(head->codes, head->row_scale, head->V, head->H, x_bf16,
                                            M, logits, static_cast<hipStream_t>(stream), nullptr,
                                            head->format == MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT),
                    "lmhead_gemv_fp8");
}

int lmhead_gemv_bf16(const uint16_t* w_bf16, int V, int H, const uint16_t* x_bf16, int M,
                     float* logits, moedec_stream_t stream) {
    if (!w_bf16 || !x_bf16 || !logits) return fail(MOEDEC_ERR_NULL, "w, x or logits is NULL");
    if (M < 1 || M > MOEDEC_MAX_M) return fail(MOEDEC_ERR_SHAPE, "M=%d not in 1..%d", M, MOEDEC_MAX_M);
    if (V < 1) return fail(MOEDEC_ERR_SHAPE, "V=%d < 1", V);
    if (H < 8 || H > 4096 || H % 8)
        return fail(MOEDEC_ERR_SHAPE, "H=%d: need 8 <= H <= 4096 and H %% 8 == 0", H);
    if (!aligned(w_bf16, 16) || !aligned(x_bf16, 4) || !aligned(logits, 4))
        return fail(MOEDEC_ERR_ALIGN, "w 16-byte, x/logits 4-byte alignment needed");
    if (int st = check_device()) return st;
    return launched(moedec::launch_gemv_bf16(w_bf16, V, H, x_bf16, M, logits,
                                             static_cast<hipStream_t>(stream)),
                    "lmhead_gemv_bf16");
}

size_t lmhead_argmax_workspace_bytes(int V, int M) {
    if (V < 1 || V > MOEDEC_MAX_EPILOGUE_V || M < 1 || M > MOEDEC_MAX_M) return 0;
    return moedec::lmhead_epilogue_bytes(V, M);
}

namespace {

// Checks shared by the greedy and the sampling epilogue calls.
int check_epilogue(const moedec_lmhead_fp8* head, const uint16_t* x_bf16, int M, const float* logits,
                   const int32_t* token_ids, const void* workspace, size_t workspace_bytes) {
    if (!head) return fail(MOEDEC_ERR_NULL, "head descriptor is NULL");
    if (head->magic != MOEDEC_LMHEAD_MAGIC)
        return fail(MOEDEC_ERR_FORMAT, "head magic 0x%08x is not an FP8 LM-head descriptor",
                    head->magic);
    if (head->format != MOEDEC_FMT_E4M3FN_ROWSCALE_F32 && head->format != MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT)
        return fail(MOEDEC_ERR_FORMAT, "head format %u is not E4M3 with per-row float32 scales",
                    head->format);
    if (!head->codes || !head->row_scale || !x_bf16 || !token_ids || !workspace)
        return fail(MOEDEC_ERR_NULL, "codes, row_scale, x, token_ids or workspace is NULL");
    if (M < 1 || M > MOEDEC_MAX_M) return fail(MOEDEC_ERR_SHAPE, "M=%d not in 1..%d", M, MOEDEC_MAX_M);
    if (head->V < 1 || head->V > MOEDEC_MAX_EPILOGUE_V)
        return fail(MOEDEC_ERR_SHAPE, "V=%d not in 1..%d", head->V, MOEDEC_MAX_EPILOGUE_V);
    if (head->H < 16 || head->H > 4096 || head->H % 16)
        return fail(MOEDEC_ERR_SHAPE, "H=%d: need 16 <= H <= 4096 and H %% 16 == 0", head->H);
    if (!aligned(head->codes, 16) || !aligned(head->row_scale, 4) || !aligned(x_bf16, 4) ||
        !aligned(logits, 4) || !aligned(token_ids, 4) || !aligned(workspace, 8))
        return fail(MOEDEC_ERR_ALIGN,
                    "codes 16-byte, row_scale/x/logits/token_ids 4-byte, workspace 8-byte alignment needed");
    const size_t need = moedec::lmhead_epilogue_bytes(head->V, M);
    if (workspace_bytes < need)
        return fail(MOEDEC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    return MOEDEC_OK;
}

}  // namespace

int lmhead_gemv_fp8_argmax(const moedec_lmhead_fp8* head, const uint16_t* x_bf16, int M, float* logits,
                           int32_t* token_ids, void* workspace, size_t workspace_bytes,
                           moedec_stream_t stream) {
    if (int st = check_epilogue(head, x_bf16, M, logits, token_ids, workspace, workspace_bytes)) return st;
    if (int st = check_device()) return st;
    const moedec::Fp8Epilogue ep{workspace, token_ids, nullptr, 1.f, 1.f, 1};
    return launched(moedec::launch_gemv_fp8(head->codes, head->row_scale, head->V, head->H, x_bf16, M,
                                            logits, static_cast<hipStream_t>(stream), &ep,
                                            head->format == MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT),
                    "lmhead_gemv_fp8_argmax");
}

int lmhead_gemv_fp8_sample(const moedec_lmhead_fp8* head, const uint16_t* x_bf16, int M,
                           float temperature, float top_p, int top_k, const float* u, float* logits,
                           int32_t* token_ids, void* workspace, size_t workspace_bytes,
                           moedec_stream_t stream) {
    if (int st = check_epilogue(head, x_bf16, M, logits, token_ids, workspace, workspace_bytes)) return st;
    if (!u) return fail(MOEDEC_ERR_NULL, "u is NULL");
    if (!aligned(u, 4)) return fail(MOEDEC_ERR_ALIGN, "u must be 4-byte aligned");
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return fail(MOEDEC_ERR_ARG, "temperature %g: need a finite value > 0", (double)temperature);
    if (!(top_p > 0.f && top_p <= 1.f)) return fail(MOEDEC_ERR_ARG, "top_p %g not in (0, 1]", (double)top_p);
    if (top_k < 1 || top_k > MOEDEC_MAX_SAMPLE_K || top_k > head->V)
        return fail(MOEDEC_ERR_ARG, "top_k=%d not in 1..min(%d, V=%d)", top_k, MOEDEC_MAX_SAMPLE_K, head->V);
    if (int st = check_device()) return st;
    const moedec::Fp8Epilogue ep{workspace, token_ids, u, temperature, top_p, top_k};
    return launched(moedec::launch_gemv_fp8(head->codes, head->row_scale, head->V, head->H, x_bf16, M,
                                            logits, static_cast<hipStream_t>(stream), &ep,
                                            head->format == MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT),
                    "lmhead_gemv_fp8_sample");
}

int moe_router_logits_bf16(const uint16_t* w_router, int E, int H, const uint16_t* x_bf16, int M,
                           float* logits, moedec_stream_t stream) {
    if (!w_router || !x_bf16 || !logits) return fail(MOEDEC_ERR_NULL, "w_router, x or logits is NULL");
    if (M < 1 || M > MOEDEC_MAX_M) return fail(MOEDEC_ERR_SHAPE, "M=%d not in 1..%d", M, MOEDEC_MAX_M);
    if (E < 1 || E > MOEDEC_MAX_E) return fail(MOEDEC_ERR_SHAPE, "E=%d not in 1..%d", E, MOEDEC_MAX_E);
    if (H < 8 || H > 4096 || H % 8)
        return fail(MOEDEC_ERR_SHAPE, "H=%d: need 8 <= H <= 4096 and H %% 8 == 0", H);
    if (!aligned(w_router, 16) || !aligned(x_bf16, 4) || !aligned(logits, 4))
        return fail(MOEDEC_ERR_ALIGN, "w_router 16-byte, x/logits 4-byte alignment needed");
    if (int st = check_device()) return st;
    return launched(moedec::launch_gemv_bf16(w_router, E, H, x_bf16, M, logits,
                                             static_cast<hipStream_t>(stream)),
                    "moe_router_logits_bf16");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Start-up self-check: closed-form cases (no stored expected values).

namespace {

constexpr int kStE = 4, kStH = 64, kStI = 32, kStK = 2;        // MoE case
constexpr int kStV = 2, kStHv = 16;                            // LM-head case

struct StLayout {
    size_t gate_c, gate_s, up_c, up_s, down_c, down_s;           // canonical routed experts
    size_t sgate_c, sgate_s, sup_c, sup_s, sdown_c, sdown_s;     // canonical shared expert
    size_t gu_c, gu_s, dn_c, dn_s, sgu_c, sgu_s, sdn_c, sdn_s;   // packed
    size_t x, logits, ids, w, disp, y, y32, ws;
    size_t lw, lcodes, lscale, lx, llogits, lid, lws;
    size_t total;
    moedec_mxfp4_sizes sz;
};

StLayout st_layout() {
    StLayout L{};
    moedec::packed_sizes(kStH, kStI, &L.sz);
    size_t off = 0;
    auto take = [&](size_t bytes) { off = (off + 255) & ~(size_t)255; const size_t at = off; off += bytes; return at; };
    const size_t gc = (size_t)kStI * kStH / 2, gs = (size_t)kStI * kStH / 32;
    const size_t dc = (size_t)kStH * kStI / 2, ds = (size_t)kStH * kStI / 32;
    L.gate_c = take(kStE * gc); L.gate_s = take(kStE * gs); L.up_c = take(kStE * gc); L.up_s = take(kStE * gs);
    L.down_c = take(kStE * dc); L.down_s = take(kStE * ds);
    L.sgate_c = take(gc); L.sgate_s = take(gs); L.sup_c = take(gc); L.sup_s = take(gs);
    L.sdown_c = take(dc); L.sdown_s = take(ds);
    L.gu_c = take(kStE * L.sz.gu_codes); L.gu_s = take(kStE * L.sz.gu_scales);
    L.dn_c = take(kStE * L.sz.dn_codes); L.dn_s = take(kStE * L.sz.dn_scales);
    L.sgu_c = take(L.sz.gu_codes); L.sgu_s = take(L.sz.gu_scales);
    L.sdn_c = take(L.sz.dn_codes); L.sdn_s = take(L.sz.dn_scales);
    L.x = take(kStH * 2); L.logits = take(kStE * 4); L.ids = take(kStK * 4); L.w = take(kStK * 4);
    L.disp = take(sizeof(moedec_dispatch)); L.y = take(kStH * 2); L.y32 = take(kStH * 4);
    L.ws = take(moedec::ffn_layout(1, kStK, kStH, kStI).total);
    L.lw = take(kStV * kStHv * 2); L.lcodes = take(kStV * kStHv); L.lscale = take(kStV * 4);
    L.lx = take(kStHv * 2); L.llogits = take(kStV * 4); L.lid = take(4);
    L.lws = take(moedec::lmhead_epilogue_bytes(kStV, 1));
    L.total = (off + 255) & ~(size_t)255;
    return L;
}

float st_bf16_to_f32(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

}  // namespace

extern "C" {

size_t moedec_selftest_bytes(void) { return st_layout().total; }

int moedec_selftest(void* scratch, size_t scratch_bytes, moedec_stream_t stream) {
    const StLayout L = st_layout();
    if (!scratch) return fail(MOEDEC_ERR_NULL, "scratch is NULL");
    if (!aligned(scratch, 256)) return fail(MOEDEC_ERR_ALIGN, "scratch must be 256-byte aligned");
    if (scratch_bytes < L.total)
        return fail(MOEDEC_ERR_WORKSPACE, "scratch %zu bytes < %zu needed", scratch_bytes, L.total);
    if (int st = check_device()) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* d = static_cast<uint8_t*>(scratch);
    // host inputs: every E2M1 nibble is code 2 (+1.0); gate/up scales 2^0, down scales 2^-5
    std::vector<uint8_t> ones(kStE * (size_t)kStI * kStH / 2, 0x22);
    std::vector<uint8_t> sc0(kStE * (size_t)kStI * kStH / 32, 127), scd(kStE * (size_t)kStH * kStI / 32, 122);
    std::vector<uint16_t> x(kStH, 0x3C80);                              // bf16 2^-6
    const float logits[kStE] = {1.5f, 0.5f, 1.5f, -1.0f};
    // LM head: row 0 = {448, -2, 1, 0.5, 0...}, row 1 = 0.25 everywhere; x = one-hot at 1
    std::vector<uint16_t> lw(kStV * kStHv, 0), lx(kStHv, 0);
    lw[0] = 0x43E0; lw[1] = 0xC000; lw[2] = 0x3F80; lw[3] = 0x3F00;
    for (int j = 0; j < kStHv; ++j) lw[kStHv + j] = 0x3E80;
    lx[1] = 0x3F80;
    const size_t gc = (size_t)kStI * kStH / 2, gs = (size_t)kStI * kStH / 32, ds = (size_t)kStH * kStI / 32;
    struct Copy { size_t at; const void* p; size_t n; } copies[] = {
        {L.gate_c, ones.data(), kStE * gc}, {L.up_c, ones.data(), kStE * gc}, {L.down_c, ones.data(), kStE * gc},
        {L.gate_s, sc0.data(), kStE * gs}, {L.up_s, sc0.data(), kStE * gs}, {L.down_s, scd.data(), kStE * ds},
        {L.sgate_c, ones.data(), gc}, {L.sup_c, ones.data(), gc}, {L.sdown_c, ones.data(), gc},
        {L.sgate_s, sc0.data(), gs}, {L.sup_s, sc0.data(), gs}, {L.sdown_s, scd.data(), ds},
        {L.x, x.data(), kStH * 2}, {L.logits, logits, sizeof(logits)},
        {L.lw, lw.data(), lw.size() * 2}, {L.lx, lx.data(), lx.size() * 2}};
    for (const Copy& c : copies)
        if (hipMemcpyAsync(d + c.at, c.p, c.n, hipMemcpyHostToDevice, s) != hipSuccess)
            return fail(MOEDEC_ERR_LAUNCH, "self-test: copy to scratch failed");
    if (hipMemsetAsync(d + L.ws, 0, moedec::ffn_layout(1, kStK, kStH, kStI).total, s) != hipSuccess ||
        hipMemsetAsync(d + L.lws, 0, moedec::lmhead_epilogue_bytes(kStV, 1), s) != hipSuccess)
        return fail(MOEDEC_ERR_LAUNCH, "self-test: workspace clear failed");
    int st;
    if ((st = moe_pack_gateup_mxfp4(d + L.gate_c, d + L.gate_s, d + L.up_c, d + L.up_s, kStE, kStH, kStI,
                                    d + L.gu_c, d + L.gu_s, stream)) ||
        (st = moe_pack_gateup_mxfp4(d + L.sgate_c, d + L.sgate_s, d + L.sup_c, d + L.sup_s, 1, kStH, kStI,
                                    d + L.sgu_c, d + L.sgu_s, stream)) ||
        (st = moe_pack_down_mxfp4(d + L.down_c, d + L.down_s, kStE, kStH, kStI, d + L.dn_c, d + L.dn_s, stream)) ||
        (st = moe_pack_down_mxfp4(d + L.sdown_c, d + L.sdown_s, 1, kStH, kStI, d + L.sdn_c, d + L.sdn_s, stream)))
        return st;
    moedec_moe_weights w{MOEDEC_MOE_MAGIC, kStE, kStH, kStI, d + L.gu_c, d + L.gu_s, d + L.dn_c, d + L.dn_s,
                         d + L.sgu_c, d + L.sgu_s, d + L.sdn_c, d + L.sdn_s};
    if ((st = moe_layer_mxfp4(&w, reinterpret_cast<uint16_t*>(d + L.x), reinterpret_cast<float*>(d + L.logits), 1,
                              kStK, reinterpret_cast<int32_t*>(d + L.ids), reinterpret_cast<float*>(d + L.w),
                              reinterpret_cast<moedec_dispatch*>(d + L.disp), reinterpret_cast<uint16_t*>(d + L.y),
                              reinterpret_cast<float*>(d + L.y32), d + L.ws,
                              moedec::ffn_layout(1, kStK, kStH, kStI).total, stream)))
        return st;
    moedec_lmhead_fp8 head{};
    if ((st = lmhead_quant_fp8(reinterpret_cast<uint16_t*>(d + L.lw), kStV, kStHv, d + L.lcodes,
                               reinterpret_cast<float*>(d + L.lscale), &head, stream)) ||
        (st = lmhead_gemv_fp8_argmax(&head, reinterpret_cast<uint16_t*>(d + L.lx), 1,
                                     reinterpret_cast<float*>(d + L.llogits), reinterpret_cast<int32_t*>(d + L.lid),
                                     d + L.lws, moedec::lmhead_epilogue_bytes(kStV, 1), stream)))
        return st;
    int32_t ids[kStK], lid = -1;
    float wts[kStK], y32[kStH], lsc[kStV], llg[kStV];
    uint16_t yb[kStH];
    uint8_t codes[kStV * kStHv];
    struct Back { void* p; size_t at; size_t n; } backs[] = {
        {ids, L.ids, sizeof(ids)}, {wts, L.w, sizeof(wts)}, {y32, L.y32, sizeof(y32)}, {yb, L.y, sizeof(yb)},
        {codes, L.lcodes, sizeof(codes)}, {lsc, L.lscale, sizeof(lsc)}, {llg, L.llogits, sizeof(llg)},
        {&lid, L.lid, sizeof(lid)}};
    for (const Back& b : backs)
        if (hipMemcpyAsync(b.p, d + b.at, b.n, hipMemcpyDeviceToHost, s) != hipSuccess)
            return fail(MOEDEC_ERR_LAUNCH, "self-test: copy back failed");
    if (hipStreamSynchronize(s) != hipSuccess) return fail(MOEDEC_ERR_LAUNCH, "self-test: stream failed");
    if (ids[0] != 0 || ids[1] != 2 || wts[0] != 0.5f || wts[1] != 0.5f)
        return fail(MOEDEC_ERR_SELFTEST, "self-test routing: ids {%d, %d} weights {%g, %g}, want {0, 2} {0.5, 0.5}",
                    ids[0], ids[1], (double)wts[0], (double)wts[1]);
    const double want = 2.0 / (1.0 + std::exp(-1.0));
    for (int r = 0; r < kStH; ++r) {
        if (!(std::fabs(y32[r] - want) <= 1e-5 * want))
            return fail(MOEDEC_ERR_SELFTEST, "self-test MoE layer: y[%d] = %.9g, want %.9g", r, (double)y32[r], want);
        if (!(std::fabs((double)st_bf16_to_f32(yb[r]) - y32[r]) <= std::ldexp(1.0, -8) * want))
            return fail(MOEDEC_ERR_SELFTEST, "self-test MoE layer: bf16 y[%d] does not round y_f32", r);
    }
    const uint8_t want_c0[5] = {0x7E, 0xC0, 0x38, 0x30, 0x00};
    for (int j = 0; j < kStHv; ++j) {
        if (codes[j] != want_c0[j < 4 ? j : 4] || codes[kStHv + j] != 0x7E)
            return fail(MOEDEC_ERR_SELFTEST, "self-test FP8 codes: column %d {0x%02x, 0x%02x}", j, codes[j],
                        codes[kStHv + j]);
    }
    if (lsc[0] != 1.0f || llg[0] != -2.0f || !(std::fabs(llg[1] - 0.25) <= 1e-6) || lid != 1)
        return fail(MOEDEC_ERR_SELFTEST, "self-test FP8 head: scale %g, logits {%g, %g}, token %d",
                    (double)lsc[0], (double)llg[0], (double)llg[1], lid);
    g_last_error[0] = '\0';
    return MOEDEC_OK;
}

}  // extern "C"
