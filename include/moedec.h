/*
 * moedec.h -- C ABI of libmoedec: batch-1 MoE decode with MXFP4 experts and
 * an FP8 LM head, hand-written HIP kernels for gfx950 (MI355X).
 *
 * Sources cited below
 *   [news] yoususu.cn/post/959 -- news article on NVIDIA's software-only DGX
 *          Spark decode speed-up (section "where the speed comes from").
 *   [ic]   ic.work article on DGX Spark running Ling-3.0-flash (section "three
 *          scalpels": 512 routed + 1 shared expert, MXFP4 routed experts,
 *          157K vocabulary).
 *   [card] ai.cheesepanini.fun knowledge card "three ways to boost MoE
 *          inference on DGX Spark" (background; method points #1 MoE kernel,
 *          #2 FP8 LM head, #3 4-token verify window).
 *   [MX]   OCP Microscaling Formats (MX) v1.0; [OFP8] OCP 8-bit Floating
 *          Point rev 1.0.
 *
 * Conventions for every call
 *   - All pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer; the library never allocates or frees device memory (the
 *     one array it holds is the scratch of moe_layer_mxfp4_noalloc, part of
 *     the library image).
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = null stream) and the
 *     call returns without waiting (moedec_selftest and
 *     moe_ffn_workspace_status are the two calls that wait for the stream).  The return value reports host-side
 *     argument checks and launch errors only; a fault inside a kernel shows
 *     up at the caller's next synchronisation.
 *   - On a non-zero return nothing was enqueued, and moedec_last_error()
 *     holds a message for the calling thread.
 *   - bf16 values are passed as uint16 bit patterns.
 *   - The library holds no state between calls other than a per-device
 *     check that the device is gfx950; calls are thread-safe.  Calls that
 *     share one workspace must be ordered (same stream or synchronised).
 */
#ifndef MOEDEC_H
#define MOEDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEDEC_ABI_VERSION 1

typedef void* moedec_stream_t;

/* Status codes. */
#define MOEDEC_OK             0
#define MOEDEC_ERR_NULL      -1   /* a required pointer is NULL */
#define MOEDEC_ERR_ALIGN     -2   /* a pointer is not aligned as documented */
#define MOEDEC_ERR_SHAPE     -3   /* a size is outside the supported range */
#define MOEDEC_ERR_FORMAT    -4   /* a descriptor's magic/format tag is wrong */
#define MOEDEC_ERR_WORKSPACE -5   /* workspace smaller than required */
#define MOEDEC_ERR_LAUNCH    -6   /* the HIP runtime rejected a launch */
#define MOEDEC_ERR_DEVICE    -7   /* the current device is not a gfx950 GPU */
#define MOEDEC_ERR_SELFTEST  -8   /* moedec_selftest: a result differs from its closed form */
#define MOEDEC_ERR_TIMEOUT   -9   /* moe_ffn_workspace_status: a cross-block wait gave up */
#define MOEDEC_ERR_ARG      -10   /* a scalar argument is outside its range (sampling settings) */

/* Limits. */
#define MOEDEC_MAX_M      4       /* tokens per call: 1, or the 4-token verify window [card #3] */
#define MOEDEC_MAX_K      32      /* experts chosen per token */
#define MOEDEC_MAX_E      1024    /* routed experts per layer */
#define MOEDEC_MAX_SLOTS  (MOEDEC_MAX_M * MOEDEC_MAX_K + 1)

int moedec_abi_version(void);
const char* moedec_status_string(int status);   /* static text, never NULL */
const char* moedec_last_error(void);            /* thread-local; "" when none */

/* ------------------------------------------------------------------------
 * Routing.  [card background; news: 8 of 512 routed experts per token;
 * card #3: a 4-token verify touches up to 32 experts]
 *
 * Per token m: the k experts with the largest float32 logits, ordered by
 * (logit descending, expert index ascending), +0.0 and -0.0 equal; weights
 * are the softmax over all E logits renormalised over the k chosen ones.
 * The dispatch table groups the tokens by expert so that each active expert's
 * weights are read once per call whatever the number of tokens using it.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t  n_slots;                              /* distinct routed experts + 1 */
    int32_t  M;                                    /* tokens */
    int32_t  expert[MOEDEC_MAX_SLOTS];             /* ascending ids, then E (= shared) */
    uint32_t token_mask[MOEDEC_MAX_SLOTS];         /* bit m: token m uses the slot */
    float    weight[MOEDEC_MAX_SLOTS][MOEDEC_MAX_M]; /* 0 where the token does not */
} moedec_dispatch;                                 /* entries >= n_slots are zero */

/*
 * logits     [M][E] float32, 4-byte aligned, finite (NaN is outside the domain)
 * topk_ids   [M][k] int32   (may be NULL)
 * topk_w     [M][k] float32 (may be NULL)
 * dispatch   one moedec_dispatch in device memory (may be NULL; at least one
 *            of the three outputs must be given), 16-byte aligned
 * 1 <= M <= 4, 1 <= E <= 1024, 1 <= k <= min(E, 32).
 */
int moe_route_topk(const float* logits, int M, int E, int k,
                   int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch,
                   moedec_stream_t stream);

/*
 * Router logits, the step before routing [card background: the router picks
 * 8 of the 512 routed experts of each layer from the token's hidden state]:
 * logits[m][e] = sum_k x[m][k] * W_router[e][k], bf16 inputs, float32
 * accumulation and output (no bias).  The same GEMV as lmhead_gemv_bf16 with
 * the expert count in place of the vocabulary, launched for a short matrix.
 * w_router [E][H] bf16, 16-byte aligned; x_bf16 [M][H], 4-byte aligned;
 * logits [M][E] float32, 4-byte aligned (moe_route_topk's input).
 * 1 <= M <= 4, 1 <= E <= 1024, 8 <= H <= 4096, H % 8 == 0.
 */
int moe_router_logits_bf16(const uint16_t* w_router, int E, int H, const uint16_t* x_bf16, int M,
                           float* logits, moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * MXFP4 expert weights.  [ic three scalpels: routed experts are MXFP4;
 * MX §5: 32 E2M1 codes share one E8M0 scale]
 *
 * Canonical layout of an N x K MXFP4 matrix: codes [N][K/2] bytes, low nibble
 * = even k; scales [N][K/32] bytes.  Experts are stacked along a leading axis.
 *
 * The FFN kernel reads a packed layout in which one 64-lane wave fetches one
 * contiguous 1 KiB chunk per load step and lane l holds the 16 code bytes (one
 * MX block) of row 16u + (l & 15), MX block 4c + (l >> 4).  Per expert, with
 * KBH4 = ceil(H/32 / 4) and KBI4 = ceil(I/32 / 4):
 *   gate/up, unit u = rows 16u..16u+15 of both W_gate and W_up:
 *     codes  [I/16][KBH4][2][64][16]   half 0 = gate rows, half 1 = the same up rows
 *     scales [I/16][KBH4][64] u16      low byte = gate scale, high byte = up scale
 *   down, unit u = output rows 16u..16u+15:
 *     codes  [H/16][KBI4][64][16]
 *     scales [H/16][KBI4][64] u8
 * MX blocks past the end of a row (block count not a multiple of four) are
 * zero codes with scale 127.  The packing is a byte permutation plus that
 * padding; it is done once, by the two calls below.
 * ---------------------------------------------------------------------- */
typedef struct {
    size_t gu_codes, gu_scales, dn_codes, dn_scales;   /* bytes per expert */
} moedec_mxfp4_sizes;

/* Per-expert packed sizes; returns MOEDEC_ERR_SHAPE unless H % 64 == 0,
 * I % 32 == 0, 64 <= H <= 4096, 32 <= I <= 2048.  `out` is host memory. */
int moedec_mxfp4_packed_sizes(int H, int I, moedec_mxfp4_sizes* out);

/* gate, up: canonical [n_experts][I][H/2] codes, [n_experts][I][H/32] scales.
 * Output: n_experts consecutive packed experts.  Code pointers 16-byte
 * aligned, the gate/up scale output 2-byte aligned. */
int moe_pack_gateup_mxfp4(const uint8_t* gate_codes, const uint8_t* gate_scales,
                          const uint8_t* up_codes, const uint8_t* up_scales,
                          int n_experts, int H, int I,
                          uint8_t* gu_codes, uint8_t* gu_scales, moedec_stream_t stream);

/* down: canonical [n_experts][H][I/2] codes, [n_experts][H][I/32] scales. */
int moe_pack_down_mxfp4(const uint8_t* down_codes, const uint8_t* down_scales,
                        int n_experts, int H, int I,
                        uint8_t* dn_codes, uint8_t* dn_scales, moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * The shared expert in FP8.  [ic three scalpels: the shared projections keep
 * a higher-precision format than the MXFP4 routed experts; card #2 and news
 * where the speed comes from: an FP8 copy built when the model is loaded
 * halves what bf16 weights cost to read]  Each of W_gate, W_up [I][H] and
 * W_down [H][I] (bf16) is quantised per output row as the LM head is: s =
 * absmax / 448 (1 for an all-zero row), code = E4M3 nearest-even,
 * saturating, of fl32(w / s).  Layout (16-byte lanes of 16 codes):
 *     gate/up codes [I/16][KH8][2][64][16]: unit rg, chunk c, half (0 gate,
 *              1 up), lane l = row 16rg + (l & 15), k = 64c + 16(l >> 4) + b
 *     down codes    [H/16][KI8][64][16]:    row block rb, chunk c, lane l =
 *              row 16rb + (l & 15), k = 64c + 16(l >> 4) + b
 *     scales   gate/up: float32 [2][I] (gate rows, then up rows); down:
 *              float32 [H]
 * KH8 = 2 * KBH4, KI8 = 2 * KBI4 (as above); codes past H or I are zero.
 * The shapes are those of moedec_mxfp4_packed_sizes.
 * ---------------------------------------------------------------------- */
int moedec_shared_fp8_packed_sizes(int H, int I, moedec_mxfp4_sizes* out);

/* Quantise and pack once.  gate_bf16, up_bf16 [I][H] and down_bf16 [H][I]
 * row-major bf16; codes 16-byte aligned, scales 4-byte aligned.  Two launches
 * on `stream` (the row scales, then the codes). */
int moe_pack_shared_fp8(const uint16_t* gate_bf16, const uint16_t* up_bf16, const uint16_t* down_bf16,
                        int H, int I, uint8_t* gu_codes, float* gu_scales, uint8_t* dn_codes,
                        float* dn_scales, moedec_stream_t stream);

#define MOEDEC_MOE_MAGIC 0x4D4F4534u             /* "MOE4": every expert MXFP4 */
#define MOEDEC_MOE_MAGIC_SHARED_FP8 0x4D4F4538u  /* "MOE8": routed MXFP4, shared FP8 */

/* Packed weights of one MoE layer.  Routed expert e starts at e * (per-expert
 * size) in each routed array; the shared expert has its own pointers, in the
 * MXFP4 layout (MOEDEC_MOE_MAGIC) or in the FP8 layout of
 * moe_pack_shared_fp8 (MOEDEC_MOE_MAGIC_SHARED_FP8: sh_gu_scales and
 * sh_dn_scales then point to the float32 row scales, 4-byte aligned).  The
 * fused layer calls take both; moe_expert_ffn_mxfp4 takes the first only
 * (MOEDEC_ERR_FORMAT). */
typedef struct {
    uint32_t magic;                    /* MOEDEC_MOE_MAGIC or MOEDEC_MOE_MAGIC_SHARED_FP8 */
    int32_t  E, H, I;
    const uint8_t* gu_codes;           /* [E] packed gate/up codes (16-byte aligned) */
    const uint8_t* gu_scales;          /* [E] packed gate/up scales (2-byte aligned) */
    const uint8_t* dn_codes;           /* [E] packed down codes */
    const uint8_t* dn_scales;          /* [E] packed down scales */
    const uint8_t* sh_gu_codes;        /* shared expert, same per-expert layout */
    const uint8_t* sh_gu_scales;
    const uint8_t* sh_dn_codes;
    const uint8_t* sh_dn_scales;
} moedec_moe_weights;                  /* host struct (pointers inside are device) */

/* ------------------------------------------------------------------------
 * Routed + shared SwiGLU expert FFN.  [card #1: MXFP4 MoE kernel, expert
 * intermediate 768; ic three scalpels: 512 routed + 1 shared expert]
 *
 * For each token m: y[m] = sum over slots s using m of
 *     weight[s][m] * W_down[e] (silu(W_gate[e] x[m]) * (W_up[e] x[m]))
 * (the shared slot has weight 1), E2M1 x E8M0 weights, bf16 x, float32
 * accumulation, h kept in float32, y rounded once to bf16 (nearest even).
 *
 * w           host pointer to the layer's packed weights
 * x_bf16      [M][H] bf16, 16-byte aligned
 * dispatch    from moe_route_topk for the same M (and k <= k_max)
 * k_max       the k used for routing (sizes the launch; 1..32)
 * y_bf16      [M][H] bf16 output, 4-byte aligned
 * y_f32       [M][H] float32 output or NULL
 * workspace   >= moe_ffn_workspace_bytes(M, k_max, H, I) bytes, 16-byte
 *             aligned, ZERO-FILLED ONCE before its first use; every call
 *             leaves it ready for the next (its counters are reset by the
 *             kernel).  Calls sharing it must not overlap.
 * One kernel launch: gate/up, SiLU*mul, down, the weighted combine and the
 * rounding are fused.  Shapes: 64 <= H <= 4096, H % 64 == 0; 32 <= I <= 2048,
 * I % 32 == 0; 1 <= E <= 1024.
 * Values outside the formats' domain (E8M0 code 0 or 255, NaN) give
 * undefined results.
 */
size_t moe_ffn_workspace_bytes(int M, int k_max, int H, int I);

/* Where an FFN / fused-layer call leaves each (slot, token)'s h in its
 * workspace, for inspecting a finished call (stream synchronised): h_words
 * is the byte offset of [M * k_max + 1][M][I] 64-bit words, slot-major: slot
 * 0 the shared expert, slot s >= 1 the routed entry s - 1 of the call's
 * dispatch table (the table's valid entries in its order); the low 32
 * bits of a word are the float32 h = silu(g) * u (before any MXFP8 rounding),
 * valid for the tokens in the slot's token mask.  Same argument ranges as
 * moe_ffn_workspace_bytes; returns MOEDEC_OK, or MOEDEC_ERR_NULL /
 * MOEDEC_ERR_SHAPE with *out untouched.
 */
typedef struct moedec_ffn_layout {
    uint64_t total_bytes;
    uint64_t h_words;
    int32_t max_slots, M;
} moedec_ffn_layout;

int moe_ffn_workspace_layout(int M, int k_max, int H, int I, moedec_ffn_layout* out);

int moe_expert_ffn_mxfp4(const moedec_moe_weights* w, const uint16_t* x_bf16, int M,
                         const moedec_dispatch* dispatch, int k_max,
                         uint16_t* y_bf16, float* y_f32,
                         void* workspace, size_t workspace_bytes,
                         moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * Fused MoE layer: moe_route_topk followed by moe_expert_ffn_mxfp4 in ONE
 * kernel launch (same results).  [card background and #1, #3; news where the
 * speed comes from]  Each block of the launch selects the top-k experts of
 * every token from the logits itself, so the FFN starts without waiting for
 * a separate routing launch.
 *
 * logits      [M][E] float32 (E = w->E), 4-byte aligned
 * k           experts per token, 1 <= k <= min(E, 32)
 * topk_ids, topk_w, dispatch   optional outputs (NULL to skip), identical to
 *             what moe_route_topk writes for the same logits
 * workspace   >= moe_ffn_workspace_bytes(M, k, H, I), as for
 *             moe_expert_ffn_mxfp4 (the two calls may share one workspace)
 * Other arguments and limits as moe_expert_ffn_mxfp4.
 * Both FFN calls run a grid whose blocks must be resident together (one
 * block per work unit at four blocks per CU for one token when the units fit,
 * otherwise three blocks per CU); they wait (boundedly) for each other's
 * blocks, so do not run them concurrently with another kernel that holds most
 * of the GPU.  The launch is refused (MOEDEC_ERR_LAUNCH) if the device cannot
 * hold that many blocks per CU.
 */
int moe_layer_mxfp4(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits,
                    int M, int k, int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch,
                    uint16_t* y_bf16, float* y_f32, void* workspace, size_t workspace_bytes,
                    moedec_stream_t stream);

/* The fused layer with 8-bit activations (W4A8), M = 1..4.  [news
 * "boundary": the measured baseline serves the model in its W4A8
 * configuration; MX Specification v1.0 §5.2 and §6.3: MXFP8 = E4M3 elements
 * sharing one E8M0 scale per 32 values]
 *
 * As moe_layer_mxfp4 with both products taking MXFP8 activations along their
 * reduction axis: x_q = MXFP8(x) per token over H, h = silu(W_gate x_q) *
 * (W_up x_q), h_q = MXFP8(h) per (token, expert) over I, y = sum_j w_j W_down
 * h_q_j + W_down,s h_q_s.  Scale and rounding as moe_layer_mxfp4_prefill_a8.
 * Each block quantises the values it reads (x as it stages it, h as it
 * stages a pair's h), so the products see exactly the MXFP8 values; the
 * weights' bytes, which bound the layer at these token counts, are the same.
 * Domain: blocks of x whose largest magnitude is 0 or at least 2^-110 (below
 * that an MXFP8 value may be a bf16 subnormal).  An FP8 shared-expert
 * descriptor is refused (MOEDEC_ERR_FORMAT).  Arguments, workspace and errors
 * as moe_layer_mxfp4.
 */
int moe_layer_mxfp4_a8(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits,
                       int M, int k, int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch,
                       uint16_t* y_bf16, float* y_f32, void* workspace, size_t workspace_bytes,
                       moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * Health of an FFN workspace.  The FFN calls above (and the residual-stream
 * call below) run blocks that wait for one another across CUs; every such
 * wait is bounded, and one that gives up -- possible only when the blocks of
 * a launch are not all resident together, e.g. beside another kernel that
 * holds most of the GPU -- records it in a status word of the workspace and
 * lets the kernel finish, so the launch returns with WRONG results and its
 * call had returned MOEDEC_OK.  This call waits for `stream`, reads that word
 * and reports it:
 *   MOEDEC_OK           no wait gave up in any call on this workspace since
 *                       the last check;
 *   MOEDEC_ERR_TIMEOUT  at least one did: the results of those calls are
 *                       invalid.  The workspace is zero-filled again before
 *                       the call returns, so it can be used right away.
 * workspace        the workspace, or NULL for the current device's scratch
 *                  of moe_layer_mxfp4_noalloc (workspace_bytes then ignored)
 * workspace_bytes  its size in bytes
 * flags_out        host, may be NULL: the raw status word (0 when clear)
 * Like moedec_selftest, this call waits for the stream.
 * ---------------------------------------------------------------------- */
int moe_ffn_workspace_status(void* workspace, size_t workspace_bytes, uint32_t* flags_out,
                             moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_layer_mxfp4 without a caller workspace, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  Same arguments and results as moe_layer_mxfp4
 * minus the workspace, and the same kernels: the workspace is a file-scope
 * device array of 4 MiB (every GPU the library runs on holds its own copy
 * until the process ends), looked up and zero-filled on the first call on a
 * device.  Nothing is allocated by this call, ever.
 *   - Sizes whose workspace (moe_ffn_workspace_bytes(M, k, H, I)) exceeds
 *     4 MiB are refused with MOEDEC_ERR_WORKSPACE; a Ling-shaped layer
 *     (H 2560, I 768, k 8) needs 1.6 MB at M = 4.
 *   - All calls on one GPU share the array: calls that overlap in time on
 *     one GPU (two streams, two threads) race and give wrong results.
 *     Order them on one stream.
 *   - moe_ffn_workspace_status(NULL, 0, ...) checks and clears its status.
 * ---------------------------------------------------------------------- */
int moe_layer_mxfp4_noalloc(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits,
                            int M, int k, int32_t* topk_ids, float* topk_w, moedec_dispatch* dispatch,
                            uint16_t* y_bf16, float* y_f32, moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * One MoE layer of a decode stack, on the residual stream.  The model the
 * pages measure stacks 42 such layers [card background]; between layers a
 * residual stream carries the sum of the layer outputs.  This call forms the
 * layer input from that stream and adds the layer output back, in the same
 * single launch as moe_layer_mxfp4:
 *     x     = bf16(RMSNorm(r_in)),  RMSNorm(r) = r / sqrt(mean(r^2) + eps)
 *             per token, unit gain, float32, rounded to nearest even
 *     y     = the MoE layer of moe_layer_mxfp4 applied to x
 *     r_out = r_in + y                                  (float32)
 * (The norm's form and its unit gain are a reading: the pages give no
 * formula for it, and its trained gains are weights this path does not have.)
 *
 * r_in        [M][H] float32, 16-byte aligned
 * r_out       [M][H] float32, 16-byte aligned; must not overlap r_in
 * eps         0 <= eps <= 1
 * x_bf16      [M][H] bf16 output (the normalised layer input) or NULL,
 *             16-byte aligned
 * y_f32       [M][H] float32 layer output or NULL
 * Other arguments, limits and the workspace as moe_layer_mxfp4.
 */
int moe_layer_rmsnorm_mxfp4(const moedec_moe_weights* w, const float* r_in, const float* logits,
                            int M, int k, float eps, float* r_out, uint16_t* x_bf16, float* y_f32,
                            void* workspace, size_t workspace_bytes, moedec_stream_t stream);

/*
 * The same layer with its router in front [card background: a router picks
 * 8 of the 512 experts for each token from its hidden state]: from the
 * residual stream alone,
 *     x      = bf16(RMSNorm(r_in))                      (as above)
 *     logits = x W_router^T                             (float32, no bias)
 *     then moe_layer_rmsnorm_mxfp4 on those logits: top-k routing, the
 *     routed + shared experts, r_out = r_in + y.
 * Two launches on `stream`: the norm and the router GEMV (one router row per
 * wave; every block forms x from r_in in the fused layer's summation order,
 * so both launches use the same x bit for bit), then the fused layer.
 * w_router    [E][H] bf16 (E = w->E, H = w->H), row-major, 16-byte aligned
 * logits      [M][E] float32 output (the second launch reads it), 4-byte
 *             aligned
 * Other arguments, limits and the workspace as moe_layer_rmsnorm_mxfp4.  If
 * the second launch is refused (MOEDEC_ERR_LAUNCH), the first has already
 * been enqueued and writes logits.
 */
int moe_layer_rmsnorm_router_mxfp4(const moedec_moe_weights* w, const uint16_t* w_router, const float* r_in,
                                   int M, int k, float eps, float* logits, float* r_out, uint16_t* x_bf16,
                                   float* y_f32, void* workspace, size_t workspace_bytes,
                                   moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * Many tokens at once: a prefill chunk or a long verify window.  [news "two
 * easily missed details": filling a long prompt is bound by matrix
 * arithmetic, decoding by bandwidth; card #3: each active expert is read once
 * for every token that chose it]
 *
 * The same layer as moe_layer_mxfp4 for T tokens,
 *     y[t] = sum_j w[t][j] FFN_{ids[t][j]}(x[t]) + FFN_shared(x[t]),
 * computed as a grouped GEMM on bf16 matrix cores: routing with per-expert
 * token counts, one token list per expert (the shared expert's list holds all
 * T), then gate/up, down and a combine.  The MXFP4 weights are used in the
 * packed layout above (the same buffers the decode calls read), dequantised
 * exactly to bf16 in registers; x is bf16; products accumulate in float32.
 * h = silu(g) * u is carried into the down product as the sum of two bf16
 * values (hi = bf16(h), lo = bf16(h - hi)), 16 significant bits, relative
 * error at most 2^-17 per element.  Each token's terms are added in float32 in
 * the order j = 0 .. k-1 then the shared expert, and rounded once to bf16.
 * Results do not depend on scheduling: every output is formed from its own
 * row and column only, in a fixed order.
 *
 * Seven launches on `stream`: routing, per-chunk expert counts, plan (one
 * block: the scans of the counts and the tile list), scatter, gate/up, down,
 * combine.
 * w             MOEDEC_MOE_MAGIC weights (an FP8 shared expert is refused
 *               with MOEDEC_ERR_FORMAT); the four scale arrays 4-byte
 *               aligned (they are read as 32-bit words)
 * x_bf16        [T][H] bf16, 16-byte aligned
 * logits        [T][E] float32 router logits, 4-byte aligned
 * T             1 .. MOEDEC_MAX_PREFILL_T tokens
 * k             1 .. min(E, MOEDEC_MAX_K)
 * topk_ids      [T][k] int32 output (selection order) or NULL
 * topk_w        [T][k] float32 output or NULL
 * group_counts  [E + 1] int32 output or NULL: tokens of each routed expert,
 *               then T for the shared expert
 * y_bf16        [T][H] bf16 output, 8-byte aligned
 * y_f32         [T][H] float32 output before rounding, or NULL; 16-byte
 *               aligned
 * workspace     moe_prefill_workspace_bytes(T, E, k, H, I) bytes, 256-byte
 *               aligned, owned by the caller; no initial contents needed.
 *               About T*(k+1)*(4H + 4I) + T*H bytes: the per-pair h and down
 *               outputs, and the W4A8 call's 8-bit x.  One call at a time per
 *               workspace.
 * Returns MOEDEC_OK, or an error code with nothing enqueued.
 */
#define MOEDEC_MAX_PREFILL_T 65536

size_t moe_prefill_workspace_bytes(int T, int E, int k, int H, int I);

int moe_layer_mxfp4_prefill(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int T,
                            int k, int32_t* topk_ids, float* topk_w, int32_t* group_counts, uint16_t* y_bf16,
                            float* y_f32, void* workspace, size_t workspace_bytes, moedec_stream_t stream);

/* The same layer with 8-bit activations (W4A8).  [news "boundary": the
 * measured baseline serves the model in its W4A8 configuration; MX
 * Specification v1.0 §5.2 and §6.3: MXFP8 = E4M3 elements sharing one E8M0
 * scale per 32 values]
 *
 * Both products take MXFP8 activations along their reduction axis and the
 * MXFP4 weights as stored, on the block-scaled fp4 x fp8 matrix instruction
 * (products of the scaled values are exact; they accumulate in float32):
 *     x_q = MXFP8(x) per token over H, h = silu(W_gate x_q) * (W_up x_q),
 *     h_q = MXFP8(h) per (token, expert) over I, y_pair = W_down h_q,
 * then the combine of moe_layer_mxfp4_prefill.  A block's scale is
 * 2^(floor(log2 max|v|) - 8), 2^-127 for an all-zero block; each element is
 * v / scale rounded to the nearest E4M3 value, ties to even, saturating at
 * +-448.  Seven launches, as above; the routing launch also quantises x.
 * Arguments, alignment, errors and workspace (moe_prefill_workspace_bytes,
 * the same size) as for moe_layer_mxfp4_prefill.
 */
int moe_layer_mxfp4_prefill_a8(const moedec_moe_weights* w, const uint16_t* x_bf16, const float* logits, int T,
                               int k, int32_t* topk_ids, float* topk_w, int32_t* group_counts, uint16_t* y_bf16,
                               float* y_f32, void* workspace, size_t workspace_bytes, moedec_stream_t stream);

/* Where the many-token calls leave their intermediates in the workspace, as
 * byte offsets from its start; for inspecting a call after it has finished
 * (the stream synchronised).  P = T*(k+1) (token, expert) pairs.
 *   pos       int32 [T][k]: pair row of token t's choice j; the shared
 *             expert's row of token t is T*k + t
 *   y_pair    float32 [P][H]: each pair's down output
 *   x_codes   uint8 [T][H], x_scales uint8 [T][x_scale_stride]: MXFP8 x
 *             (W4A8 call only; scale bytes past H/32 are padding)
 *   h_codes   uint8 [P][I], h_scales uint8 [P][h_scale_stride]: MXFP8 h
 *             (W4A8 call only; scale bytes past I/32 are not written)
 * Same argument ranges as moe_prefill_workspace_bytes; returns MOEDEC_OK or
 * MOEDEC_ERR_NULL / MOEDEC_ERR_SHAPE with *out untouched.
 */
typedef struct moedec_prefill_layout {
    uint64_t total_bytes;
    uint64_t pos, y_pair, x_codes, x_scales, h_codes, h_scales;
    int32_t x_scale_stride, h_scale_stride;
} moedec_prefill_layout;

int moe_prefill_workspace_layout(int T, int E, int k, int H, int I, moedec_prefill_layout* out);

/* ------------------------------------------------------------------------
 * LM head with online FP8 weights.  [news where the speed comes from; card
 * #2: the 157,184 x 2,560 vocabulary projection is read whole for every
 * token; a dynamic FP8 config applied when the head is built halves that
 * read; the draft must share the whole head object, not the raw weight
 * tensor, or FP8 bytes get read as bf16 -- hence the typed descriptor]
 * ---------------------------------------------------------------------- */
#define MOEDEC_LMHEAD_MAGIC 0x4C4D4838u         /* "LMH8" */
#define MOEDEC_FMT_E4M3FN_ROWSCALE_F32 1u       /* OCP E4M3, one float32 scale per row */
/* The same weights with dynamic FP8 activations [card #2: the head gets a
 * dynamic FP8 configuration]: every GEMV call quantises each token row of x
 * with the weights' rule, t_m = max_k |x[m][k]| / 448 (float32 division, 1
 * for a zero row), p = E4M3 nearest-even, saturating, of x / t_m, and
 * computes logits[m][v] = s_v * t_m * sum_k e4m3(p[m][k]) * e4m3(codes[v][k])
 * in float32.  Set desc.format to it after lmhead_quant_fp8; the GEMV, greedy
 * and sampling calls all take it.  Reads the same bytes as the weight-only
 * head (x is a few KiB). */
#define MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT 2u

typedef struct {
    uint32_t magic;                    /* MOEDEC_LMHEAD_MAGIC */
    uint32_t format;                   /* MOEDEC_FMT_E4M3FN_ROWSCALE_F32 or ..._DYNACT */
    int32_t  V, H;
    const uint8_t* codes;              /* [V][H] E4M3 codes, row-major, 16-byte aligned */
    const float* row_scale;            /* [V] */
} moedec_lmhead_fp8;                   /* host struct (pointers inside are device) */

/*
 * Quantise once: a_v = max|W[v,:]|, s_v = a_v / 448 (float32 division, 1 when
 * a_v = 0), codes = E4M3 nearest-even, saturating to +-448, of W / s_v
 * (float32 division).  w_bf16 [V][H] 16-byte aligned; codes [V][H] 16-byte
 * aligned; row_scale [V].  out_desc (host, may be NULL) is filled to describe
 * codes/row_scale.  1 <= V, 16 <= H <= 8192, H % 16 == 0.
 */
int lmhead_quant_fp8(const uint16_t* w_bf16, int V, int H,
                     uint8_t* codes, float* row_scale,
                     moedec_lmhead_fp8* out_desc, moedec_stream_t stream);

/*
 * logits[m][v] = s_v * sum_k x[m][k] * e4m3(codes[v][k]), float32 accumulation.
 * head (host) must carry the LM-head magic and an E4M3 format tag, else
 * MOEDEC_ERR_FORMAT; with MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT the
 * activations are quantised per token first (see there).  x_bf16 [M][H] 4-byte aligned; logits [M][V] float32.
 * 1 <= M <= 4, H % 16 == 0, H <= 4096.
 */
int lmhead_gemv_fp8(const moedec_lmhead_fp8* head, const uint16_t* x_bf16, int M,
                    float* logits, moedec_stream_t stream);

/*
 * Greedy decode on the FP8 head [card results: the measured decode samples
 * the next token from these logits with temperature 0.6, top-p 0.95, top-k 29;
 * greedy choice is the temperature-0 case]: the GEMV of lmhead_gemv_fp8 and
 * token_ids[m] = the row v of the largest logits[m][v], the lowest such row
 * on ties (+0.0 and -0.0 are equal), without a pass over the logits: each
 * block publishes the best (logit, row) of its rows, and the block launched
 * last waits for the others' and picks among them.  One launch on `stream`.
 * V <= MOEDEC_MAX_EPILOGUE_V, else MOEDEC_ERR_SHAPE.
 * logits      [M][V] float32, optional (NULL: not written)
 * token_ids   [M] int32, 4-byte aligned.  -1 means the polling block gave up
 *             waiting for another block's words (not expected on a working
 *             device; the call's tokens are then invalid).
 * workspace   >= lmhead_argmax_workspace_bytes(V, M) bytes, 8-byte aligned,
 *             ZERO-FILLED ONCE before its first use; every call leaves it
 *             ready for the next (launch counts, then words tagged with
 *             them).  One workspace serves one head (one V); calls sharing
 *             it must not overlap.  Layout: 8 KiB of per-block launch
 *             counts, then per token 2,048 block-key slots, 8,192 wave-key
 *             slots and V row-key slots of 8 bytes (the last two written by
 *             the sampling call).
 * Other arguments and limits as lmhead_gemv_fp8.
 */
#define MOEDEC_MAX_EPILOGUE_V (1 << 18)
size_t lmhead_argmax_workspace_bytes(int V, int M);   /* 0 for sizes out of range */
int lmhead_gemv_fp8_argmax(const moedec_lmhead_fp8* head, const uint16_t* x_bf16, int M, float* logits,
                           int32_t* token_ids, void* workspace, size_t workspace_bytes,
                           moedec_stream_t stream);

/*
 * Sampled decode on the FP8 head [card results: temperature 0.6, top-p 0.95,
 * top-k 29 in the measured decode]: the GEMV of lmhead_gemv_fp8, then per
 * token m
 *   - candidates: the top_k largest logits[m][v], ordered by (logit desc, row
 *     asc);
 *   - p_i = softmax(logit_i / temperature) over the candidates (float32);
 *   - the nucleus: the shortest prefix of the candidates whose cumulative
 *     probability reaches top_p;
 *   - token_ids[m] = the first nucleus entry whose cumulative probability,
 *     renormalised over the nucleus, exceeds u[m].
 * Every wave publishes its rows' (logit, row) keys in the workspace; the block
 * launched last selects the candidates exactly (radix selects over the
 * block maxima, the waves of the top_k blocks, then the rows of the top_k
 * waves) and draws.
 * top_k = 1 gives the greedy token.  One launch on `stream`.
 * temperature > 0 and finite; 0 < top_p <= 1; 1 <= top_k <= min(32, V), else
 * MOEDEC_ERR_ARG.
 * u           [M] float32 uniforms in [0, 1) (the caller's random draw),
 *             4-byte aligned
 * logits      [M][V] float32, optional (NULL: not written)
 * token_ids   [M] int32, as for lmhead_gemv_fp8_argmax (-1: a wait gave up)
 * workspace   as for lmhead_gemv_fp8_argmax (same size function, zero-filled
 *             once; the two calls may share one workspace if they do not
 *             overlap).
 */
#define MOEDEC_MAX_SAMPLE_K 32
int lmhead_gemv_fp8_sample(const moedec_lmhead_fp8* head, const uint16_t* x_bf16, int M,
                           float temperature, float top_p, int top_k, const float* u, float* logits,
                           int32_t* token_ids, void* workspace, size_t workspace_bytes,
                           moedec_stream_t stream);

/* Comparator: logits = W x with bf16 W [V][H] (16-byte aligned), float32
 * accumulation.  1 <= M <= 4, H % 8 == 0, H <= 4096. */
int lmhead_gemv_bf16(const uint16_t* w_bf16, int V, int H, const uint16_t* x_bf16, int M,
                     float* logits, moedec_stream_t stream);

/* ------------------------------------------------------------------------
 * Start-up self-check.  [news two easily missed details; card limits: a
 * draft model that received the FP8 head's weight tensor instead of the
 * whole head module ran silently wrong and slower; the advice is to verify
 * the wiring at start-up]  Runs small cases whose results have closed forms
 * through the calls of this library on `stream` and compares them on the host:
 *   - routing: logits {1.5, 0.5, 1.5, -1}, k = 2 -> ids {0, 2} (tie to the
 *     lower index), weights {0.5, 0.5} exactly;
 *   - the fused MXFP4 layer (H = 64, I = 32, 4 routed experts + shared, every
 *     gate/up weight 1, every down weight 2^-5, x = 2^-6): g = u = 1, every
 *     output 0.5 h + 0.5 h + h = 2 / (1 + e^-1) (float32 rounding only);
 *   - the FP8 head: codes of {448, -2, 1, 0.5, 0} and a row of 0.25 under
 *     per-row scales, the GEMV of a one-hot x, and its greedy token.
 * scratch: device memory of >= moedec_selftest_bytes() bytes, 256-byte
 * aligned, contents ignored.  Unlike every other call this one WAITS for the
 * stream.  Returns MOEDEC_OK, or MOEDEC_ERR_SELFTEST with
 * moedec_last_error() naming the first case that differs (or the status of
 * a call that failed).
 */
size_t moedec_selftest_bytes(void);
int moedec_selftest(void* scratch, size_t scratch_bytes, moedec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEDEC_H */
