/* moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer.
 *
 * The layer ("GPT-OSS on day 0", section "On Hopper" feature list and section
 * "Kernels -> MoE"; "Hosting Qwen on Blackwell", section "MoE Dispatch - Combine"):
 *
 *   logits = x . Wr^T + br                      router GEMM, fp32
 *   ids, gates = top-k(logits), softmax over the k selected logits
 *   for every expert e and the tokens routed to it (expert-major dispatch):
 *     C = deq(xq) . deq(w13_e)^T + b13_e        FP8 GEMM, 128x128-block-scaled weights
 *     h = silu(C[:, :I]) * C[:, I:]             SwiGLU (rows [0,I) of w13 = gate, [I,2I) = up)
 *     y = deq(hq) . deq(w2_e)^T + b2_e          FP8 GEMM
 *   out[t] = sum_j gates[t,j] * y(t, j)          gate-weighted combine, rounded once to bf16
 *
 * Activations x and h are quantised per token (per routed row for h) in 1x128 groups
 * along K; weights in 128x128 blocks.  A scale is fp32(amax / 448) (1 for an all-zero
 * group), a code the nearest OCP e4m3 value (ties to even) of fp32(v / scale) clamped
 * to +-448.  Blocks tile each matrix from (0,0); edge blocks are partial.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are caller-owned DEVICE pointers, row-major, contiguous,
 *     16-byte aligned.  bf16 is passed as uint16_t bit patterns, fp8 as uint8_t OCP
 *     e4m3fn codes.  `stream` is a hipStream_t (NULL = the null stream).
 *   - Arguments are validated synchronously; on error a negative status is returned
 *     and NOTHING is enqueued.  On success the work is only ENQUEUED on `stream`:
 *     no host synchronisation and no device allocation happen inside the library.
 *   - Inputs are read-only and must not alias outputs or the workspace.
 *   - Calls are re-entrant; concurrent calls must use distinct workspaces.
 *   - Every kernel a call will launch is chosen (and any large-LDS opt-in made) during
 *     validation.  MOE_ERR_HIP is returned only if the HIP runtime reports a launch
 *     failure after enqueueing began; the kernels enqueued before the failing one stay
 *     enqueued, and the outputs are then undefined.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,         /* null / misaligned pointer, non-positive size */
    MOE_ERR_UNSUPPORTED_SHAPE = -2,   /* shape outside the supported envelope below */
    MOE_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes < moe_workspace_bytes(...) */
    MOE_ERR_HIP = -4,                 /* the HIP runtime reported a launch error */
    MOE_ERR_DEVICE_WAIT = -5          /* moe_fused_status: a wait inside the fused kernel
                                         ran out (see moe_forward_fused) */
} moe_status;

/* Supported envelope: 1 <= T, 1 <= E <= 256, 1 <= top_k <= min(E, 8),
 * H and I positive multiples of 64, T * top_k < 2^31, T * H < 2^31, T * top_k * I < 2^31,
 * 2 * I * H < 2^31 (the GEMMs address A rows and one expert's weight rows with 32-bit
 * byte offsets), T * top_k * H < 2^40.  Outside it the calls return
 * MOE_ERR_UNSUPPORTED_SHAPE and moe_workspace_bytes returns 0. */

/* Routing tables, all caller-owned device buffers:
 *   topk_ids       [T, top_k] int32   expert ids per token, descending logit,
 *                                     exact ties -> lower expert index
 *   topk_gates     [T, top_k] float   softmax over the selected logits (sum = 1)
 *   expert_counts  [E]        int32   routed rows per expert
 *   expert_offsets [E + 1]    int32   exclusive prefix sum of the counts
 *   perm           [T*top_k]  int32   perm[p] = t*top_k + j of the p-th routed row, in
 *                                     expert-major, token-ascending order
 *   inv_perm       [T*top_k]  int32   inverse of perm: inv_perm[t*top_k + j] = p
 * ("Hosting Qwen on Blackwell", section "Expert Parallel": the dispatch step aggregates
 * the routing information and gathers each expert's tokens for its GEMM.) */
typedef struct {
    int32_t* topk_ids;
    float* topk_gates;
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* perm;
    int32_t* inv_perm;
} moe_routing;

/* Byte offsets of the intermediates inside a workspace (for diagnostics):
 *   xq [T, H] u8 + sx [T, ceil(H/128)] f32     quantised activations
 *   h  [T*top_k, I] u8 + sh [T*top_k, ceil(I/128)] f32   quantised SwiGLU output,
 *                                               rows in dispatch (perm) order
 *   y  [T*top_k, H] f16                        expert outputs incl. b2, dispatch order
 *                                               (IEEE half, saturated to +-65504)
 *   routing.*                                  the tables used when routing_out == NULL
 * Valid after a completed moe_forward on that workspace. */
typedef struct {
    size_t xq, sx, h, sh, y;
    size_t topk_ids, topk_gates, expert_counts, expert_offsets, perm, inv_perm;
    size_t total;
} moe_workspace_regions;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(moe_status s);

/* Bytes of device workspace moe_route / moe_forward need for this shape; 0 if the shape
 * is unsupported. */
size_t moe_workspace_bytes(int T, int H, int E, int top_k, int I);

/* Fills `out` with the workspace layout for this shape. */
moe_status moe_workspace_layout(int T, int H, int E, int top_k, int I, moe_workspace_regions* out);

/* 128x128 block quantisation of E stacked fp32 matrices ("GPT-OSS on day 0", section
 * "On Hopper": FP8 with 128x128 block scaling; weights are converted statically, as in
 * "Hosting Qwen on Blackwell", section "Quantization").
 *   w      [E, N, K] float      source weights
 *   codes  [E, N, K] uint8      e4m3 codes (output)
 *   scales [E, ceil(N/128), ceil(K/128)] float   block scales (output)
 * Requires E, N >= 1 and K a positive multiple of 16. */
moe_status moe_quantize_weights(const float* w, int E, int N, int K, uint8_t* codes,
                                float* scales, void* stream);

/* Per-token 1x128 activation quantisation (the activation side of the FP8 GEMMs).
 *   x      [T, H] bf16          input
 *   codes  [T, H] uint8         e4m3 codes (output)
 *   scales [T, ceil(H/128)] float (output)
 * Requires T >= 1 and H a positive multiple of 64. */
moe_status moe_quantize_activations(const uint16_t* x, int T, int H, uint8_t* codes,
                                    float* scales, void* stream);

/* Router GEMM + top-k + softmax over the selected logits + dispatch tables ("GPT-OSS on
 * day 0", section "Kernels -> MoE").
 *   x        [T, H] bf16        activations
 *   router_w [E, H] float       router weight (nn.Linear layout)
 *   router_b [E] float          router bias (NULL = zero)
 *   out      routing tables (all six pointers required)
 *   workspace / workspace_bytes  >= moe_workspace_bytes(T, H, E, top_k, 64) */
moe_status moe_route(const uint16_t* x, const float* router_w, const float* router_b, int T,
                     int H, int E, int top_k, const moe_routing* out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The whole layer forward.
 *   x          [T, H] bf16
 *   router_w   [E, H] float,  router_b [E] float (NULL = zero)
 *   w13        [E, 2I, H] e4m3 codes, w13_scales [E, ceil(2I/128), ceil(H/128)] float
 *   b13        [E, 2I] bf16 (NULL = zero)
 *   w2         [E, H, I] e4m3 codes,  w2_scales [E, ceil(H/128), ceil(I/128)] float
 *   b2         [E, H] bf16 (NULL = zero)
 *   out        [T, H] bf16, fully overwritten
 *   routing_out  optional (NULL allowed): also receive the routing tables
 *   workspace  >= moe_workspace_bytes(T, H, E, top_k, I) bytes of device memory */
moe_status moe_forward(const uint16_t* x, const float* router_w, const float* router_b,
                       const uint8_t* w13, const float* w13_scales, const uint16_t* b13,
                       const uint8_t* w2, const float* w2_scales, const uint16_t* b2, int T,
                       int H, int E, int top_k, int I, uint16_t* out,
                       const moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* moe_forward with per-stage timing: identical work and results, plus
 * MOE_PROFILE_EVENTS hipEvent_t handles (created by the caller) recorded on `stream`
 * before each stage and after the last one:
 *   0 router GEMM (with the 1x128 quantisation of x fused in)  1 top-k + softmax
 *   2 dispatch scan  3 dispatch scatter  4 x scale-word regrouping  5 GEMM1 (+ bias,
 *   SwiGLU, requantisation; for 256-row tiles it also stores h's scale words K-block
 *   major for GEMM2)  6 GEMM2 (+ bias)  7 combine  8 end
 * so hipEventElapsedTime(events[i], events[i+1]) is stage i's device time.  Stage 4
 * regroups the x scale words into dispatch order, K-block major, for the 256-row GEMM
 * tiles, and is empty for the other tile heights; for T > 448 the top-k + softmax runs
 * inside stage 0's kernel (the workgroup that completes a token tile's router partials
 * selects its tokens' experts) and stage 1 is empty; for T <= 256 the scatter runs inside
 * stage 2's kernel and stage 3 is empty, and when also top_k <= 4 and T * E <= 16384 one
 * kernel does top-k, scan and scatter in stage 1 and stages 2 and 3 are both empty.
 * `events` must point to MOE_PROFILE_EVENTS entries (NULL array: MOE_ERR_INVALID_ARG);
 * a NULL entry is not recorded, so a caller can time some stages only (each recorded
 * event adds a small gap between kernels). */
#define MOE_PROFILE_EVENTS 9
moe_status moe_forward_profiled(const uint16_t* x, const float* router_w, const float* router_b,
                                const uint8_t* w13, const float* w13_scales, const uint16_t* b13,
                                const uint8_t* w2, const float* w2_scales, const uint16_t* b2,
                                int T, int H, int E, int top_k, int I, uint16_t* out,
                                const moe_routing* routing_out, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* events);

/* ---- MXFP8 variant ("Hosting Qwen on Blackwell", section "Quantization": the weights
 * are converted statically to MXFP8, the microscaling format, instead of 128x128 block
 * scaling).  OCP Microscaling rule: every 32 consecutive elements along K share one
 * E8M0 scale code c (scale 2^(c - 127)), c - 127 = floor(log2(amax)) - 8 clamped to
 * [-127, 127] (0 for an all-zero block); an element code is the nearest e4m3 value
 * (ties to even) of v * 2^-(c - 127), clamped to +-448.  Weights, x and h all use 1x32
 * blocks along K.
 *
 * Scale layout: a row of K elements has K/32 codes, padded to 4 * ceil(K/128) bytes
 * (whole 4-byte words per 128-wide K-step, as the GEMMs stage them); the bytes past K/32
 * hold 127.  Activation scales (x, h) are such rows, one per token.  Weight scales are
 * stored in 16-row x 128-K tiles, the order the GEMMs read them: with KB = ceil(K/128),
 * a matrix [N, K] (N a multiple of 16) has N/16 x KB tiles of 64 bytes, tile (n, j) at
 * index n * KB + j holding row 16 n + r's four codes of K-block j at byte 4 r.  Scale
 * arrays of moe_forward_mx must be 4-byte aligned. */

/* MXFP8 quantisation of E stacked fp32 matrices.
 *   w      [E, N, K] float      source weights
 *   codes  [E, N, K] uint8      e4m3 codes (output)
 *   scales [E][N/16][KB][16][4] uint8   E8M0 codes in scale tiles (output)
 * Requires E >= 1, N a positive multiple of 16 and K a positive multiple of 32. */
moe_status moe_quantize_weights_mx(const float* w, int E, int N, int K, uint8_t* codes,
                                   uint8_t* scales, void* stream);

/* Per-token 1x32 MXFP8 activation quantisation (the rule the MXFP8 forward applies to x).
 *   x      [T, H] bf16          input
 *   codes  [T, H] uint8         e4m3 codes (output)
 *   scales [T, 4 ceil(H/128)] uint8   E8M0 codes, padded rows (output)
 * Requires T >= 1 and H a positive multiple of 64. */
moe_status moe_quantize_activations_mx(const uint16_t* x, int T, int H, uint8_t* codes,
                                       uint8_t* scales, void* stream);

/* The whole layer forward with MXFP8 experts: moe_forward's arguments and semantics, with
 * w13_scales and w2_scales the scale tiles of moe_quantize_weights_mx (2I x H and H x I
 * matrices), and x and h quantised in 1x32 MX blocks.  The workspace is the same
 * (moe_workspace_bytes). */
moe_status moe_forward_mx(const uint16_t* x, const float* router_w, const float* router_b,
                          const uint8_t* w13, const uint8_t* w13_scales, const uint16_t* b13,
                          const uint8_t* w2, const uint8_t* w2_scales, const uint16_t* b2, int T,
                          int H, int E, int top_k, int I, uint16_t* out,
                          const moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* moe_forward_mx with the per-stage events of moe_forward_profiled. */
moe_status moe_forward_mx_profiled(const uint16_t* x, const float* router_w,
                                   const float* router_b, const uint8_t* w13,
                                   const uint8_t* w13_scales, const uint16_t* b13,
                                   const uint8_t* w2, const uint8_t* w2_scales, const uint16_t* b2,
                                   int T, int H, int E, int top_k, int I, uint16_t* out,
                                   const moe_routing* routing_out, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events);

/* ---- MXFP4 expert weights ("GPT-OSS on day 0": the checkpoints ship with MXFP4 expert
 * weights).  OCP Microscaling with e2m1 elements (sign, 2 exponent bits with bias 1, 1
 * mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6): every 32 consecutive elements
 * along K share an E8M0 code c, c - 127 = floor(log2(amax)) - 2 clamped to [-127, 127] (0
 * for an all-zero block); an element is the nearest e2m1 value (ties to the even code)
 * of v * 2^-(c - 127), clamped to +-6.  Activations (x, h) stay MXFP8 (1x32 blocks, e4m3).
 *
 * Storage: 16-row x 128-K tiles, in the order the GEMMs stream them (the MXFP8 weight
 * scale tiles above, and code tiles of the same shape).  With KB = ceil(K/128), a
 * matrix [N, K] (N a multiple of 16) is N/16 x KB tiles, tile (n, j) at index n * KB + j:
 *   codes:  1024 bytes per tile; row r of the tile (matrix row 16 n + r) at byte 64 r holds
 *           K [128 j, 128 j + 128), two codes per byte (element 2i in the low nibble of
 *           byte i); codes past K are 0.  N * KB * 64 bytes per matrix.
 *   scales: 64 bytes per tile; row r's four E8M0 codes of the tile's K-block at byte 4 r
 *           (codes of blocks past K are 127).  N * 4 KB bytes per matrix. */

/* MXFP4 quantisation of E stacked fp32 matrices [E, N, K] into the tiled storage above
 * (codes [E][N/16][KB][16][64], scales [E][N/16][KB][16][4], uint8, device memory).
 * Requires E >= 1, N a positive multiple of 16 and K a positive multiple of 32. */
moe_status moe_quantize_weights_mxfp4(const float* w, int E, int N, int K, uint8_t* codes,
                                      uint8_t* scales, void* stream);

/* The whole layer forward with MXFP4 expert weights: moe_forward_mx's arguments, with w13
 * ([E] matrices [2I, H]), w2 ([E] matrices [H, I]) and their scales in the tiled storage
 * of moe_quantize_weights_mxfp4.  x and h are quantised in 1x32 MXFP8 blocks.  The
 * workspace is the same (moe_workspace_bytes).  Decode-sized layers (at most 24 routed rows
 * per expert on average) stream the weights in 16-row tiles and require H, I <= 8192
 * (MOE_ERR_UNSUPPORTED_SHAPE otherwise); larger ones take 256-row tiles. */
moe_status moe_forward_mxfp4(const uint16_t* x, const float* router_w, const float* router_b,
                             const uint8_t* w13, const uint8_t* w13_scales, const uint16_t* b13,
                             const uint8_t* w2, const uint8_t* w2_scales, const uint16_t* b2,
                             int T, int H, int E, int top_k, int I, uint16_t* out,
                             const moe_routing* routing_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* moe_forward_mxfp4 with the per-stage events of moe_forward_profiled. */
moe_status moe_forward_mxfp4_profiled(const uint16_t* x, const float* router_w,
                                      const float* router_b, const uint8_t* w13,
                                      const uint8_t* w13_scales, const uint16_t* b13,
                                      const uint8_t* w2, const uint8_t* w2_scales,
                                      const uint16_t* b2, int T, int H, int E, int top_k, int I,
                                      uint16_t* out, const moe_routing* routing_out,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* events);

/* ---- Decode: the whole layer in one persistent kernel ("Hosting Qwen on Blackwell",
 * section "Expert Parallel": for decode, dispatch, expert GEMMs and combine fuse into a
 * single kernel).  The forward of moe_forward / moe_forward_mx / moe_forward_mxfp4 for a
 * decode-sized layer, computed by one kernel launch (preceded by a one-block clear of the
 * call's counters in the workspace): router tiles, then the routing tail (top-k + softmax,
 * scan, scatter), GEMM1 and GEMM2 in 16-row M-tiles (128 h columns, 256 output columns per
 * item), and the combine,
 * taken from one work queue in dependency order, each GEMM2 tile starting as soon as its
 * M-tile's GEMM1 tiles are done.  The arithmetic of every stage is the multi-kernel path's,
 * so the results are identical to moe_forward's whenever that path also takes the
 * one-workgroup routing tail (top_k <= 4) and the row-run GEMM tiles (H and I not multiples
 * of 128); in every case they satisfy the same definitions.
 *   weight_format  0: 128x128 block scales (w13_scales / w2_scales float, as moe_forward)
 *                  1: MXFP8 (E8M0 scale tiles, as moe_forward_mx)
 *                  2: MXFP4 weights (tiled storage, as moe_forward_mxfp4)
 *   other arguments as moe_forward (scale pointers 4-byte aligned); the workspace layout
 *   is moe_workspace_layout's.
 * Envelope (MOE_ERR_UNSUPPORTED_SHAPE outside it, nothing enqueued): the general one, and
 * T <= 128, T * E <= 16384, at most 24 routed rows per expert on average
 * (T * top_k / E <= 24), H, I <= 8192.
 * Every wait of a workgroup inside the kernel is on work taken from the queue before its
 * own, so it ends once that work does; each wait is nevertheless bounded (about 2^17 polls,
 * a fraction of a second) and, past the bound, the workgroup records an error in the
 * workspace and exits, leaving `out` incomplete.  moe_fused_status reports it. */
moe_status moe_forward_fused(const uint16_t* x, const float* router_w, const float* router_b,
                             const uint8_t* w13, const void* w13_scales, const uint16_t* b13,
                             const uint8_t* w2, const void* w2_scales, const uint16_t* b2,
                             int T, int H, int E, int top_k, int I, int weight_format,
                             uint16_t* out, const moe_routing* routing_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Synchronises `stream` and returns MOE_OK if the last moe_forward_fused call on this
 * workspace (same shape) completed every wait, MOE_ERR_DEVICE_WAIT if a wait ran out
 * (MOE_ERR_HIP if the status word cannot be read). */
moe_status moe_fused_status(const void* workspace, int T, int H, int E, int top_k, int I,
                            void* stream);

/* ---- An entry point that allocates nothing ----
 * For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  moe_forward with the
 * workspace replaced by a fixed 64 MiB array that the library holds on every device it runs
 * on (allocated with its code object when the library's kernels are first loaded on that
 * device, kept until the process ends; its address is looked up once per device).  The
 * caller still owns x, the weights, out and the optional routing tables.
 * Limit: moe_workspace_bytes(T, H, E, top_k, I) must be at most 64 MiB (67108864 bytes),
 * else MOE_ERR_WORKSPACE_TOO_SMALL is returned before anything is touched; decode-sized
 * layers fit (e.g. 64 tokens at H = I = 2880, top-4), prefill-sized ones do not.
 * All calls on one device share its array: calls that overlap on one device (different
 * streams, or host threads without ordering) race and give undefined outputs.  Nothing in
 * the array has to start at zero: the forward clears what it counts into. */
moe_status moe_forward_noalloc(const uint16_t* x, const float* router_w, const float* router_b,
                               const uint8_t* w13, const float* w13_scales, const uint16_t* b13,
                               const uint8_t* w2, const float* w2_scales, const uint16_t* b2,
                               int T, int H, int E, int top_k, int I, uint16_t* out,
                               const moe_routing* routing_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
