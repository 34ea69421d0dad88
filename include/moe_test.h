/* moe_test.h -- TEST-ONLY entry points of libmoe_mi355x.so.
 *
 * Not part of the layer's API (include/moe.h): these calls exist so that a test suite can
 * pin the grouped GEMM kernels of the layer's two expert products ("GPT-OSS on day 0",
 * sections "On Hopper" and "Kernels -> MoE": the expert MLPs as FP8 grouped GEMMs with
 * 128x128 block-scaled weights; "Hosting Qwen on Blackwell", section "Quantization" for
 * the MX formats) bit for bit, independently of the bias / SwiGLU / requantisation
 * epilogues.  The kernels are the very ones moe_forward launches, with the epilogue
 * replaced by a store of the fp32 accumulators.
 *
 * Conventions are those of moe.h (caller-owned device pointers, row-major, 16-byte
 * aligned; negative status on a rejected argument, nothing enqueued then), except that
 * moe_test_gemm_raw copies a host-built tile list to the workspace and synchronises
 * `stream` before it returns.
 */
#ifndef MOE_MI355X_TEST_H
#define MOE_MI355X_TEST_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes moe_test_gemm_raw needs for `rows` routed rows over E experts with
 * reduction length K (0 if out of range). */
size_t moe_test_gemm_raw_workspace_bytes(int rows, int E, int K);

/* One grouped GEMM of the layer with its raw fp32 accumulators as the output.
 *   gemm           1: GEMM1 (routed row p reads A row perm[p] / top_k; B = w13, N = 2I:
 *                     C columns [0, I) are the gate rows, [I, 2I) the up rows);
 *                  2: GEMM2 (A rows in dispatch order, perm unused; B = w2, N = H)
 *   format         0: 128x128 block scales (A_scales fp32 [A_rows, ceil(K/128)], B_scales
 *                     fp32 [E, ceil(N/128), ceil(K/128)]);
 *                  1: MXFP8 (A_scales E8M0 rows [A_rows, 4 ceil(K/128)], B_scales E8M0
 *                     tiles as moe_quantize_weights_mx writes them);
 *                  2: MXFP4 weights (B and B_scales in moe_quantize_weights_mxfp4's tiled
 *                     storage), MXFP8 A
 *   bm             M-tile rows, which selects the kernel family exactly as moe_forward's
 *                  plan does: 256 -> the persistent large-group kernel (tiles of at most
 *                  64 rows take its narrow body; formats 0 and 1 with a mean group below
 *                  384 rows let an expert's last tile hold up to 16 more rows, as the
 *                  forward's tile list does); 16 with K = 64 mod 128 (or MXFP4) -> the
 *                  row-run streaming kernel; 16, 64 or 128 otherwise -> the LDS-ring kernel
 *                  (block scales only; MX formats take 16 or 256)
 *   A [A_rows, K]  e4m3 codes;  perm [rows] (GEMM1 only) device int32
 *   expert_counts  HOST int32 [E]: routed rows per expert (rows = their sum; the rows of
 *                  expert e are the contiguous dispatch-order segment after experts < e)
 *   B              e4m3 codes [E, N, K] (formats 0, 1) or MXFP4 tiles (format 2)
 *   C [rows, N]    float output; every element of a routed row is written
 * Requirements: K and N positive multiples of 64, rows * K < 2^31, N * K < 2^31,
 * 1 <= E <= 256, MXFP4 with bm 16: K <= 8192.  Errors: MOE_ERR_INVALID_ARG (null or
 * misaligned pointer, bad gemm / format), MOE_ERR_UNSUPPORTED_SHAPE (no kernel takes the
 * combination, or the sizes above), MOE_ERR_WORKSPACE_TOO_SMALL. */
moe_status moe_test_gemm_raw(int gemm, int format, int bm, const uint8_t* A,
                             const void* A_scales, int A_rows, const int32_t* perm, int top_k,
                             const int32_t* expert_counts, int E, const uint8_t* B,
                             const void* B_scales, int N, int K, float* C, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bound on the polls of every wait inside later moe_forward_fused launches of this process
 * (default 131072).  A negative value makes every wait give up at once, so the error path
 * (the status word that moe_fused_status reads, every workgroup exiting normally) can be
 * exercised without any wait actually running out.  Returns the previous bound. */
int moe_test_set_fused_spin_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_TEST_H */
