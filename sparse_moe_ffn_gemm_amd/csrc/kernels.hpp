// Internal launchers of the gfx950 kernels (one translation unit per kernel family).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

// One M-tile of the grouped GEMMs: rows [row_begin, row_end) of expert `expert` in
// dispatch order.
struct MTile {
  int expert, row_begin, row_end, pad;
};

// ---- quantisers ----
void launch_quantize_weights(const float* w, int E, int N, int K, uint8_t* codes, float* scales,
                             hipStream_t st);
void launch_quantize_act(const uint16_t* x, int T, int H, uint8_t* codes, float* scales,
                         hipStream_t st);
// MXFP8: codes as above; E8M0 scales in rows of 4 ceil(K/128) bytes (pads hold 127)
void launch_quantize_weights_mx(const float* w, int E, int N, int K, uint8_t* codes,
                                uint8_t* scales, hipStream_t st);
void launch_quantize_act_mx(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales,
                            hipStream_t st);
// MXFP4 weights: codes [E, N, K/2] (two e2m1 codes per byte, element 2j low), scales as MX
void launch_quantize_weights_mxfp4(const float* w, int E, int N, int K, uint8_t* codes,
                                   uint8_t* scales, hipStream_t st);

// ---- routing ----
constexpr int kRouterTile = 64;     // tokens / experts per router GEMM workgroup
constexpr int kChunk = 256;         // tokens per dispatch chunk
constexpr int kGemmQueues = 8;      // per-XCD work queues of one large-group GEMM launch
// Ints between work-queue heads (and after the tile count): 4 KB, so that each head is an
// address of its own memory channel.  Atomics that several XCDs issue to one address are
// performed one after another beyond the XCDs' own L2s; with the eight heads of a launch
// on one line, one ticket per workgroup at the start of a 1104-workgroup launch cost
// 33 us there, which the queue heads' spacing avoids.
constexpr int kQueueStride = 1024;
// Rows that an expert's last 256-row M-tile may hold beyond 256 in the block-scaled and
// MXFP8 large-group GEMMs (their full tile body takes them, the sums of the extra rows kept in
// LDS), so that an expert with up to 272 rows is one M-tile instead of a full tile and a
// 16-row tile that streams the same weights again.
constexpr int kBigExtraRows = 16;
// The extra rows of a block-scaled or MXFP8 256-row layer of `rows` routed rows over E experts:
// kBigExtraRows where the mean group is below 384 rows (most groups then hold just over
// 256 rows or fewer, and many would end in a tile of a few rows), else 0 (their
// remainders spread evenly, few end that short, and the kernel without the extra-row
// body keeps more of its registers).
inline int big_extra_rows(long rows, int E) { return rows < 384L * E ? kBigExtraRows : 0; }
// M-tiles of an expert with cnt rows in tiles of bm rows whose last one may hold xr more:
// tile i covers rows [i bm, i bm + bm), the last one [i bm, cnt).
__host__ __device__ inline int expert_tiles(int cnt, int bm, int xr) {
  if (cnt <= 0) return 0;
  const int n = (cnt - xr + bm - 1) / bm;
  return n > 1 ? n : 1;
}

// partial[s][t][e] = sum over the s-th slice of H (kslice a multiple of 128) of
// x[t,h] * W[e,h] (each tile splits its W rows into their three bf16 planes itself); also
// clears hist[0, hist_n) for the top-k step, and with xq != NULL writes the 1x128
// quantisation of x (codes xq [T,H], scales sx [T, ceil(H/128)]), the same as
// launch_quantize_act.
// With sx_mx != NULL the x quantisation is MXFP8 instead (E8M0 codes into sx_mx, rows of
// 4 ceil(H/128) bytes).
void launch_router_logits(const uint16_t* x, const float* W, int T, int H, int E, int ksplit,
                          int kslice, float* partial, int32_t* hist, int hist_n, hipStream_t st,
                          uint8_t* xq = nullptr, float* sx = nullptr, uint8_t* sx_mx = nullptr);
// Prefill-sized routing (T > 448): the weight split into W's three bf16 planes (which also
// zeroes hist [nchunks][E] and tile_done [ceil(T/64)], contiguous), then one kernel that
// computes 64-token x 128-expert router tiles over ksplit H slices of kslice columns
// (partials [ksplit][T][E], x quantised as launch_router_logits does) and, in the workgroup
// that completes each token tile, its tokens' top-k + softmax (ids, gates, the per-chunk
// histogram).  route_prefill_shape gives the H split; route_prefill_prepare makes the
// kernel's large-LDS opt-in (false if the device cannot hold it).
void route_prefill_shape(int T, int H, int E, int* ksplit, int* kslice);
bool route_prefill_prepare(int E, int top_k);
void launch_route_prefill(const uint16_t* x, const float* W, const float* bias, int T, int H, int E,
                          int top_k, int ksplit, int kslice, uint16_t* parts, float* partial,
                          uint8_t* xq, float* sx, uint8_t* sx_mx, int32_t* ids, float* gates,
                          int32_t* hist, int nchunks, int32_t* tile_done, hipStream_t st);
// ids/gates, counted into the per-chunk expert histogram hist[chunk][E] (cleared before)
void launch_topk(const float* partial, int ksplit, const float* bias, int T, int E, int top_k,
                 int32_t* ids, float* gates, int32_t* hist, hipStream_t st);
// counts, offsets, per-chunk bases and the M-tile list for tiles of `bm` rows (an expert's
// last tile up to bm + xr, expert_tiles);
// num_tiles[0] = number of M-tiles, num_tiles[1 .. 2 kGemmQueues] (the two GEMMs' work
// queues) are cleared.  With ids != NULL (only when nchunks == 1) the same workgroup also
// does the scatter (perm, inv), replacing launch_dispatch_scatter.
void launch_dispatch_scan(const int32_t* hist, int nchunks, int E, int bm, int xr, int32_t* counts,
                          int32_t* offsets, int32_t* chunk_base, MTile* tiles, int32_t* num_tiles,
                          int32_t* expert_tile_off, hipStream_t st, const int32_t* ids = nullptr,
                          int T = 0, int top_k = 0, int32_t* perm = nullptr, int32_t* inv = nullptr);
// dst[j * rows + p] = src[(perm[p] / top_k) * KB + j] (perm NULL: src[p * KB + j]): the
// scale words of the routed rows in dispatch order, K-block major
void launch_gather_row_scales(const uint32_t* src, int KB, const int32_t* perm, int top_k,
                              int rows, uint32_t* dst, hipStream_t st);
void launch_dispatch_scatter(const int32_t* ids, const int32_t* chunk_base, int T, int E,
                             int top_k, int32_t* perm, int32_t* inv, hipStream_t st);
constexpr int kTailLogits = 16384;  // largest T x E of the one-workgroup routing tail
constexpr int kTailSplit = 64;      // and its largest number of router H slices
constexpr int kTailTopK = 4;        // and its largest top_k
// T <= kChunk, T E <= kTailLogits, ksplit <= kTailSplit, top_k <= kTailTopK: top-k + softmax, scan, M-tile list and scatter in one
// workgroup (replaces
// launch_topk + launch_dispatch_scan; the router need not clear any histogram).
void launch_route_tail(const float* partial, int ksplit, const float* bias, int T, int E,
                       int top_k, int bm, int32_t* ids, float* gates, int32_t* counts,
                       int32_t* offsets, int32_t* chunk_base, MTile* tiles, int32_t* num_tiles,
                       int32_t* expert_tile_off, int32_t* perm, int32_t* inv, hipStream_t st);

// ---- grouped FP8 GEMMs ----
struct GemmArgs {
  const uint8_t* A;          // gemm1: xq [T, K] (rows gathered through perm); gemm2: h [rows, K]
  int A_rows;                // rows of A (T for gemm1, T * top_k for gemm2)
  const float* A_scale;      // [*, ceil(K/128)]
  const int32_t* perm;       // gemm1 only
  int top_k;
  const uint8_t* B;          // [E, N, K]
  const float* B_scale;      // [E, ceil(N/128), ceil(K/128)]
  const uint16_t* bias;      // [E, N] or NULL
  const MTile* tiles;
  const int32_t* num_tiles;
  const int32_t* expert_tile_off;   // [E+1] first M-tile of each expert, [E] = num_tiles
  int32_t* queue;            // kGemmQueues work-queue heads kQueueStride ints apart, zero at launch
  int E;
  int K, N, I;
  uint8_t* h_out;            // gemm1: [rows, I]
  float* h_scale;            // gemm1: [rows, ceil(I/128)]
  uint16_t* y_out;           // gemm2: [rows, N] fp16
  // MXFP8 instead of the block scales (A_scale, B_scale, h_scale unused): E8M0 codes in
  // rows of 4 ceil(K/128) bytes -- A_mx [*, ...], B_mx [E, N, ...], h_mx [rows, 4 ceil(I/128)]
  bool mx;
  bool fp4;                  // with mx: B holds MXFP4 (e2m1) codes [E, N, K/2]
  const uint8_t* A_mx;
  const uint8_t* B_mx;
  uint8_t* h_mx;
  // large-group GEMMs: the A rows' scale words (fp32 block scale or 4 E8M0 codes) per
  // K-step in dispatch order, [ceil(K/128)][sd_rows]; NULL: read A_scale / A_mx
  const uint32_t* A_sd;
  int sd_rows;
  // gemm1 of the large-group kernel: also store h's scale words in that layout,
  // [ceil(I/128)][sd_rows] (gemm2's A_sd), or NULL
  uint32_t* h_sd;
  float* c_raw;              // launch_gemm_raw only: [rows, N] fp32 accumulators
  int xr;                    // block-scaled / MXFP8 256-row tiles: rows an M-tile holds past 256 (0 or kBigExtraRows)
};

// Rows per M-tile chosen for a layer with `rows` routed rows over E experts.
int gemm_tile_rows(long rows, int E);
// Whether a kernel takes GEMM1 (swiglu) or GEMM2 launches of bm-row M-tiles over K in this
// format, with any large-LDS opt-in it needs done (a host-side call that enqueues nothing);
// launch_gemm1/2 may only be called for accepted launches.
// raw: the test-only variants that store the fp32 accumulators (launch_gemm_raw).
bool gemm_prepare(bool swiglu, bool mx, bool fp4, int K, int bm, bool raw = false);
void launch_gemm1(const GemmArgs& a, int bm, int max_tiles, hipStream_t st);
void launch_gemm2(const GemmArgs& a, int bm, int max_tiles, hipStream_t st);
// The same kernels with the epilogue replaced by a store of the fp32 accumulators (no
// bias, SwiGLU or quantisation) into a.c_raw [rows, N] at each B row's matrix row: gemm1
// gate rows j at column j, up rows I + j at column I + j.  Test infrastructure only.
void launch_gemm_raw(bool gemm1, const GemmArgs& a, int bm, int max_tiles, hipStream_t st);

// ---- decode: the whole layer in one persistent kernel ----
// Counters of one fused call in the workspace (kFusedCtrTile + M-tiles words), zeroed by the
// launch's clear kernel: the work-queue head, router tiles done, the routing-done flag,
// GEMM2 items done, the error code, and from kFusedCtrTile on the GEMM1 items done per
// M-tile.
constexpr int kFusedHead = 0, kFusedRouterDone = 1, kFusedRouted = 2, kFusedDone2 = 3,
              kFusedError = 4, kFusedCtrTile = 8;
constexpr int kFusedCombineCols = 2048;   // columns of one combine item (512 lanes x 4)
constexpr int kFusedMaxT = 128;           // tokens of a fused call (4 ceil(T / 64) <= 8 waves)
// error codes in the kFusedError word
constexpr int kFusedErrWait = 1;          // a bounded wait ran out

struct FusedArgs {
  const uint16_t* x;
  const float* rw;
  const float* rb;
  int T, H, E, top_k, I;
  int ksplit, kslice, ntx, ney;   // router tiles: token tiles x expert tiles x H slices
  float* partial;
  uint8_t* xq;
  float* sx;                       // block-scaled x scales (NULL for MX)
  uint8_t* sx_mx;                  // MX x scale codes (NULL for block scales)
  int32_t* ids;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* chunk_base;
  int32_t* perm;
  int32_t* inv;
  GemmArgs g1, g2;                 // the GEMMs (tiles, num_tiles, expert_tile_off shared)
  uint16_t* y;
  uint16_t* out;
  int32_t* ctr;
  int spin_limit;                  // polls per wait before giving up (< 0: give up at once)
};

// Dynamic LDS of the fused kernel for a shape (the largest of its stages).
size_t fused_lds_bytes(int T, int H, int E, int top_k, int I);
// Whether the fused kernel takes this format (0 block, 1 MXFP8, 2 MXFP4) with `lds` bytes
// of dynamic LDS on the current device (its large-LDS opt-in done); enqueues nothing.
bool fused_prepare(int fmt, size_t lds);
// Clears the counters (kFusedCtrTile + max_tiles words) and launches the fused kernel with
// as many workgroups as the device holds at once (at most max_items).
void launch_fused(const FusedArgs& f, int fmt, size_t lds, int max_tiles, long max_items,
                  hipStream_t st);
// Polls per wait of later launches (test hook; default 1 << 17); returns the previous bound.
int set_fused_spin_limit(int polls);

// ---- combine ----
void launch_combine(const uint16_t* y, const float* gates, const int32_t* inv, int T, int H,
                    int top_k, uint16_t* out, hipStream_t st);

}  // namespace moe
