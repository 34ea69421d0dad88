// C ABI of the MoE layer: argument validation, workspace layout and the launch
// sequence.  Everything is enqueued on the caller's stream; nothing here waits for
// the device or allocates device memory.
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "moe.h"
#include "kernels.hpp"

namespace {

using moe::ceil_div;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int T, H, E, k, I;
  long rows;
  int ksplit, kslice, nchunks, bm, max_tiles;
  int xr;          // rows an expert's last M-tile may hold beyond bm (moe::expert_tiles)
  bool presplit;   // prefill-sized routing: W split once per call, then the routing kernel
                   // (route_prefill: 64-token x 128-expert router tiles, top-k fused)
  size_t partial, hist, wparts, chunk_base, tiles, num_tiles, expert_tile_off;
  size_t ids, gates, counts, offsets, perm, inv;
  size_t xq, sx, h, sh, y;
  size_t shd;      // h scale words in dispatch order, K-block major (large-group GEMMs)
  size_t sync;     // the fused decode kernel's counters
  int max_tiles16; // M-tiles of 16 rows at most (the tile list's capacity)
  size_t total;
};

// The GEMMs address their operands with 32-bit byte offsets from a 64-bit base: row x K
// inside A (x codes [T, H] for GEMM1, h codes [T k, I] for GEMM2) and inside one expert's
// weight matrix (w13 [2I, H], w2 [H, I]).  Every such product must stay below 2^31.
bool shape_ok(int T, int H, int E, int k, int I) {
  if (T < 1 || E < 1 || E > 256 || k < 1 || k > 8 || k > E) return false;
  if (H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0) return false;
  const long rows = static_cast<long>(T) * k;
  if (rows >= (1L << 31) || static_cast<long>(T) * H >= (1L << 31)) return false;
  if (rows * I >= (1L << 31) || 2L * I * H >= (1L << 31)) return false;
  if (rows * H >= (1L << 40)) return false;
  return true;
}

// Decode-sized layers whose routing tail (top-k, scan, scatter) runs in one workgroup.
bool uses_route_tail(int T, int E, int k, int ksplit) {
  return T <= moe::kChunk && static_cast<long>(T) * E <= moe::kTailLogits &&
         k <= moe::kTailTopK && ksplit <= moe::kTailSplit;
}

// Weight formats of the forward: 128x128 block scales, MXFP8, MXFP4 (MXFP8 activations).
enum WeightFormat { kBlockFp8 = 0, kMxfp8 = 1, kMxfp4 = 2 };

// MXFP8 layers take 256-row M-tiles (the large-group kernel) except for decode-sized groups
// that the row-run kernel streams in both GEMMs; MXFP4 layers take 16-row tiles (the
// row-run kernel) for decode-sized groups and 256-row tiles otherwise.
void make_plan(int T, int H, int E, int k, int I, Plan* p, int fmt = kBlockFp8) {
  p->T = T; p->H = H; p->E = E; p->k = k; p->I = I;
  p->rows = static_cast<long>(T) * k;
  // split H across workgroups when there are few token x expert tiles (decode)
  const int tiles2d = ceil_div(T, moe::kRouterTile) * ceil_div(E, moe::kRouterTile);
  // (slices of one 128-column step each where the tiles are few: gpt-oss-20b decode, 64
  // tokens x 32 experts, 23 slices instead of 12 of two steps, routing 1 us faster)
  int ks = ceil_div(1024, tiles2d);
  ks = std::max(1, std::min(ks, ceil_div(H, moe::kBlock)));
  // the one-workgroup routing tail reads every slice of every logit: keep them few
  if (uses_route_tail(T, E, k, 0)) ks = std::min(ks, 32);
  p->kslice = ceil_div(ceil_div(H, ks), moe::kBlock) * moe::kBlock;   // whole quantisation groups
  p->ksplit = ceil_div(H, p->kslice);
  p->nchunks = ceil_div(T, moe::kChunk);
  p->presplit = ceil_div(T, moe::kRouterTile) >= 8;
  if (p->presplit) moe::route_prefill_shape(T, H, E, &p->ksplit, &p->kslice);
  // the tile list is sized for the block-scaled tile height, an upper bound for the
  // 256-row tiles of MXFP8 too, so both formats share one workspace layout
  const int bm_block = moe::gemm_tile_rows(p->rows, E);
  // MXFP8: decode-sized groups whose weight rows are not whole 128-byte lines in both GEMMs
  // (H and I = 64 mod 128, the row-run kernel) keep 16-row tiles, all others 256
  const bool mx_rowrun = bm_block == 16 && H % 128 != 0 && I % 128 != 0 && H <= 8192 && I <= 8192;
  p->bm = fmt == kMxfp4 ? (bm_block == 16 ? 16 : 256) : fmt == kMxfp8 ? (mx_rowrun ? 16 : 256) : bm_block;
  p->xr = fmt != kMxfp4 && p->bm == 256 ? moe::big_extra_rows(p->rows, E) : 0;
  p->max_tiles = static_cast<int>(p->rows / p->bm + std::min<long>(E, p->rows));
  // the tile list is sized for 16-row tiles, the most of any format, so that every format
  // shares one workspace layout
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  p->partial = take(sizeof(float) * p->ksplit * static_cast<size_t>(T) * E);
  // the dispatch histograms, then (prefill) the routing kernel's per-token-tile counters
  p->hist = take(sizeof(int32_t) * (p->nchunks * static_cast<size_t>(E) + ceil_div(T, 64)));
  p->wparts = take(p->presplit ? sizeof(uint16_t) * 3 * static_cast<size_t>(E) * H : 0);
  p->chunk_base = take(sizeof(int32_t) * p->nchunks * static_cast<size_t>(E));
  p->max_tiles16 = static_cast<int>(p->rows / 16 + std::min<long>(E, p->rows));
  p->tiles = take(sizeof(moe::MTile) * static_cast<size_t>(p->max_tiles16));
  // the tile count, then the two GEMMs' queue heads, kQueueStride ints apart
  p->num_tiles = take(sizeof(int32_t) * moe::kQueueStride * (1 + 2 * moe::kGemmQueues));
  p->expert_tile_off = take(sizeof(int32_t) * (E + 1));
  p->ids = take(sizeof(int32_t) * p->rows);
  p->gates = take(sizeof(float) * p->rows);
  p->counts = take(sizeof(int32_t) * E);
  p->offsets = take(sizeof(int32_t) * (E + 1));
  p->perm = take(sizeof(int32_t) * p->rows);
  p->inv = take(sizeof(int32_t) * p->rows);
  p->xq = take(static_cast<size_t>(T) * H);
  p->sx = take(sizeof(float) * static_cast<size_t>(T) * ceil_div(H, moe::kBlock));
  p->h = take(static_cast<size_t>(p->rows) * I);
  p->sh = take(sizeof(float) * static_cast<size_t>(p->rows) * ceil_div(I, moe::kBlock));
  p->y = take(sizeof(uint16_t) * static_cast<size_t>(p->rows) * H);
  p->shd = take(sizeof(uint32_t) * static_cast<size_t>(p->rows) * ceil_div(I, moe::kBlock));
  p->sync = take(sizeof(int32_t) * static_cast<size_t>(moe::kFusedCtrTile + p->max_tiles16));
  p->total = off;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}

moe_status finish() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// routing tables of one call: the caller's or the workspace's
struct Tables {
  int32_t* ids;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
};

// Records profiling event i on the stream (no-op without events or for a NULL entry).
void mark(hipEvent_t* ev, int i, hipStream_t st) {
  if (ev && ev[i]) (void)hipEventRecord(ev[i], st);
}

// Router (which also quantises x when `quant_x`), top-k and the dispatch tables.
void enqueue_routing(const Plan& p, const uint16_t* x, const float* rw, const float* rb,
                     const Tables& tb, void* ws, hipStream_t st, hipEvent_t* ev = nullptr,
                     bool quant_x = false, bool mx = false) {
  mark(ev, 0, st);
  if (p.presplit) {
    // prefill: router GEMM with the top-k fused (stage 0), the scan (2) and the scatter (3)
    moe::launch_route_prefill(x, rw, rb, p.T, p.H, p.E, p.k, p.ksplit, p.kslice,
                              at<uint16_t>(ws, p.wparts), at<float>(ws, p.partial),
                              quant_x ? at<uint8_t>(ws, p.xq) : nullptr,
                              quant_x && !mx ? at<float>(ws, p.sx) : nullptr,
                              quant_x && mx ? at<uint8_t>(ws, p.sx) : nullptr, tb.ids, tb.gates,
                              at<int32_t>(ws, p.hist), p.nchunks,
                              at<int32_t>(ws, p.hist) + static_cast<size_t>(p.nchunks) * p.E, st);
    mark(ev, 1, st);
    mark(ev, 2, st);
    moe::launch_dispatch_scan(at<int32_t>(ws, p.hist), p.nchunks, p.E, p.bm, p.xr, tb.counts, tb.offsets,
                              at<int32_t>(ws, p.chunk_base), at<moe::MTile>(ws, p.tiles),
                              at<int32_t>(ws, p.num_tiles), at<int32_t>(ws, p.expert_tile_off), st);
    mark(ev, 3, st);
    moe::launch_dispatch_scatter(tb.ids, at<int32_t>(ws, p.chunk_base), p.T, p.E, p.k, tb.perm,
                                 tb.inv, st);
    return;
  }
  // a single chunk of tokens (decode-sized T): one workgroup does the scan and the
  // scatter; with few logits the same workgroup also does top-k + softmax
  const bool one_chunk = p.nchunks == 1;
  const bool tail = uses_route_tail(p.T, p.E, p.k, p.ksplit);
  moe::launch_router_logits(x, rw, p.T, p.H, p.E, p.ksplit, p.kslice, at<float>(ws, p.partial),
                            at<int32_t>(ws, p.hist), tail ? 0 : p.nchunks * p.E, st,
                            quant_x ? at<uint8_t>(ws, p.xq) : nullptr,
                            quant_x && !mx ? at<float>(ws, p.sx) : nullptr,
                            quant_x && mx ? at<uint8_t>(ws, p.sx) : nullptr);
  mark(ev, 1, st);
  if (tail) {
    moe::launch_route_tail(at<float>(ws, p.partial), p.ksplit, rb, p.T, p.E, p.k, p.bm, tb.ids,
                           tb.gates, tb.counts, tb.offsets, at<int32_t>(ws, p.chunk_base),
                           at<moe::MTile>(ws, p.tiles), at<int32_t>(ws, p.num_tiles),
                           at<int32_t>(ws, p.expert_tile_off), tb.perm, tb.inv, st);
    mark(ev, 2, st);
    mark(ev, 3, st);
    return;
  }
  moe::launch_topk(at<float>(ws, p.partial), p.ksplit, rb, p.T, p.E, p.k, tb.ids, tb.gates,
                   at<int32_t>(ws, p.hist), st);
  mark(ev, 2, st);
  moe::launch_dispatch_scan(at<int32_t>(ws, p.hist), p.nchunks, p.E, p.bm, p.xr, tb.counts, tb.offsets,
                            at<int32_t>(ws, p.chunk_base), at<moe::MTile>(ws, p.tiles),
                            at<int32_t>(ws, p.num_tiles), at<int32_t>(ws, p.expert_tile_off), st,
                            one_chunk ? tb.ids : nullptr, p.T, p.k, tb.perm, tb.inv);
  mark(ev, 3, st);
  if (!one_chunk)
    moe::launch_dispatch_scatter(tb.ids, at<int32_t>(ws, p.chunk_base), p.T, p.E, p.k, tb.perm,
                                 tb.inv, st);
}

bool aligned4(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3u) == 0; }

bool routing_ok(const moe_routing* r) {
  return r && r->topk_ids && r->topk_gates && r->expert_counts && r->expert_offsets && r->perm &&
         r->inv_perm && aligned16(r->topk_ids) && aligned16(r->topk_gates) &&
         aligned16(r->perm) && aligned16(r->inv_perm);
}

}  // namespace

// The layer; `fmt` selects MXFP8 or MXFP4 weights (w13_scales / w2_scales are E8M0 code
// rows, uint8; MXFP4 codes are packed two per byte) over the 128x128 block scales (fp32).
static moe_status forward_impl(const uint16_t* x, const float* router_w, const float* router_b,
                       const uint8_t* w13, const void* w13_scales, const uint16_t* b13,
                       const uint8_t* w2, const void* w2_scales, const uint16_t* b2, int T,
                       int H, int E, int top_k, int I, uint16_t* out,
                       const moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                       void* stream, hipEvent_t* ev, int fmt = kBlockFp8) {
  const bool mx = fmt != kBlockFp8;
  if (!x || !router_w || !w13 || !w13_scales || !w2 || !w2_scales || !out || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(w13) || !aligned16(w2) ||
      !aligned16(out) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if (mx && (!aligned4(w13_scales) || !aligned4(w2_scales))) return MOE_ERR_INVALID_ARG;
  if (routing_out && !routing_ok(routing_out)) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(T, H, E, top_k, I)) return MOE_ERR_UNSUPPORTED_SHAPE;
  Plan p;
  make_plan(T, H, E, top_k, I, &p, fmt);
  // the row-run kernel stages a 16-row activation tile of all of K in LDS
  if (fmt == kMxfp4 && p.bm == 16 && (H > 8192 || I > 8192)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  // which GEMM kernels take this plan (and their large-LDS opt-in), decided before
  // anything is enqueued
  if (!moe::gemm_prepare(true, mx, fmt == kMxfp4, H, p.bm) ||
      !moe::gemm_prepare(false, mx, fmt == kMxfp4, I, p.bm))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  if (p.presplit && !moe::route_prefill_prepare(E, top_k)) return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = workspace;
  const Tables tb = routing_out
                        ? Tables{routing_out->topk_ids, routing_out->topk_gates,
                                 routing_out->expert_counts, routing_out->expert_offsets,
                                 routing_out->perm, routing_out->inv_perm}
                        : Tables{at<int32_t>(ws, p.ids), at<float>(ws, p.gates),
                                 at<int32_t>(ws, p.counts), at<int32_t>(ws, p.offsets),
                                 at<int32_t>(ws, p.perm), at<int32_t>(ws, p.inv)};
  enqueue_routing(p, x, router_w, router_b, tb, ws, st, ev, /*quant_x=*/true, mx);
  mark(ev, 4, st);   // (the x quantisation ran inside the router kernel; stage 4: scale regrouping)
  // large-group GEMM1: the x scale words of the routed rows in dispatch order, K-block
  // major, staged in the y region (written only later, by GEMM2)
  const bool gather_sx = p.bm == 256;
  if (gather_sx)
    moe::launch_gather_row_scales(at<uint32_t>(ws, p.sx), ceil_div(H, moe::kBlock), tb.perm, top_k,
                                  static_cast<int>(p.rows), at<uint32_t>(ws, p.y), st);
  mark(ev, 5, st);

  moe::GemmArgs g1{};
  g1.A = at<uint8_t>(ws, p.xq);
  g1.A_rows = T;
  g1.perm = tb.perm;
  g1.top_k = top_k;
  g1.B = w13;
  g1.mx = mx;
  g1.fp4 = fmt == kMxfp4;
  g1.xr = p.xr;
  if (mx) {
    g1.A_mx = at<uint8_t>(ws, p.sx);
    g1.B_mx = static_cast<const uint8_t*>(w13_scales);
    g1.h_mx = at<uint8_t>(ws, p.sh);
  } else {
    g1.A_scale = at<float>(ws, p.sx);
    g1.B_scale = static_cast<const float*>(w13_scales);
    g1.h_scale = at<float>(ws, p.sh);
  }
  g1.bias = b13;
  g1.tiles = at<moe::MTile>(ws, p.tiles);
  g1.num_tiles = at<int32_t>(ws, p.num_tiles);
  g1.expert_tile_off = at<int32_t>(ws, p.expert_tile_off);
  g1.E = E;
  g1.K = H;
  g1.N = 2 * I;
  g1.I = I;
  g1.h_out = at<uint8_t>(ws, p.h);
  g1.queue = at<int32_t>(ws, p.num_tiles) + moe::kQueueStride;
  if (gather_sx) {
    g1.A_sd = at<uint32_t>(ws, p.y);
    g1.sd_rows = static_cast<int>(p.rows);
    g1.h_sd = at<uint32_t>(ws, p.shd);   // GEMM2's A_sd, written by GEMM1's epilogue
  }
  moe::launch_gemm1(g1, p.bm, p.max_tiles, st);
  mark(ev, 6, st);

  moe::GemmArgs g2{};
  g2.A = at<uint8_t>(ws, p.h);
  g2.A_rows = static_cast<int>(p.rows);
  g2.perm = nullptr;
  g2.top_k = top_k;
  g2.B = w2;
  g2.mx = mx;
  g2.fp4 = fmt == kMxfp4;
  g2.xr = p.xr;
  if (mx) {
    g2.A_mx = at<uint8_t>(ws, p.sh);
    g2.B_mx = static_cast<const uint8_t*>(w2_scales);
  } else {
    g2.A_scale = at<float>(ws, p.sh);
    g2.B_scale = static_cast<const float*>(w2_scales);
  }
  g2.bias = b2;
  g2.tiles = g1.tiles;
  g2.num_tiles = g1.num_tiles;
  g2.expert_tile_off = g1.expert_tile_off;
  g2.E = E;
  g2.K = I;
  g2.N = H;
  g2.I = I;
  g2.y_out = at<uint16_t>(ws, p.y);
  g2.queue = at<int32_t>(ws, p.num_tiles) + moe::kQueueStride * (1 + moe::kGemmQueues);
  if (gather_sx) {   // h's scale words K-block major (stored by GEMM1)
    g2.A_sd = at<uint32_t>(ws, p.shd);
    g2.sd_rows = static_cast<int>(p.rows);
  }
  moe::launch_gemm2(g2, p.bm, p.max_tiles, st);
  mark(ev, 7, st);
  moe::launch_combine(at<uint16_t>(ws, p.y), tb.gates, tb.inv, T, H, top_k, out, st);
  mark(ev, 8, st);
  return finish();
}


// ---- decode: the whole layer in one persistent kernel ----

// The fused kernel's envelope (beyond shape_ok): decode-sized groups (16-row M-tiles), a
// token count and logit count the one-workgroup routing tail holds, row-run GEMM tiles.
static bool fused_shape_ok(const Plan& p) {
  if (p.T > moe::kFusedMaxT || static_cast<long>(p.T) * p.E > moe::kTailLogits) return false;
  if (p.ksplit > moe::kTailSplit) return false;
  if (moe::gemm_tile_rows(p.rows, p.E) != 16) return false;
  if (p.H > 8192 || p.I > 8192) return false;   // the row-run tiles stage all of K in LDS
  return true;
}

extern "C" moe_status moe_forward_fused(const uint16_t* x, const float* router_w,
                                        const float* router_b, const uint8_t* w13,
                                        const void* w13_scales, const uint16_t* b13,
                                        const uint8_t* w2, const void* w2_scales,
                                        const uint16_t* b2, int T, int H, int E, int top_k, int I,
                                        int weight_format, uint16_t* out,
                                        const moe_routing* routing_out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (weight_format < 0 || weight_format > 2) return MOE_ERR_INVALID_ARG;
  const bool mx = weight_format != kBlockFp8;
  if (!x || !router_w || !w13 || !w13_scales || !w2 || !w2_scales || !out || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(w13) || !aligned16(w2) ||
      !aligned16(out) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if (!aligned4(w13_scales) || !aligned4(w2_scales)) return MOE_ERR_INVALID_ARG;
  if (routing_out && !routing_ok(routing_out)) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(T, H, E, top_k, I)) return MOE_ERR_UNSUPPORTED_SHAPE;
  Plan p;
  make_plan(T, H, E, top_k, I, &p, weight_format);
  if (!fused_shape_ok(p)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const size_t lds = moe::fused_lds_bytes(T, H, E, top_k, I);
  if (!moe::fused_prepare(weight_format, lds)) return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  void* ws = workspace;
  const Tables tb = routing_out
                        ? Tables{routing_out->topk_ids, routing_out->topk_gates,
                                 routing_out->expert_counts, routing_out->expert_offsets,
                                 routing_out->perm, routing_out->inv_perm}
                        : Tables{at<int32_t>(ws, p.ids), at<float>(ws, p.gates),
                                 at<int32_t>(ws, p.counts), at<int32_t>(ws, p.offsets),
                                 at<int32_t>(ws, p.perm), at<int32_t>(ws, p.inv)};
  moe::FusedArgs f{};
  f.x = x;
  f.rw = router_w;
  f.rb = router_b;
  f.T = T; f.H = H; f.E = E; f.top_k = top_k; f.I = I;
  f.ksplit = p.ksplit;
  f.kslice = p.kslice;
  f.ntx = ceil_div(T, moe::kRouterTile);
  f.ney = ceil_div(E, moe::kRouterTile);
  f.partial = at<float>(ws, p.partial);
  f.xq = at<uint8_t>(ws, p.xq);
  f.sx = mx ? nullptr : at<float>(ws, p.sx);
  f.sx_mx = mx ? at<uint8_t>(ws, p.sx) : nullptr;
  f.ids = tb.ids;
  f.gates = tb.gates;
  f.counts = tb.counts;
  f.offsets = tb.offsets;
  f.chunk_base = at<int32_t>(ws, p.chunk_base);
  f.perm = tb.perm;
  f.inv = tb.inv;
  moe::GemmArgs& g1 = f.g1;
  g1.A = at<uint8_t>(ws, p.xq);
  g1.A_rows = T;
  g1.perm = tb.perm;
  g1.top_k = top_k;
  g1.B = w13;
  g1.mx = mx;
  g1.fp4 = weight_format == kMxfp4;
  if (mx) {
    g1.A_mx = at<uint8_t>(ws, p.sx);
    g1.B_mx = static_cast<const uint8_t*>(w13_scales);
    g1.h_mx = at<uint8_t>(ws, p.sh);
  } else {
    g1.A_scale = at<float>(ws, p.sx);
    g1.B_scale = static_cast<const float*>(w13_scales);
    g1.h_scale = at<float>(ws, p.sh);
  }
  g1.bias = b13;
  g1.tiles = at<moe::MTile>(ws, p.tiles);
  g1.num_tiles = at<int32_t>(ws, p.num_tiles);
  g1.expert_tile_off = at<int32_t>(ws, p.expert_tile_off);
  g1.E = E;
  g1.K = H;
  g1.N = 2 * I;
  g1.I = I;
  g1.h_out = at<uint8_t>(ws, p.h);
  moe::GemmArgs& g2 = f.g2;
  g2.A = at<uint8_t>(ws, p.h);
  g2.A_rows = static_cast<int>(p.rows);
  g2.top_k = top_k;
  g2.B = w2;
  g2.mx = mx;
  g2.fp4 = weight_format == kMxfp4;
  if (mx) {
    g2.A_mx = at<uint8_t>(ws, p.sh);
    g2.B_mx = static_cast<const uint8_t*>(w2_scales);
  } else {
    g2.A_scale = at<float>(ws, p.sh);
    g2.B_scale = static_cast<const float*>(w2_scales);
  }
  g2.bias = b2;
  g2.tiles = g1.tiles;
  g2.num_tiles = g1.num_tiles;
  g2.expert_tile_off = g1.expert_tile_off;
  g2.E = E;
  g2.K = I;
  g2.N = H;
  g2.I = I;
  g2.y_out = at<uint16_t>(ws, p.y);
  f.y = at<uint16_t>(ws, p.y);
  f.out = out;
  f.ctr = at<int32_t>(ws, p.sync);
  const long items = static_cast<long>(f.ntx) * f.ney * f.ksplit +
                     static_cast<long>(p.max_tiles16) * (ceil_div(I, 128) + ceil_div(H, 256)) +
                     static_cast<long>(T) * ceil_div(H, moe::kFusedCombineCols);
  moe::launch_fused(f, weight_format, lds, p.max_tiles16, items, static_cast<hipStream_t>(stream));
  return finish();
}

extern "C" moe_status moe_fused_status(const void* workspace, int T, int H, int E, int top_k,
                                       int I, void* stream) {
  if (!workspace) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(T, H, E, top_k, I)) return MOE_ERR_UNSUPPORTED_SHAPE;
  Plan p;
  make_plan(T, H, E, top_k, I, &p);
  int32_t code = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&code, at<int32_t>(const_cast<void*>(workspace), p.sync) + moe::kFusedError,
                     sizeof(code), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return MOE_ERR_HIP;
  return code == 0 ? MOE_OK : MOE_ERR_DEVICE_WAIT;
}

// ---- the workspace of moe_forward_noalloc: one fixed array per device ----
//
// A module-scope device array, allocated with the code object when it is loaded on a device
// (each device has its own copy at its own address) and held until the process ends.  In
// host code its name is only a stand-in: the address kernels must receive comes from
// hipGetSymbolAddress, looked up once per device with that device current.  Every call on a
// device shares that device's array; the forward clears what it needs cleared itself (the
// dispatch histograms in the router kernel, the GEMM work queues in the dispatch scan), so
// the contents a previous call left behind are never read.
constexpr size_t kNoallocBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch[kMaxDevices] = {};

// The current device's scratch address (NULL on failure).
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

extern "C" {

moe_status moe_forward_noalloc(const uint16_t* x, const float* router_w, const float* router_b,
                               const uint8_t* w13, const float* w13_scales, const uint16_t* b13,
                               const uint8_t* w2, const float* w2_scales, const uint16_t* b2,
                               int T, int H, int E, int top_k, int I, uint16_t* out,
                               const moe_routing* routing_out, void* stream) {
  if (!shape_ok(T, H, E, top_k, I)) return MOE_ERR_UNSUPPORTED_SHAPE;
  Plan p;
  make_plan(T, H, E, top_k, I, &p);
  if (p.total > kNoallocBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!x || !router_w || !w13 || !w13_scales || !w2 || !w2_scales || !out)
    return MOE_ERR_INVALID_ARG;   // (before the device is touched)
  void* ws = scratch_address();
  if (!ws) return MOE_ERR_HIP;
  return forward_impl(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, T, H, E,
                      top_k, I, out, routing_out, ws, kNoallocBytes, stream, nullptr);
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEVICE_WAIT: return "MOE_ERR_DEVICE_WAIT";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_bytes(int T, int H, int E, int top_k, int I) {
  if (!shape_ok(T, H, E, top_k, I)) return 0;
  Plan p;
  make_plan(T, H, E, top_k, I, &p);
  return p.total;
}

moe_status moe_workspace_layout(int T, int H, int E, int top_k, int I, moe_workspace_regions* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(T, H, E, top_k, I)) return MOE_ERR_UNSUPPORTED_SHAPE;
  Plan p;
  make_plan(T, H, E, top_k, I, &p);
  out->xq = p.xq; out->sx = p.sx; out->h = p.h; out->sh = p.sh; out->y = p.y;
  out->topk_ids = p.ids; out->topk_gates = p.gates; out->expert_counts = p.counts;
  out->expert_offsets = p.offsets; out->perm = p.perm; out->inv_perm = p.inv;
  out->total = p.total;
  return MOE_OK;
}

moe_status moe_quantize_weights(const float* w, int E, int N, int K, uint8_t* codes,
                                float* scales, void* stream) {
  if (!w || !codes || !scales || !aligned16(w) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  if (K % 16 != 0) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (static_cast<long>(E) * ceil_div(N, 128) * ceil_div(K, 128) >= (1L << 31))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  moe::launch_quantize_weights(w, E, N, K, codes, scales, static_cast<hipStream_t>(stream));
  return finish();
}

moe_status moe_quantize_activations(const uint16_t* x, int T, int H, uint8_t* codes,
                                    float* scales, void* stream) {
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || H < 1) return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || static_cast<long>(T) * H >= (1L << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  moe::launch_quantize_act(x, T, H, codes, scales, static_cast<hipStream_t>(stream));
  return finish();
}

moe_status moe_quantize_weights_mx(const float* w, int E, int N, int K, uint8_t* codes,
                                   uint8_t* scales, void* stream) {
  if (!w || !codes || !scales || !aligned16(w) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  if (K % 32 != 0 || N % 16 != 0) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (static_cast<long>(E) * N * 4 * ceil_div(K, 128) / 64 >= (1L << 31))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  moe::launch_quantize_weights_mx(w, E, N, K, codes, scales, static_cast<hipStream_t>(stream));
  return finish();
}

moe_status moe_quantize_weights_mxfp4(const float* w, int E, int N, int K, uint8_t* codes,
                                      uint8_t* scales, void* stream) {
  if (!w || !codes || !scales || !aligned16(w) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  if (K % 32 != 0 || N % 16 != 0) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (static_cast<long>(E) * N * 4 * ceil_div(K, 128) / 64 >= (1L << 31))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  moe::launch_quantize_weights_mxfp4(w, E, N, K, codes, scales, static_cast<hipStream_t>(stream));
  return finish();
}

moe_status moe_quantize_activations_mx(const uint16_t* x, int T, int H, uint8_t* codes,
                                       uint8_t* scales, void* stream) {
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || H < 1) return MOE_ERR_INVALID_ARG;
  if (H % 64 != 0 || static_cast<long>(T) * H >= (1L << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  moe::launch_quantize_act_mx(x, T, H, codes, scales, static_cast<hipStream_t>(stream));
  return finish();
}

moe_status moe_route(const uint16_t* x, const float* router_w, const float* router_b, int T,
                     int H, int E, int top_k, const moe_routing* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!x || !router_w || !workspace || !routing_ok(out) || !aligned16(x) ||
      !aligned16(router_w) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if (!shape_ok(T, H, E, top_k, 64)) return MOE_ERR_UNSUPPORTED_SHAPE;
  Plan p;
  make_plan(T, H, E, top_k, 64, &p);
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (p.presplit && !moe::route_prefill_prepare(E, top_k)) return MOE_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  const Tables tb{out->topk_ids, out->topk_gates, out->expert_counts, out->expert_offsets,
                  out->perm, out->inv_perm};
  enqueue_routing(p, x, router_w, router_b, tb, workspace, static_cast<hipStream_t>(stream));
  return finish();
}

moe_status moe_forward(const uint16_t* x, const float* router_w, const float* router_b,
                       const uint8_t* w13, const float* w13_scales, const uint16_t* b13,
                       const uint8_t* w2, const float* w2_scales, const uint16_t* b2, int T,
                       int H, int E, int top_k, int I, uint16_t* out,
                       const moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return forward_impl(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, T, H, E,
                      top_k, I, out, routing_out, workspace, workspace_bytes, stream, nullptr);
}

moe_status moe_forward_profiled(const uint16_t* x, const float* router_w, const float* router_b,
                                const uint8_t* w13, const float* w13_scales, const uint16_t* b13,
                                const uint8_t* w2, const float* w2_scales, const uint16_t* b2,
                                int T, int H, int E, int top_k, int I, uint16_t* out,
                                const moe_routing* routing_out, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* events) {
  if (!events) return MOE_ERR_INVALID_ARG;   // NULL entries: boundaries not recorded
  return forward_impl(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, T, H, E,
                      top_k, I, out, routing_out, workspace, workspace_bytes, stream,
                      reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)));
}

moe_status moe_forward_mx(const uint16_t* x, const float* router_w, const float* router_b,
                          const uint8_t* w13, const uint8_t* w13_scales, const uint16_t* b13,
                          const uint8_t* w2, const uint8_t* w2_scales, const uint16_t* b2, int T,
                          int H, int E, int top_k, int I, uint16_t* out,
                          const moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return forward_impl(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, T, H, E,
                      top_k, I, out, routing_out, workspace, workspace_bytes, stream, nullptr,
                      kMxfp8);
}

moe_status moe_forward_mx_profiled(const uint16_t* x, const float* router_w,
                                   const float* router_b, const uint8_t* w13,
                                   const uint8_t* w13_scales, const uint16_t* b13,
                                   const uint8_t* w2, const uint8_t* w2_scales, const uint16_t* b2,
                                   int T, int H, int E, int top_k, int I, uint16_t* out,
                                   const moe_routing* routing_out, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events) {
  if (!events) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, T, H, E,
                      top_k, I, out, routing_out, workspace, workspace_bytes, stream,
                      reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), kMxfp8);
}

moe_status moe_forward_mxfp4(const uint16_t* x, const float* router_w, const float* router_b,
                             const uint8_t* w13, const uint8_t* w13_scales, const uint16_t* b13,
                             const uint8_t* w2, const uint8_t* w2_scales, const uint16_t* b2,
                             int T, int H, int E, int top_k, int I, uint16_t* out,
                             const moe_routing* routing_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return forward_impl(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, T, H, E,
                      top_k, I, out, routing_out, workspace, workspace_bytes, stream, nullptr,
                      kMxfp4);
}

moe_status moe_forward_mxfp4_profiled(const uint16_t* x, const float* router_w,
                                      const float* router_b, const uint8_t* w13,
                                      const uint8_t* w13_scales, const uint16_t* b13,
                                      const uint8_t* w2, const uint8_t* w2_scales,
                                      const uint16_t* b2, int T, int H, int E, int top_k, int I,
                                      uint16_t* out, const moe_routing* routing_out,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* events) {
  if (!events) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, T, H, E,
                      top_k, I, out, routing_out, workspace, workspace_bytes, stream,
                      reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), kMxfp4);
}

}  // extern "C"
