// Router GEMM, top-k + softmax over the selected logits, and the dispatch tables.
//
// "GPT-OSS on day 0", section "Kernels -> MoE": the router takes the top-k experts
// and the softmax only over the selected logits.  "Hosting Qwen on Blackwell",
// section "Expert Parallel": dispatch aggregates the routing information and
// prepares each expert's token buffer for the grouped GEMM.
//
// The dispatch order is expert-major and token-ascending.  It is built as a stable
// counting sort that is deterministic by construction: per-chunk histograms (integer
// atomics: the counts do not depend on their order), one scan over (expert, chunk),
// then each chunk ranks its entries in token order (wave ballots on the expert bits
// give every entry the number of earlier entries of the same expert).  No slot is ever
// claimed by an atomic, so repeated runs give the same permutation bit for bit.
#include <algorithm>

#include "route_dev.hpp"

namespace moe {

// W [E, H] fp32 -> planes [3][E, H] bf16 (hi, mid, lo), once per call for layers with
// many token tiles, so the router workgroups load the parts instead of each splitting
// its weight tile again.  Also zeroes clr[0, nclr) (the routing kernel's counters and
// histograms).
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ W, long n4,
                                                           long plane, uint16_t* __restrict__ parts,
                                                           int32_t* __restrict__ clr, int nclr) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i < nclr) clr[i] = 0;
  if (i >= n4) return;
  uint2 ph, pm, pl;
  split3(reinterpret_cast<const float4*>(W)[i], ph, pm, pl);
  reinterpret_cast<uint2*>(parts)[i] = ph;
  reinterpret_cast<uint2*>(parts + plane)[i] = pm;
  reinterpret_cast<uint2*>(parts + 2 * plane)[i] = pl;
}

// ------------------------------------------------------------------------------------
// Routing of a prefill-sized layer in one kernel: router GEMM + top-k + softmax.  A
// workgroup of 512 lanes computes one router tile of 64 tokens x 128 experts over one H
// slice (grid: token tiles x expert tiles x slices, at least about one workgroup per CU)
// and stores its partial logits device-coherently; the workgroup that completes a token
// tile's last (expert tile, slice) pair sums that tile's partials and selects its tokens'
// experts (tail_topk, a lane per token), counting them into the dispatch histograms.  The
// logits never leave the chip as a whole array: only the per-slice partials of one
// tile pass between the workgroups, through the L2 / memory-side caches.  Counters and
// histograms are zeroed by the weight split that precedes the kernel.
// ------------------------------------------------------------------------------------
// 64 tokens x 128 experts per workgroup of 512 lanes (measured on the prefill layers
// against 64 x 64 (256 lanes), 128 x 64, 128 x 128 and 256 x 64: the fastest or within
// 5 %; the router GEMM is bound by the per-step load latency of its tiles, not by its
// matrix-core work)
constexpr int kRouteTT = 64, kRouteTE = 128, kRouteThreads = 512;
constexpr int kTopkRows = 64;   // tokens per top-k pass

__global__ __launch_bounds__(kRouteThreads) void route_prefill_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ parts,
    const float* __restrict__ bias, int T, int H, int E, int top_k, int kslice, int ksplit,
    float* __restrict__ partial, uint8_t* __restrict__ xq, float* __restrict__ sx,
    uint8_t* __restrict__ sx_mx, int32_t* __restrict__ ids, float* __restrict__ gates,
    int32_t* __restrict__ hist, int32_t* __restrict__ tile_done) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int word;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  // (the partials pass between this launch's workgroups; x codes and scales only to GEMM1)
  router_tile<true, kRouteThreads, true, kRouteTT, kRouteTE, false>(x, nullptr, T, H, E, kslice, blockIdx.x, blockIdx.y,
                                                   blockIdx.z, partial, xq, sx, parts, sx_mx, xs,
                                                   xs + kRouteTT * kRS);
  // every wave's partial stores acknowledged, then the token tile's counter
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) word = atomicAdd(tile_done + blockIdx.x, 1);
  __syncthreads();
  if (word != static_cast<int>(gridDim.y * gridDim.z) - 1) return;
  // the tile's last pair: logits of its tokens (device-coherent partial loads) and their
  // top-k, 64 tokens at a time (the logits of 64 tokens x 256 experts fit in LDS)
  const int SE = E | 1;
  float* logits = reinterpret_cast<float*>(lds);
  float* cv = logits + ceil_div(kTopkRows * SE, 4) * 4;
  int* ci = reinterpret_cast<int*>(cv + 32 * kTopkRows);
  int* sids = ci + 32 * kTopkRows;
  int32_t* h = hist + static_cast<size_t>(blockIdx.x * kRouteTT / kChunk) * E;   // one chunk
  for (int t0 = blockIdx.x * kRouteTT; t0 < min(T, (blockIdx.x + 1) * kRouteTT); t0 += kTopkRows) {
    const int nt = min(kTopkRows, T - t0);
    if (ksplit <= 2)
      tail_logits<2, true, 8>(partial, ksplit, bias, T, E, SE, logits, t0, nt);
    else if (ksplit <= 4)
      tail_logits<4, true, 8>(partial, ksplit, bias, T, E, SE, logits, t0, nt);
    else if (ksplit <= 8)
      tail_logits<8, true, 8>(partial, ksplit, bias, T, E, SE, logits, t0, nt);
    else if (ksplit <= 16)
      tail_logits<16, true, 8>(partial, ksplit, bias, T, E, SE, logits, t0, nt);
    else if (ksplit <= 32)
      tail_logits<32, true, 8>(partial, ksplit, bias, T, E, SE, logits, t0, nt);
    else
      tail_logits<64, true, 8>(partial, ksplit, bias, T, E, SE, logits, t0, nt);
    __syncthreads();
    int32_t* id = ids + static_cast<size_t>(t0) * top_k;
    float* gt = gates + static_cast<size_t>(t0) * top_k;
    if (top_k <= 2)
      tail_topk<2>(logits, SE, nt, E, top_k, cv, ci, kTopkRows, id, gt, sids, h);
    else if (top_k <= 4)
      tail_topk<4>(logits, SE, nt, E, top_k, cv, ci, kTopkRows, id, gt, sids, h);
    else
      tail_topk<8>(logits, SE, nt, E, top_k, cv, ci, kTopkRows, id, gt, sids, h);
    __syncthreads();
  }
}

// LDS of route_prefill_kernel: the router tile, or the top-k stage's logits, candidate
// lists and ids (whichever is larger).
static size_t route_prefill_lds(int E, int top_k) {
  const size_t tile = router_lds<kRouteTT, kRouteTE>();
  const size_t topk = 4 * static_cast<size_t>(ceil_div(kTopkRows * (E | 1), 4) * 4) +
                      2 * 4 * 32 * kTopkRows + 4 * static_cast<size_t>(kTopkRows) * top_k;
  return std::max(tile, topk);
}

// One router tile per workgroup: grid (token tiles, expert tiles, H slices).
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ W, int T,
                                                            int H, int E, int kslice,
                                                            float* __restrict__ partial,
                                                            int32_t* __restrict__ hist,
                                                            int hist_n, uint8_t* __restrict__ xq,
                                                            float* __restrict__ sx,
                                                            uint8_t* __restrict__ sx_mx) {
  __shared__ __align__(16) uint16_t xs[kRouterTile * kRS];
  __shared__ __align__(16) uint16_t wp[3][kRouterTile * kRS];   // hi, mid, lo parts of W
  {  // clear the dispatch histograms that the top-k step accumulates (a slice per block)
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    const int bid = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int per = (hist_n + nb - 1) / nb;
    const int lo = bid * per, hi = min(hist_n, lo + per);
    for (int i = lo + threadIdx.x; i < hi; i += 256) hist[i] = 0;
  }
  router_tile<false, 256>(x, W, T, H, E, kslice, blockIdx.x, blockIdx.y, blockIdx.z, partial, xq,
                          sx, nullptr, sx_mx, xs, &wp[0][0]);
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int ksplit,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int top_k, int32_t* __restrict__ ids,
                                                   float* __restrict__ gates,
                                                   int32_t* __restrict__ hist) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t TE = static_cast<size_t>(T) * E;
  float v[1][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[0][q] = e < E ? logit_of(partial, ksplit, bias, TE, static_cast<size_t>(t) * E + e, e)
                    : -INFINITY;
  }
  int id[1];
  float g[1];
  topk_select<1>(v, E, top_k, lane, id, g);
  if (lane < top_k) {
    ids[static_cast<size_t>(t) * top_k + lane] = id[0];
    gates[static_cast<size_t>(t) * top_k + lane] = g[0];
    atomicAdd(&hist[static_cast<size_t>(t / kChunk) * E + id[0]], 1);
  }
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ hist,
                                                             int nchunks, int E, int bm, int xr,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ chunk_base,
                                                             MTile* __restrict__ tiles,
                                                             int32_t* __restrict__ num_tiles,
                                                             int32_t* __restrict__ expert_tile_off,
                                                             const int32_t* __restrict__ ids, int T,
                                                             int top_k, int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv) {
  __shared__ int part[4][256];
  __shared__ int tmp[256];
  dispatch_scan_body(hist, nchunks, E, bm, xr, counts, offsets, chunk_base, tiles, num_tiles,
                     expert_tile_off, ids, T, top_k, perm, inv, part, tmp);
}

// ------------------------------------------------------------------------------------
// Routing tail of a decode-sized layer (T <= kChunk, one dispatch chunk, T E <=
// kTailLogits, at most kTailSplit H slices) in one workgroup of 16 waves: the router
// partials summed into LDS logits (all slice loads of a logit in flight together), top-k
// + softmax with a lane per token (tail_topk), then the scan, the M-tile list and the
// scatter.  Replaces three launches on the latency-bound path.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void route_tail_kernel(const float* __restrict__ partial,
                                                          int ksplit,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int top_k, int bm,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ gates,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ chunk_base,
                                                          MTile* __restrict__ tiles,
                                                          int32_t* __restrict__ num_tiles,
                                                          int32_t* __restrict__ expert_tile_off,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
  __shared__ int part[4][256];
  __shared__ int tmp[256];
  __shared__ int hist[256];
  __shared__ int sids[kChunk * 8];
  __shared__ float logits[kTailLogits + kChunk];   // rows of SE = E | 1 (odd: no bank conflicts)
  __shared__ float cv[kChunk * 4 * 8];
  __shared__ int ci[kChunk * 4 * 8];
  route_tail_body(partial, ksplit, bias, T, E, top_k, bm, ids, gates, counts, offsets, chunk_base,
                  tiles, num_tiles, expert_tile_off, perm, inv,
                  TailLds{part, tmp, hist, sids, logits, cv, ci, kChunk});
}

// One workgroup per chunk.
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids,
                                                               const int32_t* __restrict__ chunk_base,
                                                               int T, int E, int top_k,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv) {
  __shared__ int run[256];
  __shared__ int wc[4][256];
  const int chunk = blockIdx.x, tid = threadIdx.x;
  if (tid < E) run[tid] = chunk_base[static_cast<size_t>(chunk) * E + tid];
  scatter_chunk(ids, chunk, T, E, top_k, perm, inv, run, wc);
}

void launch_router_logits(const uint16_t* x, const float* W, int T, int H, int E, int ksplit,
                          int kslice, float* partial, int32_t* hist, int hist_n, hipStream_t st,
                          uint8_t* xq, float* sx, uint8_t* sx_mx) {
  dim3 grid(ceil_div(T, kRouterTile), ceil_div(E, kRouterTile), ksplit);
  router_logits_kernel<<<grid, dim3(256), 0, st>>>(x, W, T, H, E, kslice, partial, hist, hist_n, xq,
                                                   sx, sx_mx);
}

void route_prefill_shape(int T, int H, int E, int* ksplit, int* kslice) {
  const int tiles = ceil_div(T, kRouteTT) * ceil_div(E, kRouteTE);
  int ks = std::max(1, std::min(ceil_div(256, tiles), H / kBlock));
  int sl = ceil_div(ceil_div(H, ks), kBlock) * kBlock;
  *kslice = sl;
  *ksplit = ceil_div(H, sl);
}

bool route_prefill_prepare(int E, int top_k) {
  const size_t lds = route_prefill_lds(E, top_k);
  if (lds > 160 * 1024 - 256) return false;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(route_prefill_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds)) == hipSuccess;
}

void launch_route_prefill(const uint16_t* x, const float* W, const float* bias, int T, int H, int E,
                          int top_k, int ksplit, int kslice, uint16_t* parts, float* partial,
                          uint8_t* xq, float* sx, uint8_t* sx_mx, int32_t* ids, float* gates,
                          int32_t* hist, int nchunks, int32_t* tile_done, hipStream_t st) {
  const long n4 = static_cast<long>(E) * H / 4;   // H is a multiple of 64
  const int nclr = nchunks * E + ceil_div(T, kRouteTT);   // hist, then tile_done (contiguous)
  const long nsplit = std::max<long>(n4, nclr);
  router_split_kernel<<<dim3(static_cast<unsigned>((nsplit + 255) / 256)), dim3(256), 0, st>>>(
      W, n4, static_cast<long>(E) * H, parts, hist, nclr);
  dim3 grid(ceil_div(T, kRouteTT), ceil_div(E, kRouteTE), ksplit);
  route_prefill_kernel<<<grid, dim3(kRouteThreads), route_prefill_lds(E, top_k), st>>>(
      x, parts, bias, T, H, E, top_k, kslice, ksplit, partial, xq, sx, sx_mx, ids, gates, hist,
      tile_done);
}

void launch_topk(const float* partial, int ksplit, const float* bias, int T, int E, int top_k,
                 int32_t* ids, float* gates, int32_t* hist, hipStream_t st) {
  topk_kernel<<<dim3(ceil_div(T, 4)), dim3(256), 0, st>>>(partial, ksplit, bias, T, E, top_k, ids,
                                                        gates, hist);
}

void launch_dispatch_scan(const int32_t* hist, int nchunks, int E, int bm, int xr, int32_t* counts,
                          int32_t* offsets, int32_t* chunk_base, MTile* tiles, int32_t* num_tiles,
                          int32_t* expert_tile_off, hipStream_t st, const int32_t* ids, int T,
                          int top_k, int32_t* perm, int32_t* inv) {
  dispatch_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(hist, nchunks, E, bm, xr, counts, offsets,
                                                       chunk_base, tiles, num_tiles,
                                                       expert_tile_off, ids, T, top_k, perm, inv);
}

void launch_route_tail(const float* partial, int ksplit, const float* bias, int T, int E,
                       int top_k, int bm, int32_t* ids, float* gates, int32_t* counts,
                       int32_t* offsets, int32_t* chunk_base, MTile* tiles, int32_t* num_tiles,
                       int32_t* expert_tile_off, int32_t* perm, int32_t* inv, hipStream_t st) {
  route_tail_kernel<<<dim3(1), dim3(1024), 0, st>>>(partial, ksplit, bias, T, E, top_k, bm, ids,
                                                    gates, counts, offsets, chunk_base, tiles,
                                                    num_tiles, expert_tile_off, perm, inv);
}

// The activation scale words of the routed rows, in dispatch order and K-block major, for
// the large-group GEMMs (the 256 rows of a tile then read one contiguous run per K-step
// instead of a word from each row): x's gathered through perm for GEMM1, h's (already in
// dispatch order, perm NULL) for GEMM2.  Thread i = j * rows + p.
__global__ __launch_bounds__(256) void gather_row_scales_kernel(const uint32_t* __restrict__ src,
                                                                int KB,
                                                                const int32_t* __restrict__ perm,
                                                                int top_k, int rows,
                                                                uint32_t* __restrict__ dst) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long>(rows) * KB) return;
  const int j = static_cast<int>(i / rows), p = static_cast<int>(i % rows);
  const int t = perm != nullptr ? perm[p] / top_k : p;
  dst[i] = src[static_cast<long>(t) * KB + j];
}

void launch_gather_row_scales(const uint32_t* src, int KB, const int32_t* perm, int top_k,
                              int rows, uint32_t* dst, hipStream_t st) {
  const long n = static_cast<long>(rows) * KB;
  gather_row_scales_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st>>>(
      src, KB, perm, top_k, rows, dst);
}

void launch_dispatch_scatter(const int32_t* ids, const int32_t* chunk_base, int T, int E,
                             int top_k, int32_t* perm, int32_t* inv, hipStream_t st) {
  dispatch_scatter_kernel<<<dim3(ceil_div(T, kChunk)), dim3(256), 0, st>>>(ids, chunk_base, T, E,
                                                                         top_k, perm, inv);
}

}  // namespace moe
