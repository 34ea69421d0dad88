// Decode-sized layers in one persistent kernel: router GEMM (+ the quantisation of x),
// top-k + softmax, dispatch tables, GEMM1 (+ b13, SwiGLU, requantisation of h), GEMM2
// (+ b2) and the gate-weighted combine.
//
// "Hosting Qwen on Blackwell", section "Expert Parallel": for decode the whole dispatch /
// expert GEMM / combine path is fused into a single kernel, while prefill keeps several
// kernels (its routing needs far fewer workgroups than its combine).  Each stage here runs
// the arithmetic of the multi-kernel path (the same router tile, routing tail, row-run GEMM
// tiles and combine), so a call gives the same bits as the multi-kernel forward of a layer
// that path also runs with the routing tail and the row-run kernels.
//
// Work items come from one queue (a counter in the workspace), in dependency order:
//   [0, R)    router tiles (token tile, expert tile, H slice); the workgroup that finishes
//             the last of them runs the routing tail (logits, top-k + softmax, scan, the
//             16-row M-tile list, scatter) and then raises the routing flag;
//   then M-tile by M-tile the GEMM1 n-tiles (128 h columns each), then M-tile by M-tile
//   the GEMM2 n-tiles (256 output columns each), then the combine items (a token and 2048
//   output columns).
// An item waits only on items taken before it (GEMM1 on the routing flag, GEMM2 of tile m
// on m's GEMM1 n-tiles, the combine on all GEMM2 items), and only running workgroups take
// items, so every wait ends once the earlier items do, however many workgroups are
// resident.  The grid is the number the device holds at once anyway, so no workgroup
// waits for a slot.  Each wait is still bounded: past its bound the workgroup records an
// error code in the workspace and leaves (the layer's output is then incomplete).
//
// Hand-offs between workgroups (the router partials, x codes and scales, the routing
// tables, h and its scales, y) are written and read with device-coherent accesses (the sc1
// cache policy: store_c / load_c, load_lds16_c), so a counter update needs no memory fence:
// each wave waits for its own stores to be acknowledged before the workgroup's one atomic.
// Device-scope fences would write back or invalidate a whole L2 each time (measured on the
// gpt-oss-20b decode layer: with a fence pair at every item the kernel ran 2.4x slower, and
// the routing hand-offs alone cost about 8 us).
#include <algorithm>

#include "combine_dev.hpp"
#include "gemm_dev.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

int g_spin_limit = 1 << 17;   // about 0.2 s of polls (one per ~4k cycles)

// Work items: workgroup b's first ticket is b (the queue head starts at the grid size, so
// the launch does not begin with one atomic per workgroup on one address); after that,
// thread 0 claims a ticket (one atomic on the queue head) one item ahead, so the atomic's
// round trip overlaps the current item; `next_item` hands the claimed ticket to the
// workgroup through LDS and claims the one after it.  A workgroup processes its tickets in
// order, so holding the next one never blocks an earlier item another workgroup waits for.
__device__ __forceinline__ int claim(int32_t* head) {
  return threadIdx.x == 0 ? atomicAdd(head, 1) : 0;
}
__device__ __forceinline__ int next_item(int32_t* head, int& claimed, int* word) {
  __syncthreads();   // every thread has read the previous broadcast
  if (threadIdx.x == 0) *word = claimed;
  __syncthreads();
  const int q = *word;
  claimed = claim(head);
  return q;
}

// Waits until *w >= target: thread 0 polls (relaxed device-scope loads, about one per
// 4k cycles: device-scope accesses to one address are served one after another outside the
// XCDs' L2s, and tighter polling by the waiting workgroups delays the counter updates and
// ticket claims of the working ones -- one poll per 128 cycles took the gpt-oss-20b decode
// layer 227.5 us, one per 4k cycles 215.9 us), the workgroup follows; the handed-off data is
// then read with device-coherent loads.  False (and the error code recorded) after `limit`
// unsuccessful polls.
__device__ __forceinline__ bool wait_at_least(int32_t* w, int target, int32_t* err, int limit,
                                              int* word) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    if (limit < 0) {
      ok = 0;
    } else {
      for (int n = 0; __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target;
           ++n) {
        if (n >= limit) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(60);
      }
    }
    if (!ok) atomicOr(err, kFusedErrWait);
    *word = ok;
  }
  __syncthreads();
  return *word != 0;
}

// Publishes the workgroup's device-coherent stores with one counter update; returns the
// counter's previous value (in every thread).  Every wave first waits until its own stores
// are acknowledged.
__device__ __forceinline__ int publish(int32_t* w, int* word) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) *word = atomicAdd(w, 1);
  __syncthreads();
  return *word;
}

// M-tile m of the list the routing tail wrote (device-coherent loads), wave-uniform.
__device__ __forceinline__ MTile tile_at(const MTile* tiles, int m) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(tiles + m);
  const uint64_t a = load_c<true>(w), b = load_c<true>(w + 1);
  MTile mt;
  mt.expert = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  mt.row_begin = __builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32));
  mt.row_end = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b)));
  mt.pad = 0;
  return mt;
}

// LDS carve of the routing tail (see fused_lds_bytes).
__device__ __forceinline__ TailLds tail_lds(uint8_t* lds, int T, int E, int top_k) {
  const int cs = ceil_div(T, 64) * 64;
  TailLds L;
  L.part = reinterpret_cast<int(*)[256]>(lds);
  L.tmp = reinterpret_cast<int*>(lds + 4096);
  L.hist = reinterpret_cast<int*>(lds + 5120);
  L.sids = reinterpret_cast<int*>(lds + 6144);
  float* logits = reinterpret_cast<float*>(lds + 6144 + 4 * ceil_div(T * top_k, 4) * 4);
  L.logits = logits;
  L.cv = logits + ceil_div(T * (E | 1), 4) * 4;
  L.ci = reinterpret_cast<int*>(L.cv + 32 * cs);
  L.cs = cs;
  return L;
}

// The kernel walks the queue in phases, one loop per kind of item (tickets only grow, so a
// workgroup never returns to an earlier kind): each loop keeps only its own values live, so
// the register demand is the largest single stage's, not their sum.  One workgroup per CU:
// eight waves with two weight bursts each in flight already draw the CU's share of HBM
// (measured on the gpt-oss-20b decode layer: about 5.8 TB/s in the GEMM1 phase with one
// workgroup per CU, the same with two, whose items then took twice as long and stalled
// their GEMM2 successors longer).
template <bool MX, bool FP4>
__global__ __launch_bounds__(512) void moe_decode_fused_kernel(const FusedArgs f) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int word;
  constexpr int KS = 4;   // K-blocks per weight burst of the row-run tiles
  const int R = f.ntx * f.ney * f.ksplit;
  int32_t* const err = f.ctr + kFusedError;
  int32_t* const head = f.ctr + kFusedHead;
  int q = static_cast<int>(blockIdx.x);
  int claimed = claim(head);
  // ---- router tiles: partial logits of one H slice, x codes of its columns ----
  for (; q < R; q = next_item(head, claimed, &word)) {
    const int s = q % f.ksplit, rest = q / f.ksplit;
    const int ey = rest % f.ney, tx = rest / f.ney;
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
    uint16_t* wp = reinterpret_cast<uint16_t*>(lds + kRouterTile * kRS * 2);
    router_tile<false, 512, true>(f.x, f.rw, f.T, f.H, f.E, f.kslice, tx, ey, s, f.partial, f.xq,
                                  f.sx, nullptr, f.sx_mx, xs, wp);
    if (publish(f.ctr + kFusedRouterDone, &word) == R - 1) {
      // the last router tile: every partial and x code is published; route
      route_tail_body<true>(f.partial, f.ksplit, f.rb, f.T, f.E, f.top_k, 16, f.ids, f.gates, f.counts,
                      f.offsets, f.chunk_base, const_cast<MTile*>(f.g1.tiles),
                      const_cast<int32_t*>(f.g1.num_tiles),
                      const_cast<int32_t*>(f.g1.expert_tile_off), f.perm, f.inv,
                      tail_lds(lds, f.T, f.E, f.top_k));
      publish(f.ctr + kFusedRouted, &word);
    }
  }
  // ---- everything after the router waits for the routing tables ----
  if (!wait_at_least(f.ctr + kFusedRouted, 1, err, f.spin_limit, &word)) return;
  const int ntiles = __builtin_amdgcn_readfirstlane(load_c<true>(f.g1.num_tiles));
  const int NT1 = ceil_div(f.I, 128), NT2 = ceil_div(f.H, 256);   // GEMM2 items 256 columns wide
  const int end1 = R + ntiles * NT1, end2 = end1 + ntiles * NT2;
  const int end3 = end2 + f.T * ceil_div(f.H, kFusedCombineCols);
  // ---- GEMM1 n-tile (128 h columns) of M-tile m ----
  for (; q < end1; q = next_item(head, claimed, &word)) {
    const int m = (q - R) / NT1;
    const MTile mt = tile_at(f.g1.tiles, m);
    rowrun_tile<true, KS, MX, FP4, 8, false, 2, true>(f.g1, (q - R) % NT1, mt, lds);
    publish(f.ctr + kFusedCtrTile + m, &word);
  }
  // ---- GEMM2 n-tile (256 output columns: two w2 sub-tiles per wave, the same bytes per
  // item as a GEMM1 n-tile, so the per-item start and drain weigh half as much) of M-tile
  // m, once m's h is complete ----
  int ready_tile = -1;   // the last M-tile whose GEMM1 items this workgroup saw finished
  for (; q < end2; q = next_item(head, claimed, &word)) {
    const int m = (q - end1) / NT2;
    if (m != ready_tile) {
      if (!wait_at_least(f.ctr + kFusedCtrTile + m, NT1, err, f.spin_limit, &word)) return;
      ready_tile = m;
    }
    const MTile mt = tile_at(f.g2.tiles, m);
    rowrun_tile<false, KS, MX, FP4, 8, false, 2, true, true>(f.g2, (q - end1) % NT2, mt, lds);
    publish(f.ctr + kFusedDone2, &word);
  }
  // ---- combine: token t, columns [2048 c, 2048 c + 2048), once every y row is in ----
  if (q < end3 && !wait_at_least(f.ctr + kFusedDone2, ntiles * NT2, err, f.spin_limit, &word))
    return;
  const int NCC = ceil_div(f.H, kFusedCombineCols);
  for (; q < end3; q = next_item(head, claimed, &word)) {
    const int t = (q - end2) / NCC;
    const int c = ((q - end2) % NCC) * kFusedCombineCols + 4 * static_cast<int>(threadIdx.x);
    if (c < f.H) combine_quad<true>(f.y, f.gates, f.inv, f.T * f.top_k, t, c, f.H, f.top_k, f.out);
  }
  // the queue is drained
}

// Zeroes the call's counters, except the queue head: the grid size (the first tickets are
// the workgroups' own indices).
__global__ __launch_bounds__(256) void fused_clear_kernel(int32_t* __restrict__ ctr, int n,
                                                          int grid) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) ctr[i] = i == kFusedHead ? grid : 0;
}

template <bool MX, bool FP4>
const void* fused_fn() {
  return reinterpret_cast<const void*>(moe_decode_fused_kernel<MX, FP4>);
}

const void* fused_fn_of(int fmt) {
  return fmt == 0 ? fused_fn<false, false>() : fmt == 1 ? fused_fn<true, false>()
                                                         : fused_fn<true, true>();
}

}  // namespace

size_t fused_lds_bytes(int T, int H, int E, int top_k, int I) {
  const size_t cs = static_cast<size_t>(ceil_div(T, 64)) * 64;
  const size_t tail = 6144 + 16 * static_cast<size_t>(ceil_div(T * top_k, 4)) +
                      16 * static_cast<size_t>(ceil_div(T * (E | 1), 4)) + 2 * 4 * 32 * cs;
  size_t b = std::max<size_t>(kRouterLds, tail);
  b = std::max(b, rowrun_lds_bytes(H));
  b = std::max(b, rowrun_lds_bytes(I));
  return b;
}

bool fused_prepare(int fmt, size_t lds) {
  if (fmt < 0 || fmt > 2 || lds > 160 * 1024 - 256) return false;   // (+ the static word)
  return hipFuncSetAttribute(fused_fn_of(fmt), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds)) == hipSuccess;
}

int set_fused_spin_limit(int polls) {
  const int prev = g_spin_limit;
  g_spin_limit = polls;
  return prev;
}

void launch_fused(const FusedArgs& f0, int fmt, size_t lds, int max_tiles, long max_items,
                  hipStream_t st) {
  FusedArgs f = f0;
  f.spin_limit = g_spin_limit;
  int dev = 0, cus = 0, per_cu = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_fn_of(fmt), 512, lds);
  long grid = static_cast<long>(std::max(1, cus)) * std::max(1, per_cu);
  grid = std::max(1L, std::min(grid, max_items));
  const int n = kFusedCtrTile + max_tiles;
  fused_clear_kernel<<<dim3(ceil_div(n, 256)), dim3(256), 0, st>>>(f.ctr, n, static_cast<int>(grid));
  const dim3 g(static_cast<unsigned>(grid)), b(512);
  if (fmt == 0)
    moe_decode_fused_kernel<false, false><<<g, b, lds, st>>>(f);
  else if (fmt == 1)
    moe_decode_fused_kernel<true, false><<<g, b, lds, st>>>(f);
  else
    moe_decode_fused_kernel<true, true><<<g, b, lds, st>>>(f);
}

}  // namespace moe
