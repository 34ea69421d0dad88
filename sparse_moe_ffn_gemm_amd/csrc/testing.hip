// Test-only entry point: one grouped GEMM of the layer with the raw fp32 accumulators as its
// output (include/moe_test.h).  It launches the same kernels as moe_forward, on a tile list
// built here on the host from the caller's per-expert row counts.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "moe_test.h"
#include "kernels.hpp"

namespace {

using moe::ceil_div;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct RawPlan {
  size_t tiles, num_tiles, expert_tile_off, sd, total;
};

// The tile list is sized for 16-row tiles (the most of any tile height).
RawPlan raw_plan(long rows, int E, int K) {
  RawPlan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  p.tiles = take(sizeof(moe::MTile) * static_cast<size_t>(rows / 16 + std::min<long>(E, rows)));
  p.num_tiles = take(sizeof(int32_t) * moe::kQueueStride * (1 + 2 * moe::kGemmQueues));
  p.expert_tile_off = take(sizeof(int32_t) * (E + 1));
  p.sd = take(sizeof(uint32_t) * static_cast<size_t>(rows) * ceil_div(K, moe::kBlock));
  p.total = off;
  return p;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

}  // namespace

extern "C" {

size_t moe_test_gemm_raw_workspace_bytes(int rows, int E, int K) {
  if (rows < 0 || E < 1 || E > 256 || K < 64) return 0;
  return raw_plan(rows, E, K).total;
}

moe_status moe_test_gemm_raw(int gemm, int format, int bm, const uint8_t* A,
                             const void* A_scales, int A_rows, const int32_t* perm, int top_k,
                             const int32_t* expert_counts, int E, const uint8_t* B,
                             const void* B_scales, int N, int K, float* C, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if ((gemm != 1 && gemm != 2) || format < 0 || format > 2) return MOE_ERR_INVALID_ARG;
  if (!A || !A_scales || !expert_counts || !B || !B_scales || !C || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (gemm == 1 && (!perm || top_k < 1)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(A_scales) & 3u) || (reinterpret_cast<uintptr_t>(B_scales) & 3u))
    return MOE_ERR_INVALID_ARG;
  if (E < 1 || E > 256 || A_rows < 1 || N < 64 || N % 64 != 0 || K < 64 || K % 64 != 0)
    return MOE_ERR_UNSUPPORTED_SHAPE;
  if (bm != 16 && bm != 64 && bm != 128 && bm != 256) return MOE_ERR_UNSUPPORTED_SHAPE;
  long rows = 0;
  for (int e = 0; e < E; ++e) {
    if (expert_counts[e] < 0) return MOE_ERR_INVALID_ARG;
    rows += expert_counts[e];
  }
  if (rows * K >= (1L << 31) || static_cast<long>(N) * K >= (1L << 31) ||
      static_cast<long>(A_rows) * K >= (1L << 31))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  if (gemm == 2 && A_rows < rows) return MOE_ERR_UNSUPPORTED_SHAPE;
  const bool mx = format != 0, fp4 = format == 2;
  if (mx && bm != 16 && bm != 256) return MOE_ERR_UNSUPPORTED_SHAPE;   // the plan's MX tiles
  if (!moe::gemm_prepare(gemm == 1, mx, fp4, K, bm, /*raw=*/true)) return MOE_ERR_UNSUPPORTED_SHAPE;
  const RawPlan p = raw_plan(rows, E, K);
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (rows == 0) return MOE_OK;

  // the tile list: bm-row tiles per expert, expert-major, by the forward's rule (the last
  // tile of a block-scaled or MXFP8 256-row launch may hold moe::kBigExtraRows more);
  // work-queue heads zero
  const int xr = !fp4 && bm == 256 ? moe::big_extra_rows(rows, E) : 0;
  std::vector<moe::MTile> tiles;
  std::vector<int32_t> tile_off(E + 1), head(moe::kQueueStride * (1 + 2 * moe::kGemmQueues), 0);
  int off = 0;
  for (int e = 0; e < E; ++e) {
    tile_off[e] = static_cast<int32_t>(tiles.size());
    const int cnt = expert_counts[e], n = moe::expert_tiles(cnt, bm, xr);
    for (int i = 0; i < n; ++i)
      tiles.push_back(moe::MTile{e, off + i * bm, off + (i + 1 < n ? (i + 1) * bm : cnt), 0});
    off += cnt;
  }
  tile_off[E] = static_cast<int32_t>(tiles.size());
  head[0] = static_cast<int32_t>(tiles.size());

  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto* d_tiles = reinterpret_cast<moe::MTile*>(ws + p.tiles);
  auto* d_num = reinterpret_cast<int32_t*>(ws + p.num_tiles);
  auto* d_off = reinterpret_cast<int32_t*>(ws + p.expert_tile_off);
  bool ok = hipMemcpyAsync(d_tiles, tiles.data(), sizeof(moe::MTile) * tiles.size(),
                           hipMemcpyHostToDevice, st) == hipSuccess;
  ok = ok && hipMemcpyAsync(d_num, head.data(), sizeof(int32_t) * head.size(),
                            hipMemcpyHostToDevice, st) == hipSuccess;
  ok = ok && hipMemcpyAsync(d_off, tile_off.data(), sizeof(int32_t) * tile_off.size(),
                            hipMemcpyHostToDevice, st) == hipSuccess;

  moe::GemmArgs g{};
  g.A = A;
  g.A_rows = A_rows;
  g.perm = gemm == 1 ? perm : nullptr;
  g.top_k = gemm == 1 ? top_k : 1;
  g.B = B;
  g.mx = mx;
  g.fp4 = fp4;
  if (mx) {
    g.A_mx = static_cast<const uint8_t*>(A_scales);
    g.B_mx = static_cast<const uint8_t*>(B_scales);
  } else {
    g.A_scale = static_cast<const float*>(A_scales);
    g.B_scale = static_cast<const float*>(B_scales);
  }
  g.bias = nullptr;
  g.tiles = d_tiles;
  g.num_tiles = d_num;
  g.expert_tile_off = d_off;
  g.queue = d_num + moe::kQueueStride;
  g.E = E;
  g.K = K;
  g.N = N;
  g.I = gemm == 1 ? N / 2 : K;
  g.c_raw = C;
  g.xr = xr;
  if (ok && bm == 256) {   // the large-group kernels read the A scale words K-block major
    moe::launch_gather_row_scales(static_cast<const uint32_t*>(A_scales), ceil_div(K, moe::kBlock),
                                  g.perm, g.top_k, static_cast<int>(rows),
                                  reinterpret_cast<uint32_t*>(ws + p.sd), st);
    g.A_sd = reinterpret_cast<const uint32_t*>(ws + p.sd);
    g.sd_rows = static_cast<int>(rows);
  }
  if (ok) moe::launch_gemm_raw(gemm == 1, g, bm, static_cast<int>(tiles.size()), st);
  ok = ok && hipGetLastError() == hipSuccess;
  ok = (hipStreamSynchronize(st) == hipSuccess) && ok;   // the host tile list lives until here
  return ok ? MOE_OK : MOE_ERR_HIP;
}

int moe_test_set_fused_spin_limit(int polls) { return moe::set_fused_spin_limit(polls); }

}  // extern "C"
