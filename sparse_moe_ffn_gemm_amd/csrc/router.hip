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
#include "kernels.hpp"

namespace moe {

typedef float v4f __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------
// logits partials on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): products and
// sums in fp32.  Workgroup tile 64 tokens x 64 experts, 4 waves of 32x32; grid.z
// splits H so that small-T (decode) layers still spread over many CUs.
// ------------------------------------------------------------------------------------
constexpr int kRC = 32;           // H columns staged per step
constexpr int kRS = kRC + 4;      // padded LDS row (floats)

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ W, int T,
                                                            int H, int E, int kslice,
                                                            float* __restrict__ partial,
                                                            int32_t* __restrict__ hist,
                                                            int hist_n) {
  __shared__ __align__(16) float xs[kRouterTile * kRS];
  __shared__ __align__(16) float ws[kRouterTile * kRS];
  {  // clear the dispatch histograms that the top-k step accumulates (a slice per block)
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    const int bid = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int per = (hist_n + nb - 1) / nb;
    const int lo = bid * per, hi = min(hist_n, lo + per);
    for (int i = lo + threadIdx.x; i < hi; i += 256) hist[i] = 0;
  }
  const int t0 = blockIdx.x * kRouterTile, e0 = blockIdx.y * kRouterTile;
  const int h_begin = blockIdx.z * kslice;
  const int h_end = min(H, h_begin + kslice);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  // Two-level fp32 sum: the matrix cores accumulate 128 columns at a time into `acc`,
  // which is then folded into `tot`, so no long running sum absorbs small terms.
  v4f acc[2][2], tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = tot[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int h0 = h_begin; h0 < h_end; h0 += kRC) {
    {  // x: 64 rows x 32 bf16 = 4 chunks of 8 per row, one chunk per lane
      const int row = tid >> 2, c = tid & 3;
      const int t = t0 + row, h = h0 + c * 8;
      float f[8];
      if (t < T && h < h_end) {
        const uint4 raw = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + h);
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = bf16_to_f32(static_cast<uint16_t>(wd[i] & 0xFFFFu));
          f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(wd[i] >> 16));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = 0.f;
      }
      float4* d = reinterpret_cast<float4*>(xs + row * kRS + c * 8);
      d[0] = make_float4(f[0], f[1], f[2], f[3]);
      d[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // W: 64 rows x 32 floats = 8 float4 per row
      const int q = tid + 256 * i;
      const int row = q >> 3, c = q & 7;
      const int e = e0 + row, h = h0 + c * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < E && h < h_end) v = *reinterpret_cast<const float4*>(W + static_cast<size_t>(e) * H + h);
      *reinterpret_cast<float4*>(ws + row * kRS + c * 4) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRC; kk += 4) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = xs[(wm * 32 + 16 * i + (lane & 15)) * kRS + kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = ws[(wn * 32 + 16 * j + (lane & 15)) * kRS + kk + (lane >> 4)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (((h0 - h_begin) / kRC) % 4 == 3 || h0 + kRC >= h_end) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          tot[i][j] += acc[i][j];
          acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
    __syncthreads();
  }
  float* out = partial + static_cast<size_t>(blockIdx.z) * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wm * 32 + 16 * i + 4 * (lane >> 4) + r;
        const int e = e0 + wn * 32 + 16 * j + (lane & 15);
        if (t < T && e < E) out[static_cast<size_t>(t) * E + e] = tot[i][j][r];
      }
}

// ------------------------------------------------------------------------------------
// top-k + softmax: one wave per token, four tokens per workgroup.  Lane l holds experts
// l, l+64, l+128, l+192.  Each round takes the wave-wide (largest value, lowest index)
// and removes it.  The chosen experts are counted into the token's chunk histogram.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void argmax_step(float& v, int& idx, int off) {
  const float ov = __shfl_xor(v, off, 64);
  const int oi = __shfl_xor(idx, off, 64);
  if (ov > v || (ov == v && oi < idx)) {
    v = ov;
    idx = oi;
  }
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
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    if (e < E) {
      float s = 0.f;
      for (int sp = 0; sp < ksplit; ++sp) s += partial[sp * TE + static_cast<size_t>(t) * E + e];
      s += bias ? bias[e] : 0.f;
      v[q] = s == s ? s : -INFINITY;   // a NaN logit never wins
    } else {
      v[q] = -INFINITY;
    }
  }
  // k <= 8 rounds, fully unrolled so that every array stays in registers
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_v[j] = -INFINITY;
    sel_i[j] = 0;
    if (j < top_k) {
      float bv = v[0];
      int bi = lane;
#pragma unroll
      for (int q = 1; q < 4; ++q)
        if (v[q] > bv) {  // strict: ties keep the lower expert index
          bv = v[q];
          bi = lane + 64 * q;
        }
      if (bi >= E) bi = 0x7FFFFFFF;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) argmax_step(bv, bi, off);
      if (bi >= E) bi = 0;             // unreachable for finite inputs; keeps ids in range
      sel_v[j] = bv;
      sel_i[j] = bi;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (bi == lane + 64 * q) v[q] = -INFINITY;
    }
  }
  float z[8], sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    z[j] = j < top_k ? expf(sel_v[j] - sel_v[0]) : 0.f;
    sum += z[j];
  }
  int32_t* h = hist + static_cast<size_t>(t / kChunk) * E;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < top_k && lane == j) {
      ids[static_cast<size_t>(t) * top_k + j] = sel_i[j];
      gates[static_cast<size_t>(t) * top_k + j] = z[j] / sum;
      atomicAdd(&h[sel_i[j]], 1);
    }
}

// ------------------------------------------------------------------------------------
// scan: one workgroup of 1024 lanes; lane (q, e) owns expert e over the q-th quarter of
// the chunks.  counts -> offsets (LDS exclusive scan over experts) -> per-chunk bases,
// then the M-tile list (tiles of bm rows, expert-major) and each expert's first tile.
// ------------------------------------------------------------------------------------
__device__ int exclusive_scan256(int v, int* tmp) {   // lanes [0, 256) hold the values
  const int tid = threadIdx.x;
  if (tid < 256) tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = (tid < 256 && tid >= off) ? tmp[tid - off] : 0;
    __syncthreads();
    if (tid < 256) tmp[tid] += add;
    __syncthreads();
  }
  const int incl = tid < 256 ? tmp[tid] : 0;
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ hist,
                                                             int nchunks, int E, int bm,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ chunk_base,
                                                             MTile* __restrict__ tiles,
                                                             int32_t* __restrict__ num_tiles,
                                                             int32_t* __restrict__ expert_tile_off) {
  __shared__ int part[4][256];
  __shared__ int tmp[256];
  const int tid = threadIdx.x, e = tid & 255, q = tid >> 8;
  const int per = (nchunks + 3) / 4;
  const int c0 = min(nchunks, q * per), c1 = min(nchunks, c0 + per);
  int s = 0;
  if (e < E)
    for (int c = c0; c < c1; ++c) s += hist[static_cast<size_t>(c) * E + e];
  part[q][e] = s;
  __syncthreads();
  const int cnt = part[0][e] + part[1][e] + part[2][e] + part[3][e];   // zero for e >= E
  const int off = exclusive_scan256(cnt, tmp);                          // valid in lanes < 256
  if (tid < 256) tmp[e] = off;
  __syncthreads();
  if (e < E) {
    int run = tmp[e];
    for (int qq = 0; qq < q; ++qq) run += part[qq][e];
    for (int c = c0; c < c1; ++c) {
      chunk_base[static_cast<size_t>(c) * E + e] = run;
      run += hist[static_cast<size_t>(c) * E + e];
    }
    if (q == 0) {
      counts[e] = cnt;
      offsets[e] = tmp[e];
      if (e == E - 1) offsets[E] = tmp[e] + cnt;
    }
  }
  __syncthreads();
  const int ntl = (q == 0 && e < E) ? (cnt + bm - 1) / bm : 0;
  const int toff = exclusive_scan256(ntl, tmp);
  if (q == 0) {
    const int base = off;
    for (int i = 0; i < ntl; ++i) {
      MTile m;
      m.expert = e;
      m.row_begin = base + i * bm;
      m.row_end = min(base + (i + 1) * bm, base + cnt);
      m.pad = 0;
      tiles[toff + i] = m;
    }
    if (e < E) expert_tile_off[e] = toff;
    if (e == 255) {
      num_tiles[0] = toff + ntl;
      expert_tile_off[E] = toff + ntl;
    }
  }
}

// ------------------------------------------------------------------------------------
// scatter: one workgroup per chunk of kChunk tokens.  The chunk's (token, j) entries are
// taken 256 at a time in token order; inside a wave, the lanes whose expert matches a
// lane's expert bit for bit (eight ballots) give its rank; waves before it in the same
// round and earlier rounds (a running per-expert count) give the rest of its slot.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids,
                                                               const int32_t* __restrict__ chunk_base,
                                                               int T, int E, int top_k,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv) {
  __shared__ int run[256];
  __shared__ int wc[4][256];
  const int chunk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = chunk * kChunk;
  const int n = min(kChunk, T - t0) * top_k;
  const size_t flat0 = static_cast<size_t>(t0) * top_k;
  if (tid < E) run[tid] = chunk_base[static_cast<size_t>(chunk) * E + tid];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < n; r += 256) {
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) wc[ww][tid] = 0;
    __syncthreads();
    const int i = r + tid;
    const int ex = i < n ? ids[flat0 + i] : -1;
    unsigned long long peer = __ballot(ex >= 0);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = (ex >> bit) & 1;
      const unsigned long long m = __ballot(set);
      peer &= set ? m : ~m;
    }
    const int rank = __popcll(peer & below);
    if (ex >= 0 && rank == 0) wc[w][ex] = __popcll(peer);
    __syncthreads();
    if (ex >= 0) {
      int pos = run[ex] + rank;
      for (int ww = 0; ww < w; ++ww) pos += wc[ww][ex];
      const int flat = static_cast<int>(flat0) + i;   // = t * top_k + j
      perm[pos] = flat;
      inv[flat] = pos;
    }
    __syncthreads();
    if (tid < E) run[tid] += wc[0][tid] + wc[1][tid] + wc[2][tid] + wc[3][tid];
  }
}

void launch_router_logits(const uint16_t* x, const float* W, int T, int H, int E, int ksplit,
                          int kslice, float* partial, int32_t* hist, int hist_n, hipStream_t st) {
  dim3 grid(ceil_div(T, kRouterTile), ceil_div(E, kRouterTile), ksplit);
  router_logits_kernel<<<grid, dim3(256), 0, st>>>(x, W, T, H, E, kslice, partial, hist, hist_n);
}

void launch_topk(const float* partial, int ksplit, const float* bias, int T, int E, int top_k,
                 int32_t* ids, float* gates, int32_t* hist, hipStream_t st) {
  topk_kernel<<<dim3(ceil_div(T, 4)), dim3(256), 0, st>>>(partial, ksplit, bias, T, E, top_k, ids,
                                                        gates, hist);
}

void launch_dispatch_scan(const int32_t* hist, int nchunks, int E, int bm, int32_t* counts,
                          int32_t* offsets, int32_t* chunk_base, MTile* tiles, int32_t* num_tiles,
                          int32_t* expert_tile_off, hipStream_t st) {
  dispatch_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(hist, nchunks, E, bm, counts, offsets,
                                                       chunk_base, tiles, num_tiles,
                                                       expert_tile_off);
}

void launch_dispatch_scatter(const int32_t* ids, const int32_t* chunk_base, int T, int E,
                             int top_k, int32_t* perm, int32_t* inv, hipStream_t st) {
  dispatch_scatter_kernel<<<dim3(ceil_div(T, kChunk)), dim3(256), 0, st>>>(ids, chunk_base, T, E,
                                                                         top_k, perm, inv);
}

}  // namespace moe
