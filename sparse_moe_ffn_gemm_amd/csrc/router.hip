// Router GEMM, top-k + softmax over the selected logits, and the dispatch tables.
//
// "GPT-OSS on day 0", section "Kernels -> MoE": the router takes the top-k experts
// and the softmax only over the selected logits.  "Hosting Qwen on Blackwell",
// section "Expert Parallel": dispatch aggregates the routing information and
// prepares each expert's token buffer for the grouped GEMM.
//
// The dispatch order is expert-major and token-ascending.  It is built as a
// counting sort that is deterministic by construction: per-chunk histograms (LDS
// atomics, order-free), one scan, then each expert's lane walks its chunk in token
// order.  No slot is ever claimed by a global atomic, so repeated runs give the
// same permutation bit for bit.
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
                                                            float* __restrict__ partial) {
  __shared__ __align__(16) float xs[kRouterTile * kRS];
  __shared__ __align__(16) float ws[kRouterTile * kRS];
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
// top-k + softmax: one wave per token.  Lane l holds experts l, l+64, l+128, l+192.
// Each round takes the wave-wide (largest value, lowest index) and removes it.
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
  __shared__ int h_lds[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) h_lds[e] = 0;
  __syncthreads();
  const int chunk = blockIdx.x;
  const size_t TE = static_cast<size_t>(T) * E;
  for (int tt = wave; tt < kChunk; tt += 4) {
    const int t = chunk * kChunk + tt;
    if (t >= T) break;
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
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < top_k && lane == j) {
        ids[static_cast<size_t>(t) * top_k + j] = sel_i[j];
        gates[static_cast<size_t>(t) * top_k + j] = z[j] / sum;
        atomicAdd(&h_lds[sel_i[j]], 1);
      }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) hist[static_cast<size_t>(chunk) * E + e] = h_lds[e];
}

// ------------------------------------------------------------------------------------
// scan: lane e owns expert e.  counts -> offsets (LDS exclusive scan) -> per-chunk
// bases, then the M-tile list (tiles of bm rows, expert-major).
// ------------------------------------------------------------------------------------
__device__ int block_exclusive_scan(int v, int* tmp) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int incl = tmp[tid];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void dispatch_scan_kernel(const int32_t* __restrict__ hist,
                                                            int nchunks, int E, int bm,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ chunk_base,
                                                            MTile* __restrict__ tiles,
                                                            int32_t* __restrict__ num_tiles,
                                                            int32_t* __restrict__ expert_tile_off) {
  __shared__ int tmp[256];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E)
    for (int c = 0; c < nchunks; ++c) cnt += hist[static_cast<size_t>(c) * E + e];
  const int off = block_exclusive_scan(cnt, tmp);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = off + cnt;
    int run = off;
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[static_cast<size_t>(c) * E + e] = run;
      run += hist[static_cast<size_t>(c) * E + e];
    }
  }
  const int nt = e < E ? (cnt + bm - 1) / bm : 0;
  const int toff = block_exclusive_scan(nt, tmp);
  for (int i = 0; i < nt; ++i) {
    MTile m;
    m.expert = e;
    m.row_begin = off + i * bm;
    m.row_end = min(off + (i + 1) * bm, off + cnt);
    m.pad = 0;
    tiles[toff + i] = m;
  }
  if (e < E) expert_tile_off[e] = toff;
  if (e == 255) {
    num_tiles[0] = toff + nt;
    expert_tile_off[E] = toff + nt;
  }
}

// ------------------------------------------------------------------------------------
// scatter: one workgroup per chunk; lane e walks the chunk's (token, j) entries in
// token order and appends the ones routed to expert e.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids,
                                                               const int32_t* __restrict__ chunk_base,
                                                               int T, int E, int top_k,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv) {
  __shared__ int ids_lds[kChunk * 8];
  const int chunk = blockIdx.x, tid = threadIdx.x;
  const int t0 = chunk * kChunk;
  const int nt = min(kChunk, T - t0);
  const int n = nt * top_k;
  for (int i = tid; i < n; i += 256) ids_lds[i] = ids[static_cast<size_t>(t0) * top_k + i];
  __syncthreads();
  const int e = tid;
  if (e >= E) return;
  int pos = chunk_base[static_cast<size_t>(chunk) * E + e];
  for (int i = 0; i < n; ++i) {
    if (ids_lds[i] == e) {
      const int flat = t0 * top_k + i;   // = t * top_k + j
      perm[pos] = flat;
      inv[flat] = pos;
      ++pos;
    }
  }
}

void launch_router_logits(const uint16_t* x, const float* W, int T, int H, int E, int ksplit,
                          int kslice, float* partial, hipStream_t st) {
  dim3 grid(ceil_div(T, kRouterTile), ceil_div(E, kRouterTile), ksplit);
  router_logits_kernel<<<grid, dim3(256), 0, st>>>(x, W, T, H, E, kslice, partial);
}

void launch_topk(const float* partial, int ksplit, const float* bias, int T, int E, int top_k,
                 int32_t* ids, float* gates, int32_t* hist, hipStream_t st) {
  topk_kernel<<<dim3(ceil_div(T, kChunk)), dim3(256), 0, st>>>(partial, ksplit, bias, T, E, top_k,
                                                             ids, gates, hist);
}

void launch_dispatch_scan(const int32_t* hist, int nchunks, int E, int bm, int32_t* counts,
                          int32_t* offsets, int32_t* chunk_base, MTile* tiles, int32_t* num_tiles,
                          int32_t* expert_tile_off, hipStream_t st) {
  dispatch_scan_kernel<<<dim3(1), dim3(256), 0, st>>>(hist, nchunks, E, bm, counts, offsets,
                                                       chunk_base, tiles, num_tiles,
                                                       expert_tile_off);
}

void launch_dispatch_scatter(const int32_t* ids, const int32_t* chunk_base, int T, int E,
                             int top_k, int32_t* perm, int32_t* inv, hipStream_t st) {
  dispatch_scatter_kernel<<<dim3(ceil_div(T, kChunk)), dim3(256), 0, st>>>(ids, chunk_base, T, E,
                                                                         top_k, perm, inv);
}

}  // namespace moe
