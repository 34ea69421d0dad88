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
// logits partials on the bf16 matrix cores with fp32 accumulation, exactly as in fp32:
// x is bf16 already, and every fp32 weight w is split by truncation into three bf16
// parts w = hi + mid + lo (8 + 8 + 8 significant bits, no rounding anywhere), so each
// product x * part is exact in fp32 and x . w = x . hi + x . mid + x . lo is summed in
// fp32 by v_mfma_f32_16x16x32_bf16 (three times the products of an fp32 GEMM at eight
// times the fp32 matrix rate).  Workgroup tile 64 tokens x 64 experts, 4 waves of
// 32 x 32; grid.z splits H (in whole 128-column groups) so that small-T (decode) layers
// still spread over many CUs.  A step stages 128 columns of x and W in LDS while the
// next step's are loaded into registers; the matrix cores accumulate one step into
// `acc`, folded into `tot`, so no long running sum absorbs small terms.
//
// The workgroups of the first expert tile also quantise the x tile they staged (one
// 1x128 group per token and step, or four 1x32 MX blocks, the same rule and code as the
// activation quantiser), so x is read from HBM once for both uses.
// ------------------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int kRC = 128;          // H columns staged per step (one quantisation group)
constexpr int kRS = kRC + 8;      // padded LDS row (bf16): 272-byte rows spread the banks

__device__ __forceinline__ v8bf lds_bf8(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(v8bf, u);
}

// Exact three-way split of four fp32 weights into bf16 parts (hi, mid, lo), packed two
// per dword: w = hi + mid + lo by truncation, no rounding anywhere.
__device__ __forceinline__ void split3(const float4 v, uint2& ph, uint2& pm, uint2& pl) {
  const float w[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[2] = {0u, 0u}, m[2] = {0u, 0u}, l[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = __float_as_uint(w[k]);
    const float hi = __uint_as_float(u & 0xFFFF0000u);
    const float r1 = w[k] - hi;                                  // exact
    const uint32_t um = __float_as_uint(r1);
    const float mid = __uint_as_float(um & 0xFFFF0000u);
    const float lo = r1 - mid;                                   // exact, <= 8 bits
    h[k >> 1] |= (u >> 16) << (16 * (k & 1));
    m[k >> 1] |= (um >> 16) << (16 * (k & 1));
    l[k >> 1] |= (__float_as_uint(lo) >> 16) << (16 * (k & 1));
  }
  ph = make_uint2(h[0], h[1]);
  pm = make_uint2(m[0], m[1]);
  pl = make_uint2(l[0], l[1]);
}

// W [E, H] fp32 -> planes [3][E, H] bf16 (hi, mid, lo), once per call for layers with
// many token tiles, so the router workgroups load the parts instead of each splitting
// its weight tile again.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ W, long n4,
                                                           long plane, uint16_t* __restrict__ parts) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  uint2 ph, pm, pl;
  split3(reinterpret_cast<const float4*>(W)[i], ph, pm, pl);
  reinterpret_cast<uint2*>(parts)[i] = ph;
  reinterpret_cast<uint2*>(parts + plane)[i] = pm;
  reinterpret_cast<uint2*>(parts + 2 * plane)[i] = pl;
}

template <bool PRESPLIT>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ W, int T,
                                                            int H, int E, int kslice,
                                                            float* __restrict__ partial,
                                                            int32_t* __restrict__ hist,
                                                            int hist_n, uint8_t* __restrict__ xq,
                                                            float* __restrict__ sx,
                                                            const uint16_t* __restrict__ parts,
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
  const int t0 = blockIdx.x * kRouterTile, e0 = blockIdx.y * kRouterTile;
  const int h_begin = blockIdx.z * kslice;
  const int h_end = min(H, h_begin + kslice);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const bool quant = xq != nullptr && blockIdx.y == 0;
  const int KBH = ceil_div(H, kBlock);
  v4f acc[2][2], tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) tot[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // one step's global loads: x 64 rows x 16 chunks of 8 bf16; W 64 rows x 32 float4, or
  // (pre-split) three planes of 64 rows x 16 chunks of 8 bf16
  uint4 xr[4];
  float4 wr[PRESPLIT ? 1 : 8];
  uint4 pr[PRESPLIT ? 12 : 1];
  const long plane = static_cast<long>(E) * H;
  auto load = [&](int h0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      const int t = t0 + (q >> 4), h = h0 + (q & 15) * 8;
      xr[i] = make_uint4(0u, 0u, 0u, 0u);
      if (t < T && h < h_end) xr[i] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + h);
    }
    if constexpr (PRESPLIT) {
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        const int q = tid + 256 * (i & 3), pl = i >> 2;
        const int e = e0 + (q >> 4), h = h0 + (q & 15) * 8;
        pr[i] = make_uint4(0u, 0u, 0u, 0u);
        if (e < E && h < h_end)
          pr[i] = *reinterpret_cast<const uint4*>(parts + pl * plane + static_cast<size_t>(e) * H + h);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = tid + 256 * i;
        const int e = e0 + (q >> 5), h = h0 + (q & 31) * 4;
        wr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < E && h < h_end) wr[i] = *reinterpret_cast<const float4*>(W + static_cast<size_t>(e) * H + h);
      }
    }
  };
  if (h_begin < h_end) load(h_begin);
  for (int h0 = h_begin; h0 < h_end; h0 += kRC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      *reinterpret_cast<uint4*>(xs + (q >> 4) * kRS + (q & 15) * 8) = xr[i];
    }
    if constexpr (PRESPLIT) {
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        const int q = tid + 256 * (i & 3);
        *reinterpret_cast<uint4*>(&wp[i >> 2][(q >> 4) * kRS + (q & 15) * 8]) = pr[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {   // split in 3 exact bf16 parts
        const int q = tid + 256 * i;
        const int row = q >> 5, c = q & 31;
        uint2 ph, pm, pl;
        split3(wr[i], ph, pm, pl);
        *reinterpret_cast<uint2*>(&wp[0][row * kRS + c * 4]) = ph;
        *reinterpret_cast<uint2*>(&wp[1][row * kRS + c * 4]) = pm;
        *reinterpret_cast<uint2*>(&wp[2][row * kRS + c * 4]) = pl;
      }
    }
    __syncthreads();
    if (h0 + kRC < h_end) load(h0 + kRC);   // next step's loads fly during this step
    if (quant) {   // 16 lanes per token group, 16 tokens per pass
      const int g = h0 / kBlock;
#pragma unroll
      for (int pass = 0; pass < kRouterTile / 16; ++pass) {
        const int row = pass * 16 + (tid >> 4), col = 8 * (tid & 15);
        const int t = t0 + row;
        const bool in = t < T && h0 + col < h_end;
        uint8_t* codes_row = xq + static_cast<size_t>(t < T ? t : 0) * H + h0;
        if (sx_mx != nullptr) {   // MXFP8: four lanes per 32-block, pads past H get 127
          const int code = quantize_mx8(xs + row * kRS, col, in, codes_row);
          if ((tid & 3) == 0 && t < T)
            sx_mx[static_cast<size_t>(t) * 4 * KBH + (h0 + col) / kMxBlock] = static_cast<uint8_t>(code);
        } else {
          const float sc = quantize_group16(xs + row * kRS, col, in, codes_row);
          if ((tid & 15) == 0 && t < T) sx[static_cast<size_t>(t) * KBH + g] = sc;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kRC; kk += 32) {
      const int kofs = kk + 8 * (lane >> 4);
      v8bf a[2], b[3][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = lds_bf8(xs + (wm * 32 + 16 * i + (lane & 15)) * kRS + kofs);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j) b[p][j] = lds_bf8(&wp[p][(wn * 32 + 16 * j + (lane & 15)) * kRS + kofs]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int p = 0; p < 3; ++p)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[p][j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) tot[i][j] += acc[i][j];
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
// (v, idx) := the larger of (v, idx) and (ov, oi): larger value, ties to the lower index
// (a total order, so any reduction tree gives the same winner).
__device__ __forceinline__ void argmax_take(float& v, int& idx, float ov, int oi) {
  if (ov > v || (ov == v && oi < idx)) {
    v = ov;
    idx = oi;
  }
}

template <int CTRL>
__device__ __forceinline__ int dpp_row_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Wave-wide argmax, left in every lane, on the vector ALU only: DPP row rotations by 8, 4,
// 2 and 1 give every lane its row of 16's winner, then the four rows' winners are read
// from lanes 0, 16, 32 and 48 (no LDS permutes, which serialise on the CU's LDS when many
// waves select at once).
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
  argmax_take(v, idx, dpp_row<0x128>(v), dpp_row_i<0x128>(idx));
  argmax_take(v, idx, dpp_row<0x124>(v), dpp_row_i<0x124>(idx));
  argmax_take(v, idx, dpp_row<0x122>(v), dpp_row_i<0x122>(idx));
  argmax_take(v, idx, dpp_row<0x121>(v), dpp_row_i<0x121>(idx));
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(idx, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16)
    argmax_take(bv, bi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), r)),
                __builtin_amdgcn_readlane(idx, r));
  v = bv;
  idx = bi;
}

// Top-k of NT tokens for the calling wave (their dependent cross-lane steps
// interleaved), from their logits v[n][q] = logit of expert lane + 64 q (-inf past E; a
// NaN logit never wins): the k selected experts (descending logit, ties to the lower
// index) and their softmax gates, valid in lanes [0, top_k) as (id, gate) of rank
// j = lane.
template <int NT>
__device__ __forceinline__ void topk_select(float (&v)[NT][4], int E, int top_k, int lane,
                                            int (&id_out)[NT], float (&gate_out)[NT]) {
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q) v[n][q] = v[n][q] == v[n][q] ? v[n][q] : -INFINITY;
  // k <= 8 rounds, fully unrolled so that every array stays in registers
  float sel_v[NT][8];
  int sel_i[NT][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      sel_v[n][j] = -INFINITY;
      sel_i[n][j] = 0;
    }
    if (j < top_k) {
      float bv[NT];
      int bi[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        bv[n] = v[n][0];
        bi[n] = lane;
#pragma unroll
        for (int q = 1; q < 4; ++q)
          if (v[n][q] > bv[n]) {  // strict: ties keep the lower expert index
            bv[n] = v[n][q];
            bi[n] = lane + 64 * q;
          }
        if (bi[n] >= E) bi[n] = 0x7FFFFFFF;
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) wave_argmax(bv[n], bi[n]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (bi[n] >= E) bi[n] = 0;     // unreachable for finite inputs; keeps ids in range
        sel_v[n][j] = bv[n];
        sel_i[n][j] = bi[n];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (bi[n] == lane + 64 * q) v[n][q] = -INFINITY;
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float z[8], sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z[j] = j < top_k ? expf(sel_v[n][j] - sel_v[n][0]) : 0.f;
      sum += z[j];
    }
    id_out[n] = 0;
    gate_out[n] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (lane == j) {
        id_out[n] = sel_i[n][j];
        gate_out[n] = z[j] / sum;
      }
  }
}

// Logit of token t, expert e: the router partial sums over the H slices plus the bias
// (four independent partial sums so that the slice loads are in flight together).
__device__ __forceinline__ float logit_of(const float* __restrict__ partial, int ksplit,
                                          const float* __restrict__ bias, size_t TE, size_t idx,
                                          int e) {
  const float* src = partial + idx;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
  int sp = 0;
  for (; sp + 4 <= ksplit; sp += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) s4[u] += src[(sp + u) * TE];
  }
  for (; sp < ksplit; ++sp) s4[0] += src[sp * TE];
  float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  return s + (bias ? bias[e] : 0.f);
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

// ------------------------------------------------------------------------------------
// scatter of one chunk of kChunk tokens.  The chunk's (token, j) entries are taken 256 at a
// time in token order; inside a wave, the lanes whose expert matches a lane's expert bit
// for bit (eight ballots) give its rank; waves before it in the same round and earlier
// rounds (a running per-expert count) give the rest of its slot.  run[e] holds the
// chunk's first slot of expert e on entry.  Every thread of the workgroup passes the
// barriers; threads [0, 256) do the work.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void scatter_chunk(const int32_t* __restrict__ ids, int chunk, int T,
                                              int E, int top_k, int32_t* __restrict__ perm,
                                              int32_t* __restrict__ inv, int* run, int (*wc)[256]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool act = tid < 256;
  const int t0 = chunk * kChunk;
  const int n = min(kChunk, T - t0) * top_k;
  const size_t flat0 = static_cast<size_t>(t0) * top_k;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < n; r += 256) {
    if (act) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) wc[ww][tid] = 0;
    }
    __syncthreads();
    const int i = r + tid;
    const int ex = (act && i < n) ? ids[flat0 + i] : -1;
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

// ------------------------------------------------------------------------------------
// scan: one workgroup of 1024 lanes; lane (q, e) owns expert e over the q-th quarter of
// the chunks.  counts -> offsets (LDS exclusive scan over experts) -> per-chunk bases,
// then the M-tile list (tiles of bm rows, expert-major) and each expert's first tile.
// With a single chunk (decode-sized T) the same workgroup then scatters it, which saves
// a launch on the latency-bound decode path.
// ------------------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Exclusive prefix sum over lanes [0, 256) of the workgroup (4 waves): an inclusive scan
// inside each wave on DPP (row shifts by 1, 2, 4, 8 within rows of 16, then the row
// broadcasts of lanes 15 and 31), the wave totals through LDS, one barrier each way.
// Every thread of the workgroup must call it; lanes >= 256 get 0.
__device__ int exclusive_scan256(int v, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = v;
  x += dpp_i<0x111, 0xF>(x);     // row_shr:1
  x += dpp_i<0x112, 0xF>(x);     // row_shr:2
  x += dpp_i<0x114, 0xF>(x);     // row_shr:4
  x += dpp_i<0x118, 0xF>(x);     // row_shr:8
  x += dpp_i<0x142, 0xA>(x);     // row_bcast:15 into rows 1 and 3
  x += dpp_i<0x143, 0xC>(x);     // row_bcast:31 into rows 2 and 3
  if (tid < 256 && lane == 63) tmp[w] = x;
  __syncthreads();
  int base = 0;
  if (tid < 256)
    for (int ww = 0; ww < w; ++ww) base += tmp[ww];
  __syncthreads();
  return tid < 256 ? base + x - v : 0;
}

// The scan's body for a workgroup of 1024 lanes; `hist` and `ids` may point to global
// memory or to this workgroup's LDS.
__device__ __forceinline__ void dispatch_scan_body(const int32_t* hist, int nchunks, int E, int bm,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ chunk_base,
                                                   MTile* __restrict__ tiles,
                                                   int32_t* __restrict__ num_tiles,
                                                   int32_t* __restrict__ expert_tile_off,
                                                   const int32_t* ids, int T, int top_k,
                                                   int32_t* __restrict__ perm,
                                                   int32_t* __restrict__ inv, int (*part)[256],
                                                   int* tmp) {
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
  if (tid >= 1 && tid <= 2 * kGemmQueues) num_tiles[tid] = 0;   // the GEMMs' work queues
  if (ids != nullptr) {   // a single chunk (T <= kChunk): its scatter follows in this workgroup
    __syncthreads();      // every thread is past the tile scan's use of tmp and part
    if (tid < E) tmp[tid] = off;   // the chunk's first slot of each expert = its offset
    scatter_chunk(ids, 0, T, E, top_k, perm, inv, tmp, part);
  }
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ hist,
                                                             int nchunks, int E, int bm,
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
  dispatch_scan_body(hist, nchunks, E, bm, counts, offsets, chunk_base, tiles, num_tiles,
                     expert_tile_off, ids, T, top_k, perm, inv, part, tmp);
}

// ------------------------------------------------------------------------------------
// The same logit with every slice load issued at once (MAXS >= ksplit registers; the
// indices past ksplit are clamped to the last slice, so every load stays inside the
// partials, and their values are dropped), summed pairwise: one memory round trip.
template <int MAXS>
__device__ __forceinline__ float logit_wide(const float* __restrict__ partial, int ksplit,
                                            const float* __restrict__ bias, size_t TE, size_t idx,
                                            int e) {
  float r[MAXS];
#pragma unroll
  for (int u = 0; u < MAXS; ++u) r[u] = partial[static_cast<size_t>(min(u, ksplit - 1)) * TE + idx];
#pragma unroll
  for (int u = 0; u < MAXS; ++u) r[u] = u < ksplit ? r[u] : 0.f;
#pragma unroll
  for (int w = MAXS / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int u = 0; u < w; ++u) r[u] += r[u + w];
  return r[0] + (bias ? bias[e] : 0.f);
}

// logits[t * SE + e] for every (t, e), a NaN logit stored as -inf (it never wins).
template <int MAXS>
__device__ __forceinline__ void tail_logits(const float* __restrict__ partial, int ksplit,
                                            const float* __restrict__ bias, int T, int E, int SE,
                                            float* logits) {
  const int TE = T * E;
  for (int i = threadIdx.x; i < TE; i += blockDim.x) {
    const float v = logit_wide<MAXS>(partial, ksplit, bias, TE, i, i % E);
    logits[(i / E) * SE + i % E] = v == v ? v : -INFINITY;
  }
}

// Inserts candidate (v, i) (v not NaN) into the list (lv, li) of K candidates kept in
// descending order of value; empty slots hold NaN, at the end, and take any candidate.
// Candidates must arrive in ascending expert order (of equal values the earlier stays
// ahead, so ties go to the lower index).  The K compares are independent of each other
// (the list is sorted, so they switch once from false to true at the insertion point)
// and each slot then takes the candidate, its predecessor or itself: no serial chain.
template <int K>
__device__ __forceinline__ void list_insert(float (&lv)[K], int (&li)[K], float v, int i) {
  bool tk[K];
#pragma unroll
  for (int s = 0; s < K; ++s) tk[s] = !(v <= lv[s]);
#pragma unroll
  for (int s = K - 1; s >= 1; --s) {
    lv[s] = tk[s] ? (tk[s - 1] ? lv[s - 1] : v) : lv[s];
    li[s] = tk[s] ? (tk[s - 1] ? li[s - 1] : i) : li[s];
  }
  lv[0] = tk[0] ? v : lv[0];
  li[0] = tk[0] ? i : li[0];
}

// Top-k + softmax of every token with a lane per token, from logits in LDS (no NaN):
// wave (g, p), p < P, keeps the best K of experts [p E / P, (p + 1) E / P) for tokens
// 64 g + lane in registers (P = min(4, E / K) parts, so with P > 1 every list is full);
// then wave g merges each token's P lists (parts in order, so the insertions stay in
// ascending expert order), takes the softmax over the first top_k and writes ids, gates,
// the LDS copy of the ids and the LDS histogram.  The partial lists are kept as
// cv/ci[(p K + s) kChunk + t].
template <int K>
__device__ __forceinline__ void tail_topk(const float* logits, int SE, int T, int E, int top_k,
                                          float* cv, int* ci, int32_t* __restrict__ ids,
                                          float* __restrict__ gates, int* sids, int* hist) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = (T + 63) / 64;
  const int P = max(1, min(4, E / K));
  float lv[K];
  int li[K];
  if (wave < 4 * G && (wave & 3) < P) {
    const int g = wave >> 2, p = wave & 3;
    const int t = 64 * g + lane;
#pragma unroll
    for (int s = 0; s < K; ++s) {
      lv[s] = __int_as_float(0x7FC00000);   // empty (NaN)
      li[s] = 0;
    }
    if (t < T) {
      const int e1 = (p + 1) * E / P;
#pragma unroll 4
      for (int e = p * E / P; e < e1; ++e) list_insert<K>(lv, li, logits[t * SE + e], e);
      if (P > 1) {
#pragma unroll
        for (int s = 0; s < K; ++s) {
          cv[(p * K + s) * kChunk + t] = lv[s];
          ci[(p * K + s) * kChunk + t] = li[s];
        }
      }
    }
  }
  if (P > 1) {
    __syncthreads();
    if (wave < G) {
      const int t = 64 * wave + lane;
#pragma unroll
      for (int s = 0; s < K; ++s) {
        lv[s] = __int_as_float(0x7FC00000);
        li[s] = 0;
      }
      if (t < T)
        for (int c = 0; c < P * K; ++c) list_insert<K>(lv, li, cv[c * kChunk + t], ci[c * kChunk + t]);
    }
  }
  // the finished list of token 64 g + lane is in wave 4 g (P == 1) or wave g (P > 1)
  const int g = P > 1 ? wave : wave >> 2;
  const bool owner = P > 1 ? wave < G : (wave < 4 * G && (wave & 3) == 0);
  const int t = 64 * g + lane;
  if (owner && t < T) {
    float z[K], sum = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      z[j] = j < top_k ? expf(lv[j] - lv[0]) : 0.f;
      sum += z[j];
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (j < top_k) {
        ids[static_cast<size_t>(t) * top_k + j] = li[j];
        gates[static_cast<size_t>(t) * top_k + j] = z[j] / sum;
        sids[t * top_k + j] = li[j];
        atomicAdd(&hist[li[j]], 1);
      }
  }
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
  const int tid = threadIdx.x;
  const int SE = E | 1;
  if (tid < 256) hist[tid] = 0;
  if (ksplit <= 8)
    tail_logits<8>(partial, ksplit, bias, T, E, SE, logits);
  else if (ksplit <= 16)
    tail_logits<16>(partial, ksplit, bias, T, E, SE, logits);
  else if (ksplit <= 32)
    tail_logits<32>(partial, ksplit, bias, T, E, SE, logits);
  else
    tail_logits<64>(partial, ksplit, bias, T, E, SE, logits);
  __syncthreads();
  if (top_k <= 2)
    tail_topk<2>(logits, SE, T, E, top_k, cv, ci, ids, gates, sids, hist);
  else if (top_k <= 4)
    tail_topk<4>(logits, SE, T, E, top_k, cv, ci, ids, gates, sids, hist);
  else
    tail_topk<8>(logits, SE, T, E, top_k, cv, ci, ids, gates, sids, hist);
  __syncthreads();
  dispatch_scan_body(hist, 1, E, bm, counts, offsets, chunk_base, tiles, num_tiles,
                     expert_tile_off, sids, T, top_k, perm, inv, part, tmp);
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
                          uint8_t* xq, float* sx, uint16_t* parts, uint8_t* sx_mx) {
  dim3 grid(ceil_div(T, kRouterTile), ceil_div(E, kRouterTile), ksplit);
  if (parts != nullptr) {
    const long n4 = static_cast<long>(E) * H / 4;   // H is a multiple of 64
    router_split_kernel<<<dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st>>>(
        W, n4, static_cast<long>(E) * H, parts);
    router_logits_kernel<true><<<grid, dim3(256), 0, st>>>(x, W, T, H, E, kslice, partial, hist,
                                                           hist_n, xq, sx, parts, sx_mx);
  } else {
    router_logits_kernel<false><<<grid, dim3(256), 0, st>>>(x, W, T, H, E, kslice, partial, hist,
                                                            hist_n, xq, sx, nullptr, sx_mx);
  }
}

void launch_topk(const float* partial, int ksplit, const float* bias, int T, int E, int top_k,
                 int32_t* ids, float* gates, int32_t* hist, hipStream_t st) {
  topk_kernel<<<dim3(ceil_div(T, 4)), dim3(256), 0, st>>>(partial, ksplit, bias, T, E, top_k, ids,
                                                        gates, hist);
}

void launch_dispatch_scan(const int32_t* hist, int nchunks, int E, int bm, int32_t* counts,
                          int32_t* offsets, int32_t* chunk_base, MTile* tiles, int32_t* num_tiles,
                          int32_t* expert_tile_off, hipStream_t st, const int32_t* ids, int T,
                          int top_k, int32_t* perm, int32_t* inv) {
  dispatch_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(hist, nchunks, E, bm, counts, offsets,
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
