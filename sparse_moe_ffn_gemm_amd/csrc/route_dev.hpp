// Device building blocks of the router and the dispatch (router.hip), shared with the
// fused decode kernel (fused.hip): the exact bf16x3 router tile, top-k + softmax, the
// deterministic counting-sort dispatch and the one-workgroup routing tail.
#pragma once

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

// LDS bytes of one router tile of TT tokens x TE experts: the x rows and the three W planes,
// rows of kRS bf16.
template <int TT, int TE>
constexpr int router_lds() { return (TT + 3 * TE) * kRS * 2; }
constexpr int kRouterLds = router_lds<kRouterTile, kRouterTile>();

// One router tile (token tile tx of TT tokens, expert tile ey of TE experts, H slice s of
// kslice columns) by a workgroup of NTHR threads: waves in a (TT / 32) x (NTHR / 64 / (TT /
// 32)) grid, each 32 tokens x (16 NJ) experts (64 x 64 by 256 threads: 2 x 2 waves of 32 x
// 32; by 512: 2 x 4 of 32 x 16; 128 x 128 by 512: 4 x 2 of 32 x 64).  Each 16 x 16 output
// sub-tile sees the same sequence of matrix-core steps in every geometry, so the partials
// do not depend on it.  xs / wp: router_lds<TT, TE>() bytes of LDS (wp: three planes of TE
// rows).  COH: the partials are stored device-coherently (store_c), and so are the x codes
// and scales with QCOH (for a launch whose later work items read them).
template <bool PRESPLIT, int NTHR, bool COH = false, int TT = kRouterTile, int TE = kRouterTile,
          bool QCOH = COH>
__device__ __forceinline__ void router_tile(const uint16_t* __restrict__ x,
                                            const float* __restrict__ W, int T, int H, int E,
                                            int kslice, int tx, int ey, int s,
                                            float* __restrict__ partial, uint8_t* __restrict__ xq,
                                            float* __restrict__ sx,
                                            const uint16_t* __restrict__ parts,
                                            uint8_t* __restrict__ sx_mx, uint16_t* xs,
                                            uint16_t* wp) {
  static_assert(NTHR == 256 || NTHR == 512, "router workgroup width");
  constexpr int WAVES = NTHR / 64;
  constexpr int WMW = TT / 32;                    // waves along tokens
  constexpr int WNW = WAVES / WMW;                // waves along experts
  static_assert(WMW * WNW == WAVES && TE % (16 * WNW) == 0, "router tile geometry");
  constexpr int NJ = TE / WNW / 16;               // 16-expert sub-tiles per wave
  constexpr int XL = TT * 16 / NTHR;              // x loads per thread (TT rows x 16 chunks)
  constexpr int WL = TE * 32 / NTHR;              // W float4 loads per thread (TE rows x 32)
  constexpr int PX = TE * 16 / NTHR;              // pre-split part loads per thread and plane
  constexpr int PL = 3 * PX;
  constexpr int PLANE = TE * kRS;                 // LDS plane stride of wp
  const int t0 = tx * TT, e0 = ey * TE;
  const int h_begin = s * kslice;
  const int h_end = min(H, h_begin + kslice);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WMW, wn = wave / WMW;
  const bool quant = xq != nullptr && ey == 0;
  const int KBH = ceil_div(H, kBlock);
  v4f acc[2][NJ], tot[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) tot[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // one step's global loads: x TT rows x 16 chunks of 8 bf16; W TE rows x 32 float4, or
  // (pre-split) three planes of TE rows x 16 chunks of 8 bf16
  uint4 xr[XL];
  float4 wr[PRESPLIT ? 1 : WL];
  uint4 pr[PRESPLIT ? PL : 1];
  const long plane = static_cast<long>(E) * H;
  auto load = [&](int h0) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int q = tid + NTHR * i;
      const int t = t0 + (q >> 4), h = h0 + (q & 15) * 8;
      xr[i] = make_uint4(0u, 0u, 0u, 0u);
      if (t < T && h < h_end) xr[i] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + h);
    }
    if constexpr (PRESPLIT) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int q = tid + NTHR * (i % PX), pl = i / PX;
        const int e = e0 + (q >> 4), h = h0 + (q & 15) * 8;
        pr[i] = make_uint4(0u, 0u, 0u, 0u);
        if (e < E && h < h_end)
          pr[i] = *reinterpret_cast<const uint4*>(parts + pl * plane + static_cast<size_t>(e) * H + h);
      }
    } else {
#pragma unroll
      for (int i = 0; i < WL; ++i) {
        const int q = tid + NTHR * i;
        const int e = e0 + (q >> 5), h = h0 + (q & 31) * 4;
        wr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < E && h < h_end) wr[i] = *reinterpret_cast<const float4*>(W + static_cast<size_t>(e) * H + h);
      }
    }
  };
  if (h_begin < h_end) load(h_begin);
  for (int h0 = h_begin; h0 < h_end; h0 += kRC) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int q = tid + NTHR * i;
      *reinterpret_cast<uint4*>(xs + (q >> 4) * kRS + (q & 15) * 8) = xr[i];
    }
    if constexpr (PRESPLIT) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int q = tid + NTHR * (i % PX);
        *reinterpret_cast<uint4*>(wp + (i / PX) * PLANE + (q >> 4) * kRS + (q & 15) * 8) = pr[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < WL; ++i) {   // split in 3 exact bf16 parts
        const int q = tid + NTHR * i;
        const int row = q >> 5, c = q & 31;
        uint2 ph, pm, pl;
        split3(wr[i], ph, pm, pl);
        *reinterpret_cast<uint2*>(wp + row * kRS + c * 4) = ph;
        *reinterpret_cast<uint2*>(wp + PLANE + row * kRS + c * 4) = pm;
        *reinterpret_cast<uint2*>(wp + 2 * PLANE + row * kRS + c * 4) = pl;
      }
    }
    __syncthreads();
    if (h0 + kRC < h_end) load(h0 + kRC);   // next step's loads fly during this step
    if (quant) {   // 16 lanes per token group, NTHR / 16 tokens per pass
      const int g = h0 / kBlock;
#pragma unroll
      for (int pass = 0; pass < TT / (NTHR / 16); ++pass) {
        const int row = pass * (NTHR / 16) + (tid >> 4), col = 8 * (tid & 15);
        const int t = t0 + row;
        const bool in = t < T && h0 + col < h_end;
        uint8_t* codes_row = xq + static_cast<size_t>(t < T ? t : 0) * H + h0;
        if (sx_mx != nullptr) {   // MXFP8: four lanes per 32-block, pads past H get 127
          const int code = quantize_mx8<QCOH>(xs + row * kRS, col, in, codes_row);
          if ((tid & 3) == 0 && t < T)
            store_c<QCOH>(sx_mx + static_cast<size_t>(t) * 4 * KBH + (h0 + col) / kMxBlock,
                          static_cast<uint8_t>(code));
        } else {
          const float sc = quantize_group16<QCOH>(xs + row * kRS, col, in, codes_row);
          if ((tid & 15) == 0 && t < T) store_c<QCOH>(sx + static_cast<size_t>(t) * KBH + g, sc);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kRC; kk += 32) {
      const int kofs = kk + 8 * (lane >> 4);
      v8bf a[2], b[3][NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = lds_bf8(xs + (wm * 32 + 16 * i + (lane & 15)) * kRS + kofs);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          b[p][j] = lds_bf8(wp + p * PLANE + (wn * 16 * NJ + 16 * j + (lane & 15)) * kRS + kofs);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int p = 0; p < 3; ++p)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[p][j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) tot[i][j] += acc[i][j];
    __syncthreads();
  }
  float* out = partial + static_cast<size_t>(s) * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wm * 32 + 16 * i + 4 * (lane >> 4) + r;
        const int e = e0 + wn * 16 * NJ + 16 * j + (lane & 15);
        if (t < T && e < E) store_c<COH>(out + static_cast<size_t>(t) * E + e, tot[i][j][r]);
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

// ------------------------------------------------------------------------------------
// scatter of one chunk of kChunk tokens.  The chunk's (token, j) entries are taken 256 at a
// time in token order; inside a wave, the lanes whose expert matches a lane's expert bit
// for bit (eight ballots) give its rank; waves before it in the same round and earlier
// rounds (a running per-expert count) give the rest of its slot.  run[e] holds the
// chunk's first slot of expert e on entry.  Every thread of the workgroup passes the
// barriers; threads [0, 256) do the work.  COH: perm and inv are stored device-coherently.
// ------------------------------------------------------------------------------------
template <bool COH = false>
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
      store_c<COH>(perm + pos, flat);
      store_c<COH>(inv + flat, pos);
    }
    __syncthreads();
    if (tid < E) run[tid] += wc[0][tid] + wc[1][tid] + wc[2][tid] + wc[3][tid];
  }
}

// ------------------------------------------------------------------------------------
// scan: one workgroup of 256 nq lanes (nq = 2 or 4); lane (q, e) owns expert e over the
// q-th of nq parts of the chunks.  counts -> offsets (LDS exclusive scan over experts) -> per-chunk bases,
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

// The scan's body for a workgroup of 512 or 1024 lanes; `hist` and `ids` may point to global
// memory or to this workgroup's LDS.  COH: the tables are stored device-coherently.
template <bool COH = false>
__device__ __forceinline__ void dispatch_scan_body(const int32_t* hist, int nchunks, int E, int bm,
                                                   int xr,
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
  const int nq = blockDim.x >> 8;
  const int per = (nchunks + nq - 1) / nq;
  const int c0 = min(nchunks, q * per), c1 = min(nchunks, c0 + per);
  int s = 0;
  if (e < E)
    for (int c = c0; c < c1; ++c) s += hist[static_cast<size_t>(c) * E + e];
  part[q][e] = s;
  __syncthreads();
  int cnt = 0;   // zero for e >= E
  for (int qq = 0; qq < nq; ++qq) cnt += part[qq][e];
  const int off = exclusive_scan256(cnt, tmp);                          // valid in lanes < 256
  if (tid < 256) tmp[e] = off;
  __syncthreads();
  if (e < E) {
    int run = tmp[e];
    for (int qq = 0; qq < q; ++qq) run += part[qq][e];
    for (int c = c0; c < c1; ++c) {
      store_c<COH>(chunk_base + static_cast<size_t>(c) * E + e, run);
      run += hist[static_cast<size_t>(c) * E + e];
    }
    if (q == 0) {
      store_c<COH>(counts + e, cnt);
      store_c<COH>(offsets + e, tmp[e]);
      if (e == E - 1) store_c<COH>(offsets + E, tmp[e] + cnt);
    }
  }
  __syncthreads();
  const int ntl = (q == 0 && e < E) ? expert_tiles(cnt, bm, xr) : 0;
  const int toff = exclusive_scan256(ntl, tmp);
  if (q == 0) {
    const int base = off;
    for (int i = 0; i < ntl; ++i) {
      // (expert, row_begin) and (row_end, pad) as two 8-byte words
      const uint32_t rb = static_cast<uint32_t>(base + i * bm);
      const uint32_t re = static_cast<uint32_t>(i + 1 < ntl ? base + (i + 1) * bm : base + cnt);
      uint64_t* w = reinterpret_cast<uint64_t*>(tiles + toff + i);
      store_c<COH>(w, static_cast<uint64_t>(static_cast<uint32_t>(e)) | (static_cast<uint64_t>(rb) << 32));
      store_c<COH>(w + 1, static_cast<uint64_t>(re));
    }
    if (e < E) store_c<COH>(expert_tile_off + e, toff);
    if (e == 255) {
      store_c<COH>(num_tiles, toff + ntl);
      store_c<COH>(expert_tile_off + E, toff + ntl);
    }
  }
  if (tid >= 1 && tid <= 2 * kGemmQueues)   // the GEMMs' work-queue heads
    store_c<COH>(num_tiles + kQueueStride * tid, 0);
  if (ids != nullptr) {   // a single chunk (T <= kChunk): its scatter follows in this workgroup
    __syncthreads();      // every thread is past the tile scan's use of tmp and part
    if (tid < E) tmp[tid] = off;   // the chunk's first slot of each expert = its offset
    scatter_chunk<COH>(ids, 0, T, E, top_k, perm, inv, tmp, part);
  }
}

// ------------------------------------------------------------------------------------
// The same logit with every slice load issued at once (MAXS >= ksplit registers; the
// indices past ksplit are clamped to the last slice, so every load stays inside the
// partials, and their values are dropped), summed pairwise: one memory round trip.
template <int MAXS, bool COH = false>
__device__ __forceinline__ float logit_wide(const float* __restrict__ partial, int ksplit,
                                            const float* __restrict__ bias, size_t TE, size_t idx,
                                            int e) {
  float r[MAXS];
#pragma unroll
  for (int u = 0; u < MAXS; ++u)
    r[u] = load_c<COH>(partial + static_cast<size_t>(min(u, ksplit - 1)) * TE + idx);
#pragma unroll
  for (int u = 0; u < MAXS; ++u) r[u] = u < ksplit ? r[u] : 0.f;
#pragma unroll
  for (int w = MAXS / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int u = 0; u < w; ++u) r[u] += r[u + w];
  return r[0] + (bias ? bias[e] : 0.f);
}

// logits[t * SE + e] for every (t, e), a NaN logit stored as -inf (it never wins).
// Tokens [t0, t0 + nt) of T: logits[(t - t0) * SE + e].  G logits per thread and pass, so
// that G x MAXS loads are in flight together; GMAX caps G (this code runs once per
// workgroup, from a cold instruction cache: for the prefill routing kernel's few-slice sums a
// shorter unrolled body saved more instruction fetches than it cost in memory round trips).
template <int MAXS, bool COH = false, int GMAX = 64>
__device__ __forceinline__ void tail_logits(const float* __restrict__ partial, int ksplit,
                                            const float* __restrict__ bias, int T, int E, int SE,
                                            float* logits, int t0 = 0, int nt = -1) {
  constexpr int G = MAXS >= 64 ? 1 : (64 / MAXS < GMAX ? 64 / MAXS : GMAX);
  const size_t TE = static_cast<size_t>(T) * E;
  const int n = (nt < 0 ? T : nt) * E;
  const size_t base = static_cast<size_t>(t0) * E;
  const int step = static_cast<int>(blockDim.x);
  for (int i0 = threadIdx.x; i0 < n; i0 += G * step) {
    float v[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = i0 + g * step;
      v[g] = i < n ? logit_wide<MAXS, COH>(partial, ksplit, bias, TE, base + i, i % E) : 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = i0 + g * step;
      if (i < n) logits[(i / E) * SE + i % E] = v[g] == v[g] ? v[g] : -INFINITY;
    }
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
// cv/ci[(p K + s) cs + t] (cs >= T).  Needs 4 ceil(T / 64) waves.
template <int K, bool COH = false>
__device__ __forceinline__ void tail_topk(const float* logits, int SE, int T, int E, int top_k,
                                          float* cv, int* ci, int cs, int32_t* __restrict__ ids,
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
          cv[(p * K + s) * cs + t] = lv[s];
          ci[(p * K + s) * cs + t] = li[s];
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
        for (int c = 0; c < P * K; ++c) list_insert<K>(lv, li, cv[c * cs + t], ci[c * cs + t]);
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
        store_c<COH>(ids + static_cast<size_t>(t) * top_k + j, li[j]);
        store_c<COH>(gates + static_cast<size_t>(t) * top_k + j, z[j] / sum);
        sids[t * top_k + j] = li[j];
        atomicAdd(&hist[li[j]], 1);
      }
  }
}


// LDS of the routing tail: the scan's parts and scratch, the histogram, the ids of the
// chunk, the logits (rows of E | 1) and the top-k candidate lists (stride cs >= T).
struct TailLds {
  int (*part)[256];
  int* tmp;
  int* hist;
  int* sids;
  float* logits;
  float* cv;
  int* ci;
  int cs;
};

// Routing tail of a decode-sized layer (T <= kChunk, one dispatch chunk, T E <=
// kTailLogits, at most kTailSplit H slices, 4 ceil(T / 64) <= waves of the workgroup) in
// one workgroup of 512 or 1024 lanes: the router partials summed into LDS logits (all
// slice loads of a logit in flight together), top-k + softmax with a lane per token
// (tail_topk), then the scan, the M-tile list of bm-row tiles and the scatter.  COH: the
// partials are read and every table is written device-coherently.
template <bool COH = false>
__device__ __forceinline__ void route_tail_body(const float* __restrict__ partial, int ksplit,
                                                const float* __restrict__ bias, int T, int E,
                                                int top_k, int bm, int32_t* __restrict__ ids,
                                                float* __restrict__ gates,
                                                int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ chunk_base,
                                                MTile* __restrict__ tiles,
                                                int32_t* __restrict__ num_tiles,
                                                int32_t* __restrict__ expert_tile_off,
                                                int32_t* __restrict__ perm,
                                                int32_t* __restrict__ inv, const TailLds& L) {
  const int tid = threadIdx.x;
  const int SE = E | 1;
  if (tid < 256) L.hist[tid] = 0;
  if (ksplit <= 8)
    tail_logits<8, COH>(partial, ksplit, bias, T, E, SE, L.logits);
  else if (ksplit <= 16)
    tail_logits<16, COH>(partial, ksplit, bias, T, E, SE, L.logits);
  else if (ksplit <= 32)
    tail_logits<32, COH>(partial, ksplit, bias, T, E, SE, L.logits);
  else
    tail_logits<64, COH>(partial, ksplit, bias, T, E, SE, L.logits);
  __syncthreads();
  if (top_k <= 2)
    tail_topk<2, COH>(L.logits, SE, T, E, top_k, L.cv, L.ci, L.cs, ids, gates, L.sids, L.hist);
  else if (top_k <= 4)
    tail_topk<4, COH>(L.logits, SE, T, E, top_k, L.cv, L.ci, L.cs, ids, gates, L.sids, L.hist);
  else
    tail_topk<8, COH>(L.logits, SE, T, E, top_k, L.cv, L.ci, L.cs, ids, gates, L.sids, L.hist);
  __syncthreads();
  dispatch_scan_body<COH>(L.hist, 1, E, bm, 0, counts, offsets, chunk_base, tiles, num_tiles,
                          expert_tile_off, L.sids, T, top_k, perm, inv, L.part, L.tmp);
}

}  // namespace moe
