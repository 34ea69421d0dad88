// Grouped FP8 GEMMs of the experts on the gfx950 matrix cores.
//
// "GPT-OSS on day 0", section "On Hopper": FP8 with 128x128 block scaling and
// experts with biases; section "Kernels -> MoE": the bias enters the GEMM as the
// accumulator's starting value once per output tile (here it is added in the
// epilogue, which gives the same sum); section "Performance Tweaks": launch shapes
// are specialised for the hidden size 2880 rather than reused from 7168.
//
// Both GEMMs are "NT": A [rows, K] and B [N, K] are K-contiguous, the natural
// operand order of v_mfma_f32_16x16x128_f8f6f4 (lane l supplies 32 K bytes of row
// l%16, for A and B alike).  One K-step is one
// 128-wide scale block: each 16x16 sub-tile's MFMA result of that step is folded
// into the fp32 accumulator with the product of the row's activation scale and the
// sub-tile's weight block scale (block-scale promotion; the weight scale is uniform
// over every wave's column range by construction of the tiling).  Promoting every
// 128 products also bounds the error of the matrix cores' own fp8 accumulation.
//
// Memory pipeline: tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging) through a ring of STAGES K-steps,
// so STAGES-1 K-steps of loads are in flight while one is multiplied.  LDS rows are
// 128 bytes; the 16-byte chunk c of row r is stored in slot c ^ (r & 7), which each lane
// realises by choosing the global chunk it fetches.  A fragment lane (row r, K-quarter g)
// takes chunks g and g + 4 of its row rather than 2g and 2g + 1: the MFMA only needs the
// A and B lanes to agree on which K values they hold, and with this pairing the 128-bit
// fragment reads spread over all LDS banks (measured: about 1.4x the read bandwidth of
// the adjacent-chunk pairing).  Out-of-range chunks (K tail, N tail, rows past the
// expert's segment) are fetched from a zero block.
//
// Work order: blocks are numbered so that each XCD (blocks are dealt round-robin to
// the 8 XCDs) receives a contiguous range of (n-tile, m-tile) pairs with m-tiles
// fastest, so the M-tiles that share an expert's weight tile run together on one XCD
// and its L2 serves the repeated weight reads.
//
// gemm1: rows of expert e gathered from xq through perm; the 256-wide B tile holds
//   128 gate rows and the matching 128 up rows of w13, so SwiGLU pairs (j, I+j) sit
//   in the same lane; the epilogue adds b13, applies silu(gate)*up and requantises
//   each 1x128 group of h (row amax across lanes and waves) to e4m3.
// gemm2: rows of h in dispatch order, B = w2 [H, I]; the epilogue adds b2 and stores
//   y in fp16 (saturated).
//
// Kernels by group size (rows per expert): 256-row tiles over eight waves for prefill
// (grouped_gemm_big_kernel), 16/64/128-row tiles over four waves through one LDS ring
// (grouped_gemm_kernel), and for decode-sized groups whose weight rows are not whole
// cache lines, a barrier-free register stream in long per-row runs
// (grouped_gemm_rowrun_kernel).
#include <algorithm>

#include "gemm_dev.hpp"

namespace moe {


template <int BM, int BN, int WM, int WN, bool SWIGLU, int STAGES, bool RAW = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(const GemmArgs a, int max_tiles,
                                                           int ntiles, int grid) {
  constexpr int WTM = BM / WM, SM = WTM / 16;
  constexpr int WTN = BN / WN, SN = WTN / 16;
  constexpr int NG = SN / 2;                  // gemm1: gate (= up) sub-tiles per wave
  constexpr int GW = WTN / 2;                 // gemm1: gate columns per wave
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  constexpr int AROWS = BM / 4;               // A rows each wave fetches per stage
  constexpr int A_INSTR = AROWS >= 8 ? AROWS / 8 : 1;
  constexpr int BROWS = BN / 4;
  constexpr int B_INSTR = BROWS / 8;
  constexpr int LOADS = A_INSTR + B_INSTR + 1;   // vmem instructions per wave and stage
  static_assert(WM * WN == 4, "four waves");
  static_assert(SM >= 1 && SN >= 1, "sub-tiles");
  static_assert(AROWS % 8 == 0 || AROWS == 4, "A rows per wave");
  static_assert(AROWS + 2 <= 64, "one scale load per wave");
  static_assert(!SWIGLU || (BN == 256 && SN % 2 == 0 && GW <= 64), "gemm1 tile");
  static_assert(SWIGLU || WTN <= 128, "gemm2 wave columns inside one scale block");
  static_assert(STAGES >= 2 && LOADS * (STAGES - 2) < 64, "pipeline depth");

  __shared__ __align__(16) uint8_t smem[STAGES * STAGE];
  __shared__ __align__(16) float sA[STAGES][4][64];
  __shared__ int rowsrc[BM];
  __shared__ float red[SWIGLU ? WN : 1][BM];

  // ---- which tile: XCD-contiguous logical order, m-tiles fastest ----
  const int b = blockIdx.x;
  const int per_xcd = grid / 8;
  const int L = (b % 8) * per_xcd + b / 8;
  const int mti = L % max_tiles, nt = L / max_tiles;
  if (nt >= ntiles || mti >= *a.num_tiles) return;
  MTile mt = a.tiles[mti];
  mt.expert = __builtin_amdgcn_readfirstlane(mt.expert);
  mt.row_begin = __builtin_amdgcn_readfirstlane(mt.row_begin);
  mt.row_end = __builtin_amdgcn_readfirstlane(mt.row_end);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.K, N = a.N, I = a.I;
  const int KB = ceil_div(K, kBlock), NBs = ceil_div(N, kBlock);
  const int e = mt.expert;
  const uint8_t* Bexp = a.B + static_cast<size_t>(e) * N * K;
  const float* Bsc = a.B_scale + static_cast<size_t>(e) * NBs * KB;

  for (int r = tid; r < BM; r += 256) {
    const int p = mt.row_begin + r;
    int src = -1;
    if (p < mt.row_end) src = SWIGLU ? a.perm[p] / a.top_k : p;
    if (static_cast<unsigned>(src) >= static_cast<unsigned>(a.A_rows)) src = -1;   // never read past A
    rowsrc[r] = src;
  }
  __syncthreads();

  // ---- per-lane fetch descriptors (constant over K) ----
  // A: wave w fetches rows [w*AROWS, (w+1)*AROWS); lane -> (row, slot) of an 8-row group
  const int a_slot = lane & 7, a_r8 = lane >> 3;
  // Rows outside the tile are redirected to row 0 (finite codes that only feed output
  // rows/columns that are never stored); only the ragged K tail needs real zeros.
  const uint8_t* a_src[A_INSTR];
  bool a_ok[A_INSTR];
  unsigned a_off[A_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int row = wave * AROWS + i * 8 + a_r8;
    const bool live = AROWS >= 8 || lane < 32;
    const int src = live ? rowsrc[row] : -1;
    a_ok[i] = src >= 0;
    a_off[i] = static_cast<unsigned>(src < 0 ? 0 : src) * K + ((a_slot ^ swz_key(row)) << 4);
    a_src[i] = a.A + a_off[i];
  }
  const uint8_t* b_src[B_INSTR];
  bool b_ok[B_INSTR];
  unsigned b_off[B_INSTR];
#pragma unroll
  for (int i = 0; i < B_INSTR; ++i) {
    const int br = wave * BROWS + i * 8 + a_r8;
    int g = -1;
    if (SWIGLU) {
      const int j = nt * 128 + (br & 127);
      if (j < I) g = (br >> 7) * I + j;
    } else {
      const int col = nt * BN + br;
      if (col < N) g = col;
    }
    b_ok[i] = g >= 0;
    // a row past the matrix re-reads the tile's first row (already in flight, so it costs no
    // HBM traffic); it only feeds output columns that are never stored
    const int g_first = SWIGLU ? nt * 128 : nt * BN;
    b_off[i] = static_cast<unsigned>(g < 0 ? g_first : g) * K + ((a_slot ^ swz_key(br)) << 4);
    b_src[i] = Bexp + b_off[i];
  }
  // weight block-scale rows of this wave's column groups (-1: the group is empty)
  int sb_row0, sb_row1;
  if (SWIGLU) {
    const int j0 = nt * 128 + wn * GW;
    sb_row0 = j0 < I ? j0 / kBlock : -1;
    sb_row1 = j0 < I ? (I + j0) / kBlock : -1;
  } else {
    const int c0 = nt * BN + wn * WTN;
    sb_row0 = c0 < N ? c0 / kBlock : -1;
    sb_row1 = sb_row0;
  }
  // scale fetch of one K-step, one instruction per wave: lanes [0, AROWS) take the
  // activation scales of the wave's A rows, lanes AROWS and AROWS+1 the two weight block
  // scales of the wave's column groups
  const float* s_ptr = kZeroScale;
  bool s_live = false;
  if (lane < AROWS) {
    const int src = rowsrc[wave * AROWS + lane];
    s_live = src >= 0;
    s_ptr = a.A_scale + static_cast<size_t>(src < 0 ? 0 : src) * KB;
  } else if (lane < AROWS + 2) {
    const int row = lane == AROWS ? sb_row0 : sb_row1;
    s_live = row >= 0;
    s_ptr = Bsc + static_cast<size_t>(row < 0 ? 0 : row) * KB;
  }

  auto issue = [&](int kt) {   // all loads of K-step kt into ring slot kt % STAGES
    uint8_t* As = smem + (kt % STAGES) * STAGE;
    uint8_t* Bs = As + A_BYTES;
    const int k0 = kt * kBlock;
    if (k0 + kBlock <= K) {      // full K-step: scalar base + constant lane offsets
      const uint8_t* abase = a.A + k0;
      const uint8_t* bbase = Bexp + k0;
#pragma unroll
      for (int i = 0; i < A_INSTR; ++i)
        if (AROWS >= 8 || lane < 32) load_lds16_s(a_off[i], abase, As + (wave * AROWS + i * 8) * 128);
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i) load_lds16_s(b_off[i], bbase, Bs + (wave * BROWS + i * 8) * 128);
      if (lane < AROWS + 2) {
        const void* src = s_live ? static_cast<const void*>(s_ptr + kt) : kZeroScale;
        load_lds4(src, &sA[kt % STAGES][wave][0]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      const int row0 = wave * AROWS + i * 8;
      const int kk = k0 + ((a_slot ^ swz_key(row0 + a_r8)) << 4);
      const void* src = (a_ok[i] && kk < K) ? static_cast<const void*>(a_src[i] + k0) : kZeroChunk;
      if (AROWS >= 8 || lane < 32) load_lds16(src, As + row0 * 128);
    }
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
      const int row0 = wave * BROWS + i * 8;
      const int kk = k0 + ((a_slot ^ swz_key(row0 + a_r8)) << 4);
      const void* src = (b_ok[i] && kk < K) ? static_cast<const void*>(b_src[i] + k0) : kZeroChunk;
      load_lds16(src, Bs + row0 * 128);
    }
    if (lane < AROWS + 2) {
      const void* src = s_live ? static_cast<const void*>(s_ptr + kt) : kZeroScale;
      load_lds4(src, &sA[kt % STAGES][wave][0]);
    }
  };

  v4f acc[SM][SN];
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int n = 0; n < SN; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};

  auto sub_brow = [&](int n) {
    if (SWIGLU) return n < NG ? wn * GW + 16 * n : 128 + wn * GW + 16 * (n - NG);
    return wn * WTN + 16 * n;
  };

  // prologue: STAGES-1 K-steps in flight
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KB) issue(s);

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f pcar[SM];                     // last column's partial, promoted in the next step
  float scar[SM][4];
#pragma unroll
  for (int m = 0; m < SM; ++m) {
    pcar[m] = zero;
#pragma unroll
    for (int i = 0; i < 4; ++i) scar[m][i] = 0.f;
  }
  for (int kt = 0; kt < KB; ++kt) {
    // wait until this wave's loads of step kt have landed, then for every wave's
    if (kt + STAGES - 2 < KB) {
      wait_vmcnt<LOADS * (STAGES - 2)>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_only();
    // the slot consumed in step kt-1 is free: refill it with step kt+STAGES-1
    if (kt + STAGES - 1 < KB) issue(kt + STAGES - 1);

    const int slot = kt % STAGES;
    const uint8_t* As = smem + slot * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    // fragment and scale reads of this step, issued together
    const float sb0 = sA[slot][wave][AROWS];
    const float sb1 = sA[slot][wave][AROWS + 1];
    v8i af[SM];
    float4 sa4[SM];
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const int rw0 = wm * WTM + 16 * m;
      af[m] = lds_frag(As, rw0 + (lane & 15), lane >> 4);
      const int r = rw0 + 4 * (lane >> 4);          // 4 consecutive rows, one wave segment
      sa4[m] = *reinterpret_cast<const float4*>(&sA[slot][r / AROWS][r % AROWS]);
    }
    v8i bq0 = lds_frag(Bs, sub_brow(0) + (lane & 15), lane >> 4);
    v8i bq1 = lds_frag(Bs, sub_brow(SN > 1 ? 1 : 0) + (lane & 15), lane >> 4);
    // the previous step's last column, deferred to overlap the reads above
    if (kt > 0) {
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][SN - 1][i] = fmaf(pcar[m][i], scar[m][i], acc[m][SN - 1][i]);
    }
    float s0[SM][4], s1[SM][4];
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const float sa[4] = {sa4[m].x, sa4[m].y, sa4[m].z, sa4[m].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s0[m][i] = sa[i] * sb0;
        s1[m][i] = sa[i] * sb1;
      }
    }
    // Software pipeline over the n sub-tiles, pinned with scheduling fences: each MFMA
    // of column n+1 is followed by the four FMAs that fold the (finished) partial of
    // column n; B fragments are read two columns ahead.
    v4f pc[SM], pn[SM];
#pragma unroll
    for (int m = 0; m < SM; ++m)
      pc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m], bq0, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const bool second = SWIGLU && n >= NG;
      const v8i bn = bq1;
      if (n + 2 < SN) bq1 = lds_frag(Bs, sub_brow(n + 2) + (lane & 15), lane >> 4);
      if (n + 1 < SN) {
#pragma unroll
        for (int m = 0; m < SM; ++m) {
          __builtin_amdgcn_sched_barrier(0);
          pn[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m], bn, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[m][n][i] = fmaf(pc[m][i], second ? s1[m][i] : s0[m][i], acc[m][n][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < SM; ++m) pc[m] = pn[m];
      } else {
#pragma unroll
        for (int m = 0; m < SM; ++m) {
          pcar[m] = pc[m];
#pragma unroll
          for (int i = 0; i < 4; ++i) scar[m][i] = second ? s1[m][i] : s0[m][i];
        }
      }
    }
  }
  // the last step's last column
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[m][SN - 1][i] = fmaf(pcar[m][i], scar[m][i], acc[m][SN - 1][i]);
  __syncthreads();   // every wave is done with the ring before its LDS is reused

  const int rbase = wm * WTM + 4 * (lane >> 4);   // + 16 m + i
  if constexpr (RAW) {   // the fp32 accumulators, at the B row's global column of C [rows, N]
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const int br = sub_brow(n) + (lane & 15);
      int g = -1;
      if (SWIGLU) {
        const int j = nt * 128 + (br & 127);
        if (j < I) g = (br >> 7) * I + j;
      } else if (nt * BN + br < N) {
        g = nt * BN + br;
      }
      if (g < 0) continue;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = mt.row_begin + rbase + 16 * m + i;
          if (p < mt.row_end) a.c_raw[static_cast<size_t>(p) * N + g] = acc[m][n][i];
        }
    }
    return;
  }
  if constexpr (SWIGLU) {
    const uint16_t* bias = a.bias ? a.bias + static_cast<size_t>(e) * N : nullptr;
    float hv[SM][NG][4];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int j = nt * 128 + wn * GW + 16 * n + (lane & 15);
      const bool ok = j < I;
      const float bg = (ok && bias) ? bf16_to_f32(bias[j]) : 0.f;
      const float bu = (ok && bias) ? bf16_to_f32(bias[I + j]) : 0.f;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[m][n][i] + bg;
          const float u = acc[m][n + NG][i] + bu;
          hv[m][n][i] = ok ? g / (1.0f + expf(-g)) * u : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < SM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.f;
#pragma unroll
        for (int n = 0; n < NG; ++n) mx = fmaxf(mx, fabsf(hv[m][n][i]));
        mx = group_max<16>(mx);
        if ((lane & 15) == 0) red[wn][rbase + 16 * m + i] = mx;
      }
    __syncthreads();
    uint8_t* hs = smem;   // [BM][128] staging of the codes
    const int KBI = ceil_div(I, kBlock);
#pragma unroll
    for (int m = 0; m < SM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rbase + 16 * m + i;
        float amax = red[0][r];
#pragma unroll
        for (int w = 1; w < WN; ++w) amax = fmaxf(amax, red[w][r]);
        const float s = group_scale(amax);
#pragma unroll
        for (int n = 0; n < NG; ++n)
          hs[r * 128 + wn * GW + 16 * n + (lane & 15)] =
              static_cast<uint8_t>(encode2(hv[m][n][i], 0.f, s) & 0xFFu);
        const int p = mt.row_begin + r;
        if (wn == 0 && (lane & 15) == 0 && p < mt.row_end)
          a.h_scale[static_cast<size_t>(p) * KBI + nt] = s;
      }
    __syncthreads();
    for (int q = tid; q < BM * 8; q += 256) {
      const int r = q >> 3, c = q & 7;
      const int p = mt.row_begin + r, col = nt * 128 + c * 16;
      if (p < mt.row_end && col < I)
        *reinterpret_cast<uint4*>(a.h_out + static_cast<size_t>(p) * I + col) =
            *reinterpret_cast<const uint4*>(hs + r * 128 + c * 16);
    }
  } else {
    const uint16_t* bias = a.bias ? a.bias + static_cast<size_t>(e) * N : nullptr;
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const int col = nt * BN + wn * WTN + 16 * n + (lane & 15);
      if (col >= N) continue;
      const float bv = bias ? bf16_to_f32(bias[col]) : 0.f;
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = mt.row_begin + rbase + 16 * m + i;
          if (p < mt.row_end) a.y_out[static_cast<size_t>(p) * N + col] = f32_to_f16_sat(acc[m][n][i] + bv);
        }
    }
  }
}

// ------------------------------------------------------------------------------------
// Large-group variant: eight waves, two per SIMD so that one wave's promotion FMAs and
// LDS reads overlap the other's MFMAs.  A full M-tile is 256 x BN, the waves in a
// 4 (M) x 2 (N) grid, each 64 x BN/2 (4 x BN/32 sub-tiles of 16 x 16).  A (activation)
// and B (weight) tiles have rings of their own: A slots are filled SA-1 K-steps ahead, B
// slots SB-1 K-steps ahead, so the weights, which mostly come from HBM, get the longer
// lead.  Wave rows that lie entirely past the M-tile's rows skip their MFMAs.
//
// An expert's last M-tile often holds only a few rows (groups are about 256 +- 16 rows
// long).  Such a tile does a quarter of the work but, with one K-step of prefetch, waits
// a full load latency per K-step.  Tiles of at most 64 rows therefore take a narrow body
// in the same launch: 64 x BN, waves in a 2 x 4 grid of 32 x BN/4, and rings one step
// deeper (an A slot is a quarter the size), so they still run beside the expert's full
// tile on the same XCD and share its weight tile through L2.
//
// gemm1 (SWIGLU): the B tile holds BN/2 gate rows of w13 and the matching BN/2 up rows;
// wave wn takes gate and up columns [wn BN/4, (wn+1) BN/4) of them, so SwiGLU pairs sit
// in the same lane.  The weight scale is taken per 16-column sub-tile (a sub-tile never
// straddles a 128-row scale block since I is a multiple of 64).
// ------------------------------------------------------------------------------------
// LDS bytes of one tile body: A and B rings, scale slots, row sources, row-amax exchange,
// bias
template <int BN, int WM, int SM, int SA, int SB, bool FP4 = false, int XR = 0>
constexpr int big_tile_lds() {
  constexpr int BM = 16 * SM * WM + 16 * XR;
  return SA * BM * 128 + SB * BN * (FP4 ? 64 : 128) + SA * (8 + XR) * 64 * 4 + (BM + 63) / 64 * 64 * 4 +
         (8 / WM) * BM * 4 + BN * 2;
}

// Row stride (floats) of the extra rows' sums in LDS: BN + 4, so that the 16 rows of a
// fragment's float4 accesses fall in distinct banks.
template <int BN>
constexpr int big_extra_stride() { return BN + 4; }

// One M-tile x n-tile: WM x (8 / WM) waves, each SM 16-row sub-tiles by BN / (8 / WM)
// columns; SA / SB ring slots.  FP4 (with MX): MXFP4 weights in the tiled storage; a
// B-ring slot is BN / 16 weight tiles of 1 KB, each fetched whole by one load.
// Thread 0 takes the workgroup's next ticket from `queue` as the epilogue begins and
// stores it to *next (LDS) during the epilogue, so the atomic's round trip overlaps the
// epilogue's arithmetic instead of following it.
// XR = 1 (full tiles, block scales or MXFP8): the tile may hold 16 rows beyond BM (an
// expert's last rows, kBigExtraRows).  They are staged with the A ring (2 rows per wave,
// their scales in lanes 48.. of the wave's scale load, MX codes in a ninth row of the scale
// slot) and each wave multiplies them with two of its 16-column weight sub-tiles per step,
// after its own products; their sums live in LDS (accx, [16][big_extra_stride]), since the
// wave's registers are taken by its 64 x 128 accumulators, and get their own epilogue.  The
// arithmetic per element is the same as for every other row (the same promotion or the
// same scaled accumulation, in K order), so the outputs equal those of a separate tile.
template <bool SWIGLU, int BN, int WM, int SM, int SA, int SB, bool MX, bool FP4 = false, bool RAW = false,
          int XR = 0>
__device__ __forceinline__ void big_tile(const GemmArgs& a, const int nt, MTile mt, uint8_t* lds,
                                         int32_t* queue, int* next, float* accx) {
  constexpr int WAVES = 8, NT = WAVES * 64, WN = WAVES / WM, BM = 16 * SM * WM;
  constexpr int BMX = BM + 16 * XR, XPW = 16 * XR / WAVES;   // rows with the extra ones, per wave
  constexpr int XS = big_extra_stride<BN>();
  constexpr int WR = 16 * SM, WC = BN / WN;          // rows / columns of a wave
  constexpr int SN = WC / 16;                        // sub-tiles per wave along N
  constexpr int NG = SN / 2, GW = BN / (2 * WN);     // gemm1: gate sub-tiles / columns per wave
  constexpr int A_BYTES = BMX * 128, B_BYTES = BN * (FP4 ? 64 : 128);
  constexpr int A_ROWS = BM / WAVES, B_ROWS = BN / WAVES;   // rows each wave fetches per step
  constexpr int A_INSTR = A_ROWS / 8, B_INSTR = FP4 ? B_ROWS / 16 : B_ROWS / 8;
  static_assert(!FP4 || (MX && B_ROWS % 16 == 0), "MXFP4 weights: E8M0 scales, whole tiles per wave");
  static_assert(WC % 16 == 0 && BN % 64 == 0 && (!SWIGLU || SN % 2 == 0), "tile");
  static_assert(SA >= 2 && SB >= SA, "rings");
  static_assert(A_ROWS % 8 == 0 && A_ROWS <= 32 && WN * SN <= 32 && B_ROWS % 8 == 0, "scale lanes");
  // extra rows: block scales or MXFP8; two of a wave's sub-tiles each (gemm1: a gate and its
  // up sub-tile), all of a wave's columns in one 128-row weight scale block (gemm2)
  static_assert(XR == 0 || (XR == 1 && !FP4 && XPW == 2 && 32 + WN * SN <= 48 &&
                            (SWIGLU ? NG == WM : SN == 2 * WM && WC == 128)), "extra rows");

  uint8_t* ringA = lds;
  uint8_t* ringB = ringA + SA * A_BYTES;
  // per A slot and wave: lanes [0, A_ROWS) the activation scales of the wave's A rows,
  // [32, 32 + WN SN) the weight block scales of sub-tile n of column wave wn (wn SN + n)
  // (XR: a ninth row per slot, the MX codes of the extra rows: word 2 w + i = row BM + 2 w + i)
  float (*sS)[WAVES + XR][64] = reinterpret_cast<float (*)[WAVES + XR][64]>(ringB + SB * B_BYTES);
  int* rowsrc = reinterpret_cast<int*>(sS + SA);   // [BMX rounded up to 64] gemm1: perm entries
  float (*red)[BMX] = reinterpret_cast<float (*)[BMX]>(rowsrc + (BMX + 63) / 64 * 64);  // [WN][BMX]
  uint16_t* sbias = reinterpret_cast<uint16_t*>(red + WN);          // [BN] bias of the B rows (bf16)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.K, N = a.N, I = a.I;
  const int KB = ceil_div(K, kBlock), NBs = ceil_div(N, kBlock);
  const int e = mt.expert;
  // a wave computes only if some of its rows and some of its columns exist (the last
  // n-tile of a gemm1 over I = 64 mod 128 h columns, or of a gemm2 over N = 64 mod BN,
  // leaves whole column waves idle: they still fetch their share of the tile and pass the
  // barriers, but issue no fragment reads or matrix products)
  const int wave_col0 = SWIGLU ? nt * (BN / 2) + wn * GW : nt * BN + wn * WC;
  const bool wave_live = wm * WR < mt.row_end - mt.row_begin && wave_col0 < (SWIGLU ? I : N);
  const bool has_extra = XR > 0 && mt.row_end - mt.row_begin > BM;   // uniform
  const uint8_t* Bexp = a.B + static_cast<size_t>(e) * N * (FP4 ? KB * 64 : K);
  const float* Bsc = a.B_scale + static_cast<size_t>(e) * NBs * KB;

  // gemm1: the perm entries of the tile's rows go to LDS first (direct-to-LDS, so that the
  // weight prologue issued next can stay in flight while they are waited for)
  if constexpr (SWIGLU) {
    if (wave * 64 < BMX) {
      const int p = mt.row_begin + tid;
      load_lds4(p < mt.row_end ? static_cast<const void*>(a.perm + p) : static_cast<const void*>(kZeroScale),
                rowsrc + wave * 64);
    }
  }
  // source row in A of tile row r (-1: past the tile's rows; never past A)
  auto row_src = [&](int r) {
    const int p = mt.row_begin + r;
    int src = -1;
    if (p < mt.row_end) src = SWIGLU ? rowsrc[r] / a.top_k : p;
    return static_cast<unsigned>(src) < static_cast<unsigned>(a.A_rows) ? src : -1;
  };

  // global row of w13 / w2 behind B-tile row br (-1: past the matrix)
  auto b_global_row = [&](int br) {
    if (SWIGLU) {
      const int j = nt * (BN / 2) + (br % (BN / 2));
      return j < I ? (br >= BN / 2 ? I : 0) + j : -1;
    }
    const int col = nt * BN + br;
    return col < N ? col : -1;
  };

  // ---- fetch descriptors: the weight side first (it does not depend on the tile's rows),
  // so the B prologue is in flight while the activation rows are located ----
  const int a_slot = lane & 7, a_r8 = lane >> 3;
  unsigned b_off[B_INSTR];
  bool b_ok[B_INSTR];
#pragma unroll
  for (int i = 0; i < B_INSTR; ++i) {
    if constexpr (FP4) {
      // load i of the wave fetches weight tile (wave B_ROWS / 16 + i) of the B tile: lane
      // l lands at LDS byte 16 l of it, tile row l >> 2, slot l & 3, so it fetches that
      // row's chunk (l & 3) ^ swz4_key(row) (tiles past the matrix re-read the first)
      const int tr = lane >> 2, row = wave * B_ROWS + 16 * i + tr;
      const int g = b_global_row(row - tr);
      b_ok[i] = g >= 0;
      b_off[i] = static_cast<unsigned>(g < 0 ? b_global_row(0) : g) * KB * 64 + tr * 64 +
                 (((lane & 3) ^ swz4_key(tr)) << 4);
    } else {
      const int row = wave * B_ROWS + i * 8 + a_r8;
      const int g = b_global_row(row);
      b_ok[i] = g >= 0;
      // a row past the matrix re-reads the tile's first row (already in flight: no HBM
      // traffic); it only feeds output columns that are never stored
      b_off[i] = static_cast<unsigned>(g < 0 ? b_global_row(0) : g) * K + ((a_slot ^ swz_key(row)) << 4);
    }
  }
  auto issue_b = [&](int kt) {
    uint8_t* Bs = ringB + (kt % SB) * B_BYTES;
    const int k0 = kt * kBlock;
    if constexpr (FP4) {   // whole tiles (zero codes past K)
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i) load_lds16_s(b_off[i], Bexp + kt * 1024, Bs + (wave * B_ROWS + 16 * i) * 64);
    } else if (k0 + kBlock <= K) {
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i) load_lds16_s(b_off[i], Bexp + k0, Bs + (wave * B_ROWS + i * 8) * 128);
    } else {
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i) {
        const int row = wave * B_ROWS + i * 8 + a_r8;
        const int kk = k0 + ((a_slot ^ swz_key(row)) << 4);
        unsigned off = b_off[i];
        asm volatile("" : "+v"(off));
        const void* src = (b_ok[i] && kk < K) ? static_cast<const void*>(Bexp + off + k0) : kZeroChunk;
        load_lds16(src, Bs + (wave * B_ROWS + i * 8) * 128);
      }
    }
  };

  auto sub_brow = [&](int n) {   // B-tile row of sub-tile n of this wave
    if (SWIGLU) return n < NG ? wn * GW + 16 * n : BN / 2 + wn * GW + 16 * (n - NG);
    return wn * WC + 16 * n;
  };

  v4f acc[SM][SN];
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int n = 0; n < SN; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  {  // the tile's bias, staged with the first loads: wave w fetches B rows [w BN/8, (w+1) BN/8)
    const int br = wave * (BN / WAVES) + 2 * lane;
    const int g = b_global_row(br);
    const void* src = (a.bias != nullptr && g >= 0)
                          ? static_cast<const void*>(a.bias + static_cast<size_t>(e) * N + g)
                          : static_cast<const void*>(kZeroChunk);
    if (lane < BN / (2 * WAVES)) load_lds4(src, &sbias[wave * (BN / WAVES)]);
  }
  // prologue: the weight loads of steps [0, SB-1) go out first, then (gemm1) the perm
  // entries fetched above are waited for, and the activation loads of steps [0, SA-1)
  // follow; step 0 waits for all of them.  From then on every step issues A(kt + SA - 1)
  // before B(kt + SB - 1).
  for (int s = 0; s < SB - 1 && s < KB; ++s) issue_b(s);
  if constexpr (SWIGLU) {
    // the perm fetch is older than this wave's weight prologue and bias loads
    if (wave * 64 < BMX) {
      if (KB >= SB - 1) wait_vmcnt<(SB - 1) * B_INSTR + 1>();
      else wait_vmcnt<0>();
    }
    barrier_only();
  }

  unsigned a_off[A_INSTR];
  bool a_ok[A_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int row = wave * A_ROWS + i * 8 + a_r8;
    const int src = row_src(row);
    a_ok[i] = src >= 0;
    a_off[i] = static_cast<unsigned>(src < 0 ? 0 : src) * K + ((a_slot ^ swz_key(row)) << 4);
  }
  // XR: the wave's XPW extra rows, one load of lanes [0, 8 XPW) per step
  unsigned xr_off = 0;
  bool xr_ok = false;
  if constexpr (XR > 0) {
    const int row = BM + wave * XPW + a_r8;
    const int src = lane < 8 * XPW ? row_src(row) : -1;
    xr_ok = src >= 0;
    xr_off = static_cast<unsigned>(src < 0 ? 0 : src) * K + ((a_slot ^ swz_key(row)) << 4);
  }
  // A rows' scales: per token row (stride 1 per K-step), or gathered in dispatch order
  // with the K-step major (A_sd: the tile's rows of a K-step are one contiguous run)
  const float* s_ptr = kZeroScale;
  bool s_live = false;
  int s_step = 1;
  // (XR: lanes [48, 48 + XPW) the scales of the wave's extra rows)
  const bool xs_lane = XR > 0 && lane >= 48 && lane < 48 + XPW;
  if (lane < A_ROWS || xs_lane) {
    const int r = lane < A_ROWS ? wave * A_ROWS + lane : BM + wave * XPW + (lane - 48);
    const int src = row_src(r);
    s_live = src >= 0;
    if (a.A_sd != nullptr) {
      s_ptr = reinterpret_cast<const float*>(a.A_sd) + (s_live ? mt.row_begin + r : 0);
      s_step = a.sd_rows;
    } else {
      s_ptr = a.A_scale + static_cast<size_t>(src < 0 ? 0 : src) * KB;
    }
  } else if (lane >= 32 && lane < 32 + WN * SN) {
    const int q = lane - 32, qw = q / SN, n = q % SN;   // column wave qw, sub-tile n
    int row;
    if (SWIGLU) {
      const int j0 = nt * (BN / 2) + qw * GW + 16 * (n % NG);
      row = j0 < I ? ((n >= NG ? I : 0) + j0) / kBlock : -1;
    } else {
      const int c0 = nt * BN + qw * WC + 16 * n;
      row = c0 < N ? c0 / kBlock : -1;
    }
    s_live = row >= 0;
    s_ptr = Bsc + static_cast<size_t>(row < 0 ? 0 : row) * KB;
  }

  // MXFP8: every thread stages one 4-byte E8M0 row of K-step kt (the four 32-blocks of
  // its 128 columns): thread t < BM the A row t, BM <= t < BM + BN the B row t - BM; one
  // load per wave and step, like the block scales above
  // (a B row's 4 codes of step kt sit in its 16-row tile's 64-byte scale block)
  const uint8_t* x_ptr = reinterpret_cast<const uint8_t*>(kZeroScale);
  bool x_live = false;
  int x_step = 4;
  if constexpr (MX) {
    const int RS = 4 * KB;
    if (tid < BM) {
      const int src = row_src(tid);
      x_live = src >= 0;
      if (a.A_sd != nullptr) {
        x_ptr = reinterpret_cast<const uint8_t*>(a.A_sd + (x_live ? mt.row_begin + tid : 0));
        x_step = 4 * a.sd_rows;
      } else {
        x_ptr = a.A_mx + static_cast<size_t>(src < 0 ? 0 : src) * RS;
      }
    } else if (tid < BM + BN) {
      const int g = b_global_row(tid - BM);
      x_live = g >= 0;
      const int gg = g < 0 ? 0 : g;
      x_ptr = a.B_mx + (static_cast<size_t>(e) * N + (gg & ~15)) * RS + 4 * (gg & 15);
      x_step = 64;
    }
  }

  // XR with MX: lanes [0, XPW) fetch the E8M0 words of the wave's extra rows
  const uint8_t* xx_ptr = reinterpret_cast<const uint8_t*>(kZeroScale);
  bool xx_live = false;
  int xx_step = 4;
  if constexpr (MX && XR > 0) {
    if (lane < XPW) {
      const int src = row_src(BM + wave * XPW + lane);
      xx_live = src >= 0;
      if (a.A_sd != nullptr) {
        xx_ptr = reinterpret_cast<const uint8_t*>(a.A_sd + (xx_live ? mt.row_begin + BM + wave * XPW + lane : 0));
        xx_step = 4 * a.sd_rows;
      } else {
        xx_ptr = a.A_mx + static_cast<size_t>(src < 0 ? 0 : src) * 4 * KB;
      }
    }
  }

  auto issue_a = [&](int kt) {   // A rows and all scales of K-step kt
    uint8_t* As = ringA + (kt % SA) * A_BYTES;
    const int k0 = kt * kBlock;
    if (k0 + kBlock <= K) {
#pragma unroll
      for (int i = 0; i < A_INSTR; ++i) load_lds16_s(a_off[i], a.A + k0, As + (wave * A_ROWS + i * 8) * 128);
    } else {
#pragma unroll
      for (int i = 0; i < A_INSTR; ++i) {
        const int row = wave * A_ROWS + i * 8 + a_r8;
        const int kk = k0 + ((a_slot ^ swz_key(row)) << 4);
        unsigned off = a_off[i];
        asm volatile("" : "+v"(off));   // recompute the address here: no hoisted 64-bit copies
        const void* src = (a_ok[i] && kk < K) ? static_cast<const void*>(a.A + off + k0) : kZeroChunk;
        load_lds16(src, As + (wave * A_ROWS + i * 8) * 128);
      }
    }
    if constexpr (XR > 0) {
      if (lane < 8 * XPW) {
        uint8_t* dst = As + (BM + wave * XPW) * 128;
        if (k0 + kBlock <= K) {
          load_lds16_s(xr_off, a.A + k0, dst);
        } else {
          const int kk = k0 + ((a_slot ^ swz_key(BM + wave * XPW + a_r8)) << 4);
          unsigned off = xr_off;
          asm volatile("" : "+v"(off));
          load_lds16(xr_ok && kk < K ? static_cast<const void*>(a.A + off + k0) : kZeroChunk, dst);
        }
      }
    }
    if constexpr (MX) {
      const void* src = x_live ? static_cast<const void*>(x_ptr + static_cast<size_t>(x_step) * kt) : kZeroScale;
      load_lds4(src, &sS[kt % SA][wave][0]);
      if constexpr (XR > 0) {
        if (lane < XPW)
          load_lds4(xx_live ? static_cast<const void*>(xx_ptr + static_cast<size_t>(xx_step) * kt) : kZeroScale,
                    &sS[kt % SA][WAVES][wave * XPW]);
      }
    } else if (lane < A_ROWS || (lane >= 32 && lane < 32 + WN * SN) || xs_lane) {   // lanes 0.. always: one instruction
      const void* src = s_live ? static_cast<const void*>(s_ptr + static_cast<size_t>(kt) * s_step) : kZeroScale;
      load_lds4(src, &sS[kt % SA][wave][0]);
    }
  };
  for (int s = 0; s < SA - 1 && s < KB; ++s) issue_a(s);
  // "this wave's loads of step kt landed" (kt >= 1): A(j) is always followed by
  // B(j + SB - SA), and by the time step kt is waited for, A(kt + SA - 2) and
  // B(kt + SB - 2) are the last loads issued.  So with SB > SA the loads after A(kt) are B(kt + SB - SA) and the
  // SA - 2 later (A, B) step pairs; with SB == SA (B(kt) right after A(kt)) just those
  // pairs.  Near the end of K, where some of them were never issued, wait for all.
  auto wait_step = [&](int kt) {
    constexpr int PAIR = A_INSTR + 1 + (XR > 0 ? (MX ? 2 : 1) : 0) + B_INSTR;
    constexpr int AFTER = (SB > SA ? B_INSTR : 0) + (SA - 2) * PAIR;
    if (kt + SB - 2 < KB) {
      wait_vmcnt<AFTER>();
    } else {
      wait_vmcnt<0>();
    }
  };
  // The weight fragment is the MFMA's first operand and the activation fragment its
  // second, so a lane's four results are four adjacent columns of one row: the block
  // scale is one value per (m, n) and the epilogue stores are 4 or 16 bytes wide.
  v8i af[SM], bq[3];
  float sav[SM], sbv[SN];
  auto bfrag = [&](const uint8_t* Bs, int row, int g) {
    if constexpr (FP4) return lds_frag4(Bs, row, g);
    else return lds_frag(Bs, row, g);
  };
  int xa[SM], xb[SN];   // MXFP8: the lane's E8M0 codes (row lane & 15, 32-block lane >> 4)
  auto read_step = [&](int kt) {   // scales, A fragments and the first B fragment
    const int sl = kt % SA;
    const uint8_t* As = ringA + sl * A_BYTES;
    if constexpr (MX) {
      const uint8_t* xs = reinterpret_cast<const uint8_t*>(&sS[sl][0][0]);
#pragma unroll
      for (int n = 0; n < SN; ++n) xb[n] = xs[4 * (BM + sub_brow(n) + (lane & 15)) + (lane >> 4)];
#pragma unroll
      for (int m = 0; m < SM; ++m) {
        const int r = wm * WR + 16 * m + (lane & 15);
        af[m] = lds_frag(As, r, lane >> 4);
        xa[m] = xs[4 * r + (lane >> 4)];
      }
    } else {
#pragma unroll
      for (int n = 0; n < SN; ++n) sbv[n] = sS[sl][0][32 + wn * SN + n];
#pragma unroll
      for (int m = 0; m < SM; ++m) {
        const int r = wm * WR + 16 * m + (lane & 15);
        af[m] = lds_frag(As, r, lane >> 4);
        sav[m] = sS[sl][r / A_ROWS][r % A_ROWS];
      }
    }
    bq[0] = bfrag(ringB + (kt % SB) * B_BYTES, sub_brow(0) + (lane & 15), lane >> 4);
    bq[1] = bfrag(ringB + (kt % SB) * B_BYTES, sub_brow(1) + (lane & 15), lane >> 4);
  };

  // Software pipeline over the NP = SM x SN products of a step (column-major): product j
  // goes to partial j % 4 and is folded into its accumulator LAG products later (an MFMA
  // result is ready only a few MFMA issue slots after the MFMA), so the FMAs never wait
  // for the matrix pipe; B fragments are read two columns ahead.  The last LAG products of
  // a step are folded during the first MFMAs of the next one, after the barrier and the
  // next step's fragment reads have been issued, so the matrix pipe keeps running across
  // the step boundary.
  // gemm1: a wave's gate columns (GW of them, 32-aligned) lie in one 128-row scale block
  // of w13, and so do its up columns (I is a multiple of 64), so sub-tiles share two
  // weight scales and a step needs 2 SM scale products instead of SM SN
  auto scale_col = [&](int n) { return SWIGLU ? (n < NG ? 0 : NG) : n; };
  static_assert(!SWIGLU || (GW % 32 == 0 && 128 % GW == 0), "gate columns of a wave in one block");
  constexpr int NP = SM * SN, LAG = 2;
  // partials rotate through P registers; P divides NP so that a step's first products
  // never overwrite the previous step's last LAG, still unfolded
  constexpr int P = NP % 4 == 0 ? 4 : 3;
  static_assert(NP % P == 0 && LAG < P, "partials rotate across steps");
  v4f pp[P];
  float sc_tail[LAG] = {};
  wait_vmcnt<0>();   // the prologue (and the bias)
  barrier_only();
  if (wave_live) read_step(0);
  for (int kt = 0; kt < KB; ++kt) {
    // the slots of step kt-1 are free (every wave passed the barrier after reading them)
    if (kt + SA - 1 < KB) issue_a(kt + SA - 1);
    if (kt + SB - 1 < KB) issue_b(kt + SB - 1);
    if (MX && wave_live) {   // the matrix cores apply the E8M0 scales: no promotion
      const uint8_t* Bs = ringB + (kt % SB) * B_BYTES;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int n = j / SM, m = j % SM;
        if (m == 0 && n + 2 < SN) bq[(n + 2) % 3] = bfrag(Bs, sub_brow(n + 2) + (lane & 15), lane >> 4);
        acc[m][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq[n % 3], af[m], acc[m][n], FP4 ? 4 : 0,
                                                                     0, 0, xb[n], 0, xa[m]);
      }
      if constexpr (XR > 0) {   // the extra rows x the wave's sub-tiles c0, c1 (sums in accx)
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const int xr = ln & 15, xg = ln >> 4;
        const uint8_t* xs = reinterpret_cast<const uint8_t*>(&sS[kt % SA][0][0]);
        const v8i ax = lds_frag(ringA + (kt % SA) * A_BYTES, BM + xr, xg);
        const int xax = xs[4 * (WAVES * 64 + xr) + xg];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = SWIGLU ? wm + u * NG : 2 * wm + u;
          float4* d = reinterpret_cast<float4*>(accx + xr * XS + sub_brow(c) + 4 * xg);
          const float4 sm = *d;
          const v8i bx = bfrag(Bs, sub_brow(c) + xr, xg);
          const int xbx = xs[4 * (BM + sub_brow(c) + xr) + xg];
          const v4f q = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bx, ax, v4f{sm.x, sm.y, sm.z, sm.w},
                                                                         FP4 ? 4 : 0, 0, 0, xbx, 0, xax);
          *d = make_float4(q[0], q[1], q[2], q[3]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (wave_live) {
      const uint8_t* Bs = ringB + (kt % SB) * B_BYTES;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int n = j / SM, m = j % SM;
        if (m == 0 && n + 2 < SN) bq[(n + 2) % 3] = lds_frag(Bs, sub_brow(n + 2) + (lane & 15), lane >> 4);
        pp[j % P] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq[n % 3], af[m], zero, 0, 0, 0, 0, 0, 0);
        if (j >= LAG) {
          const int q = j - LAG;
          const float sc = sav[q % SM] * sbv[scale_col(q / SM)];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[q % SM][q / SM][i] = fmaf(pp[q % P][i], sc, acc[q % SM][q / SM][i]);
        } else if (kt > 0) {   // the previous step's product NP - LAG + j
          const int q = NP - LAG + j;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[q % SM][q / SM][i] = fmaf(pp[q % P][i], sc_tail[j], acc[q % SM][q / SM][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < LAG; ++j) sc_tail[j] = sav[(NP - LAG + j) % SM] * sbv[scale_col((NP - LAG + j) / SM)];
      if constexpr (XR > 0) {   // the extra rows x the wave's sub-tiles c0, c1: sums in accx
        // (the lane index is produced here, in the loop, so that no address of this block
        // stays live across the K loop: the body has no register to spare for one)
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const int xr = ln & 15, xg = ln >> 4;
        const v8i ax = lds_frag(ringA + (kt % SA) * A_BYTES, BM + xr, xg);
        const float sx = sS[kt % SA][xr / XPW][48 + xr % XPW];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = SWIGLU ? wm + u * NG : 2 * wm + u;
          float4* d = reinterpret_cast<float4*>(accx + xr * XS + sub_brow(c) + 4 * xg);
          float4 sm = *d;
          const v8i bx = lds_frag(Bs, sub_brow(c) + xr, xg);
          const v4f q = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bx, ax, zero, 0, 0, 0, 0, 0, 0);
          const float ec = sx * sbv[SWIGLU && u == 1 ? NG : 0];
          sm.x = fmaf(q[0], ec, sm.x); sm.y = fmaf(q[1], ec, sm.y);
          sm.z = fmaf(q[2], ec, sm.z); sm.w = fmaf(q[3], ec, sm.w);
          *d = sm;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (kt + 1 < KB) {
      wait_step(kt + 1);
      barrier_only();   // every wave is done with step kt's slots; step kt+1 has landed
      if (wave_live) read_step(kt + 1);
    }
  }
  if (!MX && wave_live) {      // the last step's last LAG products
#pragma unroll
    for (int j = 0; j < LAG; ++j) {
      const int q = NP - LAG + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q % SM][q / SM][i] = fmaf(pp[q % P][i], sc_tail[j], acc[q % SM][q / SM][i]);
    }
  }
  wait_vmcnt<0>();
  int ticket = 0;
  if (tid == 0) ticket = atomicAdd(queue, 1);   // lands while the epilogue computes

  // The extra rows' epilogue (has_extra, uniform): thread t takes row t / 32 of them and
  // 8 B-tile rows (gemm1: 4 h columns) of it; it clears what it read for the next tile.
  auto extra_epilogue = [&]() {
    __syncthreads();   // every wave's last accumulation into accx is done
    const int xr = tid >> 5, p = mt.row_begin + BM + xr;
    if constexpr (RAW) {
      const int c = (tid & 31) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = b_global_row(c + i);
        if (g >= 0 && p < mt.row_end) a.c_raw[static_cast<size_t>(p) * N + g] = accx[xr * XS + c + i];
        accx[xr * XS + c + i] = 0.f;
      }
    } else if constexpr (SWIGLU && MX) {   // 1x32 blocks: 8 threads of a row each
      const int hc = (tid & 31) * 4, j0 = nt * (BN / 2) + hc;
      const bool ok = j0 < I;
      float4* gp = reinterpret_cast<float4*>(accx + xr * XS + hc);
      float4* up = reinterpret_cast<float4*>(accx + xr * XS + BN / 2 + hc);
      const float4 gs = *gp, us = *up;
      *gp = make_float4(0.f, 0.f, 0.f, 0.f);
      *up = make_float4(0.f, 0.f, 0.f, 0.f);
      const float ga[4] = {gs.x, gs.y, gs.z, gs.w}, ua[4] = {us.x, us.y, us.z, us.w};
      const uint2 g2 = *reinterpret_cast<const uint2*>(&sbias[hc]);
      const uint2 u2 = *reinterpret_cast<const uint2*>(&sbias[BN / 2 + hc]);
      float bg[4], bu[4];
      bg[0] = __uint_as_float(g2.x << 16); bg[1] = __uint_as_float(g2.x & 0xFFFF0000u);
      bg[2] = __uint_as_float(g2.y << 16); bg[3] = __uint_as_float(g2.y & 0xFFFF0000u);
      bu[0] = __uint_as_float(u2.x << 16); bu[1] = __uint_as_float(u2.x & 0xFFFF0000u);
      bu[2] = __uint_as_float(u2.y << 16); bu[3] = __uint_as_float(u2.y & 0xFFFF0000u);
      float hv[4], mx = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = ga[i] + bg[i];
        const float u = ua[i] + bu[i];
        const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        hv[i] = ok ? h : 0.f;
        mx = fmaxf(mx, fabsf(hv[i]));
      }
#pragma unroll
      for (int w = 1; w < 8; w <<= 1) mx = fmaxf(mx, __shfl_xor(mx, w, 64));
      const int code = mx_scale_code(mx);
      const float mul = mx_inv_scale(code);
      if (p < mt.row_end) {
        if (ok)
          *reinterpret_cast<uint32_t*>(a.h_out + static_cast<size_t>(p) * I + j0) =
              encode4_mul(hv[0], hv[1], hv[2], hv[3], mul);
        if ((tid & 7) == 0) {   // j0 starts a 32-column block
          a.h_mx[static_cast<size_t>(p) * 4 * ceil_div(I, kBlock) + j0 / kMxBlock] = static_cast<uint8_t>(code);
          if (a.h_sd != nullptr)
            reinterpret_cast<uint8_t*>(a.h_sd)[(static_cast<size_t>(j0 / kBlock) * a.sd_rows + p) * 4 +
                                               (j0 / kMxBlock) % 4] = static_cast<uint8_t>(code);
        }
      }
    } else if constexpr (SWIGLU) {
      const int hc = (tid & 31) * 4, j0 = nt * (BN / 2) + hc;
      const bool ok = j0 < I;
      float4* gp = reinterpret_cast<float4*>(accx + xr * XS + hc);
      float4* up = reinterpret_cast<float4*>(accx + xr * XS + BN / 2 + hc);
      const float4 gs = *gp, us = *up;
      *gp = make_float4(0.f, 0.f, 0.f, 0.f);
      *up = make_float4(0.f, 0.f, 0.f, 0.f);
      const float ga[4] = {gs.x, gs.y, gs.z, gs.w}, ua[4] = {us.x, us.y, us.z, us.w};
      const uint2 g2 = *reinterpret_cast<const uint2*>(&sbias[hc]);
      const uint2 u2 = *reinterpret_cast<const uint2*>(&sbias[BN / 2 + hc]);
      float bg[4], bu[4];
      bg[0] = __uint_as_float(g2.x << 16); bg[1] = __uint_as_float(g2.x & 0xFFFF0000u);
      bg[2] = __uint_as_float(g2.y << 16); bg[3] = __uint_as_float(g2.y & 0xFFFF0000u);
      bu[0] = __uint_as_float(u2.x << 16); bu[1] = __uint_as_float(u2.x & 0xFFFF0000u);
      bu[2] = __uint_as_float(u2.y << 16); bu[3] = __uint_as_float(u2.y & 0xFFFF0000u);
      float hv[4], mx = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = ga[i] + bg[i];
        const float u = ua[i] + bu[i];
        const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        hv[i] = ok ? h : 0.f;
        mx = fmaxf(mx, fabsf(hv[i]));
      }
#pragma unroll
      for (int w = 1; w < 32; w <<= 1) mx = fmaxf(mx, __shfl_xor(mx, w, 64));
      const float sc = group_scale(mx);
      const float rs = __builtin_amdgcn_rcpf(sc);
      float q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q0 = hv[i] * rs;
        const float q1 = fmaf(fmaf(-q0, sc, hv[i]), rs, q0);
        q[i] = fminf(fmaxf(q1, -kFp8Max), kFp8Max);
      }
      if (p < mt.row_end) {
        const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false)) & 0xFFFFu;
        const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], 0, false)) & 0xFFFFu;
        if (ok) *reinterpret_cast<uint32_t*>(a.h_out + static_cast<size_t>(p) * I + j0) = lo | (hi << 16);
        if ((tid & 31) == 0) {
          a.h_scale[static_cast<size_t>(p) * ceil_div(I, kBlock) + nt] = sc;
          if (a.h_sd != nullptr) a.h_sd[static_cast<size_t>(nt) * a.sd_rows + p] = __float_as_uint(sc);
        }
      }
    } else {
      const int c = (tid & 31) * 8, c0 = nt * BN + c;
      float4* sp = reinterpret_cast<float4*>(accx + xr * XS + c);
      const float4 v0 = sp[0], v1 = sp[1];
      sp[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      sp[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 < N && p < mt.row_end) {   // N is a multiple of 64: all eight or none
        const uint4 b4 = *reinterpret_cast<const uint4*>(&sbias[c]);
        const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float blo = __uint_as_float(bw[i] << 16), bhi = __uint_as_float(bw[i] & 0xFFFF0000u);
          o[i] = f32_to_f16_sat(v[2 * i] + blo) | (static_cast<uint32_t>(f32_to_f16_sat(v[2 * i + 1] + bhi)) << 16);
        }
        *reinterpret_cast<uint4*>(a.y_out + static_cast<size_t>(p) * N + c0) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  };

  // ---- epilogue: lane holds rows r(m) = wm*WR + 16m + (lane & 15) and, per sub-tile n,
  // the four adjacent columns 16n + 4 (lane >> 4) + i of its column range ----
  const int cq = 4 * (lane >> 4);
  if constexpr (RAW) {   // the fp32 accumulators, at the B rows' global columns of C [rows, N]
    if (tid == 0) *next = ticket;
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const int g = b_global_row(sub_brow(n) + cq);   // four consecutive rows: all or none
      if (g < 0) continue;
#pragma unroll
      for (int m = 0; m < SM; ++m) {
        const int p = mt.row_begin + wm * WR + 16 * m + (lane & 15);
        if (p < mt.row_end)
          *reinterpret_cast<float4*>(a.c_raw + static_cast<size_t>(p) * N + g) =
              make_float4(acc[m][n][0], acc[m][n][1], acc[m][n][2], acc[m][n][3]);
      }
    }
    if constexpr (XR > 0) {
      if (has_extra) extra_epilogue();
    }
    return;
  }
  if constexpr (SWIGLU) {
    const int KBI = ceil_div(I, kBlock);
    float hv[SM][NG][4];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int j0 = nt * (BN / 2) + wn * GW + 16 * n + cq;
      const bool ok = j0 < I;                 // I is a multiple of 64: all four or none
      const uint2 g2 = *reinterpret_cast<const uint2*>(&sbias[sub_brow(n) + cq]);
      const uint2 u2 = *reinterpret_cast<const uint2*>(&sbias[sub_brow(n + NG) + cq]);
      float bg[4], bu[4];
      bg[0] = __uint_as_float(g2.x << 16); bg[1] = __uint_as_float(g2.x & 0xFFFF0000u);
      bg[2] = __uint_as_float(g2.y << 16); bg[3] = __uint_as_float(g2.y & 0xFFFF0000u);
      bu[0] = __uint_as_float(u2.x << 16); bu[1] = __uint_as_float(u2.x & 0xFFFF0000u);
      bu[2] = __uint_as_float(u2.y << 16); bu[3] = __uint_as_float(u2.y & 0xFFFF0000u);
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[m][n][i] + bg[i];
          const float u = acc[m][n + NG][i] + bu[i];
          const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          hv[m][n][i] = ok ? h : 0.f;
        }
    }
    if (tid == 0) *next = ticket;
    if constexpr (MX) {
      // 1x32 MX blocks of h: the wave's gate sub-tiles 2q and 2q+1 are 32 aligned
      // columns; the block maximum of a row is the lane's 8 values and those of the row's
      // other 3 lanes (lane >> 4).  Blocks past I (h = 0 there) get the pad code 127.
      static_assert(NG % 2 == 0, "whole MX blocks per wave");
      const int RSI = 4 * KBI;
#pragma unroll
      for (int m = 0; m < SM; ++m) {
        const int p = mt.row_begin + wm * WR + 16 * m + (lane & 15);
#pragma unroll
        for (int q = 0; q < NG / 2; ++q) {
          float mx = 0.f;
#pragma unroll
          for (int n = 2 * q; n < 2 * q + 2; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(hv[m][n][i]));
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const int code = mx_scale_code(mx);
          const float mul = mx_inv_scale(code);
          const int jb = nt * (BN / 2) + wn * GW + 32 * q;
          if (p < mt.row_end) {
            uint8_t* hrow = a.h_out + static_cast<size_t>(p) * I;
#pragma unroll
            for (int n = 2 * q; n < 2 * q + 2; ++n) {
              const int j0 = jb + 16 * (n - 2 * q) + cq;
              if (j0 < I)
                *reinterpret_cast<uint32_t*>(hrow + j0) =
                    encode4_mul(hv[m][n][0], hv[m][n][1], hv[m][n][2], hv[m][n][3], mul);
            }
            if ((lane >> 4) == 0) {
              a.h_mx[static_cast<size_t>(p) * RSI + jb / kMxBlock] = static_cast<uint8_t>(code);
              if (a.h_sd != nullptr)   // byte (jb / 32) mod 4 of word [jb / 128][p]
                reinterpret_cast<uint8_t*>(a.h_sd)[(static_cast<size_t>(jb / kBlock) * a.sd_rows + p) * 4 +
                                                   (jb / kMxBlock) % 4] = static_cast<uint8_t>(code);
            }
          }
        }
      }
      if constexpr (XR > 0) {
        if (has_extra) extra_epilogue();
      }
      return;
    }
    // Each 1x128 group of h is a row's 128 columns [128 c, 128 c + 128); a tile holds
    // BN/2 of them starting at nt * BN/2.  The scale of a group is only complete when
    // every tile that covers part of it has contributed, so tiles whose column range is
    // not a whole number of groups (BN/2 != 128) reduce per group across the tile.
    static_assert(!SWIGLU || BN == 256, "gemm1 groups are whole tiles");
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      float mx = 0.f;
#pragma unroll
      for (int n = 0; n < NG; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(hv[m][n][i]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (lane < 16) red[wn][wm * WR + 16 * m + lane] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const int r = wm * WR + 16 * m + (lane & 15);
      const int p = mt.row_begin + r;
      float amax = red[0][r];
#pragma unroll
      for (int w = 1; w < WN; ++w) amax = fmaxf(amax, red[w][r]);
      const float sc = group_scale(amax);   // exact fp32(amax / 448)
      // quotient h / sc: reciprocal estimate plus one residual correction
      const float rs = __builtin_amdgcn_rcpf(sc);
      if (p < mt.row_end) {
        uint8_t* hrow = a.h_out + static_cast<size_t>(p) * I;
#pragma unroll
        for (int n = 0; n < NG; ++n) {
          const int j0 = nt * (BN / 2) + wn * GW + 16 * n + cq;
          float q[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float q0 = hv[m][n][i] * rs;
            const float q1 = fmaf(fmaf(-q0, sc, hv[m][n][i]), rs, q0);
            q[i] = fminf(fmaxf(q1, -kFp8Max), kFp8Max);
          }
          const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false)) & 0xFFFFu;
          const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], 0, false)) & 0xFFFFu;
          if (j0 < I) *reinterpret_cast<uint32_t*>(hrow + j0) = lo | (hi << 16);
        }
        if (wn == 0 && lane < 16) {
          a.h_scale[static_cast<size_t>(p) * KBI + nt] = sc;
          if (a.h_sd != nullptr) a.h_sd[static_cast<size_t>(nt) * a.sd_rows + p] = __float_as_uint(sc);
        }
      }
    }
    if constexpr (XR > 0) {
      if (has_extra) extra_epilogue();
    }
  } else {
    if (tid == 0) *next = ticket;
#pragma unroll
    for (int n = 0; n < SN; ++n) {
      const int c0 = nt * BN + wn * WC + 16 * n + cq;
      if (c0 >= N) continue;                  // N is a multiple of 64: all four or none
      const uint2 b2 = *reinterpret_cast<const uint2*>(&sbias[sub_brow(n) + cq]);
      float bv[4];
      bv[0] = __uint_as_float(b2.x << 16); bv[1] = __uint_as_float(b2.x & 0xFFFF0000u);
      bv[2] = __uint_as_float(b2.y << 16); bv[3] = __uint_as_float(b2.y & 0xFFFF0000u);
#pragma unroll
      for (int m = 0; m < SM; ++m) {
        const int p = mt.row_begin + wm * WR + 16 * m + (lane & 15);
        if (p < mt.row_end)
          *reinterpret_cast<uint2*>(a.y_out + static_cast<size_t>(p) * N + c0) = make_uint2(
              f32_to_f16_sat(acc[m][n][0] + bv[0]) | (static_cast<uint32_t>(f32_to_f16_sat(acc[m][n][1] + bv[1])) << 16),
              f32_to_f16_sat(acc[m][n][2] + bv[2]) | (static_cast<uint32_t>(f32_to_f16_sat(acc[m][n][3] + bv[3])) << 16));
      }
    }
    if constexpr (XR > 0) {
      if (has_extra) extra_epilogue();
    }
  }
}

// Large-group GEMM launch: full M-tiles (256 rows, rings SA / SB) and narrow ones (at
// most 64 rows, rings SAN / SBN) share the launch and the work order.
//
// Persistent: one workgroup per CU (the LDS of a tile body is most of a CU's), each
// taking tiles from work queues until they run dry.  Tiles take from about 25 to 65 us,
// and with one workgroup per block the in-order dealing of blocks to XCDs left CUs idle
// between tiles (measured: busy about 77% of the launch).  The expert-major tile order is
// cut into eight contiguous ranges, one queue per XCD (block b runs on XCD b mod 8), so
// the workgroups of an XCD run neighbouring tiles together and share the expert's
// activation rows and weight tiles in their L2; a workgroup whose XCD's queue is empty
// takes from the other XCDs' queues.  Every queue head only grows, so every workgroup
// leaves after at most total + 8 of its fetches.  A tile's successor in the same queue is
// claimed during its epilogue (big_tile), the first ticket of each queue before its loop.
// XR = 1 (block scales or MXFP8, a.xr = kBigExtraRows): full tiles of up to 256 + 16 rows take
// the extra-row body; a separate instantiation, so that launches without such tiles keep
// the two-body kernel and its register allocation.
template <bool SWIGLU, int BN, int SA, int SB, int SAN, int SBN, bool MX = false, bool FP4 = false,
          bool RAW = false, int XR = 0>
__global__ __launch_bounds__(512) void grouped_gemm_big_kernel(const GemmArgs a, int ntiles) {
  static_assert(XR == 0 || (!FP4 && 16 * XR == kBigExtraRows), "extra rows of the tile list");
  constexpr int kFull = big_tile_lds<BN, 4, 4, SA, SB, FP4, XR>(), kNarrow = big_tile_lds<BN, 2, 2, SAN, SBN, FP4>();
  __shared__ __align__(16) uint8_t lds[kFull > kNarrow ? kFull : kNarrow];
  __shared__ __align__(16) float accx[XR ? 16 * big_extra_stride<BN>() : 4];
  __shared__ int s_next;
  __shared__ int32_t s_eto[257];   // expert_tile_off, read by every tile's lookup
  for (int i = threadIdx.x; i <= a.E; i += blockDim.x) s_eto[i] = a.expert_tile_off[i];
  for (int i = threadIdx.x; i < (XR ? 16 * big_extra_stride<BN>() : 4); i += blockDim.x) accx[i] = 0.f;
  const int total = __builtin_amdgcn_readfirstlane(*a.num_tiles) * ntiles;
  const int per_xcd = (total + kGemmQueues - 1) / kGemmQueues;
  const int x0 = blockIdx.x % kGemmQueues;
  for (int d = 0; d < kGemmQueues; ++d) {
    const int x = (x0 + d) % kGemmQueues;
    const int lo = x * per_xcd;
    const int n = total - lo < per_xcd ? total - lo : per_xcd;   // may be <= 0
    __syncthreads();   // the previous tile is done with LDS, every thread has read s_next
    int32_t* head = a.queue + x * kQueueStride;
    if (threadIdx.x == 0) s_next = n > 0 ? atomicAdd(head, 1) : n;
    __syncthreads();
    int t = __builtin_amdgcn_readfirstlane(s_next);
    while (t < n) {
      int nt;
      MTile mt;
      tile_of(a, s_eto, ntiles, lo + t, nt, mt);
      // (big_tile's first barrier precedes its write of s_next: every thread has read t)
      if (mt.row_end - mt.row_begin <= 64) {
        big_tile<SWIGLU, BN, 2, 2, SAN, SBN, MX, FP4, RAW>(a, nt, mt, lds, head, &s_next, accx);
      } else if (XR > 0 && mt.row_end - mt.row_begin > 256) {
        big_tile<SWIGLU, BN, 4, 4, SA, SB, MX, FP4, RAW, XR>(a, nt, mt, lds, head, &s_next, accx);
      } else {
        big_tile<SWIGLU, BN, 4, 4, SA, SB, MX, FP4, RAW>(a, nt, mt, lds, head, &s_next, accx);
      }
      __syncthreads();   // the tile is done with LDS; its successor's ticket is in s_next
      t = __builtin_amdgcn_readfirstlane(s_next);
    }
  }
}

// The row-run variant (its tile body is rowrun_tile): one launch-order tile per workgroup.
template <bool SWIGLU, int KS, bool MX = false, bool FP4 = false, int NW = 8, bool RAW = false>
__global__ __launch_bounds__(512) void grouped_gemm_rowrun_kernel(const GemmArgs a, int ntiles) {
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  int nt;
  MTile mt;
  if (!pick_tile(a, ntiles, nt, mt)) return;
  rowrun_tile<SWIGLU, KS, MX, FP4, NW, RAW>(a, nt, mt, dyn_lds);
}

// Block-scaled gemm1 on the row-run body at three workgroups per CU: bursts of 3 K-blocks
// keep it within 80 VGPRs (six waves per SIMD; with 4 it needs 94), so the gemm1
// workgroups of a decode layer (an M-tile x 128 h columns each; 736 on the 64-token
// gpt-oss-20b layer) are all resident at once instead of running in two rounds of 512
// (GEMM1 101.5 -> 95.7 us there, same box).  gemm2 at six waves either spills (3 K-blocks)
// or streams no faster (2), so it keeps the kernel above.
template <bool RAW>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(6, 6)))
void grouped_gemm_rowrun_g1_kernel(const GemmArgs a, int ntiles) {
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  int nt;
  MTile mt;
  if (!pick_tile(a, ntiles, nt, mt)) return;
  rowrun_tile<true, 3, false, false, 8, RAW>(a, nt, mt, dyn_lds);
}

// Large-group launch shapes (workgroup tile 256 x BN, A / B ring depths).  gemm2 takes the
// same 256-column tiles as gemm1 (a 64 x 128 tile per wave: fewer LDS fragment bytes per
// matrix product than 192 columns' 64 x 96); the waves whose columns lie past N skip their
// work, so an N that is not a multiple of 256 costs little (gemm2 453.9 -> 446.1 us at
// gpt-oss-120b prefill, N = 2880; 364 -> 341 us at qwen3 prefill; 3049 -> 2775 us at the
// DeepSeek-shaped layer, against 192-column tiles with a 3-deep weight ring).
constexpr int kG1BN = 256, kG1SA = 2, kG1SB = 2;
constexpr int kG2BN = 256, kG2SA = 2, kG2SB = 2;
// Ring depth of narrow (at most 64-row) tiles in the large-group launch.
constexpr int kNarrowS = 3;
// MXFP4 weights (half the B bytes per step): both GEMMs 256 wide, B rings one deeper,
// gemm2's A ring too (gemm2 352 vs 372 us on the gpt-oss-120b prefill layer; gemm1 no
// faster; 128-wide gemm2 tiles 495 us).
constexpr int kF4BN = 256, kF4SA1 = 2, kF4SA2 = 3, kF4SB = 3;
// Dynamic LDS of the row-run kernel at its largest K (64 blocks).
constexpr int kRowrunMaxLds = 64 * 2048 + 16 * 256 + 8 * 16 * 4;

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int gemm_tile_rows(long rows, int E) {
  const long avg = rows / (E > 0 ? E : 1);
  if (avg <= 24) return 16;
  if (avg <= 96) return 64;
  if (avg <= 160) return 128;
  return 256;
}

// Large dynamic LDS (above 64 KB) must be opted into per kernel; the row-run kernels stage
// up to 64 K-blocks of their 16-row activation tile.
static bool lds_opt_in(const void* kernel, size_t lds) {
  if (lds <= 64 * 1024) return true;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kRowrunMaxLds) == hipSuccess;
}
template <bool SWIGLU, int KS, bool MX, bool FP4, int NW, bool RAW>
static bool rowrun_lds_ok(size_t lds) {
  return lds_opt_in(reinterpret_cast<const void*>(grouped_gemm_rowrun_kernel<SWIGLU, KS, MX, FP4, NW, RAW>), lds);
}
// The block-scaled row-run launch of gemm1 (SWIGLU) or gemm2.
template <bool SWIGLU, bool RAW>
static bool rowrun_block_lds_ok(size_t lds) {
  if constexpr (SWIGLU) return lds_opt_in(reinterpret_cast<const void*>(grouped_gemm_rowrun_g1_kernel<RAW>), lds);
  else return rowrun_lds_ok<false, 4, false, false, 8, RAW>(lds);
}

static size_t rowrun_lds(int K) { return rowrun_lds_bytes(K); }

// Which kernel family takes a launch of bm-row M-tiles over K (the order of the tests in
// launch_gemm below).
enum class Family { kBig, kBigFp4, kRowrunFp4, kRowrun, kRing, kNone };

static Family family(bool mx, bool fp4, int K, int bm) {
  const int KB = ceil_div(K, kBlock);
  if (fp4) return bm == 256 ? Family::kBigFp4 : (bm == 16 && KB <= 64) ? Family::kRowrunFp4 : Family::kNone;
  if (bm == 256 || (mx && bm != 16)) return Family::kBig;
  if (bm == 16 && K % kBlock != 0 && KB <= 64) return Family::kRowrun;
  return mx ? Family::kNone : Family::kRing;
}

template <bool SWIGLU, bool RAW>
static bool prepare(bool mx, bool fp4, int K, int bm) {
  constexpr int KS = 4;
  const size_t lds = rowrun_lds(K);
  switch (family(mx, fp4, K, bm)) {
    case Family::kNone:
      return false;
    case Family::kRowrunFp4:
      return rowrun_lds_ok<SWIGLU, 4, true, true, 8, RAW>(lds) && rowrun_lds_ok<SWIGLU, 4, true, true, 2, RAW>(lds);
    case Family::kRowrun:
      // block-scaled: without the opt-in the LDS-ring kernel takes the launch instead
      return mx ? rowrun_lds_ok<SWIGLU, KS, true, false, 8, RAW>(lds)
                : (rowrun_block_lds_ok<SWIGLU, RAW>(lds), true);
    default:
      return true;
  }
}

bool gemm_prepare(bool swiglu, bool mx, bool fp4, int K, int bm, bool raw) {
  if (raw) return swiglu ? prepare<true, true>(mx, fp4, K, bm) : prepare<false, true>(mx, fp4, K, bm);
  return swiglu ? prepare<true, false>(mx, fp4, K, bm) : prepare<false, false>(mx, fp4, K, bm);
}

// Enqueues one grouped GEMM; gemm_prepare has accepted (mx, fp4, K, bm) on this device.
template <bool SWIGLU, bool RAW>
static void launch_gemm(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  // decode-sized groups stream weights: gemm2 takes 128-column tiles there, twice as many
  // workgroups over the same bytes, so the last round of tiles is not half empty
  const int bn = (!SWIGLU && bm == 16) ? 128 : 256;
  const int ntiles = SWIGLU ? ceil_div(a.I, 128) : ceil_div(a.N, bn);
  const long total = static_cast<long>(max_tiles) * ntiles;
  const int grid = static_cast<int>((total + 7) / 8 * 8);
  const long cus = device_cus();
  switch (family(a.mx, a.fp4, a.K, bm)) {
    case Family::kNone:
      return;
    case Family::kBigFp4: {
      // MXFP4 weights, large groups: 256-row tiles, persistent (one workgroup per CU)
      const int nt_big = SWIGLU ? ceil_div(a.I, kF4BN / 2) : ceil_div(a.N, kF4BN);
      const long tot = static_cast<long>(max_tiles) * nt_big;
      const int g = static_cast<int>(std::min((tot + 7) / 8 * 8, (cus + 7) / 8 * 8));
      grouped_gemm_big_kernel<SWIGLU, kF4BN, SWIGLU ? kF4SA1 : kF4SA2, kF4SB, kNarrowS, kNarrowS, true, true, RAW>
          <<<g, 512, 0, st>>>(a, nt_big);
      return;
    }
    case Family::kRowrunFp4: {
      const int cols = SWIGLU ? a.I : a.N;
      const size_t lds = rowrun_lds(a.K);
      // fewer 128-column workgroups than half the CUs (a few experts of a few tokens):
      // 32-column ones (gemm1 still covers whole 128-column groups: the idle waves past I
      // write the pad codes 127 of h's last scale word)
      const bool narrow = static_cast<long>(max_tiles) * ceil_div(cols, 128) < cus / 2;
      const int nts = !narrow ? ceil_div(cols, 128) : SWIGLU ? 4 * ceil_div(cols, 128) : ceil_div(cols, 32);
      const int g = static_cast<int>((static_cast<long>(max_tiles) * nts + 7) / 8 * 8);
      if (narrow)
        grouped_gemm_rowrun_kernel<SWIGLU, 4, true, true, 2, RAW><<<g, 128, lds, st>>>(a, nts);
      else
        grouped_gemm_rowrun_kernel<SWIGLU, 4, true, true, 8, RAW><<<g, 512, lds, st>>>(a, nts);
      return;
    }
    case Family::kBig: {
      constexpr int BN = SWIGLU ? kG1BN : kG2BN;
      const int nt_big = SWIGLU ? ceil_div(a.I, BN / 2) : ceil_div(a.N, BN);
      const long tot = static_cast<long>(max_tiles) * nt_big;
      // persistent: one workgroup per CU (a multiple of the queue count), at most one per tile
      const int g = static_cast<int>(std::min((tot + 7) / 8 * 8, (cus + 7) / 8 * 8));
      if (a.mx && a.xr > 0) {   // M-tiles of up to 256 + kBigExtraRows rows
        if constexpr (SWIGLU)
          grouped_gemm_big_kernel<true, kG1BN, kG1SA, kG1SB, kNarrowS, kNarrowS, true, false, RAW, 1><<<g, 512, 0, st>>>(a, nt_big);
        else
          grouped_gemm_big_kernel<false, kG2BN, kG2SA, kG2SB, kNarrowS, kNarrowS, true, false, RAW, 1><<<g, 512, 0, st>>>(a, nt_big);
      } else if (a.mx) {
        if constexpr (SWIGLU)
          grouped_gemm_big_kernel<true, kG1BN, kG1SA, kG1SB, kNarrowS, kNarrowS, true, false, RAW><<<g, 512, 0, st>>>(a, nt_big);
        else
          grouped_gemm_big_kernel<false, kG2BN, kG2SA, kG2SB, kNarrowS, kNarrowS, true, false, RAW><<<g, 512, 0, st>>>(a, nt_big);
      } else if (a.xr > 0) {   // M-tiles of up to 256 + kBigExtraRows rows
        if constexpr (SWIGLU)
          grouped_gemm_big_kernel<true, kG1BN, kG1SA, kG1SB, kNarrowS, kNarrowS, false, false, RAW, 1><<<g, 512, 0, st>>>(a, nt_big);
        else
          grouped_gemm_big_kernel<false, kG2BN, kG2SA, kG2SB, kNarrowS, kNarrowS, false, false, RAW, 1><<<g, 512, 0, st>>>(a, nt_big);
      } else if constexpr (SWIGLU) {
        grouped_gemm_big_kernel<true, kG1BN, kG1SA, kG1SB, kNarrowS, kNarrowS, false, false, RAW><<<g, 512, 0, st>>>(a, nt_big);
      } else {
        grouped_gemm_big_kernel<false, kG2BN, kG2SA, kG2SB, kNarrowS, kNarrowS, false, false, RAW><<<g, 512, 0, st>>>(a, nt_big);
      }
      return;
    }
    case Family::kRowrun: {
      // Decode-sized groups whose weight rows are not whole 128-byte lines (K = 64 mod 128,
      // so every other row starts mid-line and each 128-byte block of it spans two lines):
      // the row-run kernel, which fetches 64-byte pieces (always within one line) in long
      // per-row runs.  Rows that are whole lines stream faster through the LDS ring below.
      constexpr int KS = 4;
      const int nts = ceil_div(SWIGLU ? a.I : a.N, 128);
      const int g = static_cast<int>((static_cast<long>(max_tiles) * nts + 7) / 8 * 8);
      const size_t lds = rowrun_lds(a.K);
      if (a.mx) {
        grouped_gemm_rowrun_kernel<SWIGLU, KS, true, false, 8, RAW><<<g, 512, lds, st>>>(a, nts);
        return;
      }
      if (rowrun_block_lds_ok<SWIGLU, RAW>(lds)) {
        if constexpr (SWIGLU)
          grouped_gemm_rowrun_g1_kernel<RAW><<<g, 512, lds, st>>>(a, nts);
        else
          grouped_gemm_rowrun_kernel<false, KS, false, false, 8, RAW><<<g, 512, lds, st>>>(a, nts);
        return;
      }
      break;   // no large-LDS opt-in: the LDS-ring kernel
    }
    case Family::kRing:
      break;
  }
  switch (bm) {
    case 16:
      if constexpr (SWIGLU)
        grouped_gemm_kernel<16, 256, 1, 4, true, 4, RAW><<<grid, 256, 0, st>>>(a, max_tiles, ntiles, grid);
      else
        grouped_gemm_kernel<16, 128, 1, 4, false, 4, RAW><<<grid, 256, 0, st>>>(a, max_tiles, ntiles, grid);
      break;
    case 64:
      grouped_gemm_kernel<64, 256, 1, 4, SWIGLU, 3, RAW><<<grid, 256, 0, st>>>(a, max_tiles, ntiles, grid);
      break;
    default:
      grouped_gemm_kernel<128, 256, 2, 2, SWIGLU, 3, RAW><<<grid, 256, 0, st>>>(a, max_tiles, ntiles, grid);
      break;
  }
}

void launch_gemm1(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  launch_gemm<true, false>(a, bm, max_tiles, st);
}
void launch_gemm2(const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  launch_gemm<false, false>(a, bm, max_tiles, st);
}
void launch_gemm_raw(bool gemm1, const GemmArgs& a, int bm, int max_tiles, hipStream_t st) {
  if (gemm1)
    launch_gemm<true, true>(a, bm, max_tiles, st);
  else
    launch_gemm<false, true>(a, bm, max_tiles, st);
}

}  // namespace moe
